"""Shared helpers of the GPU parity tests: tolerance checks and oracle plumbing."""
import os
import sys

import numpy as np
import torch

# Output rows: BF16 rows within rel-L2 <= 1e-2 and max-abs <= 2e-2 x row RMS of the
# oracle's rows (FP32 accumulation order differs from the oracle's exact sums).
REL_L2 = 1e-2
MAX_ABS_RMS = 2e-2
# Hidden requantization: >= 99.9% of the e4m3 codes identical.
HIDDEN_MATCH = 0.999


def host_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return os.cpu_count() or 1


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(u16)).view(torch.bfloat16).double().numpy()


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _fp4_table():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    return np.array([float(v) for _, v in rows])


FP4 = _fp4_table()
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E8M0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def dq_fp4(codes_packed, scales):
    """[..., n/2] packed e2m1 + [..., n/32] E8M0 -> float64 [..., n] (test-side decoder)."""
    lo = FP4[codes_packed & 15]
    hi = FP4[codes_packed >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(codes_packed.shape[:-1] + (-1,))
    return v * np.repeat(E8M0[scales], 32, axis=-1)


def dq_fp8(codes, scales):
    return E4M3[codes] * np.repeat(E8M0[scales], 32, axis=-1)


def check_rows(got_u16: np.ndarray, ref_u16, what: str = ""):
    """ref: BF16 bits (uint16) or float64 reference rows."""
    g = bf16_to_f64(got_u16)
    r = bf16_to_f64(ref_u16) if ref_u16.dtype == np.uint16 else np.asarray(ref_u16, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite outputs"
    err = g - r
    rms = np.sqrt(np.mean(r * r, axis=-1))
    rel = np.linalg.norm(err, axis=-1) / np.maximum(np.linalg.norm(r, axis=-1), 1e-300)
    mx = np.abs(err).max(axis=-1)
    zero = rms == 0
    assert np.all(mx[zero] == 0), f"{what}: rows that must be zero are not"
    bad = np.flatnonzero(~zero & ((rel > REL_L2) | (mx > MAX_ABS_RMS * rms)))
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance, first {bad[:5]}: "
                           f"rel {rel[bad[:5]]}, maxabs/rms {(mx / np.maximum(rms, 1e-300))[bad[:5]]}")
    return float(rel.max()), float((mx / np.maximum(rms, 1e-300))[~zero].max() if (~zero).any() else 0.0)


def record_stats(stats: dict):
    """Append one parity record (JSON line) to gpurun_out/parity_stats.jsonl when that
    folder exists (GPU runs collect them; elsewhere nothing is written)."""
    import json
    d = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
    if os.path.isdir(d):
        with open(os.path.join(d, "parity_stats.jsonl"), "a") as f:
            f.write(json.dumps(stats) + "\n")


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()
