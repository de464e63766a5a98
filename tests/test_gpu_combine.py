"""The weighted top-k combine (moe_combine) against the oracle's combine.

The oracle sums w[t, s] * y[t*K + s, d] exactly (FP64) and rounds once (to FP32, then
BF16); the kernel accumulates FP32 fused multiply-adds in slot order and rounds to BF16.
The two BF16 results are identical except where the exact sum lies within the FP32
accumulation error bound (K + 1 roundings of at most 2^-24 of the summed magnitudes) of
a BF16 rounding boundary.  There the kernel's value must still be a BF16 rounding of a
value within that bound of the exact sum (one ulp from the oracle's, or more where the
sum cancels).  No other element may differ at all.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import bf16_to_f64, log

DEV = "cuda"


def _lib():
    import moe_routed_expert_mx_amd as m
    return m


def _bf16_rows(n, D, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(n, D, generator=g).to(torch.bfloat16).view(torch.uint16).numpy()


def _check(rows, w, got):
    B, K = w.shape
    ref = oracle.combine(rows, w, B, K)
    y = bf16_to_f64(rows).reshape(B, K, -1)
    terms = w.astype(np.float64)[:, :, None] * y
    exact = terms.sum(axis=1)
    bound = (K + 1) * 2.0 ** -24 * np.abs(terms).sum(axis=1)
    g, r = got.astype(np.int32), ref.astype(np.int32)
    diff = g != r
    # distance of the exact sum to the nearest BF16 rounding boundary: the midpoints
    # between the reference value and its two neighbours (codes one above and one
    # below in magnitude; the same sign)
    rv = bf16_to_f64(ref)
    r32 = ref.astype(np.uint32)
    up = bf16_to_f64((r32 + 1).astype(np.uint16))
    dn = np.where((r32 & 0x7FFF) > 0, bf16_to_f64((r32 - 1).astype(np.uint16)), -rv)
    ulp = np.abs(up - rv)
    near = np.minimum(np.abs(exact - (rv + up) / 2), np.abs(exact - (rv + dn) / 2)) <= bound + 1e-300
    bad = diff & ~near
    assert not bad.any(), f"{bad.sum()} elements differ away from a rounding boundary"
    # every kernel value is a BF16 rounding of some value within the FP32 error bound of
    # the exact sum (one ulp apart from the oracle, or more where the sum cancels)
    gv = bf16_to_f64(got)
    gulp = np.abs(bf16_to_f64((got.astype(np.uint32) + 1).astype(np.uint16)) - gv)
    ok = np.abs(gv - exact) <= bound + gulp / 2 * 1.0000001
    assert np.all(ok), f"{(~ok).sum()} elements are not a rounding of a value within the FP32 error bound"
    return int(diff.sum())


@pytest.mark.gpu
@pytest.mark.parametrize("name", workloads.ORDER)
def test_combine_workload_shapes(name):
    m = _lib()
    w = workloads.WORKLOADS[name]
    d = workloads.generate(name)
    log(f"combine {name}")
    rows = _bf16_rows(w.B * w.K, w.D, seed=100 + w.seed)
    weights = d["weights"].astype(np.float32)
    out = torch.empty(w.B, w.D, dtype=torch.bfloat16, device=DEV)
    m.moe_combine(torch.from_numpy(rows).to(DEV), torch.from_numpy(weights).to(DEV), out)
    torch.cuda.synchronize()
    n = _check(rows, weights, out.view(torch.uint16).cpu().numpy())
    log(f"  {n} near-boundary one-ulp differences of {w.B * w.D}")


@pytest.mark.gpu
@pytest.mark.parametrize("B,K,D", [(1, 1, 8), (3, 1, 512), (5, 7, 24), (2, 64, 4096)])
def test_combine_edge_shapes(B, K, D):
    m = _lib()
    log(f"combine edge B={B} K={K} D={D}")
    rows = _bf16_rows(B * K, D, seed=B * 1000 + K * 10 + D)
    g = torch.Generator("cpu").manual_seed(K)
    weights = torch.softmax(torch.randn(B, K, generator=g), dim=1).numpy().astype(np.float32)
    out = torch.empty(B, D, dtype=torch.bfloat16, device=DEV)
    m.moe_combine(torch.from_numpy(rows).to(DEV), torch.from_numpy(weights).to(DEV), out)
    torch.cuda.synchronize()
    got = out.view(torch.uint16).cpu().numpy()
    n = _check(rows, weights, got)
    if K == 1:  # a single product is exact in FP32: bit-identical
        assert n == 0


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["tiny", "decode_b8"])
def test_combine_after_experts(name):
    """End to end: the experts kernel's rows, combined on the GPU, against the oracle's
    rows combined by the oracle (rows are within the output tolerance of each other)."""
    from moe_routed_expert_mx_amd.layer import MoeLayer
    m = _lib()
    d = workloads.generate(name)
    w = d["workload"]
    log(f"combine after experts {name}")
    layer = MoeLayer(d["w13"], d["s13"], d["w2"], d["s2"], B_max=w.B, topk=w.K, device=DEV)
    x = torch.from_numpy(d["x"]).to(DEV)
    ids = torch.from_numpy(d["ids"]).to(DEV)
    rows = layer.forward(x, ids)
    out = torch.empty(w.B, w.D, dtype=torch.bfloat16, device=DEV)
    m.moe_combine(rows, torch.from_numpy(d["weights"].astype(np.float32)).to(DEV), out)
    torch.cuda.synchronize()
    codes, scales = oracle.plan(d["x"])
    ref_rows = oracle.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                              hidden_floor=oracle.default_hidden_floor(w.I))["out"]
    ref = bf16_to_f64(oracle.combine(ref_rows, d["weights"].astype(np.float32), w.B, w.K))
    got = bf16_to_f64(out.view(torch.uint16).cpu().numpy())
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    assert np.all(rel <= 1e-2), rel.max()
    assert np.all(np.abs(got - ref).max(axis=1) <= 2e-2 * rms * 4)
