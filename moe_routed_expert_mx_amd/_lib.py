"""ctypes binding of libmoe_mx.so (include/moe_mx.h): argument marshalling only.

Every entry point keeps the C name.  Tensors are torch tensors on the GPU (PyTorch is
used for device memory and streams only); every step of the path runs in the HIP
library.  Errors from the library raise ``MoeError``.  There is no fallback: if the
library is not built, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch first: the library runs on torch's streams and memory, so it must bind to the
# HIP runtime torch has loaded.  Loaded the other way round, the process holds two HIP
# runtimes and launches on torch's streams fail.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mx.so")

MOE_OK, MOE_EINVAL, MOE_ENOSPACE, MOE_EHIP, MOE_ELIMIT = 0, -1, -2, -3, -4


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} ({status})")
        self.status = status


class moe_weights_t(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("D", ctypes.c_int32), ("I", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("s13", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("s2", ctypes.c_void_p)]


class moe_run_opts_t(ctypes.Structure):
    _fields_ = [("hidden_rule", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("col_tiles", ctypes.c_int32), ("ring", ctypes.c_int32), ("exchange", ctypes.c_int32),
                ("fc2_claims", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2),
                ("hidden_codes_dev", ctypes.c_void_p), ("hidden_scales_dev", ctypes.c_void_p),
                ("plan_dev", ctypes.c_void_p), ("plan_bytes", ctypes.c_size_t), ("status_dev", ctypes.c_void_p),
                ("ahead", ctypes.c_void_p), ("ahead_rows", ctypes.c_int32)]


class moe_prefetch_row_t(ctypes.Structure):
    _fields_ = [("addr", ctypes.c_void_p), ("bytes", ctypes.c_uint64)]


def prefetch_rows(tensors_or_ranges):
    """A next-layer prefetch table (ctypes array of moe_prefetch_row_t, row count) from device
    tensors or (address, bytes) pairs."""
    rows = []
    for t in tensors_or_ranges:
        if isinstance(t, tuple):
            rows.append(moe_prefetch_row_t(t[0], t[1]))
        else:
            rows.append(moe_prefetch_row_t(t.data_ptr(), t.numel() * t.element_size()))
    return (moe_prefetch_row_t * max(len(rows), 1))(*rows), len(rows)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python moe_routed_expert_mx_amd/build.py` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    c, P = ctypes, ctypes.c_void_p
    sig = {
        "moe_status_string": (c.c_char_p, [c.c_int]),
        "moe_plan_bytes": (c.c_size_t, [c.c_int32, c.c_int32]),
        "moe_units_bytes": (c.c_size_t, [c.c_int32, c.c_int32, c.c_int32]),
        "moe_workspace_bytes": (c.c_size_t, [c.c_int32] * 5),
        "moe_packed_weight_bytes": (c.c_int, [c.c_int32] * 3 + [c.POINTER(c.c_size_t)] * 4),
        "moe_pack_weights": (c.c_int, [c.c_int32] * 3 + [P] * 9),
        "moe_workspace_init": (c.c_int, [P, c.c_size_t, P]),
        "moe_plan": (c.c_int, [P, c.c_int32, c.c_int32, P, c.c_size_t, P]),
        "moe_group": (c.c_int, [P, c.c_int32, c.c_int32, c.c_int32, P, c.c_size_t, P]),
        "moe_plan_group": (c.c_int, [P, P, c.c_int32, c.c_int32, c.c_int32, c.c_int32, P, c.c_size_t, P, c.c_size_t,
                                     P]),
        "moe_units_export": (c.c_int, [P, c.c_size_t, c.c_int32, c.c_int32, c.c_int32, P, P, P,
                                       c.c_int32, P]),
        "moe_experts_run": (c.c_int, [c.POINTER(moe_weights_t), c.POINTER(moe_run_opts_t), P, P, c.c_size_t,
                                      c.c_int32, c.c_int32, P, c.c_size_t, P, c.c_size_t, P]),
        "moe_decode_run": (c.c_int, [c.POINTER(moe_weights_t), c.POINTER(moe_run_opts_t), P, P, c.c_int32,
                                     c.c_int32, P, c.c_size_t, P, c.c_size_t, P]),
        "moe_decode_run_noalloc": (c.c_int, [c.POINTER(moe_weights_t), c.POINTER(moe_run_opts_t), P, P, c.c_int32,
                                             c.c_int32, P, c.c_size_t, P]),
        "moe_combine": (c.c_int, [P, c.c_size_t, P, c.c_int32, c.c_int32, c.c_int32, P, c.c_size_t, P]),
        "moe_work_split": (c.c_int, [c.c_int32] * 6 + [P, P]),
        "moe_grouped_runs": (c.c_int, [c.c_int32, P, c.c_int32, c.c_int32, c.c_int32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    return L


lib = _load()
EXPORTED = ("moe_status_string", "moe_plan_bytes", "moe_units_bytes", "moe_workspace_bytes", "moe_packed_weight_bytes",
            "moe_pack_weights", "moe_workspace_init", "moe_plan", "moe_group", "moe_plan_group", "moe_units_export",
            "moe_experts_run", "moe_decode_run", "moe_decode_run_noalloc", "moe_combine", "moe_work_split",
            "moe_grouped_runs")


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ------------------------------------------------------------------- entry points
def moe_plan_bytes(B: int, D: int) -> int:
    return lib.moe_plan_bytes(B, D)


def moe_units_bytes(B: int, topk: int, E: int) -> int:
    return lib.moe_units_bytes(B, topk, E)


def moe_workspace_bytes(E: int, D: int, I: int, B_max: int, topk: int) -> int:
    return lib.moe_workspace_bytes(E, D, I, B_max, topk)


def moe_packed_weight_bytes(E: int, D: int, I: int):
    out = [ctypes.c_size_t(0) for _ in range(4)]
    _check("moe_packed_weight_bytes", lib.moe_packed_weight_bytes(E, D, I, *[ctypes.byref(o) for o in out]))
    return tuple(o.value for o in out)


def moe_work_split(form: int, groups: int, D: int, I: int, grid: int, claims_ring: int = 0):
    """Host-side static split of an experts launch: (split [grid, 6], items [groups*I/32, 2])
    as numpy int32 arrays (no device call)."""
    import numpy as np
    split = np.zeros((grid, 6), np.int32)
    items = np.zeros((max(groups * (I // 32), 1), 2), np.int32)
    _check("moe_work_split", lib.moe_work_split(form, groups, D, I, grid, claims_ring, split.ctypes.data,
                                                items.ctypes.data))
    return split, items[:groups * (I // 32)]


def moe_grouped_runs(chunk_cols, D: int, I: int, grid: int):
    """Host-side FC2 runs of the grouped form's three-call launch: [grid, 2] int32
    {first tile, tiles} from the chunks' live column counts (no device call)."""
    import numpy as np
    cols = np.ascontiguousarray(chunk_cols, dtype=np.int32)
    runs = np.zeros((grid, 2), np.int32)
    _check("moe_grouped_runs", lib.moe_grouped_runs(len(cols), cols.ctypes.data if len(cols) else None, D, I, grid,
                                                    runs.ctypes.data))
    return runs


def moe_pack_weights(E, D, I, w13, s13, w2, s2, w13p, s13p, w2p, s2p, stream=None):
    _check("moe_pack_weights", lib.moe_pack_weights(E, D, I, *map(_ptr, (w13, s13, w2, s2, w13p, s13p, w2p, s2p)),
                                                    _stream(stream)))


def moe_workspace_init(ws, stream=None):
    _check("moe_workspace_init", lib.moe_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream)))


def moe_plan(x, plan, stream=None):
    B, D = x.shape
    _check("moe_plan", lib.moe_plan(_ptr(x), B, D, _ptr(plan), _nbytes(plan), _stream(stream)))


def moe_group(ids, E: int, units, stream=None):
    B, K = ids.shape
    _check("moe_group", lib.moe_group(_ptr(ids), B, K, E, _ptr(units), _nbytes(units), _stream(stream)))


def moe_plan_group(x, ids, E: int, plan, units, stream=None):
    """moe_plan and moe_group in one launch."""
    B, D = x.shape
    K = ids.shape[1]
    _check("moe_plan_group", lib.moe_plan_group(_ptr(x), _ptr(ids), B, D, K, E, _ptr(plan), _nbytes(plan),
                                                _ptr(units), _nbytes(units), _stream(stream)))


def moe_units_export(units, B, topk, E, header, unit_expert, unit_rows, stream=None):
    _check("moe_units_export", lib.moe_units_export(_ptr(units), _nbytes(units), B, topk, E, _ptr(header),
                                                    _ptr(unit_expert), _ptr(unit_rows), unit_expert.numel(),
                                                    _stream(stream)))


def _opts(hidden_rule, grid, col_tiles, ring, hidden_codes, hidden_scales, plan=None, status=None, exchange=0,
          fc2_claims=0, ahead=None):
    """ahead: None or (ctypes array of moe_prefetch_row_t, rows), e.g. from prefetch_rows();
    the caller keeps the array alive until the call returns."""
    table, rows = ahead if ahead is not None else (None, 0)
    return moe_run_opts_t(hidden_rule, grid, col_tiles, ring, exchange, fc2_claims, (ctypes.c_int32 * 2)(0, 0),
                          _ptr(hidden_codes), _ptr(hidden_scales), _ptr(plan), 0 if plan is None else _nbytes(plan),
                          _ptr(status), None if table is None else ctypes.cast(table, ctypes.c_void_p), rows)


def moe_experts_run(weights: moe_weights_t, plan, units, B: int, topk: int, ws, out, *, hidden_rule=0, grid=0,
                    col_tiles=0, ring=0, hidden_codes=None, hidden_scales=None, stream=None):
    opts = _opts(hidden_rule, grid, col_tiles, ring, hidden_codes, hidden_scales)
    _check("moe_experts_run", lib.moe_experts_run(ctypes.byref(weights), ctypes.byref(opts), _ptr(plan),
                                                  _ptr(units), _nbytes(units), B, topk, _ptr(ws), _nbytes(ws),
                                                  _ptr(out), _nbytes(out), _stream(stream)))


def moe_decode_run(weights: moe_weights_t, x, ids, ws, out, *, hidden_rule=0, grid=0, ring=0, exchange=0,
                   fc2_claims=0, ahead=None, hidden_codes=None, hidden_scales=None, plan=None, status=None,
                   stream=None):
    """The whole step of a batch in one launch (B <= 8: the decode kernel; B > 8: the
    grouped kernel making its own plan and chunk table): x BF16 [B, D] (or uint16
    bits), ids int32 [B, topk] -> out BF16 [B*topk, D]; optional plan (u8, the moe_plan
    layout) and status (int32 [1]) outputs; exchange 0 (whole-K hidden blocks, the
    default), 1 (tagged partial sums) or 2 (finished split blocks); fc2_claims 1 turns
    on the FC2 tail claims of exchange 0; ahead (from prefetch_rows) names the next layer's
    weights for the whole-K kernel to read into the Infinity Cache."""
    B, K = ids.shape
    opts = _opts(hidden_rule, grid, 0, ring, hidden_codes, hidden_scales, plan, status, exchange, fc2_claims,
                 ahead)
    _check("moe_decode_run", lib.moe_decode_run(ctypes.byref(weights), ctypes.byref(opts), _ptr(x), _ptr(ids), B, K,
                                                _ptr(ws), _nbytes(ws), _ptr(out), _nbytes(out), _stream(stream)))


def moe_decode_run_noalloc(weights: moe_weights_t, x, ids, out, *, hidden_rule=0, grid=0, ring=0, fc2_claims=0,
                           ahead=None, hidden_codes=None, hidden_scales=None, plan=None, status=None, stream=None):
    """moe_decode_run with the library's fixed per-device scratch instead of a workspace
    (no allocation; the whole-K decode form only, MOE_ELIMIT beyond its limits)."""
    B, K = ids.shape
    opts = _opts(hidden_rule, grid, 0, ring, hidden_codes, hidden_scales, plan, status, 0, fc2_claims, ahead)
    _check("moe_decode_run_noalloc", lib.moe_decode_run_noalloc(ctypes.byref(weights), ctypes.byref(opts), _ptr(x),
                                                                _ptr(ids), B, K, _ptr(out), _nbytes(out),
                                                                _stream(stream)))


def moe_combine(rows, weights, out, stream=None):
    """rows: BF16 [B*topk, D] (or uint16 bits), weights: FP32 [B, topk], out: BF16 [B, D]."""
    B, K = weights.shape
    D = rows.shape[-1]
    _check("moe_combine", lib.moe_combine(_ptr(rows), _nbytes(rows), _ptr(weights), B, K, D, _ptr(out), _nbytes(out),
                                          _stream(stream)))
