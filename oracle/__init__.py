"""CPU oracle for the routed-experts MoE decode step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  It wraps ``moe_oracle.c`` (plain C, FP64 sums) through
ctypes and shares nothing with the HIP library: no code, headers, tables or helpers.

Sources: the vLLM API pages "…cutedsl.moe.experts" (mx_block, plan_chunk,
ExpertsKernel.group / store_hidden / fc2 / finalize) and "…cutedsl.moe.experts_runtime"
(PersistentExperts.run: plan, then units, then the experts).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (IEEE semantics: no FMA contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        c = ctypes
        P = c.c_void_p
        L.oracle_e2m1_value.restype = c.c_double
        L.oracle_e2m1_value.argtypes = [c.c_uint]
        L.oracle_e4m3_value.restype = c.c_double
        L.oracle_e4m3_value.argtypes = [c.c_uint]
        L.oracle_e8m0_value.restype = c.c_double
        L.oracle_e8m0_value.argtypes = [c.c_uint]
        L.oracle_e4m3_encode.restype = c.c_uint
        L.oracle_e4m3_encode.argtypes = [c.c_float]
        L.oracle_float_to_bf16.restype = c.c_uint16
        L.oracle_float_to_bf16.argtypes = [c.c_float]
        L.oracle_block_exponent.restype = c.c_int
        L.oracle_block_exponent.argtypes = [c.c_float, c.c_int]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_e4m3_encode_array.argtypes = [P, c.c_int64, P]
        L.oracle_block_exponent_array.restype = None
        L.oracle_block_exponent_array.argtypes = [P, c.c_int64, c.c_int, P]
        L.oracle_quantize_blocks.restype = None
        L.oracle_quantize_blocks.argtypes = [P, c.c_int64, c.c_int, P, P]
        L.oracle_plan.restype = c.c_int
        L.oracle_plan.argtypes = [P, c.c_int, c.c_int, P, P]
        L.oracle_group.restype = c.c_int
        L.oracle_group.argtypes = [P, c.c_int, c.c_int, c.c_int, P, P]
        L.oracle_experts.restype = c.c_int
        L.oracle_experts.argtypes = [c.c_int, c.c_int, c.c_int, P, P, P, P, P, P, P, c.c_int,
                                     c.c_int, P, c.c_int, c.c_int, P, P, P, P, P, P, P, c.c_int, P]
        L.oracle_combine.restype = c.c_int
        L.oracle_combine.argtypes = [P, P, c.c_int, c.c_int, c.c_int, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------------------- formats
def e2m1_value(nibble: int) -> float:
    return lib().oracle_e2m1_value(nibble)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e8m0_value(code: int) -> float:
    return lib().oracle_e8m0_value(code)


def e4m3_encode(values) -> np.ndarray:
    v = _c(values, np.float32).ravel()
    out = np.empty(v.size, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out.reshape(np.shape(values))


def block_exponent(amax, floor_rule: bool) -> np.ndarray:
    a = _c(amax, np.float32).ravel()
    out = np.empty(a.size, np.int32)
    lib().oracle_block_exponent_array(_ptr(a), a.size, int(floor_rule), _ptr(out))
    return out.reshape(np.shape(amax))


def float_to_bf16(value: float) -> int:
    return lib().oracle_float_to_bf16(value)


def quantize_blocks(values, floor_rule: bool):
    """MXFP8 of consecutive 32-value blocks: returns (codes u8 [..., n], scales u8 [..., n/32])."""
    v = _c(values, np.float32)
    assert v.shape[-1] % 32 == 0
    nb = v.size // 32
    codes = np.empty(v.shape, np.uint8)
    scales = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint8)
    lib().oracle_quantize_blocks(_ptr(v), nb, int(floor_rule), _ptr(codes), _ptr(scales))
    return codes, scales


# ----------------------------------------------------------------------------- method
def plan(x_bf16: np.ndarray):
    """MXFP8 plan of BF16 rows (given as uint16 bits) -> (codes [B, D], scales [B, D/32])."""
    x = _c(x_bf16, np.uint16)
    B, D = x.shape
    codes = np.empty((B, D), np.uint8)
    scales = np.empty((B, D // 32), np.uint8)
    rc = lib().oracle_plan(_ptr(x), B, D, _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("oracle_plan: invalid arguments")
    return codes, scales


def group(ids: np.ndarray, E: int):
    """Unit table: (unit_expert [n], unit_rows [n, 8]) with -1 padding."""
    ids = _c(ids, np.int32)
    B, K = ids.shape
    ue = np.empty(max(B * K, 1), np.int32)
    ur = np.empty((max(B * K, 1), 8), np.int32)
    n = lib().oracle_group(_ptr(ids), B, K, E, _ptr(ue), _ptr(ur))
    if n < 0:
        raise ValueError("oracle_group: ids out of range or repeated within a token")
    return ue[:n].copy(), ur[:n].copy()


def experts(w13, s13, w2, s2, codes, scales, ids, *, hidden_floor: bool, routes=None,
            nthreads: int = 1, want_fc1: bool = False, want_hidden: bool = True,
            want_hidden_f32: bool = False, want_fc1_abs: bool = False):
    """Per-route FC1 -> SwiGLU -> MXFP8 requant -> FC2.  Canonical weight layouts:
    w13 [E, 2I, D/2], s13 [E, 2I, D/32], w2 [E, D, I/2], s2 [E, D, I/32].

    Returns dict(out=BF16 bits [n, D], out_f32=[n, D] (the rows before BF16 rounding),
    fc1=[n, 2I] f32 | None, fc1_abs=[n, 2I] f64 (sum of |w*x| of each FC1 row) | None,
    hidden=[n, I] f32 (the gated activation before its requantization) | None, hcodes=[n, I], hscales=[n, I/32], inexact=int)."""
    w13, s13, w2, s2 = (_c(a, np.uint8) for a in (w13, s13, w2, s2))
    codes, scales = _c(codes, np.uint8), _c(scales, np.uint8)
    ids = _c(ids, np.int32)
    E, I2, Dh = w13.shape
    D, I = Dh * 2, I2 // 2
    B, K = ids.shape
    r = None if routes is None else _c(routes, np.int32)
    n = B * K if r is None else r.size
    out = np.empty((n, D), np.uint16)
    out32 = np.empty((n, D), np.float32)
    fc1 = np.empty((n, 2 * I), np.float32) if want_fc1 else None
    hf = np.empty((n, I), np.float32) if want_hidden_f32 else None
    fa = np.empty((n, 2 * I), np.float64) if want_fc1_abs else None
    hc = np.empty((n, I), np.uint8) if want_hidden else None
    hs = np.empty((n, I // 32), np.uint8) if want_hidden else None
    inexact = ctypes.c_int64(0)
    rc = lib().oracle_experts(E, D, I, _ptr(w13), _ptr(s13), _ptr(w2), _ptr(s2), _ptr(codes),
                              _ptr(scales), _ptr(ids), B, K, _ptr(r), n, int(hidden_floor),
                              _ptr(out), _ptr(out32), _ptr(fc1), _ptr(fa), _ptr(hf), _ptr(hc), _ptr(hs), int(nthreads),
                              ctypes.byref(inexact))
    if rc:
        raise ValueError("oracle_experts: invalid arguments")
    return {"out": out, "out_f32": out32, "fc1": fc1, "fc1_abs": fa, "hidden": hf, "hcodes": hc, "hscales": hs,
            "inexact": inexact.value}


def combine(rows_bf16: np.ndarray, weights: np.ndarray, B: int, K: int) -> np.ndarray:
    rows = _c(rows_bf16, np.uint16)
    w = _c(weights, np.float32)
    D = rows.shape[-1]
    out = np.empty((B, D), np.uint16)
    rc = lib().oracle_combine(_ptr(rows), _ptr(w), B, K, D, _ptr(out))
    if rc:
        raise ValueError("oracle_combine: invalid arguments")
    return out


def default_hidden_floor(I: int) -> bool:
    """The pages requantize the hidden with the floor exponent rule on the TP8 shard
    (w13 of 768 rows, i.e. I = 384) and with the default rule otherwise
    (ExpertsKernel.store_hidden: mx_exponent(..., floor=tp == 8);
    PersistentExperts.__init__: tp = 8 iff w13 has 768 rows)."""
    return I == 384
