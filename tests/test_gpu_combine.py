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
    """End to end: the experts kernel's rows, combined on the GPU.

    Two bars.  (1) The combine itself, on the kernel's own rows: the _check bar above.
    (2) Against the oracle's rows combined by the oracle: per token, rel-L2 <= 1e-2, and
    each element within the route bar carried through the weighted sum.  A route's bar is
    max-abs <= 2e-2 x RMS of its oracle row plus half a BF16 ulp of its largest element;
    a route with a hidden code that FP32 summation order flipped may exceed it (the
    experts parity tests bound each such route by its flip's FC2 image), so such routes
    are counted (at most 1 %) and carry their own measured deviation.  The combine adds
    K route errors with weights w[t, s], so the token's bound is sum_s w[t, s] x (route
    bar), plus the FP32 accumulation bound and half a BF16 ulp of each combined row.  A
    bar scaled by the combined row's own RMS would not hold: the errors add linearly,
    while the RMS of a weighted sum of K nearly independent rows adds in quadrature."""
    from moe_routed_expert_mx_amd.layer import MoeLayer
    m = _lib()
    d = workloads.generate(name)
    w = d["workload"]
    log(f"combine after experts {name}")
    layer = MoeLayer(d["w13"], d["s13"], d["w2"], d["s2"], B_max=w.B, topk=w.K, device=DEV)
    x = torch.from_numpy(d["x"]).to(DEV)
    ids = torch.from_numpy(d["ids"]).to(DEV)
    rows = layer.forward(x, ids)
    weights = d["weights"].astype(np.float32)
    out = torch.empty(w.B, w.D, dtype=torch.bfloat16, device=DEV)
    m.moe_combine(rows, torch.from_numpy(weights).to(DEV), out)
    torch.cuda.synchronize()
    got16 = out.view(torch.uint16).cpu().numpy()
    _check(rows.view(torch.uint16).cpu().numpy(), weights, got16)
    codes, scales = oracle.plan(d["x"])
    ref_rows = oracle.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                              hidden_floor=oracle.default_hidden_floor(w.I))["out"]
    ref = bf16_to_f64(oracle.combine(ref_rows, weights, w.B, w.K))
    got = bf16_to_f64(got16)
    rel = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert np.all(rel <= 1e-2), rel.max()
    r = bf16_to_f64(ref_rows).reshape(w.B, w.K, w.D)
    y = bf16_to_f64(rows.view(torch.uint16).cpu().numpy()).reshape(w.B, w.K, w.D)
    plain = 2e-2 * np.sqrt(np.mean(r * r, axis=2)) + _half_ulp(np.abs(r).max(axis=2))
    dev = np.abs(y - r).max(axis=2)
    n_over = int((dev > plain).sum())
    assert n_over <= max(1, w.B * w.K // 100), f"{n_over} routes over the plain route bar"
    route_bar = np.maximum(plain, dev)
    wt = weights.astype(np.float64)
    acc = (w.K + 1) * 2.0 ** -24 * (np.abs(wt)[:, :, None] * np.abs(y)).sum(axis=1).max(axis=1)
    # both combined rows are rounded to BF16 once: half an ulp each
    bound = (np.abs(wt) * route_bar).sum(axis=1) + acc + _half_ulp(np.abs(ref).max(axis=1)) + \
        _half_ulp(np.abs(got).max(axis=1))
    worst = np.abs(got - ref).max(axis=1)
    assert np.all(worst <= bound), f"max-abs over the carried bar: {(worst / bound).max()}"
    log(f"  routes over the plain bar: {n_over}")
    log(f"  max-abs / carried bar: {(worst / bound).max():.3f}")


def _half_ulp(a):
    """Half a BF16 ulp at magnitude a (normal range)."""
    ex = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (ex - 8), 0.0)
