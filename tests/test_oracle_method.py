"""Pins of the oracle's method (plan, unit table, FC1 -> SwiGLU -> requant -> FC2,
combine) against things other than itself: dense FP64 matmuls of operands decoded
with torch and the OCP FP4 table, torch's float8 cast, closed forms (one-hot x,
all-ones weights, zero gate), brute-force constructions of the unit table, and the
routing invariants the pages state (rows in the caller's top-k order; routes to one
expert independent of each other)."""
import os

import numpy as np
import pytest
import torch

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fp4_table():
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    return np.array([float(v) for _, v in rows])


FP4 = _fp4_table()
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
E8M0 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()


def dq_fp4(codes_packed, scales):
    """[..., n/2] packed e2m1 + [..., n/32] E8M0 -> float64 [..., n]."""
    lo = FP4[codes_packed & 15]
    hi = FP4[codes_packed >> 4]
    v = np.stack([lo, hi], axis=-1).reshape(codes_packed.shape[:-1] + (-1,))
    return v * np.repeat(E8M0[scales], 32, axis=-1)


def dq_fp8(codes, scales):
    return E4M3[codes] * np.repeat(E8M0[scales], 32, axis=-1)


def bf16_bits(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.uint16).numpy()


def small(seed=0, **kw):
    base = dict(B=5, E=6, K=3, D=256, I=64, routing="uniform", scale_lo=-9, scale_hi=-5, seed=seed)
    base.update(kw)
    return workloads.generate(workloads.custom(**base))


# ------------------------------------------------------------------------------ plan
def test_plan_codes_match_torch_cast(orc):
    d = workloads.generate("decode_b8", with_weights=False)    # includes the x30 row
    codes, scales = orc.plan(d["x"])
    x = torch.from_numpy(d["x"]).view(torch.bfloat16).double().numpy()
    B, D = x.shape
    blocks = x.reshape(B, D // 32, 32)
    e = scales.astype(np.int64) - 127
    amax = np.abs(blocks).max(-1)
    # ceil rule: the smallest power of two keeping the block inside e4m3's range
    assert np.all(amax * 2.0 ** -e <= 448) and np.all(amax * 2.0 ** -(e - 1) > 448)
    scaled = (blocks * 2.0 ** -e[..., None]).astype(np.float32)
    ref = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes.reshape(B, D // 32, 32), ref)


def test_plan_exact_for_representable_rows(orc):
    """x built from e4m3 values times a per-block power of two (and a block maximum
    of 448 * 2^k) quantizes with no loss: codes decode back to x exactly."""
    rng = np.random.default_rng(7)
    B, D = 3, 512
    c = rng.integers(0, 126, (B, D // 32, 32))
    c[..., 0] = 0x7E                                 # block max 448 -> exponent k exactly
    sgn = np.where(rng.random((B, D // 32, 32)) < 0.5, -1.0, 1.0)
    k = rng.integers(-20, 20, (B, D // 32, 1))
    x = (E4M3[c] * sgn * 2.0 ** k).reshape(B, D).astype(np.float32)
    xb = bf16_bits(x)
    assert np.array_equal(torch.from_numpy(xb).view(torch.bfloat16).float().numpy(), x)
    codes, scales = orc.plan(xb)
    assert np.array_equal(scales.astype(np.int64) - 127, k[..., 0])
    assert np.array_equal(dq_fp8(codes, scales), x.astype(np.float64))


# ------------------------------------------------------------------------------ units
def _units_by_sorting(ids, E):
    """Independent construction: sort routes by (expert, token), cut in runs of 8."""
    B, K = ids.shape
    pairs = np.arange(B * K)
    e = ids.ravel()
    order = np.lexsort((pairs // K, e))
    ue, rows = [], []
    for ex in np.unique(e[order]):
        sel = order[e[order] == ex]
        for i in range(0, len(sel), 8):
            ue.append(ex)
            r = -np.ones(8, np.int64)
            r[: len(sel[i:i + 8])] = sel[i:i + 8]
            rows.append(r)
    return np.array(ue), np.array(rows).reshape(-1, 8)


@pytest.mark.parametrize("name", workloads.ORDER)
def test_group_matches_sorted_construction(orc, name):
    d = workloads.generate(name, with_weights=False)
    w = d["workload"]
    ue, ur = orc.group(d["ids"], w.E)
    ue2, ur2 = _units_by_sorting(d["ids"], w.E)
    assert np.array_equal(ue, ue2) and np.array_equal(ur, ur2)
    # every route exactly once
    real = ur[ur >= 0]
    assert np.array_equal(np.sort(real), np.arange(w.B * w.K))


def test_group_rejects_repeated_or_out_of_range(orc):
    with pytest.raises(ValueError):
        orc.group(np.array([[1, 1]], np.int32), 4)
    with pytest.raises(ValueError):
        orc.group(np.array([[1, 4]], np.int32), 4)


def test_group_many_tokens_one_expert(orc):
    ids = np.zeros((21, 1), np.int32)
    ids[5, 0] = 2
    ue, ur = orc.group(ids, 3)
    assert list(ue) == [0, 0, 0, 2]
    assert list(ur[0]) == [0, 1, 2, 3, 4, 6, 7, 8] and list(ur[1]) == list(range(9, 17))
    assert list(ur[2]) == [17, 18, 19, 20, -1, -1, -1, -1] and list(ur[3][:2]) == [5, -1]


# ------------------------------------------------------------------------------ experts
def _dense_reference(d, codes, scales, res, hidden_floor):
    """FP64 dense per-route matmuls of independently decoded operands."""
    w = d["workload"]
    I = w.I
    ids = d["ids"]
    X = dq_fp8(codes, scales)
    fc1 = np.empty((w.B * w.K, 2 * I))
    out = np.empty((w.B * w.K, w.D), np.uint16)
    for r in range(w.B * w.K):
        t, e = r // w.K, ids.ravel()[r]
        W13 = dq_fp4(d["w13"][e], d["s13"][e])
        fc1[r] = W13 @ X[t]
        W2 = dq_fp4(d["w2"][e], d["s2"][e])
        H = dq_fp8(res["hcodes"][r], res["hscales"][r])
        out[r] = bf16_bits((W2 @ H).astype(np.float32))
    return fc1.astype(np.float32), out


@pytest.mark.parametrize("which", ["tiny", "small", "small_floor"])
def test_experts_match_dense_fp64(orc, which):
    d = workloads.generate("tiny") if which == "tiny" else small(seed=3, B=4, E=5, K=3)
    floor = which == "small_floor"
    codes, scales = orc.plan(d["x"])
    res = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                      hidden_floor=floor, want_fc1=True, nthreads=4)
    assert res["inexact"] == 0                        # FP64 sums were exact
    fc1, out = _dense_reference(d, codes, scales, res, floor)
    assert np.array_equal(res["fc1"], fc1)
    assert np.array_equal(res["out"], out)
    # the sums of the FC1 terms' magnitudes: dense |W13| @ |X| of the same operands
    res2 = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                       hidden_floor=floor, want_fc1_abs=True, nthreads=2)
    X = np.abs(dq_fp8(codes, scales))
    for r in range(d["workload"].B * d["workload"].K):
        e = d["ids"].ravel()[r]
        mag = np.abs(dq_fp4(d["w13"][e], d["s13"][e])) @ X[r // d["workload"].K]
        assert np.allclose(res2["fc1_abs"][r], mag, rtol=1e-12, atol=0)
    # SwiGLU + requant of the FP32 FC1 values (torch's cast, exponent rule pinned in
    # test_oracle_formats): at least 99.9% identical, the rest one code apart
    g, u = fc1[:, : d["workload"].I].astype(np.float64), fc1[:, d["workload"].I:].astype(np.float64)
    h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
    hb = h.reshape(h.shape[0], -1, 32)
    e = res["hscales"].astype(np.int64) - 127
    amax = np.abs(hb).astype(np.float64).max(-1)
    if floor:
        assert np.all((amax == 0) | ((amax * 2.0 ** -e >= 256) & (amax * 2.0 ** -e < 512)))
    else:
        assert np.all((amax == 0) | (amax * 2.0 ** -e <= 448))
    ref = torch.from_numpy(np.clip(hb * 2.0 ** -e[..., None], -448, 448).astype(np.float32)) \
        .to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(h.shape)
    assert np.mean(ref == res["hcodes"]) >= 0.999


def test_experts_full_decode_b1_dense(orc):
    d = workloads.generate("decode_b1")
    codes, scales = orc.plan(d["x"])
    res = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                      hidden_floor=True, want_fc1=True, nthreads=8, routes=[0, 7, 15])
    assert res["inexact"] == 0
    X = dq_fp8(codes, scales)
    for i, r in enumerate([0, 7, 15]):
        e = d["ids"].ravel()[r]
        fc1 = (dq_fp4(d["w13"][e], d["s13"][e]) @ X[0]).astype(np.float32)
        assert np.array_equal(res["fc1"][i], fc1)
        H = dq_fp8(res["hcodes"][i], res["hscales"][i])
        out = bf16_bits((dq_fp4(d["w2"][e], d["s2"][e]) @ H).astype(np.float32))
        assert np.array_equal(res["out"][i], out)


def test_one_hot_x_selects_a_weight_column(orc):
    """x = e_k: the plan quantizes it exactly (scale 2^-8, code 0x78) and FC1 row r is
    dq(W13[e, r, k]) exactly."""
    d = small(seed=5, B=1, E=3, K=2, D=256, I=64)
    k = 77
    x = np.zeros((1, 256), np.float32)
    x[0, k] = 1.0
    xb = bf16_bits(x)
    codes, scales = orc.plan(xb)
    assert codes[0, k] == 0x78 and scales[0, k // 32] == 127 - 8
    res = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                      hidden_floor=False, want_fc1=True)
    for r in range(2):
        e = d["ids"].ravel()[r]
        col = dq_fp4(d["w13"][e], d["s13"][e])[:, k]
        assert np.array_equal(res["fc1"][r], col.astype(np.float32))


def test_all_ones_weights_sum_x(orc):
    """FP4 codes all 1.0 with unit scales: every FC1 row is sum_k dq(x_k)."""
    d = small(seed=6, B=2, E=2, K=1, D=512, I=32)
    d["w13"][:] = 0x22
    d["s13"][:] = 127
    codes, scales = orc.plan(d["x"])
    res = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                      hidden_floor=False, want_fc1=True)
    X = dq_fp8(codes, scales)
    for t in range(2):
        assert np.all(res["fc1"][t] == np.float32(X[t].sum()))


def _golden_swiglu():
    rows = []
    with open(os.path.join(GOLDEN, "swiglu.txt")) as f:
        for ln in f:
            if ln.strip() and not ln.startswith("#"):
                g, u, h = ln.split()[:3]
                rows.append((float(g), float(u), h))
    return rows


def _fp4_code_and_exponent(v):
    """v = FP4(code) * 2^k with code's magnitude in the OCP table: the (code, k) pair
    with the smallest |k| (found by search over the table, not by any oracle code)."""
    if v == 0:
        return 0, 0
    for k in sorted(range(-12, 13), key=abs):
        m = abs(v) / 2.0 ** k
        hit = np.flatnonzero(FP4[:8] == m)
        if hit.size:
            return int(hit[0]) | (8 if v < 0 else 0), k
    raise ValueError(v)


def test_swiglu_closed_forms(orc):
    """The gated activation on exact FC1 values (tests/golden/swiglu.txt): x = e_0
    quantizes exactly to 1.0, so FC1 row r is the hand-set weight W13[0, r, 0] and
    gate i / up i take the golden pair (g_i, u_i).  The oracle's FP32 hidden must equal
    the closed form g*u/(1+e^-g) rounded to FP32 -- a swapped gate/up half or a flipped
    sign inside the sigmoid changes almost every row."""
    gold = _golden_swiglu()
    I, D = 32, 64
    assert len(gold) == I
    w13 = np.zeros((1, 2 * I, D // 2), np.uint8)
    s13 = np.full((1, 2 * I, D // 32), 127, np.uint8)
    for i, (g, u, _) in enumerate(gold):
        for r, v in ((i, g), (I + i, u)):
            code, k = _fp4_code_and_exponent(v)
            w13[0, r, 0] = code                       # low nibble = k index 0
            s13[0, r, 0] = 127 + k
    w2 = np.zeros((1, D, I // 2), np.uint8)
    s2 = np.full((1, D, I // 32), 127, np.uint8)
    x = np.zeros((1, D), np.float32)
    x[0, 0] = 1.0
    codes, scales = orc.plan(bf16_bits(x))
    res = orc.experts(w13, s13, w2, s2, codes, scales, np.zeros((1, 1), np.int32), hidden_floor=False,
                      want_fc1=True, want_hidden_f32=True)
    # the FC1 values are exactly the pairs (the construction is right)
    assert np.array_equal(res["fc1"][0, :I], np.array([g for g, _, _ in gold], np.float32))
    assert np.array_equal(res["fc1"][0, I:], np.array([u for _, u, _ in gold], np.float32))
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    for i, (g, u, lit) in enumerate(gold):
        # the literal is the closed form (re-derived here at 50 digits as a typo guard)
        exact = Decimal(repr(g)) / (1 + (-Decimal(repr(g))).exp()) * Decimal(repr(u))
        assert abs(Decimal(lit) - exact) <= abs(exact) * Decimal("1e-25"), (i, lit, exact)
        assert res["hidden"][0, i] == np.float32(float(lit)), (i, g, u, res["hidden"][0, i], lit)
    swapped = [np.float32(u / (1 + np.exp(-u)) * g) for g, u, _ in gold]
    flipped = [np.float32(g / (1 + np.exp(g)) * u) for g, u, _ in gold]
    assert np.sum(res["hidden"][0] != swapped) >= 20 and np.sum(res["hidden"][0] != flipped) >= 20


def test_swiglu_matches_torch_silu(orc):
    """On a random layer, the oracle's FP32 hidden is torch's SiLU (its own FP64
    implementation) of the gate times the up value, rounded once to FP32."""
    d = small(seed=21, B=4, E=5, K=3, I=96)
    codes, scales = orc.plan(d["x"])
    res = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"], hidden_floor=False,
                      want_fc1=True, want_hidden_f32=True)
    I = d["workload"].I
    g = torch.from_numpy(res["fc1"][:, :I].astype(np.float64))
    u = torch.from_numpy(res["fc1"][:, I:].astype(np.float64))
    ref = (torch.nn.functional.silu(g) * u).to(torch.float32).numpy()
    ulp = np.spacing(np.abs(ref).astype(np.float32))
    assert np.all(np.abs(res["hidden"] - ref) <= ulp)      # at most one FP32 rounding apart
    assert np.mean(res["hidden"] == ref) >= 0.999
    # and the hidden codes are the MXFP8 of exactly that FP32 hidden
    c2, s2 = orc.quantize_blocks(res["hidden"], floor_rule=False)
    assert np.array_equal(c2, res["hcodes"]) and np.array_equal(s2, res["hscales"])


def test_zero_gate_gives_zero_hidden_and_output(orc):
    d = small(seed=8, B=2, E=3, K=2, D=256, I=64)
    d["w13"][:, :64] = 0                              # gate rows -> g = 0 -> h = 0
    codes, scales = orc.plan(d["x"])
    res = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                      hidden_floor=False)
    assert np.all(res["hcodes"] & 0x7F == 0) and np.all(res["hscales"] == 0)
    assert np.all(res["out"] & 0x7FFF == 0)


def test_rows_follow_topk_order(orc):
    """Permuting a token's top-k slots permutes its output rows the same way."""
    d = small(seed=9, B=3, E=8, K=4)
    codes, scales = orc.plan(d["x"])
    a = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"], hidden_floor=False)
    perm = np.array([2, 0, 3, 1])
    ids2 = d["ids"][:, perm]
    b = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, ids2, hidden_floor=False)
    for t in range(3):
        assert np.array_equal(b["out"][t * 4:(t + 1) * 4], a["out"][t * 4:(t + 1) * 4][perm])


def test_routes_are_independent(orc):
    """A route's row equals a run of that single (token, expert) pair, whatever else
    is in the batch (the dedupe only shares weight streaming)."""
    d = small(seed=10, B=6, E=3, K=2)                 # few experts: many tokens share one
    codes, scales = orc.plan(d["x"])
    full = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"], hidden_floor=False)
    for r in range(12):
        t = r // 2
        single = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes[t:t + 1], scales[t:t + 1],
                             d["ids"][t:t + 1, r % 2:r % 2 + 1], hidden_floor=False)
        assert np.array_equal(single["out"][0], full["out"][r])


def test_route_subset_matches_full_run(orc):
    d = small(seed=11, B=4, E=5, K=3)
    codes, scales = orc.plan(d["x"])
    full = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"], hidden_floor=False)
    sub = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                      hidden_floor=False, routes=[11, 0, 5], nthreads=3)
    assert np.array_equal(sub["out"], full["out"][[11, 0, 5]])


def test_combine_matches_weighted_sum(orc):
    d = small(seed=12, B=3, E=4, K=3)
    codes, scales = orc.plan(d["x"])
    r = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"], hidden_floor=False)
    out = orc.combine(r["out"], d["weights"], 3, 3)
    y = torch.from_numpy(r["out"]).view(torch.bfloat16).double().numpy().reshape(3, 3, -1)
    ref = bf16_bits((d["weights"].astype(np.float64)[..., None] * y).sum(1).astype(np.float32))
    assert np.array_equal(out, ref)


def test_out_f32_rounds_to_out(orc):
    """The FP32 rows the oracle exposes are the rows before their BF16 rounding, and
    equal the dense FP64 FC2 of its hidden rounded once to FP32."""
    d = small(seed=13, B=3, E=4, K=2)
    codes, scales = orc.plan(d["x"])
    r = orc.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"], hidden_floor=False)
    assert np.array_equal(bf16_bits(r["out_f32"]), r["out"])
    for i in range(6):
        e = d["ids"].ravel()[i]
        y = dq_fp4(d["w2"][e], d["s2"][e]) @ dq_fp8(r["hcodes"][i], r["hscales"][i])
        assert np.array_equal(r["out_f32"][i], y.astype(np.float32))
