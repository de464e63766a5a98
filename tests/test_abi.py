"""The C ABI library loads, exports every entry point include/moe_mx.h declares, and
rejects bad arguments on the host (no GPU needed: all of these return before any
HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mx.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def m():
    import moe_routed_expert_mx_amd as pkg
    return pkg


def test_every_declared_symbol_is_exported(m):
    names = _declared()
    assert len(names) >= 10
    lib = ctypes.CDLL(m._lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m.EXPORTED)


def test_status_strings(m):
    assert m.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert m.status_string(s) != "unknown status"


def test_sizes(m):
    assert m.moe_plan_bytes(1, 3584) == 3584 + 112
    assert m.moe_plan_bytes(256, 3584) == 256 * 3584 * 33 // 32
    assert m.moe_plan_bytes(0, 3584) == 0 and m.moe_plan_bytes(4, 100) == 0
    w13, s13, w2, s2 = m.moe_packed_weight_bytes(160, 3584, 384)
    # the packing only reorders: same bytes as the canonical layout when I % 128 == 0
    assert (w13, s13, w2, s2) == (160 * 768 * 1792, 160 * 768 * 112, 160 * 3584 * 192, 160 * 224 * 256)
    w13, s13, w2, s2 = m.moe_packed_weight_bytes(8, 512, 96)          # I padded to 128 for FC2
    assert w2 == 8 * 32 * 1 * 1024 and s2 == 8 * 32 * 256
    assert m.moe_workspace_bytes(160, 3584, 384, 256, 16) > m.moe_workspace_bytes(160, 3584, 384, 1, 16) > 0
    assert m.moe_workspace_bytes(160, 3584, 385, 8, 16) == 0            # I % 32 != 0
    assert m.moe_workspace_bytes(160, 3000, 384, 8, 16) == 0            # D % 512 != 0
    with pytest.raises(m.MoeError):
        m.moe_packed_weight_bytes(0, 3584, 384)


def test_host_side_argument_errors(m):
    L = m._lib.lib
    fake = ctypes.c_void_p(0x1000)      # never dereferenced: every call below fails its checks first
    assert L.moe_plan(None, 1, 512, fake, 10**6, None) == m._lib.MOE_EINVAL
    assert L.moe_plan(fake, 1, 500, fake, 10**6, None) == m._lib.MOE_EINVAL
    assert L.moe_plan(fake, 2, 512, fake, 100, None) == m._lib.MOE_ENOSPACE
    assert L.moe_group(fake, 1, 0, 16, fake, 10**6, None) == m._lib.MOE_EINVAL
    assert L.moe_group(fake, 1, 4, 16, fake, 10, None) == m._lib.MOE_ENOSPACE
    assert m.moe_units_bytes(1, 4, 16) > 0 and m.moe_units_bytes(0, 4, 16) == 0
    w = m.moe_weights_t(16, 512, 128, 0x1000, 0x1000, 0x1000, 0x1000)
    o = m.moe_run_opts_t()
    big = 10**9

    def run(B, K, units, ws, out, opts=o, wts=w):
        return L.moe_experts_run(ctypes.byref(wts), ctypes.byref(opts), fake, fake, units, B, K, fake, ws, fake, out,
                                 None)

    assert run(1, 4, big, big, 16) == m._lib.MOE_ENOSPACE              # output too small
    assert run(1, 4, big, 100, big) == m._lib.MOE_ENOSPACE             # workspace too small
    assert run(1, 4, 10, big, big) == m._lib.MOE_ENOSPACE              # unit table too small
    assert run(0, 4, big, big, big) == m._lib.MOE_EINVAL
    o.col_tiles = 4
    assert run(1, 4, big, big, big) == m._lib.MOE_EINVAL
    o.col_tiles, o.hidden_rule = 0, 5
    assert run(1, 4, big, big, big) == m._lib.MOE_EINVAL
    o.hidden_rule = 0
    o.col_tiles = 3     # 0 (default), 1 (one-tile kernel) or 2 (grouped kernel only)
    assert run(1, 4, big, big, big) == m._lib.MOE_EINVAL
    o.col_tiles = 1
    for bad_ring in (1, 5, -1):
        o.ring = bad_ring
        assert run(1, 4, big, big, big) == m._lib.MOE_EINVAL
    o.ring = 0
    ws1 = m.moe_workspace_bytes(16, 512, 128, 1, 4)
    assert run(2, 4, big, ws1, big) == m._lib.MOE_ENOSPACE          # workspace sized for one token
    bad = m.moe_weights_t(16, 512, 100, 0x1000, 0x1000, 0x1000, 0x1000)
    assert run(1, 4, big, big, big, m.moe_run_opts_t(), bad) == m._lib.MOE_EINVAL
    assert L.moe_pack_weights(16, 512, 128, None, fake, fake, fake, fake, fake, fake, fake, None) == m._lib.MOE_EINVAL
    assert L.moe_workspace_init(None, 1024, None) == m._lib.MOE_EINVAL


def test_product_does_not_reach_the_oracle():
    """The HIP path and the oracle share nothing: no imports either way, no shared
    sources."""
    pkg = os.path.join(ROOT, "moe_routed_expert_mx_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in re.sub(r"#.*|//.*", "", src).lower().replace("oracle_", ""), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            src = open(os.path.join(ROOT, "oracle", f)).read()
            assert "moe_routed_expert_mx_amd" not in src and "moe_mx.h" not in src


def test_combine_argument_checks():
    """moe_combine rejects bad arguments on the host, before any launch."""
    import ctypes
    import moe_routed_expert_mx_amd as m
    L = m._lib.lib
    fake = ctypes.c_void_p(0x1000)
    big = 1 << 40
    assert L.moe_combine(None, big, fake, 1, 4, 512, fake, big, None) == m._lib.MOE_EINVAL
    assert L.moe_combine(fake, big, fake, 1, 4, 500, fake, big, None) == m._lib.MOE_EINVAL   # D % 8
    assert L.moe_combine(fake, big, fake, 0, 4, 512, fake, big, None) == m._lib.MOE_EINVAL
    assert L.moe_combine(fake, 4 * 512 * 2 - 1, fake, 1, 4, 512, fake, big, None) == m._lib.MOE_ENOSPACE
    assert L.moe_combine(fake, big, fake, 1, 4, 512, fake, 512 * 2 - 1, None) == m._lib.MOE_ENOSPACE


def test_decode_run_argument_checks(m):
    """moe_decode_run (the whole step in one launch) checks its arguments on the host;
    the decode-only options are refused by moe_experts_run."""
    L = m._lib.lib
    fake = ctypes.c_void_p(0x1000)
    big = 10**9
    w = m.moe_weights_t(16, 512, 128, 0x1000, 0x1000, 0x1000, 0x1000)

    def dec(B, K, ws=big, out=big, opts=None, x=fake, ids=fake):
        o = opts if opts is not None else m.moe_run_opts_t()
        return L.moe_decode_run(ctypes.byref(w), ctypes.byref(o), x, ids, B, K, fake, ws, fake, out, None)

    # more than 8 tokens: the grouped kernel in one launch, which refuses the options of
    # the whole-K decode kernel and the split-block exchanges on the host
    for field, value in (("fc2_claims", 1), ("exchange", 1), ("col_tiles", 1)):
        o = m.moe_run_opts_t()
        setattr(o, field, value)
        assert dec(9, 4, opts=o) == m._lib.MOE_EINVAL, field
    table, n = m._lib.prefetch_rows([(0x1000, 4096)])
    o = m.moe_run_opts_t()
    o.ahead, o.ahead_rows = ctypes.cast(table, ctypes.c_void_p), n
    assert dec(9, 4, opts=o) == m._lib.MOE_EINVAL
    assert dec(9, 4, out=9 * 4 * 512 * 2 - 1) == m._lib.MOE_ENOSPACE
    assert dec(0, 4) == m._lib.MOE_EINVAL
    assert dec(1, 0) == m._lib.MOE_EINVAL
    assert dec(1, 4, x=None) == m._lib.MOE_EINVAL
    assert dec(1, 4, ids=None) == m._lib.MOE_EINVAL
    assert dec(2, 4, out=2 * 4 * 512 * 2 - 1) == m._lib.MOE_ENOSPACE
    assert dec(2, 4, ws=100) == m._lib.MOE_ENOSPACE
    o = m.moe_run_opts_t()
    o.plan_dev, o.plan_bytes = 0x1000, 2 * 512 // 32 * 33 - 1  # plan dump too small
    assert dec(2, 4, opts=o) == m._lib.MOE_ENOSPACE
    o.plan_dev, o.plan_bytes = None, 64                        # a size without a buffer
    assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL
    o = m.moe_run_opts_t()
    o.exchange = 3
    assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL              # no such exchange
    # next-layer prefetch table: at most 64 rows, 16-byte aligned, below 2^31 bytes each
    table, n = m._lib.prefetch_rows([(0x1000, 4096)] * 65)
    o = m.moe_run_opts_t()
    o.ahead, o.ahead_rows = ctypes.cast(table, ctypes.c_void_p), 65
    assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL
    o.ahead_rows = 0
    o.ahead = None
    o.ahead_rows = 3                                           # rows without a table
    assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL
    for row in ((0x1008, 4096), (0x1000, 1 << 31), (0, 16)):
        table, n = m._lib.prefetch_rows([row])
        o.ahead, o.ahead_rows = ctypes.cast(table, ctypes.c_void_p), n
        assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL, row
        assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 2, 4, fake, big,
                                        None) == m._lib.MOE_EINVAL
    table, n = m._lib.prefetch_rows([(0x1000, 4096)])
    o.ahead, o.ahead_rows = ctypes.cast(table, ctypes.c_void_p), n
    assert L.moe_experts_run(ctypes.byref(w), ctypes.byref(o), fake, fake, big, 1, 4, fake, big, fake, big,
                             None) == m._lib.MOE_EINVAL             # the decode form's option
    o = m.moe_run_opts_t()
    o.fc2_claims = 2
    assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL              # FC2 claims: 0 (off) or 1 (on)
    assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 2, 4, fake, big,
                                    None) == m._lib.MOE_EINVAL
    o = m.moe_run_opts_t()
    o.col_tiles = 2
    assert dec(2, 4, opts=o) == m._lib.MOE_EINVAL              # the grouped kernel is not a decode form
    assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 2, 4, fake, big,
                                    None) == m._lib.MOE_EINVAL
    o = m.moe_run_opts_t()
    o.exchange = 1                                             # a decode-form option
    assert L.moe_experts_run(ctypes.byref(w), ctypes.byref(o), fake, fake, big, 1, 4, fake, big, fake, big,
                             None) == m._lib.MOE_EINVAL
    o = m.moe_run_opts_t()
    o.status_dev = 0x1000
    assert L.moe_experts_run(ctypes.byref(w), ctypes.byref(o), fake, fake, big, 1, 4, fake, big, fake, big,
                             None) == m._lib.MOE_EINVAL
    # a workspace sized for decode batches serves every B <= B_max of the form
    assert m.moe_workspace_bytes(160, 3584, 384, 8, 16) >= m.moe_workspace_bytes(160, 3584, 384, 1, 16)


def test_noalloc_host_side_limits(m):
    """The allocation-free entry point checks its limits on the host before any HIP call:
    B > 8 or an exchange other than 0 is MOE_EINVAL; a batch whose whole-K exchange would
    not fit its fixed scratch (here more than 128 distinct experts) is MOE_ELIMIT."""
    L = m._lib.lib
    fake = ctypes.c_void_p(0x1000)
    w = m.moe_weights_t(400, 512, 64, fake, fake, fake, fake)
    o = m.moe_run_opts_t()
    big = 8 * 40 * 512 * 2
    assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 9, 4, fake, big, None) \
        == m._lib.MOE_EINVAL
    assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 8, 40, fake, big, None) \
        == m._lib.MOE_ELIMIT
    o.exchange = 2
    assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 2, 4, fake, big, None) \
        == m._lib.MOE_EINVAL
    o.exchange = 0
    assert L.moe_decode_run_noalloc(ctypes.byref(w), ctypes.byref(o), fake, fake, 2, 4, fake, 16, None) \
        == m._lib.MOE_ENOSPACE
