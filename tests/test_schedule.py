"""The experts launches' static work split and their waves' wait protocol, checked on
the CPU.

The split comes from the library itself (moe_work_split evaluates the kernels' own
split functions on the host), so these tests check the code that runs, not a copy.

* Cover: every FC1 item (one 32-wide hidden block of one group) goes to exactly one
  workgroup, and the FC2 runs partition the output tiles (the grouped form's three-call
  launch balances its runs on bytes: moe_grouped_runs, also checked for balance).
* Protocol: each workgroup's waves are modelled as ordered lists of posts and waits on
  their workgroup's LDS words, and on global block flags, in the order the kernels take
  them (experts page, ExpertsKernel: a co-resident grid whose CTAs wait on other CTAs'
  hidden blocks).  Running every wave as far as its waits allow must finish every wave:
  no wait cycle, for every split tested.
* Give-up: with one published block missing, the bounded waits end every wave, and the
  global waits end within one status poll period of the first give-up (each reads the
  status word every 256 polls).
"""
import itertools
import math

import numpy as np
import pytest

INF = 1 << 30
QSTREAM = 8          # streaming waves of either form (returned by moe_work_split too)


@pytest.fixture(scope="module")
def m():
    import moe_routed_expert_mx_amd as pkg
    return pkg


def _cases():
    shapes = [(3584, 384), (7168, 256), (512, 32), (1024, 96), (2048, 512), (7168, 384)]
    groups = [0, 1, 2, 3, 7, 13, 65, 128]
    grids = [1, 2, 7, 8, 33, 64, 256, 257]
    return shapes, groups, grids


# ---------------------------------------------------------------------------- cover
@pytest.mark.parametrize("form", [0, 1])
def test_split_covers_items_and_tiles(m, form):
    shapes, groups, grids = _cases()
    for (D, I), G, grid in itertools.product(shapes, groups, grids):
        if form == 1 and I > 384:
            continue
        HB, TPE = I // 32, D // 16
        split, items = m.moe_work_split(form, G, D, I, grid)
        n1, first2, n2 = split[:, 0], split[:, 1], split[:, 2]
        assert (split[:, 3] == QSTREAM).all()
        # FC1: item i to workgroup i mod grid, n1[c] of them
        assert n1.sum() == G * HB
        for c in range(grid):
            assert n1[c] == len(range(c, G * HB, grid)), (form, D, I, G, grid, c)
        # items are a bijection onto (group, block)
        pairs = set(map(tuple, items.tolist()))
        assert len(pairs) == G * HB
        assert pairs == {(g, j) for g in range(G) for j in range(HB)}
        # FC2 runs partition [0, G * TPE)
        assert (n2 >= 0).all() and n2.sum() == G * TPE
        live = np.flatnonzero(n2 > 0)
        order = live[np.argsort(first2[live], kind="stable")]
        pos = 0
        for c in order:
            assert first2[c] == pos, (form, D, I, G, grid, c)
            pos += n2[c]
        assert pos == G * TPE


def test_grouped_items_of_a_chunk_share_an_xcd(m):
    """Grouped form: with a grid that is a multiple of eight, the blocks of a chunk in a
    full group of eight chunks go to workgroups congruent mod 8 (one XCD: workgroup c
    runs on XCD c mod 8), so its hidden is exchanged within one L2."""
    for G, grid, (D, I) in itertools.product([8, 16, 61, 300], [8, 64, 256], [(7168, 256), (3584, 384)]):
        HB = I // 32
        _, items = m.moe_work_split(1, G, D, I, grid)
        xcd = {}
        for i, (ch, j) in enumerate(items.tolist()):
            if ch < G // 8 * 8:
                xcd.setdefault(ch, set()).add((i % grid) % 8)
        assert all(len(v) == 1 for v in xcd.values()), (G, grid, D, I)


def test_grouped_consecutive_chunks_stream_together(m):
    """Grouped form: in the groups of 32 chunks, four consecutive chunks share an XCD and
    a hidden block's items of those chunks lie within 24 of each other (the same round of
    items at a grid of 256), so an expert cut into two chunks mostly reads its weights
    once per XCD at the same time."""
    for G, (D, I) in itertools.product([32, 64, 170, 300], [(3584, 256), (3584, 384)]):
        HB = I // 32
        _, items = m.moe_work_split(1, G, D, I, 256)
        where = {}
        for i, (ch, j) in enumerate(items.tolist()):
            where[(ch, j)] = i
        big = G // 32 * 32
        for ch in range(0, big, 4):
            for j in range(HB):
                idx = [where[(c, j)] for c in range(ch, ch + 4)]
                assert len({x % 8 for x in idx}) == 1, (G, ch, j)
                assert max(idx) - min(idx) <= 24, (G, ch, j)


# ------------------------------------------------------- grouped form: byte-balanced runs
def _chunk_cols(rng, n, kind):
    if kind == "full":
        return np.full(n, 32, np.int32)
    if kind == "zipf":  # a few experts with several full chunks, then one small chunk each
        return np.where(rng.random(n) < 0.3, 32, rng.integers(1, 6, n)).astype(np.int32)
    return rng.integers(1, 33, n).astype(np.int32)


def _tile_costs(cols, D, I):
    """Cost of each FC2 tile in 16-byte units: its weights and scales, 16 (I/2 + I/32)
    bytes, and its BF16 output rows, 16 rows x 2 bytes per live column of its chunk."""
    return np.repeat(17 * I // 32 + 2 * cols.astype(np.int64), D // 16)


@pytest.mark.parametrize("kind", ["uniform", "zipf", "full"])
def test_grouped_runs_partition_and_balance(m, kind):
    """The three-call grouped launch's FC2 runs: contiguous, in chunk order, covering every
    tile once, each run's cost within one tile of the mean share."""
    rng = np.random.default_rng({"uniform": 1, "zipf": 2, "full": 3}[kind])
    for D, I in [(3584, 384), (3584, 256), (512, 32), (7168, 128)]:
        for n in [0, 1, 7, 151, 169, 1024]:
            if n * 32 > 65536 and kind == "full":
                continue
            cols = _chunk_cols(rng, n, kind)
            cost = _tile_costs(cols, D, I)
            for grid in [1, 7, 8, 256, 257]:
                runs = m.moe_grouped_runs(cols, D, I, grid)
                first, n2 = runs[:, 0], runs[:, 1]
                assert (n2 >= 0).all() and n2.sum() == n * (D // 16), (D, I, n, grid)
                assert first[0] == 0 and (first[1:] == first[:-1] + n2[:-1]).all(), (D, I, n, grid)
                if n == 0:
                    continue
                S = np.concatenate([[0], np.cumsum(cost)])
                share = S[-1] / grid
                run_cost = S[first + n2] - S[first]
                assert (np.abs(run_cost - share) <= cost.max() + 1).all(), (D, I, n, grid)
                if kind == "full":  # equal tile costs: tile counts differ by at most one
                    assert n2.max() - n2.min() <= 1


def test_grouped_runs_balance_a_skewed_batch(m):
    """Chunks of a Zipf-routed batch (popular experts in full chunks first, then one
    small chunk per tail expert): equal tile counts put ~1.3x the mean bytes on the first
    workgroups; the byte-balanced runs stay within a tile of the mean."""
    cols = np.array([32] * 40 + [3] * 110, np.int32)
    D, I, grid = 3584, 256, 256
    cost = _tile_costs(cols, D, I)
    S = np.concatenate([[0], np.cumsum(cost)])
    runs = m.moe_grouped_runs(cols, D, I, grid)
    bal = S[runs[:, 0] + runs[:, 1]] - S[runs[:, 0]]
    split, _ = m.moe_work_split(1, len(cols), D, I, grid)
    eq = S[split[:, 1] + split[:, 2]] - S[split[:, 1]]
    assert eq.max() / eq.mean() > 1.25
    assert bal.max() / bal.mean() < 1.02


def test_grouped_runs_protocol_has_no_cycle(m):
    """The grouped kernel's wait protocol with byte-balanced runs in place of equal ones."""
    rng = np.random.default_rng(4)
    for D, I in [(3584, 384), (512, 32)]:
        for n in [1, 13, 65, 128]:
            cols = _chunk_cols(rng, n, "zipf")
            for grid in [1, 8, 33, 256]:
                split, items = m.moe_work_split(1, n, D, I, grid)
                split[:, 1:3] = m.moe_grouped_runs(cols, D, I, grid)
                blocked, _, _ = _run(_grouped_actors(split, items, D, I))
                assert not blocked, (D, I, n, grid, blocked[:4])


def test_grouped_runs_reject_bad_arguments(m):
    L, E = m._lib.lib, m._lib.MOE_EINVAL
    cols = np.full(4, 8, np.int32)
    runs = np.zeros((4, 2), np.int32)
    ok = L.moe_grouped_runs(4, cols.ctypes.data, 3584, 384, 4, runs.ctypes.data)
    assert ok == m._lib.MOE_OK
    bad = np.array([8, 0, 8, 8], np.int32)
    assert L.moe_grouped_runs(4, bad.ctypes.data, 3584, 384, 4, runs.ctypes.data) == E     # 0 columns
    bad = np.array([8, 33, 8, 8], np.int32)
    assert L.moe_grouped_runs(4, bad.ctypes.data, 3584, 384, 4, runs.ctypes.data) == E     # > 32 columns
    assert L.moe_grouped_runs(1025, cols.ctypes.data, 3584, 384, 4, runs.ctypes.data) == E  # > 1024 chunks
    assert L.moe_grouped_runs(4, cols.ctypes.data, 3584, 512, 4, runs.ctypes.data) == E    # I > 384
    assert L.moe_grouped_runs(4, cols.ctypes.data, 3000, 384, 4, runs.ctypes.data) == E    # D % 512
    assert L.moe_grouped_runs(4, cols.ctypes.data, 3584, 384, 0, runs.ctypes.data) == E    # grid
    assert L.moe_grouped_runs(4, None, 3584, 384, 4, runs.ctypes.data) == E
    assert L.moe_grouped_runs(4, cols.ctypes.data, 3584, 384, 4, None) == E


def test_split_rejects_bad_arguments(m):
    L = m._lib.lib
    buf = np.zeros((4, 6), np.int32)
    E = m._lib.MOE_EINVAL
    assert L.moe_work_split(2, 1, 3584, 384, 4, 0, buf.ctypes.data, None) == E
    assert L.moe_work_split(0, 129, 3584, 384, 4, 0, buf.ctypes.data, None) == E
    assert L.moe_work_split(1, 1025, 3584, 384, 4, 0, buf.ctypes.data, None) == E
    assert L.moe_work_split(0, 1, 3584, 384, 0, 0, buf.ctypes.data, None) == E
    assert L.moe_work_split(0, 1, 3584, 384, 2049, 0, buf.ctypes.data, None) == E
    assert L.moe_work_split(0, 1, 3000, 384, 4, 0, buf.ctypes.data, None) == E
    assert L.moe_work_split(0, 1, 3584, 384, 4, 0, None, None) == E
    assert L.moe_work_split(0, 1, 3584, 384, 4, 1, buf.ctypes.data, None) == E      # ring 2..4
    assert L.moe_work_split(1, 1, 3584, 384, 4, 2, buf.ctypes.data, None) == E      # decode form only
    assert L.moe_work_split(0, 1, 3584, 384, 4, 2, buf.ctypes.data, None) == m._lib.MOE_OK


# ------------------------------------------------------------------------ protocol
def _wave_tiles(first2, n2, w):
    """FC2 tiles of streaming wave w: w, w + 8, ... of the workgroup's run."""
    return [first2 + t for t in range(w, n2, QSTREAM)]


def _fc2_ops(first2, n2, w, TPE, c):
    """A streaming wave's FC2 part: on entering a new hidden sequence (the run's groups,
    in order) it posts that it is done with the earlier ones, then waits for the
    loader's copy; at the end it posts that it is done with all."""
    ops, cur = [], None
    g0 = first2 // TPE
    for t in _wave_tiles(first2, n2, w):
        seq = t // TPE - g0
        if seq != cur:
            cur = seq
            ops += [("post", (c, "prog2", w), seq), ("wait", (c, "ready"), seq + 1)]
    ops.append(("post", (c, "prog2", w), INF))
    return ops


def _nseq(first2, n2, TPE):
    return (first2 + n2 - 1) // TPE - first2 // TPE + 1 if n2 > 0 else 0


def _decode_actors(split, items, D, I):
    """decode_whole_kernel: eight streaming waves (FC1 K steps w, w + 8, ... of each of
    the workgroup's items, then FC2 tiles), the finisher (adds the waves' partial tiles
    of each item, SwiGLU, publishes the block) and the loader (per hidden sequence: waits
    until the waves are done with the buffer it reuses, two back, then for the group's
    blocks, then copies)."""
    NS1, HB, TPE = D // 128, I // 32, D // 16
    grid = split.shape[0]
    actors = []
    for c in range(grid):
        n1, first2, n2 = (int(v) for v in split[c, :3])
        nw1 = min(NS1, QSTREAM)
        for w in range(QSTREAM):
            m1 = -(-(NS1 - w) // QSTREAM) if w < NS1 else 0
            ops = [("add", (c, "xdone"))]
            if n1 * m1 > 0:
                ops.append(("wait", (c, "xdone"), QSTREAM + 2))
            if m1 > 0:
                for k in range(n1):
                    ops += [("wait", (c, "cons"), k), ("post", (c, "prog", w), k + 1)]
            actors.append(ops + _fc2_ops(first2, n2, w, TPE, c))
        fin = [("add", (c, "xdone"))]
        for k in range(n1):
            fin += [("wait", (c, "prog", ww), k + 1) for ww in range(nw1)]
            fin.append(("post", (c, "cons"), k + 1))
            fin.append(("gpost", tuple(items[c + k * grid])))
        actors.append(fin)
        ld = [("add", (c, "xdone"))]
        g0 = first2 // TPE
        for seq in range(_nseq(first2, n2, TPE)):
            if seq >= 2:
                ld += [("wait", (c, "prog2", ww), seq - 1) for ww in range(QSTREAM)]
            ld += [("gwait", (g0 + seq, j)) for j in range(HB)]
            ld.append(("post", (c, "ready"), seq + 1))
        actors.append(ld)
    return actors


def _grouped_actors(split, items, D, I):
    """grouped_kernel: eight streaming waves (wave w runs the workgroup's items w, w + 8,
    ... whole, stages each finished block once the loader has published its previous
    one, then its FC2 tiles) and the loader (publishes the staged blocks in item order,
    then per hidden sequence: waits until every wave is done with the one buffer, then
    for the chunk's blocks, then copies)."""
    HB, TPE = I // 32, D // 16
    grid = split.shape[0]
    actors = []
    for c in range(grid):
        n1, first2, n2 = (int(v) for v in split[c, :3])
        for w in range(QSTREAM):
            n1w = -(-(n1 - w) // QSTREAM) if n1 > w else 0
            ops = []
            for mm in range(n1w):
                ops += [("wait", (c, "pub", w), mm), ("post", (c, "staged", w), mm + 1)]
            actors.append(ops + _fc2_ops(first2, n2, w, TPE, c))
        ld = []
        for k in range(n1):
            ww, mm = k % QSTREAM, k // QSTREAM
            ld += [("wait", (c, "staged", ww), mm + 1), ("gpost", tuple(items[c + k * grid])),
                   ("post", (c, "pub", ww), mm + 1)]
        g0 = first2 // TPE
        for seq in range(_nseq(first2, n2, TPE)):
            if seq >= 1:
                ld += [("wait", (c, "prog2", ww), seq) for ww in range(QSTREAM)]
            ld += [("gwait", (g0 + seq, j)) for j in range(HB)]
            ld.append(("post", (c, "ready"), seq + 1))
        actors.append(ld)
    return actors


def _run(actors, drop=None, bounded=False, lds_limit=64, poll_limit=4096, period=256):
    """Runs the waves.  Unbounded: every wave advances while its next wait holds; returns
    the waves left blocked (none means no wait cycle).  Bounded (a time-stepped model of
    the kernels' bounded waits, one poll per step): an LDS wait gives up after lds_limit
    polls; a global wait after poll_limit polls, or at a multiple of `period` polls once
    any wait has given up.  Returns (blocked waves, step of the first give-up, step of
    the last global give-up)."""
    lds, flags = {}, set()
    pc = [0] * len(actors)
    polls = [0] * len(actors)
    first_give_up, last_global = None, None
    step = 0
    while True:
        moved = False
        for a, ops in enumerate(actors):
            while pc[a] < len(ops):
                op = ops[pc[a]]
                kind = op[0]
                if kind == "post":
                    lds[op[1]] = max(lds.get(op[1], 0), op[2])
                elif kind == "add":
                    lds[op[1]] = lds.get(op[1], 0) + 1
                elif kind == "gpost":
                    if op[1] != drop:
                        flags.add(op[1])
                elif kind == "wait":
                    if lds.get(op[1], 0) < op[2]:
                        break
                elif kind == "gwait":
                    if op[1] not in flags:
                        break
                pc[a] += 1
                polls[a] = 0
                moved = True
        blocked = [a for a in range(len(actors)) if pc[a] < len(actors[a])]
        if not blocked:
            return [], first_give_up, last_global
        if moved:
            continue
        if not bounded:
            return blocked, None, None
        # one poll for every blocked wave; those past their bound give up and go on
        step += 1
        gave = []
        for a in blocked:
            polls[a] += 1
            kind = actors[a][pc[a]][0]
            if kind == "wait":
                out = polls[a] >= lds_limit
            else:
                out = polls[a] >= poll_limit or (first_give_up is not None and polls[a] % period == 0)
            if out:
                gave.append(a)
                if kind == "gwait":
                    last_global = step
        for a in gave:
            pc[a] += 1
            polls[a] = 0
        if gave and first_give_up is None:
            first_give_up = step


def _all_splits(m, form):
    shapes, groups, grids = _cases()
    for (D, I), G, grid in itertools.product(shapes[:4], groups, grids):
        if form == 1 and I > 384:
            continue
        split, items = m.moe_work_split(form, G, D, I, grid)
        yield D, I, G, grid, split, items


@pytest.mark.parametrize("form", [0, 1])
def test_wait_protocol_has_no_cycle(m, form):
    build = _decode_actors if form == 0 else _grouped_actors
    for D, I, G, grid, split, items in _all_splits(m, form):
        blocked, _, _ = _run(build(split, items, D, I))
        assert not blocked, (form, D, I, G, grid, blocked[:4])


@pytest.mark.parametrize("form", [0, 1])
def test_missing_block_gives_up_together(m, form):
    """A planted fault in the model (one block's flag never published): without bounds
    the consumers of its group block for good; with them every wave ends, and every
    global wait that gave up did so within one status period of the first give-up
    (it reads the status word every 256 polls), not after its own full bound."""
    build = _decode_actors if form == 0 else _grouped_actors
    D, I, G, grid = 3584, 384, 13, 33
    split, items = m.moe_work_split(form, G, D, I, grid)
    actors = build(split, items, D, I)
    drop = tuple(items[len(items) // 2])
    blocked, _, _ = _run(actors, drop=drop)
    assert blocked, "the planted fault blocks nobody: the model does not see the flags"
    blocked, first, last = _run(actors, drop=drop, bounded=True, lds_limit=10**6, poll_limit=4096, period=256)
    assert not blocked
    assert first is not None and first >= 4096
    assert last - first <= 256 + 1, (first, last)


# ------------------------------------------------------------- FC2 tail claims
def _kernel_constants():
    """The claim constants, read from the kernel source (so that the model follows it)."""
    import os
    import re
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "moe_routed_expert_mx_amd", "csrc", "moe_mx.hip")).read()
    get = lambda n: int(re.search(r"constexpr int %s = (\d+);" % n, src).group(1))
    return {"ahead": get("kQAhead"), "victims": get("kQVictims"), "ring": get("kQRing"), "grain": 8}


def _claims_model(split, items, D, I, R, K, rng):
    """decode_whole_kernel with FC2 tail claims, as interleavable generators (each yields
    the condition it waits on).  Streaming waves issue R slots ahead of what they consume;
    a slot past the wave's head takes the next queue entry (waiting until it is posted) and
    reports it taken.  The finisher, after FC1, re-arms its counter, claims its zone's
    grains from the front (each claim once every wave has taken all but `ahead` of the
    posted grains), then the zones of the next `victims` workgroups from the back where
    they lie in its last group, then posts the end entry; without a zone it posts the end
    entry first.  The counter is re-armed when the finisher starts; a claim that reaches a
    counter not yet re-armed sees the old call's tag and takes nothing.  Returns the
    generators and the record of computed tiles."""
    NS1, HB, TPE = D // 128, I // 32, D // 16
    grid = split.shape[0]
    A, V, RING, GR = K["ahead"], K["victims"], K["ring"], K["grain"]
    flags, ctr, done = set(), {}, []
    call = 7

    def wg(c):
        n1, first2, n2, _, zb, Z = (int(v) for v in split[c])
        st = {"prog": [0] * 8, "prog2": [0] * 8, "cons": 0, "ready": 0, "xdone": 0, "taken": [0] * 8,
              "posted": 0, "queue": [None] * RING, "history": []}
        g0 = first2 // TPE
        glast = (first2 + n2 - 1) // TPE if n2 > 0 else -1

        def post(first):
            st["queue"][st["posted"] % RING] = first
            st["history"].append(first)
            st["posted"] += 1

        def wave(w):
            m1 = -(-(NS1 - w) // 8) if w < NS1 else 0
            n1el = n1 * m1
            issued = []
            cur = {"t": first2 + w, "q": 0, "end": False}

            def issue():
                if len(issued) < n1el:
                    issued.append(("fc1",))
                    return
                if cur["t"] < zb:
                    issued.append(("tile", cur["t"]))
                    cur["t"] += 8
                    return
                if cur["end"]:
                    issued.append(("dummy",))
                    return
                q = cur["q"]
                yield lambda: st["posted"] >= q + 1
                s = st["queue"][q % RING]
                assert s == st["history"][q], "a queue entry was overwritten before its issue read it"
                cur["q"] += 1
                st["taken"][w] = cur["q"]
                if s < 0:
                    cur["end"] = True
                    issued.append(("dummy",))
                else:
                    issued.append(("tile", s + w))

            for _ in range(R):
                yield from issue()
            st["xdone"] += 1
            if n1el:
                yield lambda: st["xdone"] >= 10
            k = 0
            for item in range(n1 if m1 else 0):
                for _ in range(m1):
                    assert issued[k] == ("fc1",)
                    yield from issue()
                    k += 1
                yield lambda: st["cons"] >= item
                st["prog"][w] = item + 1
            # the consume side walks the same sequence R slots behind; every entry it
            # reads was taken by the issue side, and is still in the ring
            ch = {"t": first2 + w, "q": 0}
            cur_seq = None
            while True:
                if ch["t"] < zb:
                    t = ch["t"]
                    ch["t"] += 8
                else:
                    q = ch["q"]
                    assert q < st["posted"] and st["queue"][q % RING] == st["history"][q]
                    s = st["history"][q]
                    ch["q"] += 1
                    if s < 0:
                        break
                    t = s + w
                assert k < len(issued) and issued[k] == ("tile", t), "consume side off the issue side"
                g = t // TPE
                seq = g - g0
                if seq != cur_seq:
                    cur_seq = seq
                    st["prog2"][w] = seq
                    yield lambda: st["ready"] >= seq + 1
                done.append((c, t, glast))
                yield from issue()
                k += 1
            st["prog2"][w] = INF

        def finisher():
            ctr[c] = [call, 0, 0]   # re-armed for the call
            if Z == 0:
                post(-1)
            st["xdone"] += 1
            for kk in range(n1):
                for ww in range(min(NS1, 8)):
                    yield lambda: st["prog"][ww] >= kk + 1
                st["cons"] = kk + 1
                flags.add(tuple(items[c + kk * grid]))
            if Z == 0:
                return

            def pace():
                if st["posted"] >= A:
                    need = st["posted"] - A + 1
                    yield lambda: all(v >= need for v in st["taken"])

            while True:
                yield from pace()
                tag, f, r = ctr[c]
                ctr[c][1] += 1
                if tag != call or f + r >= Z:
                    break
                post(zb + f * GR)
            for vc in range(c + 1, min(c + V, grid - 1) + 1):
                vn1, vf, vn2, _, vzb, vZ = (int(v) for v in split[vc])
                if vZ == 0 or vzb // TPE != glast or (vf + vn2 - 1) // TPE != glast:
                    continue
                while True:
                    yield from pace()
                    word = ctr.setdefault(vc, ["old", 0, 0])   # not re-armed yet: an old tag
                    tag, f, r = list(word)
                    word[2] += 1
                    if tag != call or f + r >= vZ:
                        break
                    post(vzb + (vZ - 1 - r) * GR)
            post(-1)

        def loader():
            st["xdone"] += 1
            for seq in range(_nseq(first2, n2, TPE)):
                if seq >= 2:
                    for ww in range(8):
                        yield lambda: st["prog2"][ww] >= seq - 1
                for j in range(HB):
                    yield lambda: (g0 + seq, j) in flags
                st["ready"] = seq + 1

        return [wave(w) for w in range(8)] + [finisher(), loader()]

    gens = []
    for c in rng.permutation(grid):
        gens += wg(int(c))
    return gens, done


def _interleave(gens, rng):
    """Advances the generators in random order, one step at a time, until all are done;
    returns the generators still blocked when nothing can move (none: no deadlock)."""
    live = {i: (g, None) for i, g in enumerate(gens)}
    while live:
        moved = False
        for i in rng.permutation(list(live)):
            g, cond = live[i]
            if cond is not None and not cond():
                continue
            try:
                live[i] = (g, next(g))
            except StopIteration:
                del live[i]
            moved = True
        if not moved:
            return list(live)
    return []


def _claims_runs(m, case, seeds=3):
    """Runs the claims model of one case over `seeds` random interleavings, checking
    every property; returns the tiles computed by thieves."""
    G, D, I, grid = case
    K = _kernel_constants()
    R = 2
    split, items = m.moe_work_split(0, G, D, I, grid, R)
    assert split[:, 5].sum() > 0, "the case has no claimable zone"
    TPE = D // 16
    stolen = 0
    for seed in range(seeds):
        rng = np.random.default_rng(seed)
        gens, done = _claims_model(split, items, D, I, R, K, rng)
        blocked = _interleave(gens, rng)
        assert not blocked, (case, seed, len(blocked))
        tiles = sorted(t for _, t, _ in done)
        assert tiles == list(range(G * TPE)), (case, seed)
        for c, t, glast in done:
            n1, first2, n2 = (int(v) for v in split[c, :3])
            if not first2 <= t < first2 + n2:
                assert t // TPE == glast, (case, seed, c, t)
                stolen += 1
    return stolen


@pytest.mark.parametrize("case", [(13, 1024, 128, 33), (24, 1024, 128, 3), (65, 3584, 384, 61),
                                  (9, 2048, 256, 7), (40, 512, 64, 16)])
def test_claims_protocol_covers_every_tile_once(m, case):
    """FC2 tail claims (experts page, ExpertsKernel steal and claims), modelled over random
    interleavings: no wave waits for good, every FC2 tile is computed exactly once (a
    grain goes to its owner or to one thief, never both), a thief computes only tiles of
    its last group (whose hidden it holds), and no queue entry is read before it is
    posted or after it is overwritten."""
    _claims_runs(m, case)


def test_claims_model_takes_grains_from_victims(m):
    """The model reaches the thieves' path: in this case some interleavings hand zone
    grains to the workgroup before their owner."""
    assert _claims_runs(m, (13, 1024, 128, 33)) > 0
