"""moe_decode_run_noalloc (the entry point for callers that cannot allocate) against
moe_decode_run on the same inputs: rows, hidden dump and plan bit-identical, and both
within the output bars against the oracle; two calls in a row, the second with a
smaller batch, then the first batch again; the allocation-free call also once with the
FC2 tail claims on (their counters live in the same fixed scratch)."""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_routed_expert_mx_amd as m
    from moe_routed_expert_mx_amd.layer import MoeLayer
    return m, MoeLayer


def _both(m, layer, d, claims=0):
    w = d["workload"]
    x = torch.from_numpy(d["x"]).to(DEV)
    ids = torch.from_numpy(d["ids"]).to(DEV)
    res = []
    for fn in ("workspace", "noalloc"):
        out = layer.out_buffer(w.B)
        hc = torch.zeros(w.B * w.K, w.I, dtype=torch.uint8, device=DEV)
        hs = torch.zeros(w.B * w.K, w.I // 32, dtype=torch.uint8, device=DEV)
        plan = torch.zeros(m.moe_plan_bytes(w.B, w.D), dtype=torch.uint8, device=DEV)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        if fn == "workspace":
            m.moe_decode_run(layer.structs[0], x, ids, layer.ws, out, hidden_codes=hc, hidden_scales=hs, plan=plan,
                             status=status)
        else:
            m.moe_decode_run_noalloc(layer.structs[0], x, ids, out, hidden_codes=hc, hidden_scales=hs, plan=plan,
                                     status=status, fc2_claims=claims)
        torch.cuda.synchronize()
        res.append((out.view(torch.uint16).cpu().numpy(), hc.cpu().numpy(), hs.cpu().numpy(), plan.cpu().numpy(),
                    int(status.item())))
    return res


def test_noalloc_matches_workspace_form(lib):
    from test_gpu_parity import _check_all, _oracle
    m, MoeLayer = lib
    d8 = workloads.generate("decode_b8")
    w = d8["workload"]
    layer = MoeLayer(d8["w13"], d8["s13"], d8["w2"], d8["s2"], B_max=8, topk=w.K, device=DEV)
    d3 = dict(d8)
    d3["x"], d3["ids"] = np.ascontiguousarray(d8["x"][:3]), np.ascontiguousarray(d8["ids"][:3])
    d3["workload"] = workloads.custom("b3", B=3, E=w.E, K=w.K, D=w.D, I=w.I)
    for name, d, claims in (("b8", d8, 0), ("b3", d3, 0), ("b8 again", d8, 0), ("b8 claims", d8, 1)):
        print(f"noalloc vs workspace: {name}", flush=True)
        (a, ahc, ahs, ap, ast), (b, bhc, bhs, bp, bst) = _both(m, layer, d, claims)
        assert ast == 0 and bst == 0
        assert np.array_equal(a, b) and np.array_equal(ahc, bhc) and np.array_equal(ahs, bhs)
        assert np.array_equal(ap, bp)
        _check_all(d, b, bhc, bhs, _oracle(d), what=f"noalloc/{name}")
