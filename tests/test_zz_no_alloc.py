"""The allocation-free decode step (ckv_decode_step_noalloc) against the decode
step with a caller's workspace (ckv_decode_step): two calls in a row on one GPU,
the second on a smaller workload, every output and every state array identical."""
from __future__ import annotations

import pytest
import torch

from sparse_long_context_centroid_amd import binding as Bd
from sparse_long_context_centroid_amd import inputs as I

pytestmark = pytest.mark.gpu

STATE = ("scores", "selected", "num_selected", "cand", "index_len", "index_list", "assigned",
         "out", "centroids", "comm_size", "members", "seq_len", "err")


def _snap(layer):
    torch.cuda.synchronize()
    return {k: getattr(layer, k).detach().cpu().clone() for k in STATE}


def _same(a, b, what):
    for k in STATE:
        x, y = a[k], b[k]
        if x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"{what}: {k} differs"


@pytest.mark.parametrize("first,second", [
    ((3, dict(steps=2)), (1, dict(context=4096, steps=2))),
    ((2, dict(steps=2)), (0, dict(steps=1))),
])
def test_noalloc_step_matches_workspace_step(first, second):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bd.load()
    for cfg, kw in (first, second):
        print(f"\n[case] noalloc cfg{cfg} {kw}", flush=True)
        wl = I.make_workload(cfg, device="cuda", **kw)
        L = wl.layers[0]
        # separate K/V pools so that each path appends into its own cache
        ref = Bd.decode_layer_from_workload(wl, 0)
        ref.k, ref.v = ref.k.clone(), ref.v.clone()
        ref.kv = Bd.make_kv(ref.k, ref.v, ref.page_table, wl.page_size, ref.seq_len)
        dut = Bd.decode_layer_from_workload(wl, 0)
        for t in range(wl.steps):
            q, kn, vn = L.q[t].contiguous(), L.k_new[t].contiguous(), L.v_new[t].contiguous()
            ref.step_fused(q, kn, vn, wl.scale)
            dut.step_noalloc(q, kn, vn, wl.scale)
            _same(_snap(ref), _snap(dut), f"cfg{cfg} step {t}")
            assert int(dut.err.item()) == 0
        torch.cuda.synchronize()
        assert torch.equal(ref.k, dut.k) and torch.equal(ref.v, dut.v)
        del ref, dut, wl, L
        torch.cuda.empty_cache()
