"""The fused decode step (ckv_decode_step: the update in extra workgroups of the
attention launch, seq_len advanced by the merge) against the four separate calls of
the C ABI on the same state, over graph granularities, dtypes, head dims, sink
counts, community sizes down to one or two tokens, and a list longer than its
stride:

* identical index lists, lengths, sets, candidates, assignments, error bits and
  updated state (centroids bit for bit, sizes, member pools, seq_len); attention
  outputs equal within float rounding (the two paths run the same attention code in
  two kernel instances);
* a list that runs past its stride is flagged (CKV_DEVERR_INDEX_RANGE) and stops at
  the stride on both paths;
* the workloads of communities of one to three tokens (hundreds of kept communities,
  most of an attention piece's tokens in different communities) against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_parity import run_parity
from sparse_long_context_centroid_amd import binding as Bd
from sparse_long_context_centroid_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bd.load()


def _spec(name, B, Hq, Hkv, d, ctx, budget, *, dtype=I.DT_BF16, head=False, layer=False,
          S=4, M=8, mean=64.0, steps=2):
    return I.ConfigSpec(name, B, Hq, Hkv, d, ctx, head, budget, steps, dtype, num_sinks=S,
                        n_cand=M, shuffled_pages=True, layer_graph=layer, mean_comm_size=mean)


# (spec, contexts, index_stride or None for sinks + budget)
CASES = [
    (_spec("group-bf16-d128", 2, 8, 2, 128, 3000, 300), [3000, 1800], None),
    (_spec("group-bf16-d128-tiny-communities", 2, 8, 2, 128, 6000, 1000, mean=1.5),
     [6000, 2500], None),
    (_spec("perhead-bf16-d128-small-communities", 1, 8, 2, 128, 4000, 600, head=True, mean=3.0),
     [4000], None),
    (_spec("layer-bf16-d64-tiny-communities", 2, 8, 4, 64, 5000, 800, layer=True, mean=2.0),
     [5000, 3100], None),
    (_spec("group-fp32-d64-tiny-communities", 1, 4, 1, 64, 4000, 700, dtype=I.DT_F32, mean=1.5),
     [4000], None),
    (_spec("group-fp32-d128", 2, 8, 2, 128, 2500, 400, dtype=I.DT_F32), [2500, 900], None),
    (_spec("group-bf16-no-sinks", 2, 8, 2, 128, 2000, 250, S=0), [2000, 1500], None),
    (_spec("group-bf16-context-below-sinks", 3, 8, 2, 128, 1000, 200, S=7), [1000, 5, 3], None),
    (_spec("group-bf16-budget-zero", 1, 8, 2, 128, 1500, 0), [1500], None),
    (_spec("group-bf16-list-past-stride", 2, 8, 2, 128, 3000, 600), [3000, 2000], 250),
]


def _state(layer):
    torch.cuda.synchronize()
    return {k: getattr(layer, k).detach().cpu().clone() for k in
            ("scores", "selected", "num_selected", "cand", "index_len", "index_list",
             "assigned", "out", "centroids", "comm_size", "members", "seq_len", "err")}


@pytest.mark.parametrize("spec,contexts,stride", CASES, ids=[c[0].name for c in CASES])
def test_fused_step_matches_four_calls(spec, contexts, stride):
    print(f"\n[case] fused step vs four calls: {spec.name} contexts={contexts} "
          f"stride={stride}", flush=True)
    wl = I.make_workload(spec, 57_000, device="cuda", contexts=contexts)
    if stride is None:
        stride = int(wl.S + int(wl.budget.max()))
    L = wl.layers[0]
    # both layers read the same K/V pools: each step appends row n with the same
    # bytes in both, and attention reads only the rows below n
    four = Bd.decode_layer_from_workload(wl, 0, index_stride=stride)
    fused = Bd.decode_layer_from_workload(wl, 0, index_stride=stride)
    for t in range(wl.steps):
        q, kn, vn = L.q[t].contiguous(), L.k_new[t].contiguous(), L.v_new[t].contiguous()
        four.step(q, kn, vn, wl.scale)
        a = _state(four)
        fused.step_fused(q, kn, vn, wl.scale)
        b = _state(fused)
        for k in a:
            if k == "out":
                continue
            x, y = a[k], b[k]
            if k == "index_list":
                for g in range(x.shape[0]):
                    n = int(a["index_len"][g])
                    assert torch.equal(x[g, :n], y[g, :n]), f"step {t} graph {g}: index lists"
                continue
            if x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), f"step {t}: {k} differs between the two paths"
        d = (a["out"] - b["out"]).abs().max().item()
        assert d <= 1e-5, f"step {t}: outputs differ by {d}"
    if stride < int(wl.S + int(wl.budget.max())):
        # the list ran past its stride: flagged, stopped at the stride
        assert int(a["err"].item()) & Bd.DEVERR_INDEX_RANGE
        assert int(a["index_len"].max().item()) == stride
    else:
        assert int(a["err"].item()) == 0


@pytest.mark.parametrize("spec,contexts", [(c[0], c[1]) for c in CASES[1:5]],
                         ids=[c[0].name for c in CASES[1:5]])
def test_tiny_communities_match_oracle(spec, contexts):
    """Communities of one to three tokens: hundreds of kept communities per list."""
    print(f"\n[case] tiny communities vs oracle: {spec.name} contexts={contexts}", flush=True)
    wl = I.make_workload(spec, 58_000, device="cuda", contexts=contexts)
    run_parity(wl, fused=True)


def test_fused_step_follows_replaced_buffers():
    """step_fused marshals the layer's own buffers once and reuses them while the
    same objects stay in place: after buffers are replaced, the next step writes
    into the new ones (and leaves the old ones as they were), equal to a layer whose
    every step marshals its arguments afresh (the path with timing events)."""
    spec = _spec("group-bf16-d128-rebound", 2, 8, 2, 128, 3000, 300, steps=3)
    print(f"\n[case] fused step after replaced buffers: {spec.name}", flush=True)
    wl = I.make_workload(spec, 57_100, device="cuda", contexts=[3000, 1700])
    L = wl.layers[0]
    cached = Bd.decode_layer_from_workload(wl, 0)
    fresh = Bd.decode_layer_from_workload(wl, 0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for t in range(wl.steps):
        q, kn, vn = L.q[t].contiguous(), L.k_new[t].contiguous(), L.v_new[t].contiguous()
        old = None
        if t > 0:
            old = {k: getattr(cached, k) for k in ("out", "index_list", "cand", "assigned")}
            snap = {k: v.detach().clone() for k, v in old.items()}
            cached.out = torch.full_like(cached.out, float("nan"))
            cached.index_list = torch.full_like(cached.index_list, -7)
            cached.cand = torch.full_like(cached.cand, -7)
            cached.assigned = torch.full_like(cached.assigned, -7)
        cached.step_fused(q, kn, vn, wl.scale)
        fresh.step_fused(q, kn, vn, wl.scale, events=ev)
        a, b = _state(cached), _state(fresh)
        for k in a:
            if k == "out":
                continue
            x, y = a[k], b[k]
            if k == "index_list":
                for g in range(x.shape[0]):
                    n = int(b["index_len"][g])
                    assert torch.equal(x[g, :n], y[g, :n]), f"step {t} graph {g}: index lists"
                continue
            if x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), f"step {t}: {k} differs"
        assert torch.equal(a["out"], b["out"]), f"step {t}: outputs differ"
        if old is not None:
            for k, v in old.items():
                assert torch.equal(v.cpu(), snap[k].cpu()), f"step {t}: the replaced {k} was written"
    assert int(b["err"].item()) == 0


@pytest.mark.parametrize("fused", [True, False], ids=["fused-step", "four-calls"])
def test_step_on_a_side_stream(fused):
    """Every launch of a call goes to the stream it is given: the same steps on a
    second stream (torch's current stream inside the block; default priority) give
    the state and outputs of the default stream bit for bit."""
    spec = _spec("group-bf16-d128-stream", 2, 8, 2, 128, 3000, 300, steps=3)
    print(f"\n[case] side stream: {spec.name} fused={fused}", flush=True)
    wl = I.make_workload(spec, 57_200, device="cuda", contexts=[3000, 2200])
    L = wl.layers[0]
    main = Bd.decode_layer_from_workload(wl, 0)
    side = Bd.decode_layer_from_workload(wl, 0)
    # the two layers own separate K/V pools: each appends its own rows
    side.k, side.v = side.k.clone(), side.v.clone()
    side.kv = Bd.make_kv(side.k, side.v, side.page_table, wl.page_size, side.seq_len)
    s = torch.cuda.Stream()
    for t in range(wl.steps):
        q, kn, vn = L.q[t].contiguous(), L.k_new[t].contiguous(), L.v_new[t].contiguous()
        torch.cuda.synchronize()
        (main.step_fused if fused else main.step)(q, kn, vn, wl.scale)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            (side.step_fused if fused else side.step)(q, kn, vn, wl.scale)
        torch.cuda.synchronize()
        a, b = _state(main), _state(side)
        for k in a:
            x, y = a[k], b[k]
            if k == "index_list":
                for g in range(x.shape[0]):
                    n = int(a["index_len"][g])
                    assert torch.equal(x[g, :n], y[g, :n]), f"step {t} graph {g}: index lists"
                continue
            if x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), f"step {t}: {k} differs between the streams"
    assert int(a["err"].item()) == 0
    assert torch.equal(main.k, side.k) and torch.equal(main.v, side.v)
