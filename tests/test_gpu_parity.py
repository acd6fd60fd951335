"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes are chosen so that the oracle finishes in seconds while the kernels still
span several tiles / splits and a ragged tail; the full-size cases run the
configurations' real shapes for a few steps.  Every case prints its name first.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import brute
import helpers as H
from gpu_parity import run_parity
from sparse_long_context_centroid_amd import binding as Bd
from sparse_long_context_centroid_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    Bd.load()


def _case(name):
    print(f"\n[case] {name}", flush=True)


REDUCED = [
    (0, dict()),
    (1, dict(context=8192, steps=4)),
    (2, dict(context=8192, steps=3)),
    (3, dict(context=16384, steps=3)),
    (4, dict(context=16384, steps=2, layers=2, batch=6)),
]


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
@pytest.mark.parametrize("cfg,kw", REDUCED)
def test_parity_reduced(cfg, kw, fused):
    _case(f"cfg{cfg} {kw} fused={fused}")
    wl = I.make_workload(cfg, device="cuda", **kw)
    run_parity(wl, li=len(wl.layers) - 1, fused=fused)


def test_parity_budget_zero_sinks_only():
    _case("budget 0")
    wl = I.make_workload(1, device="cuda", context=2048, steps=2, budget=0)
    s = run_parity(wl)
    assert s["mean_idx_len"] == wl.S


def test_parity_full_budget_equals_dense():
    _case("full budget == dense")
    wl = I.make_workload(1, device="cuda", context=1536, steps=1, budget=1 << 20)
    layer = Bd.decode_layer_from_workload(wl, 0, index_stride=2048)
    L = wl.layers[0]
    K, V = H.logical_kv(wl, L)
    layer.step(L.q[0].contiguous(), L.k_new[0].contiguous(), L.v_new[0].contiguous(), wl.scale)
    torch.cuda.synchronize()
    assert int(layer.err.item()) == 0
    out = layer.out.cpu().numpy()
    q = H.raw_np(L.q[0])
    n = int(wl.seq_len0[0])
    assert (layer.index_len.cpu().numpy() == n).all()
    for h in range(wl.Hq):
        ref = brute.dense_attention(q[0, h], K[0, h // 4], V[0, h // 4], n, wl.scale)
        assert np.max(np.abs(out[0, h] - ref.astype(np.float64))) < 2e-3


def test_parity_single_candidate():
    _case("M = 1")
    wl = I.make_workload(1, device="cuda", context=4096, steps=3, n_cand=1)
    run_parity(wl)


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
def test_parity_exact_score_ties(fused):
    """Duplicated centroids give exactly equal scores; the (score desc, id asc)
    order must be reproduced bit for bit."""
    _case("tied scores")
    wl = I.make_workload(1, device="cuda", context=4096, steps=3)
    cen = wl.layers[0].centroids
    C = int(wl.layers[0].num_comms.min())
    cen[:, 1:C:2] = cen[:, 0:C - 1:2]
    run_parity(wl, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
def test_parity_zero_query(fused):
    _case("q = 0")
    wl = I.make_workload(1, device="cuda", context=4096, steps=2)
    wl.layers[0].q.zero_()
    run_parity(wl, fused=fused)


def test_capacity_overflow_is_flagged():
    _case("capacity overflow")
    wl = I.make_workload(1, device="cuda", context=2048, steps=1, slack=0)
    layer = Bd.decode_layer_from_workload(wl, 0)
    L = wl.layers[0]
    layer.step(L.q[0].contiguous(), L.k_new[0].contiguous(), L.v_new[0].contiguous(), wl.scale)
    torch.cuda.synchronize()
    assert int(layer.err.item()) & Bd.DEVERR_CAPACITY
    assert (layer.assigned.cpu().numpy() == -1).all()
    assert np.array_equal(layer.comm_size.cpu().numpy().reshape(L.comm_size.shape), L.comm_size)
    assert (layer.seq_len.cpu().numpy() == wl.seq_len0 + 1).all()


def test_unmapped_page_is_flagged_and_skipped():
    _case("unmapped page")
    wl = I.make_workload(1, device="cuda", context=2048, steps=1, budget=1 << 20)
    layer = Bd.decode_layer_from_workload(wl, 0, index_stride=2048)
    layer.page_table[0, 5] = -1      # tokens 80..95 become unreachable
    L = wl.layers[0]
    layer.step(L.q[0].contiguous(), L.k_new[0].contiguous(), L.v_new[0].contiguous(), wl.scale)
    torch.cuda.synchronize()
    assert int(layer.err.item()) & Bd.DEVERR_UNMAPPED_PAGE
    K, V = H.logical_kv(wl, L)
    q = H.raw_np(L.q[0])
    keep = np.array([j for j in range(2048) if not 80 <= j < 96])
    out = layer.out.cpu().numpy()
    for h in (0, 13):
        z =(brute.bf16_bits_to_ld(K[0, h // 4][keep]) @ brute.bf16_bits_to_ld(q[0, h])) \
            * brute.LD(np.float32(wl.scale))
        w = np.exp(z - z.max())
        ref = (w[:, None] * brute.bf16_bits_to_ld(V[0, h // 4][keep])).sum(0) / w.sum()
        assert np.max(np.abs(out[0, h] - ref.astype(np.float64))) < 2e-3


def test_out_of_range_entries_are_flagged_and_skipped():
    """Index-list entries outside [0, seq_len) given to the attention call (negative,
    at n, past n, far past the cache) are skipped and flagged; the output is the
    oracle's attention over the list's valid entries, on lists long enough to span
    several attention workgroups, with bad entries at both ends of the lists."""
    import oracle.ckv_oracle as O
    _case("out-of-range index entries")
    wl = I.make_workload(4, device="cuda", contexts=[3000, 1200], steps=1, layers=1)
    stride = 1024
    layer = Bd.decode_layer_from_workload(wl, 0, index_stride=stride)
    rng = np.random.default_rng(11)
    lists, lens, valid = np.zeros((layer.NG, stride), np.int32), np.zeros(layer.NG, np.int32), []
    for g in range(layer.NG):
        n = int(wl.seq_len0[g // wl.Hkv])
        m = 700 + 17 * g
        good = rng.choice(n, m - 6, replace=False).astype(np.int32)
        bad = np.array([-1, n, n + 5, -7, 1 << 30, n + 1000], np.int32)
        lst = np.concatenate([bad[:1], good, bad[1:]])
        lst[[191, 192, 383]] = bad[[1, 2, 3]]          # inside and between pieces
        lists[g, :m] = lst
        lens[g] = m
        valid.append(lst[(lst >= 0) & (lst < n)])
    layer.index_list.copy_(torch.from_numpy(lists))
    layer.index_len.copy_(torch.from_numpy(lens))
    L = wl.layers[0]
    q = L.q[0].contiguous()
    layer.attend(q, wl.scale)
    torch.cuda.synchronize()
    assert int(layer.err.item()) & Bd.DEVERR_INDEX_RANGE
    out = layer.out.cpu().numpy().astype(np.float64)
    K, V = H.logical_kv(wl, L)
    qn = H.raw_np(q)
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        for h in range(wl.Hq):
            g = b * wl.Hkv + h // G
            ref = O.attend(qn[b, h], K[b, h // G], V[b, h // G], valid[g], wl.scale)
            err = np.abs(out[b, h] - ref)
            rel = np.linalg.norm(out[b, h] - ref) / max(np.linalg.norm(ref), 1e-30)
            assert err.max() <= 2e-3 and rel <= 1e-3, (b, h, err.max(), rel)


@pytest.mark.parametrize("cfg,kw", [
    (1, dict(steps=16)),
    (2, dict(steps=8)),
    (3, dict(steps=3)),
])
def test_parity_full_size(cfg, kw):
    """The configurations' real shapes, in the launch configuration the benchmark
    times (the fused decode step)."""
    _case(f"full size cfg{cfg} {kw}")
    wl = I.make_workload(cfg, device="cuda", **kw)
    run_parity(wl, fused=True)


def test_parity_full_size_ragged_paged():
    _case("full size cfg4, 1 of 36 layers")
    wl = I.make_workload(4, device="cuda", steps=2, layers=1)
    run_parity(wl, fused=True)


def test_parity_full_size_ragged_paged_deep_layer():
    """A later layer of a multi-layer workload: every layer shares one community
    stride, whatever its own partition sizes."""
    _case("full size cfg4, layer 7 of 8")
    wl = I.make_workload(4, device="cuda", steps=2, layers=8)
    run_parity(wl, li=7, fused=True)


@pytest.mark.parametrize("cfg,kw,sample", [
    (0, dict(steps=1), None),
    (1, dict(context=6000, steps=1), None),
    (4, dict(contexts=[8192, 3000, 12345, 700], steps=1, layers=1), None),
    (3, dict(steps=1), 12),
    (I.ConfigSpec("bf16-d128-g8-group", 2, 16, 2, 128, 2300, False, 256, 1, I.DT_BF16),
     dict(), None),
])
def test_dense_baseline_matches_oracle(cfg, kw, sample):
    """The dense baseline (every cached token, through the page table) against the
    oracle's attention over the full list 0..n-1; `sample` checks that many
    (sequence, head) pairs of a full-size case."""
    import oracle.ckv_oracle as O
    _case(f"dense cfg{cfg} {kw}")
    wl = I.make_workload(cfg, device="cuda", **kw)
    layer = Bd.decode_layer_from_workload(wl, 0)
    L = wl.layers[0]
    q = L.q[0].contiguous()
    layer.dense(q, wl.scale)
    torch.cuda.synchronize()
    assert int(layer.err.item()) == 0
    out = layer.out.cpu().numpy().astype(np.float64)
    K, V = H.logical_kv(wl, L)
    qn = H.raw_np(q)
    G = wl.Hq // wl.Hkv
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.Hq)]
    if sample:
        rng = np.random.default_rng(5)
        pairs = [pairs[i] for i in rng.choice(len(pairs), sample, replace=False)]
    for b, h in pairs:
        n = int(wl.seq_len0[b])
        ref = O.attend(qn[b, h], K[b, h // G], V[b, h // G], np.arange(n, dtype=np.int32),
                       wl.scale)
        err = np.abs(out[b, h] - ref)
        rel = np.linalg.norm(out[b, h] - ref) / max(np.linalg.norm(ref), 1e-30)
        assert err.max() <= 2e-3 and rel <= 1e-3, (b, h, err.max(), rel)


@pytest.mark.parametrize("cfg,kw", [
    (1, dict(context=4096, steps=4)),
    (4, dict(contexts=[5000, 2100, 8192, 777], steps=3, layers=1)),
    (0, dict(steps=1)),
])
def test_rebuild_and_drift_match_oracle(cfg, kw):
    """After some decode steps (members appended, centroids moved), the centroids
    recomputed from the member lists are bit-exact with the oracle's, and the
    per-graph drift of the running means agrees with the oracle's."""
    import oracle.ckv_oracle as O
    _case(f"rebuild cfg{cfg} {kw}")
    wl = I.make_workload(cfg, device="cuda", **kw)
    _, layer, st = run_parity(wl, fused=True, return_state=True)
    reb = layer.rebuild()
    drift = layer.drift(reb).cpu().numpy()
    torch.cuda.synchronize()
    assert int(layer.err.item()) == 0
    rows = torch.empty((layer.NG, layer.Cmax, layer.d), dtype=torch.float32, device="cuda")
    Bd.ckv_centroids_to_rows(layer.dims, reb, rows)
    rows = rows.cpu().numpy()
    for g in range(layer.NG):
        b = g // (wl.Hkv * wl.gpk)
        kvh = (g // wl.gpk) % wl.Hkv
        C = int(st.num_comms[g])
        ref = O.rebuild(st.K[b, kvh], st.members, st.start[g, :C], st.size[g, :C])
        assert np.array_equal(rows[g, :C].view(np.uint32), ref.view(np.uint32)), g
        dref = O.drift(st.cent[g, :C], ref, st.size[g, :C])
        assert abs(float(drift[g]) - dref) <= 1e-5 * dref + 1e-12, (g, drift[g], dref)


# Shapes beyond the five workloads: every (dtype, head_dim, heads-per-graph)
# combination the library builds, in both graph modes.
_SHAPES = [
    I.ConfigSpec("bf16-d64-g8-group", 2, 16, 2, 64, 3000, False, 300, 3, I.DT_BF16),
    I.ConfigSpec("bf16-d64-g8-perhead", 1, 16, 2, 64, 2000, True, 256, 2, I.DT_BF16),
    I.ConfigSpec("fp32-d128-g2-perhead", 1, 4, 2, 128, 2500, True, 256, 3, I.DT_F32),
    I.ConfigSpec("fp32-d128-g4-group", 2, 8, 2, 128, 2200, False, 200, 2, I.DT_F32),
    I.ConfigSpec("bf16-d128-g1-mha", 2, 4, 4, 128, 2000, False, 200, 3, I.DT_BF16),
    I.ConfigSpec("fp32-d64-g1-mha", 1, 2, 2, 64, 1500, False, 128, 2, I.DT_F32),
    I.ConfigSpec("bf16-d128-g2-group", 3, 8, 4, 128, 1800, False, 160, 2, I.DT_BF16),
    I.ConfigSpec("fp32-d64-g8-group", 1, 8, 1, 64, 2600, False, 256, 2, I.DT_F32),
    # 8 heads x d 128 = 1024 outputs per graph: more than the merge's 512 threads
    I.ConfigSpec("bf16-d128-g8-group", 2, 16, 2, 128, 2300, False, 256, 2, I.DT_BF16),
]


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
@pytest.mark.parametrize("spec", _SHAPES, ids=[s.name for s in _SHAPES])
def test_parity_shapes(spec, fused):
    _case(f"shape {spec.name} fused={fused}")
    wl = I.make_workload(spec, device="cuda")
    run_parity(wl, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
def test_parity_contexts_shorter_than_sinks(fused):
    """Sequences of 3, 4 and 5 tokens (no communities, or only sinks) next to a
    normal one: sinks only, no candidates, the token still appended."""
    _case("short contexts")
    wl = I.make_workload(1, device="cuda", contexts=[3, 4, 5, 700], steps=2)
    run_parity(wl, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
def test_parity_all_sinks_null_member_pool(fused):
    """Every sequence holds sinks only: no community exists, the member pool is
    empty and reaches the library as a null pointer; the lists are the sinks and
    the new token is still appended."""
    _case("all sinks, null member pool")
    wl = I.make_workload(1, device="cuda", contexts=[3, 4, 2], steps=2)
    assert wl.layers[0].members.size == 0
    layer = Bd.decode_layer_from_workload(wl, 0)
    assert layer.graphs.members is None
    run_parity(wl, fused=fused)


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
def test_parity_empty_communities(fused):
    """Communities of size 0 (members never listed) score -inf and are never kept
    or candidates."""
    _case("empty communities")
    wl = I.make_workload(1, device="cuda", context=4096, steps=3)
    L = wl.layers[0]
    L.comm_size[:, 1:40:3] = 0
    run_parity(wl, fused=fused)


def test_parity_maximum_sizes():
    """A long sequence (250K tokens: ~3900 communities, four per select thread),
    the largest candidate count (16) and a 16K budget (86 attention splits per
    graph, past one merge load round)."""
    _case("maximum sizes")
    spec = I.ConfigSpec("max-sizes", 1, 4, 1, 128, 250000, False, 16384, 2, I.DT_BF16,
                        n_cand=16)
    wl = I.make_workload(spec, device="cuda")
    assert wl.Cmax > 3584 and wl.Cmax <= 4096
    run_parity(wl, fused=True)
    run_parity(I.make_workload(spec, device="cuda"), fused=False)


def test_parity_community_cap():
    """Near the community cap (8192 per graph): 128K tokens over ~8100 communities,
    a mean community size of 16, eight communities per select thread."""
    _case("community cap")
    spec = I.ConfigSpec("comm-cap", 1, 8, 2, 128, 131072, False, 4096, 2, I.DT_BF16,
                        markov_labels=8100)
    wl = I.make_workload(spec, device="cuda")
    assert 7168 < wl.Cmax <= 8192
    run_parity(wl, fused=True)
    run_parity(I.make_workload(spec, device="cuda"), fused=False)


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
def test_parity_persistent_attention_grid(fused):
    """A list grid larger than one round of resident workgroups (64 group graphs x
    22 splits) runs as the persistent attention grid; ragged contexts leave many
    split slots empty."""
    _case(f"persistent attention grid fused={fused}")
    spec = I.ConfigSpec("persist-grid", 8, 32, 8, 128, 32768, False, 4096, 2, I.DT_BF16)
    wl = I.make_workload(spec, device="cuda",
                         contexts=[32768, 5000, 20000, 9000, 32768, 3000, 12000, 26000])
    assert wl.NG * ((wl.S + int(wl.budget.max()) + 191) // 192) > 1024
    run_parity(wl, fused=fused)


def test_parity_persistent_grid_at_its_graph_limit():
    """The persistent attention grid at its largest graph count (1024 group graphs:
    128 sequences x 8 KV heads, every thread of the prologue holding 4 graphs), with
    one- and two-split lists."""
    _case("persistent grid, 1024 graphs")
    spec = I.ConfigSpec("persist-1024", 128, 32, 8, 128, 600, False, 200, 2, I.DT_BF16)
    rng = np.random.default_rng(5)
    wl = I.make_workload(spec, device="cuda", contexts=[int(x) for x in rng.integers(150, 600, 128)])
    assert wl.NG == 1024
    run_parity(wl, fused=True)


@pytest.mark.parametrize("per_head", [False, True], ids=["group", "per-head"])
def test_parity_past_the_persistent_graph_limit(per_head):
    """More graphs than the persistent attention grid takes (1280 > 1024) with a
    list grid of several rounds: the launcher falls back to the direct grid, whose
    empty split slots still mark their partials; group graphs of 160 ragged
    sequences, or per-head graphs of 40."""
    B = 40 if per_head else 160
    _case(f"past the persistent graph limit, per_head={per_head}")
    spec = I.ConfigSpec("many-graphs", B, 32, 8, 128, 2000, per_head, 400, 2, I.DT_BF16)
    rng = np.random.default_rng(6)
    wl = I.make_workload(spec, device="cuda", contexts=[int(x) for x in rng.integers(120, 2000, B)])
    assert wl.NG == 1280
    run_parity(wl, fused=True)


def test_parity_persistent_grid_with_every_list_empty():
    """No sinks and a zero budget: every list is empty, the persistent grid has no
    busy split (its workers only mark the empty slots) and every output is 0."""
    _case("persistent grid, empty lists")
    spec = I.ConfigSpec("persist-empty", 8, 32, 8, 128, 4096, False, 0, 2, I.DT_BF16,
                        num_sinks=0)
    wl = I.make_workload(spec, device="cuda")
    s = run_parity(wl, fused=True, index_stride=4096)
    assert s["mean_idx_len"] == 0
