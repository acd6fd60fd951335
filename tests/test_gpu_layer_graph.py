"""GPU parity of the whole-layer graph (graphs_per_kv = 0) with the fp64 oracle.

One graph per sequence serves every head of the layer: the score is the max over
all query heads of their own KV head's centroid slice, one index list feeds every
KV head's attention, and the update compares whole centroid rows (Hkv*d values).
The same acceptance as the other graph modes: scores, sets, candidates, lists,
assignments, members, sizes, K/V appends and centroids bit-exact; attention within
max-abs 2e-3 and relative L2 1e-3.
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


def _case(name):
    print(f"\n[case] {name}", flush=True)


def _layer(cfg):
    return I.granularity_spec(I.CONFIGS[cfg] if isinstance(cfg, int) else cfg, "layer")


LAYER_REDUCED = [
    (1, dict(context=8192, steps=4)),
    (3, dict(context=16384, steps=3)),
    (0, dict(steps=1)),
]


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
@pytest.mark.parametrize("cfg,kw", LAYER_REDUCED)
def test_layer_graph_parity_reduced(cfg, kw, fused):
    _case(f"layer graph cfg{cfg} {kw} fused={fused}")
    wl = I.make_workload(_layer(cfg), device="cuda", **kw)
    assert wl.gpk == 0 and wl.NG == wl.B
    run_parity(wl, fused=fused)


_LAYER_SHAPES = [
    I.ConfigSpec("bf16-d64-g8-layer", 2, 16, 2, 64, 3000, False, 300, 3, I.DT_BF16,
                 layer_graph=True),
    I.ConfigSpec("fp32-d128-g2-layer", 1, 8, 4, 128, 2500, False, 256, 3, I.DT_F32,
                 layer_graph=True),
    I.ConfigSpec("bf16-d128-g1-layer", 2, 4, 4, 128, 2000, False, 200, 3, I.DT_BF16,
                 layer_graph=True),
    I.ConfigSpec("bf16-d128-g8-layer", 1, 16, 2, 128, 2300, False, 256, 2, I.DT_BF16,
                 layer_graph=True),
]


@pytest.mark.parametrize("fused", [False, True], ids=["four-calls", "fused-step"])
@pytest.mark.parametrize("spec", _LAYER_SHAPES, ids=[s.name for s in _LAYER_SHAPES])
def test_layer_graph_parity_shapes(spec, fused):
    _case(f"layer shape {spec.name} fused={fused}")
    run_parity(I.make_workload(spec, device="cuda"), fused=fused)


@pytest.mark.parametrize("n_cand", [8, 12], ids=["update-in-attention", "update-in-merge"])
def test_layer_graph_update_host_launch(n_cand):
    """8 KV heads x d 128: with 8 candidates the layer update's staging fits the
    attention launch's update rows and runs there; with 12 it does not, and the
    merge launch runs it (each sequence advancing its own seq_len)."""
    _case(f"layer graph update host, n_cand={n_cand}")
    spec = I.ConfigSpec("layer-host", 3, 32, 8, 128, 3000, False, 300, 3, I.DT_BF16,
                        n_cand=n_cand, layer_graph=True)
    wl = I.make_workload(spec, device="cuda")
    assert wl.M == n_cand and wl.Hkv * wl.d == 1024
    run_parity(wl, fused=True)


def test_layer_graph_ties_and_zero_query():
    _case("layer graph tied centroids, q = 0")
    wl = I.make_workload(_layer(1), device="cuda", context=4096, steps=3)
    cen = wl.layers[0].centroids
    C = int(wl.layers[0].num_comms.min())
    cen[:, 1:C:2] = cen[:, 0:C - 1:2]
    wl.layers[0].q[1].zero_()
    run_parity(wl, fused=True)


def test_layer_graph_full_size_32k():
    _case("layer graph full size 32K")
    wl = I.make_workload(_layer(1), device="cuda", steps=8)
    run_parity(wl, fused=True)


def test_layer_graph_rebuild_and_drift():
    import oracle.ckv_oracle as O
    _case("layer graph rebuild / drift")
    wl = I.make_workload(_layer(1), device="cuda", context=4096, steps=4)
    _, layer, st = run_parity(wl, fused=True, return_state=True)
    reb = layer.rebuild()
    drift = layer.drift(reb).cpu().numpy()
    torch.cuda.synchronize()
    assert int(layer.err.item()) == 0
    rows = torch.empty((layer.NG, layer.Cmax, layer.cdim), dtype=torch.float32, device="cuda")
    Bd.ckv_centroids_to_rows(layer.dims, reb, rows)
    rows = rows.cpu().numpy()
    d = wl.d
    for b in range(layer.NG):
        C = int(st.num_comms[b])
        ref = np.concatenate([O.rebuild(st.K[b, kvh], st.members, st.start[b, :C],
                                        st.size[b, :C]) for kvh in range(wl.Hkv)], axis=1)
        assert ref.shape == (C, wl.Hkv * d)
        assert np.array_equal(rows[b, :C].view(np.uint32), ref.view(np.uint32)), b
        dref = O.drift(st.cent[b, :C], ref, st.size[b, :C])
        assert abs(float(drift[b]) - dref) <= 1e-5 * dref + 1e-12, (b, drift[b], dref)


def test_layer_graph_capacity_overflow_is_flagged():
    _case("layer graph capacity overflow")
    wl = I.make_workload(_layer(1), device="cuda", context=2048, steps=1, slack=0)
    layer = Bd.decode_layer_from_workload(wl, 0)
    L = wl.layers[0]
    layer.step_fused(L.q[0].contiguous(), L.k_new[0].contiguous(), L.v_new[0].contiguous(),
                     wl.scale)
    torch.cuda.synchronize()
    assert int(layer.err.item()) & Bd.DEVERR_CAPACITY
    assert (layer.assigned.cpu().numpy() == -1).all()
    assert (layer.seq_len.cpu().numpy() == wl.seq_len0 + 1).all()
