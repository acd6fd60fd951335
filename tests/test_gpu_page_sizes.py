"""Paged KV caches of other page sizes than the workloads' 16 tokens: one token per
page, a few tokens, 64, 256 and a page of 4096 tokens that holds a whole short
sequence.  Every page table is shuffled, and the decode steps append tokens across
page boundaries.  Through the C ABI against the fp64 oracle: the decode step (fused
and as four calls) in every graph mode, the dense baseline and the centroid rebuild,
which all read K/V rows through the page table."""
from __future__ import annotations

import numpy as np
import pytest
import torch

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


def _spec(name, B, Hq, Hkv, d, ctx, budget, *, dtype=I.DT_BF16, head=False, layer=False,
          steps=3):
    return I.ConfigSpec(name, B, Hq, Hkv, d, ctx, head, budget, steps, dtype,
                        shuffled_pages=True, layer_graph=layer)


MODES = [
    (_spec("group-bf16-d128", 3, 8, 2, 128, 5000, 400), [5000, 1100, 3071]),
    (_spec("perhead-bf16-d128", 2, 8, 2, 128, 3000, 300, head=True), [3000, 1500]),
    (_spec("layer-bf16-d64", 2, 8, 2, 64, 3000, 300, layer=True), [3000, 2049]),
    (_spec("group-fp32-d64", 2, 4, 1, 64, 2500, 250, dtype=I.DT_F32), [2500, 1023]),
]
PAGE_SIZES = [1, 2, 4, 64, 256, 4096]


@pytest.mark.parametrize("ps", PAGE_SIZES)
@pytest.mark.parametrize("spec,contexts", MODES, ids=[m[0].name for m in MODES])
def test_decode_step_with_page_size(spec, contexts, ps):
    print(f"\n[case] page size {ps}: {spec.name} contexts={contexts} fused", flush=True)
    wl = I.make_workload(spec, 61_000 + ps, device="cuda", contexts=contexts, page_size=ps)
    assert wl.page_size == ps
    run_parity(wl, fused=True)


@pytest.mark.parametrize("ps", [1, 64, 4096])
def test_four_calls_with_page_size(ps):
    spec, contexts = MODES[0]
    print(f"\n[case] page size {ps}: {spec.name} contexts={contexts} four calls", flush=True)
    wl = I.make_workload(spec, 62_000 + ps, device="cuda", contexts=contexts, page_size=ps)
    run_parity(wl, fused=False)


@pytest.mark.parametrize("ps", [1, 4, 256, 4096])
def test_dense_baseline_with_page_size(ps):
    """Attention over every cached token, read through a page table of this page
    size, against the oracle's attention over 0..n-1."""
    import oracle.ckv_oracle as O
    spec, contexts = MODES[0]
    print(f"\n[case] page size {ps}: dense baseline {spec.name} contexts={contexts}", flush=True)
    wl = I.make_workload(spec, 63_000 + ps, device="cuda", contexts=contexts, page_size=ps,
                         steps=1)
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
    for b in range(wl.B):
        n = int(wl.seq_len0[b])
        for h in range(wl.Hq):
            ref = O.attend(qn[b, h], K[b, h // G], V[b, h // G], np.arange(n, dtype=np.int32),
                           wl.scale)
            err = np.abs(out[b, h] - ref)
            rel = np.linalg.norm(out[b, h] - ref) / max(np.linalg.norm(ref), 1e-30)
            assert err.max() <= 2e-3 and rel <= 1e-3, (b, h, err.max(), rel)


@pytest.mark.parametrize("ps", [1, 256])
def test_rebuild_with_page_size(ps):
    """After decode steps, the centroids recomputed from the member rows (read
    through the page table) are bit-exact with the oracle's."""
    import oracle.ckv_oracle as O
    spec, contexts = MODES[0]
    print(f"\n[case] page size {ps}: rebuild {spec.name} contexts={contexts}", flush=True)
    wl = I.make_workload(spec, 64_000 + ps, device="cuda", contexts=contexts, page_size=ps)
    _, layer, st = run_parity(wl, fused=True, return_state=True)
    reb = layer.rebuild()
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
