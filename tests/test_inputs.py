"""The seeded workload generator: shapes and CSR consistency on the host (no GPU).

Every layer of a multi-layer workload must use the workload's one community
stride, and every graph's member lists must hold positions of its own sequence
only (past the sinks, below the context length), without overlapping regions."""
from __future__ import annotations

import numpy as np
import pytest

from sparse_long_context_centroid_amd import inputs as I


@pytest.mark.parametrize("cfg,kw", [
    (4, dict(layers=6, contexts=[8192, 9100, 8400, 8800], steps=2)),
    (2, dict(context=4096, steps=2)),
    (0, dict()),
])
def test_layers_share_stride_and_members_are_own_positions(cfg, kw):
    wl = I.make_workload(cfg, device="cpu", **kw)
    gps = wl.Hkv * wl.gpk
    for L in wl.layers:
        assert L.centroids.shape[1] == wl.Cmax
        for a in (L.comm_start, L.comm_size, L.comm_cap):
            assert a.shape == (wl.NG, wl.Cmax)
        assert (L.num_comms <= wl.Cmax).all()
        spans = []
        for g in range(wl.NG):
            n = int(wl.seq_len0[g // gps])
            C = int(L.num_comms[g])
            st, sz, cap = L.comm_start[g, :C], L.comm_size[g, :C], L.comm_cap[g, :C]
            assert (sz <= cap).all() and (L.comm_size[g, C:] == 0).all()
            pos = np.concatenate([L.members[s:s + k] for s, k in zip(st, sz)]) if C else []
            assert len(pos) == max(n - wl.S, 0)
            assert np.array_equal(np.sort(pos), np.arange(min(wl.S, n), n))
            spans += [(int(s), int(s + c)) for s, c in zip(st, cap)]
        spans.sort()
        assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))


@pytest.mark.parametrize("ps", [None, 1, 4, 256])
def test_logical_kv_gather_matches_the_page_walk(ps):
    """The test-side gather of the paged pools into token order equals a plain walk
    over the page table (unmapped pages stay zero), at the default and other page
    sizes."""
    import helpers as H
    wl = I.make_workload(4, contexts=[700, 1600, 33], steps=2, layers=1, page_size=ps)
    assert wl.page_size == (I.PAGE_SIZE if ps is None else ps)
    assert tuple(wl.layers[0].k_pages.shape[1:]) == (wl.Hkv, wl.page_size, wl.d)
    L = wl.layers[0]
    K, V = H.logical_kv(wl, L)
    pt = wl.page_table.cpu().numpy()
    kp, vp = H.raw_np(L.k_pages), H.raw_np(L.v_pages)
    B, P = pt.shape
    ps = wl.page_size
    K2 = np.zeros((B, wl.Hkv, P * ps, wl.d), kp.dtype)
    V2 = np.zeros_like(K2)
    for b in range(B):
        for p in range(P):
            if pt[b, p] >= 0:
                K2[b, :, p * ps:(p + 1) * ps] = kp[pt[b, p]]
                V2[b, :, p * ps:(p + 1) * ps] = vp[pt[b, p]]
    assert (pt < 0).any()
    assert np.array_equal(K, K2) and np.array_equal(V, V2)


def test_page_size_must_be_a_power_of_two():
    with pytest.raises(ValueError):
        I.make_workload(0, page_size=48)
