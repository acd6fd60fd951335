"""GPU parity of the prefill edge kernel (ckv_prefill_edges) with the fp64 oracle.

Small cases compare every query row (several 64-query workgroups, key tiles and a
ragged tail) for every built (head_dim, heads per graph) combination and both
graph modes; the full-size cases run the Qwen3-8B-shaped prefill of one layer at
32K and 128K positions and compare sampled rows.  Ties are exact when keys repeat:
then the lists must equal the oracle's bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import edge_parity as E
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


def _check_all(pf, Hq, Hkv, gpk, topk, rows=None, graphs=None, label=""):
    idx, sc, pr = E.run_edges(pf, Hq, Hkv, gpk, topk)
    qb, kb = E.bits(pf.q), E.bits(pf.k)
    B, n = pf.q.shape[:2]
    G = Hq // Hkv
    NG = B * Hkv * gpk
    rows = np.arange(n) if rows is None else np.asarray(rows)
    near = 0
    for g in (range(NG) if graphs is None else graphs):
        Q, K = E.graph_qk(qb, kb, g, Hkv, gpk, G)
        near += E.check_graph(idx[g], sc[g], None if pr is None else pr[g], Q, K, pf.S,
                              pf.scale, topk, rows, f"{label} graph {g}")
    print(f"[edges] {label}: rows with near-ties {near}", flush=True)
    return idx, sc


# (head_dim, Hq, Hkv, gpk): every heads-per-graph the kernel is built for
_SHAPES = [(128, 8, 2, 1), (128, 8, 4, 1), (128, 4, 4, 1), (128, 8, 1, 1), (128, 8, 2, 4),
           (64, 8, 2, 1), (64, 8, 4, 1), (64, 4, 4, 1), (64, 8, 1, 1), (64, 8, 1, 8)]


@pytest.mark.parametrize("d,Hq,Hkv,gpk", _SHAPES)
def test_edges_small(d, Hq, Hkv, gpk):
    _case(f"edges small d={d} Hq={Hq} Hkv={Hkv} gpk={gpk}")
    pf = I.make_prefill(11 + d + Hq + Hkv + gpk, B=1, n=333, Hq=Hq, Hkv=Hkv, d=d, S=4,
                        device="cuda", mean_size=16)
    _check_all(pf, Hq, Hkv, gpk, 8, label=f"d{d} G{Hq // Hkv} gpk{gpk}")


@pytest.mark.parametrize("topk", [1, 2, 5, 8])
def test_edges_topk_and_batch(topk):
    _case(f"edges topk={topk} batch=2")
    pf = I.make_prefill(40 + topk, B=2, n=200, Hq=8, Hkv=2, d=128, S=4, device="cuda",
                        mean_size=16)
    _check_all(pf, 8, 2, 1, topk, label=f"topk{topk}")


@pytest.mark.parametrize("n,S", [(1, 4), (3, 4), (5, 4), (9, 4), (64, 0), (65, 0), (130, 70)])
def test_edges_short_and_sink_heavy(n, S):
    _case(f"edges n={n} S={S}")
    pf = I.make_prefill(50 + n + S, B=1, n=n, Hq=8, Hkv=2, d=128, S=S, device="cuda",
                        mean_size=8)
    _check_all(pf, 8, 2, 1, 8, label=f"n{n} S{S}")


def test_edges_exact_ties_resolve_by_position():
    """Keys drawn from 5 distinct rows: equal scores are exactly equal on both sides,
    and the lists must match the oracle's (lowest position first) bit for bit."""
    _case("edges exact ties")
    pf = I.make_prefill(60, B=1, n=300, Hq=8, Hkv=2, d=128, S=4, device="cuda")
    pat = pf.k[:, :5].clone()
    rep = torch.arange(300, device="cuda") % 5
    pf.k[:] = pat[:, rep]
    idx, sc, pr = E.run_edges(pf, 8, 2, 1, 8)
    qb, kb = E.bits(pf.q), E.bits(pf.k)
    from oracle import ckv_oracle as O
    for g in range(2):
        Q, K = E.graph_qk(qb, kb, g, 2, 1, 4)
        oi, os_ = O.edges(Q, K, pf.S, pf.scale, 8)
        assert np.array_equal(idx[g], oi), g
        assert np.array_equal(pr[g], O.coattention_pairs(oi, 8)), g


def test_edges_zero_queries_take_the_earliest_keys():
    _case("edges zero queries")
    pf = I.make_prefill(61, B=1, n=150, Hq=8, Hkv=2, d=128, S=4, device="cuda")
    pf.q.zero_()
    idx, sc, _ = E.run_edges(pf, 8, 2, 1, 8)
    for i in range(150):
        k = min(8, max(i - 4, 0))
        assert list(idx[0, i, :k]) == list(range(4, 4 + k)), i
        assert (sc[0, i, :k] == 0).all()


def test_edges_without_pairs_and_argument_errors():
    _case("edges no pairs / errors")
    pf = I.make_prefill(62, B=1, n=100, Hq=8, Hkv=2, d=128, S=4, device="cuda")
    idx, sc, pr = E.run_edges(pf, 8, 2, 1, 8, pairs=False)
    assert pr is None
    idx2, sc2, _ = E.run_edges(pf, 8, 2, 1, 8)
    assert np.array_equal(idx, idx2) and np.array_equal(sc, sc2)
    dims = Bd.ckv_dims(1, 8, 2, 128, 1, 64, 4, I.DT_BF16)
    o_i = torch.empty((2, 100, 9), dtype=torch.int32, device="cuda")
    o_s = torch.empty((2, 100, 9), dtype=torch.float32, device="cuda")
    with pytest.raises(Bd.CkvError):
        Bd.ckv_prefill_edges(dims, pf.q, pf.k, 100, 9, pf.scale, o_i, o_s)
    with pytest.raises(Bd.CkvError):
        Bd.ckv_prefill_edges(dims, pf.q, pf.k, 0, 8, pf.scale, o_i, o_s)
    f32 = Bd.ckv_dims(1, 8, 2, 128, 1, 64, 4, I.DT_F32)
    with pytest.raises(Bd.CkvError):
        Bd.ckv_prefill_edges(f32, pf.q, pf.k, 100, 8, pf.scale, o_i, o_s)


def _sample_rows(n, S, seed):
    r = np.random.default_rng(seed)
    fixed = [0, S - 1, S, S + 1, S + 8, 63, 64, 65, 127, 128, n // 2, n - 65, n - 64, n - 2, n - 1]
    return np.unique(np.concatenate([[x for x in fixed if 0 <= x < n],
                                     r.integers(0, n, size=9)]))


@pytest.mark.parametrize("gpk", [1, 4])
def test_edges_full_32k(gpk):
    """Qwen3-8B-shaped layer (32 query / 8 KV heads, d 128) over a 32K prefill."""
    _case(f"edges full n=32768 gpk={gpk}")
    n = 32768
    pf = I.make_prefill(70 + gpk, B=1, n=n, Hq=32, Hkv=8, d=128, S=4, device="cuda")
    graphs = [0, 5] if gpk == 1 else [0, 13, 31]
    _check_all(pf, 32, 8, gpk, 8, rows=_sample_rows(n, 4, 3), graphs=graphs,
               label=f"32K gpk{gpk}")


def test_edges_full_128k():
    _case("edges full n=131072 gpk=1")
    n = 131072
    pf = I.make_prefill(72, B=1, n=n, Hq=32, Hkv=8, d=128, S=4, device="cuda")
    _check_all(pf, 32, 8, 1, 8, rows=_sample_rows(n, 4, 4)[::2], graphs=[3],
               label="128K gpk1")
