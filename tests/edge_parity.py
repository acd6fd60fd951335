"""Parity of the prefill edge kernel (ckv_prefill_edges) with the fp64 oracle.

The kernel forms q.k on the matrix cores (bf16 products are exact, the d-term sum
is fp32); the oracle sums in fp64.  For a query row the fp32 sum of d exact
products differs from the exact one by at most gamma_d * sum_e |q_e k_e|
(gamma_d = d u / (1 - d u), u = 2^-24), whatever the order; the group max and the
positive scale keep that bound, so scores may differ by at most

    tol_i = gamma_d * scale * max_{h, j < i} sum_e |q_h[i]_e k[j]_e|  (+ one fp32 ulp).

Ranks are compared in order: a rank where the two lists hold different keys is
accepted only if the oracle's score of the kernel's key lies within 2 tol_i of
the oracle's score at that rank (a near-tie, where the kernel may legally choose
the other key).  Everything else -- counts, padding, positions -- must match
exactly.  The co-attention pairs must equal the oracle's pairs
(ckvo_coattention_pairs) of the oracle's own edge list, or, on a row where a
near-tie changed the list, the oracle's pairs of the kernel's list.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import ckv_oracle as O
from sparse_long_context_centroid_amd import binding as Bd
from sparse_long_context_centroid_amd import inputs as I


def run_edges(pf: I.Prefill, Hq: int, Hkv: int, gpk: int, topk: int, pairs: bool = True,
              events=None):
    """Launch the kernel; return (idx, score, pairs) as host arrays [NG, n, ...]."""
    B, n, _, d = pf.q.shape
    dims = Bd.ckv_dims(B, Hq, Hkv, d, gpk, 64, pf.S, I.DT_BF16)
    NG = B * Hkv * gpk
    dev = pf.q.device
    idx = torch.full((NG, n, topk), -7, dtype=torch.int32, device=dev)
    sc = torch.full((NG, n, topk), 7.0, dtype=torch.float32, device=dev)
    npair = topk * (topk - 1) // 2
    pr = torch.full((NG, n, max(npair, 1), 2), -7, dtype=torch.int32, device=dev) if pairs else None
    Bd.ckv_prefill_edges(dims, pf.q, pf.k, n, topk, pf.scale, idx, sc, pr if npair else None,
                         events=events)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), sc.cpu().numpy(),
            pr.cpu().numpy()[:, :, :npair] if (pairs and npair) else None)


def graph_qk(q_bits: np.ndarray, k_bits: np.ndarray, g: int, Hkv: int, gpk: int, G: int):
    """Oracle operands of graph g: Q [n, heads, d] and K [n, d] as bf16 bits."""
    per_seq = Hkv * gpk
    b, gs = divmod(g, per_seq)
    kvh = gs // gpk
    h0, hpg = (kvh * G, G) if gpk == 1 else (gs, 1)
    Q = np.ascontiguousarray(q_bits[b, :, h0:h0 + hpg, :])
    K = np.ascontiguousarray(k_bits[b, :, kvh, :])
    return Q, K


def bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_tolerance(Q: np.ndarray, K: np.ndarray, S: int, scale: float, rows) -> np.ndarray:
    """tol_i of the module docstring for each query row."""
    n, G, d = Q.shape
    u = 2.0 ** -24
    gamma = d * u / (1 - d * u)
    Qa = np.abs(bf16_to_f64(Q))
    Ka = np.abs(bf16_to_f64(K))
    out = np.zeros(len(rows))
    for r, i in enumerate(rows):
        if i - S <= 0:
            continue
        m = (Qa[i] @ Ka[S:i].T).max()
        out[r] = gamma * abs(scale) * m
    return out


def check_graph(idx_g, sc_g, pr_g, Q, K, S, scale, topk, rows, label=""):
    """Compare one graph's kernel rows with the oracle; returns the near-tie count."""
    rows = np.asarray(rows, np.int32)
    idx_o, sc_o = O.edges(Q, K, S, scale, topk, rows)
    pr_o = O.coattention_pairs(idx_o, topk) if pr_g is not None else None
    tol = row_tolerance(Q, K, S, scale, rows)
    near = 0
    for r, i in enumerate(rows):
        gi, gs_, oi, os_ = idx_g[i], sc_g[i], idx_o[r], sc_o[r]
        nv = min(topk, max(int(i) - S, 0))
        where = f"{label} row {i}"
        assert (oi[:nv] >= 0).all() and (oi[nv:] == -1).all(), where
        assert (gi[:nv] >= 0).all(), (where, gi)
        assert (gi[nv:] == -1).all() and np.isneginf(gs_[nv:]).all(), (where, gi, gs_)
        assert len(set(gi[:nv].tolist())) == nv, (where, gi)
        assert ((gi[:nv] >= S) & (gi[:nv] < i)).all(), (where, gi)
        t = tol[r] + 2 * np.spacing(np.float32(np.abs(os_[:nv]).max(initial=0.0)))
        assert (np.abs(gs_[:nv].astype(np.float64) - os_[:nv]) <= t).all(), \
            (where, gs_[:nv], os_[:nv], t)
        # the kernel's own order: score desc, position asc on equal scores
        for x in range(nv - 1):
            assert gs_[x] > gs_[x + 1] or (gs_[x] == gs_[x + 1] and gi[x] < gi[x + 1]), \
                (where, gi, gs_)
        diff = np.nonzero(gi[:nv] != oi[:nv])[0]
        if len(diff):
            near += 1
            zg = O.edge_scores(Q, K, scale, np.full(len(diff), i, np.int32),
                               gi[diff].astype(np.int32))
            assert (np.abs(zg - os_[diff].astype(np.float64)) <= 2 * t + 1e-30).all(), \
                (where, "not a near-tie", gi, oi, zg, os_[diff], t)
        if pr_g is not None:
            # the oracle's pairs of the oracle's own list; where a near-tie put a
            # different key in the kernel's list, the oracle's pairs of that list
            want = pr_o[r] if not len(diff) else O.coattention_pairs(gi[None], topk)[0]
            assert np.array_equal(pr_g[i], want), (where, pr_g[i], want)
    return near
