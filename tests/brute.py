"""A second, tiny, independent reference used only to pin the oracle.

Everything here is written from the definitions in a different form from the
oracle's: scores from member-by-member logits instead of centroids, selection by
enumerating every subset of communities, attention as a dense masked softmax, the
centroid invariant as a direct mean.  Arithmetic is numpy longdouble or exact
Python integers/fractions; it is meant for inputs of a few dozen tokens.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

LD = np.longdouble


def bf16_bits_to_ld(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(LD)
    return a.astype(LD)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (finite inputs)."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def order_key(score: float, cid: int):
    return (-float(score), cid)


def select_by_subsets(score, size, budget):
    """Largest set X of non-empty communities with (a) sum of sizes <= budget and
    (b) X closed upward in the order (score desc, id asc): nothing outside X comes
    before anything inside X.  Found by enumerating all subsets."""
    C = len(score)
    ids = [c for c in range(C) if size[c] > 0]
    best = ()
    for r in range(len(ids) + 1):
        for X in itertools.combinations(ids, r):
            if sum(int(size[c]) for c in X) > budget:
                continue
            inside = set(X)
            ok = all(order_key(score[c], c) < order_key(score[o], o)
                     for c in X for o in ids if o not in inside)
            if ok and len(X) > len(best):
                best = X
    return set(best)


def dense_attention(q, K, V, n, scale):
    """Softmax attention of one query over rows 0..n-1, longdouble, masked form."""
    q = bf16_bits_to_ld(q)
    K = bf16_bits_to_ld(K)[:n]
    V = bf16_bits_to_ld(V)[:n]
    z = (K @ q) * LD(np.float32(scale))
    w = np.exp(z - z.max())
    return (w[:, None] * V).sum(0) / w.sum()


def attention_over(q, K, V, idx, scale):
    q = bf16_bits_to_ld(q)
    Kr = bf16_bits_to_ld(K)[np.asarray(idx)]
    Vr = bf16_bits_to_ld(V)[np.asarray(idx)]
    z = np.array([sum(q[i] * Kr[t, i] for i in range(len(q))) for t in range(len(idx))],
                 dtype=LD) * LD(np.float32(scale))
    w = np.exp(z - z.max())
    return np.array([sum(w[t] * Vr[t, i] for t in range(len(idx))) for i in range(len(q))],
                    dtype=LD) / w.sum()


def mean_member_logit(q_rows, K, members, scale):
    """Score of a community computed from its members: max over heads of the mean
    logit (q_h . K_j) over the members j, as an exact Fraction when the inputs are
    exactly representable."""
    best = None
    for qh in q_rows:
        tot = Fraction(0)
        for j in members:
            tot += sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qh, K[j]))
        m = tot / len(members)
        best = m if best is None or m > best else best
    return best * Fraction(float(scale))


def sq_dist(a, b):
    a = bf16_bits_to_ld(a)
    b = np.asarray(b).astype(LD)
    return ((a - b) ** 2).sum()
