"""Python driver for the fp64 CPU oracle (ckv_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark may use it; the product path never imports it.  It shares no
code with the HIP library and does not import it.

The C file implements one graph's score, selection, index list, attention and
local update in fp64.  This driver holds the host state of a whole decode layer
(centroids, CSR member lists, the logical K/V cache, sequence lengths) and runs
the per-graph functions for every graph of a decode step, the graphs spread over
a thread pool (ctypes releases the GIL during each C call).

Graph numbering follows the GQA layout: graph g = (b*Hkv + kvh)*gpk + j, where
gpk = 1 (one graph per query group: heads kvh*G .. kvh*G+G-1 share it) or
gpk = G (one graph per query head, j = head index inside the group), or gpk = 0:
one graph per layer (graph g = sequence b), shared by every head of the layer
(rit.work post "CommunityKV long-context decoding", sections on how many graphs a
model keeps and where to start: the group graph, the per-head graph, and the
whole layer in one graph, which the post reports as the least accurate).

Readings for the layer graph: a community holds one centroid per KV head (the
mean of its members' keys in that head), stored as one row of Hkv*d values,
KV head after KV head; its score is the max over all query heads of
q_h . mu_{c, kv head of h} * scale (the group reading, over the whole layer);
one index list serves every KV head; the new token joins the nearest candidate
in squared L2 over the whole row (all KV heads' keys), one fp64 sum over the
row in element order (ckvo_update_layer).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ckv_oracle.c")
LIB = os.path.join(HERE, "libckv_oracle.so")
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

DT_F32 = 0
DT_BF16 = 1

_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no contraction of multiply-adds)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            path = os.environ.get("CKV_ORACLE_LIB")   # a planted-mistake build, in tests
            if path is None:
                path = LIB
                if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
                    build()
            L = C.CDLL(path)
            P = C.c_void_p
            i32 = C.c_int
            L.ckvo_score.argtypes = [i32, i32, P, i32, P, P, i32, C.c_float, P]
            L.ckvo_score.restype = None
            L.ckvo_select.argtypes = [i32, P, P, i32, i32, P, P, C.POINTER(C.c_int)]
            L.ckvo_select.restype = i32
            L.ckvo_index_list.argtypes = [i32, i32, i32, P, P, P, P, P]
            L.ckvo_index_list.restype = i32
            L.ckvo_attend.argtypes = [i32, P, i32, P, P, i32, C.c_long, P, i32, C.c_float, P]
            L.ckvo_attend.restype = None
            L.ckvo_update.argtypes = [i32, P, i32, P, i32, P, P, P, P, P, i32,
                                      C.POINTER(C.c_long)]
            L.ckvo_update.restype = i32
            L.ckvo_rebuild.argtypes = [i32, P, i32, P, P, P, i32, P]
            L.ckvo_rebuild.restype = None
            L.ckvo_drift.argtypes = [i32, P, P, P, i32]
            L.ckvo_drift.restype = C.c_double
            L.ckvo_edges.argtypes = [i32, i32, P, P, i32, i32, C.c_float, i32, P, i32, P, P]
            L.ckvo_edges.restype = None
            L.ckvo_edge_scores.argtypes = [i32, i32, P, P, i32, C.c_float, P, P, i32, P]
            L.ckvo_edge_scores.restype = None
            L.ckvo_update_layer.argtypes = [i32, i32, P, i32, P, i32, P, P, P, P, P, i32]
            L.ckvo_update_layer.restype = i32
            L.ckvo_coattention_pairs.argtypes = [i32, P, i32, P]
            L.ckvo_coattention_pairs.restype = None
            _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    raise TypeError(f"oracle inputs are bf16 bits (uint16) or float32, got {a.dtype}")


# ---- single-graph wrappers (numpy in, numpy out) ---------------------------------

def score(q: np.ndarray, cent: np.ndarray, size: np.ndarray, scale: float) -> np.ndarray:
    """q [G, d] (uint16 bf16 bits or float32), cent [C, d] fp32, size [C] -> fp32 [C]."""
    q = np.ascontiguousarray(q)
    cent = np.ascontiguousarray(cent, np.float32)
    size = np.ascontiguousarray(size, np.int32)
    G, d = q.shape
    Cn = cent.shape[0]
    out = np.empty(Cn, np.float32)
    lib().ckvo_score(d, G, _p(q), _dt(q), _p(cent), _p(size), Cn, scale, _p(out))
    return out


def select(score: np.ndarray, size: np.ndarray, budget: int, M: int):
    """-> (sel u8 [C], k*, cand int32 [<=M])."""
    score = np.ascontiguousarray(score, np.float32)
    size = np.ascontiguousarray(size, np.int32)
    Cn = score.shape[0]
    sel = np.zeros(max(Cn, 1), np.uint8)
    cand = np.full(max(M, 1), -1, np.int32)
    nc = C.c_int(0)
    k = lib().ckvo_select(Cn, _p(score), _p(size), int(budget), int(M), _p(sel), _p(cand),
                          C.byref(nc))
    return sel[:Cn], k, cand[:nc.value]


def index_list(n: int, S: int, sel: np.ndarray, start: np.ndarray, size: np.ndarray,
               members: np.ndarray, max_len: int) -> np.ndarray:
    sel = np.ascontiguousarray(sel, np.uint8)
    start = np.ascontiguousarray(start, np.int32)
    size = np.ascontiguousarray(size, np.int32)
    members = np.ascontiguousarray(members, np.int32)
    idx = np.empty(max(max_len, 1), np.int32)
    ln = lib().ckvo_index_list(int(n), int(S), sel.shape[0], _p(sel), _p(start), _p(size),
                               _p(members), _p(idx))
    assert ln <= max_len
    return idx[:ln].copy()


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray, scale: float):
    """q [d]; K, V [rows, d] (same dtype); idx [len] -> fp64 [d]."""
    q = np.ascontiguousarray(q)
    K = np.ascontiguousarray(K)
    V = np.ascontiguousarray(V)
    idx = np.ascontiguousarray(idx, np.int32)
    d = q.shape[0]
    out = np.empty(d, np.float64)
    lib().ckvo_attend(d, _p(q), _dt(q), _p(K), _p(V), _dt(K), K.shape[1], _p(idx),
                      idx.shape[0], scale, _p(out))
    return out


def update(k_new: np.ndarray, cand: np.ndarray, cent: np.ndarray, size: np.ndarray,
           cap: np.ndarray, start: np.ndarray, members: np.ndarray, n: int):
    """In-place update of cent/size/members.  -> (chosen id or <0, multiply-adds)."""
    for a in (cent, size, members):
        assert a.flags["C_CONTIGUOUS"] and a.flags["WRITEABLE"]
    cand = np.ascontiguousarray(cand, np.int32)
    cap = np.ascontiguousarray(cap, np.int32)
    start = np.ascontiguousarray(start, np.int32)
    k_new = np.ascontiguousarray(k_new)
    ops = C.c_long(0)
    r = lib().ckvo_update(cent.shape[1], _p(k_new), _dt(k_new), _p(cand), cand.shape[0],
                          _p(cent), _p(size), _p(cap), _p(start), _p(members), int(n),
                          C.byref(ops))
    return r, ops.value


# ---- a whole decode layer -----------------------------------------------------------

ERR_CAPACITY = 1


def rebuild(K: np.ndarray, members: np.ndarray, start: np.ndarray, size: np.ndarray):
    """K [rows, d] (bf16 bits or fp32); CSR of C communities -> fp32 [C, d]."""
    K = np.ascontiguousarray(K)
    members = np.ascontiguousarray(members, np.int32)
    start = np.ascontiguousarray(start, np.int32)
    size = np.ascontiguousarray(size, np.int32)
    C, d = size.shape[0], K.shape[1]
    out = np.zeros((C, d), np.float32)
    lib().ckvo_rebuild(d, _p(K), _dt(K), _p(members), _p(start), _p(size), C, _p(out))
    return out


def drift(cent: np.ndarray, ref: np.ndarray, size: np.ndarray) -> float:
    """Largest relative L2 distance of cent from ref over non-empty communities."""
    cent = np.ascontiguousarray(cent, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    size = np.ascontiguousarray(size, np.int32)
    return float(lib().ckvo_drift(cent.shape[1], _p(cent), _p(ref), _p(size), size.shape[0]))


def edges(Q: np.ndarray, K: np.ndarray, S: int, scale: float, topk: int, rows=None):
    """Q [n, G, d], K [n, d] (bf16 bits or fp32) of one KV head -> (idx, score)
    [len(rows), topk]: each query position's strongest earlier non-sink keys."""
    Q = np.ascontiguousarray(Q)
    K = np.ascontiguousarray(K)
    n, G, d = Q.shape
    rows = np.arange(n, dtype=np.int32) if rows is None else np.ascontiguousarray(rows, np.int32)
    idx = np.empty((len(rows), topk), np.int32)
    score = np.empty((len(rows), topk), np.float32)
    lib().ckvo_edges(d, G, _p(Q), _p(K), _dt(K), int(S), scale, int(topk), _p(rows), len(rows),
                     _p(idx), _p(score))
    return idx, score


def coattention_pairs(idx: np.ndarray, topk: int) -> np.ndarray:
    """idx [rows, topk] direct-edge key positions (-1 padded) -> co-attention pairs
    [rows, topk*(topk-1)/2, 2]: every pair of a row's keys, (lower, higher)."""
    idx = np.ascontiguousarray(idx, np.int32).reshape(-1, topk)
    npair = topk * (topk - 1) // 2
    out = np.empty((idx.shape[0], npair, 2), np.int32)
    if npair and idx.shape[0]:
        lib().ckvo_coattention_pairs(int(topk), _p(idx), idx.shape[0], _p(out))
    return out


def update_layer(k_new: np.ndarray, cand: np.ndarray, cent: np.ndarray, size: np.ndarray,
                 cap: np.ndarray, start: np.ndarray, members: np.ndarray, n: int, nseg: int):
    """The layer graph's update: rows of nseg slices (one per KV head); in place
    like update().  -> chosen id or <0."""
    for a in (cent, size, members):
        assert a.flags["C_CONTIGUOUS"] and a.flags["WRITEABLE"]
    cand = np.ascontiguousarray(cand, np.int32)
    cap = np.ascontiguousarray(cap, np.int32)
    start = np.ascontiguousarray(start, np.int32)
    k_new = np.ascontiguousarray(k_new)
    row = cent.shape[1]
    assert row % nseg == 0 and k_new.size == row
    return lib().ckvo_update_layer(row // nseg, nseg, _p(k_new), _dt(k_new), _p(cand),
                                   cand.shape[0], _p(cent), _p(size), _p(cap), _p(start),
                                   _p(members), int(n))


def edge_scores(Q: np.ndarray, K: np.ndarray, scale: float, rows, keys) -> np.ndarray:
    """fp64 group scores z of (query rows[r], key keys[r]) pairs, as in edges()."""
    Q = np.ascontiguousarray(Q)
    K = np.ascontiguousarray(K)
    n, G, d = Q.shape
    rows = np.ascontiguousarray(rows, np.int32)
    keys = np.ascontiguousarray(keys, np.int32)
    assert rows.shape == keys.shape and rows.ndim == 1
    assert ((rows >= 0) & (rows < n) & (keys >= 0) & (keys < n)).all()
    z = np.empty(len(rows), np.float64)
    lib().ckvo_edge_scores(d, G, _p(Q), _p(K), _dt(K), scale, _p(rows), _p(keys), len(rows),
                           _p(z))
    return z


class OracleState:
    """Host state of one decode layer, advanced one step at a time.

    centroids [NG, Cmax, d] fp32 ([B, Cmax, Hkv*d] for the layer graph); num_comms [NG]; comm_start/size/cap [NG, Cmax];
    members [pool]; K, V [B, Hkv, n_alloc, d] raw (uint16 bf16 bits or float32),
    logical token order; seq_len [B].
    """

    def __init__(self, *, B, Hq, Hkv, d, gpk, S, centroids, num_comms, comm_start,
                 comm_size, comm_cap, members, K, V, seq_len, threads=None):
        self.B, self.Hq, self.Hkv, self.d, self.gpk, self.S = B, Hq, Hkv, d, gpk, S
        self.G = Hq // Hkv
        self.layer = gpk == 0
        self.NG = B if self.layer else B * Hkv * gpk
        self.cent = np.array(centroids, np.float32, copy=True, order="C")
        self.num_comms = np.array(num_comms, np.int32, copy=True)
        self.start = np.array(comm_start, np.int32, copy=True, order="C")
        self.size = np.array(comm_size, np.int32, copy=True, order="C")
        self.cap = np.array(comm_cap, np.int32, copy=True, order="C")
        self.members = np.array(members, np.int32, copy=True, order="C")
        self.K = np.array(K, copy=True, order="C")
        self.V = np.array(V, copy=True, order="C")
        self.seq_len = np.array(seq_len, np.int32, copy=True)
        self.threads = threads or len(os.sched_getaffinity(0))
        self._layer_undo = {}

    def layer_candidate_rows(self, g: int):
        """Layer graph g: (candidate ids, their centroid rows before the last step's
        update, the new token's key row) of the last step."""
        before, cand, krow, _ = self._layer_undo[g]
        return cand, (before[0] if before is not None else None), krow

    def adopt_layer_choice(self, g: int, c: int):
        """Replace the last step's layer-graph choice of graph g by community c (one
        of its candidates): the state goes back to before that update, then the
        update runs with c as the only candidate.  -> the new result code."""
        before, cand, krow, n = self._layer_undo[g]
        assert before is not None and c in set(int(x) for x in cand)
        rows, size, slots, vals = before
        self.cent[g, cand] = rows
        self.size[g, cand] = size
        ok = slots >= 0
        self.members[slots[ok]] = vals[ok]
        Cn = int(self.num_comms[g])
        return update_layer(krow, np.array([c], np.int32), self.cent[g, :Cn],
                            self.size[g, :Cn], self.cap[g, :Cn], self.start[g, :Cn],
                            self.members, n, self.Hkv)

    def heads_of(self, g: int):
        if self.layer:
            return list(range(self.Hq))
        j = g % self.gpk
        kvh = (g // self.gpk) % self.Hkv
        if self.gpk == 1:
            return list(range(kvh * self.G, (kvh + 1) * self.G))
        return [kvh * self.G + j]

    def _layer_step(self, g, q, k_new, budget, scale, M, max_len, res):
        """One whole-layer graph (g = sequence b)."""
        b, d, G = g, self.d, self.G
        n = int(self.seq_len[b])
        Cn = int(self.num_comms[g])
        size = self.size[g, :Cn].copy()
        # per KV head: its G heads against its slice of the centroid rows; the max
        # of the fp32-rounded scores equals the rounding of the max (rounding is
        # monotone)
        s = np.full(Cn, -np.inf, np.float32)
        for kvh in range(self.Hkv):
            part = np.ascontiguousarray(self.cent[g, :Cn, kvh * d:(kvh + 1) * d])
            s = np.maximum(s, score(q[b, kvh * G:(kvh + 1) * G], part, size, scale))
        sel, k, cand = select(s, size, int(budget[b]), M)
        idx = index_list(n, self.S, sel, self.start[g, :Cn], size, self.members, max_len)
        outs = {}
        for kvh in range(self.Hkv):
            for h in range(kvh * G, (kvh + 1) * G):
                outs[h] = attend(q[b, h], self.K[b, kvh], self.V[b, kvh], idx, scale)
        krow = np.ascontiguousarray(k_new[b]).reshape(-1)
        # the candidates' rows before the update, kept so that a caller may replace
        # the choice (adopt_layer_choice)
        before = None
        if len(cand):
            st_, sz_, cp_ = self.start[g, cand], self.size[g, cand], self.cap[g, cand]
            slots = np.where(sz_ < cp_, st_ + sz_, -1)
            before = (self.cent[g, cand].copy(), sz_.copy(), slots,
                      np.where(slots >= 0, self.members[np.maximum(slots, 0)], 0))
        r = update_layer(krow, cand, self.cent[g, :Cn], self.size[g, :Cn], self.cap[g, :Cn],
                         self.start[g, :Cn], self.members, n, self.Hkv) if Cn else -2
        self._layer_undo[g] = (before, cand, krow, n)
        res[g] = (s, sel, k, cand, idx, outs, r)

    def _graph_step(self, g, q, k_new, budget, scale, M, max_len, res):
        if self.layer:
            return self._layer_step(g, q, k_new, budget, scale, M, max_len, res)
        b = g // (self.Hkv * self.gpk)
        kvh = (g // self.gpk) % self.Hkv
        n = int(self.seq_len[b])
        Cn = int(self.num_comms[g])
        heads = self.heads_of(g)
        size = self.size[g, :Cn].copy()
        s = score(q[b, heads], self.cent[g, :Cn], size, scale)
        sel, k, cand = select(s, size, int(budget[b]), M)
        idx = index_list(n, self.S, sel, self.start[g, :Cn], size, self.members, max_len)
        K = self.K[b, kvh]
        V = self.V[b, kvh]
        outs = {h: attend(q[b, h], K, V, idx, scale) for h in heads}
        # local update on this graph's own rows (views into the state arrays)
        cent_g = self.cent[g, :Cn]
        size_g = self.size[g, :Cn]
        r, _ = update(k_new[b, kvh], cand, cent_g, size_g, self.cap[g, :Cn],
                      self.start[g, :Cn], self.members, n) if Cn else (-2, 0)
        res[g] = (s, sel, k, cand, idx, outs, r)

    def step(self, q, k_new, v_new, budget, scale, M, max_len):
        """One decode step for every graph.  q [B, Hq, d], k_new/v_new [B, Hkv, d] raw."""
        q = np.ascontiguousarray(q)
        k_new = np.ascontiguousarray(k_new)
        res = [None] * self.NG
        with ThreadPoolExecutor(self.threads) as ex:
            list(ex.map(lambda g: self._graph_step(g, q, k_new, budget, scale, M, max_len,
                                                   res), range(self.NG)))
        Cmax = self.cent.shape[1]
        out = {
            "scores": np.full((self.NG, Cmax), -np.inf, np.float32),
            "selected": np.zeros((self.NG, Cmax), np.uint8),
            "kstar": np.zeros(self.NG, np.int32),
            "cand": np.full((self.NG, M), -1, np.int32),
            "idx": [None] * self.NG,
            "idx_len": np.zeros(self.NG, np.int32),
            "out": np.zeros((self.B, self.Hq, self.d), np.float64),
            "assigned": np.full(self.NG, -1, np.int32),
            "err": np.zeros(self.NG, np.int32),
        }
        for g, (s, sel, k, cand, idx, outs, r) in enumerate(res):
            b = g if self.layer else g // (self.Hkv * self.gpk)
            Cn = len(s)
            out["scores"][g, :Cn] = s
            out["selected"][g, :Cn] = sel
            out["kstar"][g] = k
            out["cand"][g, :len(cand)] = cand
            out["idx"][g] = idx
            out["idx_len"][g] = len(idx)
            for h, o in outs.items():
                out["out"][b, h] = o
            if r >= 0:
                out["assigned"][g] = r
            elif r == -1:
                out["err"][g] |= ERR_CAPACITY
        # append the new token's key/value at position n, then grow the sequence
        for b in range(self.B):
            n = int(self.seq_len[b])
            self.K[b, :, n] = k_new[b]
            self.V[b, :, n] = v_new[b]
            self.seq_len[b] = n + 1
        return out
