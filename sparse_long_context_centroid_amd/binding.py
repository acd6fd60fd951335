"""ctypes binding of libckv.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch tensors
that already live on the GPU; it passes their raw device pointers and the current
HIP stream.  No computation happens here, and there is no fallback: if the HIP
library is missing or fails, the call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libckv.so")

CKV_OK = 0
CKV_DT_F32 = 0
CKV_DT_BF16 = 1
DEVERR_CAPACITY = 1
DEVERR_UNMAPPED_PAGE = 2
DEVERR_INDEX_RANGE = 4


class ckv_dims(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("graphs_per_kv", C.c_int32), ("max_comms", C.c_int32),
                ("num_sinks", C.c_int32), ("dtype", C.c_int32)]


class ckv_graphs(C.Structure):
    _fields_ = [("centroids", C.c_void_p), ("num_comms", C.c_void_p), ("comm_start", C.c_void_p),
                ("comm_size", C.c_void_p), ("comm_cap", C.c_void_p), ("members", C.c_void_p)]


class ckv_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("page_table", C.c_void_p),
                ("page_size", C.c_int32), ("max_pages_per_seq", C.c_int32),
                ("num_pages", C.c_int32), ("seq_len", C.c_void_p)]


class CkvError(RuntimeError):
    pass


_lib = None


def load(path: str = LIB_PATH):
    """Load libckv.so (built by sparse_long_context_centroid_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CkvError(f"{path} is missing: build it with "
                       "`python -m sparse_long_context_centroid_amd.build`")
    L = C.CDLL(path)
    P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    pd, pg, pk = C.POINTER(ckv_dims), C.POINTER(ckv_graphs), C.POINTER(ckv_kv)
    sig = {
        "ckv_workspace_size": (sz, [pd, i32]),
        "ckv_centroids_from_rows": (i32, [pd, P, P, P]),
        "ckv_centroids_to_rows": (i32, [pd, P, P, P]),
        "ckv_score_centroids": (i32, [pd, P, pg, C.c_float, P, P]),
        "ckv_select": (i32, [pd, P, pg, P, P, i32, P, i32, P, P, P, P, P, P]),
        "ckv_sparse_decode_attn": (i32, [pd, P, pk, P, i32, P, C.c_float, P, P, sz, P, P]),
        "ckv_local_update": (i32, [pd, P, P, P, i32, pg, pk, P, P, P]),
        "ckv_decode_step": (i32, [pd, P, P, P, pg, pk, P, i32, C.c_float, P, P, i32, P, P, P,
                                  P, P, P, P, sz, P, P, P]),
        "ckv_decode_step_noalloc": (i32, [pd, P, P, P, pg, pk, P, i32, C.c_float, P, P, i32, P,
                                          P, P, P, P, P, P, P, P]),
        "ckv_dense_workspace_size": (sz, [pd, pk]),
        "ckv_dense_decode_attn": (i32, [pd, P, pk, C.c_float, P, P, sz, P, P]),
        "ckv_rebuild_centroids": (i32, [pd, pg, pk, P, P, P]),
        "ckv_centroid_drift": (i32, [pd, pg, P, P, P]),
        "ckv_prefill_edges": (i32, [pd, P, P, i32, i32, C.c_float, P, P, P, P, P]),
        "ckv_status_string": (C.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


EXPORTED = ("ckv_workspace_size", "ckv_centroids_from_rows", "ckv_centroids_to_rows",
            "ckv_score_centroids", "ckv_select", "ckv_sparse_decode_attn", "ckv_local_update",
            "ckv_decode_step", "ckv_decode_step_noalloc", "ckv_dense_workspace_size",
            "ckv_dense_decode_attn",
            "ckv_rebuild_centroids", "ckv_centroid_drift", "ckv_prefill_edges",
            "ckv_status_string")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise CkvError("libckv takes device tensors")
    if not t.is_contiguous():
        raise CkvError("libckv takes contiguous tensors")
    return C.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != CKV_OK:
        msg = load().ckv_status_string(status).decode()
        raise CkvError(f"{what} failed: {msg} ({status})")


def make_dims(B, Hq, Hkv, d, gpk, Cmax, S, dtype) -> ckv_dims:
    return ckv_dims(B, Hq, Hkv, d, gpk, Cmax, S, dtype)


def make_graphs(centroids, num_comms, comm_start, comm_size, comm_cap, members) -> ckv_graphs:
    return ckv_graphs(_ptr(centroids), _ptr(num_comms), _ptr(comm_start), _ptr(comm_size),
                      _ptr(comm_cap), _ptr(members))


def make_kv(k, v, page_table, page_size, seq_len) -> ckv_kv:
    return ckv_kv(_ptr(k), _ptr(v), _ptr(page_table), page_size, page_table.shape[1],
                  k.shape[0], _ptr(seq_len))


# ---- entry points ---------------------------------------------------------------------

def ckv_workspace_size(dims: ckv_dims, index_stride: int) -> int:
    return load().ckv_workspace_size(C.byref(dims), index_stride)


def ckv_centroids_from_rows(dims, rows, centroids, stream=None):
    _check(load().ckv_centroids_from_rows(C.byref(dims), _ptr(rows), _ptr(centroids),
                                          _stream(stream)), "ckv_centroids_from_rows")


def ckv_centroids_to_rows(dims, centroids, rows, stream=None):
    _check(load().ckv_centroids_to_rows(C.byref(dims), _ptr(centroids), _ptr(rows),
                                        _stream(stream)), "ckv_centroids_to_rows")


def ckv_score_centroids(dims, q, graphs, scale, scores, stream=None):
    _check(load().ckv_score_centroids(C.byref(dims), _ptr(q), C.byref(graphs), scale,
                                      _ptr(scores), _stream(stream)), "ckv_score_centroids")


def ckv_select(dims, scores, graphs, budget, seq_len, n_cand, index_list, index_len,
               num_selected, cand, selected, err_flag, stream=None):
    _check(load().ckv_select(C.byref(dims), _ptr(scores), C.byref(graphs), _ptr(budget),
                             _ptr(seq_len), n_cand, _ptr(index_list), index_list.shape[1],
                             _ptr(index_len), _ptr(num_selected), _ptr(cand), _ptr(selected),
                             _ptr(err_flag), _stream(stream)), "ckv_select")


def ckv_sparse_decode_attn(dims, q, kv, index_list, index_len, scale, out, ws, err_flag,
                           stream=None):
    _check(load().ckv_sparse_decode_attn(C.byref(dims), _ptr(q), C.byref(kv), _ptr(index_list),
                                         index_list.shape[1], _ptr(index_len), scale, _ptr(out),
                                         _ptr(ws), ws.numel() * ws.element_size(), _ptr(err_flag),
                                         _stream(stream)), "ckv_sparse_decode_attn")


def ckv_dense_workspace_size(dims, kv) -> int:
    return int(load().ckv_dense_workspace_size(C.byref(dims), C.byref(kv)))


def ckv_dense_decode_attn(dims, q, kv, scale, out, ws, err_flag, stream=None):
    _check(load().ckv_dense_decode_attn(C.byref(dims), _ptr(q), C.byref(kv), scale, _ptr(out),
                                        _ptr(ws), ws.numel() * ws.element_size(), _ptr(err_flag),
                                        _stream(stream)), "ckv_dense_decode_attn")


def ckv_rebuild_centroids(dims, graphs, kv, centroids_out, err_flag, stream=None):
    _check(load().ckv_rebuild_centroids(C.byref(dims), C.byref(graphs), C.byref(kv),
                                        _ptr(centroids_out), _ptr(err_flag), _stream(stream)),
           "ckv_rebuild_centroids")


def ckv_centroid_drift(dims, graphs, reference, drift, stream=None):
    _check(load().ckv_centroid_drift(C.byref(dims), C.byref(graphs), _ptr(reference),
                                     _ptr(drift), _stream(stream)), "ckv_centroid_drift")


def ckv_prefill_edges(dims, q, k, n, topk, scale, edge_idx, edge_score, edge_pairs=None,
                      events=None, stream=None):
    """events: None or 2 torch.cuda.Event(enable_timing=True) bound to the kernel."""
    ev = None
    if events is not None:
        if len(events) != 2:
            raise CkvError("ckv_prefill_edges takes 2 events")
        for e in events:
            if e.cuda_event == 0:        # torch creates the HIP event at first record
                e.record()
        ev = (C.c_void_p * 2)(*[e.cuda_event for e in events])
    _check(load().ckv_prefill_edges(C.byref(dims), _ptr(q), _ptr(k), n, topk, scale,
                                    _ptr(edge_idx), _ptr(edge_score), _ptr(edge_pairs), ev,
                                    _stream(stream)), "ckv_prefill_edges")


def ckv_local_update(dims, k_new, v_new, cand, n_cand, graphs, kv, assigned, err_flag,
                     stream=None):
    _check(load().ckv_local_update(C.byref(dims), _ptr(k_new), _ptr(v_new), _ptr(cand), n_cand,
                                   C.byref(graphs), C.byref(kv), _ptr(assigned), _ptr(err_flag),
                                   _stream(stream)), "ckv_local_update")


def ckv_decode_step(dims, q, k_new, v_new, graphs, kv, budget, n_cand, scale, scores,
                    index_list, index_len, num_selected, cand, selected, assigned, out, ws,
                    err_flag, events=None, stream=None):
    """events: None or 8 torch.cuda.Event(enable_timing=True): the start / stop pair
    of each of the 4 kernels (score, select, attention + update, merge), bound to
    the kernels' own execution."""
    ev = None
    if events is not None:
        if len(events) != 8:
            raise CkvError("ckv_decode_step takes 8 timing events")
        for e in events:
            if e.cuda_event == 0:        # torch creates the HIP event at first record
                e.record()
        ev = (C.c_void_p * 8)(*[e.cuda_event for e in events])
    _check(load().ckv_decode_step(C.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new),
                                  C.byref(graphs), C.byref(kv), _ptr(budget), n_cand, scale,
                                  _ptr(scores), _ptr(index_list), index_list.shape[1],
                                  _ptr(index_len), _ptr(num_selected), _ptr(cand),
                                  _ptr(selected), _ptr(assigned), _ptr(out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _ptr(err_flag), ev,
                                  _stream(stream)), "ckv_decode_step")


def ckv_decode_step_noalloc(dims, q, k_new, v_new, graphs, kv, budget, n_cand, scale, scores,
                            index_list, index_len, num_selected, cand, selected, assigned, out,
                            err_flag, events=None, stream=None):
    """ckv_decode_step without a workspace argument: the library's own device array."""
    ev = None
    if events is not None:
        if len(events) != 8:
            raise CkvError("ckv_decode_step_noalloc takes 8 timing events")
        for e in events:
            if e.cuda_event == 0:
                e.record()
        ev = (C.c_void_p * 8)(*[e.cuda_event for e in events])
    _check(load().ckv_decode_step_noalloc(C.byref(dims), _ptr(q), _ptr(k_new), _ptr(v_new),
                                          C.byref(graphs), C.byref(kv), _ptr(budget), n_cand,
                                          scale, _ptr(scores), _ptr(index_list),
                                          index_list.shape[1], _ptr(index_len),
                                          _ptr(num_selected), _ptr(cand), _ptr(selected),
                                          _ptr(assigned), _ptr(out), _ptr(err_flag), ev,
                                          _stream(stream)), "ckv_decode_step_noalloc")


def ckv_status_string(status: int) -> str:
    return load().ckv_status_string(status).decode()


# ---- device state of one decode layer ----------------------------------------------------

class DecodeLayer:
    """Device buffers of one layer (graphs, paged KV, outputs, workspaces) and the
    four calls of one decode step.  Built from host/device arrays; every step of
    the path runs in libckv's kernels."""

    def __init__(self, *, B, Hq, Hkv, d, gpk, S, dtype, Cmax, M, index_stride, page_size,
                 centroid_rows, num_comms, comm_start, comm_size, comm_cap, members,
                 k_pages, v_pages, page_table, seq_len, budget, device="cuda"):
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.dims = make_dims(B, Hq, Hkv, d, gpk, Cmax, S, dtype)
        self.B, self.Hq, self.Hkv, self.d, self.gpk, self.S, self.M = B, Hq, Hkv, d, gpk, S, M
        self.Cmax = Cmax
        # gpk = 0: one graph per layer (per sequence) whose centroid rows hold one
        # d-slice per KV head
        self.NG = B if gpk == 0 else B * Hkv * gpk
        self.cdim = Hkv * d if gpk == 0 else d
        self.page_size = page_size
        t = lambda a: torch.as_tensor(a).to(**i32).contiguous()
        self.num_comms = t(num_comms)
        self.comm_start = t(comm_start)
        self.comm_size = t(comm_size)
        self.comm_cap = t(comm_cap)
        self.members = t(members)
        self.centroids = torch.empty(self.NG * Cmax * self.cdim, dtype=torch.float32,
                                     device=dev)
        rows = centroid_rows.to(dev, torch.float32).contiguous()
        ckv_centroids_from_rows(self.dims, rows, self.centroids)
        self.k = k_pages.to(dev).contiguous()
        self.v = v_pages.to(dev).contiguous()
        self.page_table = t(page_table)
        self.seq_len = t(seq_len)
        self.budget = t(budget)
        self.graphs = make_graphs(self.centroids, self.num_comms, self.comm_start,
                                  self.comm_size, self.comm_cap, self.members)
        self.kv = make_kv(self.k, self.v, self.page_table, page_size, self.seq_len)
        # outputs and workspaces
        self.scores = torch.full((self.NG, Cmax), float("-inf"), dtype=torch.float32, device=dev)
        self.index_list = torch.zeros((self.NG, index_stride), **i32)
        self.index_len = torch.zeros(self.NG, **i32)
        self.num_selected = torch.zeros(self.NG, **i32)
        self.cand = torch.zeros((self.NG, M), **i32)
        self.selected = torch.zeros((self.NG, Cmax), dtype=torch.uint8, device=dev)
        self.assigned = torch.zeros(self.NG, **i32)
        self.err = torch.zeros(1, **i32)
        self.out = torch.zeros((B, Hq, d), dtype=torch.float32, device=dev)
        wsz = ckv_workspace_size(self.dims, index_stride)
        if wsz == 0:
            raise CkvError("invalid dims for the workspace")
        self.ws = torch.empty(wsz, dtype=torch.uint8, device=dev)

    # individual stages
    def score(self, q, scale):
        ckv_score_centroids(self.dims, q, self.graphs, scale, self.scores)

    def select(self):
        ckv_select(self.dims, self.scores, self.graphs, self.budget, self.seq_len, self.M,
                   self.index_list, self.index_len, self.num_selected, self.cand,
                   self.selected, self.err)

    def attend(self, q, scale):
        ckv_sparse_decode_attn(self.dims, q, self.kv, self.index_list, self.index_len, scale,
                               self.out, self.ws, self.err)

    def dense(self, q, scale, out=None):
        """Dense baseline: attention over every cached token (no selection)."""
        if getattr(self, "dense_ws", None) is None:
            n = ckv_dense_workspace_size(self.dims, self.kv)
            if n == 0:
                raise CkvError("invalid dims for the dense workspace")
            self.dense_ws = torch.empty(n, dtype=torch.uint8, device=self.out.device)
        out = self.out if out is None else out
        ckv_dense_decode_attn(self.dims, q, self.kv, scale, out, self.dense_ws, self.err)

    def rebuild(self, out=None):
        """Centroids recomputed from the member lists (interleaved layout)."""
        out = torch.empty_like(self.centroids) if out is None else out
        ckv_rebuild_centroids(self.dims, self.graphs, self.kv, out, self.err)
        return out

    def drift(self, reference):
        """Per-graph largest relative distance of the running centroids from `reference`."""
        d = torch.empty(self.NG, dtype=torch.float32, device=self.centroids.device)
        ckv_centroid_drift(self.dims, self.graphs, reference, d)
        return d

    def update(self, k_new, v_new):
        ckv_local_update(self.dims, k_new, v_new, self.cand, self.M, self.graphs, self.kv,
                         self.assigned, self.err)

    def step(self, q, k_new, v_new, scale):
        """The four calls of the C ABI, in order."""
        self.score(q, scale)
        self.select()
        self.attend(q, scale)
        self.update(k_new, v_new)

    def step_fused(self, q, k_new, v_new, scale, events=None):
        """The same step through ckv_decode_step (4 launches; 5 for the layer graph).
        Without events the layer's own arguments are marshalled once and reused
        while the same objects stay in place, so a call converts only q, k_new,
        v_new, the scale and the stream."""
        if events is not None:
            ckv_decode_step(self.dims, q, k_new, v_new, self.graphs, self.kv, self.budget,
                            self.M, scale, self.scores, self.index_list, self.index_len,
                            self.num_selected, self.cand, self.selected, self.assigned, self.out,
                            self.ws, self.err, events=events)
            return
        own = (self.dims, self.graphs, self.kv, self.budget, self.scores, self.index_list,
               self.index_len, self.num_selected, self.cand, self.selected, self.assigned,
               self.out, self.ws, self.err)
        key = tuple(map(id, own)) + (self.M,)
        cached = getattr(self, "_fused_args", None)
        if cached is None or cached[0] != key:
            head = (C.byref(self.dims),)
            mid = (C.byref(self.graphs), C.byref(self.kv), _ptr(self.budget), self.M)
            tail = (_ptr(self.scores), _ptr(self.index_list), self.index_list.shape[1],
                    _ptr(self.index_len), _ptr(self.num_selected), _ptr(self.cand),
                    _ptr(self.selected), _ptr(self.assigned), _ptr(self.out), _ptr(self.ws),
                    self.ws.numel() * self.ws.element_size(), _ptr(self.err), None)
            cached = self._fused_args = (key, own, head, mid, tail)
        _, _, head, mid, tail = cached
        _check(load().ckv_decode_step(*head, _ptr(q), _ptr(k_new), _ptr(v_new), *mid, scale,
                                      *tail, _stream(None)), "ckv_decode_step")

    def step_noalloc(self, q, k_new, v_new, scale, events=None):
        """The same step through ckv_decode_step_noalloc (no workspace argument)."""
        ckv_decode_step_noalloc(self.dims, q, k_new, v_new, self.graphs, self.kv, self.budget,
                                self.M, scale, self.scores, self.index_list, self.index_len,
                                self.num_selected, self.cand, self.selected, self.assigned,
                                self.out, self.err, events=events)

    def centroid_rows(self) -> torch.Tensor:
        rows = torch.empty((self.NG, self.Cmax, self.cdim), dtype=torch.float32,
                           device=self.centroids.device)
        ckv_centroids_to_rows(self.dims, self.centroids, rows)
        return rows


def decode_layer_from_workload(wl, li: int = 0, index_stride: Optional[int] = None,
                               device: str = "cuda") -> DecodeLayer:
    """Device state of layer `li` of a generated workload (inputs.make_workload)."""
    L = wl.layers[li]
    if index_stride is None:
        index_stride = int(wl.S + wl.budget.max())
    if tuple(L.comm_start.shape) != (wl.NG, wl.Cmax) or L.centroids.shape[1] != wl.Cmax:
        raise CkvError(f"layer {li}: per-community arrays are not [NG, Cmax] = "
                       f"[{wl.NG}, {wl.Cmax}]")
    return DecodeLayer(B=wl.B, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, gpk=wl.gpk, S=wl.S,
                       dtype=wl.dtype, Cmax=wl.Cmax, M=wl.M, index_stride=index_stride,
                       page_size=wl.page_size, centroid_rows=L.centroids,
                       num_comms=L.num_comms, comm_start=L.comm_start, comm_size=L.comm_size,
                       comm_cap=L.comm_cap, members=L.members, k_pages=L.k_pages,
                       v_pages=L.v_pages, page_table=wl.page_table, seq_len=wl.seq_len0,
                       budget=wl.budget, device=device)
