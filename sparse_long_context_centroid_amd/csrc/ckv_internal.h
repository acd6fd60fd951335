// ckv_internal.h -- host-side problem description and kernel launchers of libckv.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ckv.h"

namespace ckv {

// Validated copy of ckv_dims with derived sizes.
struct Problem {
    int B, Hq, Hkv, D, gpk, Cmax, S, dtype;
    // attention only: consecutive graphs that read one index list (the layer
    // graph's list serves the graphs of its Hkv KV heads)
    int list_div = 1;
    // optional timing of the next launch: events bound to the kernel's own start
    // and end (hipExtLaunchKernelGGL), null for none
    hipEvent_t ev_start = nullptr, ev_stop = nullptr;
    int G() const { return Hq / Hkv; }
    // gpk = 0: one graph per layer (per sequence), shared by every head
    bool layer() const { return gpk == 0; }
    int NG() const { return layer() ? B : B * Hkv * gpk; }
    int heads_per_graph() const { return layer() ? Hq : (gpk == 1 ? G() : 1); }
    int graphs_per_seq() const { return layer() ? 1 : Hkv * gpk; }
    // centroid row length: one d-slice per KV head for the layer graph
    int cdim() const { return layer() ? Hkv * D : D; }
    int elem_bytes() const { return dtype == CKV_DT_BF16 ? 2 : 4; }
};

// Attention workgroup: kAttnWaves wavefronts, each issuing kAttnLoads wave-wide
// 16-byte-per-lane loads of K and of V; a row of d elements takes d*elem/16 lanes,
// so one load covers 1024/(d*elem) rows.  Tokens per workgroup:
constexpr int kAttnWaves = 4;
constexpr int kAttnLoads = 12;
// Largest graph count of a persistent attention grid (its per-graph split prefix
// lives in LDS); more graphs always take the direct grid.
constexpr int kAttnPersistMaxGraphs = 1024;
constexpr int attn_chunk(int D, int elem_bytes) {
    return kAttnWaves * kAttnLoads * (1024 / (D * elem_bytes));
}
inline int attn_max_splits(const Problem &p, int index_stride) {
    const int ch = attn_chunk(p.D, p.elem_bytes());
    return (index_stride + ch - 1) / ch;
}

// Compute units of the current device (queried once per device; 256, the MI355X
// count, if the query fails).
int device_cu_count();

inline int log2_pow2(int x) {
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

// Dense baseline: one graph per KV head holding its G query heads (every cached
// token is read, so no graph structure applies).  A workgroup covers cpw chunks
// so that a graph has at most 64 pieces (one merge load round).
inline Problem dense_problem(const Problem &p) {
    Problem d = p;
    d.gpk = 1;
    d.list_div = 1;
    return d;
}
// Attention runs per (sequence, KV head) with that head's G query heads; the
// layer graph's one index list is read by all Hkv of them.
inline Problem attn_problem(const Problem &p) {
    Problem a = p;
    if (p.layer()) {
        a.gpk = 1;
        a.list_div = p.Hkv;
    }
    return a;
}
inline int dense_max_splits(const Problem &p, const ckv_kv &kv, int *cpw) {
    const int ch = attn_chunk(p.D, p.elem_bytes());
    const long long max_ctx = (long long)kv.max_pages_per_seq * kv.page_size;
    const long long c = (max_ctx + (long long)ch * 64 - 1) / ((long long)ch * 64);
    *cpw = c < 1 ? 1 : (int)c;
    const long long span = (long long)ch * *cpw;
    const long long ms = (max_ctx + span - 1) / span;
    return ms < 1 ? 1 : (int)ms;
}
inline size_t dense_partial_floats(const Problem &p, const ckv_kv &kv) {
    const Problem d = dense_problem(p);
    int cpw;
    return (size_t)d.NG() * d.heads_per_graph() * dense_max_splits(d, kv, &cpw) * (d.D + 2);
}

// Workspace of the attention call: partials NG * GH * max_splits * (D + 2) fp32.
inline size_t attn_partial_floats(const Problem &pg, int index_stride) {
    const Problem p = attn_problem(pg);
    return (size_t)p.NG() * p.heads_per_graph() * attn_max_splits(p, index_stride) * (p.D + 2);
}

hipError_t launch_score(const Problem &p, const void *q, const ckv_graphs &gr, double scale,
                        float *scores, hipStream_t st);
hipError_t launch_rows_to_interleaved(const Problem &p, const float *rows, float *cent,
                                      hipStream_t st);
hipError_t launch_interleaved_to_rows(const Problem &p, const float *cent, float *rows,
                                      hipStream_t st);
hipError_t launch_select(const Problem &p, const float *scores, const ckv_graphs &gr,
                         const int32_t *budget, const int32_t *seq_len, int n_cand,
                         int32_t *idx, int idx_stride, int32_t *idx_len, int32_t *num_sel,
                         int32_t *cand, uint8_t *selected, int32_t *err, hipStream_t st);
// Local update run inside the attention launch (fused decode step).
struct UpdateSpec {
    const void *k_new, *v_new;
    const int32_t *cand;
    int n_cand;
    const ckv_graphs *graphs;
    int32_t *assigned;
};
hipError_t launch_attn_partials(const Problem &p, const void *q, const ckv_kv &kv,
                                const int32_t *idx, int idx_stride, const int32_t *idx_len,
                                float scale, float *partials, int32_t *err, const UpdateSpec *upd,
                                hipStream_t st);
hipError_t launch_attn_merge(const Problem &p, int idx_stride, float *out, const float *partials,
                             int32_t *bump_seq_len, hipStream_t st);
// Whether the layer graph's update fits the attention launch's update rows (then the
// decode step runs it there, under the K/V stream).
bool layer_update_in_attention_fits(const Problem &p, int n_cand);
// The layer graph's merge with the step's layer update in extra workgroups (one per
// sequence; each advances its seq_len), when it does not fit the attention launch.
hipError_t launch_attn_merge_layer_update(const Problem &p, int idx_stride, float *out,
                                         const float *partials, const void *k_new,
                                         const void *v_new, const int32_t *cand, int n_cand,
                                         const ckv_graphs &gr, const ckv_kv &kv,
                                         int32_t *assigned, int32_t *err, hipStream_t st);
// Dense baseline: attention over every cached token of each sequence.
hipError_t launch_dense_partials(const Problem &p, const void *q, const ckv_kv &kv, float scale,
                                 float *partials, int32_t *err, hipStream_t st);
hipError_t launch_dense_merge(const Problem &p, const ckv_kv &kv, float *out,
                              const float *partials, hipStream_t st);
// Centroids recomputed from the member lists; drift of the running means.
hipError_t launch_rebuild(const Problem &p, const ckv_graphs &gr, const ckv_kv &kv, float *out,
                          int32_t *err, hipStream_t st);
hipError_t launch_drift(const Problem &p, const ckv_graphs &gr, const float *ref, float *drift,
                        hipStream_t st);
// Prefill token graph: per-query top-k direct edges and their co-attention pairs.
int edge_queries_per_block(const Problem &p);
hipError_t launch_edges(const Problem &p, const void *q, const void *k, int n, float scale,
                        int topk, int32_t *idx, float *score, int32_t *pairs, hipStream_t st);
// The layer graph's update (one workgroup per sequence); bump: seq_len += 1.
bool layer_update_fits(const Problem &p, int n_cand);
hipError_t launch_layer_update(const Problem &p, const void *k_new, const void *v_new,
                               const int32_t *cand, int n_cand, const ckv_graphs &gr,
                               const ckv_kv &kv, int32_t *assigned, int32_t *err, bool bump,
                               hipStream_t st);
hipError_t launch_update(const Problem &p, const void *k_new, const void *v_new,
                         const int32_t *cand, int n_cand, const ckv_graphs &gr, const ckv_kv &kv,
                         int32_t *assigned, int32_t *err, hipStream_t st);

}  // namespace ckv
