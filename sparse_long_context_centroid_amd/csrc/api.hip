// api.hip -- the extern "C" entry points of libckv.so: host-side validation, then
// launches on the caller's stream.  No allocation, no synchronisation, no state.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "ckv.h"
#include "ckv_internal.h"

using ckv::Problem;

namespace ckv {
int device_cu_count() {
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}
}  // namespace ckv

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

ckv_status make_problem(const ckv_dims *d, Problem &p) {
    if (!d) return CKV_ERR_INVALID_ARG;
    if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->num_sinks < 0 ||
        d->max_comms < 64 || d->max_comms % 64 != 0)
        return CKV_ERR_INVALID_ARG;
    if (d->num_q_heads % d->num_kv_heads != 0) return CKV_ERR_INVALID_ARG;
    const int G = d->num_q_heads / d->num_kv_heads;
    if (d->graphs_per_kv != 0 && d->graphs_per_kv != 1 && d->graphs_per_kv != G)
        return CKV_ERR_INVALID_ARG;
    if (G != 1 && G != 2 && G != 4 && G != 8) return CKV_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128) return CKV_ERR_UNSUPPORTED;
    if (d->dtype != CKV_DT_BF16 && d->dtype != CKV_DT_F32) return CKV_ERR_UNSUPPORTED;
    if (d->max_comms > CKV_MAX_COMMS) return CKV_ERR_UNSUPPORTED;
    p.B = d->batch;
    p.Hq = d->num_q_heads;
    p.Hkv = d->num_kv_heads;
    p.D = d->head_dim;
    p.gpk = d->graphs_per_kv;
    p.Cmax = d->max_comms;
    p.S = d->num_sinks;
    p.dtype = d->dtype;
    if ((long long)p.NG() * p.Cmax * p.cdim() > (1LL << 40)) return CKV_ERR_INVALID_ARG;
    return CKV_OK;
}

// members may be null: an empty pool (no community has a member slot) has no
// address, and no kernel reads or writes the pool of a community without slots
ckv_status check_graphs(const ckv_graphs *g) {
    if (!g || !g->centroids || !g->num_comms || !g->comm_start || !g->comm_size ||
        !g->comm_cap)
        return CKV_ERR_INVALID_ARG;
    return CKV_OK;
}

ckv_status check_kv(const ckv_kv *kv, const Problem &p) {
    if (!kv || !kv->k || !kv->v || !kv->page_table || !kv->seq_len) return CKV_ERR_INVALID_ARG;
    if (!is_pow2(kv->page_size) || kv->page_size > 4096 || kv->max_pages_per_seq < 1 ||
        kv->num_pages < 1)
        return CKV_ERR_INVALID_ARG;
    // row indices (page, head, slot) are 32-bit inside the kernels
    if ((long long)kv->num_pages * p.Hkv * kv->page_size >= (1LL << 31))
        return CKV_ERR_UNSUPPORTED;
    return CKV_OK;
}

ckv_status hip_status(hipError_t e) { return e == hipSuccess ? CKV_OK : CKV_ERR_HIP; }

// The split merge keeps one weight per (head, split) in LDS.
ckv_status check_splits(const Problem &p, int index_stride) {
    const Problem a = ckv::attn_problem(p);
    const size_t lds = (size_t)a.heads_per_graph() * ckv::attn_max_splits(a, index_stride) * 4;
    return lds <= 65536 ? CKV_OK : CKV_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

size_t ckv_workspace_size(const ckv_dims *dims, int32_t index_stride) {
    Problem p;
    if (make_problem(dims, p) != CKV_OK || index_stride < 1) return 0;
    return ckv::attn_partial_floats(p, index_stride) * sizeof(float);
}

ckv_status ckv_centroids_from_rows(const ckv_dims *dims, const float *rows, float *centroids,
                                   void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if (!rows || !centroids || rows == centroids) return CKV_ERR_INVALID_ARG;
    return hip_status(ckv::launch_rows_to_interleaved(p, rows, centroids,
                                                       static_cast<hipStream_t>(stream)));
}

ckv_status ckv_centroids_to_rows(const ckv_dims *dims, const float *centroids, float *rows,
                                 void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if (!rows || !centroids || rows == centroids) return CKV_ERR_INVALID_ARG;
    return hip_status(ckv::launch_interleaved_to_rows(p, centroids, rows,
                                                       static_cast<hipStream_t>(stream)));
}

ckv_status ckv_score_centroids(const ckv_dims *dims, const void *q, const ckv_graphs *graphs,
                               float scale, float *scores, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_graphs(graphs)) != CKV_OK) return s;
    if (!q || !scores) return CKV_ERR_INVALID_ARG;
    return hip_status(ckv::launch_score(p, q, *graphs, (double)scale, scores,
                                        static_cast<hipStream_t>(stream)));
}

ckv_status ckv_select(const ckv_dims *dims, const float *scores, const ckv_graphs *graphs,
                      const int32_t *budget, const int32_t *kv_seq_len, int32_t n_cand,
                      int32_t *index_list, int32_t index_stride, int32_t *index_len,
                      int32_t *num_selected, int32_t *cand, uint8_t *selected,
                      int32_t *err_flag, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_graphs(graphs)) != CKV_OK) return s;
    if (!scores || !budget || !kv_seq_len || !index_list || !index_len || !cand)
        return CKV_ERR_INVALID_ARG;
    if (n_cand < 1 || n_cand > CKV_MAX_CAND || index_stride < 1) return CKV_ERR_INVALID_ARG;
    return hip_status(ckv::launch_select(p, scores, *graphs, budget, kv_seq_len, n_cand,
                                         index_list, index_stride, index_len, num_selected, cand,
                                         selected, err_flag, static_cast<hipStream_t>(stream)));
}

ckv_status ckv_sparse_decode_attn(const ckv_dims *dims, const void *q, const ckv_kv *kv,
                                  const int32_t *index_list, int32_t index_stride,
                                  const int32_t *index_len, float scale, float *out, void *ws,
                                  size_t ws_bytes, int32_t *err_flag, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_kv(kv, p)) != CKV_OK) return s;
    if (!q || !index_list || !index_len || !out || index_stride < 1) return CKV_ERR_INVALID_ARG;
    if ((s = check_splits(p, index_stride)) != CKV_OK) return s;
    if (!ws || ws_bytes < ckv_workspace_size(dims, index_stride)) return CKV_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = hip_status(ckv::launch_attn_partials(p, q, *kv, index_list, index_stride, index_len,
                                                  scale, static_cast<float *>(ws), err_flag,
                                                  nullptr, st))) != CKV_OK)
        return s;
    return hip_status(
        ckv::launch_attn_merge(p, index_stride, out, static_cast<float *>(ws), nullptr, st));
}

size_t ckv_dense_workspace_size(const ckv_dims *dims, const ckv_kv *kv) {
    Problem p;
    if (make_problem(dims, p) != CKV_OK || check_kv(kv, p) != CKV_OK) return 0;
    return ckv::dense_partial_floats(p, *kv) * sizeof(float);
}

ckv_status ckv_dense_decode_attn(const ckv_dims *dims, const void *q, const ckv_kv *kv,
                                 float scale, float *out, void *ws, size_t ws_bytes,
                                 int32_t *err_flag, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_kv(kv, p)) != CKV_OK) return s;
    if (!q || !out) return CKV_ERR_INVALID_ARG;
    if (!ws || ws_bytes < ckv_dense_workspace_size(dims, kv)) return CKV_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((s = hip_status(ckv::launch_dense_partials(p, q, *kv, scale, static_cast<float *>(ws),
                                                   err_flag, st))) != CKV_OK)
        return s;
    return hip_status(ckv::launch_dense_merge(p, *kv, out, static_cast<float *>(ws), st));
}

ckv_status ckv_rebuild_centroids(const ckv_dims *dims, const ckv_graphs *graphs,
                                 const ckv_kv *kv, float *centroids_out, int32_t *err_flag,
                                 void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_graphs(graphs)) != CKV_OK) return s;
    if ((s = check_kv(kv, p)) != CKV_OK) return s;
    if (!centroids_out) return CKV_ERR_INVALID_ARG;
    return hip_status(ckv::launch_rebuild(p, *graphs, *kv, centroids_out, err_flag,
                                          static_cast<hipStream_t>(stream)));
}

ckv_status ckv_centroid_drift(const ckv_dims *dims, const ckv_graphs *graphs,
                              const float *reference, float *drift, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_graphs(graphs)) != CKV_OK) return s;
    if (!reference || !drift) return CKV_ERR_INVALID_ARG;
    return hip_status(
        ckv::launch_drift(p, *graphs, reference, drift, static_cast<hipStream_t>(stream)));
}

ckv_status ckv_prefill_edges(const ckv_dims *dims, const void *q, const void *k, int32_t n,
                             int32_t topk, float scale, int32_t *edge_idx, float *edge_score,
                             int32_t *edge_pairs, void *const *events, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if (p.dtype != CKV_DT_BF16 || p.layer()) return CKV_ERR_UNSUPPORTED;
    if (!q || !k || !edge_idx || !edge_score) return CKV_ERR_INVALID_ARG;
    if (n < 1 || topk < 1 || topk > CKV_MAX_EDGES || !std::isfinite(scale))
        return CKV_ERR_INVALID_ARG;
    if ((long long)p.B * n * p.Hq * p.D >= (1LL << 40)) return CKV_ERR_INVALID_ARG;
    if (events) {
        p.ev_start = static_cast<hipEvent_t>(events[0]);
        p.ev_stop = static_cast<hipEvent_t>(events[1]);
    }
    return hip_status(ckv::launch_edges(p, q, k, n, scale, topk, edge_idx, edge_score,
                                        edge_pairs, static_cast<hipStream_t>(stream)));
}

ckv_status ckv_local_update(const ckv_dims *dims, const void *k_new, const void *v_new,
                            const int32_t *cand, int32_t n_cand, const ckv_graphs *graphs,
                            const ckv_kv *kv, int32_t *assigned, int32_t *err_flag,
                            void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_graphs(graphs)) != CKV_OK) return s;
    if ((s = check_kv(kv, p)) != CKV_OK) return s;
    if (!k_new || !v_new || !cand || !assigned) return CKV_ERR_INVALID_ARG;
    if (n_cand < 1 || n_cand > CKV_MAX_CAND) return CKV_ERR_INVALID_ARG;
    if (p.layer() && !ckv::layer_update_fits(p, n_cand)) return CKV_ERR_UNSUPPORTED;
    return hip_status(ckv::launch_update(p, k_new, v_new, cand, n_cand, *graphs, *kv, assigned,
                                         err_flag, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// The decode step behind ckv_decode_step and ckv_decode_step_noalloc; ws holds
// ws_bytes of device scratch.
ckv_status decode_step_impl(const ckv_dims *dims, const void *q, const void *k_new,
                            const void *v_new, const ckv_graphs *graphs, const ckv_kv *kv,
                            const int32_t *budget, int32_t n_cand, float scale, float *scores,
                            int32_t *index_list, int32_t index_stride, int32_t *index_len,
                            int32_t *num_selected, int32_t *cand, uint8_t *selected,
                            int32_t *assigned, float *out, void *ws, size_t ws_bytes,
                            int32_t *err_flag, void *const *events, void *stream) {
    Problem p;
    ckv_status s = make_problem(dims, p);
    if (s != CKV_OK) return s;
    if ((s = check_graphs(graphs)) != CKV_OK) return s;
    if ((s = check_kv(kv, p)) != CKV_OK) return s;
    if (!q || !k_new || !v_new || !budget || !scores || !index_list || !index_len || !cand ||
        !assigned || !out)
        return CKV_ERR_INVALID_ARG;
    if (n_cand < 1 || n_cand > CKV_MAX_CAND || index_stride < 1) return CKV_ERR_INVALID_ARG;
    if ((s = check_splits(p, index_stride)) != CKV_OK) return s;
    if (p.layer() && !ckv::layer_update_fits(p, n_cand)) return CKV_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < ckv_workspace_size(dims, index_stride)) return CKV_ERR_WORKSPACE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // launch k's timing events, bound to the kernel's own start and end
    auto timed = [&](int k) {
        Problem t = p;
        if (events) {
            t.ev_start = static_cast<hipEvent_t>(events[2 * k]);
            t.ev_stop = static_cast<hipEvent_t>(events[2 * k + 1]);
        }
        return t;
    };
    if ((s = hip_status(ckv::launch_score(timed(0), q, *graphs, (double)scale, scores, st))) !=
        CKV_OK)
        return s;
    if ((s = hip_status(ckv::launch_select(timed(1), scores, *graphs, budget, kv->seq_len, n_cand,
                                           index_list, index_stride, index_len, num_selected,
                                           cand, selected, err_flag, st))) != CKV_OK)
        return s;
    if (p.layer()) {
        // the layer graph: its update runs in extra workgroups of the attention launch
        // when its staging fits there (then the merge advances seq_len), else in extra
        // workgroups of the merge launch (each advancing its sequence's seq_len)
        if (ckv::layer_update_in_attention_fits(p, n_cand)) {
            const ckv::UpdateSpec lupd{k_new, v_new, cand, n_cand, graphs, assigned};
            if ((s = hip_status(ckv::launch_attn_partials(timed(2), q, *kv, index_list,
                                                          index_stride, index_len, scale,
                                                          static_cast<float *>(ws), err_flag,
                                                          &lupd, st))) != CKV_OK)
                return s;
            return hip_status(ckv::launch_attn_merge(timed(3), index_stride, out,
                                                     static_cast<float *>(ws), kv->seq_len, st));
        }
        if ((s = hip_status(ckv::launch_attn_partials(timed(2), q, *kv, index_list,
                                                      index_stride, index_len, scale,
                                                      static_cast<float *>(ws), err_flag,
                                                      nullptr, st))) != CKV_OK)
            return s;
        return hip_status(ckv::launch_attn_merge_layer_update(
            timed(3), index_stride, out, static_cast<float *>(ws), k_new, v_new, cand, n_cand,
            *graphs, *kv, assigned, err_flag, st));
    }
    const ckv::UpdateSpec upd{k_new, v_new, cand, n_cand, graphs, assigned};
    if ((s = hip_status(ckv::launch_attn_partials(timed(2), q, *kv, index_list, index_stride,
                                                  index_len, scale, static_cast<float *>(ws),
                                                  err_flag, &upd, st))) != CKV_OK)
        return s;
    return hip_status(ckv::launch_attn_merge(timed(3), index_stride, out,
                                             static_cast<float *>(ws), kv->seq_len, st));
}

// Scratch of ckv_decode_step_noalloc: one array per GPU the library runs on, held
// until the process ends.  In host code `scratch` only names the symbol; its
// device address on each GPU comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address reaches the kernels.
constexpr size_t kNoallocScratchBytes = (size_t)CKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call on that
// device; nullptr on failure.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

ckv_status ckv_decode_step(const ckv_dims *dims, const void *q, const void *k_new,
                           const void *v_new, const ckv_graphs *graphs, const ckv_kv *kv,
                           const int32_t *budget, int32_t n_cand, float scale, float *scores,
                           int32_t *index_list, int32_t index_stride, int32_t *index_len,
                           int32_t *num_selected, int32_t *cand, uint8_t *selected,
                           int32_t *assigned, float *out, void *ws, size_t ws_bytes,
                           int32_t *err_flag, void *const *events, void *stream) {
    return decode_step_impl(dims, q, k_new, v_new, graphs, kv, budget, n_cand, scale, scores,
                            index_list, index_stride, index_len, num_selected, cand, selected,
                            assigned, out, ws, ws_bytes, err_flag, events, stream);
}

ckv_status ckv_decode_step_noalloc(const ckv_dims *dims, const void *q, const void *k_new,
                                   const void *v_new, const ckv_graphs *graphs, const ckv_kv *kv,
                                   const int32_t *budget, int32_t n_cand, float scale,
                                   float *scores, int32_t *index_list, int32_t index_stride,
                                   int32_t *index_len, int32_t *num_selected, int32_t *cand,
                                   uint8_t *selected, int32_t *assigned, float *out,
                                   int32_t *err_flag, void *const *events, void *stream) {
    // the size check needs no device: a step whose scratch exceeds the array is
    // refused before anything is looked up or enqueued
    const size_t need = ckv_workspace_size(dims, index_stride);
    if (need == 0) {
        Problem p;
        const ckv_status s = make_problem(dims, p);
        return s != CKV_OK ? s : CKV_ERR_INVALID_ARG;
    }
    if (need > kNoallocScratchBytes) return CKV_ERR_WORKSPACE;
    void *ws = device_scratch();
    if (!ws) return CKV_ERR_HIP;
    return decode_step_impl(dims, q, k_new, v_new, graphs, kv, budget, n_cand, scale, scores,
                            index_list, index_stride, index_len, num_selected, cand, selected,
                            assigned, out, ws, kNoallocScratchBytes, err_flag, events, stream);
}

const char *ckv_status_string(ckv_status status) {
    switch (status) {
        case CKV_OK: return "ok";
        case CKV_ERR_INVALID_ARG: return "invalid argument";
        case CKV_ERR_UNSUPPORTED: return "unsupported configuration";
        case CKV_ERR_WORKSPACE: return "workspace missing or too small";
        case CKV_ERR_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
