// update.hip -- the standalone local-update call.
//
// Per graph g of sequence b, n = seq_len[b] (rule in update_rule.h):
//   c* = nearest candidate centroid to k_new; members[...] <- n; size += 1;
//   centroid <- running mean; once per (b, KV head) K/V row n <- k_new / v_new;
// and finally seq_len[b] += 1.
//
// One workgroup per sequence, so reading n and incrementing seq_len cannot race;
// one wavefront per graph of the sequence (looping when there are more than 8).
// The fused decode step runs the same update in extra workgroups of the attention
// launch instead (attention reads neither centroids, member lists nor row n).
#include "ckv_device.h"
#include "ckv_internal.h"
#include "update_rule.h"

namespace ckv {

template <typename T, int D>
__global__ __launch_bounds__(512) void update_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, const int32_t *__restrict__ cand,
    int M, float *__restrict__ cent, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_start, int32_t *__restrict__ comm_size,
    const int32_t *__restrict__ comm_cap, int32_t *__restrict__ members, int Cmax, int Hkv,
    int gpk, T *__restrict__ kc, T *__restrict__ vc, const int32_t *__restrict__ page_table,
    int log2ps, int max_pages, int num_pages, int32_t *__restrict__ seq_len,
    int32_t *__restrict__ assigned, int32_t *__restrict__ err) {
    __shared__ __align__(16) float s_rows[8 * kUpdLdsFloats(D)];
    sequence_update<T, D>(blockIdx.x, k_new, v_new, cand, M, cent, num_comms, comm_start,
                          comm_size, comm_cap, members, Cmax, Hkv, gpk, kc, vc, page_table,
                          log2ps, max_pages, num_pages, seq_len, assigned, err, s_rows);
}

template <typename T, int D>
static void launch_update_t(const Problem &p, const void *k_new, const void *v_new,
                            const int32_t *cand, int M, const ckv_graphs &gr, const ckv_kv &kv,
                            int32_t *assigned, int32_t *err, hipStream_t st) {
    const int nw = p.graphs_per_seq() < 8 ? p.graphs_per_seq() : 8;
    hipLaunchKernelGGL((update_kernel<T, D>), dim3(p.B), dim3(nw * kWave), 0, st,
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), cand, M,
                       gr.centroids, gr.num_comms, gr.comm_start, gr.comm_size, gr.comm_cap,
                       gr.members, p.Cmax, p.Hkv, p.gpk, static_cast<T *>(kv.k),
                       static_cast<T *>(kv.v), kv.page_table, log2_pow2(kv.page_size),
                       kv.max_pages_per_seq, kv.num_pages, kv.seq_len, assigned, err);
}

template <typename T, int D>
__global__ __launch_bounds__(kLayerUpdThreads) void layer_update_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, const int32_t *__restrict__ cand,
    int M, float *__restrict__ cent, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_start, int32_t *__restrict__ comm_size,
    const int32_t *__restrict__ comm_cap, int32_t *__restrict__ members, int Cmax, int Hkv,
    T *__restrict__ kc, T *__restrict__ vc, const int32_t *__restrict__ page_table, int log2ps,
    int max_pages, int num_pages, int32_t *__restrict__ seq_len, int bump,
    int32_t *__restrict__ assigned, int32_t *__restrict__ err) {
    extern __shared__ __align__(16) unsigned char s_raw[];
    layer_update_seq<T, D>(blockIdx.x, k_new, v_new, cand, M, cent, num_comms, comm_start,
                           comm_size, comm_cap, members, Cmax, Hkv, kc, vc, page_table, log2ps,
                           max_pages, num_pages, seq_len, bump, assigned, err, s_raw);
}

template <typename T, int D>
static void launch_layer_update_t(const Problem &p, const void *k_new, const void *v_new,
                                  const int32_t *cand, int M, const ckv_graphs &gr,
                                  const ckv_kv &kv, int32_t *assigned, int32_t *err, bool bump,
                                  hipStream_t st) {
    hipLaunchKernelGGL((layer_update_kernel<T, D>), dim3(p.B), dim3(kLayerUpdThreads),
                       layer_update_lds(p.cdim(), M, p.Hkv), st, static_cast<const T *>(k_new),
                       static_cast<const T *>(v_new), cand, M, gr.centroids, gr.num_comms,
                       gr.comm_start, gr.comm_size, gr.comm_cap, gr.members, p.Cmax, p.Hkv,
                       static_cast<T *>(kv.k), static_cast<T *>(kv.v), kv.page_table,
                       log2_pow2(kv.page_size), kv.max_pages_per_seq, kv.num_pages, kv.seq_len,
                       bump ? 1 : 0, assigned, err);
}

bool layer_update_fits(const Problem &p, int n_cand) {
    return p.cdim() <= 4096 && p.Hkv <= kLayerUpdMaxHeads &&
           layer_update_lds(p.cdim(), n_cand, p.Hkv) <= 65536;
}

hipError_t launch_layer_update(const Problem &p, const void *k_new, const void *v_new,
                               const int32_t *cand, int n_cand, const ckv_graphs &gr,
                               const ckv_kv &kv, int32_t *assigned, int32_t *err, bool bump,
                               hipStream_t st) {
    if (!layer_update_fits(p, n_cand)) return hipErrorInvalidValue;
#define CKV_LUPD_CASE(TT, DT, DD)                                                              \
    if (p.dtype == DT && p.D == DD) {                                                          \
        launch_layer_update_t<TT, DD>(p, k_new, v_new, cand, n_cand, gr, kv, assigned, err,    \
                                      bump, st);                                               \
        return hipGetLastError();                                                              \
    }
    CKV_LUPD_CASE(bf16_t, CKV_DT_BF16, 128) CKV_LUPD_CASE(bf16_t, CKV_DT_BF16, 64)
    CKV_LUPD_CASE(float, CKV_DT_F32, 128) CKV_LUPD_CASE(float, CKV_DT_F32, 64)
#undef CKV_LUPD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_update(const Problem &p, const void *k_new, const void *v_new,
                         const int32_t *cand, int n_cand, const ckv_graphs &gr, const ckv_kv &kv,
                         int32_t *assigned, int32_t *err, hipStream_t st) {
    if (p.layer())
        return launch_layer_update(p, k_new, v_new, cand, n_cand, gr, kv, assigned, err, true,
                                   st);
#define CKV_UPD_CASE(TT, DT, DD)                                                               \
    if (p.dtype == DT && p.D == DD) {                                                          \
        launch_update_t<TT, DD>(p, k_new, v_new, cand, n_cand, gr, kv, assigned, err, st);     \
        return hipGetLastError();                                                              \
    }
    CKV_UPD_CASE(bf16_t, CKV_DT_BF16, 128) CKV_UPD_CASE(bf16_t, CKV_DT_BF16, 64)
    CKV_UPD_CASE(float, CKV_DT_F32, 128) CKV_UPD_CASE(float, CKV_DT_F32, 64)
#undef CKV_UPD_CASE
    return hipErrorInvalidValue;
}

}  // namespace ckv
