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

// The layer graph: one graph per sequence b, whose centroid rows hold one d-slice
// per KV head (E = Hkv*d values, KV head after KV head).  The new token's key row
// is the concatenation of its Hkv keys; it joins the candidate whose row is
// nearest in squared L2 over all E values, accumulated per KV head (each slice
// summed in fp64 in element order, then the slices in head order; lower id on
// equal distance); that community's whole row moves to the running mean, and K/V
// row n is written in every KV head.
//
// One workgroup per sequence: k_new is widened to fp64 in LDS and the candidates'
// rows are staged there by the whole workgroup (every load in flight at once);
// one thread per (candidate, slice) sums that slice, and the first wave's lanes
// 0..M-1 add their candidate's slices in order.  LDS: E doubles plus M rows of
// E+4 floats (the host checks the size).
constexpr int kLayerUpdThreads = 256;
constexpr int kLayerUpdMaxHeads = 32;  // KV heads (slices) per row
inline size_t layer_update_lds(int E, int M) {
    return (size_t)E * sizeof(double) + (size_t)M * (E + 4) * sizeof(float);
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
#pragma clang fp contract(off)
    extern __shared__ __align__(16) unsigned char s_raw[];
    __shared__ int s_best, s_slot, s_new;
    __shared__ int s_cl[CKV_MAX_CAND];
    __shared__ double s_part[CKV_MAX_CAND * kLayerUpdMaxHeads];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int E = Hkv * D, E4 = E / 4, CS = E + 4;
    double *kn64 = reinterpret_cast<double *>(s_raw);
    float *lc = reinterpret_cast<float *>(kn64 + E);
    const int n = seq_len[b];
    const int C = min(num_comms[b], Cmax);
    const T *kn = k_new + (size_t)b * E;
    const T *vn = v_new + (size_t)b * E;
    // round 1: the candidate ids (to LDS) and k_new (widened to fp64)
    if (tid < M) {
        const int cc = cand[(size_t)b * M + tid];
        s_cl[tid] = (cc >= 0 && cc < C) ? cc : -1;
    }
    {
        // E / 256 elements per thread, loaded together (clamped indexes: a loop of
        // load-then-store would wait for each load in turn)
        constexpr int kMaxPer = 16;  // E <= 4096
        T kv[kMaxPer];
#pragma unroll
        for (int r = 0; r < kMaxPer; ++r) kv[r] = kn[min(tid + r * kLayerUpdThreads, E - 1)];
#pragma unroll
        for (int r = 0; r < kMaxPer; ++r)
            if (tid + r * kLayerUpdThreads < E)
                kn64[tid + r * kLayerUpdThreads] = (double)to_f32(kv[r]);
    }
    __syncthreads();
    // round 2: the candidates' rows, element 4*k4 .. +3 of community c at float4
    // (b*E4 + k4)*Cmax + c, 8 loads per thread in flight per pass
    const float4 *c4 = reinterpret_cast<const float4 *>(cent) + (size_t)b * E4 * Cmax;
    const int total = M * E4;
    for (int t0 = 0; t0 < total; t0 += 8 * kLayerUpdThreads) {
        float4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = min(t0 + k * kLayerUpdThreads + tid, total - 1);
            v[k] = c4[(size_t)(t % E4) * Cmax + max(s_cl[t / E4], 0)];
        }
        __builtin_amdgcn_sched_barrier(0);
        // stores at the same clamped slots (past the end: a repeat of the last
        // slot's own value), so no store waits behind a branch
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int t = min(t0 + k * kLayerUpdThreads + tid, total - 1);
            *reinterpret_cast<float4 *>(lc + (t / E4) * CS + 4 * (t % E4)) = v[k];
        }
    }
    __syncthreads();
    // one (candidate, KV head slice) per thread: the slice's squared distance in
    // element order, 4 at a time from LDS
    for (int pr = tid; pr < M * Hkv; pr += kLayerUpdThreads) {
        const int sl = pr / Hkv, kh = pr % Hkv;
        const float4 *mu4 = reinterpret_cast<const float4 *>(lc + sl * CS + kh * D);
        const double2 *k2 = reinterpret_cast<const double2 *>(kn64 + kh * D);
        double s = 0.0;
#pragma unroll 8
        for (int i4 = 0; i4 < D / 4; ++i4) {
            const float4 m = mu4[i4];
            const double2 ka = k2[2 * i4], kb = k2[2 * i4 + 1];
            const double d0 = ka.x - (double)m.x, d1 = ka.y - (double)m.y;
            const double d2 = kb.x - (double)m.z, d3 = kb.y - (double)m.w;
            const double q0 = d0 * d0, q1 = d1 * d1, q2 = d2 * d2, q3 = d3 * d3;
            s = s + q0;
            s = s + q1;
            s = s + q2;
            s = s + q3;
        }
        s_part[pr] = s;
    }
    __syncthreads();
    if (tid < kWave) {
        const int lane = tid;
        const int c = lane < M ? s_cl[lane] : -1;
        double dist = __builtin_inf();
        if (c >= 0) {
            double s = 0.0;
            for (int kh = 0; kh < Hkv; ++kh) s = s + s_part[lane * Hkv + kh];
            dist = s;
        }
        int best = c, slot = c >= 0 ? lane : -1;
        double bd = dist;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double od = __shfl_xor(bd, off);
            const int oc = __shfl_xor(best, off);
            const int os = __shfl_xor(slot, off);
            if (oc >= 0 && (best < 0 || od < bd || (od == bd && oc < best))) {
                bd = od;
                best = oc;
                slot = os;
            }
        }
        if (lane == 0) {
            int slot_new = -1;
            if (best >= 0) {
                const size_t gc = (size_t)b * Cmax + best;
                const int sz = comm_size[gc];
                if (sz < comm_cap[gc]) {
                    members[(size_t)comm_start[gc] + sz] = n;
                    comm_size[gc] = sz + 1;
                    slot_new = sz;
                } else {
                    set_err(err, CKV_DEVERR_CAPACITY);
                }
            }
            assigned[b] = slot_new >= 0 ? best : -1;
            s_best = best;
            s_slot = slot;
            s_new = slot_new;
        }
    }
    __syncthreads();
    const int best = s_best, slot_new = s_new;
    if (slot_new >= 0) {
        // running mean of the winner's whole row, from its LDS copy
        const double cnt = (double)(slot_new + 1);
        const float *mu = lc + s_slot * CS;
        for (int i = tid; i < E; i += kLayerUpdThreads) {
            const double m0 = (double)mu[i];
            const double step = (kn64[i] - m0) / cnt;
            cent[(((size_t)b * E4 + i / 4) * Cmax + best) * 4 + i % 4] = (float)(m0 + step);
        }
    }
    // K/V row n in every KV head
    const int lp = n >> log2ps;
    const int pg = lp < max_pages ? page_table[(size_t)b * max_pages + lp] : -1;
    if (pg >= 0 && pg < num_pages) {
        for (int i = tid; i < E; i += kLayerUpdThreads) {
            const int kvh = i / D, e = i % D;
            const size_t row =
                (((size_t)pg * Hkv + kvh) << log2ps) + (n & ((1 << log2ps) - 1));
            kc[row * D + e] = kn[i];
            vc[row * D + e] = vn[i];
        }
    } else if (tid == 0) {
        set_err(err, CKV_DEVERR_UNMAPPED_PAGE);
    }
    if (bump) {
        __syncthreads();
        if (tid == 0) seq_len[b] = n + 1;
    }
}

template <typename T, int D>
static void launch_layer_update_t(const Problem &p, const void *k_new, const void *v_new,
                                  const int32_t *cand, int M, const ckv_graphs &gr,
                                  const ckv_kv &kv, int32_t *assigned, int32_t *err, bool bump,
                                  hipStream_t st) {
    hipLaunchKernelGGL((layer_update_kernel<T, D>), dim3(p.B), dim3(kLayerUpdThreads),
                       layer_update_lds(p.cdim(), M), st, static_cast<const T *>(k_new),
                       static_cast<const T *>(v_new), cand, M, gr.centroids, gr.num_comms,
                       gr.comm_start, gr.comm_size, gr.comm_cap, gr.members, p.Cmax, p.Hkv,
                       static_cast<T *>(kv.k), static_cast<T *>(kv.v), kv.page_table,
                       log2_pow2(kv.page_size), kv.max_pages_per_seq, kv.num_pages, kv.seq_len,
                       bump ? 1 : 0, assigned, err);
}

bool layer_update_fits(const Problem &p, int n_cand) {
    return p.cdim() <= 4096 && p.Hkv <= kLayerUpdMaxHeads &&
           layer_update_lds(p.cdim(), n_cand) <= 65536;
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
