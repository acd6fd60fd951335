// update.hip -- constant-time local update of one community per graph.
//
// rit.work post "CommunityKV long-context decoding", token-graph section: a new
// token does not re-partition the graph; it is attached to a suitable neighbouring
// community and only that community's centre is updated, at a cost that depends on
// the model dimension and not on the context length.  The CommunityKV abstract
// (McKenna et al., 2026) calls it a constant-time local update rule.
//
// Per graph g of sequence b, n = seq_len[b]:
//   c* = argmin_{c in cand[g]} ||k_new - mu_c||^2   (fp64, element order, no FMA;
//        lower id on ties)
//   members[start_c* + size_c*] = n; size_c* += 1
//   mu_c* <- fp32( mu + (k_new - mu) / size )      (fp64 per element)
// once per (b, KV head): K/V row n <- k_new / v_new; then seq_len[b] += 1.
//
// One workgroup per sequence (so reading n and incrementing seq_len cannot race);
// its 4 wavefronts loop over the sequence's graphs.  Lane m owns candidate m and
// accumulates its distance sequentially in fp64 so the result matches a plain
// element-order sum bit for bit; the work is M*d + d per graph, independent of n.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kUpdThreads = 256;
constexpr int kUpdWaves = kUpdThreads / kWave;

#pragma clang fp contract(off)

template <typename T, int D>
__device__ double sq_dist(const T *__restrict__ kn, const float *__restrict__ cent, size_t g,
                          int Cmax, int c) {
    double s = 0.0;
    const float4 *cp = reinterpret_cast<const float4 *>(cent) + (size_t)g * (D / 4) * Cmax + c;
#pragma unroll 8
    for (int k = 0; k < D / 4; ++k) {
        const float4 v = cp[(size_t)k * Cmax];
        const float m4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double diff = (double)to_f32(kn[k * 4 + e]) - (double)m4[e];
            const double sq = diff * diff;
            s = s + sq;
        }
    }
    return s;
}

template <typename T, int D>
__global__ __launch_bounds__(kUpdThreads) void update_kernel(
    const T *__restrict__ k_new, const T *__restrict__ v_new, const int32_t *__restrict__ cand,
    int M, float *__restrict__ cent, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_start, int32_t *__restrict__ comm_size,
    const int32_t *__restrict__ comm_cap, int32_t *__restrict__ members, int Cmax, int Hkv,
    int gpk, T *__restrict__ kc, T *__restrict__ vc, const int32_t *__restrict__ page_table,
    int log2ps, int max_pages, int num_pages, int32_t *__restrict__ seq_len,
    int32_t *__restrict__ assigned, int32_t *__restrict__ err) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int n = seq_len[b];
    const int gps = Hkv * gpk;

    for (int gl = w; gl < gps; gl += kUpdWaves) {
        const size_t g = (size_t)b * gps + gl;
        const int kvh = gl / gpk;
        const T *kn = k_new + ((size_t)b * Hkv + kvh) * D;
        const int C = min(num_comms[g], Cmax);
        // candidate distances, one candidate per lane
        int c = -1;
        double dist = __builtin_inf();
        if (lane < M) {
            const int cc = cand[g * M + lane];
            if (cc >= 0 && cc < C) {
                c = cc;
                dist = sq_dist<T, D>(kn, cent, g, Cmax, cc);
            }
        }
        // wave argmin over (dist, id)
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const double od = __shfl_xor(dist, off);
            const int oc = __shfl_xor(c, off);
            const bool take = oc >= 0 && (c < 0 || od < dist || (od == dist && oc < c));
            if (take) {
                dist = od;
                c = oc;
            }
        }
        int best = c;
        int slot = -1;
        if (lane == 0) {
            if (best >= 0) {
                const int sz = comm_size[g * Cmax + best];
                if (sz < comm_cap[g * Cmax + best]) {
                    slot = sz;
                    members[(size_t)comm_start[g * Cmax + best] + sz] = n;
                    comm_size[g * Cmax + best] = sz + 1;
                } else {
                    set_err(err, CKV_DEVERR_CAPACITY);
                }
            }
            assigned[g] = slot >= 0 ? best : -1;
        }
        slot = __shfl(slot, 0);
        if (slot >= 0) {
            const double cnt = (double)(slot + 1);
            float *cp = cent + (size_t)g * (D / 4) * Cmax * 4;
            for (int i = lane; i < D; i += kWave) {
                float &mu = cp[((size_t)(i / 4) * Cmax + best) * 4 + i % 4];
                const double m0 = (double)mu;
                const double step = ((double)to_f32(kn[i]) - m0) / cnt;
                mu = (float)(m0 + step);
            }
        }
        // K/V row n, once per KV head
        if (gl % gpk == 0) {
            const int lp = n >> log2ps;
            const int pg = lp < max_pages ? page_table[(size_t)b * max_pages + lp] : -1;
            if (pg >= 0 && pg < num_pages) {
                const size_t ro = ((((size_t)pg * Hkv + kvh) << log2ps) + (n & ((1 << log2ps) - 1))) * D;
                const T *vn = v_new + ((size_t)b * Hkv + kvh) * D;
                for (int i = lane; i < D; i += kWave) {
                    kc[ro + i] = kn[i];
                    vc[ro + i] = vn[i];
                }
            } else if (lane == 0) {
                set_err(err, CKV_DEVERR_UNMAPPED_PAGE);
            }
        }
    }
    __syncthreads();
    if (tid == 0) seq_len[b] = n + 1;
}

template <typename T, int D>
static void launch_update_t(const Problem &p, const void *k_new, const void *v_new,
                            const int32_t *cand, int M, const ckv_graphs &gr, const ckv_kv &kv,
                            int32_t *assigned, int32_t *err, hipStream_t st) {
    int log2ps = 0;
    while ((1 << log2ps) < kv.page_size) ++log2ps;
    hipLaunchKernelGGL((update_kernel<T, D>), dim3(p.B), dim3(kUpdThreads), 0, st,
                       static_cast<const T *>(k_new), static_cast<const T *>(v_new), cand, M,
                       gr.centroids, gr.num_comms, gr.comm_start, gr.comm_size, gr.comm_cap,
                       gr.members, p.Cmax, p.Hkv, p.gpk, static_cast<T *>(kv.k),
                       static_cast<T *>(kv.v), kv.page_table, log2ps, kv.max_pages_per_seq,
                       kv.num_pages, kv.seq_len, assigned, err);
}

hipError_t launch_update(const Problem &p, const void *k_new, const void *v_new,
                         const int32_t *cand, int n_cand, const ckv_graphs &gr, const ckv_kv &kv,
                         int32_t *assigned, int32_t *err, hipStream_t st) {
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

// ---- workspace zero fill (a kernel, so it is safe inside captured graphs) ----------
__global__ void fill_zero_kernel(uint32_t *p, size_t words) {
    for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < words;
         t += (size_t)gridDim.x * blockDim.x)
        p[t] = 0u;
}

hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t st) {
    const size_t words = bytes / 4;
    if (words == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(256), dim3(256), 0, st,
                       static_cast<uint32_t *>(ptr), words);
    return hipGetLastError();
}

}  // namespace ckv
