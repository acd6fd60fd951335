// rebuild.hip -- centroids recomputed from the member lists, and their drift.
//
// rit.work post "CommunityKV long-context decoding": each community carries a
// centre (token-graph section); local assignments drift away from the best
// partition over long generations and the partition is refreshed from time to
// time (infrastructure section).  The rebuild is the plain definition of the
// centre -- the mean of the member keys -- and the drift compares the running
// means kept by the local update with it.
//
//   rebuild: mu_c[i] = fp32( (sum over members j of K[j][i], stored order, fp64) / size_c )
//   drift  : max over non-empty c of ||mu_c - ref_c||_2 / ||ref_c||_2  (per graph)
//
// Design: one wavefront per community.  Lane l owns elements l*E .. l*E+E-1 of the
// row (E = d/64), so every member row is one coalesced wave-wide load; the
// members of a batch are resolved to physical rows once (lane j: member j), their
// rows broadcast with a lane shuffle, and the loads of a 16-member batch are all
// issued before the element sums walk them in member order (which keeps the sum
// order of the definition).
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kRebuildWaves = 4;
constexpr int kRebuildBatch = 16;

template <typename T, int D>
__global__ __launch_bounds__(kRebuildWaves * kWave) void rebuild_kernel(
    const T *__restrict__ kc, const int32_t *__restrict__ page_table, int log2ps, int max_pages,
    int num_pages, const int32_t *__restrict__ seq_len, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_start, const int32_t *__restrict__ comm_size,
    const int32_t *__restrict__ members, int Cmax, int Hkv, int gpk, float *__restrict__ out,
    int32_t *__restrict__ err) {
    // blockIdx.y is the centroid set: the graph itself, or for the layer graph
    // (gpk = 0) one KV head's slice of the sequence's graph (set = b*Hkv + kvh)
    constexpr int E = D / kWave;  // elements per lane
    static_assert(E >= 1 && D % kWave == 0, "row split");
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int set = blockIdx.y;
    const int g = gpk == 0 ? set / Hkv : set;  // graph of the community arrays
    const int c = blockIdx.x * kRebuildWaves + w;
    const int C = min(num_comms[g], Cmax);
    if (c >= C) return;
    const int b = gpk == 0 ? g : g / (Hkv * gpk);
    const int kvh = gpk == 0 ? set % Hkv : (g / gpk) % Hkv;
    const int n = seq_len[b];
    const int sz = comm_size[(size_t)g * Cmax + c];
    const int st = comm_start[(size_t)g * Cmax + c];
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    bool bad = false;
    for (int m0 = 0; m0 < sz; m0 += kWave) {
        // lane j resolves member m0 + j to a physical row (-1: invalid, flagged)
        int row = -1;
        if (m0 + lane < sz) {
            const int pos = members[(size_t)st + m0 + lane];
            if (pos >= 0 && pos < n) {
                const int lp = pos >> log2ps;
                const int pg = lp < max_pages ? page_table[(size_t)b * max_pages + lp] : -1;
                if (pg >= 0 && pg < num_pages)
                    row = ((pg * Hkv + kvh) << log2ps) + (pos & ((1 << log2ps) - 1));
            }
            bad |= row < 0;
        }
        const int nb = min(kWave, sz - m0);
        for (int k0 = 0; k0 < nb; k0 += kRebuildBatch) {
            T v[kRebuildBatch][E];
            int rr[kRebuildBatch];
#pragma unroll
            for (int k = 0; k < kRebuildBatch; ++k) {
                rr[k] = __shfl(row, k0 + k);
                const T *src = kc + (size_t)(rr[k] < 0 ? 0 : rr[k]) * D + lane * E;
#pragma unroll
                for (int e = 0; e < E; ++e) v[k][e] = src[e];
            }
#pragma unroll
            for (int k = 0; k < kRebuildBatch; ++k) {
                if (k0 + k < nb && rr[k] >= 0) {
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = acc[e] + (double)to_f32(v[k][e]);
                }
            }
        }
    }
    if (__ballot(bad) && lane == 0) set_err(err, CKV_DEVERR_INDEX_RANGE);
    float *og = out + (size_t)set * (D / 4) * Cmax * 4;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = lane * E + e;
        og[((size_t)(i / 4) * Cmax + c) * 4 + i % 4] =
            sz > 0 ? (float)(acc[e] / (double)sz) : 0.f;
    }
}

// One workgroup per graph; thread t takes communities t, t+256, ...: in the
// community-interleaved layout lane c reads community c, so every wave-wide load is
// one contiguous 1 KiB line and no cross-lane sum is needed.
constexpr int kDriftThreads = 256;
// d4: float4 chunks of a centroid row (d/4, or Hkv*d/4 for the layer graph), a
// multiple of KC
__global__ __launch_bounds__(kDriftThreads) void drift_kernel(
    const float *__restrict__ cent, const float *__restrict__ ref,
    const int32_t *__restrict__ num_comms, const int32_t *__restrict__ comm_size, int Cmax,
    int d4, float *__restrict__ drift) {
    constexpr int KC = 8;  // float4 chunks in flight per operand
    __shared__ double s_worst[kDriftThreads / kWave];
    const int g = blockIdx.x;
    const int C = min(num_comms[g], Cmax);
    const float4 *cg = reinterpret_cast<const float4 *>(cent) + (size_t)g * d4 * Cmax;
    const float4 *rg = reinterpret_cast<const float4 *>(ref) + (size_t)g * d4 * Cmax;
    double worst = 0.0;
    for (int c = threadIdx.x; c < C; c += kDriftThreads) {
        if (comm_size[(size_t)g * Cmax + c] <= 0) continue;
        double num = 0.0, den = 0.0;
#pragma unroll 1
        for (int k0 = 0; k0 < d4; k0 += KC) {
            float4 a[KC], r[KC];
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                a[k] = cg[(size_t)(k0 + k) * Cmax + c];
                r[k] = rg[(size_t)(k0 + k) * Cmax + c];
            }
#pragma unroll
            for (int k = 0; k < KC; ++k) {
                const double ax[4] = {a[k].x, a[k].y, a[k].z, a[k].w};
                const double rx[4] = {r[k].x, r[k].y, r[k].z, r[k].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double diff = ax[e] - rx[e];
                    num += diff * diff;
                    den += rx[e] * rx[e];
                }
            }
        }
        const double rel = den > 0.0 ? sqrt(num) / sqrt(den) : sqrt(num);
        worst = rel > worst ? rel : worst;
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_xor(worst, off);
        worst = o > worst ? o : worst;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) s_worst[threadIdx.x / kWave] = worst;
    __syncthreads();
    if (threadIdx.x == 0) {
        double m = 0.0;
        for (int i = 0; i < kDriftThreads / kWave; ++i) m = s_worst[i] > m ? s_worst[i] : m;
        drift[g] = (float)m;
    }
}

hipError_t launch_rebuild(const Problem &p, const ckv_graphs &gr, const ckv_kv &kv, float *out,
                          int32_t *err, hipStream_t st) {
    const dim3 grid((p.Cmax + kRebuildWaves - 1) / kRebuildWaves,
                    p.layer() ? p.B * p.Hkv : p.NG());
#define CKV_REBUILD_CASE(TT, DT, DD)                                                           \
    if (p.dtype == DT && p.D == DD) {                                                          \
        hipExtLaunchKernelGGL((rebuild_kernel<TT, DD>), grid, dim3(kRebuildWaves * kWave), 0,  \
                              st, p.ev_start, p.ev_stop, 0, static_cast<const TT *>(kv.k),     \
                              kv.page_table, log2_pow2(kv.page_size), kv.max_pages_per_seq,    \
                              kv.num_pages, kv.seq_len, gr.num_comms, gr.comm_start,           \
                              gr.comm_size, gr.members, p.Cmax, p.Hkv, p.gpk, out, err);       \
        return hipGetLastError();                                                              \
    }
    CKV_REBUILD_CASE(bf16_t, CKV_DT_BF16, 128) CKV_REBUILD_CASE(bf16_t, CKV_DT_BF16, 64)
    CKV_REBUILD_CASE(float, CKV_DT_F32, 128) CKV_REBUILD_CASE(float, CKV_DT_F32, 64)
#undef CKV_REBUILD_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_drift(const Problem &p, const ckv_graphs &gr, const float *ref, float *drift,
                        hipStream_t st) {
    if ((p.cdim() / 4) % 8 != 0) return hipErrorInvalidValue;
    hipExtLaunchKernelGGL(drift_kernel, dim3(p.NG()), dim3(kDriftThreads), 0, st, p.ev_start,
                          p.ev_stop, 0, gr.centroids, ref, gr.num_comms, gr.comm_size, p.Cmax,
                          p.cdim() / 4, drift);
    return hipGetLastError();
}

}  // namespace ckv
