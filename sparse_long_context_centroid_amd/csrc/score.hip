// score.hip -- centroid scoring (rit.work post "CommunityKV long-context decoding",
// token-graph section: the decode query is compared with the community centres
// only; granularity section: one graph may serve a whole group of heads).
//
//   s[g][c] = fp32( max_{h in heads(g)} (q_h . mu_{g,c}) * scale ),  -inf if empty.
//
// Design for gfx950: the centroids are stored community-interleaved,
// [NG][d/4][Cmax][4] fp32, so lane c of a wavefront owns centroid c and every
// wave-wide load is one contiguous 1 KiB line of 64 float4 -- no cross-lane
// reduction at all.  The inner products are accumulated in fp64 in element order:
// each product of a bf16/fp32 query element with an fp32 centroid element is exact
// in fp64, so the score is a deterministic function of the stored bytes.  Each
// workgroup widens the graph's queries to fp64 in LDS, [d/4][GH][4], so the
// per-element query values are wave-uniform broadcast reads.
#include <type_traits>
#include <utility>

#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

// One wavefront per workgroup: many small workgroups spread the 1 KiB centroid
// lines over every CU, and the query staging needs no workgroup barrier.
constexpr int kScoreThreads = 64;
// float4 chunks of a centroid in flight per lane: the next chunk's loads are
// issued before the current one is consumed (two chunks of registers).  A grid of
// at most one wave per SIMD streams 8-float4 chunks; a larger grid (several
// rounds of waves) takes 4-float4 chunks: its rounds overlap anyway, and a
// workgroup past its graph's community count (ragged batches) fetches half as
// much before it learns that and leaves.
constexpr int kScoreChunk = 8;
constexpr int kScoreChunkRounds = 4;

// v_fmac_f64 whose first factor comes from lane N of this lane's 16-lane row (DPP
// row_newbcast, a gfx90a+ 64-bit DPP control): acc = q[row lane N] * m + acc with
// one rounding, exactly as fma().  q must not be written by a VALU instruction in
// the two instructions before (the DPP read hazard; the compiler does not look
// inside inline asm): callers load q from LDS and issue s_nop 1 first.
template <int N>
__device__ __forceinline__ void fmac_row_bcast(double &acc, double q, double m) {
    asm volatile("v_fmac_f64_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                 : "+v"(acc)
                 : "v"(q), "v"(m), "n"(N));
}

// The FMAs of float4 step KK of a chunk, in element order and, per element, head
// order: query value v = (4*KK + c)*GH + h of the chunk sits in register v / 16 at
// row lane v % 16.
template <int GH, int NRP, int KK, int I>
__device__ __forceinline__ void score_fma(double (&acc)[GH], const double (&qr)[NRP],
                                          const double (&e)[4]) {
    constexpr int c = I / GH, h = I % GH, v = (4 * KK + c) * GH + h;
    fmac_row_bcast<v % 16>(acc[h], qr[v / 16], e[c]);
}
template <int GH, int NRP, int KK, int... I>
__device__ __forceinline__ void score_step(double (&acc)[GH], const double (&qr)[NRP],
                                           const float4 &f, std::integer_sequence<int, I...>) {
    const double e[4] = {f.x, f.y, f.z, f.w};
    asm volatile("s_nop 1");
    (score_fma<GH, NRP, KK, I>(acc, qr, e), ...);
}
template <int GH, int NRP, int KC, int... KK>
__device__ __forceinline__ void score_chunk(double (&acc)[GH], const double (&qr)[NRP],
                                            const float4 (&cur)[KC],
                                            std::integer_sequence<int, KK...>) {
    (score_step<GH, NRP, KK>(acc, qr, cur[KK], std::make_integer_sequence<int, 4 * GH>{}), ...);
}

// One workgroup = 64 consecutive communities of one graph, one per lane.  The
// graph's GH query rows are widened to fp64 once into LDS, in value order
// v = element*GH + head.  Per chunk of 4*KC elements each lane fetches 4*KC*GH/16
// of the chunk's values (lane p of a 16-lane row: values p, 16 + p, ...), and the
// FMAs take each value from its row lane with a DPP broadcast: the chunk costs a
// few LDS reads per lane instead of one broadcast LDS read per value.
template <typename T, int D, int GH, int KC>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const T *__restrict__ q, const float *__restrict__ cent, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_size, int Cmax, int Hq, int Hkv, int gpk, double scale,
    float *__restrict__ scores) {
    static_assert((D / 4) % KC == 0, "whole chunks");
    // lane j stages elements 4k..4k+3 of head h, k = j / GH, h = j % GH, with one
    // vector load
    constexpr int NQ = (D * GH / 4 + kScoreThreads - 1) / kScoreThreads;
    constexpr int NRP = 4 * KC * GH / 16;  // query registers per lane per chunk
    static_assert((4 * KC * GH) % 16 == 0, "whole 16-lane rows of query values");
    __shared__ double sq[D * GH];
    const int g = blockIdx.y;
    const int c0 = blockIdx.x * kScoreThreads + threadIdx.x;
    const int c = min(c0, Cmax - 1);
    const int G = Hq / Hkv;
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int h0 = kvh * G + (gpk == 1 ? 0 : g % gpk);
    // every load is issued before any result is waited for: the query chunk, the
    // first centroid chunk, the size and the community count
    using Q4 = typename std::conditional<sizeof(T) == 2, uint2, float4>::type;
    Q4 qraw[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int jq = min((int)threadIdx.x + j * kScoreThreads, D * GH / 4 - 1);
        qraw[j] = *reinterpret_cast<const Q4 *>(q + ((size_t)b * Hq + h0 + jq % GH) * D +
                                                (jq / GH) * 4);
    }
    const float4 *cp = reinterpret_cast<const float4 *>(cent) + (size_t)g * (D / 4) * Cmax + c;
    float4 cur[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) cur[k] = cp[(size_t)k * Cmax];
    const int sz = comm_size[(size_t)g * Cmax + c];
    const int C = min(num_comms[g], Cmax);
    // a workgroup wholly past the graph's count leaves now: only its first chunk
    // (issued before the count was known) was fetched in vain
    if ((int)(blockIdx.x * kScoreThreads) >= C) return;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        float e4[4];
        if constexpr (sizeof(T) == 2) {
            const uint2 w = reinterpret_cast<const uint2 &>(qraw[j]);
            e4[0] = bf16_lo(w.x);
            e4[1] = bf16_hi(w.x);
            e4[2] = bf16_lo(w.y);
            e4[3] = bf16_hi(w.y);
        } else {
            const float4 w = reinterpret_cast<const float4 &>(qraw[j]);
            e4[0] = w.x;
            e4[1] = w.y;
            e4[2] = w.z;
            e4[3] = w.w;
        }
        const int jq = min((int)threadIdx.x + j * kScoreThreads, D * GH / 4 - 1);
        const int k = jq / GH, h = jq % GH;
#pragma unroll
        for (int e = 0; e < 4; ++e) sq[(4 * k + e) * GH + h] = (double)e4[e];
    }
    __syncthreads();

    double acc[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) acc[h] = 0.0;
    // (kept rolled: unrolled, the compiler moves each load down to its use and the
    // chunks' round trips serialise)
#pragma unroll 1
    for (int k0 = 0; k0 < D / 4; k0 += KC) {
        float4 nxt[KC];
        const int kn = min(k0 + KC, D / 4 - KC);  // the last pass reloads a chunk, unused
#pragma unroll
        for (int k = 0; k < KC; ++k) nxt[k] = cp[(size_t)(kn + k) * Cmax];
        double qr[NRP];
        const double *qc = sq + 4 * k0 * GH + (threadIdx.x & 15);
#pragma unroll
        for (int j = 0; j < NRP; ++j) qr[j] = qc[16 * j];
        score_chunk<GH, NRP, KC>(acc, qr, cur, std::make_integer_sequence<int, KC>{});
#pragma unroll
        for (int k = 0; k < KC; ++k) cur[k] = nxt[k];
    }
    double best = acc[0];
#pragma unroll
    for (int h = 1; h < GH; ++h)
        if (acc[h] > best) best = acc[h];
    if (c0 < C) scores[(size_t)g * Cmax + c] = sz > 0 ? (float)(best * scale) : -__builtin_inff();
}

// The layer graph (one graph per sequence b, shared by every head; same post,
// granularity section): a community carries one centroid per KV head, and its
// score is the max over every query head h of q_h . mu_{c, kv head of h}:
//   s[b][c] = max over KV heads k of fp32( max_{h in group k} (q_h . mu_{b,k,c}) * scale ).
// The centroid of (b, k) is set b*Hkv + k of the interleaved layout.  A workgroup
// holds one wave per KV head (up to kLayerScoreWaves; more heads loop): each wave
// runs the lane-per-community stream above on its head's slice with its G queries
// in its own LDS rows, and the waves' maxima meet in LDS.  A workgroup covers CPW
// communities: 64, or 32 when the grid would otherwise leave most compute units
// idle (lanes 32-63 then repeat lanes 0-31: the same addresses in the same load
// instructions, so no extra bytes, and only lanes 0-31 write).
constexpr int kLayerScoreWaves = 8;

template <typename T, int D, int GH, int CPW>
__global__ __launch_bounds__(kLayerScoreWaves * kWave) void layer_score_kernel(
    const T *__restrict__ q, const float *__restrict__ cent, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_size, int Cmax, int Hq, int Hkv, double scale,
    float *__restrict__ scores) {
    constexpr int KC = kScoreChunk;
    static_assert((D / 4) % KC == 0, "whole chunks");
    constexpr int NQ = (D * GH / 4 + kWave - 1) / kWave;
    constexpr int NRP = 4 * KC * GH / 16;  // query registers per lane per chunk
    static_assert((4 * KC * GH) % 16 == 0, "whole 16-lane rows of query values");
    __shared__ double sq[kLayerScoreWaves][D * GH];
    __shared__ float s_best[kLayerScoreWaves][kWave];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    static_assert(CPW == 32 || CPW == 64, "communities per workgroup");
    const int c0 = blockIdx.x * CPW + (lane & (CPW - 1));
    const int c = min(c0, Cmax - 1);
    const int C = min(num_comms[b], Cmax);
    if ((int)(blockIdx.x * CPW) >= C) return;
    using Q4 = typename std::conditional<sizeof(T) == 2, uint2, float4>::type;
    double *sqw = sq[w];
    float best = -__builtin_inff();
#pragma unroll 1
    for (int kvh = w; kvh < Hkv; kvh += nw) {
        const int h0 = kvh * GH;
        Q4 qraw[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int jq = min(lane + j * kWave, D * GH / 4 - 1);
            qraw[j] = *reinterpret_cast<const Q4 *>(q + ((size_t)b * Hq + h0 + jq % GH) * D +
                                                    (jq / GH) * 4);
        }
        const float4 *cp = reinterpret_cast<const float4 *>(cent) +
                           ((size_t)b * Hkv + kvh) * (D / 4) * Cmax + c;
        float4 cur[KC];
#pragma unroll
        for (int k = 0; k < KC; ++k) cur[k] = cp[(size_t)k * Cmax];
        // this wave's previous head is no longer read (LDS rows private to the wave)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float e4[4];
            if constexpr (sizeof(T) == 2) {
                const uint2 wv = reinterpret_cast<const uint2 &>(qraw[j]);
                e4[0] = bf16_lo(wv.x);
                e4[1] = bf16_hi(wv.x);
                e4[2] = bf16_lo(wv.y);
                e4[3] = bf16_hi(wv.y);
            } else {
                const float4 wv = reinterpret_cast<const float4 &>(qraw[j]);
                e4[0] = wv.x;
                e4[1] = wv.y;
                e4[2] = wv.z;
                e4[3] = wv.w;
            }
            const int jq = min(lane + j * kWave, D * GH / 4 - 1);
            const int k = jq / GH, h = jq % GH;
#pragma unroll
            for (int e = 0; e < 4; ++e) sqw[(4 * k + e) * GH + h] = (double)e4[e];
        }
        __builtin_amdgcn_wave_barrier();
        double acc[GH];
#pragma unroll
        for (int h = 0; h < GH; ++h) acc[h] = 0.0;
#pragma unroll 1
        for (int k0 = 0; k0 < D / 4; k0 += KC) {
            float4 nxt[KC];
            const int kn = min(k0 + KC, D / 4 - KC);
#pragma unroll
            for (int k = 0; k < KC; ++k) nxt[k] = cp[(size_t)(kn + k) * Cmax];
            double qr[NRP];
            const double *qc = sqw + 4 * k0 * GH + (lane & 15);
#pragma unroll
            for (int j = 0; j < NRP; ++j) qr[j] = qc[16 * j];
            score_chunk<GH, NRP, KC>(acc, qr, cur, std::make_integer_sequence<int, KC>{});
#pragma unroll
            for (int k = 0; k < KC; ++k) cur[k] = nxt[k];
        }
        double m = acc[0];
#pragma unroll
        for (int h = 1; h < GH; ++h)
            if (acc[h] > m) m = acc[h];
        const float v = (float)(m * scale);
        best = v > best ? v : best;
    }
    s_best[w][lane] = best;
    __syncthreads();
    if (w == 0) {
        for (int i = 1; i < nw; ++i) best = s_best[i][lane] > best ? s_best[i][lane] : best;
        if (c0 < C && lane < CPW)
            scores[(size_t)b * Cmax + c] =
                comm_size[(size_t)b * Cmax + c] > 0 ? best : -__builtin_inff();
    }
}

// ---- layout helpers ---------------------------------------------------------------
__global__ void rows_to_interleaved_kernel(const float *__restrict__ rows, float *__restrict__ out,
                                           int NG, int Cmax, int D) {
    const size_t total = (size_t)NG * Cmax * D;
    for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
         t += (size_t)gridDim.x * blockDim.x) {
        const size_t g = t / ((size_t)Cmax * D);
        const int c = (int)((t / D) % Cmax);
        const int i = (int)(t % D);
        out[((g * (D / 4) + i / 4) * Cmax + c) * 4 + i % 4] = rows[t];
    }
}

__global__ void interleaved_to_rows_kernel(const float *__restrict__ cent, float *__restrict__ rows,
                                           int NG, int Cmax, int D) {
    const size_t total = (size_t)NG * Cmax * D;
    for (size_t t = blockIdx.x * (size_t)blockDim.x + threadIdx.x; t < total;
         t += (size_t)gridDim.x * blockDim.x) {
        const size_t g = t / ((size_t)Cmax * D);
        const int c = (int)((t / D) % Cmax);
        const int i = (int)(t % D);
        rows[t] = cent[((g * (D / 4) + i / 4) * Cmax + c) * 4 + i % 4];
    }
}

// ---- launchers ----------------------------------------------------------------------
template <typename T, int D, int GH>
static void launch_score_t(const Problem &p, const void *q, const ckv_graphs &gr, double scale,
                           float *scores, hipStream_t st) {
    const dim3 grid((p.Cmax + kScoreThreads - 1) / kScoreThreads, p.NG());
    const bool rounds = (long long)grid.x * grid.y > 4LL * device_cu_count();
    auto kernel = rounds ? score_kernel<T, D, GH, kScoreChunkRounds>
                         : score_kernel<T, D, GH, kScoreChunk>;
    hipExtLaunchKernelGGL(kernel, grid, dim3(kScoreThreads), 0, st, p.ev_start, p.ev_stop, 0,
                          static_cast<const T *>(q), gr.centroids, gr.num_comms, gr.comm_size,
                          p.Cmax, p.Hq, p.Hkv, p.gpk, scale, scores);
}

template <typename T, int D, int GH>
static void launch_layer_score_t(const Problem &p, const void *q, const ckv_graphs &gr,
                                 double scale, float *scores, hipStream_t st) {
    const int nw = p.Hkv < kLayerScoreWaves ? p.Hkv : kLayerScoreWaves;
    // narrow workgroups only for a grid of at most a quarter as many workgroups as
    // compute units (1 x 32K: 9 -> 18 workgroups, 9.0 -> 7.5 us); at 4 x 128K (132
    // workgroups) the repeated lanes' requests made it slower (10.4 -> 13.0 us)
    const bool narrow = 4LL * ((p.Cmax + kWave - 1) / kWave) * p.B <= device_cu_count();
    auto kernel = narrow ? layer_score_kernel<T, D, GH, 32> : layer_score_kernel<T, D, GH, 64>;
    const int cpw = narrow ? 32 : 64;
    hipExtLaunchKernelGGL(kernel, dim3((p.Cmax + cpw - 1) / cpw, p.B), dim3(nw * kWave), 0, st,
                          p.ev_start, p.ev_stop, 0,
                          static_cast<const T *>(q), gr.centroids, gr.num_comms, gr.comm_size,
                          p.Cmax, p.Hq, p.Hkv, scale, scores);
}

hipError_t launch_score(const Problem &p, const void *q, const ckv_graphs &gr, double scale,
                        float *scores, hipStream_t st) {
    if (p.layer()) {
        const int G = p.G();
#define CKV_LSCORE_CASE(TT, DT, DD, HH)                                                        \
        if (p.dtype == DT && p.D == DD && G == HH) {                                           \
            launch_layer_score_t<TT, DD, HH>(p, q, gr, scale, scores, st);                     \
            return hipGetLastError();                                                          \
        }
        CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 128, 1) CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 128, 2)
        CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 128, 4) CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 128, 8)
        CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 64, 1) CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 64, 2)
        CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 64, 4) CKV_LSCORE_CASE(bf16_t, CKV_DT_BF16, 64, 8)
        CKV_LSCORE_CASE(float, CKV_DT_F32, 128, 1) CKV_LSCORE_CASE(float, CKV_DT_F32, 128, 2)
        CKV_LSCORE_CASE(float, CKV_DT_F32, 128, 4) CKV_LSCORE_CASE(float, CKV_DT_F32, 128, 8)
        CKV_LSCORE_CASE(float, CKV_DT_F32, 64, 1) CKV_LSCORE_CASE(float, CKV_DT_F32, 64, 2)
        CKV_LSCORE_CASE(float, CKV_DT_F32, 64, 4) CKV_LSCORE_CASE(float, CKV_DT_F32, 64, 8)
#undef CKV_LSCORE_CASE
        return hipErrorInvalidValue;
    }
    const int GH = p.heads_per_graph();
#define CKV_SCORE_CASE(TT, DT, DD, HH)                                                         \
    if (p.dtype == DT && p.D == DD && GH == HH) {                                              \
        launch_score_t<TT, DD, HH>(p, q, gr, scale, scores, st);                               \
        return hipGetLastError();                                                              \
    }
    CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 128, 1) CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 128, 2)
    CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 128, 4) CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 128, 8)
    CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 64, 1) CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 64, 2)
    CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 64, 4) CKV_SCORE_CASE(bf16_t, CKV_DT_BF16, 64, 8)
    CKV_SCORE_CASE(float, CKV_DT_F32, 128, 1) CKV_SCORE_CASE(float, CKV_DT_F32, 128, 2)
    CKV_SCORE_CASE(float, CKV_DT_F32, 128, 4) CKV_SCORE_CASE(float, CKV_DT_F32, 128, 8)
    CKV_SCORE_CASE(float, CKV_DT_F32, 64, 1) CKV_SCORE_CASE(float, CKV_DT_F32, 64, 2)
    CKV_SCORE_CASE(float, CKV_DT_F32, 64, 4) CKV_SCORE_CASE(float, CKV_DT_F32, 64, 8)
#undef CKV_SCORE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_rows_to_interleaved(const Problem &p, const float *rows, float *cent,
                                      hipStream_t st) {
    hipLaunchKernelGGL(rows_to_interleaved_kernel, dim3(1024), dim3(256), 0, st, rows, cent,
                       p.NG(), p.Cmax, p.cdim());
    return hipGetLastError();
}

hipError_t launch_interleaved_to_rows(const Problem &p, const float *cent, float *rows,
                                      hipStream_t st) {
    hipLaunchKernelGGL(interleaved_to_rows_kernel, dim3(1024), dim3(256), 0, st, cent, rows,
                       p.NG(), p.Cmax, p.cdim());
    return hipGetLastError();
}

}  // namespace ckv
