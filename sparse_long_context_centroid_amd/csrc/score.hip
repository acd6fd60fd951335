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
// in fp64, so the score is a deterministic function of the stored bytes.  The
// group's queries are staged once per step as fp64 in [g][d/4][GH][4] order so the
// per-element query values are wave-uniform and are fetched with scalar loads.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kScoreThreads = 256;

// One workgroup = 256 consecutive communities of one graph, one per lane.  The
// graph's GH query rows are widened to fp64 once into LDS, laid out [d/4][GH][4]
// so that each step's 4*GH values are one contiguous broadcast read.
template <typename T, int D, int GH>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    const T *__restrict__ q, const float *__restrict__ cent, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_size, int Cmax, int Hq, int Hkv, int gpk, double scale,
    float *__restrict__ scores) {
    __shared__ double sq[D * GH];
    const int g = blockIdx.y;
    const int C = min(num_comms[g], Cmax);
    const int base = blockIdx.x * kScoreThreads;
    if (base >= C) return;
    const int c = base + threadIdx.x;
    const bool live = c < C;
    const int G = Hq / Hkv;
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int h0 = kvh * G + (gpk == 1 ? 0 : g % gpk);
    // Stage the graph's queries in LDS before the centroid stream starts: a query
    // load issued behind 32 KiB of centroid requests per wave would wait for the
    // whole stream.
    for (int t = threadIdx.x; t < D * GH; t += kScoreThreads) {
        const int k = t / (GH * 4), h = (t / 4) % GH, e = t % 4;
        sq[t] = (double)to_f32(q[((size_t)b * Hq + h0 + h) * D + k * 4 + e]);
    }
    __syncthreads();
    const float4 *cp = reinterpret_cast<const float4 *>(cent) + (size_t)g * (D / 4) * Cmax +
                       (live ? c : base);
    float4 v[D / 4];
#pragma unroll
    for (int k = 0; k < D / 4; ++k) v[k] = cp[(size_t)k * Cmax];
    const int sz = live ? comm_size[(size_t)g * Cmax + c] : 0;

    double acc[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) acc[h] = 0.0;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) {
        const double e0 = v[k].x, e1 = v[k].y, e2 = v[k].z, e3 = v[k].w;
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            const double *qq = sq + (k * GH + h) * 4;
            acc[h] = fma(qq[0], e0, acc[h]);
            acc[h] = fma(qq[1], e1, acc[h]);
            acc[h] = fma(qq[2], e2, acc[h]);
            acc[h] = fma(qq[3], e3, acc[h]);
        }
    }
    double best = acc[0];
#pragma unroll
    for (int h = 1; h < GH; ++h)
        if (acc[h] > best) best = acc[h];
    if (live) scores[(size_t)g * Cmax + c] = sz > 0 ? (float)(best * scale) : -__builtin_inff();
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
    hipLaunchKernelGGL((score_kernel<T, D, GH>),
                       dim3((p.Cmax + kScoreThreads - 1) / kScoreThreads, p.NG()),
                       dim3(kScoreThreads), 0, st, static_cast<const T *>(q), gr.centroids,
                       gr.num_comms, gr.comm_size, p.Cmax, p.Hq, p.Hkv, p.gpk, scale, scores);
}

hipError_t launch_score(const Problem &p, const void *q, const ckv_graphs &gr, double scale,
                        float *scores, hipStream_t st) {
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
                       p.NG(), p.Cmax, p.D);
    return hipGetLastError();
}

hipError_t launch_interleaved_to_rows(const Problem &p, const float *cent, float *rows,
                                      hipStream_t st) {
    hipLaunchKernelGGL(interleaved_to_rows_kernel, dim3(1024), dim3(256), 0, st, cent, rows,
                       p.NG(), p.Cmax, p.D);
    return hipGetLastError();
}

}  // namespace ckv
