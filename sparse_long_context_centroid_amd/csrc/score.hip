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

// q [B][Hq][d] (T) -> q64 [NG][d/4][GH][4] fp64; GH = heads per graph.
template <typename T>
__global__ __launch_bounds__(256) void stage_query_kernel(const T *__restrict__ q,
                                                          double *__restrict__ q64, int Hq,
                                                          int Hkv, int gpk, int D, int GH) {
    const int g = blockIdx.x;
    const int G = Hq / Hkv;
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int j = g % gpk;
    const int h0 = kvh * G + (gpk == 1 ? 0 : j);
    const int total = GH * D;
    for (int t = threadIdx.x; t < total; t += blockDim.x) {
        // destination order: k = i/4, h, e = i%4
        const int k = t / (GH * 4);
        const int h = (t / 4) % GH;
        const int e = t % 4;
        const int i = k * 4 + e;
        q64[(size_t)g * total + t] = (double)to_f32(q[((size_t)b * Hq + h0 + h) * D + i]);
    }
}

template <int D, int GH>
__global__ __launch_bounds__(64) void score_kernel(const double *__restrict__ q64,
                                                   const float *__restrict__ cent,
                                                   const int32_t *__restrict__ num_comms,
                                                   const int32_t *__restrict__ comm_size,
                                                   int Cmax, double scale,
                                                   float *__restrict__ scores) {
    const int g = blockIdx.y;
    const int C = min(num_comms[g], Cmax);
    const int c = blockIdx.x * kWave + threadIdx.x;
    if (blockIdx.x * kWave >= C) return;
    const bool live = c < C;
    const int cc = live ? c : 0;
    const float4 *cp = reinterpret_cast<const float4 *>(cent) + (size_t)g * (D / 4) * Cmax + cc;
    const double *qg = q64 + (size_t)g * (D / 4) * GH * 4;

    float4 v[D / 4];
#pragma unroll
    for (int k = 0; k < D / 4; ++k) v[k] = cp[(size_t)k * Cmax];

    double acc[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) acc[h] = 0.0;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) {
        const double e0 = v[k].x, e1 = v[k].y, e2 = v[k].z, e3 = v[k].w;
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            const double *qq = qg + (k * GH + h) * 4;
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
    if (live) {
        const int sz = comm_size[(size_t)g * Cmax + c];
        scores[(size_t)g * Cmax + c] = sz > 0 ? (float)(best * scale) : -__builtin_inff();
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
hipError_t launch_stage_query(const Problem &p, const void *q, double *q64, hipStream_t st) {
    const int GH = p.heads_per_graph();
    if (p.dtype == CKV_DT_BF16)
        hipLaunchKernelGGL(stage_query_kernel<bf16_t>, dim3(p.NG()), dim3(256), 0, st,
                           static_cast<const bf16_t *>(q), q64, p.Hq, p.Hkv, p.gpk, p.D, GH);
    else
        hipLaunchKernelGGL(stage_query_kernel<float>, dim3(p.NG()), dim3(256), 0, st,
                           static_cast<const float *>(q), q64, p.Hq, p.Hkv, p.gpk, p.D, GH);
    return hipGetLastError();
}

template <int D, int GH>
static void launch_score_t(const Problem &p, const double *q64, const ckv_graphs &gr,
                           double scale, float *scores, hipStream_t st) {
    hipLaunchKernelGGL((score_kernel<D, GH>), dim3(p.Cmax / kWave, p.NG()), dim3(kWave), 0, st,
                       q64, gr.centroids, gr.num_comms, gr.comm_size, p.Cmax, scale, scores);
}

hipError_t launch_score(const Problem &p, const double *q64, const ckv_graphs &gr, double scale,
                        float *scores, hipStream_t st) {
    const int GH = p.heads_per_graph();
#define CKV_SCORE_CASE(DD, HH) \
    if (p.D == DD && GH == HH) { launch_score_t<DD, HH>(p, q64, gr, scale, scores, st); return hipGetLastError(); }
    CKV_SCORE_CASE(64, 1) CKV_SCORE_CASE(64, 2) CKV_SCORE_CASE(64, 4) CKV_SCORE_CASE(64, 8)
    CKV_SCORE_CASE(128, 1) CKV_SCORE_CASE(128, 2) CKV_SCORE_CASE(128, 4) CKV_SCORE_CASE(128, 8)
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
