// attn.hip -- indexed split-K flash-decode over the selected tokens.
//
// rit.work post "CommunityKV long-context decoding", token-graph section: the
// chosen communities are loaded from the full (never evicted) KV cache and
// attention is computed exactly over that reduced token set.  For every query head
// h of sequence b, with graph g(h) and index list I_g:
//   o_h = sum_{j in I_g} exp(z_j - max z) V_j / sum_{j in I_g} exp(z_j - max z),
//   z_j = scale * q_h . K_j.
//
// gfx950 design (VALU path):
// * One workgroup = 4 wavefronts = 4*16*RPW consecutive entries (256 for bf16
//   d=128) of one
//   graph's index list; grid = (max splits, NG); workgroups past the list exit.
// * A K or V row (d*elem bytes = 256 B for bf16 d=128 or fp32 d=64) is read by
//   LPR = row_bytes/16 lanes with one 16-byte load each, so one wave-wide load
//   gathers 64/LPR whole rows (1 KiB) -- coalesced row gathers through the page
//   table.  All 2*(64/RPW) loads of a wave are issued before any arithmetic.
// * Logits are reduced over the LPR lanes of a row with DPP adds; softmax runs in
//   the log2 domain in fp32; each wave keeps (m, l, acc) per head, the 4 waves are
//   merged in LDS and the workgroup writes one partial (m, l, acc[d]) per head.
// * The last workgroup of a graph to finish (device-scope arrival counter) merges
//   the partials with the log-sum-exp rule and writes the fp32 output, then resets
//   the counter -- no second launch.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int EPL>
__device__ __forceinline__ void unpack(const uint4 &u, float (&x)[EPL]);

template <>
__device__ __forceinline__ void unpack<bf16_t, 8>(const uint4 &u, float (&x)[8]) {
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x);
    x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z);
    x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void unpack<float, 4>(const uint4 &u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x); x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z); x[3] = __uint_as_float(u.w);
}

template <typename T, int D, int GH>
__global__ __launch_bounds__(256) void attn_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const int32_t *__restrict__ page_table, int log2ps, int max_pages, int num_pages,
    const int32_t *__restrict__ seq_len, const int32_t *__restrict__ idx, int idx_stride,
    const int32_t *__restrict__ idx_len, int Hq, int Hkv, int gpk, float scale_log2,
    float *__restrict__ out, uint32_t *__restrict__ counters, float *__restrict__ part,
    int max_splits, int32_t *__restrict__ err) {
    constexpr int EPL = 16 / sizeof(T);      // row elements per lane
    constexpr int LPR = D / EPL;             // lanes per row
    constexpr int RPW = kWave / LPR;         // rows per wave-wide load
    constexpr int NLD = kAttnLoads;          // loads per wave for K (and for V)
    constexpr int kTokPerWave = NLD * RPW;
    constexpr int kChunk = kTokPerWave * kAttnWaves;
    static_assert(kChunk == attn_chunk(D, sizeof(T)), "chunk");
    static_assert(LPR >= 1 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row split");

    __shared__ float s_m[kAttnWaves][GH];
    __shared__ float s_l[kAttnWaves][GH];
    __shared__ float s_acc[kAttnWaves][GH][D];
    __shared__ int s_last;

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int G = Hq / Hkv;
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int h0 = kvh * G + (gpk == 1 ? 0 : g % gpk);
    const int len = min(idx_len[g], idx_stride);
    const int nsplit = (len + kChunk - 1) / kChunk;

    if (len <= 0) {
        if (split == 0)
            for (int t = tid; t < GH * D; t += blockDim.x)
                out[((size_t)b * Hq + h0 + t / D) * D + t % D] = 0.f;
        return;
    }
    if (split >= nsplit) return;

    const int n = seq_len[b];
    const int ls = lane % LPR;  // slice of the row this lane reads
    const int rs = lane / LPR;  // row slot inside a wave-wide load

    // query slice, pre-scaled into the log2 domain
    float qv[GH][EPL];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        const uint4 u = *reinterpret_cast<const uint4 *>(q + ((size_t)b * Hq + h0 + h) * D + ls * EPL);
        float x[EPL];
        unpack<T, EPL>(u, x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[h][e] = x[e] * scale_log2;
    }

    // this wave's tokens: entries t0 .. t0+63 of the list
    const int t0 = split * kChunk + w * kTokPerWave;
    const int te = t0 + lane;
    size_t rowoff = 0;
    bool ok = false;
    if (te < len) {
        const int pos = idx[(size_t)g * idx_stride + te];
        if (pos >= 0 && pos < n) {
            const int lp = pos >> log2ps;
            const int pg = lp < max_pages ? page_table[(size_t)b * max_pages + lp] : -1;
            if (pg >= 0 && pg < num_pages) {
                rowoff = ((((size_t)pg * Hkv + kvh) << log2ps) + (pos & ((1 << log2ps) - 1))) * D;
                ok = true;
            } else {
                set_err(err, CKV_DEVERR_UNMAPPED_PAGE);
            }
        } else {
            set_err(err, CKV_DEVERR_INDEX_RANGE);
        }
    }

    uint4 kr[NLD], vr[NLD];
    bool okr[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int src = i * RPW + rs;
        const size_t ro = (size_t)__shfl((long long)rowoff, src);
        okr[i] = __shfl((int)ok, src) != 0;
        kr[i] = okr[i] ? *reinterpret_cast<const uint4 *>(kc + ro + ls * EPL) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int src = i * RPW + rs;
        const size_t ro = (size_t)__shfl((long long)rowoff, src);
        vr[i] = okr[i] ? *reinterpret_cast<const uint4 *>(vc + ro + ls * EPL) : make_uint4(0, 0, 0, 0);
    }

    // logits (log2 domain), one per (load, head); identical on the LPR lanes of a row
    float z[NLD][GH];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        float x[EPL];
        unpack<T, EPL>(kr[i], x);
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) s = fmaf(qv[h][e], x[e], s);
            s = group_sum<LPR>(s);
            z[i][h] = okr[i] ? s : -__builtin_inff();
        }
    }
    // wave-wide max per head
    float m[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        float mm = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < NLD; ++i) mm = fmaxf(mm, z[i][h]);
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
        m[h] = mm;
    }
    float l[GH], acc[GH][EPL];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        float x[EPL];
        unpack<T, EPL>(vr[i], x);
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            const float p = okr[i] ? fast_exp2(z[i][h] - m[h]) : 0.f;
            l[h] += p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
        }
    }
    // merge the RPW row slots of the wave (same dims, disjoint tokens, same m)
#pragma unroll
    for (int h = 0; h < GH; ++h) {
#pragma unroll
        for (int off = LPR; off < kWave; off <<= 1) {
            l[h] += __shfl_xor(l[h], off);
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
        }
    }
    if (lane < LPR) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) s_acc[w][h][lane * EPL + e] = acc[h][e];
            if (lane == 0) {
                s_m[w][h] = m[h];
                s_l[w][h] = l[h];
            }
        }
    }
    __syncthreads();

    // merge the waves; write this workgroup's partial (m, l, acc[D]) per head
    float *pbase = part + ((size_t)g * GH * max_splits) * (D + 2);
    for (int t = tid; t < GH * D; t += blockDim.x) {
        const int h = t / D, i = t % D;
        float mm = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < kAttnWaves; ++v) mm = fmaxf(mm, s_m[v][h]);
        float a = 0.f, ll = 0.f;
#pragma unroll
        for (int v = 0; v < kAttnWaves; ++v) {
            const float f = s_m[v][h] == -__builtin_inff() ? 0.f : fast_exp2(s_m[v][h] - mm);
            a += s_acc[v][h][i] * f;
            ll += s_l[v][h] * f;
        }
        float *pp = pbase + ((size_t)h * max_splits + split) * (D + 2);
        pp[2 + i] = a;
        if (i == 0) {
            pp[0] = mm;
            pp[1] = ll;
        }
    }

    // last workgroup of this graph merges all partials
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&counters[g], 1u);
        s_last = (prev == (uint32_t)(nsplit - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int t = tid; t < GH * D; t += blockDim.x) {
        const int h = t / D, i = t % D;
        const float *ph = pbase + (size_t)h * max_splits * (D + 2);
        float mm = -__builtin_inff();
        for (int s = 0; s < nsplit; ++s) mm = fmaxf(mm, __builtin_nontemporal_load(ph + (size_t)s * (D + 2)));
        float a = 0.f, ll = 0.f;
        for (int s = 0; s < nsplit; ++s) {
            const float ms = __builtin_nontemporal_load(ph + (size_t)s * (D + 2));
            const float f = ms == -__builtin_inff() ? 0.f : fast_exp2(ms - mm);
            ll += __builtin_nontemporal_load(ph + (size_t)s * (D + 2) + 1) * f;
            a += __builtin_nontemporal_load(ph + (size_t)s * (D + 2) + 2 + i) * f;
        }
        out[((size_t)b * Hq + h0 + h) * D + i] = ll > 0.f ? a / ll : 0.f;
    }
    if (tid == 0) counters[g] = 0u;
}

template <typename T, int D, int GH>
static void launch_attn_t(const Problem &p, const void *q, const ckv_kv &kv, const int32_t *idx,
                          int idx_stride, const int32_t *idx_len, float scale, float *out,
                          uint32_t *counters, float *partials, int32_t *err, hipStream_t st) {
    int log2ps = 0;
    while ((1 << log2ps) < kv.page_size) ++log2ps;
    const int ms = attn_max_splits(p, idx_stride);
    hipLaunchKernelGGL((attn_kernel<T, D, GH>), dim3(ms, p.NG()), dim3(256), 0, st,
                       static_cast<const T *>(q), static_cast<const T *>(kv.k),
                       static_cast<const T *>(kv.v), kv.page_table, log2ps, kv.max_pages_per_seq,
                       kv.num_pages, kv.seq_len, idx, idx_stride, idx_len, p.Hq, p.Hkv, p.gpk,
                       scale * kLog2e, out, counters, partials, ms, err);
}

hipError_t launch_attn(const Problem &p, const void *q, const ckv_kv &kv, const int32_t *idx,
                       int idx_stride, const int32_t *idx_len, float scale, float *out,
                       uint32_t *counters, float *partials, int32_t *err, hipStream_t st) {
    const int GH = p.heads_per_graph();
#define CKV_ATTN_CASE(TT, DT, DD, HH)                                                          \
    if (p.dtype == DT && p.D == DD && GH == HH) {                                              \
        launch_attn_t<TT, DD, HH>(p, q, kv, idx, idx_stride, idx_len, scale, out, counters,    \
                                  partials, err, st);                                          \
        return hipGetLastError();                                                              \
    }
    CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 128, 1) CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 128, 2)
    CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 128, 4) CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 128, 8)
    CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 64, 1) CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 64, 2)
    CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 64, 4) CKV_ATTN_CASE(bf16_t, CKV_DT_BF16, 64, 8)
    CKV_ATTN_CASE(float, CKV_DT_F32, 64, 1) CKV_ATTN_CASE(float, CKV_DT_F32, 64, 2)
    CKV_ATTN_CASE(float, CKV_DT_F32, 64, 4) CKV_ATTN_CASE(float, CKV_DT_F32, 64, 8)
    CKV_ATTN_CASE(float, CKV_DT_F32, 128, 1) CKV_ATTN_CASE(float, CKV_DT_F32, 128, 2)
    CKV_ATTN_CASE(float, CKV_DT_F32, 128, 4) CKV_ATTN_CASE(float, CKV_DT_F32, 128, 8)
#undef CKV_ATTN_CASE
    return hipErrorInvalidValue;
}

}  // namespace ckv
