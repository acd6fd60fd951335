// update_rule.h -- the constant-time local update of one graph, run by one wavefront.
//
// rit.work post "CommunityKV long-context decoding", token-graph section: the new
// token is attached to a suitable neighbouring community and only that community's
// centre is updated, at a cost set by the model dimension, not by the context
// length; the CommunityKV abstract (McKenna et al., 2026) calls it a constant-time
// local update rule.  Reading used here: the neighbours are the graph's top-M
// communities of this step's score order; the new key joins the one whose
// centroid is nearest in squared L2 (lower id on equal distance); its centroid
// becomes the running mean of its members.
//
// Precision: the distance of each candidate is summed in fp64 in element order by
// one lane (no contraction into FMA: every product and sum rounds once), and the
// centroid moves by mu <- fp32(mu + (k - mu) / size) in fp64 -- a deterministic
// function of the stored bytes.
#pragma once

#include "ckv_device.h"

namespace ckv {

// LDS floats one updating wavefront needs: k_new widened to fp64.
constexpr int kUpdLdsFloats(int D) { return 2 * D; }

// One wavefront updates graph g.  cand[0..M) are community ids (-1 = none);
// C communities are in use.  lds_row holds kUpdLdsFloats(D) floats of LDS private
// to this wave (k_new widened to fp64).
// When write_kv, the wave also stores k_new / v_new into K/V row `kv_row`
// (element offset), or flags an unmapped page.
template <typename T, int D>
__device__ __forceinline__ void local_update_wave(const T *__restrict__ kn, const T *__restrict__ vn,
                                  const int *cand, int M, int C, size_t g, int Cmax,
                                  float *__restrict__ cent, const int32_t *__restrict__ comm_start,
                                  int32_t *__restrict__ comm_size,
                                  const int32_t *__restrict__ comm_cap,
                                  int32_t *__restrict__ members, int n, bool write_kv,
                                  T *__restrict__ kc, T *__restrict__ vc, size_t kv_row,
                                  bool kv_ok, int32_t *__restrict__ assigned,
                                  int32_t *__restrict__ err, float *lds_row) {
#pragma clang fp contract(off)
    const int lane = threadIdx.x & (kWave - 1);
    // k_new widened to fp64 once, into LDS, so the candidate lanes read it there
    // instead of issuing one dependent scalar load per element
    double *kn64 = reinterpret_cast<double *>(lds_row);
    for (int i = lane; i < D; i += kWave) kn64[i] = (double)to_f32(kn[i]);
    __builtin_amdgcn_wave_barrier();
    // lane m < M owns candidate m: its size, capacity and start are fetched with
    // the first chunk of its centroid; the centroid streams through registers in
    // chunks of 8 float4 (the distance stays an element-order sum)
    int c = -1;
    if (lane < M) {
        const int cc = cand[lane];
        if (cc >= 0 && cc < C) c = cc;
    }
    int sz = 0, cap = 0, st = 0;
    double dist = __builtin_inf();
    if (c >= 0) {
        const float4 *cp = reinterpret_cast<const float4 *>(cent) + g * (D / 4) * Cmax + c;
        sz = comm_size[g * Cmax + c];
        cap = comm_cap[g * Cmax + c];
        st = comm_start[g * Cmax + c];
        double s = 0.0;
#pragma unroll 1
        for (int k0 = 0; k0 < D / 4; k0 += 8) {
            float4 v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = cp[(size_t)(k0 + k) * Cmax];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float m4[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double diff = kn64[(k0 + k) * 4 + e] - (double)m4[e];
                    const double sq = diff * diff;
                    s = s + sq;
                }
            }
        }
        dist = s;
    }
    // argmin over (distance, id) across the wave
    int best = c;
    double bd = dist;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double od = __shfl_xor(bd, off);
        const int oc = __shfl_xor(best, off);
        if (oc >= 0 && (best < 0 || od < bd || (od == bd && oc < best))) {
            bd = od;
            best = oc;
        }
    }
    const unsigned long long win = __ballot(c >= 0 && c == best);
    int slot = -1;
    int wl = 0;
    if (win) {
        wl = __ffsll((long long)win) - 1;
        sz = __shfl(sz, wl);
        cap = __shfl(cap, wl);
        st = __shfl(st, wl);
        __builtin_amdgcn_wave_barrier();
        if (sz < cap) {
            slot = sz;
            if (lane == 0) {
                members[(size_t)st + sz] = n;
                comm_size[g * Cmax + best] = sz + 1;
            }
        } else if (lane == 0) {
            set_err(err, CKV_DEVERR_CAPACITY);
        }
    }
    if (lane == 0) assigned[g] = slot >= 0 ? best : -1;
    if (slot >= 0) {
        const double cnt = (double)(slot + 1);
        float *mu = cent + g * (D / 4) * Cmax * 4;
        for (int i = lane; i < D; i += kWave) {
            const double m0 = (double)mu[((size_t)(i / 4) * Cmax + best) * 4 + i % 4];
            const double step = (kn64[i] - m0) / cnt;
            mu[((size_t)(i / 4) * Cmax + best) * 4 + i % 4] = (float)(m0 + step);
        }
    }
    if (write_kv) {
        if (kv_ok) {
            for (int i = lane; i < D; i += kWave) {
                kc[kv_row + i] = kn[i];
                vc[kv_row + i] = vn[i];
            }
        } else if (lane == 0) {
            set_err(err, CKV_DEVERR_UNMAPPED_PAGE);
        }
    }
}

// Graph g (sequence b = g / (Hkv*gpk)) by one wavefront: the new token is row n =
// seq_len[b]; the first graph of each KV head also writes K/V row n.  seq_len is
// left as it is.
template <typename T, int D>
__device__ __forceinline__ void graph_update(size_t g, const T *__restrict__ k_new,
                                             const T *__restrict__ v_new,
                                             const int32_t *__restrict__ cand, int M,
                                             float *__restrict__ cent,
                                             const int32_t *__restrict__ num_comms,
                                             const int32_t *__restrict__ comm_start,
                                             int32_t *__restrict__ comm_size,
                                             const int32_t *__restrict__ comm_cap,
                                             int32_t *__restrict__ members, int Cmax, int Hkv,
                                             int gpk, T *__restrict__ kc, T *__restrict__ vc,
                                             const int32_t *__restrict__ page_table, int log2ps,
                                             int max_pages, int num_pages,
                                             const int32_t *__restrict__ seq_len,
                                             int32_t *__restrict__ assigned,
                                             int32_t *__restrict__ err, float *lds_row) {
    const int gps = Hkv * gpk;
    const int b = (int)(g / gps);
    const int gl = (int)(g % gps);
    const int n = seq_len[b];
    const int kvh = gl / gpk;
    const T *kn = k_new + ((size_t)b * Hkv + kvh) * D;
    const T *vn = v_new + ((size_t)b * Hkv + kvh) * D;
    const int C = min(num_comms[g], Cmax);
    const int lp = n >> log2ps;
    const int pg = lp < max_pages ? page_table[(size_t)b * max_pages + lp] : -1;
    const bool ok = pg >= 0 && pg < num_pages;
    const size_t row =
        ok ? ((((size_t)pg * Hkv + kvh) << log2ps) + (n & ((1 << log2ps) - 1))) * D : 0;
    local_update_wave<T, D>(kn, vn, cand + g * M, M, C, g, Cmax, cent, comm_start, comm_size,
                            comm_cap, members, n, gl % gpk == 0, kc, vc, row, ok, assigned, err,
                            lds_row);
}

// All graphs of sequence b, one wavefront per graph (looping when the workgroup
// has fewer waves than graphs), then seq_len[b] += 1.  One workgroup per sequence,
// so reading n and advancing seq_len cannot race.  lds_rows: kUpdLdsFloats(D)
// floats per wave.
template <typename T, int D>
__device__ __forceinline__ void sequence_update(int b, const T *__restrict__ k_new, const T *__restrict__ v_new,
                                const int32_t *__restrict__ cand, int M, float *__restrict__ cent,
                                const int32_t *__restrict__ num_comms,
                                const int32_t *__restrict__ comm_start,
                                int32_t *__restrict__ comm_size,
                                const int32_t *__restrict__ comm_cap,
                                int32_t *__restrict__ members, int Cmax, int Hkv, int gpk,
                                T *__restrict__ kc, T *__restrict__ vc,
                                const int32_t *__restrict__ page_table, int log2ps, int max_pages,
                                int num_pages, int32_t *__restrict__ seq_len,
                                int32_t *__restrict__ assigned, int32_t *__restrict__ err,
                                float *lds_rows) {
    const int w = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int gps = Hkv * gpk;
    const int n = seq_len[b];
    for (int gl = w; gl < gps; gl += nw)
        graph_update<T, D>((size_t)b * gps + gl, k_new, v_new, cand, M, cent, num_comms,
                           comm_start, comm_size, comm_cap, members, Cmax, Hkv, gpk, kc, vc,
                           page_table, log2ps, max_pages, num_pages, seq_len, assigned, err,
                           lds_rows + (size_t)w * kUpdLdsFloats(D));
    __syncthreads();
    if (threadIdx.x == 0) seq_len[b] = n + 1;
}

}  // namespace ckv
