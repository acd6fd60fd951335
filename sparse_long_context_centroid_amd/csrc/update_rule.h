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

// Lanes per candidate slot: the wave's 64 lanes cover CKV_MAX_CAND slots.
constexpr int kUpdLanesPerCand = kWave / CKV_MAX_CAND;
// Row stride (floats) of a candidate centroid parked in LDS: padded by one float4
// so that the candidate lanes' element-order reads fall in different banks.
constexpr int kUpdCentStride(int D) { return D + 4; }
// LDS floats one updating wavefront needs: k_new widened to fp64, then the
// candidates' centroids.
constexpr int kUpdLdsFloats(int D) { return 2 * D + CKV_MAX_CAND * kUpdCentStride(D); }

// One wavefront updates graph g.  cand[0..M) are community ids (-1 = none);
// C communities are in use.  lds_row holds kUpdLdsFloats(D) floats of LDS private
// to this wave.  When write_kv, the wave also stores k_new / v_new into K/V row n
// of KV head kvh (seq_pages: the sequence's page-table row), or flags an unmapped
// page.
//
// Every global read is issued before any is waited for, in two dependent rounds:
// the candidate ids (beside the caller's seq_len and community-count loads), then
// all candidates' centroids (4 lanes per candidate) with their sizes, capacities
// and starts, and the page-table entry of row n.  The page-table load is issued
// after the candidate ids and unconditionally (clamped slot, validity by selects),
// so that waiting for the ids never waits for it.  The centroids are parked in
// LDS; the lane that owns a candidate then sums its distance there, in element
// order.
template <typename T, int D>
__device__ __forceinline__ void local_update_wave(const T *__restrict__ kn, const T *__restrict__ vn,
                                  const int *cand, int M, int C, size_t g, int Cmax,
                                  float *__restrict__ cent, const int32_t *__restrict__ comm_start,
                                  int32_t *__restrict__ comm_size,
                                  const int32_t *__restrict__ comm_cap,
                                  int32_t *__restrict__ members, int n, bool write_kv,
                                  T *__restrict__ kc, T *__restrict__ vc,
                                  const int32_t *__restrict__ seq_pages, int log2ps,
                                  int max_pages, int num_pages, int kvh, int Hkv,
                                  int32_t *__restrict__ assigned,
                                  int32_t *__restrict__ err, float *lds_row) {
#pragma clang fp contract(off)
    constexpr int LPC = kUpdLanesPerCand;
    constexpr int CS = kUpdCentStride(D);
    constexpr int KPL = D / 4 / LPC;  // float4 chunks of a centroid per lane
    static_assert((D / 4) % LPC == 0, "whole chunks per lane");
    const int lane = threadIdx.x & (kWave - 1);
    const int slot = lane / LPC, part = lane % LPC;
    double *kn64 = reinterpret_cast<double *>(lds_row);
    float *lc = lds_row + 2 * D;
    // round 1: this lane's candidate id and its share of k_new
    const int cc = cand[min(slot, M - 1)];
    T knr[D / kWave > 0 ? D / kWave : 1];
#pragma unroll
    for (int r = 0; r < D / kWave; ++r) knr[r] = kn[lane + r * kWave];
    // K/V row n: its page-table entry, requested behind the ids
    const int lp = n >> log2ps;
    const int pg = seq_pages[min(lp, max_pages - 1)];
    const int c = (slot < M && cc >= 0 && cc < C) ? cc : -1;
    const int cl = c >= 0 ? c : 0;  // loads below are unconditional
    // round 2: the centroid share, size, capacity and start of the candidate
    const float4 *cp = reinterpret_cast<const float4 *>(cent) + g * (D / 4) * Cmax + cl;
    float4 v[KPL];
#pragma unroll
    for (int k = 0; k < KPL; ++k) v[k] = cp[(size_t)(part + k * LPC) * Cmax];
    int sz = comm_size[g * Cmax + cl];
    const int cap = comm_cap[g * Cmax + cl];
    const int st = comm_start[g * Cmax + cl];
#pragma unroll
    for (int r = 0; r < D / kWave; ++r) kn64[lane + r * kWave] = (double)to_f32(knr[r]);
#pragma unroll
    for (int k = 0; k < KPL; ++k)
        *reinterpret_cast<float4 *>(lc + slot * CS + (part + k * LPC) * 4) = v[k];
    __builtin_amdgcn_wave_barrier();
    // the first lane of each candidate slot sums the distance in element order
    double dist = __builtin_inf();
    if (part == 0 && c >= 0) {
        double s = 0.0;
        const float *mu = lc + slot * CS;
#pragma unroll 8
        for (int i = 0; i < D; ++i) {
            const double diff = kn64[i] - (double)mu[i];
            const double sq = diff * diff;
            s = s + sq;
        }
        dist = s;
    }
    // argmin over (distance, id) among the slot-owning lanes (lanes 0, LPC, 2*LPC,
    // ...: a butterfly over distances LPC..32 stays inside that set), then made
    // wave-uniform from lane 0
    int best = part == 0 ? c : -1;
    double bd = dist;
#pragma unroll
    for (int off = LPC; off < kWave; off <<= 1) {
        const double od = __shfl_xor(bd, off);
        const int oc = __shfl_xor(best, off);
        if (oc >= 0 && (best < 0 || od < bd || (od == bd && oc < best))) {
            bd = od;
            best = oc;
        }
    }
    best = __shfl(best, 0);
    const unsigned long long win = __ballot(part == 0 && c >= 0 && c == best);
    int slot_new = -1;
    int wl = 0;
    if (win) {
        wl = __ffsll((long long)win) - 1;
        const int wsz = __shfl(sz, wl);
        const int wcap = __shfl(cap, wl);
        const int wst = __shfl(st, wl);
        if (wsz < wcap) {
            slot_new = wsz;
            if (lane == 0) {
                members[(size_t)wst + wsz] = n;
                comm_size[g * Cmax + best] = wsz + 1;
            }
        } else if (lane == 0) {
            set_err(err, CKV_DEVERR_CAPACITY);
        }
    }
    if (lane == 0) assigned[g] = slot_new >= 0 ? best : -1;
    if (slot_new >= 0) {
        // running mean of the winner, from its LDS copy
        const double cnt = (double)(slot_new + 1);
        const float *mu = lc + (wl / LPC) * CS;
        float *out = cent + g * (D / 4) * Cmax * 4;
        for (int i = lane; i < D; i += kWave) {
            const double m0 = (double)mu[i];
            const double step = (kn64[i] - m0) / cnt;
            out[((size_t)(i / 4) * Cmax + best) * 4 + i % 4] = (float)(m0 + step);
        }
    }
    if (write_kv) {
        const bool kv_ok = lp < max_pages && pg >= 0 && pg < num_pages;
        const size_t kv_row =
            kv_ok ? ((((size_t)pg * Hkv + kvh) << log2ps) + (n & ((1 << log2ps) - 1))) * D : 0;
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
    local_update_wave<T, D>(kn, vn, cand + g * M, M, C, g, Cmax, cent, comm_start, comm_size,
                            comm_cap, members, n, gl % gpk == 0, kc, vc,
                            page_table + (size_t)b * max_pages, log2ps, max_pages, num_pages, kvh,
                            Hkv, assigned, err, lds_row);
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

// The layer graph: one graph per sequence b, whose centroid rows hold one d-slice
// per KV head (E = Hkv*d values, KV head after KV head).  The new token's key row
// is the concatenation of its Hkv keys; it joins the candidate whose row is
// nearest in squared L2 over all E values, accumulated per KV head (each slice
// summed in fp64 in element order, then the slices in head order; lower id on
// equal distance); that community's whole row moves to the running mean, and K/V
// row n is written in every KV head.
//
// One workgroup (of at least kLayerUpdThreads threads) per sequence: k_new (as
// fp32, exact for both input types) and the candidates' rows are staged in LDS by
// the whole workgroup (every load in flight at once); one thread per (candidate,
// slice) sums that slice in fp64, and the first wave's lanes 0..M-1 add their
// candidate's slices in order.  All of its LDS comes from one buffer of
// layer_update_lds(E, M, Hkv) bytes (the host checks the size): the slice sums
// (M*Hkv doubles), the M rows of E+4 floats, k_new (E floats), then M candidate
// ids and three ints.
constexpr int kLayerUpdThreads = 256;
constexpr int kLayerUpdMaxHeads = 32;  // KV heads (slices) per row
__host__ __device__ constexpr size_t layer_update_part_bytes(int M, int Hkv) {
    return ((size_t)M * Hkv * sizeof(double) + 15) / 16 * 16;
}
inline size_t layer_update_lds(int E, int M, int Hkv) {
    return layer_update_part_bytes(M, Hkv) + (size_t)M * (E + 4) * sizeof(float) +
           (size_t)E * sizeof(float) + (size_t)(M + 3) * sizeof(int);
}

template <typename T, int D>
__device__ __forceinline__ void layer_update_seq(
    int b, const T *__restrict__ k_new, const T *__restrict__ v_new,
    const int32_t *__restrict__ cand, int M, float *__restrict__ cent,
    const int32_t *__restrict__ num_comms, const int32_t *__restrict__ comm_start,
    int32_t *__restrict__ comm_size, const int32_t *__restrict__ comm_cap,
    int32_t *__restrict__ members, int Cmax, int Hkv, T *__restrict__ kc, T *__restrict__ vc,
    const int32_t *__restrict__ page_table, int log2ps, int max_pages, int num_pages,
    int32_t *__restrict__ seq_len, int bump, int32_t *__restrict__ assigned,
    int32_t *__restrict__ err, unsigned char *__restrict__ s_raw) {
#pragma clang fp contract(off)
    const int tid = threadIdx.x;
    // threads past the first kLayerUpdThreads (a larger host workgroup) only join
    // the barriers
    const bool act = tid < kLayerUpdThreads;
    const int E = Hkv * D, E4 = E / 4, CS = E + 4;
    double *s_part = reinterpret_cast<double *>(s_raw);
    float *lc = reinterpret_cast<float *>(s_raw + layer_update_part_bytes(M, Hkv));
    float *knf = lc + (size_t)M * CS;
    int *s_cl = reinterpret_cast<int *>(knf + E);
    int &s_best = s_cl[M], &s_slot = s_cl[M + 1], &s_new = s_cl[M + 2];
    const int n = seq_len[b];
    const int C = min(num_comms[b], Cmax);
    const T *kn = k_new + (size_t)b * E;
    const T *vn = v_new + (size_t)b * E;
    // round 1: the candidate ids and k_new (as fp32) to LDS
    if (tid < M) {
        const int cc = cand[(size_t)b * M + tid];
        s_cl[tid] = (cc >= 0 && cc < C) ? cc : -1;
    }
    if (act) {
        // E / 256 elements per thread, loaded together (clamped indexes: a loop of
        // load-then-store would wait for each load in turn)
        constexpr int kMaxPer = 16;  // E <= 4096
        T kv[kMaxPer];
#pragma unroll
        for (int r = 0; r < kMaxPer; ++r) kv[r] = kn[min(tid + r * kLayerUpdThreads, E - 1)];
#pragma unroll
        for (int r = 0; r < kMaxPer; ++r)
            if (tid + r * kLayerUpdThreads < E)
                knf[tid + r * kLayerUpdThreads] = to_f32(kv[r]);
    }
    __syncthreads();
    // round 2: the candidates' rows, element 4*k4 .. +3 of community c at float4
    // (b*E4 + k4)*Cmax + c, 8 loads per thread in flight per pass
    const float4 *c4 = reinterpret_cast<const float4 *>(cent) + (size_t)b * E4 * Cmax;
    const int total = M * E4;
    for (int t0 = 0; act && t0 < total; t0 += 8 * kLayerUpdThreads) {
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
    for (int pr = tid; act && pr < M * Hkv; pr += kLayerUpdThreads) {
        const int sl = pr / Hkv, kh = pr % Hkv;
        const float4 *mu4 = reinterpret_cast<const float4 *>(lc + sl * CS + kh * D);
        const float4 *k4 = reinterpret_cast<const float4 *>(knf + kh * D);
        double s = 0.0;
#pragma unroll 8
        for (int i4 = 0; i4 < D / 4; ++i4) {
            const float4 m = mu4[i4];
            const float4 k = k4[i4];
            const double d0 = (double)k.x - (double)m.x, d1 = (double)k.y - (double)m.y;
            const double d2 = (double)k.z - (double)m.z, d3 = (double)k.w - (double)m.w;
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
        for (int i = tid; act && i < E; i += kLayerUpdThreads) {
            const double m0 = (double)mu[i];
            const double step = ((double)knf[i] - m0) / cnt;
            cent[(((size_t)b * E4 + i / 4) * Cmax + best) * 4 + i % 4] = (float)(m0 + step);
        }
    }
    // K/V row n in every KV head
    const int lp = n >> log2ps;
    const int pg = lp < max_pages ? page_table[(size_t)b * max_pages + lp] : -1;
    if (pg >= 0 && pg < num_pages) {
        for (int i = tid; act && i < E; i += kLayerUpdThreads) {
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


}  // namespace ckv
