// edges.hip -- direct edges of the prefill token graph from QK^T tiles on MFMA.
//
// rit.work post "CommunityKV long-context decoding", token-graph section: the
// graph is built during the prefill pass from the QK^T scores the model computes
// anyway; a direct edge links a query to a key it attends strongly, a second kind
// links keys that are looked at together; the initial sink tokens are no nodes.
// Readings: the strength of query position i -> key position j in a graph is
//   z_ij = max over the graph's query heads h of q_h[i] . k[j] * scale,
// causal and without self-links (S <= j < i); the direct edges of i are its
// `topk` strongest keys in (z desc, j asc) order; the co-attention pairs of i are
// all pairs of those keys (lower position first, pairs in ascending order).
//
// Design for gfx950: QK^T is a dense contraction, so it runs on the matrix cores
// (v_mfma_f32_16x16x32_bf16: exact products, fp32 accumulation).  A workgroup
// owns 4 waves of consecutive queries of one graph.  The MFMA rows of a wave are
// its (query, head) pairs, query-major: a lane's four accumulator rows are heads
// of the same query (or queries), so the group max needs no lane exchange (one
// 16-lane swap for 8 heads).  Key tiles of 64 rows are staged in LDS (row stride
// padded by 16 B: conflict-free 16-byte reads), shared by the four waves.  Every
// lane keeps a sorted top-8 list per query for the key columns it owns (key =
// 16-key block + lane % 16); since a lane meets its keys in ascending position,
// a new score enters only if strictly above the list's last entry, which a
// wave-wide ballot tests before the rare insertion.  At the end the 16 lanes of a
// row merge their lists with lane shuffles.
#include "ckv_device.h"
#include "ckv_internal.h"

#include <type_traits>

namespace ckv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#ifndef CKV_EDGE_WAVES
#define CKV_EDGE_WAVES 4
#endif
constexpr int kEdgeWaves = CKV_EDGE_WAVES;  // waves (query blocks) sharing a key tile
#ifndef CKV_EDGE_KT
#define CKV_EDGE_KT 64
#endif
constexpr int kEdgeKT = CKV_EDGE_KT;  // keys per LDS tile
constexpr int kEdgeList = 8; // list length kept per query (largest topk)
#ifndef CKV_EDGE_REFRESH
#define CKV_EDGE_REFRESH 4
#endif
constexpr int kEdgeRefresh = CKV_EDGE_REFRESH;  // tiles between row-bound refreshes
#ifndef CKV_EDGE_QPW1
#define CKV_EDGE_QPW1 16
#endif
// queries per wave: 64 MFMA rows of (query, head) pairs, or with one head per
// graph CKV_EDGE_QPW1 queries (16 or 32: two M-blocks share each key block)
constexpr int edge_queries_per_wave(int hpg) {
    return hpg == 1 ? CKV_EDGE_QPW1 : (hpg <= 4 ? 16 : 8);
}

// (a, ia) before (b, ib) in the (score desc, position asc) order.
__device__ __forceinline__ bool edge_before(float a, int ia, float b, int ib) {
    return a > b || (a == b && ia < ib);
}

// Insert (v, vi) into a sorted list (the last entry falls off): from the first
// slot it goes before, every later slot takes the entry displaced from the one
// above.  LATEST: vi is larger than every position in the list, so ties keep the
// listed entry first.
template <bool LATEST>
__device__ __forceinline__ void edge_insert(float (&ts)[kEdgeList], int (&ti)[kEdgeList],
                                            float v, int vi) {
    bool shifting = false;
#pragma unroll
    for (int p = 0; p < kEdgeList; ++p) {
        const bool take =
            shifting || (LATEST ? v > ts[p] : edge_before(v, vi, ts[p], ti[p]));
        shifting = take;
        const float ov = ts[p];
        const int oi = ti[p];
        ts[p] = take ? v : ov;
        ti[p] = take ? vi : oi;
        v = take ? ov : v;
        vi = take ? oi : vi;
    }
}

// The 8th largest of the values held by the 16 lanes of a row, in every lane of
// the row (a bitonic sort across the row, descending by lane, then a broadcast).
__device__ __forceinline__ float row16_eighth_largest(float v, int r16) {
#pragma unroll
    for (int k = 2; k <= 16; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float o = __shfl_xor(v, j, 16);
            const bool keep_max = ((r16 & j) == 0) == ((r16 & k) == 0);
            v = keep_max ? fmaxf(v, o) : fminf(v, o);
        }
    }
    return __shfl(v, 7, 16);
}

template <int D, int HPG>
__global__ __launch_bounds__(kEdgeWaves * kWave) void edges_kernel(
    const bf16_t *__restrict__ q, const bf16_t *__restrict__ k, int n, int Hq, int Hkv, int gpk,
    int S, float scale, int topk, int32_t *__restrict__ out_idx, float *__restrict__ out_score,
    int32_t *__restrict__ out_pairs) {
    constexpr int EK = kEdgeList;
    constexpr int T = D / 32;                          // MFMA steps over the head dimension
    constexpr int QPW = edge_queries_per_wave(HPG);    // queries per wave
    constexpr int QPB = kEdgeWaves * QPW;              // queries per workgroup
    constexpr int MB = QPW * HPG / 16;                 // 16-row M-blocks per wave
    constexpr int HL = HPG < 4 ? HPG : 4;              // heads of a query in one lane
    constexpr int QPL = 4 / HL;                        // queries per lane per M-block
    constexpr int NQ = MB * QPL;                       // query slots per lane (= 4)
    constexpr int LDSR = D + 8;                        // LDS row stride in bf16
    constexpr int KT = kEdgeKT;
    constexpr int kPieces = KT * D / 8 / (kEdgeWaves * kWave);  // 16-byte loads per thread
    static_assert(HPG == 1 || HPG == 2 || HPG == 4 || HPG == 8, "heads per graph");
    static_assert(NQ == 4 || NQ == 8, "query slots");
    static_assert(kPieces * kEdgeWaves * kWave * 8 == KT * D, "tile split");
    __shared__ __align__(16) bf16_t s_k[2][KT * LDSR];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int gs = blockIdx.y;             // graph of the sequence
    const int b = blockIdx.z;
    const int kvh = gs / gpk;
    const int h0 = gs * HPG;               // first query head (graph = head when HPG = 1)
    // the largest query blocks first (they see the most keys)
    const int q0 = ((int)gridDim.x - 1 - (int)blockIdx.x) * QPB;
    const int qw = q0 + w * QPW;
    const int r16 = lane & 15, g4 = lane >> 4;
    const bf16_t *qb = q + (size_t)b * n * Hq * D;
    const bf16_t *kb_ = k + (size_t)b * n * Hkv * D;

    // A operands: row R = m*16 + r16 of the wave is (query R / HPG, head R % HPG);
    // lane (r16, g4) holds elements 32t + 8g4 .. +8 of that row
    bf16x8_t a[MB][T];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int R = m * 16 + r16;
        // queries past n read row n-1 (their results are not written)
        const int qi = min(qw + R / HPG, n - 1), h = R % HPG;
#pragma unroll
        for (int t = 0; t < T; ++t)
            a[m][t] = __builtin_bit_cast(
                bf16x8_t, *reinterpret_cast<const uint4 *>(qb + ((size_t)qi * Hq + h0 + h) * D +
                                                           32 * t + 8 * g4));
    }
    // query of slot s = m*QPL + jq: accumulator rows 4g4 + jq*HL .. +HL of block m
    int qpos[NQ];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int jq = 0; jq < QPL; ++jq)
            qpos[m * QPL + jq] = qw + (m * 16 + 4 * g4 + jq * HL) / HPG;
    float ts[NQ][EK];
    int ti[NQ][EK];
#pragma unroll
    for (int s = 0; s < NQ; ++s)
#pragma unroll
        for (int p = 0; p < EK; ++p) {
            ts[s][p] = -__builtin_inff();
            ti[s][p] = -1;
        }
    // thr[s]: a key of slot s can only matter if its score is above thr[s] = the
    // larger of this lane's 8th entry and a lower bound of the row's 8th best
    // (keys arrive in ascending position, so an equal score loses the tie)
    float thr[NQ];
#pragma unroll
    for (int s = 0; s < NQ; ++s) thr[s] = -__builtin_inff();

    const int qlast = min(q0 + QPB, n) - 1;  // largest query of the workgroup
    const int wlast = min(qw + QPW, n) - 1;  // ... of this wave
    // key tiles S, S+KT, ... below qlast; tile it+1 is fetched into registers
    // while tile it is computed, then stored into the other LDS buffer.  Rows
    // past n are clamped to row n-1: such keys are only ever compared for
    // queries past n, whose results are not written.
    u32x4_t pre[kPieces];
    // one 16-key block on the matrix cores: T MFMAs per M-block
    auto mma = [&](const bf16_t *sk, f32x4_t (&acc)[MB]) __attribute__((always_inline)) {
        // B operand: lane (r16, g4) holds elements 32t + 8g4 .. +8 of key k16 + r16
        bf16x8_t bb[T];
#pragma unroll
        for (int t = 0; t < T; ++t)
            bb[t] = *reinterpret_cast<const bf16x8_t *>(sk + r16 * LDSR + 32 * t + 8 * g4);
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][t], bb[t], acc[m], 0, 0, 0);
        }
    };
    // the block's group max, scale and list filter (MASKED applies j < i: only
    // tiles that reach the wave's queries); one wave-wide branch per block
    auto filter = [&](const f32x4_t (&acc)[MB], int k16, auto masked_c)
                      __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int j = k16 + r16;  // this lane's accumulator column
        float zs[NQ];
        bool ins[NQ];
        bool any = false;
#pragma unroll
        for (int m = 0; m < MB; ++m) {
#pragma unroll
            for (int jq = 0; jq < QPL; ++jq) {
                float z = acc[m][jq * HL];
#pragma unroll
                for (int h = 1; h < HL; ++h) z = fmaxf(z, acc[m][jq * HL + h]);
                if constexpr (HPG == 8) {
                    // the other four heads sit in the lane 16 apart
                    const uint32_t u = __float_as_uint(z);
                    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                    z = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
                }
                const int s = m * QPL + jq;
                z *= scale;
                if constexpr (MASKED) z = j < qpos[s] ? z : -__builtin_inff();
                zs[s] = z;
                ins[s] = z > thr[s];
                any |= ins[s];
            }
        }
        if (__ballot(any)) {
#pragma unroll
            for (int s = 0; s < NQ; ++s) {
                if (ins[s]) {
                    edge_insert<true>(ts[s], ti[s], zs[s], j);
                    thr[s] = fmaxf(thr[s], ts[s][EK - 1]);
                }
            }
        }
    };
    // the blocks of a tile, software-pipelined: block b+1's MFMAs are issued
    // before block b is filtered, so the matrix cores run under the filter
    auto tile = [&](const bf16_t *sk, int kt, int nb, auto masked_c) __attribute__((always_inline)) {
        static_assert(KT == 64, "four blocks per tile");
        f32x4_t x0[MB], x1[MB];
        mma(sk, x0);
        __builtin_amdgcn_sched_barrier(0);
        if (nb > 1) mma(sk + 16 * LDSR, x1);
        filter(x0, kt, masked_c);
        __builtin_amdgcn_sched_barrier(0);
        if (nb > 2) mma(sk + 32 * LDSR, x0);
        if (nb > 1) filter(x1, kt + 16, masked_c);
        __builtin_amdgcn_sched_barrier(0);
        if (nb > 3) mma(sk + 48 * LDSR, x1);
        if (nb > 2) filter(x0, kt + 32, masked_c);
        __builtin_amdgcn_sched_barrier(0);
        if (nb > 3) filter(x1, kt + 48, masked_c);
    };
    const int ntiles = qlast > S ? (qlast - S + KT - 1) / KT : 0;
    // Tile it is stored into LDS buffer it & 1 at the top of iteration it, from
    // registers loaded during iteration it-1's compute (a loop-carried prefetch,
    // which the compiler cannot sink next to the store).  One barrier per tile:
    // the buffer written at the top of iteration it was last read in iteration
    // it-2, which every wave finished before the barrier of iteration it-1.
    // Piece p of a tile: row (tid + 256p) / (D/8), 16-byte column (tid + 256p) % (D/8);
    // rows are clamped to n-1 (the last prefetch re-reads valid rows).
#pragma unroll
    for (int p = 0; p < kPieces; ++p) {
        const int c = tid + p * kEdgeWaves * kWave;
        const int j = min(S + c / (D / 8), n - 1);
        pre[p] = *reinterpret_cast<const u32x4_t *>(kb_ + ((size_t)j * Hkv + kvh) * D +
                                                  8 * (c % (D / 8)));
    }
    // the A operands are complete before the loop (an empty use of each): left in
    // flight, they make the compiler wait for every outstanding load -- the next
    // tile's included -- at the first MFMA of every tile
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int t = 0; t < T; ++t) asm volatile("" ::"v"(a[m][t]));
#pragma unroll 1
    for (int it = 0; it < ntiles; ++it) {
        const int kt = S + it * KT;
        bf16_t *sk = s_k[it & 1];
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            const int c = tid + p * kEdgeWaves * kWave;
            *reinterpret_cast<u32x4_t *>(sk + (c / (D / 8)) * LDSR + 8 * (c % (D / 8))) = pre[p];
        }
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kPieces; ++p) {
            const int c = tid + p * kEdgeWaves * kWave;
            const int j = min(kt + KT + c / (D / 8), n - 1);
            pre[p] = *reinterpret_cast<const u32x4_t *>(kb_ + ((size_t)j * Hkv + kvh) * D +
                                                      8 * (c % (D / 8)));
        }
        // blocks of this tile below the wave's last query (wave-uniform)
        const int nb = min(max((wlast - kt + 15) / 16, 0), KT / 16);
        if (nb > 0) {
            if (kt + KT <= qw)
                tile(sk, kt, nb, std::integral_constant<bool, false>{});
            else
                tile(sk, kt, nb, std::integral_constant<bool, true>{});
        }
        // row bound: the 8 largest lane maxima are 8 distinct keys, so the row's
        // 8th best is at least the 8th largest of the 16 maxima (refreshed every
        // kEdgeRefresh tiles: it tightens slowly once the lists have filled)
        if (it % kEdgeRefresh == kEdgeRefresh - 1) {
#pragma unroll
            for (int s = 0; s < NQ; ++s)
                thr[s] = fmaxf(thr[s], row16_eighth_largest(ts[s][0], r16));
        }
    }

    // merge the 16 lanes of a row (same queries, disjoint key columns)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
        for (int s = 0; s < NQ; ++s) {
            float ps[EK];
            int pi[EK];
#pragma unroll
            for (int p = 0; p < EK; ++p) {
                ps[p] = __shfl_xor(ts[s][p], off);
                pi[p] = __shfl_xor(ti[s][p], off);
            }
#pragma unroll
            for (int p = 0; p < EK; ++p)
                if (pi[p] >= 0) edge_insert<false>(ts[s], ti[s], ps[p], pi[p]);
        }
    }

    // lane r16 == s of a row writes query slot s (with 8 heads, rows g4 and g4^1
    // hold the same queries: the even one writes)
    const int npairs = topk * (topk - 1) / 2;
    const size_t gq = ((size_t)b * gridDim.y + gs) * n;  // graph row base
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
        const int i = qpos[s];
        if (r16 != s || i >= n || (HPG == 8 && (g4 & 1))) continue;
        const size_t o = gq + i;
        int kept[EK];
#pragma unroll
        for (int p = 0; p < EK; ++p) {
            const bool v = p < topk && ti[s][p] >= 0;
            if (p < topk) {
                out_idx[o * topk + p] = v ? ti[s][p] : -1;
                out_score[o * topk + p] = v ? ts[s][p] : -__builtin_inff();
            }
            kept[p] = v ? ti[s][p] : 0x7fffffff;
        }
        if (out_pairs) {
            // ascending positions, missing entries last (odd-even transposition sort)
#pragma unroll
            for (int r = 0; r < EK; ++r)
#pragma unroll
                for (int x = r & 1; x + 1 < EK; x += 2) {
                    const int lo = min(kept[x], kept[x + 1]), hi = max(kept[x], kept[x + 1]);
                    kept[x] = lo;
                    kept[x + 1] = hi;
                }
            int32_t *pp = out_pairs + o * npairs * 2;
#pragma unroll
            for (int x = 0; x < EK; ++x)
#pragma unroll
                for (int y = x + 1; y < EK; ++y) {
                    if (y >= topk) continue;
                    const int c = x * topk - x * (x + 1) / 2 + (y - x - 1);
                    const bool v = kept[y] != 0x7fffffff;
                    pp[2 * c] = v ? kept[x] : -1;
                    pp[2 * c + 1] = v ? kept[y] : -1;
                }
        }
    }
}

int edge_queries_per_block(const Problem &p) {
    return kEdgeWaves * edge_queries_per_wave(p.heads_per_graph());
}

hipError_t launch_edges(const Problem &p, const void *q, const void *k, int n, float scale,
                        int topk, int32_t *idx, float *score, int32_t *pairs, hipStream_t st) {
    const int hpg = p.heads_per_graph();
    const dim3 grid((n + edge_queries_per_block(p) - 1) / edge_queries_per_block(p),
                    p.graphs_per_seq(), p.B);
#define CKV_EDGE_CASE(DD, HH)                                                                  \
    if (p.D == DD && hpg == HH) {                                                              \
        hipExtLaunchKernelGGL((edges_kernel<DD, HH>), grid, dim3(kEdgeWaves * kWave), 0, st,   \
                              p.ev_start, p.ev_stop, 0, static_cast<const bf16_t *>(q),        \
                              static_cast<const bf16_t *>(k), n, p.Hq, p.Hkv, p.gpk, p.S,      \
                              scale, topk, idx, score, pairs);                                 \
        return hipGetLastError();                                                              \
    }
    CKV_EDGE_CASE(128, 1) CKV_EDGE_CASE(128, 2) CKV_EDGE_CASE(128, 4) CKV_EDGE_CASE(128, 8)
    CKV_EDGE_CASE(64, 1) CKV_EDGE_CASE(64, 2) CKV_EDGE_CASE(64, 4) CKV_EDGE_CASE(64, 8)
#undef CKV_EDGE_CASE
    return hipErrorInvalidValue;
}

}  // namespace ckv
