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

namespace ckv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kEdgeWaves = 4;
constexpr int kEdgeKT = 64;  // keys per LDS tile
constexpr int kEdgeList = 8; // list length kept per query (largest topk)
constexpr int edge_queries_per_wave(int hpg) { return hpg <= 4 ? 16 : 8; }

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
    static_assert(HPG == 1 || HPG == 2 || HPG == 4 || HPG == 8, "heads per graph");
    static_assert(NQ == 4, "query slots");
    __shared__ __align__(16) bf16_t s_k[kEdgeKT * LDSR];

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
        const int qi = qw + R / HPG, h = R % HPG;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qi < n)
                u = *reinterpret_cast<const uint4 *>(qb + ((size_t)qi * Hq + h0 + h) * D +
                                                     32 * t + 8 * g4);
            a[m][t] = __builtin_bit_cast(bf16x8_t, u);
        }
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

    const int qlast = min(q0 + QPB, n) - 1;  // largest query of the workgroup
    const int wlast = min(qw + QPW, n) - 1;  // ... of this wave
    for (int kt = S; kt < qlast; kt += kEdgeKT) {
        // stage keys kt .. kt+63 (zeros past n)
        __syncthreads();
        constexpr int kChunks = kEdgeKT * D / 8;  // 16-byte pieces of a tile
#pragma unroll
        for (int c = tid; c < kChunks; c += kEdgeWaves * kWave) {
            const int row = c / (D / 8), col = c % (D / 8);
            const int j = kt + row;
            uint4 u = make_uint4(0, 0, 0, 0);
            if (j < n)
                u = *reinterpret_cast<const uint4 *>(kb_ + ((size_t)j * Hkv + kvh) * D + 8 * col);
            *reinterpret_cast<uint4 *>(s_k + row * LDSR + 8 * col) = u;
        }
        __syncthreads();
        for (int sb = 0; sb < kEdgeKT; sb += 16) {
            const int k16 = kt + sb;
            if (k16 >= wlast) break;  // every key from here on is at or past the wave's queries
            // B operand: lane (r16, g4) holds elements 32t + 8g4 .. +8 of key k16 + r16
            bf16x8_t bb[T];
#pragma unroll
            for (int t = 0; t < T; ++t)
                bb[t] = *reinterpret_cast<const bf16x8_t *>(s_k + (sb + r16) * LDSR + 32 * t +
                                                            8 * g4);
            const int j = k16 + r16;  // this lane's accumulator column
            f32x4_t acc[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < T; ++t)
                    acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[m][t], bb[t], acc[m], 0, 0, 0);
            }
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
                    z = j < qpos[s] ? z * scale : -__builtin_inff();
                    const bool ins = z > ts[s][EK - 1];
                    if (__ballot(ins)) {
                        if (ins) edge_insert<true>(ts[s], ti[s], z, j);
                    }
                }
            }
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
