// attn.hip -- indexed split-K flash-decode over the selected tokens, and the
// log-sum-exp merge of the splits.
//
// rit.work post "CommunityKV long-context decoding", token-graph section: the
// chosen communities are loaded from the full (never evicted) KV cache and
// attention is computed exactly over that reduced token set.  For every query head
// h of sequence b, with graph g(h) and index list I_g:
//   o_h = sum_{j in I_g} exp(z_j - max z) V_j / sum_{j in I_g} exp(z_j - max z),
//   z_j = scale * q_h . K_j.
//
// gfx950 design:
// * grid = (NG, splits): the graph index varies fastest, so the workgroups of one
//   graph share an XCD (and its L2) and the short last splits are dispatched last;
//   a graph's list is cut into `nsplit` balanced chunks of <= CH entries.
// * Phase A: each thread resolves one list entry -> page-table lookup -> row index
//   (or -1 when out of range / unmapped), into LDS.
// * Phase B: a K or V row (d*elem bytes, 256 B for bf16 d=128) is read by LPR =
//   row_bytes/16 lanes with one 16-byte load each, so a wave-wide load gathers
//   64/LPR whole rows (1 KiB); every wave issues its 2*NLD loads back to back with
//   no branches (rows of invalid entries point at row 0 and are masked), so with
//   NLD = 12 and 3 waves per SIMD a 128K-token step's whole K/V working set is
//   requested in one round of workgroups.
// * bf16 q.K on the matrix cores: the wave's rows form groups of 16.  A group's K
//   rows pass through a per-wave LDS tile into the B operand of
//   v_mfma_f32_16x16x32_bf16 (exact bf16 products, fp32 sums); the A operand
//   repeats the graph's query heads down its 16 rows, so accumulator register i of
//   lane (row r, quarter t) holds the logit of row r for head (4t + i) % GH.  Each
//   (row, head) then takes one exp, and p reaches the lanes that hold the row's V
//   pieces through LDS.  For d = 128 and up to 4 heads the operands are swapped:
//   the output is indexed (row, head), lane (quarter t, column c) holds rows 4t+i
//   for head c % GH -- the rows whose V pieces the lane reads -- and lane h of each
//   quad holds head h, so p reaches the FMAs by a DPP quad broadcast, not LDS.  The
//   wave keeps one softmax reference per head, rescaled lazily in the log2 domain;
//   P.V is fp32 FMAs on the vector ALUs.
// * fp32 rows: dot products over the LPR lanes of a row with DPP sums, online
//   softmax per row slot.
// * The wave's row slots and then the 4 waves are merged; the workgroup writes one
//   partial (m, l, acc[d]) per head.
// * The merge (next launch, so no device-wide fences are needed) combines the
//   partials: m* = max m_s, l = sum l_s 2^(m_s-m*), o = sum acc_s 2^(m_s-m*) / l.
// * In the fused decode step grid row 0 holds extra workgroups, one wave per
//   graph, that run the local update while the other workgroups stream K/V.
// * A list grid that needs several rounds of resident workgroups (ragged batches:
//   many short lists and a few long ones) runs as one persistent round instead:
//   `workers` workgroups (the launch's capacity) each build the compact list of
//   busy splits (graph g owns items pfx[g] .. pfx[g+1]-1, from the list lengths)
//   and walk it with stride `workers`, after marking the grid's empty split slots
//   for the merge.  No workgroup is dispatched for an empty split, and every slot
//   keeps a busy workgroup until the list runs out.
#include <atomic>
#include <type_traits>

#include "ckv_device.h"
#include "ckv_internal.h"
#include "update_rule.h"

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

// Graph handled by grid column x: for per-head graphs whose count is a multiple of
// 8*gpk, the gpk graphs of a KV head are placed on one XCD (x % 8) so that their
// overlapping lists hit the same L2.
__device__ __forceinline__ int graph_of_column(int x, int NG, int gpk) {
    if (gpk > 1 && NG % (8 * gpk) == 0) {
        const int xcd = x & 7, rest = x >> 3;
        return ((rest / gpk) * 8 + xcd) * gpk + rest % gpk;
    }
    return x;
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Value of lane H of this lane's quad (DPP quad_perm [H,H,H,H]).
__device__ __forceinline__ float quad_bcast(float x, int h) {
    switch (h) {
        case 0: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x00, 0xF, 0xF, false));
        case 1: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x55, 0xF, 0xF, false));
        case 2: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xAA, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xFF, 0xF, 0xF, false));
    }
}

// Maximum over the 16 lanes of a row, in every lane of the row.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    return fmaxf(x, dpp<0x140>(x));
}

struct OpAdd {
    __device__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
    __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// op(x[L], x[L ^ OFF]) in every lane L (the same value in both lanes of a pair),
// for OFF = 8 (DPP rotate by 8 inside a 16-lane row), 16 or 32 (gfx950 lane-swap
// instructions: after the swap the two registers hold the even and the odd
// 16-lane rows, resp. the low and the high 32 lanes, of x in both halves).
template <int OFF, typename Op>
__device__ __forceinline__ float pair_op(float x, Op op) {
    static_assert(OFF == 8 || OFF == 16 || OFF == 32, "pair distance");
    const uint32_t u = __float_as_uint(x);
    if constexpr (OFF == 8) {
        return op(x, __uint_as_float(__builtin_amdgcn_update_dpp(u, u, 0x128, 0xF, 0xF, false)));
    } else if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
}

// Partial q.K over this lane's 4 fp32 elements of a row, for one head.
__device__ __forceinline__ float qk_part_f32(const float (&qf)[4], const uint4 &k) {
    float s = 0.f;
    s = fmaf(qf[0], __uint_as_float(k.x), s);
    s = fmaf(qf[1], __uint_as_float(k.y), s);
    s = fmaf(qf[2], __uint_as_float(k.z), s);
    s = fmaf(qf[3], __uint_as_float(k.w), s);
    return s;
}

// Fused decode step: the local update runs in extra workgroups of this launch.
struct UpdateArgs {
    const void *k_new, *v_new;
    const int32_t *cand;
    int M;
    float *cent;
    const int32_t *num_comms, *comm_start;
    int32_t *comm_size;
    const int32_t *comm_cap;
    int32_t *members;
    int Cmax, NG;
    int32_t *assigned;
    // the layer graph: NG sequences, one update workgroup each (layer_update_seq,
    // its LDS from the update rows' staging area)
    int layer;
};

// What a launch of attn_kernel reads as its token list.
enum AttnMode {
    kAttnIndexed = 0,        // the index list of each graph
    kAttnIndexedUpdate = 1,  // the same, plus the local update in grid row 0
    kAttnDense = 2           // every cached token 0..seq_len-1 (the dense baseline)
};

template <typename T, int D, int GH, int MODE, bool PERSIST>
__global__ __launch_bounds__(256) void attn_kernel(
    const T *__restrict__ q, T *__restrict__ kc, T *__restrict__ vc,
    const int32_t *__restrict__ page_table, int log2ps, int max_pages, int num_pages,
    int32_t *__restrict__ seq_len, const int32_t *__restrict__ idx, int idx_stride,
    int list_div, const int32_t *__restrict__ idx_len, int Hq, int Hkv, int gpk,
    float scale_log2,
    float *__restrict__ part, int max_splits, int chunks_per_wg, int32_t *__restrict__ err,
    UpdateArgs u, int n_graphs, int workers) {
    constexpr int EPL = 16 / sizeof(T);     // row elements per lane
    constexpr int LPR = D / EPL;            // lanes per row
    constexpr int RPW = kWave / LPR;        // rows per wave-wide load
    constexpr int NLD = kAttnLoads;         // loads per wave for K (and for V)
    constexpr int TPW = NLD * RPW;          // tokens per wave
    constexpr int CH = TPW * kAttnWaves;    // tokens per workgroup (max)
    constexpr int kSub = 2;                 // loads per online-softmax batch
    static_assert(CH == attn_chunk(D, sizeof(T)), "chunk");
    static_assert(LPR >= 1 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row split");
    static_assert(NLD % 4 == 0 && NLD % kSub == 0, "row slots are read as int4");

    constexpr bool kMfma = sizeof(T) == 2;  // bf16: q.K on the matrix cores
    // bf16, d = 128, up to 4 heads: the MFMA output is indexed (row, head), so a lane
    // holds the logits of the 4 rows whose V pieces it reads
    constexpr bool kSwap = kMfma && D == 128 && GH <= 4;
    __shared__ __align__(16) int s_row[CH];
    __shared__ float s_m[kAttnWaves][GH];
    __shared__ float s_l[kAttnWaves][GH];
    __shared__ float s_acc[kAttnWaves][GH][D];
    __shared__ __align__(16) float s_p[kAttnWaves][16 * GH];  // bf16 path: p of one group
    // s_big, bf16 path: one tile per wave for the K rows of a 16-row group (16 x D
    // bf16), then the graph's GH query rows (bf16).  In the fused step, grid row 0
    // runs only the local update and uses the same memory for its candidate rows.
    constexpr int kStageFloats = kMfma ? kAttnWaves * 16 * D / 2 + GH * D / 2 : 1;
    constexpr int kUpdFloats = MODE == kAttnIndexedUpdate ? kAttnWaves * kUpdLdsFloats(D) : 1;
    // persistent grid: the busy-split prefix and list length of every graph, after
    // the stage (the update rows' staging overlaps them; those workgroups do no
    // attention)
    constexpr int kPfxInts = PERSIST ? 2 * kAttnPersistMaxGraphs + 1 : 0;
    constexpr int kWorkFloats = kStageFloats + kPfxInts;
    __shared__ __align__(16) float s_big[kWorkFloats > kUpdFloats ? kWorkFloats : kUpdFloats];
    __shared__ int s_wsum[kAttnWaves];
    constexpr bool persist = PERSIST;
    static_assert(!PERSIST || MODE != kAttnDense, "the dense grid is always direct");

    if constexpr (MODE == kAttnIndexedUpdate) {
        // grid row 0: the local update, one wave per graph (dispatched first, so it
        // runs under the K/V stream of the attention workgroups); seq_len advances
        // in the merge launch
        // direct grid: row 0; persistent grid: the workgroups before the workers
        if (persist ? (int)blockIdx.x < (int)gridDim.x - workers : blockIdx.y == 0) {
            if (u.layer) {
                if ((int)blockIdx.x < u.NG)
                    layer_update_seq<T, D>(
                        blockIdx.x, static_cast<const T *>(u.k_new),
                        static_cast<const T *>(u.v_new), u.cand, u.M, u.cent, u.num_comms,
                        u.comm_start, u.comm_size, u.comm_cap, u.members, u.Cmax, Hkv, kc, vc,
                        page_table, log2ps, max_pages, num_pages, seq_len, 0, u.assigned, err,
                        reinterpret_cast<unsigned char *>(s_big));
                return;
            }
            const int w = threadIdx.x / kWave;
            const size_t gu = (size_t)blockIdx.x * kAttnWaves + w;
            if (gu < u.NG)
                graph_update<T, D>(gu, static_cast<const T *>(u.k_new),
                                   static_cast<const T *>(u.v_new), u.cand, u.M, u.cent,
                                   u.num_comms, u.comm_start, u.comm_size, u.comm_cap, u.members,
                                   u.Cmax, Hkv, gpk, kc, vc, page_table, log2ps, max_pages,
                                   num_pages, seq_len, u.assigned, err,
                                   s_big + w * kUpdLdsFloats(D));
            return;
        }
    }
    const int NG = n_graphs;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int G = Hq / Hkv;
    const int span = CH * chunks_per_wg;  // tokens one workgroup may cover
    int *s_pfx = reinterpret_cast<int *>(s_big + kStageFloats);  // [NG + 1]
    int *s_len = s_pfx + kAttnPersistMaxGraphs + 1;               // [NG]
    int item = 0, item_end = 1, item_step = 1;
    if (persist) {
        // list lengths and split counts of all graphs, kPT consecutive graphs per
        // thread, and their exclusive prefix over the workgroup (wave scans by
        // shuffles, then the wave totals)
        constexpr int kPT = (kAttnPersistMaxGraphs + 255) / 256;
        int lens[kPT], cnt[kPT], tsum = 0;
#pragma unroll
        for (int j = 0; j < kPT; ++j) {
            const int gg = tid * kPT + j;
            const int L = gg < NG ? min(idx_len[gg / list_div], idx_stride) : 0;
            lens[j] = L;
            cnt[j] = (L + span - 1) / span;
            tsum += cnt[j];
        }
        int incl = tsum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int v = __shfl_up(incl, o);
            incl += lane >= o ? v : 0;
        }
        if (lane == kWave - 1) s_wsum[w] = incl;
        __syncthreads();
        int off = incl - tsum;
        for (int v = 0; v < w; ++v) off += s_wsum[v];
#pragma unroll
        for (int j = 0; j < kPT; ++j) {
            const int gg = tid * kPT + j;
            if (gg < NG) {
                s_pfx[gg] = off;
                s_len[gg] = lens[j];
            }
            off += cnt[j];
        }
        if (tid == blockDim.x - 1) s_pfx[NG] = off;  // every busy split of the grid
        __syncthreads();
        // empty split slots keep a weight-0 partial for the merge, as in the direct
        // grid; each slot is marked by one thread of the workers
        const int worker = (int)blockIdx.x - ((int)gridDim.x - workers);
        for (int sl = worker * (int)blockDim.x + tid; sl < NG * max_splits;
             sl += workers * (int)blockDim.x) {
            const int gg = sl / max_splits, sp = sl % max_splits;
            if (sp >= s_pfx[gg + 1] - s_pfx[gg]) {
#pragma unroll
                for (int h = 0; h < GH; ++h) {
                    float *pp = part + (((size_t)gg * GH + h) * max_splits + sp) * (D + 2);
                    pp[0] = -__builtin_inff();
                    pp[1] = 0.f;
                }
            }
        }
        item = worker;
        item_end = s_pfx[NG];
        item_step = workers;
    }
    for (; item < item_end; item += item_step) {
    int g, split;
    if (persist) {
        // the graph whose items hold this one: the last g with pfx[g] <= item
        int lo = 0, hi = NG;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pfx[mid] <= item) lo = mid;
            else hi = mid;
        }
        g = lo;
        split = item - s_pfx[g];
    } else {
        g = graph_of_column(blockIdx.x, NG, gpk);
        split = (int)blockIdx.y - (MODE == kAttnIndexedUpdate ? 1 : 0);
    }
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int h0 = kvh * G + (gpk == 1 ? 0 : g % gpk);
    // bf16: the graph's GH query rows (one 16-byte piece per thread) are requested
    // first and stored to LDS only after phase A's loads, so that their round trip
    // runs beside the list's instead of ahead of it
    static_assert(!kMfma || GH * D / 8 <= 256, "one query piece per thread");
    uint4 qv = make_uint4(0, 0, 0, 0);
    if constexpr (kMfma)
        qv = reinterpret_cast<const uint4 *>(q + ((size_t)b * Hq + h0) * D)[min(tid, GH * D / 8 - 1)];
    const int n = seq_len[b];
    // index list of this graph (one list serves list_div consecutive graphs)
    const int gl = g / list_div;
    const int len = persist ? s_len[g] : MODE == kAttnDense ? n : min(idx_len[gl], idx_stride);
    const int nsplit = (len + span - 1) / span;
    if (!persist && split >= nsplit) {
        // an empty split still marks its partial (weight 0) so the merge can read
        // every split without knowing the list length
        if (tid < GH) {
            float *pp = part + (((size_t)g * GH + tid) * max_splits + split) * (D + 2);
            pp[0] = -__builtin_inff();
            pp[1] = 0.f;
        }
        return;
    }
    // balanced cut of the list into nsplit pieces of at most `span` tokens
    const int t_begin = (int)(((long long)len * split) / nsplit);
    const int t_end = (int)(((long long)len * (split + 1)) / nsplit);
    const int ls = lane % LPR;  // slice of the row this lane reads
    const int rs = lane / LPR;  // row slot inside a wave-wide load

    // bf16 rows: q.K of 16 rows at a time on the matrix cores; fp32 rows: dot
    // products on the vector ALUs (below)
    const int r16 = lane & 15, t4 = lane >> 4;  // matrix-core lane coordinates

    // fp32 query slice of this lane; the scale is applied to the sum
    float qf[GH][EPL];
    // matrix-core A operand (bf16): row r16 is head r16 % GH (the heads repeat down
    // the 16 rows), k-block j of 32 elements, this lane's 8 at 32j + 8*t4.  The GH
    // query rows wait in LDS behind the K tiles and are read per group, which keeps
    // 16 registers free for loads in flight.
    constexpr int KB = kMfma ? D / 32 : 1;
    const uint4 *s_q = reinterpret_cast<const uint4 *>(s_big + kAttnWaves * 16 * D / 2);
    if constexpr (!kMfma) {
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            const uint4 u =
                *reinterpret_cast<const uint4 *>(q + ((size_t)b * Hq + h0 + h) * D + ls * EPL);
            qf[h][0] = __uint_as_float(u.x); qf[h][1] = __uint_as_float(u.y);
            qf[h][2] = __uint_as_float(u.z); qf[h][3] = __uint_as_float(u.w);
        }
    }

    // fp32 path: running (m, l, acc) of this lane's row slot
    float m[GH], l[GH], acc[GH][EPL];
    // bf16 path: one reference per head for the whole wave (mv, in the scaled log2
    // domain), and lane partial sums of p; register i of a lane serves head
    // (4*t4 + i) % GH, the head of accumulator row 4*t4 + i
    float mv[4], thr[4], lsum[4];
    float mv0 = -__FLT_MAX__, thr0 = -__FLT_MAX__, lsum0 = 0.f;  // swap layout: one head per lane
    constexpr float kLazy = 8.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // finite start: z > thr holds for every finite logit, and 2^(-inf - mv) = 0
        mv[i] = -__FLT_MAX__;
        thr[i] = -__FLT_MAX__;
        lsum[i] = 0.f;
    }
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        m[h] = -__builtin_inff();
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }
    // one chunk of at most CH tokens [c0, c_end): rows to LDS, then the K/V rows of
    // this wave, folded into the running state
    auto chunk = [&](const int c0, const int c_end) {
    // ---- phase A: list entries -> row indices in LDS
    // both loads at clamped slots, unconditionally (a load under a branch makes the
    // compiler wait for it there); validity is decided by selects afterwards.
    // c0 < c_end <= idx_stride, so the clamped list slot is always in the list.
    for (int t = tid; t < CH; t += blockDim.x) {
        const int te = c0 + t;
        const bool in = te < c_end;
        const int pos = MODE == kAttnDense ? te : idx[(size_t)gl * idx_stride + min(te, c_end - 1)];
        const bool pos_ok = in & (pos >= 0) & (pos < n);
        const int lp = pos_ok ? pos >> log2ps : 0;
        const int pg = page_table[(size_t)b * max_pages + min(lp, max_pages - 1)];
        const bool pg_ok = pos_ok & (lp < max_pages) & (pg >= 0) & (pg < num_pages);
        s_row[t] = pg_ok ? ((pg * Hkv + kvh) << log2ps) + (pos & ((1 << log2ps) - 1)) : -1;
        if (in & !pos_ok) set_err(err, CKV_DEVERR_INDEX_RANGE);
        if (pos_ok & !pg_ok) set_err(err, CKV_DEVERR_UNMAPPED_PAGE);
    }
    if constexpr (kMfma) {
        // the query rows, requested at the start (visible after this barrier)
        if (c0 == t_begin && tid < GH * D / 8)
            reinterpret_cast<uint4 *>(s_big + kAttnWaves * 16 * D / 2)[tid] = qv;
    }
    __syncthreads();

    if constexpr (kMfma) {
        // ---- phase B (bf16).  The wave's TPW tokens form NGRP groups of 16 rows.
        // K and V rows are both read whole, LPR lanes per row and RPW rows per load;
        // lane slot rs takes rows rs*VL .. rs*VL + VL-1 of a group.  Each group's K
        // rows then pass through this wave's LDS tile into the MFMA B operand: lane
        // (r16, t4) needs row r16, elements 32j + 8*t4 .. +7 for k-block j.  The
        // 16-byte pieces of row r sit at slot (piece ^ swz(r)) in the tile, so both
        // the row-wise writes and the column-wise reads spread over all banks.
        constexpr int NGRP = TPW / 16;
        constexpr int VL = 16 / RPW;
        static_assert(TPW % 16 == 0 && VL == KB && NGRP * VL == NLD, "group shape");
        const int *sw = s_row + w * TPW;
        int vrow[NGRP][VL];
#pragma unroll
        for (int gi = 0; gi < NGRP; ++gi) {
            if constexpr (VL == 4) {
                const int4 r4 = *reinterpret_cast<const int4 *>(sw + 16 * gi + rs * VL);
                vrow[gi][0] = r4.x; vrow[gi][1] = r4.y; vrow[gi][2] = r4.z; vrow[gi][3] = r4.w;
            } else {
                static_assert(VL == 2, "V loads per group");
                const int2 r2 = *reinterpret_cast<const int2 *>(sw + 16 * gi + rs * VL);
                vrow[gi][0] = r2.x; vrow[gi][1] = r2.y;
            }
        }
        // validity of the row this lane scores (row r16 of each group)
        uint32_t kvalid = 0;
#pragma unroll
        for (int gi = 0; gi < NGRP; ++gi) kvalid |= (sw[16 * gi + r16] >= 0 ? 1u : 0u) << gi;
        uint32_t rvalid = 0;  // swap layout: rows 4*t4 .. 4*t4+3 of each group
        if constexpr (kSwap) {
#pragma unroll
            for (int gi = 0; gi < NGRP; ++gi) {
                const int4 r4 = *reinterpret_cast<const int4 *>(sw + 16 * gi + 4 * t4);
                rvalid |= ((r4.x >= 0 ? 1u : 0u) | (r4.y >= 0 ? 2u : 0u) | (r4.z >= 0 ? 4u : 0u) |
                           (r4.w >= 0 ? 8u : 0u)) << (4 * gi);
            }
        }
        // all loads in flight together, K then V of each group in turn, so the
        // first group can start while the later ones arrive
        uint4 kr[NGRP][VL], vr[NGRP][VL];
#pragma unroll
        for (int gi = 0; gi < NGRP; ++gi) {
#pragma unroll
            for (int jj = 0; jj < VL; ++jj)
                kr[gi][jj] = load_nt(kc + (size_t)(vrow[gi][jj] < 0 ? 0 : vrow[gi][jj]) * D +
                                     ls * EPL);
#pragma unroll
            for (int jj = 0; jj < VL; ++jj)
                vr[gi][jj] = load_nt(vc + (size_t)(vrow[gi][jj] < 0 ? 0 : vrow[gi][jj]) * D +
                                     ls * EPL);
        }
        __builtin_amdgcn_sched_barrier(0);

        // swz(r): 16-byte slot rotation of tile row r (LPR slots per row)
        constexpr int kSwzShift = LPR == 16 ? 0 : LPR == 8 ? 1 : -1;
        static_assert(kSwzShift >= 0, "tile rows of 8 or 16 pieces");
        uint4 *tile = reinterpret_cast<uint4 *>(s_big) + w * 16 * LPR;
        float *sp = s_p[w];
#pragma unroll
        for (int gi = 0; gi < NGRP; ++gi) {
            // K rows of the group through the tile
#pragma unroll
            for (int jj = 0; jj < VL; ++jj) {
                const int r = rs * VL + jj;
                tile[r * LPR + (ls ^ ((r >> kSwzShift) & (LPR - 1)))] = kr[gi][jj];
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            uint4 kb[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j)
                kb[j] = tile[r16 * LPR + ((4 * j + t4) ^ ((r16 >> kSwzShift) & (LPR - 1)))];
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if constexpr (kSwap) {
                // C[row][col] = K_row . q_{col % GH}: lane (t4, r16) gets rows 4*t4 + i
                // for head r16 % GH; the heads repeat every 4 columns, so lane j of each
                // quad holds head j
                f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KB; ++j)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, kb[j]),
                        __builtin_bit_cast(bf16x8_t, s_q[(r16 % GH) * (D / 8) + 4 * j + t4]), c,
                        0, 0, 0);
                float z[4];
                bool need = false;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[i] = (rvalid >> (4 * gi + i)) & 1u ? c[i] * scale_log2 : -__builtin_inff();
                    need |= z[i] > thr0;
                }
                if (__builtin_amdgcn_ballot_w64(need) != 0) {
                    // this head's maximum over the 16 rows: the lane's 4, then the 4 quarters
                    float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
                    mx = pair_op<16>(mx, OpMax{});
                    mx = pair_op<32>(mx, OpMax{});
                    const float mn = fmaxf(mv0, mx);
                    const float cf = fast_exp2(mv0 - mn);
                    mv0 = mn;
                    thr0 = mn + kLazy;
                    lsum0 *= cf;
#pragma unroll
                    for (int h = 0; h < GH; ++h) {
                        const float f = GH == 1 ? cf : quad_bcast(cf, h);
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[h][e] *= f;
                    }
                }
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(z[i] - mv0);
                    lsum0 += p[i];
                }
                // V lane (t4, ls) reads rows 4*t4 + jj: the rows of p[jj]; head h's weight
                // comes from lane h of the lane's quad
#pragma unroll
                for (int jj = 0; jj < VL; ++jj) {
                    float x[EPL];
                    unpack<T, EPL>(vr[gi][jj], x);
#pragma unroll
                    for (int h = 0; h < GH; ++h) {
                        const float ph = GH == 1 ? p[jj] : quad_bcast(p[jj], h);
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(ph, x[e], acc[h][e]);
                    }
                }
                continue;
            }
            // S[4*t4 + i][r16] = q_head . K_row over KB k-blocks
            f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KB; ++j)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, s_q[(r16 % GH) * (D / 8) + 4 * j + t4]),
                    __builtin_bit_cast(bf16x8_t, kb[j]), c, 0, 0, 0);
            const bool ok = (kvalid >> gi) & 1u;
            float z[4];
            bool need = false;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                z[i] = ok ? c[i] * scale_log2 : -__builtin_inff();
                need |= z[i] > thr[i];
            }
            // lazy reference: (l, acc) are rescaled only when a logit of the wave
            // passes its head's reference by more than 2^kLazy, so p <= 2^kLazy
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                float cf[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float mn = fmaxf(mv[i], row_max16(z[i]));
                    cf[i] = fast_exp2(mv[i] - mn);
                    mv[i] = mn;
                    thr[i] = mn + kLazy;
                    lsum[i] *= cf[i];
                }
                float hf[GH];  // the factor of each head, in every lane
                if constexpr (GH <= 4) {
#pragma unroll
                    for (int h = 0; h < GH; ++h) hf[h] = cf[h];
                } else {
                    // heads 0-3 sit in even 16-lane rows, 4-7 in odd ones
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t u = __float_as_uint(cf[i]);
                        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
                        hf[i] = __uint_as_float(r[0]);
                        hf[4 + i] = __uint_as_float(r[1]);
                    }
                }
#pragma unroll
                for (int h = 0; h < GH; ++h)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] *= hf[h];
            }
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(z[i] - mv[i]);
                lsum[i] += p[i];
            }
            // p of (row r16, head) to the wave's LDS slots, read back in the V layout
            // (lanes repeating a head store the same value)
            if constexpr (GH == 8)
                *reinterpret_cast<float4 *>(sp + r16 * 8 + 4 * (t4 & 1)) =
                    make_float4(p[0], p[1], p[2], p[3]);
            else if constexpr (GH == 4)
                *reinterpret_cast<float4 *>(sp + r16 * 4) = make_float4(p[0], p[1], p[2], p[3]);
            else if constexpr (GH == 2)
                *reinterpret_cast<float2 *>(sp + r16 * 2) = make_float2(p[0], p[1]);
            else
                sp[r16] = p[0];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
            for (int jj = 0; jj < VL; ++jj) {
                const float *pr = sp + (rs * VL + jj) * GH;
                float pv[GH];
#pragma unroll
                for (int h = 0; h < GH; ++h) pv[h] = pr[h];
                float x[EPL];
                unpack<T, EPL>(vr[gi][jj], x);
#pragma unroll
                for (int h = 0; h < GH; ++h)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pv[h], x[e], acc[h][e]);
            }
            // the next group's stores must not overtake these loads
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    } else {
    // ---- phase B (fp32): this lane's NLD row slots are contiguous in LDS
    int rows[NLD];
    {
        const int4 *sr = reinterpret_cast<const int4 *>(s_row + w * TPW + rs * NLD);
#pragma unroll
        for (int i = 0; i < NLD / 4; ++i) {
            const int4 r4 = sr[i];
            rows[4 * i + 0] = r4.x;
            rows[4 * i + 1] = r4.y;
            rows[4 * i + 2] = r4.z;
            rows[4 * i + 3] = r4.w;
        }
    }
    uint32_t valid = 0;
#pragma unroll
    for (int i = 0; i < NLD; ++i) valid |= (rows[i] >= 0 ? 1u : 0u) << i;
    uint4 kr[NLD], vr[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i)
        kr[i] = load_nt(kc + (size_t)(rows[i] < 0 ? 0 : rows[i]) * D + ls * EPL);
#pragma unroll
    for (int i = 0; i < NLD; ++i)
        vr[i] = load_nt(vc + (size_t)(rows[i] < 0 ? 0 : rows[i]) * D + ls * EPL);
    // all 2*NLD row loads stay in flight together: without this fence the
    // scheduler sinks most of them below the first softmax batch, which splits
    // the gather into dependent round trips
    __builtin_amdgcn_sched_barrier(0);

    // online softmax over batches of kSub loads; m, l, acc are per row slot.  m is
    // a reference, not necessarily the running maximum: (l, acc) are rescaled only
    // when a logit exceeds it by more than 2^kLazy (so p = 2^(z-m) <= 2^kLazy and
    // acc stays far from fp32 overflow); (m, l, acc) always describe the same sum.
    // Rows past the chunk's end take no part (z = -inf, p = 0).
#pragma unroll
    for (int i0 = 0; i0 < NLD; i0 += kSub) {
        float z[kSub][GH];
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                const float s = group_sum<LPR>(qk_part_f32(qf[h], kr[i0 + j]));
                z[j][h] = (valid >> (i0 + j)) & 1u ? s * scale_log2 : -__builtin_inff();
            }
        }
#pragma unroll
        for (int h = 0; h < GH; ++h) {
            float mn = m[h];
#pragma unroll
            for (int j = 0; j < kSub; ++j) mn = fmaxf(mn, z[j][h]);
            if (mn > m[h] + kLazy) {
                const float c = fast_exp2(m[h] - mn);  // 0 when m was -inf
                l[h] *= c;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] *= c;
                m[h] = mn;
            }
        }
#pragma unroll
        for (int j = 0; j < kSub; ++j) {
            float x[EPL];
            unpack<T, EPL>(vr[i0 + j], x);
#pragma unroll
            for (int h = 0; h < GH; ++h) {
                float p = fast_exp2(z[j][h] - m[h]);
                p = (valid >> (i0 + j)) & 1u ? p : 0.f;
                l[h] += p;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, x[e], acc[h][e]);
            }
        }
    }
    }
    };
    if constexpr (MODE == kAttnDense) {
        for (int c0 = t_begin; c0 < t_end; c0 += CH) {
            if (c0 != t_begin) __syncthreads();  // every wave has read s_row
            chunk(c0, min(c0 + CH, t_end));
        }
    } else {
        chunk(t_begin, t_end);  // an indexed piece is one chunk
    }
    if constexpr (kMfma) {
        // one reference per head: the RPW row slots of acc simply add up; l is the
        // sum of p over the 16 rows of a 16-lane row
        if constexpr (LPR == 16) {
            // reduce-scatter over the 4 row slots: a lane swap of two registers
            // followed by one add sums both over row pairs (xor 16, then xor 32), so
            // register 4q + rho ends up summed in 16-lane row rho of T[q]
            constexpr int NR = GH * EPL;
            static_assert(NR % 4 == 0, "acc registers in fours");
            float *a = &acc[0][0];
            float S[NR / 2], Tq[NR / 4];
#pragma unroll
            for (int k = 0; k < NR / 2; ++k) {
                const auto r = __builtin_amdgcn_permlane16_swap(
                    __float_as_uint(a[2 * k]), __float_as_uint(a[2 * k + 1]), false, false);
                S[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            }
#pragma unroll
            for (int k = 0; k < NR / 4; ++k) {
                const auto r = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(S[2 * k]), __float_as_uint(S[2 * k + 1]), false, false);
                Tq[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            }
            // lane (rho = rs, ls) holds element ls*EPL + (4q + rho) % EPL of head
            // (4q + rho) / EPL in Tq[q]
#pragma unroll
            for (int k = 0; k < NR / 4; ++k) {
                const int reg = 4 * k + rs;
                s_acc[w][reg / EPL][ls * EPL + reg % EPL] = Tq[k];
            }
        } else {
#pragma unroll
            for (int h = 0; h < GH; ++h) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    if constexpr (LPR <= 8) acc[h][e] = pair_op<8>(acc[h][e], OpAdd{});
                    if constexpr (LPR <= 16) acc[h][e] = pair_op<16>(acc[h][e], OpAdd{});
                    acc[h][e] = pair_op<32>(acc[h][e], OpAdd{});
                }
            }
            if (lane < LPR) {
#pragma unroll
                for (int h = 0; h < GH; ++h)
#pragma unroll
                    for (int e = 0; e < EPL; ++e) s_acc[w][h][lane * EPL + e] = acc[h][e];
            }
        }
        float lt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lt[i] = group_sum<16>(lsum[i]);
        if constexpr (kSwap) {
            // l of head r16 % GH: the lane's rows, then the 4 quarters
            float l0 = pair_op<16>(lsum0, OpAdd{});
            l0 = pair_op<32>(l0, OpAdd{});
            if (t4 == 0 && r16 < GH) {
                s_m[w][r16] = mv0;
                s_l[w][r16] = l0;
            }
        } else
        // lane 0 holds heads 0..min(GH,4)-1, lane 16 heads 4-7
        if (r16 == 0 && t4 < (GH > 4 ? 2 : 1)) {
#pragma unroll
            for (int i = 0; i < (GH < 4 ? GH : 4); ++i) {
                s_m[w][4 * t4 + i] = mv[i];
                s_l[w][4 * t4 + i] = lt[i];
            }
        }
    } else {
    // merge the RPW row slots of the wave (same dims, disjoint tokens, own maxima);
    // lanes L and L^off pair up with VALU lane swaps, no LDS round trips
#pragma unroll
    for (int h = 0; h < GH; ++h) {
        float mm = m[h];
        if constexpr (LPR <= 8) mm = pair_op<8>(mm, OpMax{});
        if constexpr (LPR <= 16) mm = pair_op<16>(mm, OpMax{});
        mm = pair_op<32>(mm, OpMax{});
        const float c = mm == -__builtin_inff() ? 0.f : fast_exp2(m[h] - mm);
        l[h] *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= c;
        m[h] = mm;
        if constexpr (LPR <= 8) {
            l[h] = pair_op<8>(l[h], OpAdd{});
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = pair_op<8>(acc[h][e], OpAdd{});
        }
        if constexpr (LPR <= 16) {
            l[h] = pair_op<16>(l[h], OpAdd{});
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = pair_op<16>(acc[h][e], OpAdd{});
        }
        l[h] = pair_op<32>(l[h], OpAdd{});
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = pair_op<32>(acc[h][e], OpAdd{});
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
    if (persist) __syncthreads();  // the next item reuses the workgroup's LDS
    }
}

// Merge of one graph's split partials into out, in one 512-thread workgroup (the
// layer graph's merge launch, whose extra workgroups run its update) (m* = max m_s, weights
// 2^(m_s - m*) / sum_s l_s 2^(m_s - m*)).  Every split slot holds a valid (m, l)
// -- empty splits carry m = -inf -- so all loads are issued at once, without first
// reading the list length; acc values of weight-0 splits are never used.
template <int D, int GH>
__device__ __forceinline__ void merge_graph(int g, int Hq, int Hkv, int gpk,
                                            float *__restrict__ out,
                                            const float *__restrict__ part, int max_splits,
                                            float *s_w) {
    constexpr int kBatch = 32;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int G = Hq / Hkv;
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int h0 = kvh * G + (gpk == 1 ? 0 : g % gpk);
    const float *pbase = part + ((size_t)g * GH * max_splits) * (D + 2);
    // this thread's output element and the first batch of its partial values
    const int t0 = tid < GH * D ? tid : 0;
    const int h = t0 / D, i = t0 % D;
    const float *pa = pbase + (size_t)h * max_splits * (D + 2) + 2 + i;
    // loads at clamped slots, unconditionally: a load inside a branch would make the
    // compiler wait for each one in turn
    float x[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) x[k] = pa[(size_t)min(k, max_splits - 1) * (D + 2)];
    // weights: one wave per head
    for (int hh = w; hh < GH; hh += blockDim.x / kWave) {
        const float *ph = pbase + (size_t)hh * max_splits * (D + 2);
        if (max_splits <= kWave) {
            // one split per lane: (m, l) fetched once, reduced with DPP
            float2 ml = make_float2(-__builtin_inff(), 0.f);
            if (lane < max_splits) ml = *reinterpret_cast<const float2 *>(ph + (size_t)lane * (D + 2));
            const float mm = wave_max_f(ml.x);
            const float f = ml.x == -__builtin_inff() ? 0.f : fast_exp2(ml.x - mm);
            const float ll = wave_sum_f(ml.y * f);
            const float inv = ll > 0.f ? 1.f / ll : 0.f;
            if (lane < max_splits) s_w[hh * max_splits + lane] = f * inv;
            continue;
        }
        float mm = -__builtin_inff();
        for (int s = lane; s < max_splits; s += kWave) mm = fmaxf(mm, ph[(size_t)s * (D + 2)]);
        mm = wave_max_f(mm);
        float ll = 0.f;
        for (int s = lane; s < max_splits; s += kWave) {
            const float ms = ph[(size_t)s * (D + 2)];
            const float f = ms == -__builtin_inff() ? 0.f : fast_exp2(ms - mm);
            s_w[hh * max_splits + s] = f;
            ll += ph[(size_t)s * (D + 2) + 1] * f;
        }
        ll = wave_sum_f(ll);
        const float inv = ll > 0.f ? 1.f / ll : 0.f;
        for (int s = lane; s < max_splits; s += kWave) s_w[hh * max_splits + s] *= inv;
    }
    __syncthreads();
    // GH*D output elements over the workgroup's threads (more than one per thread
    // when GH*D exceeds the workgroup: 8 heads x 128); the first element's first
    // batch was loaded above
    for (int t = tid; t < GH * D; t += blockDim.x) {
        const int ht = t / D, it = t % D;
        const float *pt = pbase + (size_t)ht * max_splits * (D + 2) + 2 + it;
        float a = 0.f;
        for (int s0 = 0; s0 < max_splits; s0 += kBatch) {
            if (s0 > 0 || t != tid) {
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    x[k] = pt[(size_t)min(s0 + k, max_splits - 1) * (D + 2)];
            }
            // weight 0 (an empty split, or a slot past the last) contributes nothing,
            // whatever its never-written acc holds; selects, no branches
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float wk = s_w[ht * max_splits + min(s0 + k, max_splits - 1)];
                const bool use = (s0 + k < max_splits) & (wk != 0.f);
                const float term = x[k] * wk;
                a += use ? term : 0.f;
            }
        }
        out[((size_t)b * Hq + h0 + ht) * D + it] = a;
    }
}

// Merge of one head's split partials into out (m* = max m_s, weights
// 2^(m_s - m*) / sum_s l_s 2^(m_s - m*)): one single-wave workgroup per 64 output
// elements of a (graph, head), one element per lane (many small workgroups: the
// launch is a single load round trip, and this grid starts and drains sooner than
// one workgroup per graph).  With up to 64 splits, lane s derives split s's weight
// and the FMAs take it by readlane (no LDS, no barrier); more splits go through
// LDS.  Every split slot holds a valid (m, l) -- empty splits carry m = -inf -- so
// all loads are issued at once, without first reading the list length; acc values
// of weight-0 splits are never used.  With seq_len_bump (fused decode step) the
// first workgroup of every sequence also advances seq_len, after the step's update
// has been made.
template <int D, int GH>
__global__ __launch_bounds__(kWave) void merge_kernel(int Hq, int Hkv, int gpk,
                                                      float *__restrict__ out,
                                                      const float *__restrict__ part,
                                                      int max_splits,
                                                      int32_t *__restrict__ seq_len_bump) {
    extern __shared__ float s_w[];
    static_assert(D % kWave == 0, "whole waves per head");
    constexpr int kBatch = 32;
    constexpr int WPH = D / kWave;  // workgroups per head
    const int g = blockIdx.x / (GH * WPH), hh = (blockIdx.x / WPH) % GH;
    const int lane = threadIdx.x;
    const int i = (blockIdx.x % WPH) * kWave + lane;
    const int G = Hq / Hkv;
    const int b = g / (Hkv * gpk);
    const int kvh = (g / gpk) % Hkv;
    const int h0 = kvh * G + (gpk == 1 ? 0 : g % gpk);
    const float *ph = part + ((size_t)g * GH + hh) * max_splits * (D + 2);
    // loads at clamped slots, unconditionally: a load inside a branch would make the
    // compiler wait for each one in turn
    float x[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) x[k] = ph[(size_t)min(k, max_splits - 1) * (D + 2) + 2 + i];
    float a = 0.f;
    if (max_splits <= kWave) {
        // lane s: split s's weight
        float2 ml = make_float2(-__builtin_inff(), 0.f);
        if (lane < max_splits) ml = *reinterpret_cast<const float2 *>(ph + (size_t)lane * (D + 2));
        const float mm = wave_max_f(ml.x);
        const float f = ml.x == -__builtin_inff() ? 0.f : fast_exp2(ml.x - mm);
        const float ll = wave_sum_f(ml.y * f);
        const float wl = ll > 0.f ? f / ll : 0.f;
#pragma unroll
        for (int s0 = 0; s0 < kWave; s0 += kBatch) {
            if (s0 >= max_splits) break;
            if (s0 > 0) {
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    x[k] = ph[(size_t)min(s0 + k, max_splits - 1) * (D + 2) + 2 + i];
            }
            // weight 0 (an empty split, or a slot past the last) contributes nothing,
            // whatever its never-written acc holds; selects, no branches
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s0 + k));
                const bool use = (s0 + k < max_splits) & (wk != 0.f);
                const float term = x[k] * wk;
                a += use ? term : 0.f;
            }
        }
    } else {
        float mm = -__builtin_inff();
        for (int s = lane; s < max_splits; s += kWave) mm = fmaxf(mm, ph[(size_t)s * (D + 2)]);
        mm = wave_max_f(mm);
        float ll = 0.f;
        for (int s = lane; s < max_splits; s += kWave) {
            const float ms = ph[(size_t)s * (D + 2)];
            const float f = ms == -__builtin_inff() ? 0.f : fast_exp2(ms - mm);
            s_w[s] = f;
            ll += ph[(size_t)s * (D + 2) + 1] * f;
        }
        ll = wave_sum_f(ll);
        const float inv = ll > 0.f ? 1.f / ll : 0.f;
        for (int s = lane; s < max_splits; s += kWave) s_w[s] *= inv;
        __syncthreads();
        for (int s0 = 0; s0 < max_splits; s0 += kBatch) {
            if (s0 > 0) {
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    x[k] = ph[(size_t)min(s0 + k, max_splits - 1) * (D + 2) + 2 + i];
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const float wk = s_w[min(s0 + k, max_splits - 1)];
                const bool use = (s0 + k < max_splits) & (wk != 0.f);
                const float term = x[k] * wk;
                a += use ? term : 0.f;
            }
        }
    }
    out[((size_t)b * Hq + h0 + hh) * D + i] = a;
    // after the merge, as an add that returns nothing: a read of seq_len first would
    // hold this workgroup's partial loads behind its round trip
    if (seq_len_bump && lane == 0 && blockIdx.x % (GH * WPH) == 0 && g % (Hkv * gpk) == 0)
        __hip_atomic_fetch_add(seq_len_bump + g / (Hkv * gpk), 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroups of attn_kernel<T, D, GH, MODE> resident on the current device at
// once (queried once per device and instance; 0 if the query fails).
template <typename T, int D, int GH, int MODE>
static int attn_persist_capacity() {
    constexpr int kDevices = 64;
    static std::atomic<int> cache[kDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 0;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<T, D, GH, MODE, true>,
                                                     256, 0) != hipSuccess ||
        per_cu <= 0)
        return 0;
    c = per_cu * device_cu_count();
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <typename T, int D, int GH, int MODE>
static void launch_partials_t(const Problem &p, const void *q, const ckv_kv &kv,
                              const int32_t *idx, int idx_stride, const int32_t *idx_len,
                              float scale, float *partials, int32_t *err, const UpdateArgs &u,
                              int ms, int cpw, hipStream_t st) {
    const int NG = p.NG();
    const int upd_wgs = MODE != kAttnIndexedUpdate ? 0
                        : u.layer                  ? u.NG
                                                   : (NG + kAttnWaves - 1) / kAttnWaves;
    // a list grid larger than one round of resident workgroups runs persistent (group
    // graphs only: per-head graphs keep the direct grid's column order, which puts
    // the graphs of a KV head on one XCD)
    if constexpr (MODE != kAttnDense) {
        if (p.gpk == 1 && NG <= kAttnPersistMaxGraphs) {
            const int cap = attn_persist_capacity<T, D, GH, MODE>();
            if ((long long)NG * ms + upd_wgs > cap && cap > upd_wgs) {
                const int workers = cap - upd_wgs;
                hipExtLaunchKernelGGL(
                    (attn_kernel<T, D, GH, MODE, true>), dim3(upd_wgs + workers), dim3(256), 0,
                    st, p.ev_start, p.ev_stop, 0, static_cast<const T *>(q),
                    static_cast<T *>(kv.k), static_cast<T *>(kv.v), kv.page_table,
                    log2_pow2(kv.page_size), kv.max_pages_per_seq, kv.num_pages, kv.seq_len, idx,
                    idx_stride, p.list_div, idx_len, p.Hq, p.Hkv, p.gpk, scale * kLog2e, partials,
                    ms, cpw, err, u, NG, workers);
                return;
            }
        }
    }
    hipExtLaunchKernelGGL((attn_kernel<T, D, GH, MODE, false>),
                          dim3(NG, ms + (MODE == kAttnIndexedUpdate ? 1 : 0)), dim3(256), 0, st,
                          p.ev_start, p.ev_stop, 0, static_cast<const T *>(q),
                          static_cast<T *>(kv.k), static_cast<T *>(kv.v), kv.page_table,
                          log2_pow2(kv.page_size), kv.max_pages_per_seq, kv.num_pages,
                          kv.seq_len, idx, idx_stride, p.list_div, idx_len, p.Hq, p.Hkv, p.gpk,
                          scale * kLog2e, partials, ms, cpw, err, u, NG, 0);
}

// One launcher for the three modes; GH = heads per graph of `p`.
static hipError_t launch_mode(const Problem &p, int mode, const void *q, const ckv_kv &kv,
                              const int32_t *idx, int idx_stride, const int32_t *idx_len,
                              float scale, float *partials, int32_t *err, const UpdateArgs &u,
                              int ms, int cpw, hipStream_t st) {
    const int GH = p.heads_per_graph();
#define CKV_ATTN_CASE(TT, DT, DD, HH)                                                          \
    if (p.dtype == DT && p.D == DD && GH == HH) {                                              \
        if (mode == kAttnIndexedUpdate)                                                        \
            launch_partials_t<TT, DD, HH, kAttnIndexedUpdate>(p, q, kv, idx, idx_stride,       \
                                                              idx_len, scale, partials, err,   \
                                                              u, ms, cpw, st);                 \
        else if (mode == kAttnDense)                                                           \
            launch_partials_t<TT, DD, HH, kAttnDense>(p, q, kv, idx, idx_stride, idx_len,      \
                                                      scale, partials, err, u, ms, cpw, st);   \
        else                                                                                   \
            launch_partials_t<TT, DD, HH, kAttnIndexed>(p, q, kv, idx, idx_stride, idx_len,    \
                                                        scale, partials, err, u, ms, cpw, st); \
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

bool layer_update_in_attention_fits(const Problem &p, int n_cand) {
    // the update rows' staging area of the attention launch: kAttnWaves wave slots
    const size_t area = (size_t)kAttnWaves * kUpdLdsFloats(p.D) * sizeof(float);
    return p.layer() && layer_update_fits(p, n_cand) &&
           layer_update_lds(p.cdim(), n_cand, p.Hkv) <= area;
}

hipError_t launch_attn_partials(const Problem &pg, const void *q, const ckv_kv &kv,
                                const int32_t *idx, int idx_stride, const int32_t *idx_len,
                                float scale, float *partials, int32_t *err, const UpdateSpec *upd,
                                hipStream_t st) {
    // the layer graph's update runs here only when its staging fits the launch's
    // update rows (else the merge launch takes it)
    if (upd && pg.layer() && !layer_update_in_attention_fits(pg, upd->n_cand))
        return hipErrorInvalidValue;
    const Problem p = attn_problem(pg);
    UpdateArgs u{};
    if (upd) {
        u = UpdateArgs{upd->k_new, upd->v_new, upd->cand, upd->n_cand, upd->graphs->centroids,
                       upd->graphs->num_comms, upd->graphs->comm_start, upd->graphs->comm_size,
                       upd->graphs->comm_cap, upd->graphs->members, p.Cmax,
                       pg.layer() ? pg.B : p.NG(), upd->assigned, pg.layer() ? 1 : 0};
    }
    return launch_mode(p, upd ? kAttnIndexedUpdate : kAttnIndexed, q, kv, idx, idx_stride,
                       idx_len, scale, partials, err, u, attn_max_splits(p, idx_stride), 1, st);
}

hipError_t launch_dense_partials(const Problem &p, const void *q, const ckv_kv &kv, float scale,
                                 float *partials, int32_t *err, hipStream_t st) {
    const Problem pd = dense_problem(p);
    int cpw = 1;
    const int ms = dense_max_splits(pd, kv, &cpw);
    return launch_mode(pd, kAttnDense, q, kv, nullptr, 0, nullptr, scale, partials, err,
                       UpdateArgs{}, ms, cpw, st);
}

// The layer graph's merge launch also runs the step's update: B extra workgroups,
// one per sequence, each running the layer update (which advances its sequence's
// seq_len itself, after reading n).  The update writes centroids, member lists and
// K/V row n, none of which the merge reads; the merge reads only the partials.
struct LayerUpdArgs {
    const void *k_new, *v_new;
    const int32_t *cand;
    int M;
    float *cent;
    const int32_t *num_comms, *comm_start;
    int32_t *comm_size;
    const int32_t *comm_cap;
    int32_t *members;
    int Cmax, Hkv;
    void *kc, *vc;
    const int32_t *page_table;
    int log2ps, max_pages, num_pages;
    int32_t *seq_len, *assigned, *err;
};

template <typename T, int D, int GH>
__global__ __launch_bounds__(512) void merge_layer_update_kernel(int Hq, int Hkv,
                                                                 float *__restrict__ out,
                                                                 const float *__restrict__ part,
                                                                 int max_splits, int n_merge,
                                                                 LayerUpdArgs a) {
    extern __shared__ __align__(16) float s_dyn[];
    if ((int)blockIdx.x >= n_merge) {
        layer_update_seq<T, D>((int)blockIdx.x - n_merge, static_cast<const T *>(a.k_new),
                               static_cast<const T *>(a.v_new), a.cand, a.M, a.cent,
                               a.num_comms, a.comm_start, a.comm_size, a.comm_cap, a.members,
                               a.Cmax, a.Hkv, static_cast<T *>(a.kc), static_cast<T *>(a.vc),
                               a.page_table, a.log2ps, a.max_pages, a.num_pages, a.seq_len, 1,
                               a.assigned, a.err, reinterpret_cast<unsigned char *>(s_dyn));
        return;
    }
    merge_graph<D, GH>(blockIdx.x, Hq, Hkv, 1, out, part, max_splits, s_dyn);
}

static hipError_t launch_merge(const Problem &p, int ms, float *out, const float *partials,
                               int32_t *bump_seq_len, hipStream_t st) {
    const int GH = p.heads_per_graph();
#define CKV_MERGE_CASE(DD, HH)                                                                 \
    if (p.D == DD && GH == HH) {                                                               \
        hipExtLaunchKernelGGL((merge_kernel<DD, HH>), dim3(p.NG() * HH * (DD / kWave)),        \
                              dim3(kWave), (size_t)ms * sizeof(float), st, p.ev_start,         \
                              p.ev_stop, 0, p.Hq, p.Hkv, p.gpk, out, partials, ms,             \
                              bump_seq_len);                                                   \
        return hipGetLastError();                                                              \
    }
    CKV_MERGE_CASE(128, 1) CKV_MERGE_CASE(128, 2) CKV_MERGE_CASE(128, 4) CKV_MERGE_CASE(128, 8)
    CKV_MERGE_CASE(64, 1) CKV_MERGE_CASE(64, 2) CKV_MERGE_CASE(64, 4) CKV_MERGE_CASE(64, 8)
#undef CKV_MERGE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const Problem &pg, int idx_stride, float *out, const float *partials,
                             int32_t *bump_seq_len, hipStream_t st) {
    const Problem p = attn_problem(pg);
    return launch_merge(p, attn_max_splits(p, idx_stride), out, partials, bump_seq_len, st);
}

hipError_t launch_dense_merge(const Problem &p, const ckv_kv &kv, float *out,
                              const float *partials, hipStream_t st) {
    const Problem pd = dense_problem(p);
    int cpw = 1;
    return launch_merge(pd, dense_max_splits(pd, kv, &cpw), out, partials, nullptr, st);
}

hipError_t launch_attn_merge_layer_update(const Problem &pg, int idx_stride, float *out,
                                         const float *partials, const void *k_new,
                                         const void *v_new, const int32_t *cand, int n_cand,
                                         const ckv_graphs &gr, const ckv_kv &kv,
                                         int32_t *assigned, int32_t *err, hipStream_t st) {
    if (!pg.layer() || !layer_update_fits(pg, n_cand)) return hipErrorInvalidValue;
    const Problem p = attn_problem(pg);
    const int ms = attn_max_splits(p, idx_stride);
    const int GH = p.heads_per_graph();
    const size_t merge_lds = (size_t)GH * ms * sizeof(float);
    const size_t upd_lds = layer_update_lds(pg.cdim(), n_cand, pg.Hkv);
    const size_t lds = merge_lds > upd_lds ? merge_lds : upd_lds;
    const LayerUpdArgs a{k_new, v_new, cand, n_cand, gr.centroids, gr.num_comms, gr.comm_start,
                         gr.comm_size, gr.comm_cap, gr.members, pg.Cmax, pg.Hkv, kv.k, kv.v,
                         kv.page_table, log2_pow2(kv.page_size), kv.max_pages_per_seq,
                         kv.num_pages, kv.seq_len, assigned, err};
#define CKV_MLU_CASE(TT, DT, DD, HH)                                                           \
    if (p.dtype == DT && p.D == DD && GH == HH) {                                              \
        hipExtLaunchKernelGGL((merge_layer_update_kernel<TT, DD, HH>), dim3(p.NG() + pg.B),    \
                              dim3(512), lds, st, p.ev_start, p.ev_stop, 0, p.Hq, p.Hkv, out,   \
                              partials, ms, p.NG(), a);                                        \
        return hipGetLastError();                                                              \
    }
    CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 128, 1) CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 128, 2)
    CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 128, 4) CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 128, 8)
    CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 64, 1) CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 64, 2)
    CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 64, 4) CKV_MLU_CASE(bf16_t, CKV_DT_BF16, 64, 8)
    CKV_MLU_CASE(float, CKV_DT_F32, 128, 1) CKV_MLU_CASE(float, CKV_DT_F32, 128, 2)
    CKV_MLU_CASE(float, CKV_DT_F32, 128, 4) CKV_MLU_CASE(float, CKV_DT_F32, 128, 8)
    CKV_MLU_CASE(float, CKV_DT_F32, 64, 1) CKV_MLU_CASE(float, CKV_DT_F32, 64, 2)
    CKV_MLU_CASE(float, CKV_DT_F32, 64, 4) CKV_MLU_CASE(float, CKV_DT_F32, 64, 8)
#undef CKV_MLU_CASE
    return hipErrorInvalidValue;
}

}  // namespace ckv
