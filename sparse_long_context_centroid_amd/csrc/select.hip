// select.hip -- budgeted community selection, sinks and CSR compaction.
//
// rit.work post "CommunityKV long-context decoding": the granularity section keeps
// a small active token budget; the token-graph section loads chosen communities
// whole and always adds the initial sink tokens.  Per graph:
//   order  : non-empty communities by (score desc, id asc)
//   keep   : the longest prefix of that order whose sizes sum to <= budget
//   cand   : the first n_cand communities of the same order (update candidates)
//   list   : 0..min(S,n)-1, then members of kept communities in ascending id.
//
// One 1024-thread workgroup per graph; thread t holds communities t*IPT ..
// t*IPT+IPT-1 in registers, so every block scan runs in id order.
//
// The kept prefix is found without sorting.  Fast path: the scores are binned
// into 256 buckets linear in the score between the graph's min and max (a
// monotone map, so each bucket is a contiguous stretch of the order); one
// size-weighted histogram (and one unit-weighted for the candidates) gives the
// crossing bucket; buckets above it are kept, below dropped, and the communities
// inside it (a handful) are ranked exactly by one wavefront.  General path, when
// the crossing bucket holds more than 64 communities (e.g. many equal scores):
// with u32 keys that preserve the fp32 score order, the prefix is {key > T*} plus
// an id-ordered prefix of {key == T*}, where T* is the smallest key with
// W(key > T*) <= budget (W = sum of sizes); W(key > T) does not increase with T,
// so T* is found by a 4-ary search on the key, one size-weighted block reduction
// per probe.  Both paths give exactly the (score desc, id asc) prefix.  The member
// lists of the kept communities are then copied with one flat, balanced pass
// (each thread finds its communities by lockstep binary searches over the
// compacted offsets), so all member loads are in flight at once.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
// Longest kept-member list expanded into an LDS slot map (longer lists search).
constexpr int kSelSrcMax = 8192;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int x) {
    // lanes whose source is outside the row (or whose row is masked off) read 0
    return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive wavefront scan (sum) of an int with DPP only: Hillis-Steele inside each
// row of 16 lanes (row_shr 1, 2, 4, 8), then row_bcast 15 / 31 carry the row
// totals into the following rows.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += dpp_i<0x111>(x);        // row_shr:1
    x += dpp_i<0x112>(x);        // row_shr:2
    x += dpp_i<0x114>(x);        // row_shr:4
    x += dpp_i<0x118>(x);        // row_shr:8
    x += dpp_i<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x += dpp_i<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

// Sum of an int over the wavefront, as a wave-uniform value.
__device__ __forceinline__ int wave_sum(int x) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x), kWave - 1);
}

// Block sums of N ints (all threads get all N); `buf` holds N*kSelWaves ints and
// must not be written again before the next barrier.
template <int N>
__device__ __forceinline__ void block_sums(int (&v)[N], int *buf) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = wave_sum(v[j]);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < N; ++j) buf[j * kSelWaves + w] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) {
        int t = 0;
#pragma unroll
        for (int i = 0; i < kSelWaves; ++i) t += buf[j * kSelWaves + i];
        v[j] = t;
    }
}

// Block maxima of two floats (all threads get both); `buf` holds 2*kSelWaves.
__device__ __forceinline__ void block_max2(float (&v)[2], float *buf) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < 2; ++j) v[j] = wave_max_f(v[j]);
    if (lane == 0) {
        buf[w] = v[0];
        buf[kSelWaves + w] = v[1];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float t = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < kSelWaves; ++i) t = fmaxf(t, buf[j * kSelWaves + i]);
        v[j] = t;
    }
}

// One wavefront: given a 256-bin histogram, the bin where the weight summed from
// the top first exceeds `cap` (-1 when the whole histogram fits) and the weight of
// the bins above it, as wave-uniform values.
__device__ __forceinline__ int2 find_crossing(const int *hist, int cap) {
    const int lane = threadIdx.x & (kWave - 1);
    int h[4];
    int t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = hist[lane * 4 + i];
        t += h[i];
    }
    const int incl = wave_incl_scan(t);
    const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (total <= cap) return make_int2(-1, total);
    // weight of the bins above this lane's four (lanes above hold the higher bins)
    int above = total - incl;
    int bin = -1, at = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        const int next = above + h[i];
        const bool here = (above <= cap) & (next > cap);
        bin = here ? lane * 4 + i : bin;
        at = here ? above : at;
        above = next;
    }
    // exactly one lane holds the crossing: broadcast it
    const uint64_t m = __ballot(bin >= 0);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    return make_int2(__builtin_amdgcn_readlane(bin, src), __builtin_amdgcn_readlane(at, src));
}

// Communities inside the crossing bucket that the fast path ranks exactly.
constexpr int kPend = 64;

// One round of the 4-ary search for the smallest T in [lo, hi] with f(T) <= cap,
// f non-increasing; f1..f3 are f at the three probe points t1 < t2 < t3.
__device__ __forceinline__ void narrow(uint32_t &lo, uint32_t &hi, const uint32_t (&t)[3],
                                       const int (&f)[3], int cap) {
    if (f[0] <= cap) {
        hi = t[0];
    } else if (f[1] <= cap) {
        lo = t[0] + 1;
        hi = t[1];
    } else if (f[2] <= cap) {
        lo = t[1] + 1;
        hi = t[2];
    } else {
        lo = t[2] + 1;
    }
}

__device__ __forceinline__ void probes(uint32_t lo, uint32_t hi, uint32_t (&t)[3]) {
    const uint64_t wdt = (uint64_t)hi - lo;
    t[0] = lo + (uint32_t)(wdt / 4);
    t[1] = lo + (uint32_t)(wdt / 2);
    t[2] = lo + (uint32_t)(wdt * 3 / 4);
}

// Exclusive block scan of two ints; also returns the totals.  With TAIL, ends with a
// barrier (so that `tmp` may be written again at once).
template <bool TAIL>
__device__ __forceinline__ void block_excl_scan2(int a, int b, int &ea, int &eb, int &ta, int &tb,
                                                 int *tmp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int ia = wave_incl_scan(a);
    const int ib = wave_incl_scan(b);
    if (lane == kWave - 1) {
        tmp[w] = ia;
        tmp[kSelWaves + w] = ib;
    }
    __syncthreads();
    int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; ++i) {
        const int va = tmp[i], vb = tmp[kSelWaves + i];
        if (i < w) {
            pa += va;
            pb += vb;
        }
        sa += va;
        sb += vb;
    }
    ea = pa + ia - a;
    eb = pb + ib - b;
    ta = sa;
    tb = sb;
    if (TAIL) __syncthreads();
}

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_start, int32_t *__restrict__ comm_size,
    int32_t *__restrict__ members, int Cmax, int graphs_per_seq,
    const int32_t *__restrict__ budget, const int32_t *__restrict__ seq_len, int S, int M,
    int32_t *__restrict__ idx, int idx_stride, int32_t *__restrict__ idx_len,
    int32_t *__restrict__ num_sel, int32_t *__restrict__ cand, uint8_t *__restrict__ selected,
    int32_t *__restrict__ err) {
    __shared__ int red[2][6 * kSelWaves];
    __shared__ int scan_tmp[2 * kSelWaves];
    // kept communities of the graph (at most IPT per thread), in id order
    __shared__ int list_start[IPT * kSelThreads];
    __shared__ int list_off[IPT * kSelThreads + 1];
    __shared__ int s_src[kSelSrcMax];
    __shared__ uint32_t cand_key[CKV_MAX_CAND];
    __shared__ int cand_id[CKV_MAX_CAND];
    __shared__ int cand_n;
    __shared__ int histA[256], histB[256];
    __shared__ float fred[2 * kSelWaves];
    // pending entries as (key, id, weight, -) so one LDS read fetches an entry
    __shared__ int4 pendA[kPend], pendB[kPend];
    __shared__ bool pendA_sel[kPend], pendB_sel[kPend];
    __shared__ int pendA_n, pendB_n;

    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int b = g / graphs_per_seq;
    const int C = min(num_comms[g], Cmax);
    const int n = seq_len[b];
    const int Bt = budget[b] < 0 ? 0 : budget[b];

    // sizes, scores and member offsets of this thread's communities, all in flight
    // (loaded unconditionally at clamped slots, so none waits for the community
    // count; slots past it are masked afterwards)
    uint32_t key[IPT];
    float sc[IPT];
    int wt[IPT], cst[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int c = min(tid * IPT + i, Cmax - 1);
        const size_t o = (size_t)g * Cmax + c;
        wt[i] = comm_size[o];
        sc[i] = scores[o];
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        // valid keys are >= 1; 0 marks an empty or unused community
        const bool live = tid * IPT + i < C && wt[i] > 0;
        wt[i] = live ? wt[i] : 0;
        sc[i] = live ? sc[i] : 0.f;
        key[i] = live ? max(order_key(sc[i]), 1u) : 0u;
    }
    // histograms and counters cleared here: the barrier of the range reduction
    // below orders these writes before the first use
    for (int t = tid; t < 256; t += kSelThreads) {
        histA[t] = 0;
        histB[t] = 0;
    }
    if (tid == 0) {
        cand_n = 0;
        pendA_n = 0;
        pendB_n = 0;
    }

    // ---- fast path: one size-weighted histogram over 256 score buckets that are
    // linear in the fp32 score (monotone, so every bucket is a contiguous range of
    // the order); everything above the crossing bucket is kept, everything below
    // dropped, and the few communities inside it are ranked exactly by one wave.
    bool selA[IPT], selB[IPT];
    float lo_s = __builtin_inff(), hi_s = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (wt[i] > 0) {
            lo_s = fminf(lo_s, sc[i]);
            hi_s = fmaxf(hi_s, sc[i]);
        }
    }
    {
        float v2[2] = {-lo_s, hi_s};
        block_max2(v2, fred);
        lo_s = -v2[0];
        hi_s = v2[1];
    }
    const bool spread = hi_s > lo_s && hi_s - lo_s < __builtin_inff();
    const float bscale = spread ? 255.99f / (hi_s - lo_s) : 0.f;
    int bk[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const float x = (sc[i] - lo_s) * bscale;
        bk[i] = wt[i] > 0 ? min(255, max(0, (int)x)) : -1;
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (bk[i] >= 0) {
            atomicAdd(&histA[bk[i]], wt[i]);
            atomicAdd(&histB[bk[i]], 1);
        }
    }
    __syncthreads();
    // every wave finds both crossings itself (no hand-over through LDS and a barrier)
    const int2 cA = find_crossing(histA, Bt), cB = find_crossing(histB, M);
    const int bA = cA.x, aboveA_b = cA.y, bB = cB.x, aboveB_b = cB.y;
    // member offsets, requested now: only the compaction below needs them
#pragma unroll
    for (int i = 0; i < IPT; ++i) cst[i] = comm_start[(size_t)g * Cmax + min(tid * IPT + i, Cmax - 1)];
    int slotA[IPT], slotB[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        slotA[i] = -1;
        slotB[i] = -1;
        selA[i] = bk[i] >= 0 && (bA < 0 || bk[i] > bA);
        selB[i] = bk[i] >= 0 && (bB < 0 || bk[i] > bB);
        if (bk[i] >= 0 && bk[i] == bA) {
            slotA[i] = atomicAdd(&pendA_n, 1);
            if (slotA[i] < kPend)
                pendA[slotA[i]] = make_int4((int)key[i], tid * IPT + i, wt[i], 0);
        }
        if (bk[i] >= 0 && bk[i] == bB) {
            slotB[i] = atomicAdd(&pendB_n, 1);
            if (slotB[i] < kPend) pendB[slotB[i]] = make_int4((int)key[i], tid * IPT + i, 1, 0);
        }
    }
    __syncthreads();
    const int nPA = pendA_n, nPB = pendB_n;
    if (nPA <= kPend && nPB <= kPend) {
        // exact rank of each pending community among the pending ones, in the
        // (score desc, id asc) order: kept iff everything before it still fits
        if (w < 2) {
            // wave 0 ranks the budget crossing (size weights), wave 1 the candidate
            // crossing (unit weights)
            const int4 *pend = w == 0 ? pendA : pendB;
            const int np = w == 0 ? nPA : nPB;
            // one entry per lane (np <= kPend = kWave); the others arrive by readlane
            const int4 me = pend[lane < np ? lane : 0];
            const uint32_t k0 = (uint32_t)me.x;
            int before = 0;
            for (int j = 0; j < np; ++j) {
                const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane(me.x, j);
                const int ij = __builtin_amdgcn_readlane(me.y, j);
                const int wj = __builtin_amdgcn_readlane(me.z, j);
                // bitwise, not short-circuit: the loop stays free of branches
                before += ((kj > k0) | ((kj == k0) & (ij < me.y))) ? wj : 0;
            }
            if (lane < np) {
                if (w == 0) pendA_sel[lane] = aboveA_b + before + me.z <= Bt;
                else pendB_sel[lane] = aboveB_b + before + 1 <= M;
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            if (slotA[i] >= 0) selA[i] = pendA_sel[slotA[i]];
            if (slotB[i] >= 0) selB[i] = pendB_sel[slotB[i]];
        }
    } else {
        // ---- general path (e.g. many equal scores): exact 4-ary search on the keys
        // for the smallest T with W(key > T) <= Bt (A, size weights) and the
        // smallest U with N(key > U) <= M (B, unit weights); W(key > 0xFFFFFFFF) = 0,
        // so the answer always lies in [lo, hi].  Ties at T / U are resolved by
        // an id-ordered prefix sum.
        uint32_t loA = 0, hiA = 0xFFFFFFFFu, loB = 0, hiB = 0xFFFFFFFFu;
        for (int it = 0; (loA != hiA || loB != hiB) && it < 40; ++it) {
            uint32_t tA[3], tB[3];
            probes(loA, hiA, tA);
            probes(loB, hiB, tB);
            int v[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int i = 0; i < IPT; ++i) {
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    v[j] += key[i] > tA[j] ? wt[i] : 0;
                    v[3 + j] += key[i] > tB[j] ? 1 : 0;
                }
            }
            block_sums<6>(v, red[it & 1]);
            const int fA[3] = {v[0], v[1], v[2]}, fB[3] = {v[3], v[4], v[5]};
            if (loA != hiA) narrow(loA, hiA, tA, fA, Bt);
            if (loB != hiB) narrow(loB, hiB, tB, fB, M);
        }
        const uint32_t TA = loA, TB = loB;
        int aboveA = 0, aboveB = 0, tieA = 0, tieB = 0;
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            aboveA += key[i] > TA ? wt[i] : 0;
            aboveB += key[i] > TB ? 1 : 0;
            tieA += (key[i] == TA && TA > 0) ? wt[i] : 0;
            tieB += (key[i] == TB && TB > 0) ? 1 : 0;
        }
        int exA, exB, totTieA, totTieB;
        block_excl_scan2<true>(tieA, tieB, exA, exB, totTieA, totTieB, scan_tmp);
        int remA, remB;
        {
            int v[2] = {aboveA, aboveB};
            block_sums<2>(v, red[0]);
            remA = Bt - v[0];
            remB = M - v[1];
        }
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            bool sa = key[i] > TA;
            bool sb = key[i] > TB;
            if (key[i] == TA && TA > 0) {
                sa = exA + wt[i] <= remA;
                exA += wt[i];
            }
            if (key[i] == TB && TB > 0) {
                sb = exB + 1 <= remB;
                exB += 1;
            }
            selA[i] = sa && wt[i] > 0;
            selB[i] = sb && wt[i] > 0;
        }
    }
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (selB[i]) {
            const int slot = atomicAdd(&cand_n, 1);
            if (slot < CKV_MAX_CAND) {
                cand_key[slot] = key[i];
                cand_id[slot] = tid * IPT + i;
            }
        }
    }

    // compaction offsets in id order
    int la = 0, lc = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        la += selA[i] ? wt[i] : 0;
        lc += selA[i] ? 1 : 0;
    }
    int ea, ec, total, ksel;
    // (scan_tmp is not written again before the barrier after the lists)
    block_excl_scan2<false>(la, lc, ea, ec, total, ksel, scan_tmp);
#pragma unroll
    for (int i = 0; i < IPT; ++i) cst[i] = selA[i] ? cst[i] : 0;  // waited for before any store
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int c = tid * IPT + i;
        if (selA[i]) {
            list_start[ec] = cst[i];
            list_off[ec] = ea;
            ea += wt[i];
            ec += 1;
        }
        if (selected && c < Cmax) selected[(size_t)g * Cmax + c] = selA[i] ? 1 : 0;
    }
    if (tid == 0) list_off[ksel] = total;
    if (w == 0) {
        // the candidates (at most M <= CKV_MAX_CAND, unordered in LDS) go out in
        // (key desc, id asc) order: each one's rank is the number it yields to; one
        // candidate per lane, the others compared through readlane
        const int nc = cand_n < M ? cand_n : M;
        const uint32_t kk = cand_key[lane < nc ? lane : 0];
        const int ii = cand_id[lane < nc ? lane : 0];
        int r = 0;
        for (int j = 0; j < nc; ++j) {
            const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)kk, j);
            const int ij = __builtin_amdgcn_readlane(ii, j);
            r += ((kj > kk) | ((kj == kk) & (ij < ii))) ? 1 : 0;
        }
        if (lane < nc) cand[(size_t)g * M + r] = ii;
        else if (lane < M) cand[(size_t)g * M + lane] = -1;
    }
    __syncthreads();

    const int ns = S < n ? S : n;
    int32_t *out = idx + (size_t)g * idx_stride;
    bool overflow = false;
    // flat copy of the kept member lists: output slot p (0 <= p < total) belongs
    // to the compacted community e with list_off[e] <= p < list_off[e+1].  When the
    // list fits s_src, each wave first expands its share of the communities into a
    // slot -> pool-index map (LDS only); otherwise the slots find their community by
    // lockstep binary searches.
    constexpr int kBatch = 4;
    const bool mapped = total <= kSelSrcMax;
    if (mapped) {
        // four communities per round: their offsets are read together, then written
        for (int e0 = w; e0 < ksel; e0 += 4 * kSelWaves) {
            int off[4], len[4], st0[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int e = e0 + u * kSelWaves;
                const int ec = min(e, ksel - 1);
                off[u] = list_off[ec];
                len[u] = e < ksel ? list_off[ec + 1] - off[u] : 0;
                st0[u] = list_start[ec];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                for (int j = lane; j < len[u]; j += kWave) s_src[off[u] + j] = st0[u] + j;
        }
        __syncthreads();
    }
    int top = 1;  // largest power of two <= ksel (ksel >= 1 whenever total > 0)
    while (top * 2 <= ksel) top *= 2;
    for (int p0 = 0; p0 < total; p0 += kBatch * kSelThreads) {
        int src[kBatch];
        if (mapped) {
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int p = p0 + k * kSelThreads + tid;
                const int v = s_src[min(p, kSelSrcMax - 1)];  // read unconditionally
                src[k] = p < total ? v : -1;
            }
        } else {
            // last e with list_off[e] <= p, for the kBatch slots at once: the
            // searches advance in lockstep, one LDS read per slot per halving step
            int lo[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; ++k) lo[k] = 0;
            for (int st = top; st > 0; st >>= 1) {
                // branch-free: all kBatch LDS reads of a step are issued back to back
                int v[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k) v[k] = list_off[min(lo[k] + st, ksel - 1)];
#pragma unroll
                for (int k = 0; k < kBatch; ++k) {
                    const int p = p0 + k * kSelThreads + tid;
                    lo[k] = (lo[k] + st < ksel && v[k] <= p) ? lo[k] + st : lo[k];
                }
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                const int p = p0 + k * kSelThreads + tid;
                const int st0 = list_start[lo[k]], of0 = list_off[lo[k]];  // unconditional
                src[k] = p < total ? st0 + (p - of0) : -1;
            }
        }
        // unconditional loads (slot 0 for idle lanes; total > 0 here, so the pool is
        // not empty): loads inside branches make the compiler wait for every
        // outstanding access, stores included, before each store
        int val[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) val[k] = members[(size_t)max(src[k], 0)];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int o = ns + p0 + k * kSelThreads + tid;
            if (src[k] >= 0 && o < idx_stride) out[o] = val[k];
            overflow |= src[k] >= 0 && o >= idx_stride;
        }
    }
    // the sinks go out last: stored before the copy, they would hold up the copy's
    // loads behind them (one in-order counter covers loads and stores)
    for (int t = tid; t < ns; t += kSelThreads) {
        if (t < idx_stride) out[t] = t;
        else overflow = true;
    }
    if (overflow) set_err(err, CKV_DEVERR_INDEX_RANGE);
    if (tid == 0) {
        const int len = ns + total;
        idx_len[g] = len < idx_stride ? len : idx_stride;
        if (num_sel) num_sel[g] = ksel;
    }

}

hipError_t launch_select(const Problem &p, const float *scores, const ckv_graphs &gr,
                         const int32_t *budget, const int32_t *seq_len, int n_cand,
                         int32_t *idx, int idx_stride, int32_t *idx_len, int32_t *num_sel,
                         int32_t *cand, uint8_t *selected, int32_t *err, hipStream_t st) {
    const int ipt = (p.Cmax + kSelThreads - 1) / kSelThreads;
#define CKV_SEL_CASE(I)                                                                         \
    if (ipt <= I) {                                                                             \
        hipExtLaunchKernelGGL(select_kernel<I>, dim3(p.NG()), dim3(kSelThreads), 0, st,         \
                              p.ev_start, p.ev_stop, 0, scores,                                 \
                           gr.num_comms, gr.comm_start, gr.comm_size, gr.members, p.Cmax,       \
                           p.graphs_per_seq(), budget, seq_len, p.S, n_cand, idx, idx_stride,   \
                           idx_len, num_sel, cand, selected, err);                              \
        return hipGetLastError();                                                               \
    }
    static_assert(CKV_MAX_COMMS <= 8 * kSelThreads, "instances up to the community cap");
    CKV_SEL_CASE(1) CKV_SEL_CASE(2) CKV_SEL_CASE(3) CKV_SEL_CASE(4)
    CKV_SEL_CASE(6) CKV_SEL_CASE(8)
#undef CKV_SEL_CASE
    return hipErrorInvalidValue;
}

}  // namespace ckv
