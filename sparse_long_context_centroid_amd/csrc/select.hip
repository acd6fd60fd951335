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
// One 1024-thread workgroup per graph; everything lives in LDS / registers.
// The prefix is found without sorting: a most-significant-digit-first radix
// select over order-preserving u32 score keys (4 passes of 8 bits) whose
// histograms are weighted by community size (the kept prefix) and by 1 (the
// candidates) at the same time; a wavefront suffix scan over each 256-bin
// histogram finds the digit where the running weight crosses the remaining
// budget.  Communities still tied on the full 32-bit key after 4 passes are
// resolved by an id-ordered prefix sum, which is exactly the (score desc, id asc)
// order restricted to the tie.  Thread t holds communities t*IPT .. t*IPT+IPT-1,
// so the block scans are in id order.
#include "ckv_device.h"
#include "ckv_internal.h"

namespace ckv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;

enum : uint8_t { ST_REJ = 0, ST_PEND = 1, ST_SEL = 2 };

// Inclusive wave scan (sum) of an int.
__device__ __forceinline__ int wave_incl_scan(int x) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// Exclusive block scan of two ints at once; returns the exclusive prefixes and
// the block totals.  `tmp` holds 2*kSelWaves ints.  Ends with a barrier, so the
// caller may reuse `tmp` only after another barrier.
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
    __syncthreads();
}

// Wave 0: given a 256-bin histogram, find the crossing digit.
//   out[0] = digit (or -1 when the whole histogram fits in `rem`)
//   out[1] = weight of the bins above that digit
__device__ __forceinline__ void find_crossing(const int *hist, int rem, int *out) {
    const int lane = threadIdx.x;  // wave 0 only
    int h[4];
    int t = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = hist[lane * 4 + i];
        t += h[i];
    }
    // suffix over lanes: S_l = sum_{l' >= l} t_l'
    int s = t;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int y = __shfl_down(s, off);
        if (lane + off < kWave) s += y;
    }
    const int total = __shfl(s, 0);
    if (total <= rem) {
        if (lane == 0) {
            out[0] = -1;
            out[1] = total;
        }
        return;
    }
    int above = s - t;  // weight of the bins of higher lanes
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        const int incl = above + h[i];
        if (above <= rem && incl > rem) {
            out[0] = lane * 4 + i;
            out[1] = above;
        }
        above = incl;
    }
}

template <int IPT>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ num_comms,
    const int32_t *__restrict__ comm_start, const int32_t *__restrict__ comm_size,
    const int32_t *__restrict__ members, int Cmax, int graphs_per_seq,
    const int32_t *__restrict__ budget, const int32_t *__restrict__ seq_len, int S, int M,
    int32_t *__restrict__ idx, int idx_stride, int32_t *__restrict__ idx_len,
    int32_t *__restrict__ num_sel, int32_t *__restrict__ cand, uint8_t *__restrict__ selected,
    int32_t *__restrict__ err) {
    __shared__ int histA[256];
    __shared__ int histB[256];
    __shared__ int cross[4];
    __shared__ int scan_tmp[2 * kSelWaves];
    __shared__ int list_start[CKV_MAX_COMMS];
    __shared__ int list_off[CKV_MAX_COMMS + 1];
    __shared__ uint32_t cand_key[CKV_MAX_CAND];
    __shared__ int cand_id[CKV_MAX_CAND];
    __shared__ int cand_n;

    const int g = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = tid / kWave;
    const int b = g / graphs_per_seq;
    const int C = min(num_comms[g], Cmax);
    const int n = seq_len[b];
    int remA = budget[b] < 0 ? 0 : budget[b];
    int remB = M;

    uint32_t key[IPT];
    int wt[IPT];
    uint8_t stA[IPT], stB[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int c = tid * IPT + i;
        const bool v = c < C && comm_size[(size_t)g * Cmax + c] > 0;
        wt[i] = v ? comm_size[(size_t)g * Cmax + c] : 0;
        key[i] = v ? order_key(scores[(size_t)g * Cmax + c]) : 0u;
        stA[i] = v ? ST_PEND : ST_REJ;
        stB[i] = v ? ST_PEND : ST_REJ;
    }
    if (tid == 0) cand_n = 0;

    bool doneA = false, doneB = false;
    for (int pass = 0; pass < 4 && !(doneA && doneB); ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) {
            histA[tid] = 0;
            histB[tid] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int dg = (key[i] >> shift) & 255;
            if (stA[i] == ST_PEND) atomicAdd(&histA[dg], wt[i]);
            if (stB[i] == ST_PEND) atomicAdd(&histB[dg], 1);
        }
        __syncthreads();
        if (w == 0) {
            if (!doneA) find_crossing(histA, remA, cross);
            if (!doneB) find_crossing(histB, remB, cross + 2);
        }
        __syncthreads();
        if (!doneA) {
            const int dA = cross[0];
#pragma unroll
            for (int i = 0; i < IPT; ++i) {
                if (stA[i] != ST_PEND) continue;
                const int dg = (key[i] >> shift) & 255;
                stA[i] = (dA < 0 || dg > dA) ? ST_SEL : (dg < dA ? ST_REJ : ST_PEND);
            }
            remA -= cross[1];
            doneA = dA < 0;
        }
        if (!doneB) {
            const int dB = cross[2];
#pragma unroll
            for (int i = 0; i < IPT; ++i) {
                if (stB[i] != ST_PEND) continue;
                const int dg = (key[i] >> shift) & 255;
                stB[i] = (dB < 0 || dg > dB) ? ST_SEL : (dg < dB ? ST_REJ : ST_PEND);
            }
            remB -= cross[3];
            doneB = dB < 0;
        }
        __syncthreads();
    }

    // Ties on the full key: keep the id-ordered prefix that fits.
    {
        int la = 0, lb = 0;
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            la += stA[i] == ST_PEND ? wt[i] : 0;
            lb += stB[i] == ST_PEND ? 1 : 0;
        }
        int ea, eb, ta, tb;
        block_excl_scan2(la, lb, ea, eb, ta, tb, scan_tmp);
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            if (stA[i] == ST_PEND) {
                stA[i] = (ea + wt[i] <= remA) ? ST_SEL : ST_REJ;
                ea += wt[i];
            }
            if (stB[i] == ST_PEND) {
                stB[i] = (eb + 1 <= remB) ? ST_SEL : ST_REJ;
                eb += 1;
            }
        }
    }

    // Candidates: at most M, gathered then ordered by (key desc, id asc).
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        if (stB[i] == ST_SEL) {
            const int slot = atomicAdd(&cand_n, 1);
            if (slot < CKV_MAX_CAND) {
                cand_key[slot] = key[i];
                cand_id[slot] = tid * IPT + i;
            }
        }
    }

    // Compaction offsets in id order.
    int la = 0, lc = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        la += stA[i] == ST_SEL ? wt[i] : 0;
        lc += stA[i] == ST_SEL ? 1 : 0;
    }
    int ea, ec, total, ksel;
    block_excl_scan2(la, lc, ea, ec, total, ksel, scan_tmp);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
        const int c = tid * IPT + i;
        if (stA[i] == ST_SEL) {
            list_start[ec] = comm_start[(size_t)g * Cmax + c];
            list_off[ec] = ea;
            ea += wt[i];
            ec += 1;
        }
        if (selected && c < Cmax) selected[(size_t)g * Cmax + c] = stA[i] == ST_SEL ? 1 : 0;
    }
    if (tid == 0) list_off[ksel] = total;
    __syncthreads();

    const int ns = S < n ? S : n;
    int32_t *out = idx + (size_t)g * idx_stride;
    bool overflow = false;
    for (int t = tid; t < ns; t += kSelThreads) {
        if (t < idx_stride) out[t] = t;
        else overflow = true;
    }
    for (int e = w; e < ksel; e += kSelWaves) {
        const int st = list_start[e];
        const int o0 = ns + list_off[e];
        const int sz = list_off[e + 1] - list_off[e];
        for (int j = lane; j < sz; j += kWave) {
            const int o = o0 + j;
            if (o < idx_stride) out[o] = members[(size_t)st + j];
            else overflow = true;
        }
    }
    if (overflow) set_err(err, CKV_DEVERR_INDEX_RANGE);

    if (tid == 0) {
        const int len = ns + total;
        idx_len[g] = len < idx_stride ? len : idx_stride;
        if (num_sel) num_sel[g] = ksel;
        // order the candidates (at most CKV_MAX_CAND) by (key desc, id asc)
        const int nc = cand_n < M ? cand_n : M;
        for (int a = 1; a < nc; ++a) {
            const uint32_t kk = cand_key[a];
            const int ii = cand_id[a];
            int p = a - 1;
            while (p >= 0 && (cand_key[p] < kk || (cand_key[p] == kk && cand_id[p] > ii))) {
                cand_key[p + 1] = cand_key[p];
                cand_id[p + 1] = cand_id[p];
                --p;
            }
            cand_key[p + 1] = kk;
            cand_id[p + 1] = ii;
        }
        for (int a = 0; a < M; ++a) cand[(size_t)g * M + a] = a < nc ? cand_id[a] : -1;
    }
}

hipError_t launch_select(const Problem &p, const float *scores, const ckv_graphs &gr,
                         const int32_t *budget, const int32_t *seq_len, int n_cand,
                         int32_t *idx, int idx_stride, int32_t *idx_len, int32_t *num_sel,
                         int32_t *cand, uint8_t *selected, int32_t *err, hipStream_t st) {
    const int ipt = (p.Cmax + kSelThreads - 1) / kSelThreads;
#define CKV_SEL_CASE(I)                                                                        \
    if (ipt <= I) {                                                                            \
        hipLaunchKernelGGL(select_kernel<I>, dim3(p.NG()), dim3(kSelThreads), 0, st, scores,   \
                           gr.num_comms, gr.comm_start, gr.comm_size, gr.members, p.Cmax,      \
                           p.graphs_per_seq(), budget, seq_len, p.S, n_cand, idx, idx_stride,  \
                           idx_len, num_sel, cand, selected, err);                             \
        return hipGetLastError();                                                              \
    }
    CKV_SEL_CASE(1) CKV_SEL_CASE(2) CKV_SEL_CASE(4)
#undef CKV_SEL_CASE
    return hipErrorInvalidValue;
}

}  // namespace ckv
