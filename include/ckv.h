/*
 * ckv.h -- C ABI of libckv.so, the CommunityKV decode hot path for MI355X (gfx950).
 *
 * Sources for the operations (the method is described in prose only):
 *   [RIT-graph]  rit.work post "CommunityKV long-context decoding", section
 *                "Граф токенов заменяет повторную кластеризацию" (the token graph
 *                replaces repeated clustering): centres per community, the query
 *                compared with the centres only, chosen communities loaded from
 *                the full cache, exact attention inside them, sinks always added,
 *                the cache never evicted, new tokens attached locally with one
 *                centre updated.
 *   [RIT-granul] same post, section "Ускорение зависит от того, сколько графов
 *                хранит модель": one graph per group of heads sharing K/V, or one
 *                per query head; a small active token budget.
 *   [RIT-plan]   same post, section "Когда CommunityKV стоит включить в план
 *                инфраструктуры": drift of local assignments, periodic
 *                re-partitioning, the group graph as the starting point and the
 *                whole-layer graph as the less accurate variant.
 *   [ABSTRACT]   "CommunityKV: Efficient Long-Context Decoding via Graph
 *                Partitioning" (McKenna et al., 2026), abstract: constant-time
 *                local update rule, per-head and query-group graphs.
 *
 * One decode step of one layer is, in stream order:
 *   ckv_score_centroids -> ckv_select -> ckv_sparse_decode_attn -> ckv_local_update
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every array pointer is DEVICE memory owned by the caller; the library never
 *   allocates or frees memory, keeps no pointer after a call returns and holds no
 *   global state.  Structs (ckv_dims, ckv_graphs, ckv_kv) are read on the host
 *   during the call only.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call only enqueues work on it and returns; there is no host synchronisation.
 * - Host-detectable errors are returned synchronously and nothing is enqueued.
 *   Data-dependent anomalies found on the device set bits in the caller's int32
 *   `err_flag` (device memory, OR-ed, sticky) and the affected graph or token is
 *   skipped; kernels never trap.  CKV_ERR_HIP reports a failed launch.
 * - Graphs: NG = batch * num_kv_heads * graphs_per_kv.  Graph g of sequence b,
 *   KV head kvh and sub-index j is g = (b*num_kv_heads + kvh)*graphs_per_kv + j.
 *   With graphs_per_kv == 1 the G = num_q_heads/num_kv_heads query heads
 *   kvh*G .. kvh*G+G-1 share one graph (query-group graph); with
 *   graphs_per_kv == G query head kvh*G + j owns graph g (per-head graph); with
 *   graphs_per_kv == 0 graph g = b serves every head of the layer (NG = batch;
 *   see "Graph granularity" below).
 * - Not reentrant across overlapping calls that share a workspace.
 */
#ifndef CKV_H
#define CKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CKV_API __attribute__((visibility("default")))

typedef int32_t ckv_status;
enum {
    CKV_OK = 0,
    CKV_ERR_INVALID_ARG = -1, /* null pointer, inconsistent sizes            */
    CKV_ERR_UNSUPPORTED = -2, /* head_dim / dtype / group size not built      */
    CKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
    CKV_ERR_HIP = -4          /* a kernel launch failed                       */
};

enum { CKV_DT_F32 = 0, CKV_DT_BF16 = 1 };

/* Sticky device error bits OR-ed into *err_flag. */
enum {
    CKV_DEVERR_CAPACITY = 1,      /* chosen community has no free member slot   */
    CKV_DEVERR_UNMAPPED_PAGE = 2, /* page_table entry < 0 or >= num_pages        */
    CKV_DEVERR_INDEX_RANGE = 4    /* index list entry outside [0, seq_len)       */
};

/* Largest supported values. */
enum { CKV_MAX_COMMS = 8192, CKV_MAX_CAND = 16, CKV_MAX_EDGES = 8 };

typedef struct ckv_dims {
    int32_t batch;         /* B sequences                                          */
    int32_t num_q_heads;   /* Hq                                                   */
    int32_t num_kv_heads;  /* Hkv; Hq % Hkv == 0, G = Hq/Hkv in {1,2,4,8}           */
    int32_t head_dim;      /* d in {64, 128}                                       */
    int32_t graphs_per_kv; /* 1 (query-group graph), G (one graph per query head),  */
                           /* or 0 (one graph per layer, shared by all heads; see   */
                           /* "Graph granularity" below)                            */
    int32_t max_comms;     /* Cmax: stride of per-community arrays; multiple of 64, */
                           /* <= CKV_MAX_COMMS                                      */
    int32_t num_sinks;     /* S >= 0: positions 0..S-1 are attention sinks          */
    int32_t dtype;         /* CKV_DT_BF16 or CKV_DT_F32: q, K, V, k_new, v_new      */
} ckv_dims;

/*
 * Graph granularity [RIT-granul: one graph per group of heads that share keys and
 * values is the fast default; one graph per query head is slower and needs more
 * memory.  RIT-plan: putting a whole layer into one graph was clearly less
 * accurate].
 * graph g of a batch, NG graphs:
 *   graphs_per_kv = 1: g = b*Hkv + kvh, heads kvh*G .. kvh*G+G-1, NG = B*Hkv
 *   graphs_per_kv = G: g = (b*Hkv + kvh)*G + j, head kvh*G + j,    NG = B*Hq
 *   graphs_per_kv = 0: g = b, every head of the layer,              NG = B
 * Readings for the layer graph: a community carries one centroid per KV head (a
 * centroid row of Hkv*d values, KV head after KV head, the centroid of KV head kvh
 * at elements kvh*d .. kvh*d+d-1); its score is the max over all query heads of
 * q_h . (head kvh(h)'s centroid) * scale; one index list serves every KV head;
 * the new token's key row (its Hkv keys, in order) joins the nearest candidate in
 * squared L2 over the whole row (fp64; the kernel sums each KV head's slice in
 * element order, then the slices in head order -- an order that can only swap
 * candidates whose distances agree to within rounding), and every KV head's K/V
 * row n is written.  The layer graph's update stages M centroid rows in LDS:
 * Hkv <= 32, Hkv*d <= 4096 and M*(Hkv*d+4)*4 + Hkv*d*8 bytes within 64 KiB, else
 * CKV_ERR_UNSUPPORTED.  ckv_prefill_edges does not
 * take the layer graph.
 */

/* Community state of NG graphs.  Community c of graph g owns member slots
 * members[comm_start[g*Cmax+c] .. + comm_cap[g*Cmax+c]); the first
 * comm_size[g*Cmax+c] hold token positions in ascending order of insertion. */
typedef struct ckv_graphs {
    float *centroids;    /* fp32, "community-interleaved": element i of centroid c of
                            graph g at centroids[((g*(R/4) + i/4)*Cmax + c)*4 + i%4],
                            R = d (R = Hkv*d for the layer graph)              */
    int32_t *num_comms;  /* [NG] communities in use, C_g <= Cmax                     */
    int32_t *comm_start; /* [NG*Cmax]                                                 */
    int32_t *comm_size;  /* [NG*Cmax]                                                 */
    int32_t *comm_cap;   /* [NG*Cmax]                                                 */
    int32_t *members;    /* member pool (token positions); NULL allowed only for an
                            empty pool: every comm_cap of every graph is 0 (e.g.
                            every sequence holds sinks only)                        */
} ckv_graphs;

/* Full, never-evicted paged KV cache of one layer. */
typedef struct ckv_kv {
    void *k;                  /* [num_pages][Hkv][page_size][d] in dims.dtype        */
    void *v;                  /* same layout                                         */
    const int32_t *page_table; /* [B][max_pages_per_seq]: physical page of logical
                                  page p of sequence b; < 0 = unmapped               */
    int32_t page_size;         /* tokens per page, power of two                      */
    int32_t max_pages_per_seq;
    int32_t num_pages;
    int32_t *seq_len;          /* [B] tokens in cache; ckv_local_update adds one     */
} ckv_kv;

/* Bytes of workspace ckv_sparse_decode_attn and ckv_decode_step need for index
 * lists of up to `index_stride` entries per graph (split partials; no state is
 * kept in it between calls).  Returns 0 for invalid dims. */
CKV_API size_t ckv_workspace_size(const ckv_dims *dims, int32_t index_stride);

/* Layout helpers: rows [NG][Cmax][d] fp32 <-> community-interleaved centroids. */
CKV_API ckv_status ckv_centroids_from_rows(const ckv_dims *dims, const float *rows,
                                   float *centroids, void *stream);
CKV_API ckv_status ckv_centroids_to_rows(const ckv_dims *dims, const float *centroids,
                                 float *rows, void *stream);

/*
 * Centroid scoring [RIT-graph: the decode query is compared with the community
 * centres only; RIT-granul: a group graph serves all heads of the group].
 *   scores[g*Cmax + c] = fp32( max_{h in heads(g)} (q_h . mu_{g,c}) * scale )
 * with the inner products accumulated in fp64 in element order (the products of
 * bf16/fp32 inputs and fp32 centroids are exact in fp64); -inf if the community
 * is empty.  Entries c >= num_comms[g] are not written.
 *   q      : [B][Hq][d] in dims.dtype
 *   scale  : usually 1/sqrt(d)
 */
CKV_API ckv_status ckv_score_centroids(const ckv_dims *dims, const void *q,
                                       const ckv_graphs *graphs, float scale, float *scores,
                                       void *stream);

/*
 * Budgeted community selection, sinks and compaction [RIT-granul: small active
 * token budget; RIT-graph: whole communities are loaded, sinks always added].
 * Per graph: order the non-empty communities by (score desc, id asc) and keep
 * the longest prefix whose sizes sum to <= budget[b] (sinks not counted; stop at
 * the first community that does not fit).  Then
 *   index_list[g*index_stride ..] = 0..min(S,n)-1, then the members of the kept
 *   communities in ascending id, each in member order;   n = kv_seq_len[b]
 *   index_len[g] = its length;  num_selected[g] = number kept (may be NULL)
 *   cand[g*n_cand + i] = i-th community of the same order (i < n_cand), -1 if none
 *   selected[g*Cmax + c] = 1 if kept else 0 (may be NULL)
 * Returns CKV_ERR_INVALID_ARG if index_stride < S + max budget is not
 * guaranteed by the caller; budgets are read on the device, so the caller must
 * ensure S + budget[b] <= index_stride (entries beyond are dropped and flagged
 * CKV_DEVERR_INDEX_RANGE).
 */
CKV_API ckv_status ckv_select(const ckv_dims *dims, const float *scores, const ckv_graphs *graphs,
                      const int32_t *budget, const int32_t *kv_seq_len, int32_t n_cand,
                      int32_t *index_list, int32_t index_stride, int32_t *index_len,
                      int32_t *num_selected, int32_t *cand, uint8_t *selected,
                      int32_t *err_flag, void *stream);

/*
 * Sparse exact attention over the index lists [RIT-graph: exact attention inside
 * the reduced token set; the cache stays full, so any token can be chosen].
 * For every query head h of sequence b, with graph g(h):
 *   out[(b*Hq + h)*d + i] = sum_j softmax_j(scale * q_h . K_j) V_j[i]
 * over j in index_list[g*index_stride .. + index_len[g]), K/V rows read through
 * the page table.  fp32 accumulation, fp32 output; an empty list gives 0.
 * Entries outside [0, seq_len[b]) or on unmapped pages are skipped and flagged.
 * ws: ckv_workspace_size(dims, index_stride) bytes of scratch.
 */
CKV_API ckv_status ckv_sparse_decode_attn(const ckv_dims *dims, const void *q, const ckv_kv *kv,
                                  const int32_t *index_list, int32_t index_stride,
                                  const int32_t *index_len, float scale, float *out,
                                  void *ws, size_t ws_bytes, int32_t *err_flag, void *stream);

/*
 * Constant-time local update [RIT-graph: the new token joins a neighbouring
 * community and one centre moves, at a cost set by d and not by the context;
 * ABSTRACT: constant-time local update rule].  For every graph g of sequence b,
 * with n = kv->seq_len[b] before the call:
 *   c* = argmin over the candidates cand[g*n_cand ..] (entries < 0 ignored) of
 *        ||k_new - mu_c||^2 (fp64, element order, lower id on ties)
 *   members[start + size] = n; size += 1;
 *   mu_c* = fp32( mu + (k_new - mu) / size )   (fp64 arithmetic per element)
 *   assigned[g] = c* (-1 if no candidate or the community is full -> CAPACITY bit)
 * and, once per (b, KV head), K/V row n <- k_new/v_new; finally seq_len[b] += 1.
 *   k_new, v_new: [B][Hkv][d] in dims.dtype
 */
CKV_API ckv_status ckv_local_update(const ckv_dims *dims, const void *k_new, const void *v_new,
                            const int32_t *cand, int32_t n_cand, const ckv_graphs *graphs,
                            const ckv_kv *kv, int32_t *assigned, int32_t *err_flag,
                            void *stream);

/*
 * Dense decode attention, the baseline the sparse path is measured against: for
 * every query head h of sequence b, exact softmax attention over all cached tokens
 * 0..seq_len[b]-1 of its KV head, read through the page table -- the same
 * computation as ckv_sparse_decode_attn with a full index list [RIT-graph: the
 * method keeps the whole cache and attends over chosen communities instead].
 * dims.graphs_per_kv and max_comms are validated but play no part.
 *   q    : [B][Hq][d] (dims.dtype);  out : [B][Hq][d] fp32
 *   ws   : >= ckv_dense_workspace_size(dims, kv) bytes (split partials; pieces are
 *          sized so that a KV head has at most 64 of them for the largest context
 *          max_pages_per_seq * page_size)
 * err_flag: CKV_DEVERR_UNMAPPED_PAGE for unmapped pages below seq_len (skipped).
 * Returns 0 from the size query for invalid dims or kv.
 */
CKV_API size_t ckv_dense_workspace_size(const ckv_dims *dims, const ckv_kv *kv);
CKV_API ckv_status ckv_dense_decode_attn(const ckv_dims *dims, const void *q, const ckv_kv *kv,
                                         float scale, float *out, void *ws, size_t ws_bytes,
                                         int32_t *err_flag, void *stream);

/*
 * Centroids recomputed from the member lists: for every community c < num_comms
 * of every graph, mu_c = the mean of the keys of its members (stored member order,
 * fp64 sums, one rounding to fp32; 0 for an empty community) -- the centre each
 * community carries [RIT-graph], as a refresh when the running means of the local
 * update have drifted over a long generation [RIT-plan: "Когда CommunityKV стоит
 * включить в план инфраструктуры", drift of local assignments and periodic
 * re-partitioning].  Keys are read through the page table of kv.
 *   centroids_out : [NG][d/4][max_comms][4] fp32 (the layout of graphs->centroids);
 *                   may be graphs->centroids itself (each output depends on keys only).
 * err_flag: CKV_DEVERR_INDEX_RANGE when a member is outside [0, seq_len) or on an
 * unmapped page (that member is left out of the sum, the count is not changed).
 */
CKV_API ckv_status ckv_rebuild_centroids(const ckv_dims *dims, const ckv_graphs *graphs,
                                         const ckv_kv *kv, float *centroids_out,
                                         int32_t *err_flag, void *stream);

/*
 * Drift of the running-mean centroids (graphs->centroids) from `reference` (same
 * layout, e.g. the output of ckv_rebuild_centroids): drift[g] = the largest, over
 * the non-empty communities of graph g, of ||mu_c - ref_c||_2 / ||ref_c||_2 (fp64,
 * rounded to fp32; a zero reference row counts its absolute distance).
 *   drift : [NG] fp32 (device)
 */
CKV_API ckv_status ckv_centroid_drift(const ckv_dims *dims, const ckv_graphs *graphs,
                                      const float *reference, float *drift, void *stream);

/*
 * Direct edges of the prefill token graph, from the QK^T scores of the prefill
 * [RIT-graph: the token graph is built during prefill from the QK^T the model
 * computes anyway; one kind of edge links a query to a key it attends strongly,
 * another links keys that are attended together; the initial sink tokens are
 * not graph nodes].  Readings: graph g (the graphs of dims, graphs_per_kv) links
 * query position i to key position j with strength
 *   z_ij = max over the graph's query heads h of (q_h[i] . k[j]) * scale,
 * causal and without self-links (num_sinks <= j < i); the direct edges of i are
 * its `topk` strongest keys, in (z desc, j asc) order, fewer (padded with -1 and
 * -inf) when i - num_sinks < topk; its co-attention pairs are all pairs of those
 * keys, each as (lower position, higher position), listed in ascending order.
 * Pairs are emitted per query, unaggregated: counting how often a pair recurs
 * is left to the graph builder.  QK^T is computed on the matrix cores (bf16
 * products, fp32 sums): keys whose z differ by less than the fp32 rounding of a
 * d-term sum can swap places.
 *   dims      : batch B (each of n positions), heads, head_dim, graphs_per_kv,
 *               num_sinks; dtype must be CKV_DT_BF16 (else CKV_ERR_UNSUPPORTED);
 *               max_comms is only validated
 *   q         : [B][n][Hq][d] bf16 (prefill queries, contiguous)
 *   k         : [B][n][Hkv][d] bf16 (prefill keys, contiguous)
 *   topk      : 1 .. CKV_MAX_EDGES
 *   edge_idx  : [NG][n][topk] int32 key positions (NG = B * Hkv * graphs_per_kv)
 *   edge_score: [NG][n][topk] fp32 z
 *   edge_pairs: NULL, or [NG][n][topk*(topk-1)/2][2] int32; a pair is (-1, -1)
 *               when either key is missing
 *   events    : NULL, or 2 hipEvent_t (as void*) with timing, bound to the
 *               kernel's own start and end
 * All buffers are the caller's device memory.  Returns CKV_ERR_INVALID_ARG for
 * null buffers, n < 1, topk out of range or a non-finite scale.
 */
CKV_API ckv_status ckv_prefill_edges(const ckv_dims *dims, const void *q, const void *k,
                                     int32_t n, int32_t topk, float scale, int32_t *edge_idx,
                                     float *edge_score, int32_t *edge_pairs,
                                     void *const *events, void *stream);

/*
 * One whole decode step, the four operations above in 4 kernel launches:
 * scoring; selection + compaction; sparse attention (split partials) with the
 * local update running in extra workgroups of the same launch (attention reads
 * neither centroids, member lists nor row n); and the split merge with the
 * seq_len advance.  Arguments and results are those of the four calls
 * (num_selected and selected may be NULL), and every result equals the sequence
 *   ckv_score_centroids; ckv_select; ckv_sparse_decode_attn; ckv_local_update.
 * events: NULL, or 8 hipEvent_t (as void*) created with timing enabled: the
 * start / stop pair of each of the 4 kernels in the order above, bound to the
 * kernel's own execution (hipExtLaunchKernelGGL), so hipEventElapsedTime of a
 * pair is that kernel's duration without launch gaps.
 * The layer graph (graphs_per_kv = 0) also takes 4 launches: its update runs in
 * extra workgroups of the attention launch, one per sequence, when its staging (the
 * n_cand candidate rows of Hkv*d floats) fits there, as for d = 128, Hkv <= 8 and
 * n_cand <= 8; otherwise in extra workgroups of the merge launch (each advancing
 * its sequence's seq_len), whose event pair then covers it.
 */
CKV_API ckv_status ckv_decode_step(const ckv_dims *dims, const void *q, const void *k_new,
                                   const void *v_new, const ckv_graphs *graphs, const ckv_kv *kv,
                                   const int32_t *budget, int32_t n_cand, float scale,
                                   float *scores, int32_t *index_list, int32_t index_stride,
                                   int32_t *index_len, int32_t *num_selected, int32_t *cand,
                                   uint8_t *selected, int32_t *assigned, float *out, void *ws,
                                   size_t ws_bytes, int32_t *err_flag, void *const *events,
                                   void *stream);

/*
 * ckv_decode_step for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same step and results, with the scratch in an array the library
 * holds in device memory (one per GPU it runs on, kept until the process ends)
 * instead of a caller's workspace.  No call allocates or frees memory.
 *   - a step whose ckv_workspace_size(dims, index_stride) exceeds
 *     CKV_NOALLOC_SCRATCH_BYTES returns CKV_ERR_WORKSPACE before anything is
 *     enqueued;
 *   - the array holds no state a step relies on (every step writes the scratch it
 *     reads); calls that overlap on one GPU (several streams or threads at once)
 *     share it and race: serialise them;
 *   - CKV_ERR_HIP when the array's device address cannot be obtained.
 * Other arguments and the events are those of ckv_decode_step.
 */
#define CKV_NOALLOC_SCRATCH_BYTES (32u << 20)
CKV_API ckv_status ckv_decode_step_noalloc(const ckv_dims *dims, const void *q,
                                           const void *k_new, const void *v_new,
                                           const ckv_graphs *graphs, const ckv_kv *kv,
                                           const int32_t *budget, int32_t n_cand, float scale,
                                           float *scores, int32_t *index_list,
                                           int32_t index_stride, int32_t *index_len,
                                           int32_t *num_selected, int32_t *cand,
                                           uint8_t *selected, int32_t *assigned, float *out,
                                           int32_t *err_flag, void *const *events, void *stream);

CKV_API const char *ckv_status_string(ckv_status status);

#ifdef __cplusplus
}
#endif
#endif /* CKV_H */
