/*
 * ckv_oracle.c -- plain, slow, fp64 CPU oracle of the CommunityKV decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file; only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header, table or helper with the HIP library.
 *
 * Sources (the method is described only in prose; no listing exists):
 *   [RIT-graph]   rit.work post "CommunityKV long-context decoding", section
 *                 "Граф токенов заменяет повторную кластеризацию" (the token graph
 *                 replaces repeated clustering).
 *   [RIT-granul]  same post, section "Ускорение зависит от того, сколько графов
 *                 хранит модель" (speed-up depends on how many graphs are kept).
 *   [ABSTRACT]    "CommunityKV: Efficient Long-Context Decoding via Graph
 *                 Partitioning" (McKenna, Alexandridis, Susanj, Liu, 2026), abstract.
 *
 * Per graph and decode step the method (a) compares the query only with the
 * community centres, (b) keeps communities under a small token budget, (c) always
 * adds the initial sink tokens, (d) computes exact attention over the chosen
 * tokens of the full cache and (e) attaches the new token to one neighbouring
 * community and moves that single centre [RIT-graph; ABSTRACT].  The pages leave
 * the score formula, the fill rule, the tie-break, "neighbouring" and the
 * precision open; the readings taken here are stated at each function.
 *
 * Arithmetic: every sum, product, exponential and quotient is fp64, compiled with
 * -ffp-contract=off so each operation rounds once, in source order.  Inputs are
 * the stored bytes (bf16 or fp32) widened exactly to fp64.  Two values are kept
 * in fp32 because they are fp32 state of the method: the per-community score used
 * for ordering, and the centroid (fp64 update, rounded once per update).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define CKVO_DT_F32 0
#define CKVO_DT_BF16 1

/* Widen element i of a bf16 or fp32 array to fp64 (exact in both cases). */
static double widen(const void *p, long i, int dtype)
{
    if (dtype == CKVO_DT_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[i];
}

/*
 * Centroid score of one graph [RIT-graph: the decode query is compared with the
 * community centres only; RIT-granul: one graph can serve a group of heads].
 * Reading: the score of community c is the largest, over the graph's query heads
 * h, of the inner product q_h . mu_c, times `scale` (1/sqrt(d)), in fp64; it is
 * then stored as fp32.  Empty communities (size 0) score -inf.
 *
 *   q      : G query rows of d elements, row h at q + h*d  (dtype q_dtype)
 *   cent   : C rows of d fp32, row c at cent + c*d
 *   size   : C community sizes
 *   out    : C fp32 scores
 */
void ckvo_score(int d, int G, const void *q, int q_dtype, const float *cent,
                const int32_t *size, int C, float scale, float *out)
{
    for (int c = 0; c < C; ++c) {
        if (size[c] <= 0) {
            out[c] = -INFINITY;
            continue;
        }
        double best = -INFINITY;
        for (int h = 0; h < G; ++h) {
            double dot = 0.0;
            for (int i = 0; i < d; ++i)
                dot = dot + widen(q, (long)h * d + i, q_dtype) * (double)cent[(long)c * d + i];
            if (dot > best)
                best = dot;
        }
        out[c] = (float)(best * (double)scale);
    }
}

/* Order used for selection: higher score first, lower community id on equal score. */
typedef struct {
    float s;
    int c;
} ckvo_item;

static int item_cmp(const void *a, const void *b)
{
    const ckvo_item *x = (const ckvo_item *)a, *y = (const ckvo_item *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->c < y->c) ? -1 : (x->c > y->c);
}

/*
 * Budgeted community selection and update candidates for one graph
 * [RIT-granul: a small active token budget; RIT-graph: chosen communities are
 * loaded whole].  Reading: sort the non-empty communities by (score desc, id asc);
 * keep the longest prefix of that order whose sizes sum to at most `budget`
 * (sinks are not counted); stop at the first community that does not fit.
 * The first min(M, #non-empty) communities of the same order are the
 * "neighbouring" communities offered to the local update.
 *
 *   sel   : C flags, 1 = selected            cand : up to M community ids
 *   returns k* (number selected); *n_cand gets the number of candidates.
 */
int ckvo_select(int C, const float *score, const int32_t *size, int budget, int M,
                uint8_t *sel, int32_t *cand, int *n_cand)
{
    ckvo_item *it = (ckvo_item *)malloc(sizeof(ckvo_item) * (size_t)(C > 0 ? C : 1));
    int m = 0;
    for (int c = 0; c < C; ++c) {
        sel[c] = 0;
        if (size[c] > 0) {
            it[m].s = score[c];
            it[m].c = c;
            ++m;
        }
    }
    qsort(it, (size_t)m, sizeof(ckvo_item), item_cmp);
    long total = 0;
    int k = 0;
    while (k < m && total + size[it[k].c] <= (long)budget) {
        total += size[it[k].c];
        sel[it[k].c] = 1;
        ++k;
    }
    int nc = m < M ? m : M;
    for (int i = 0; i < nc; ++i)
        cand[i] = it[i].c;
    *n_cand = nc;
    free(it);
    return k;
}

/*
 * Token index list of one graph [RIT-graph: the initial sink tokens are kept out
 * of the graph and always added; the chosen communities are then read from the
 * cache].  Reading: positions 0..min(S,n)-1 first, then the members of every
 * selected community in ascending community id, each in stored member order.
 * Returns the list length.
 */
int ckvo_index_list(int n, int S, int C, const uint8_t *sel, const int32_t *start,
                    const int32_t *size, const int32_t *members, int32_t *idx)
{
    int len = 0;
    int ns = S < n ? S : n;
    for (int j = 0; j < ns; ++j)
        idx[len++] = j;
    for (int c = 0; c < C; ++c) {
        if (!sel[c])
            continue;
        for (int j = 0; j < size[c]; ++j)
            idx[len++] = members[start[c] + j];
    }
    return len;
}

/*
 * Exact softmax attention of one query head over the listed tokens [RIT-graph:
 * exact attention inside the reduced token set, read from the full cache].
 *   z_j = (q . K_j) * scale,   o = sum_j exp(z_j - max z) V_j / sum_j exp(z_j - max z)
 * K and V rows: element i of token j at K + j*row_stride + i.  An empty list
 * gives o = 0.
 */
void ckvo_attend(int d, const void *q, int q_dtype, const void *K, const void *V,
                 int kv_dtype, long row_stride, const int32_t *idx, int len,
                 float scale, double *out)
{
    for (int i = 0; i < d; ++i)
        out[i] = 0.0;
    if (len <= 0)
        return;
    double *z = (double *)malloc(sizeof(double) * (size_t)len);
    double zmax = -INFINITY;
    for (int t = 0; t < len; ++t) {
        long row = (long)idx[t] * row_stride;
        double dot = 0.0;
        for (int i = 0; i < d; ++i)
            dot = dot + widen(q, i, q_dtype) * widen(K, row + i, kv_dtype);
        z[t] = dot * (double)scale;
        if (z[t] > zmax)
            zmax = z[t];
    }
    double denom = 0.0;
    for (int t = 0; t < len; ++t) {
        double w = exp(z[t] - zmax);
        long row = (long)idx[t] * row_stride;
        denom = denom + w;
        for (int i = 0; i < d; ++i)
            out[i] = out[i] + w * widen(V, row + i, kv_dtype);
    }
    for (int i = 0; i < d; ++i)
        out[i] = out[i] / denom;
    free(z);
}

/*
 * Local update of one graph for the new token at position n [RIT-graph: the new
 * token is attached to a suitable neighbouring community and only that centre is
 * updated, at a cost set by the model dimension and not by the context length;
 * ABSTRACT: constant-time local update rule].
 * Reading: among the candidate communities pick the one whose centroid is nearest
 * to k_new in squared L2 (fp64; lower id on equal distance), append n to its
 * member list, grow its size by one and move its centroid to the running mean
 *   mu <- fp32( mu + (k_new - mu) / size_new )        (fp64 arithmetic).
 * Returns the chosen id, or -1 when that community is full (nothing changes),
 * or -2 when there are no candidates.  *madds counts the multiply-adds done.
 */
int ckvo_update(int d, const void *k_new, int dtype, const int32_t *cand, int n_cand,
                float *cent, int32_t *size, const int32_t *cap, const int32_t *start,
                int32_t *members, int n, long *madds)
{
    long ops = 0;
    int best = -1;
    double best_d = INFINITY;
    for (int m = 0; m < n_cand; ++m) {
        int c = cand[m];
        double dist = 0.0;
        for (int i = 0; i < d; ++i) {
            double diff = widen(k_new, i, dtype) - (double)cent[(long)c * d + i];
            dist = dist + diff * diff;
            ++ops;
        }
        if (dist < best_d || (dist == best_d && c < best)) {
            best_d = dist;
            best = c;
        }
    }
    if (madds)
        *madds = ops;
    if (best < 0)
        return -2;
    if (size[best] >= cap[best])
        return -1;
    members[start[best] + size[best]] = n;
    size[best] += 1;
    double cnt = (double)size[best];
    for (int i = 0; i < d; ++i) {
        double mu = (double)cent[(long)best * d + i];
        double nu = mu + (widen(k_new, i, dtype) - mu) / cnt;
        cent[(long)best * d + i] = (float)nu;
        ++ops;
    }
    if (madds)
        *madds = ops;
    return best;
}

/*
 * The update of a whole-layer graph [RIT-granul, RIT-plan: one graph may serve a
 * whole layer].  A centroid row is nseg slices of d values, one slice per KV head
 * (row length nseg*d), and k_new is the matching row of the new token's keys.
 * Reading: the new token is one node of the one graph, so the distance of a
 * candidate is the plain squared L2 distance over the whole row -- one fp64 sum
 * over all nseg*d elements in element order; lower id on equal distance.  The
 * winner's whole row moves to the running mean, exactly as in ckvo_update.
 */
int ckvo_update_layer(int d, int nseg, const void *k_new, int dtype, const int32_t *cand,
                      int n_cand, float *cent, int32_t *size, const int32_t *cap,
                      const int32_t *start, int32_t *members, int n)
{
    const long row = (long)d * nseg;
    int win = -1;
    double win_dist = INFINITY;
    for (int m = 0; m < n_cand; ++m) {
        const int c = cand[m];
        double total = 0.0;
        for (long e = 0; e < row; ++e) {
            const double gap = widen(k_new, e, dtype) - (double)cent[(long)c * row + e];
            total = total + gap * gap;
        }
        if (total < win_dist || (total == win_dist && c < win)) {
            win_dist = total;
            win = c;
        }
    }
    if (win < 0)
        return -2;
    if (size[win] >= cap[win])
        return -1;
    members[start[win] + size[win]] = n;
    size[win] += 1;
    const double count = (double)size[win];
    for (long e = 0; e < row; ++e) {
        const double old_mu = (double)cent[(long)win * row + e];
        cent[(long)win * row + e] = (float)(old_mu + (widen(k_new, e, dtype) - old_mu) / count);
    }
    return win;
}

/*
 * Centroid of every community recomputed from its member list: the plain mean of
 * the member keys [RIT-graph: each community has a centre; RIT-plan: local
 * assignments drift over long generations, and the partition is refreshed from
 * time to time].  Reading: mu_c[i] = fp32( (sum over members j of K[j][i], in
 * stored member order, fp64) / size_c ); empty communities get 0.
 *
 *   K       : key rows of one KV head, row j at K + j*d (dtype)
 *   members : the pool; community c holds members[start[c] .. start[c]+size[c])
 *   out     : C rows of d fp32
 */
void ckvo_rebuild(int d, const void *K, int dtype, const int32_t *members,
                  const int32_t *start, const int32_t *size, int C, float *out)
{
    for (int c = 0; c < C; ++c) {
        for (int i = 0; i < d; ++i) {
            double s = 0.0;
            for (int m = 0; m < size[c]; ++m)
                s = s + widen(K, (long)members[start[c] + m] * d + i, dtype);
            out[(long)c * d + i] = size[c] > 0 ? (float)(s / (double)size[c]) : 0.0f;
        }
    }
}

/*
 * Drift of running-mean centroids from reference ones (e.g. rebuilt): the largest,
 * over the non-empty communities, of ||mu_c - ref_c||_2 / ||ref_c||_2 (fp64;
 * a zero reference row counts its absolute distance).  0 when none is non-empty.
 */
double ckvo_drift(int d, const float *cent, const float *ref, const int32_t *size, int C)
{
    double worst = 0.0;
    for (int c = 0; c < C; ++c) {
        if (size[c] <= 0)
            continue;
        double num = 0.0, den = 0.0;
        for (int i = 0; i < d; ++i) {
            double diff = (double)cent[(long)c * d + i] - (double)ref[(long)c * d + i];
            num = num + diff * diff;
            den = den + (double)ref[(long)c * d + i] * (double)ref[(long)c * d + i];
        }
        double r = den > 0.0 ? sqrt(num) / sqrt(den) : sqrt(num);
        if (r > worst)
            worst = r;
    }
    return worst;
}

/*
 * Direct edges of the prefill token graph of one KV head [RIT-graph: the graph is
 * built during the prefill pass from the QK^T scores the model computes anyway;
 * a direct edge links a query to a key it attends strongly; the initial sink
 * tokens are not graph nodes].  Readings: the strength of the link from query
 * position i to key position j is the group score
 *   z_ij = max over the KV head's G query heads of q_h[i] . k[j] * scale  (fp64),
 * causal and without self-links (S <= j < i); the edges of query i are its
 * `topk` strongest keys, in (z desc, j asc) order, fewer when i - S < topk.
 *
 *   Q     : query rows, head h of position i at Q + (i*G + h)*d    (dtype)
 *   K     : key rows, position j at K + j*d                        (dtype)
 *   rows  : the query positions to compute (nrows of them)
 *   idx   : [nrows][topk] key positions, -1 padded;  score: [nrows][topk] fp32 z
 */
/*
 * The group score z_ij of the edges below for given pairs: query position rows[r],
 * key position keys[r] (fp64, not rounded).
 */
void ckvo_edge_scores(int d, int G, const void *Q, const void *K, int dtype, float scale,
                      const int32_t *rows, const int32_t *keys, int npairs, double *z)
{
    for (int r = 0; r < npairs; ++r) {
        long i = rows[r], j = keys[r];
        double best = -INFINITY;
        for (int h = 0; h < G; ++h) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot = dot + widen(Q, (i * G + h) * d + e, dtype) * widen(K, j * d + e, dtype);
            best = dot > best ? dot : best;
        }
        z[r] = best * (double)scale;
    }
}

void ckvo_edges(int d, int G, const void *Q, const void *K, int dtype, int S, float scale,
                int topk, const int32_t *rows, int nrows, int32_t *idx, float *score)
{
    for (int r = 0; r < nrows; ++r) {
        int i = rows[r];
        int32_t *oi = idx + (long)r * topk;
        float *os = score + (long)r * topk;
        for (int t = 0; t < topk; ++t) {
            oi[t] = -1;
            os[t] = -INFINITY;
        }
        int lo = S;
        int cnt = i - lo > 0 ? i - lo : 0;
        if (cnt == 0)
            continue;
        double *z = (double *)malloc(sizeof(double) * (size_t)cnt);
        for (int j = lo; j < i; ++j) {
            double best = -INFINITY;
            for (int h = 0; h < G; ++h) {
                double dot = 0.0;
                for (int e = 0; e < d; ++e)
                    dot = dot + widen(Q, ((long)i * G + h) * d + e, dtype) *
                                widen(K, (long)j * d + e, dtype);
                if (dot > best)
                    best = dot;
            }
            z[j - lo] = best * (double)scale;
        }
        /* repeated extraction of the strongest remaining key (lowest j on ties) */
        int k = topk < cnt ? topk : cnt;
        for (int t = 0; t < k; ++t) {
            int arg = -1;
            for (int j = 0; j < cnt; ++j)
                if (z[j] != -INFINITY && (arg < 0 || z[j] > z[arg]))
                    arg = j;
            oi[t] = lo + arg;
            os[t] = (float)z[arg];
            z[arg] = -INFINITY;
        }
        free(z);
    }
}

/*
 * Co-attention edges of the prefill token graph [RIT-graph: besides the direct
 * query->key links, the graph links keys that are attended together; abstract:
 * the token graph is built from the prefill's QK^T scores].  Readings: two keys
 * are attended together when both are among one query's `topk` strongest keys
 * (the direct edges of ckvo_edges); every such pair is emitted once per query,
 * unaggregated, as (lower position, higher position).  The valid keys of a row
 * are sorted ascending, a[0] < a[1] < ... < a[cnt-1]; the pair slots of a row are
 * the index pairs (x, y), 0 <= x < y < topk, in lexicographic order, and slot
 * (x, y) holds (a[x], a[y]) when y < cnt, else (-1, -1).
 *
 *   idx   : [nrows][topk] key positions, -1 where a query has fewer keys
 *   pairs : [nrows][topk*(topk-1)/2][2]
 */
void ckvo_coattention_pairs(int topk, const int32_t *idx, int nrows, int32_t *pairs)
{
    int32_t *keys = (int32_t *)malloc(sizeof(int32_t) * (size_t)(topk > 0 ? topk : 1));
    const long per_row = (long)topk * (topk - 1) / 2;
    for (int r = 0; r < nrows; ++r) {
        int cnt = 0;
        for (int t = 0; t < topk; ++t) {
            int32_t j = idx[(long)r * topk + t];
            if (j < 0)
                continue;
            /* insertion into the ascending list of the row's keys */
            int at = cnt;
            while (at > 0 && keys[at - 1] > j) {
                keys[at] = keys[at - 1];
                --at;
            }
            keys[at] = j;
            ++cnt;
        }
        int32_t *out = pairs + (long)r * per_row * 2;
        long slot = 0;
        for (int x = 0; x < topk; ++x) {
            for (int y = x + 1; y < topk; ++y) {
                out[2 * slot] = y < cnt ? keys[x] : -1;
                out[2 * slot + 1] = y < cnt ? keys[y] : -1;
                ++slot;
            }
        }
    }
    free(keys);
}
