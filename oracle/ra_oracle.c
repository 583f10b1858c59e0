/*
 * ra_oracle.c -- plain, slow, fp64 CPU oracle for one rank's share of ring
 * (blockwise) attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the only thing both sides
 * share is the seeded input generator.
 *
 * What it computes, and the passages it follows (glossary page "sequence
 * parallelism transformers"):
 *   - "Fundamentals / Sequence Dimension Splitting": N tokens are cut into P
 *     contiguous chunks of N/P; rank r owns tokens [r*N/P, (r+1)*N/P).
 *   - "Ring Attention / Ring Communication": in each of P steps GPU i passes
 *     its current block to GPU i+1 and takes one from GPU i-1, so at step s
 *     rank r holds block (r - s) mod P  (orc_ring_block).
 *   - "Ring Attention / Computation": for every block it holds, a rank
 *     attends its local queries to that block's keys/values and accumulates
 *     the result, which equals full attention (orc_block_partial,
 *     orc_merge, orc_rank_share).
 *   - "Ulysses Sequence Parallelism / Attention Computation": full attention
 *     over all tokens for a subset of heads (orc_attention with P = 1).
 *   - "Implementation Considerations / Numerical Stability": the softmax
 *     normalisation across blocks is carried as (running max m, running sum
 *     l, unnormalised output o) and merged by rescaling to the common max.
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes of this repository):
 *   - softmax scale 1/sqrt(d) is an argument; logits s_ij = scale * <q_i, k_j>;
 *   - causal: key at global position kv_off + j is visible to query at global
 *     position q_off + i iff kv_off + j <= q_off + i;
 *   - grouped-query attention: query head h reads kv head h / (Hq / Hkv);
 *   - an empty visible set gives the merge identity (m, l, o) = (-inf, 0, 0);
 *   - LSE is the natural-log log-sum-exp of the scaled logits.
 *
 * Arithmetic is fp64 with plain loops in index order; no BLAS, no SIMD
 * intrinsics, no blocking or reordering beyond what the definition states.
 * Threads (pthreads) only split the list of independent output rows.
 *
 * Layout: q is [B, nq_rows, Hq, d], k and v are [B, nkv_rows, Hkv, d], all
 * contiguous fp64; the *_rows arguments give the batch stride in rows.  A row
 * list is an int64 array of (b, h, i) triples; outputs are compact,
 * o[r*d + c], lse[r], m[r], l[r] for the r-th listed row.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const double *q, *k, *v;
    int64_t q_rows, kv_rows;   /* rows per batch entry of the q and k/v buffers */
    int64_t nq, nkv, hq, hkv, d;
    int64_t q_off, kv_off;     /* global position of local query 0 / key 0 */
    int causal;
    double scale;
} orc_problem;

static int visible(const orc_problem *p, int64_t i, int64_t j)
{
    if (!p->causal) return 1;
    return p->kv_off + j <= p->q_off + i;
}

/* Unnormalised softmax partial of query row (b, h, i) over the keys of *p:
 *   m = max_j s_ij,  l = sum_j exp(s_ij - m),  o = sum_j exp(s_ij - m) v_j
 * over the visible j.  s is scratch of nkv doubles. */
static void partial_row(const orc_problem *p, int64_t b, int64_t h, int64_t i,
                        double *s, double *m_out, double *l_out, double *o_out)
{
    const int64_t d = p->d;
    const int64_t g = h / (p->hq / p->hkv);
    const double *qi = p->q + ((b * p->q_rows + i) * p->hq + h) * d;
    double m = -INFINITY;
    for (int64_t j = 0; j < p->nkv; ++j) {
        if (!visible(p, i, j)) continue;
        const double *kj = p->k + ((b * p->kv_rows + j) * p->hkv + g) * d;
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += qi[c] * kj[c];
        s[j] = p->scale * dot;
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c) o_out[c] = 0.0;
    if (m != -INFINITY) {
        for (int64_t j = 0; j < p->nkv; ++j) {
            if (!visible(p, i, j)) continue;
            const double *vj = p->v + ((b * p->kv_rows + j) * p->hkv + g) * d;
            double w = exp(s[j] - m);
            l += w;
            for (int64_t c = 0; c < d; ++c) o_out[c] += w * vj[c];
        }
    }
    *m_out = m;
    *l_out = l;
}

typedef struct {
    const orc_problem *p;
    const int64_t *rows;
    int64_t r0, r1;
    int normalise;            /* 1: full attention (O, LSE); 0: partial (m, l, o) */
    double *o, *a, *bb;       /* normalise: a = lse; else a = m, bb = l */
    int err;
} orc_job;

static void *run_rows(void *arg)
{
    orc_job *J = (orc_job *)arg;
    const orc_problem *p = J->p;
    double *s = (double *)malloc(sizeof(double) * (size_t)(p->nkv > 0 ? p->nkv : 1));
    if (!s) { J->err = 1; return NULL; }
    for (int64_t r = J->r0; r < J->r1; ++r) {
        int64_t b = J->rows[3 * r], h = J->rows[3 * r + 1], i = J->rows[3 * r + 2];
        double m, l;
        double *o = J->o + r * p->d;
        partial_row(p, b, h, i, s, &m, &l, o);
        if (J->normalise) {
            for (int64_t c = 0; c < p->d; ++c) o[c] = o[c] / l;
            J->a[r] = m + log(l);
        } else {
            J->a[r] = m;
            J->bb[r] = l;
        }
    }
    free(s);
    return NULL;
}

static int check_rows(const orc_problem *p, const int64_t *rows, int64_t nrows, int64_t B)
{
    if (p->d <= 0 || p->hq <= 0 || p->hkv <= 0 || p->hq % p->hkv != 0) return -3;
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= p->hq || i < 0 || i >= p->nq) return -5;
    }
    return 0;
}

static int run_threads(const orc_problem *p, const int64_t *rows, int64_t nrows, int normalise,
                       double *o, double *a, double *bb, int nthreads)
{
    if (nrows <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    orc_job *jobs = (orc_job *)calloc((size_t)nthreads, sizeof(orc_job));
    pthread_t *tid = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    int *joined = (int *)calloc((size_t)nthreads, sizeof(int));
    if (!jobs || !tid || !joined) { free(jobs); free(tid); free(joined); return -8; }
    int64_t per = (nrows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        orc_job *J = &jobs[t];
        J->p = p; J->rows = rows; J->normalise = normalise;
        J->o = o; J->a = a; J->bb = bb;
        J->r0 = t * per;
        J->r1 = (t + 1) * per < nrows ? (t + 1) * per : nrows;
        if (J->r0 >= J->r1) continue;
        if (pthread_create(&tid[t], NULL, run_rows, J) == 0) joined[t] = 1;
        else run_rows(J);                 /* no thread: do the rows here */
    }
    int err = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (joined[t]) pthread_join(tid[t], NULL);
        if (jobs[t].err) err = -8;
    }
    free(jobs); free(tid); free(joined);
    return err;
}

/* Full softmax attention of the listed query rows over all keys of the block
 * (the plain definition): O_i = sum_j softmax_j(s_ij) v_j, LSE_i = log sum_j e^{s_ij}. */
int orc_attention(const double *q, const double *k, const double *v,
                  int64_t B, int64_t q_rows, int64_t kv_rows, int64_t nq, int64_t nkv,
                  int64_t hq, int64_t hkv, int64_t d, int64_t q_off, int64_t kv_off,
                  int causal, double scale, const int64_t *rows, int64_t nrows,
                  double *o, double *lse, int nthreads)
{
    orc_problem p = {q, k, v, q_rows, kv_rows, nq, nkv, hq, hkv, d, q_off, kv_off, causal, scale};
    int e = check_rows(&p, rows, nrows, B);
    if (e) return e;
    return run_threads(&p, rows, nrows, 1, o, lse, NULL, nthreads);
}

/* Unnormalised partial (m, l, o) of the listed rows against one key/value block. */
int orc_block_partial(const double *q, const double *k, const double *v,
                      int64_t B, int64_t q_rows, int64_t kv_rows, int64_t nq, int64_t nkv,
                      int64_t hq, int64_t hkv, int64_t d, int64_t q_off, int64_t kv_off,
                      int causal, double scale, const int64_t *rows, int64_t nrows,
                      double *m, double *l, double *o, int nthreads)
{
    orc_problem p = {q, k, v, q_rows, kv_rows, nq, nkv, hq, hkv, d, q_off, kv_off, causal, scale};
    int e = check_rows(&p, rows, nrows, B);
    if (e) return e;
    return run_threads(&p, rows, nrows, 0, o, m, l, nthreads);
}

/* Merge two partials over disjoint key sets A and B:
 *   sum_{j in A u B} e^{s_j - m} = e^{m_a - m} sum_A e^{s_j - m_a} + e^{m_b - m} sum_B e^{s_j - m_b}
 * with m = max(m_a, m_b); a side with m = -inf holds no keys and weighs 0. */
void orc_merge(int64_t nrows, int64_t d,
               const double *ma, const double *la, const double *oa,
               const double *mb, const double *lb, const double *ob,
               double *m, double *l, double *o)
{
    for (int64_t r = 0; r < nrows; ++r) {
        double mm = ma[r] > mb[r] ? ma[r] : mb[r];
        double wa = ma[r] == -INFINITY ? 0.0 : exp(ma[r] - mm);
        double wb = mb[r] == -INFINITY ? 0.0 : exp(mb[r] - mm);
        double ll = wa * la[r] + wb * lb[r];
        for (int64_t c = 0; c < d; ++c) o[r * d + c] = wa * oa[r * d + c] + wb * ob[r * d + c];
        m[r] = mm;
        l[r] = ll;
    }
}

/* O = o / l, LSE = m + ln l. */
void orc_finalize(int64_t nrows, int64_t d, const double *m, const double *l, const double *o,
                  double *out, double *lse)
{
    for (int64_t r = 0; r < nrows; ++r) {
        for (int64_t c = 0; c < d; ++c) out[r * d + c] = o[r * d + c] / l[r];
        lse[r] = m[r] + log(l[r]);
    }
}

/* Ring position: at step s rank r holds the block that started at rank (r - s) mod P. */
int64_t orc_ring_block(int64_t P, int64_t rank, int64_t s)
{
    int64_t j = (rank - s) % P;
    return j < 0 ? j + P : j;
}

/* One rank's share: the local query block (q, [B, N/P, Hq, d]) against the P
 * key/value blocks of k, v ([B, N, Hkv, d]) visited in ring order, each
 * block's partial folded into the running state, then normalised. */
int orc_rank_share(const double *q, const double *k, const double *v,
                   int64_t B, int64_t N, int64_t P, int64_t rank,
                   int64_t hq, int64_t hkv, int64_t d, int causal, double scale,
                   const int64_t *rows, int64_t nrows, double *out, double *lse, int nthreads)
{
    if (P <= 0 || N % P != 0) return -3;
    if (rank < 0 || rank >= P) return -5;
    const int64_t nb = N / P;
    size_t nd = (size_t)(nrows > 0 ? nrows : 1) * (size_t)d;
    size_t n1 = (size_t)(nrows > 0 ? nrows : 1);
    double *m = malloc(n1 * sizeof(double)), *l = malloc(n1 * sizeof(double));
    double *o = malloc(nd * sizeof(double));
    double *pm = malloc(n1 * sizeof(double)), *pl = malloc(n1 * sizeof(double));
    double *po = malloc(nd * sizeof(double));
    int e = 0;
    if (!m || !l || !o || !pm || !pl || !po) { e = -8; goto done; }
    for (int64_t r = 0; r < nrows; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0;
        for (int64_t c = 0; c < d; ++c) o[r * d + c] = 0.0;
    }
    for (int64_t s = 0; s < P; ++s) {
        int64_t j = orc_ring_block(P, rank, s);
        e = orc_block_partial(q, k + j * nb * hkv * d, v + j * nb * hkv * d,
                              B, nb, N, nb, nb, hq, hkv, d, rank * nb, j * nb,
                              causal, scale, rows, nrows, pm, pl, po, nthreads);
        if (e) goto done;
        orc_merge(nrows, d, m, l, o, pm, pl, po, m, l, o);
    }
    orc_finalize(nrows, d, m, l, o, out, lse);
done:
    free(m); free(l); free(o); free(pm); free(pl); free(po);
    return e;
}

/* Share of an explicitly padded sequence (mvp-engine skill page
 * "sequence-parallel": pad and mask explicitly when the length is not a
 * multiple of the shard count): k, v hold N rows of which the first n_valid
 * are real; a key at position >= n_valid is visible to no query.  The ring
 * is unchanged; block j contributes its keys before n_valid (none: the merge
 * identity). */
int orc_rank_share_padded(const double *q, const double *k, const double *v,
                          int64_t B, int64_t N, int64_t P, int64_t rank,
                          int64_t hq, int64_t hkv, int64_t d, int causal, double scale, int64_t n_valid,
                          const int64_t *rows, int64_t nrows, double *out, double *lse, int nthreads)
{
    if (P <= 0 || N % P != 0) return -3;
    if (rank < 0 || rank >= P || n_valid < 1 || n_valid > N) return -5;
    const int64_t nb = N / P;
    size_t nd = (size_t)(nrows > 0 ? nrows : 1) * (size_t)d;
    size_t n1 = (size_t)(nrows > 0 ? nrows : 1);
    double *m = malloc(n1 * sizeof(double)), *l = malloc(n1 * sizeof(double));
    double *o = malloc(nd * sizeof(double));
    double *pm = malloc(n1 * sizeof(double)), *pl = malloc(n1 * sizeof(double));
    double *po = malloc(nd * sizeof(double));
    int e = 0;
    if (!m || !l || !o || !pm || !pl || !po) { e = -8; goto done; }
    for (int64_t r = 0; r < nrows; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.0;
        for (int64_t c = 0; c < d; ++c) o[r * d + c] = 0.0;
    }
    for (int64_t s = 0; s < P; ++s) {
        const int64_t j = orc_ring_block(P, rank, s);
        const int64_t real = n_valid - j * nb;         /* real keys of block j */
        const int64_t nk = real < 0 ? 0 : (real > nb ? nb : real);
        if (nk == 0) continue;
        e = orc_block_partial(q, k + j * nb * hkv * d, v + j * nb * hkv * d,
                              B, nb, N, nb, nk, hq, hkv, d, rank * nb, j * nb,
                              causal, scale, rows, nrows, pm, pl, po, nthreads);
        if (e) goto done;
        orc_merge(nrows, d, m, l, o, pm, pl, po, m, l, o);
    }
    orc_finalize(nrows, d, m, l, o, out, lse);
done:
    free(m); free(l); free(o); free(pm); free(pl); free(po);
    return e;
}

/* Load-balanced ("zigzag") share, the reading of "Implementation
 * Considerations / Load Balancing" used here: the sequence is cut into 2P
 * chunks of c = N/(2P) tokens and rank r owns chunks r and 2P-1-r, so under
 * causal masking every rank gets the same number of visible pairs.  The
 * local query block is [chunk r | chunk 2P-1-r] (2c rows): local row i sits
 * at global position r*c + i for i < c and (2P-1-r)*c + (i - c) otherwise.
 * The ring is unchanged: at step s rank r holds the block of rank
 * j = (r - s) mod P, i.e. key chunks j and 2P-1-j (k, v are the whole
 * sequence, [B, N, Hkv, d]); every local query attends to both chunks and
 * the partials are merged as in orc_rank_share.  Listed rows of the two
 * query chunks are handled as two row lists, each with its own position of
 * local row 0 (q_off = r*c, and (2P-1-r)*c - c for the second chunk). */
int orc_rank_share_zigzag(const double *q, const double *k, const double *v,
                          int64_t B, int64_t N, int64_t P, int64_t rank,
                          int64_t hq, int64_t hkv, int64_t d, int causal, double scale,
                          const int64_t *rows, int64_t nrows, double *out, double *lse, int nthreads)
{
    if (P <= 0 || N % (2 * P) != 0) return -3;
    if (rank < 0 || rank >= P) return -5;
    const int64_t c = N / (2 * P), nq = 2 * c;
    const int64_t q_off[2] = {rank * c, (2 * P - 1 - rank) * c - c};
    size_t n1 = (size_t)(nrows > 0 ? nrows : 1), nd = n1 * (size_t)d;
    int64_t *sub = malloc(3 * n1 * sizeof(int64_t)), *idx = malloc(n1 * sizeof(int64_t));
    double *m = malloc(n1 * sizeof(double)), *l = malloc(n1 * sizeof(double)), *o = malloc(nd * sizeof(double));
    double *pm = malloc(n1 * sizeof(double)), *pl = malloc(n1 * sizeof(double)), *po = malloc(nd * sizeof(double));
    double *so = malloc(nd * sizeof(double)), *sl = malloc(n1 * sizeof(double));
    int e = 0;
    if (!sub || !idx || !m || !l || !o || !pm || !pl || !po || !so || !sl) { e = -8; goto done; }
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[3 * r + 2] < 0 || rows[3 * r + 2] >= nq) { e = -5; goto done; }
    for (int half = 0; half < 2; ++half) {
        /* the listed rows of this query chunk */
        int64_t n = 0;
        for (int64_t r = 0; r < nrows; ++r) {
            if ((rows[3 * r + 2] >= c) != half) continue;
            sub[3 * n] = rows[3 * r]; sub[3 * n + 1] = rows[3 * r + 1]; sub[3 * n + 2] = rows[3 * r + 2];
            idx[n++] = r;
        }
        if (n == 0) continue;
        for (int64_t r = 0; r < n; ++r) {
            m[r] = -INFINITY;
            l[r] = 0.0;
            for (int64_t x = 0; x < d; ++x) o[r * d + x] = 0.0;
        }
        for (int64_t s = 0; s < P; ++s) {
            const int64_t j = orc_ring_block(P, rank, s);
            const int64_t chunks[2] = {j, 2 * P - 1 - j};
            for (int t = 0; t < 2; ++t) {
                const int64_t kc = chunks[t];
                e = orc_block_partial(q, k + kc * c * hkv * d, v + kc * c * hkv * d,
                                      B, nq, N, nq, c, hq, hkv, d, q_off[half], kc * c,
                                      causal, scale, sub, n, pm, pl, po, nthreads);
                if (e) goto done;
                orc_merge(n, d, m, l, o, pm, pl, po, m, l, o);
            }
        }
        orc_finalize(n, d, m, l, o, so, sl);
        for (int64_t r = 0; r < n; ++r) {
            lse[idx[r]] = sl[r];
            for (int64_t x = 0; x < d; ++x) out[idx[r] * d + x] = so[r * d + x];
        }
    }
done:
    free(sub); free(idx); free(m); free(l); free(o); free(pm); free(pl); free(po); free(so); free(sl);
    return e;
}

/* Block class of (query positions [q_off, q_off+nq), key positions
 * [kv_off, kv_off+nkv)): 0 = no visible pair (SKIP), 1 = every pair visible
 * (FULL), 2 = some but not all (PARTIAL). */
int orc_classify(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal)
{
    if (nq <= 0 || nkv <= 0) return 0;
    if (!causal) return 1;
    if (kv_off > q_off + nq - 1) return 0;          /* first key after last query */
    if (kv_off + nkv - 1 <= q_off) return 1;        /* last key at or before first query */
    return 2;
}

/* Number of visible (query, key) pairs, counted row by row. */
int64_t orc_visible_pairs(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal)
{
    int64_t n = 0;
    for (int64_t i = 0; i < nq; ++i) {
        int64_t c = causal ? q_off + i - kv_off + 1 : nkv;
        if (c < 0) c = 0;
        if (c > nkv) c = nkv;
        n += c;
    }
    return n;
}

/* Algorithmic FLOP of one rank's share, "4 * Nq * Nkv * d * H, causal-halved":
 * each block counts 4 * d * Hq * Nq * Nkv * B weighted 1 (FULL), 1/2 (PARTIAL)
 * or 0 (SKIP). */
double orc_share_flops(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d, int causal)
{
    const int64_t nb = N / P;
    double f = 0.0;
    for (int64_t s = 0; s < P; ++s) {
        int64_t j = orc_ring_block(P, rank, s);
        int cls = orc_classify(rank * nb, nb, j * nb, nb, causal);
        double w = cls == 1 ? 1.0 : (cls == 2 ? 0.5 : 0.0);
        f += w * 4.0 * (double)d * (double)hq * (double)nb * (double)nb * (double)B;
    }
    return f;
}

/* The same FLOP rule for the load-balanced share: each (query chunk, key
 * chunk) pair of c x c tokens counts 4 * d * Hq * c * c * B weighted by its
 * class. */
double orc_share_flops_zigzag(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d, int causal)
{
    const int64_t c = N / (2 * P);
    const int64_t qpos[2] = {rank * c, (2 * P - 1 - rank) * c};
    double f = 0.0;
    for (int64_t s = 0; s < P; ++s) {
        const int64_t j = orc_ring_block(P, rank, s);
        const int64_t kpos[2] = {j * c, (2 * P - 1 - j) * c};
        for (int a = 0; a < 2; ++a)
            for (int t = 0; t < 2; ++t) {
                const double weight[3] = {0.0, 1.0, 0.5};   /* SKIP, FULL, PARTIAL */
                f += weight[orc_classify(qpos[a], c, kpos[t], c, causal)] * 4.0 * (double)d * (double)hq *
                     (double)c * (double)c * (double)B;
            }
    }
    return f;
}

/* ---------------------------------------------------------------- backward
 *
 * Gradients of one rank's share ("Implementation Considerations / Gradient
 * Synchronization": the backward pass uses the same communication pattern as
 * the forward pass, so the ring visits the same blocks).  With the share's
 * forward P_ij = exp(s_ij - LSE_i) over the visible keys, s_ij = scale
 * <q_i, k_j>, O_i = sum_j P_ij v_j and an upstream gradient dO_i, the chain
 * rule through the softmax gives (the plain definition, written out):
 *   D_i   = <dO_i, O_i>
 *   dP_ij = <dO_i, v_j>,   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale * sum_j dS_ij k_j
 *   dK_j  = scale * sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i
 * dQ rows sum over every visible key, block by block in ring order; dK and
 * dV rows are this rank's contribution (its local queries, all query heads
 * of the kv head) to key j, which the ring would carry back to its owner.
 *
 * Layout: q, dout [B, N/P, Hq, d]; k, v [B, N, Hkv, d]; contiguous fp64.
 * qrows: (b, h, i) triples of dQ rows, dq[r*d + c]; krows: (b, g, j)
 * triples (j a row of k/v, g a kv head) of dK/dV rows, dk/dv[r*d + c].
 * Under the load-balanced layout (zigzag) the N/P local rows are chunks
 * rank and 2P-1-rank of 2P, and the block a ring step brings is the
 * sender's two chunks; the formulas are unchanged, only positions differ.
 * For an explicitly padded sequence, keys at positions >= kv_end are visible
 * to no query (their gradients are zero). */

typedef struct {
    const double *q, *k, *v, *dout;
    int64_t B, N, P, rank, nb, hq, hkv, d;
    int causal;
    double scale;
    int zigzag;
    int64_t kv_end;
} orc_bwd;

/* sequence position of local query row i */
static int64_t bwd_qpos(const orc_bwd *w, int64_t i)
{
    if (!w->zigzag) return w->rank * w->nb + i;
    const int64_t c = w->nb / 2;
    return i < c ? w->rank * c + i : (2 * w->P - 1 - w->rank) * c + (i - c);
}

/* key rows [lo[x], hi[x]) of the block at ring step st; returns their count */
static int bwd_step_keys(const orc_bwd *w, int64_t st, int64_t lo[2], int64_t hi[2])
{
    const int64_t blk = orc_ring_block(w->P, w->rank, st);
    if (!w->zigzag) {
        lo[0] = blk * w->nb; hi[0] = lo[0] + w->nb;
        return 1;
    }
    const int64_t c = w->nb / 2;
    lo[0] = blk * c; hi[0] = lo[0] + c;
    lo[1] = (2 * w->P - 1 - blk) * c; hi[1] = lo[1] + c;
    return 2;
}

static int bwd_visible(const orc_bwd *w, int64_t i, int64_t j)
{
    return j < w->kv_end && (!w->causal || j <= bwd_qpos(w, i));
}

static double bwd_dot(const double *a, const double *b, int64_t d)
{
    double s = 0.0;
    for (int64_t c = 0; c < d; ++c) s += a[c] * b[c];
    return s;
}

/* LSE_i and D_i of local query row (b, h, i): the forward by definition over
 * all visible keys (block by block in ring order), then D = <dO, O>.
 * o is scratch of d doubles, s of N doubles. */
static void bwd_row_stats(const orc_bwd *w, int64_t b, int64_t h, int64_t i, double *s, double *o,
                          double *lse_out, double *D_out)
{
    const int64_t d = w->d, g = h / (w->hq / w->hkv);
    const double *qi = w->q + ((b * w->nb + i) * w->hq + h) * d;
    double m = -INFINITY;
    for (int64_t st = 0; st < w->P; ++st) {
        int64_t lo[2], hi[2];
        const int nr = bwd_step_keys(w, st, lo, hi);
        for (int x = 0; x < nr; ++x)
            for (int64_t j = lo[x]; j < hi[x]; ++j) {
                if (!bwd_visible(w, i, j)) continue;
                s[j] = w->scale * bwd_dot(qi, w->k + ((b * w->N + j) * w->hkv + g) * d, d);
                if (s[j] > m) m = s[j];
            }
    }
    double l = 0.0;
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < w->N; ++j) {
        if (!bwd_visible(w, i, j)) continue;
        const double e = exp(s[j] - m);
        const double *vj = w->v + ((b * w->N + j) * w->hkv + g) * d;
        l += e;
        for (int64_t c = 0; c < d; ++c) o[c] += e * vj[c];
    }
    const double lse = m + log(l);
    for (int64_t c = 0; c < d; ++c) o[c] /= l;
    *lse_out = lse;
    *D_out = bwd_dot(w->dout + ((b * w->nb + i) * w->hq + h) * d, o, d);
}

typedef struct {
    const orc_bwd *w;
    int kind;                 /* 0: stats of all rows of listed heads; 1: dQ rows; 2: dK/dV rows */
    const int64_t *rows;
    int64_t r0, r1;
    const double *lse, *D;    /* kind 2: per (head slot, i) */
    const int64_t *slot;      /* kind 2: head slot of (b, h), or -1 */
    double *out0, *out1;
    int err;
} orc_bwd_job;

static void *bwd_run(void *arg)
{
    orc_bwd_job *J = (orc_bwd_job *)arg;
    const orc_bwd *w = J->w;
    const int64_t d = w->d, G = w->hq / w->hkv;
    double *s = malloc(sizeof(double) * (size_t)(w->N > 0 ? w->N : 1));
    double *o = malloc(sizeof(double) * (size_t)d);
    if (!s || !o) { J->err = 1; free(s); free(o); return NULL; }
    for (int64_t r = J->r0; r < J->r1; ++r) {
        if (J->kind == 0) {            /* rows = (b, h) heads: all local rows of each */
            const int64_t b = J->rows[2 * (r / w->nb)], h = J->rows[2 * (r / w->nb) + 1], i = r % w->nb;
            bwd_row_stats(w, b, h, i, s, o, &J->out0[r], &J->out1[r]);
        } else if (J->kind == 1) {     /* dQ row (b, h, i) */
            const int64_t b = J->rows[3 * r], h = J->rows[3 * r + 1], i = J->rows[3 * r + 2];
            const int64_t g = h / G;
            double lse, D;
            bwd_row_stats(w, b, h, i, s, o, &lse, &D);
            const double *doi = w->dout + ((b * w->nb + i) * w->hq + h) * d;
            double *dq = J->out0 + r * d;
            for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;
            for (int64_t st = 0; st < w->P; ++st) {
                int64_t lo[2], hi[2];
                const int nr = bwd_step_keys(w, st, lo, hi);
                for (int x = 0; x < nr; ++x)
                    for (int64_t j = lo[x]; j < hi[x]; ++j) {
                        if (!bwd_visible(w, i, j)) continue;
                        const double *kj = w->k + ((b * w->N + j) * w->hkv + g) * d;
                        const double p = exp(s[j] - lse);
                        const double dp = bwd_dot(doi, w->v + ((b * w->N + j) * w->hkv + g) * d, d);
                        const double ds = p * (dp - D);
                        for (int64_t c = 0; c < d; ++c) dq[c] += w->scale * ds * kj[c];
                    }
            }
        } else {                       /* dK, dV row (b, g, j) */
            const int64_t b = J->rows[3 * r], g = J->rows[3 * r + 1], j = J->rows[3 * r + 2];
            const double *kj = w->k + ((b * w->N + j) * w->hkv + g) * d;
            const double *vj = w->v + ((b * w->N + j) * w->hkv + g) * d;
            double *dk = J->out0 + r * d, *dv = J->out1 + r * d;
            for (int64_t c = 0; c < d; ++c) dk[c] = dv[c] = 0.0;
            for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                const int64_t sl = J->slot[b * w->hq + h];
                for (int64_t i = 0; i < w->nb; ++i) {
                    if (!bwd_visible(w, i, j)) continue;
                    const double *qi = w->q + ((b * w->nb + i) * w->hq + h) * d;
                    const double *doi = w->dout + ((b * w->nb + i) * w->hq + h) * d;
                    const double p = exp(w->scale * bwd_dot(qi, kj, d) - J->lse[sl * w->nb + i]);
                    const double ds = p * (bwd_dot(doi, vj, d) - J->D[sl * w->nb + i]);
                    for (int64_t c = 0; c < d; ++c) {
                        dk[c] += w->scale * ds * qi[c];
                        dv[c] += p * doi[c];
                    }
                }
            }
        }
    }
    free(s); free(o);
    return NULL;
}

static int bwd_threads(orc_bwd_job proto, int64_t n, int nthreads)
{
    if (n <= 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > n) nthreads = (int)n;
    orc_bwd_job *jobs = calloc((size_t)nthreads, sizeof(orc_bwd_job));
    pthread_t *tid = calloc((size_t)nthreads, sizeof(pthread_t));
    int *joined = calloc((size_t)nthreads, sizeof(int));
    if (!jobs || !tid || !joined) { free(jobs); free(tid); free(joined); return -8; }
    const int64_t per = (n + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = proto;
        jobs[t].r0 = t * per;
        jobs[t].r1 = (t + 1) * per < n ? (t + 1) * per : n;
        if (jobs[t].r0 >= jobs[t].r1) continue;
        if (pthread_create(&tid[t], NULL, bwd_run, &jobs[t]) == 0) joined[t] = 1;
        else bwd_run(&jobs[t]);
    }
    int err = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (joined[t]) pthread_join(tid[t], NULL);
        if (jobs[t].err) err = -8;
    }
    free(jobs); free(tid); free(joined);
    return err;
}

static int rank_share_bwd(const double *q, const double *k, const double *v, const double *dout,
                          int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d,
                          int causal, double scale,
                          const int64_t *qrows, int64_t nqrows, const int64_t *krows, int64_t nkrows,
                          double *dq, double *dk, double *dv, int nthreads, int zigzag, int64_t kv_end)
{
    if (P <= 0 || N % (zigzag ? 2 * P : P) != 0 || hkv <= 0 || hq % hkv != 0 || d <= 0) return -3;
    if (rank < 0 || rank >= P || kv_end < 1 || kv_end > N) return -5;
    const orc_bwd w = {q, k, v, dout, B, N, P, rank, N / P, hq, hkv, d, causal, scale, zigzag, kv_end};
    const int64_t G = hq / hkv;
    for (int64_t r = 0; r < nqrows; ++r)
        if (qrows[3 * r] < 0 || qrows[3 * r] >= B || qrows[3 * r + 1] < 0 || qrows[3 * r + 1] >= hq ||
            qrows[3 * r + 2] < 0 || qrows[3 * r + 2] >= w.nb) return -5;
    for (int64_t r = 0; r < nkrows; ++r)
        if (krows[3 * r] < 0 || krows[3 * r] >= B || krows[3 * r + 1] < 0 || krows[3 * r + 1] >= hkv ||
            krows[3 * r + 2] < 0 || krows[3 * r + 2] >= N) return -5;
    orc_bwd_job proto;
    memset(&proto, 0, sizeof proto);
    proto.w = &w;
    int e = 0;
    if (nqrows > 0) {
        proto.kind = 1; proto.rows = qrows; proto.out0 = dq;
        if ((e = bwd_threads(proto, nqrows, nthreads))) return e;
    }
    if (nkrows <= 0) return 0;
    /* LSE and D of every local row of the query heads the listed kv rows need */
    int64_t *slot = malloc(sizeof(int64_t) * (size_t)(B * hq));
    int64_t *heads = malloc(sizeof(int64_t) * (size_t)(2 * B * hq));
    if (!slot || !heads) { free(slot); free(heads); return -8; }
    for (int64_t x = 0; x < B * hq; ++x) slot[x] = -1;
    int64_t nh = 0;
    for (int64_t r = 0; r < nkrows; ++r) {
        const int64_t b = krows[3 * r], g = krows[3 * r + 1];
        for (int64_t h = g * G; h < (g + 1) * G; ++h)
            if (slot[b * hq + h] < 0) {
                slot[b * hq + h] = nh;
                heads[2 * nh] = b; heads[2 * nh + 1] = h;
                ++nh;
            }
    }
    double *lse = malloc(sizeof(double) * (size_t)(nh * w.nb + 1));
    double *D = malloc(sizeof(double) * (size_t)(nh * w.nb + 1));
    if (!lse || !D) { e = -8; goto done; }
    proto.kind = 0; proto.rows = heads; proto.out0 = lse; proto.out1 = D;
    if ((e = bwd_threads(proto, nh * w.nb, nthreads))) goto done;
    proto.kind = 2; proto.rows = krows; proto.lse = lse; proto.D = D; proto.slot = slot;
    proto.out0 = dk; proto.out1 = dv;
    e = bwd_threads(proto, nkrows, nthreads);
done:
    free(slot); free(heads); free(lse); free(D);
    return e;
}

int orc_rank_share_bwd(const double *q, const double *k, const double *v, const double *dout,
                       int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d,
                       int causal, double scale,
                       const int64_t *qrows, int64_t nqrows, const int64_t *krows, int64_t nkrows,
                       double *dq, double *dk, double *dv, int nthreads)
{
    return rank_share_bwd(q, k, v, dout, B, N, P, rank, hq, hkv, d, causal, scale, qrows, nqrows, krows, nkrows,
                          dq, dk, dv, nthreads, 0, N);
}

/* Backward of the padded share (orc_rank_share_padded's forward): keys at
 * positions >= n_valid are masked out. */
int orc_rank_share_padded_bwd(const double *q, const double *k, const double *v, const double *dout,
                              int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d,
                              int causal, double scale, int64_t n_valid,
                              const int64_t *qrows, int64_t nqrows, const int64_t *krows, int64_t nkrows,
                              double *dq, double *dk, double *dv, int nthreads)
{
    return rank_share_bwd(q, k, v, dout, B, N, P, rank, hq, hkv, d, causal, scale, qrows, nqrows, krows, nkrows,
                          dq, dk, dv, nthreads, 0, n_valid);
}

/* Backward of the load-balanced share: q, dout hold the rank's 2 N/(2P)
 * rows (chunk rank, then chunk 2P-1-rank). */
int orc_rank_share_zigzag_bwd(const double *q, const double *k, const double *v, const double *dout,
                              int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d,
                              int causal, double scale,
                              const int64_t *qrows, int64_t nqrows, const int64_t *krows, int64_t nkrows,
                              double *dq, double *dk, double *dv, int nthreads)
{
    return rank_share_bwd(q, k, v, dout, B, N, P, rank, hq, hkv, d, causal, scale, qrows, nqrows, krows, nkrows,
                          dq, dk, dv, nthreads, 1, N);
}
