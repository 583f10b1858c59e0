/*
 * libringattn -- one rank's share of ring (blockwise) attention on MI355X (gfx950).
 *
 * The operation (glossary page "sequence parallelism transformers"):
 *   - section "Fundamentals", item "Sequence Dimension Splitting": the N tokens
 *     are split into P contiguous chunks of N/P; rank r owns the queries and the
 *     key/value block at positions [r*N/P, (r+1)*N/P);
 *   - section "Ring Attention", item "Ring Communication": in P steps each rank
 *     passes its current block to rank r+1 and receives from rank r-1, so at
 *     step s rank r holds block (r - s) mod P;
 *   - section "Ring Attention", item "Computation": at every step the rank
 *     attends its local queries to the held block and accumulates; the
 *     accumulated result equals full softmax attention;
 *   - section "Implementation Considerations", item "Numerical Stability": the
 *     accumulation carries the softmax normalisation as a running maximum m and
 *     running sum l per query row (log-sum-exp rescaling);
 *   - section "Ulysses Sequence Parallelism", item "Attention Computation":
 *     after the all-to-all a GPU holds all N tokens for a subset of heads and
 *     runs full attention on them: ra_rank_share with P = 1.
 *
 * On one GPU all P blocks are resident in device memory and the ring is
 * replayed as sequential steps; no inter-GPU traffic happens in this library.
 *
 * Conventions shared by every call
 *   - Tensors are described by ra_tensor: a DEVICE pointer owned by the caller
 *     (the library never allocates, frees or keeps it), an element type, a
 *     4-d shape and 4 strides counted in elements.
 *   - q, k, v, o_acc, o_out use the [B, S, H, d] layout (batch, sequence,
 *     heads, head_dim; the sequence on dim 1 as the mvp-engine
 *     sequence-parallel skill page fixes for [batch, seq, hidden]).  stride[3]
 *     must be 1; data and stride[0..2] * element size must be multiples of
 *     16 bytes (128-bit loads).  Any other strides are accepted, so a
 *     [B, H, S, d] buffer can be passed as a permuted view; the sequence
 *     stride of k and v (stride[1]) must be at most 2^24 elements and a
 *     k/v block at most 2^29 keys long (RA_E_RANGE otherwise).
 *   - Per-row statistics m, l, lse are fp32 with shape [B, H, S, 1]
 *     (stride[3] ignored), any strides.
 *   - Query position i of the local block is global position q_off + i; key j
 *     of a block is global position kv_off + j.  With causal != 0 a key is
 *     visible iff its global position <= the query's global position.
 *   - Grouped-query attention: Hq must be a multiple of Hkv; query head h
 *     reads kv head h / (Hq / Hkv).
 *   - The softmax scale is opts->scale, or 1/sqrt(d) when opts is NULL or
 *     opts->scale <= 0.  Logits are scaled in fp32 (never folded into bf16 Q).
 *   - Running state (o_acc, m, l): o_acc fp32 [B, Nq, Hq, d] holds the
 *     unnormalised output sum_j e^{s_j - m} v_j, m the running max of the
 *     scaled logits (natural-log units), l the running sum sum_j e^{s_j - m}.
 *     The empty state is (o_acc, m, l) = (0, -inf, 0) (ra_state_init).
 *   - Supported: q/k/v dtype RA_BF16 (bf16 MFMA, fp32 accumulation) or RA_F32
 *     (fp32 arithmetic), all three the same; d in {64, 128}.
 *   - Every call validates all arguments on the host before touching the GPU
 *     and returns RA_OK (0) or a negative ra_status; the reason is then in
 *     ra_last_error() (thread-local).  Work is enqueued asynchronously on
 *     opts->stream (a hipStream_t; NULL = the default stream); a fault inside
 *     a kernel surfaces at the caller's next synchronisation.
 *   - Empty work (B == 0, Nq == 0, a block with no visible key) returns RA_OK
 *     without a launch.
 */
#ifndef LIBRINGATTN_H
#define LIBRINGATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RA_OK = 0,
    RA_E_NULL = -1,        /* a required pointer or tensor is NULL */
    RA_E_DTYPE = -2,       /* unsupported or mismatched element type */
    RA_E_SHAPE = -3,       /* inconsistent shapes; N % P != 0; Hq % Hkv != 0 */
    RA_E_LAYOUT = -4,      /* stride[3] != 1 or a 16-byte alignment rule broken */
    RA_E_RANGE = -5,       /* rank outside [0, P), P < 1, negative offset, size too large */
    RA_E_UNSUPPORTED = -6, /* head_dim not 64 or 128 */
    RA_E_HIP = -7          /* the HIP runtime refused a launch */
} ra_status;

typedef enum { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

typedef struct {
    void *data;          /* device pointer, caller-owned */
    int32_t dtype;       /* ra_dtype */
    int64_t shape[4];
    int64_t stride[4];   /* in elements */
} ra_tensor;

typedef struct {
    void *stream;               /* hipStream_t; NULL = default stream */
    float scale;                /* softmax scale; <= 0 selects 1/sqrt(d) */
    const ra_tensor *m;         /* ra_finalize: running max, needed for lse_out */
    const ra_tensor *o_out;     /* normalised output O [B, Nq, Hq, d], bf16 or fp32 */
    const ra_tensor *lse_out;   /* log-sum-exp [B, Hq, Nq, 1] fp32, natural log; optional */
} ra_opts;

/* Fill the running state with the empty state: o_acc = 0, m = -inf, l = 0
 * (the state before the first block of "Ring Attention" / "Computation";
 * as a merge operand it changes nothing).  o_acc fp32 [B, Nq, H, d] with
 * d in {64, 128}; m, l fp32 [B, H, Nq, 1].  Caller-owned, written in place. */
int ra_state_init(const ra_tensor *o_acc, const ra_tensor *m, const ra_tensor *l,
                  const ra_opts *opts);

/* One ring step ("Ring Attention" / "Computation"): attend the local queries
 * q [B, Nq, Hq, d] (global positions q_off..) to one key/value block
 * k_blk, v_blk [B, Nkv, Hkv, d] (global positions kv_off..) and fold the
 * result into the running state (o_acc, m, l) in place (log-sum-exp
 * rescaling to the common maximum).  A block with no visible key (causal
 * SKIP) returns RA_OK without a launch.  Steps may come in any order; the
 * result after all blocks equals full attention up to rounding. */
int ra_step(const ra_tensor *q, const ra_tensor *k_blk, const ra_tensor *v_blk,
            const ra_tensor *o_acc, const ra_tensor *m, const ra_tensor *l,
            int64_t q_off, int64_t kv_off, int causal, const ra_opts *opts);

/* Normalise the running state: O = o_acc / l, and LSE = m + ln l.
 * Source: glossary page "sequence parallelism transformers", section
 * "Implementation Considerations", item "Numerical Stability" (the softmax
 * normalisation is carried as (m, l) and applied once all blocks are in),
 * and section "Ring Attention", item "Computation" (the accumulated result
 * is then full softmax attention).  The LSE output (natural log) is the one
 * statistic the backward needs.
 *   o_acc: fp32 [B, S, H, d], d in {64, 128}, read (or overwritten in place);
 *   l, opts->m: fp32 [B, H, S, 1], read;
 *   opts->o_out: [B, S, H, d] bf16 or fp32, written, optional (NULL: O is
 *   written in place into o_acc); opts->lse_out: fp32 [B, H, S, 1], written,
 *   optional, needs opts->m (RA_E_NULL otherwise).
 * A row with l = 0 (no visible key) gives 0/0 like the definition.  All
 * buffers are the caller's; errors as for every call.  One launch,
 * HBM-bound: (6d + 12) bytes per row for a bf16 O. */
int ra_finalize(const ra_tensor *o_acc, const ra_tensor *l, const ra_opts *opts);

/* Merge a second partial state into the running state, in place:
 *   m' = max(m, m_b); w = e^{m - m'}, w_b = e^{m_b - m'} (0 for a side with
 *   m = -inf); l' = w l + w_b l_b; o_acc' = w o_acc + w_b o_b.
 * Source: glossary page "sequence parallelism transformers", section "Ring
 * Attention", item "Computation" (each block's result is accumulated and
 * the accumulation equals full attention), and section "Implementation
 * Considerations", item "Numerical Stability" (the running maximum and sum
 * per row).  The pages print no formula: this is the exact log-sum-exp
 * rescaling to the common maximum, the only combination of two partials
 * over disjoint key sets that gives the softmax over their union.  The
 * empty state (0, -inf, 0) is its identity, and it is commutative and
 * associative up to rounding, so blocks may arrive in any order.
 *   o_acc, o_b: fp32 [B, S, H, d], d in {64, 128} (o_acc read and written,
 *               o_b read);
 *   m, l, m_b, l_b: fp32 [B, H, S, 1] (m, l read and written).
 * All buffers are the caller's.  One launch, HBM-bound: 3 (4d + 8) bytes per
 * row.  Errors as for every call. */
int ra_merge(const ra_tensor *o_acc, const ra_tensor *m, const ra_tensor *l,
             const ra_tensor *o_b, const ra_tensor *m_b, const ra_tensor *l_b, const ra_opts *opts);

/* One rank's whole share in one launch: the local query block
 * q [B, N/P, Hq, d] of rank `rank` (global positions rank*N/P..) against the
 * P blocks of k, v [B, N, Hkv, d] visited in ring order (block (rank - s) mod P
 * at step s), causal blocks skipped per (q_off, kv_off), the running state
 * kept on chip, normalised at the end.  Writes O to opts->o_out (required)
 * and LSE to opts->lse_out (optional).  N % P != 0 or Nq != N/P is
 * RA_E_SHAPE: uneven lengths are not padded silently.
 * Source: glossary page "sequence parallelism transformers", section
 * "Fundamentals", item "Sequence Dimension Splitting" (contiguous chunks of
 * N/P), section "Ring Attention", items "Ring Communication" (the block
 * order) and "Computation" (attend, accumulate; equal to full attention),
 * section "Implementation Considerations", item "Numerical Stability" (the
 * running max and sum); with P = 1, section "Ulysses Sequence Parallelism",
 * item "Attention Computation".  The causal rule and the skipping of blocks
 * with no visible key are not on the pages: a key is visible iff its global
 * position is at or before the query's (the usual autoregressive mask), and
 * a block that holds no visible key for any local query is never read.
 *   q: [B, N/P, Hq, d]; k, v: [B, N, Hkv, d] (the whole sequence, block j =
 *   rows [j N/P, (j+1) N/P)); o_out [B, N/P, Hq, d] bf16 or fp32; lse_out
 *   [B, Hq, N/P, 1] fp32 natural log.  All device buffers are the caller's. */
int ra_rank_share(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                  int P, int rank, int causal, const ra_opts *opts);

/* One rank's share of an explicitly PADDED sequence (mvp-engine skill page
 * "sequence-parallel": when the sequence length is not a multiple of the
 * shard count, pad and mask explicitly).  k, v hold N = P * ceil(n_valid/P)
 * rows, the first n_valid real and the rest padding; keys at positions
 * >= n_valid are masked out for every query.  Query rows at positions
 * >= n_valid (padding) are computed like the others, against the real keys,
 * and are the caller's to ignore.  Shapes, outputs and errors as for
 * ra_rank_share; n_valid outside [1, N] is RA_E_RANGE. */
int ra_rank_share_padded(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                         int P, int rank, int causal, int64_t n_valid, const ra_opts *opts);

/* One rank's LOAD-BALANCED share in one launch (glossary page "sequence
 * parallelism transformers", section "Implementation Considerations", item
 * "Load Balancing": under causal masking contiguous shards leave rank 0 with
 * half a block of work and rank P-1 with P - 1/2).  The sequence is cut into
 * 2P chunks of c = N/(2P) tokens and rank r owns chunks r and 2P-1-r, so
 * every rank gets the same number of visible pairs.
 *   q:    [B, 2c, Hq, d] = [chunk r | chunk 2P-1-r]: local row i is global
 *         position r*c + i for i < c and (2P-1-r)*c + (i - c) otherwise;
 *   k, v: [B, N, Hkv, d], the whole sequence in natural order (the ring
 *         block of rank j is key chunks j and 2P-1-j);
 *   opts->o_out (required) [B, 2c, Hq, d] and opts->lse_out (optional)
 *         [B, Hq, 2c] in the same local row order.
 * Every key chunk is folded into both query chunks; the fold order differs
 * from the ring's only in rounding.  N % (2P) != 0 or Nq != 2 N/(2P) is
 * RA_E_SHAPE; other errors as for ra_rank_share. */
int ra_rank_share_zigzag(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                         int P, int rank, int causal, const ra_opts *opts);

/* Backward of one rank's (contiguous) share (glossary page "sequence
 * parallelism transformers", section "Implementation Considerations", item
 * "Gradient Synchronization": the backward pass runs the same ring).  With
 * the forward's P_ij = exp(s_ij - LSE_i) and dO the gradient arriving at O:
 * D_i = <dO_i, O_i>, dS_ij = P_ij (<dO_i, v_j> - D_i), dQ_i = scale *
 * sum_j dS_ij k_j, dK_j = scale * sum_i dS_ij q_i, dV_j = sum_i P_ij dO_i.
 *   q, o, dout: [B, N/P, Hq, d] bf16 (o and lse as ra_rank_share returned
 *               them; dout the upstream gradient);
 *   k, v:       [B, N, Hkv, d] bf16, the whole sequence;
 *   lse:        [B, Hq, N/P] fp32;
 *   dq:         [B, N/P, Hq, d] fp32, written;
 *   dk, dv:     [B, N, Hkv, d] fp32, written: this rank's contribution for
 *               every key (zero for keys none of its queries sees), which
 *               the ring would carry back to the key's owner;
 *   delta:      [B, Hq, N/P] fp32 workspace owned by the caller (D_i).
 * bf16 q/k/v only (RA_E_UNSUPPORTED otherwise); shapes and strides as for
 * ra_rank_share, and the sequence stride of q and dout (stride[1]) also at
 * most 2^24 elements (RA_E_RANGE otherwise).  Four launches on opts->stream. */
int ra_rank_share_bwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                      const ra_tensor *o, const ra_tensor *lse, const ra_tensor *dout,
                      int P, int rank, int causal,
                      const ra_tensor *dq, const ra_tensor *dk, const ra_tensor *dv,
                      const ra_tensor *delta, const ra_opts *opts);

/* ra_rank_share_bwd without the caller's `delta` workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  D_i = <dO_i, O_i> goes to a
 * workspace the library holds in a static device array, one per device, of
 * 2^20 fp32 rows (4 MiB, kept until the process ends): B * Hq * N/P above
 * 2^20 is RA_E_RANGE.  The call allocates nothing.  Every call on one device
 * uses that device's array, so calls that may overlap on one device (other
 * streams, other host threads) race: order them.  Arguments, outputs and
 * errors otherwise as ra_rank_share_bwd. */
int ra_rank_share_bwd_noalloc(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                              const ra_tensor *o, const ra_tensor *lse, const ra_tensor *dout,
                              int P, int rank, int causal,
                              const ra_tensor *dq, const ra_tensor *dk, const ra_tensor *dv,
                              const ra_opts *opts);

/* Backward of the load-balanced share (ra_rank_share_zigzag's forward):
 * the same computation as ra_rank_share_bwd with the rank's N/P local rows
 * being chunk `rank` (rows [0, N/(2P))) and chunk 2P-1-rank (the rest) of
 * 2P equal chunks, at those chunks' sequence positions; dk, dv again hold
 * this rank's contribution for every key row.  Arguments, layouts, dtypes
 * and ownership as ra_rank_share_bwd (o and lse from ra_rank_share_zigzag);
 * N not divisible by 2P is RA_E_SHAPE. */
int ra_rank_share_zigzag_bwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                             const ra_tensor *o, const ra_tensor *lse, const ra_tensor *dout,
                             int P, int rank, int causal,
                             const ra_tensor *dq, const ra_tensor *dk, const ra_tensor *dv,
                             const ra_tensor *delta, const ra_opts *opts);

/* Backward of the padded share (ra_rank_share_padded's forward, same n_valid):
 * keys at positions >= n_valid see no query, so their dk, dv rows are zero
 * and their k, v contents are never read.  Padding query rows (positions >=
 * n_valid) are differentiated like the others through their dout rows; a
 * caller whose loss ignores them passes zeros there.  Arguments otherwise as
 * ra_rank_share_bwd; n_valid outside [1, N] is RA_E_RANGE. */
int ra_rank_share_padded_bwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                             const ra_tensor *o, const ra_tensor *lse, const ra_tensor *dout,
                             int P, int rank, int causal, int64_t n_valid,
                             const ra_tensor *dq, const ra_tensor *dk, const ra_tensor *dv,
                             const ra_tensor *delta, const ra_opts *opts);

/* ---- host-only queries (no GPU needed) --------------------------------- */

/* Block held by `rank` at ring step s: (rank - s) mod P.  -1 if P < 1.
 * Source: glossary page "sequence parallelism transformers", section "Ring
 * Attention", item "Ring Communication" (blocks move one rank up the ring
 * per step, so a rank receives from the rank below it).  Host only. */
int64_t ra_ring_block(int64_t P, int64_t rank, int64_t s);

/* Class of the (query positions [q_off, q_off+nq), key positions
 * [kv_off, kv_off+nkv)) pair: 0 = SKIP (no visible pair), 1 = FULL (all
 * visible), 2 = PARTIAL.  The pages define neither causal masking nor block
 * skipping: the rule is that of causal attention at global positions (a key
 * is visible iff kv <= q, all keys visible when causal == 0), applied per
 * (q_off, kv_off) pair; the kernels take their block and tile decisions
 * with the same function.  Host only. */
int ra_classify(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal);

/* Tile plan of one step as the kernels use it: out[ti * ceil(nkv/bn) + tj] =
 * ra_classify of query tile ti (bm rows) and key tile tj (bn keys), tails
 * ragged.  Returns the number of tiles written, or a negative ra_status.
 * Same source as ra_classify (glossary page "sequence parallelism
 * transformers", section "Flash Attention with Sequence Parallelism", item
 * "Tiled Computation", for the tiling; the causal classes are not on the
 * pages).  out: host array of out_len entries, caller-owned.  Host only. */
int64_t ra_plan_tiles(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal,
                      int64_t bm, int64_t bn, int8_t *out, int64_t out_len);

/* Query/key tile shape (rows bm, keys bn) the kernels use for this dtype and d. */
int ra_tile_shape(int32_t dtype, int64_t d, int64_t *bm, int64_t *bn);

/* Algorithmic FLOP of one (query block, key block) pair as one ra_step
 * folds it, per batch entry: 4 * nq * nkv * d * hq weighted 1 for FULL, 1/2
 * for PARTIAL, 0 for SKIP (the classes of ra_classify).  -1 for a negative
 * argument.  Host only.  The pages give no FLOP count: 4 d per (query, key)
 * pair is the two products Q K^T and P V of 2 d FLOP each, and the causal
 * diagonal block is halved (its visible pairs are half the block, up to the
 * diagonal itself). */
double ra_flops(int64_t nq, int64_t nkv, int64_t q_off, int64_t kv_off, int64_t hq, int64_t d, int causal);

/* Algorithmic FLOP of one rank's share, 4 * Nq * Nkv * d * Hq * B per block,
 * weighted 1 for FULL, 1/2 for PARTIAL (the causal diagonal), 0 for SKIP. */
double ra_share_flops(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d,
                      int causal);

/* The same FLOP rule for ra_rank_share_zigzag's share: each (query chunk,
 * key chunk) pair of c x c tokens counts 4 * c * c * d * Hq * B, weighted by
 * its class.  -1 if N % (2P) != 0 or rank is outside [0, P). */
double ra_share_flops_zigzag(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d,
                             int causal);

/* Description of the last error on this thread ("" if none). */
const char *ra_last_error(void);

/* Library version string. */
const char *ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBRINGATTN_H */
