/*
 * dsa.h — C ABI of libdsa.so: DSA sparse attention over a block-paged KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * The hot path has three stages (web page "Day-0 Adaptation of
 * Trillion-Parameter MoE Models on Domestic GPUs", section 3 "Adapting
 * Sparse Attention (DSA)"):
 *   1. index selection: a low-dimensional indexer scores every past position
 *      (dsa_index_score) and a block-wise Top-K keeps the K best positions
 *      (dsa_topk), item (1);
 *   2. the kept K/V rows are gathered from a paged cache through a block
 *      table, item (2);
 *   3. exact softmax attention runs over the kept rows only, with separate
 *      prefill and decode kernels (dsa_sparse_attn_prefill,
 *      dsa_sparse_attn_decode), item (3).
 * The Top-K output layout is exactly what the attention calls read (page
 * "Technical Path for Day-0 Adaptation of Trillion-Parameter Models on
 * Domestic GPUs", section 3.1, requirement 1), and one block table maps the
 * cache for every call (page "Day-0 Adaptation of Ultra-Large-Scale MoE
 * Models on Heterogeneous AI Accelerators", section 4, cache layout
 * alignment).
 *
 * Conventions for every call
 *   - Memory: every pointer argument is DEVICE memory owned by the caller,
 *     except `cache` (a host struct holding device pointers).  The library
 *     allocates nothing and keeps no state between calls.
 *   - Streams: work is enqueued on `stream` and is asynchronous; results are
 *     valid once the stream has been synchronised.
 *   - Errors: arguments are checked on the host before anything is launched;
 *     a failing check returns its status and launches nothing.  Device
 *     contents (block table entries, lengths, indices) are trusted: they are
 *     not read on the host.  A launch failure returns DSA_ERR_HIP.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Alignment: kv, v, k_idx, q, q_idx, out and the attention workspace
 *     must start 16-byte aligned and row strides must be multiples of 8
 *     elements (every HIP and torch allocation is aligned); otherwise
 *     DSA_ERR_UNSUPPORTED.
 *   - Shapes supported by the kernels (others return DSA_ERR_UNSUPPORTED):
 *       indexer   (H_idx, d_idx) = (64, 128) or (4, 32);
 *       attention (H, d_qk, d_v) = (128, 576, 512) with V the first 512
 *                 columns of each K row (cache->v == NULL), or (8, 64, 64)
 *                 with a separate V pool;
 *       1 <= K <= 2048; any lengths, except that one dsa_index_score
 *       DSA_PREFILL call takes at most 1048560 queries (chunk longer
 *       prefills) and a DSA_DECODE call with more than 1024 queries at most
 *       65535;
 *       block_size a multiple of 16 for dsa_index_score, any block_size >= 1
 *       for the other calls.
 *   - Softmax scale: sm_scale may be any finite value (zero and negative
 *     included); a non-finite scale returns DSA_ERR_SHAPE.
 *   - Precision of attention: q.K in bf16 with fp32 accumulation.  In the
 *     (128, 576, 512) family the P.V product runs in fp16 with fp32
 *     accumulation: the weights carry 11 significant bits and the values are
 *     converted from bf16, exactly for magnitudes in [2^-17, 65504], so value
 *     entries must stay within the fp16 range (|v| <= 65504); the decode
 *     split partials (each split's normalised output) are kept in fp16 too,
 *     while the log-sum-exp merge runs in fp32.  The (8, 64, 64)
 *     family carries each weight as a bf16 pair (16 bits) and has no range
 *     limit beyond bf16's.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,         /* a required pointer is NULL                       */
  DSA_ERR_SHAPE = 2,        /* a size or stride is out of range or inconsistent */
  DSA_ERR_UNSUPPORTED = 3,  /* no kernel for this head count / width            */
  DSA_ERR_WORKSPACE = 4,    /* workspace_bytes below the matching *_workspace_size */
  DSA_ERR_DEVICE = 5,       /* current device is not gfx950 or not usable       */
  DSA_ERR_HIP = 6,          /* a HIP launch failed                              */
  DSA_ERR_BOUNDS = 7        /* device data out of range (debug builds only)     */
} dsa_status_t;

typedef enum { DSA_PREFILL = 0, DSA_DECODE = 1 } dsa_phase_t;

/* Block-paged cache (page 1, section 3 item (2)): position p of sequence b
 * lives in physical block block_table[b * max_blocks_per_seq + p / block_size],
 * slot p % block_size.  A pool row of block blk, slot s starts at element
 * (blk * block_size + s) * row_stride.  All pointers are device memory. */
typedef struct {
  const uint16_t *kv;         /* bf16 key rows, d_qk columns used (the latent row when v == NULL) */
  int64_t kv_row_stride;      /* elements between consecutive slots, >= d_qk                    */
  const uint16_t *v;          /* bf16 value rows (d_v columns), or NULL: V = first d_v columns of kv */
  int64_t v_row_stride;       /* elements between slots of v (ignored when v == NULL)           */
  const uint16_t *k_idx;      /* bf16 indexer keys, one row of d_idx per position               */
  int64_t k_idx_row_stride;   /* elements between slots of k_idx, >= d_idx                      */
  const int32_t *block_table; /* [n_seq, max_blocks_per_seq] physical block ids                  */
  const int32_t *seq_lens;    /* [n_seq] cached positions per sequence (current token included) */
  int32_t n_seq;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;         /* blocks in each pool                                            */
  int32_t block_size;
  int32_t d_qk, d_v, d_idx;
} dsa_paged_cache_t;

/* Index score (page 1, section 3 item (1): low-dimensional similarity
 * scoring of every past position).  Query i belongs to sequence seq_i and
 * sits at position pos_i of it; its candidates are positions 0 .. pos_i:
 *   scores[i * ld + s] = sum_h w[i*H_idx + h] * max(0, q_idx[i,h,:] . k_idx(seq_i, s))
 * for s = 0 .. pos_i; other entries of the row are left unspecified.  Sums
 * are exact for integer-valued inputs below 2^24.
 *   q_seq, q_pos: int32 [n_q] device arrays giving seq_i and pos_i (page
 *     "Day-0 Adaptation of Ultra-Large-Scale MoE Models on Heterogeneous AI
 *     Accelerators", section 3.3: shapes are run-time values), with
 *     0 <= seq_i < n_seq and 0 <= pos_i < min(ld, max_blocks_per_seq *
 *     block_size) (device data: not checked by release builds).  Both NULL
 *     (DSA_DECODE only): query i is the last cached token of sequence i,
 *     pos_i = seq_lens[i] - 1, and n_q must equal cache->n_seq.
 *   phase selects the kernel.  DSA_DECODE streams each query's indexer keys
 *     from HBM (one query per sequence, or a few); DSA_PREFILL stages key
 *     tiles in LDS and shares them among blocks of 16 consecutive queries,
 *     which is fastest when consecutive queries are consecutive positions
 *     of one sequence (a causal prefill chunk), though any mix is allowed.
 * q_idx: bf16 [n_q, H_idx, d_idx]; w: fp32 [n_q, H_idx]; scores: fp32 [n_q, ld].
 * DSA_PREFILL takes at most 1048560 queries per call (chunk longer prefills).
 * workspace: dsa_index_score_ws(phase, n_q, ld) bytes (may be NULL when
 * that is 0). */
dsa_status_t dsa_index_score(const dsa_paged_cache_t *cache, dsa_phase_t phase,
                             const uint16_t *q_idx, const float *w, const int32_t *q_seq,
                             const int32_t *q_pos, int32_t n_q, int32_t H_idx, float *scores,
                             int64_t ld, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Workspace bytes dsa_index_score needs (0 for every size today). */
size_t dsa_index_score_ws(dsa_phase_t phase, int32_t n_q, int64_t ld);

/* Workspace bytes dsa_topk needs for these sizes (0 is possible). */
size_t dsa_topk_workspace_size(int32_t n_q, int64_t ld, int32_t K);

/* Top-K (page 1, section 3 item (1): block-wise scoring, intra-block
 * reduction, cross-block merge; no global sort).  Row i has n_i candidates
 * scores[i * ld + 0 .. n_i - 1], where n_i = n_valid[i] if n_valid != NULL,
 * else causal_base + i + 1 (the rows of a causal prefill chunk).
 * idx[i * K + r] receives the positions of the K largest scores, equal scores
 * ordered by lower position first, listed in ascending position order;
 * when n_i < K the row holds 0 .. n_i - 1 followed by -1.
 * -0.0 and +0.0 compare equal; NaN scores are not allowed.
 * n_i must satisfy 0 <= n_i <= ld (not checked: device data).
 * 1 <= K <= 2048 and ld <= 16777216, else DSA_ERR_SHAPE.  Rows of
 * ld <= 16384 need no workspace; longer rows need
 * dsa_topk_workspace_size(n_q, ld, K) bytes (about 8 * n_q * ld), whose
 * contents need no initialisation and are scratch after the call.  The
 * result is exact for every input; only the speed depends on the values
 * (a pruning bound drawn from a strided sample of each long row). */
dsa_status_t dsa_topk(const float *scores, int64_t ld, int32_t n_q, int32_t K,
                      const int32_t *n_valid, int32_t causal_base, int32_t *idx, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Flags of dsa_index_topk_decode. */
#define DSA_TOPK_SEED_PREVIOUS 1
#define DSA_INDEX_TOPK_SCORE_ONLY 2   /* run only the first launch (scores, group maxima) */
#define DSA_INDEX_TOPK_SELECT_ONLY 4  /* run only the second launch, on the workspace of a
                                         SCORE_ONLY call with the same arguments */

/* Workspace bytes dsa_index_topk_decode needs: for ld <= 262144 two fp32
 * group maxima per 16 positions of a row and one word per row (about
 * n_q * ld / 2 bytes); above, the long-row Top-K's (about 8 * n_q * ld). */
size_t dsa_index_topk_decode_ws(int32_t n_q, int64_t ld, int32_t K);

/* Index score and Top-K fused for decode rows (page 1, section 3 item (1):
 * block-wise scoring, intra-block reduction and cross-block merge; item
 * (3): decode reuses the previous step's index structure).  Computes what
 * dsa_index_score (DSA_DECODE) followed by dsa_topk computes -- the same
 * scores, written to `scores` [n_q, ld], and the same kept positions,
 * written to `idx` [n_q, K] (ascending, ties to the lower position, -1
 * padded) -- for the queries that q_seq / q_pos (or, both NULL, the last
 * token of each sequence, n_q == n_seq) describe, with row i's candidates
 * 0 .. pos_i.  The index kernel also writes, for every 16-position group,
 * its two largest scores into the workspace; the K-th largest of those
 * bounds the row's K-th largest score from below, so the Top-K step reads
 * only the groups that reach the bound, then selects exactly among them.
 * Rows capacities ld above 262144 (a million-token context) take the
 * long-row selection of dsa_topk instead, which spreads a row over many
 * workgroups.  The call makes two launches (the long-row path four);
 * flags DSA_INDEX_TOPK_SCORE_ONLY and DSA_INDEX_TOPK_SELECT_ONLY run the
 * index score, resp. the selection, on its own (for timing each apart).
 * DSA_TOPK_SEED_PREVIOUS tries each row's K-th largest score of the
 * previous call on this workspace as the bound (ld <= 262144; used only
 * when it is verified to be one; results never depend on it).  ld must be a multiple
 * of 4 and at most 2^24; scores must be 16-byte aligned; 1 <= K <= 2048.
 * Workspace: dsa_index_topk_decode_ws(n_q, ld, K) bytes, 16-byte aligned,
 * no initialisation needed (with DSA_TOPK_SEED_PREVIOUS it must hold the
 * previous call's results for the same rows to be of use). */
dsa_status_t dsa_index_topk_decode(const dsa_paged_cache_t *cache, const uint16_t *q_idx,
                                   const float *w, const int32_t *q_seq, const int32_t *q_pos,
                                   int32_t n_q, int32_t H_idx, int32_t K, float *scores,
                                   int64_t ld, int32_t *idx, int32_t flags, void *workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes dsa_index_topk_prefill needs: one 512 KB score slot per
 * workgroup of its persistent grid, min(256, ceil(n_q / 16)) slots (at most
 * 128 MiB whatever n_q), or 0 for n_q < 1. */
size_t dsa_index_topk_prefill_ws(int32_t n_q);

/* Index score and Top-K fused for prefill rows (page 1, section 3 item (3):
 * the prefill path fuses index selection into large-granularity operators),
 * with no n_q x ld score matrix: idx[i * K ..] receives what
 * dsa_index_score (DSA_PREFILL) followed by dsa_topk would give for query i
 * (position q_pos[i] of sequence q_seq[i], candidates 0 .. q_pos[i];
 * ascending, ties to the lower position, -1 padded), and no scores are
 * written.  A persistent grid (one workgroup per CU) takes blocks of 16
 * queries; the scores of a block's rows pass through the workgroup's slot
 * of the workspace and are selected there (a row with at most K
 * candidates keeps them all and is not scored).  Rows are limited to 8192
 * candidates: q_pos[i] < 8192 (device data: a debug build reports a larger
 * position, a release build selects among the first 8192); chunk longer
 * prefills through the two separate calls.  Indexer shape (64, 128) only;
 * block_size a multiple of 16; 1 <= K <= 2048.  q_seq and q_pos are
 * required.  Workspace: dsa_index_topk_prefill_ws(n_q) bytes, 16-byte
 * aligned, no initialisation; calls that share a workspace must not
 * overlap. */
dsa_status_t dsa_index_topk_prefill(const dsa_paged_cache_t *cache, const uint16_t *q_idx,
                                    const float *w, const int32_t *q_seq, const int32_t *q_pos,
                                    int32_t n_q, int32_t H_idx, int32_t K, int32_t *idx,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes dsa_sparse_attn_decode needs (split-K partial results). */
size_t dsa_sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t K, int32_t d_v);

/* Sparse attention, decode path (page 1, section 3 item (3): one token per
 * step, bandwidth bound).  Query b is the last token of sequence b
 * (B == cache->n_seq).  For every head h:
 *   l_j = sm_scale * q[b,h,:] . K_j,  p = softmax(l) over the kept j,
 *   out[b,h,:] = sum_j p_j V_j,       lse[b,h] = ln sum_j exp(l_j)
 * where j runs over idx[b*K + r] for r < min(K, seq_lens[b]) with
 * idx >= 0; entries < 0 are skipped.  K_j / V_j are rows of position j read
 * through the block table.  q: bf16 [B, H, d_qk]; out: bf16 [B, H, d_v];
 * lse: fp32 [B, H] or NULL.  A row with nothing kept gives out = 0,
 * lse = -inf.  The work is split over the kept positions and merged by
 * log-sum-exp; `workspace` holds the partial results. */
dsa_status_t dsa_sparse_attn_decode(const dsa_paged_cache_t *cache, const uint16_t *q,
                                    const int32_t *idx, int32_t B, int32_t H, int32_t K,
                                    float sm_scale, uint16_t *out, float *lse, void *workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* Sparse attention, decode path, allocating nothing: for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * kernels and results as dsa_sparse_attn_decode, but the split partial
 * results live in a static device array of the library: 48 MiB (50331648
 * bytes) per GPU, held from the library's load until the process ends.
 * Sizes whose dsa_sparse_attn_decode_workspace_size exceeds that return
 * DSA_ERR_WORKSPACE before anything is launched.  Every call on one GPU uses
 * the same array, so calls that overlap on one GPU (concurrent streams,
 * threads) race; calls ordered on one stream do not. */
dsa_status_t dsa_sparse_attn_decode_static(const dsa_paged_cache_t *cache, const uint16_t *q,
                                           const int32_t *idx, int32_t B, int32_t H, int32_t K,
                                           float sm_scale, uint16_t *out, float *lse,
                                           hipStream_t stream);

/* Sparse attention, prefill path (page 1, section 3 item (3): many queries,
 * compute bound).  Query t belongs to sequence q_seq[t] at position
 * q_pos[t] (int32 [T] device arrays, 0 <= q_seq[t] < n_seq, 0 <= q_pos[t] <
 * max_blocks_per_seq * block_size; queries of several sequences may share a
 * call); same formula as decode, with j over idx[t*K + r] for
 * r < min(K, q_pos[t] + 1) and idx >= 0.  q: bf16 [T, H, d_qk]; out: bf16
 * [T, H, d_v]; lse: fp32 [T, H] or NULL.  No workspace. */
dsa_status_t dsa_sparse_attn_prefill(const dsa_paged_cache_t *cache, const uint16_t *q,
                                     const int32_t *q_seq, const int32_t *q_pos,
                                     const int32_t *idx, int32_t T, int32_t H, int32_t K,
                                     float sm_scale, uint16_t *out, float *lse,
                                     hipStream_t stream);

/* Cache write (page 1, section 3 item (2), the paged layout; page
 * "Day-0 Adaptation of Ultra-Large-Scale MoE Models on Heterogeneous AI
 * Accelerators", section 4: what a prefill writes is what a decode reads).
 * Token i of sequence seq[i] at logical position pos[i] is stored in the
 * physical row block_table[seq[i] * max_blocks_per_seq + pos[i] / block_size]
 * * block_size + pos[i] % block_size of each pool: kv_new row i (d_qk
 * columns) into kv, v_new row i (d_v columns) into v, k_idx_new row i (d_idx
 * columns) into k_idx.  The pools are written in place through the cache's
 * pointers.  kv_new: bf16 [n, d_qk]; v_new: bf16 [n, d_v], NULL exactly when
 * cache->v is NULL (the latent family, whose V is part of the kv row);
 * k_idx_new: bf16 [n, d_idx]; seq, pos: int32 [n].  A token whose sequence,
 * position or physical block lies outside the cache description is skipped.
 * Two tokens must not map to the same row (their order is then undefined).
 * seq_lens is neither read nor updated.  n == 0 is a no-op. */
dsa_status_t dsa_cache_write(const dsa_paged_cache_t *cache, const int32_t *seq,
                             const int32_t *pos, int32_t n, const uint16_t *kv_new,
                             const uint16_t *v_new, const uint16_t *k_idx_new,
                             hipStream_t stream);

/* Static text for a status code. */
const char *dsa_status_string(dsa_status_t status);

/* Checks of device data (a debug aid; page "Day-0 Adaptation of
 * Ultra-Large-Scale MoE Models on Heterogeneous AI Accelerators", section 4:
 * the index results decide the cache addresses, so a bad entry must be
 * found where it is read).  In a library built with DSA_DEBUG_BOUNDS, every
 * kernel checks the device data the host cannot see -- block-table entries
 * (0 <= entry < num_blocks), sequence lengths and query positions against
 * the cache description and ld, kept indices against their row's candidate
 * count, Top-K candidate counts against ld -- replaces an out-of-range value
 * by a safe one (block 0, nothing to score, a skipped index) and records
 * it.  This call synchronises `stream`, then returns DSA_ERR_BOUNDS if any
 * call since the previous check met such a value (and clears the record),
 * else DSA_OK.  A release build checks nothing and returns
 * DSA_ERR_UNSUPPORTED. */
dsa_status_t dsa_check_device_errors(hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
