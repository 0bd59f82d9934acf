/*
 * DSA sparse attention: the oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU statement of what the DSA hot path computes.  Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the GPU
 * library never does, and the two share no code.
 *
 * The method (web pages: "Day-0 Adaptation of Trillion-Parameter MoE Models
 * on Domestic GPUs", section 3 "Adapting Sparse Attention (DSA)", items (1)
 * Index Selection, (2) KV Cache Layout and (3) Two Compute Paths; "Technical
 * Path for Day-0 Adaptation of Trillion-Parameter Models on Domestic GPUs",
 * section 3.1 "Implementing Sparse Attention"; "Day-0 Adaptation of
 * Ultra-Large-Scale MoE Models on Heterogeneous AI Accelerators", sections
 * 3.2 "Operator Layer" and 4 "Joint Debugging Essentials"):
 *   a lightweight indexer scores every past position, the K best positions
 *   are kept, and exact softmax attention runs over those positions only,
 *   reading K/V rows from a block-paged cache through a block table.
 *
 * Readings taken where the pages are silent (each is a plain reading):
 *   - index score of query i against position s of its sequence:
 *       score = sum_h w[i,h] * max(0, q_idx[i,h,:] . k_idx[s,:])
 *     with one indexer key per position shared by all indexer heads.  The
 *     pages only say "similarity scoring" after a dimension-reducing
 *     projection; a per-head ReLU is what keeps several weighted heads from
 *     collapsing into one.  `relu = 0` switches to the identity (a test aid).
 *   - candidates of the query at position t are positions 0..t (its own
 *     position included);
 *   - Top-K keeps the K largest scores, equal scores ordered by lower
 *     position first; fewer than K candidates -> all of them; the kept
 *     positions are listed ascending and padded with -1 up to K;
 *   - attention: logits = sm_scale * q . K_j over the kept j, ordinary
 *     softmax, output = sum_j p_j V_j, and lse = natural log of the softmax
 *     normaliser (max-shifted).  No kept position -> output 0, lse = -inf.
 *
 * Arithmetic: every sum is accumulated in double; results are stored as
 * fp32.  bf16 inputs are passed as raw 16-bit patterns.
 *
 * Paged cache (item (2) above): position p of sequence b lives at physical
 * row block_table[b][p / block_size] * block_size + p % block_size of a pool
 * whose rows are `row_stride` elements apart.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static int64_t physical_row(const int32_t *block_table, int32_t max_blocks, int32_t block_size,
                            int32_t seq, int64_t pos) {
  int32_t block = block_table[(int64_t)seq * max_blocks + pos / block_size];
  return (int64_t)block * block_size + pos % block_size;
}

/* Index score (item (1), "similarity scoring").
 * scores[i * ld + s] for s = 0..q_pos[i]; other entries are left untouched. */
void oracle_index_score(const uint16_t *k_idx, int64_t k_idx_row_stride,
                        const int32_t *block_table, int32_t max_blocks, int32_t block_size,
                        int32_t d_idx, const uint16_t *q_idx, const float *w,
                        const int32_t *q_seq, const int32_t *q_pos, int32_t n_q, int32_t H_idx,
                        int32_t relu, float *scores, int64_t ld) {
  for (int32_t i = 0; i < n_q; ++i) {
    const int64_t n = (int64_t)q_pos[i] + 1;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < n; ++s) {
      const uint16_t *key =
          k_idx + physical_row(block_table, max_blocks, block_size, q_seq[i], s) * k_idx_row_stride;
      double total = 0.0;
      for (int32_t h = 0; h < H_idx; ++h) {
        const uint16_t *qh = q_idx + ((int64_t)i * H_idx + h) * d_idx;
        double dot = 0.0;
        for (int32_t d = 0; d < d_idx; ++d) dot += bf16_value(qh[d]) * bf16_value(key[d]);
        if (relu && dot < 0.0) dot = 0.0;
        total += (double)w[(int64_t)i * H_idx + h] * dot;
      }
      scores[(int64_t)i * ld + s] = (float)total;
    }
  }
}

typedef struct {
  float score;
  int32_t pos;
} candidate;

/* larger score first; equal scores: lower position first */
static int by_score_then_position(const void *a, const void *b) {
  const candidate *x = (const candidate *)a, *y = (const candidate *)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->pos > y->pos) - (x->pos < y->pos);
}

static int ascending_int(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* Top-K (item (1), "Top-K filtering").  Row i holds n_valid[i] candidates
 * scores[i * ld + 0 .. n_valid[i]-1].  idx[i * K + r] receives the kept
 * positions ascending, then -1.  The definition is written out directly:
 * order all candidates by (score desc, position asc), keep the first K. */
void oracle_topk(const float *scores, int64_t ld, const int32_t *n_valid, int32_t n_q, int32_t K,
                 int32_t *idx) {
#pragma omp parallel for schedule(dynamic)
  for (int32_t i = 0; i < n_q; ++i) {
    const int64_t n = n_valid[i];
    candidate *c = (candidate *)malloc((size_t)(n > 0 ? n : 1) * sizeof(candidate));
    for (int64_t s = 0; s < n; ++s) {
      c[s].score = scores[(int64_t)i * ld + s];
      c[s].pos = (int32_t)s;
    }
    qsort(c, (size_t)n, sizeof(candidate), by_score_then_position);
    const int64_t kept = n < K ? n : K;
    int32_t *row = idx + (int64_t)i * K;
    for (int64_t r = 0; r < kept; ++r) row[r] = c[r].pos;
    qsort(row, (size_t)kept, sizeof(int32_t), ascending_int);
    for (int64_t r = kept; r < K; ++r) row[r] = -1;
    free(c);
  }
}

/* Exact attention over the kept positions (section 3 of the first page: exact
 * attention only over the selected positions; item (2): rows gathered through
 * the block table).  q: [n_q, H, d_qk]; idx: [n_q, K] (-1 = none);
 * out: [n_q, H, d_v] fp32; lse: [n_q, H] fp32 (may be NULL).
 * K_j = k_pool row of position j (d_qk columns); V_j = v_pool row of position
 * j (its first d_v columns; v_pool may be the same pool as k_pool). */
void oracle_sparse_attn(const uint16_t *k_pool, int64_t k_row_stride, const uint16_t *v_pool,
                        int64_t v_row_stride, const int32_t *block_table, int32_t max_blocks,
                        int32_t block_size, int32_t d_qk, int32_t d_v, const uint16_t *q,
                        const int32_t *q_seq, const int32_t *idx, int32_t n_q, int32_t H,
                        int32_t K, double sm_scale, float *out, float *lse) {
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int32_t i = 0; i < n_q; ++i) {
    for (int32_t h = 0; h < H; ++h) {
      const uint16_t *qh = q + ((int64_t)i * H + h) * d_qk;
      const int32_t *sel = idx + (int64_t)i * K;
      double *logit = (double *)malloc((size_t)K * sizeof(double));
      double *acc = (double *)calloc((size_t)d_v, sizeof(double));
      double m = -INFINITY;
      for (int32_t j = 0; j < K; ++j) {
        logit[j] = -INFINITY;
        if (sel[j] < 0) continue;
        const uint16_t *kr =
            k_pool + physical_row(block_table, max_blocks, block_size, q_seq[i], sel[j]) *
                         k_row_stride;
        double dot = 0.0;
        for (int32_t d = 0; d < d_qk; ++d) dot += bf16_value(qh[d]) * bf16_value(kr[d]);
        logit[j] = sm_scale * dot;
        if (logit[j] > m) m = logit[j];
      }
      double z = 0.0;
      for (int32_t j = 0; j < K; ++j) {
        if (sel[j] < 0) continue;
        const double p = exp(logit[j] - m);
        const uint16_t *vr =
            v_pool + physical_row(block_table, max_blocks, block_size, q_seq[i], sel[j]) *
                         v_row_stride;
        z += p;
        for (int32_t d = 0; d < d_v; ++d) acc[d] += p * bf16_value(vr[d]);
      }
      float *o = out + ((int64_t)i * H + h) * d_v;
      for (int32_t d = 0; d < d_v; ++d) o[d] = z > 0.0 ? (float)(acc[d] / z) : 0.0f;
      if (lse) lse[(int64_t)i * H + h] = z > 0.0 ? (float)(m + log(z)) : -INFINITY;
      free(logit);
      free(acc);
    }
  }
}
