/*
 * MoE expert GEMM with online MXFP4 -> FP8 conversion: the oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  The plain, slow CPU statement of what the expert
 * path computes; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code with the GPU path.
 *
 * The method (web pages "Day-0 Adaptation of Trillion-Parameter MoE Models on
 * Domestic GPUs", section 4 "Online Conversion of 4-Bit Expert Weights and
 * FP8 Workspace Reuse"; "Technical Path for Day-0 Adaptation of
 * Trillion-Parameter Models on Domestic GPUs", section 3.2 "Online Conversion
 * of Low-Precision Expert Weights"): expert weights are stored in MXFP4; just
 * before the matrix product they are converted to 8-bit floating point, and
 * the product of the routed tokens with the converted weights is computed.
 *
 * Formats (the OCP Microscaling (MX) specification, v1.0, which the pages
 * name by "MXFP4"; "8-bit floating point" read as FP8 E4M3):
 *   - MXFP4 block: 32 consecutive elements along K share one E8M0 scale
 *     X = 2^(code - 127) (code 255 is NaN); each element is FP4 E2M1: sign,
 *     2 exponent bits (bias 1), 1 mantissa bit; exponent field 0 is the
 *     subnormal range (0 or 0.5).  Element 2i of a byte pair sits in the low
 *     nibble, 2i+1 in the high nibble.
 *   - FP8 E4M3 (the OCP "E4M3FN" encoding): sign, 4 exponent bits (bias 7),
 *     3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite 448.
 *     Conversion of a real value rounds to nearest, ties to even, and
 *     saturates at +-448 ("satfinite").
 * Readings taken where the pages are silent: the conversion applies the
 * block scale (the FP8 weight equals scale x element, exactly so whenever
 * that value is an E4M3 number, which holds for every element when the
 * scale code is in 119..133), the routed tokens are FP8 E4M3 as well (an
 * "8-bit matrix multiply"), and the product accumulates in double here and
 * is stored as fp32.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* FP4 E2M1 code (low 4 bits) -> value, from its fields. */
double oracle_fp4_value(uint8_t code) {
  const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E8M0 scale code -> value (NaN for 255). */
double oracle_e8m0_value(uint8_t code) {
  return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
}

/* E4M3 code -> value. */
double oracle_e4m3_value(uint8_t code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double mag = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* Real value -> E4M3 code: round to nearest (ties to even) among the finite
 * E4M3 values, saturating at +-448; NaN -> 0x7f.  Written as a search over
 * the 127 non-negative finite codes, which are ordered by value. */
uint8_t oracle_e4m3_encode(double x) {
  if (isnan(x)) return 0x7f;
  const uint8_t sign = (signbit(x) ? 0x80 : 0);
  double a = fabs(x);
  if (a >= 448.0) return sign | 0x7e;
  uint8_t best = 0;
  for (int c = 1; c < 0x7f; ++c) {  /* largest code whose value <= a */
    if (oracle_e4m3_value((uint8_t)c) <= a) best = (uint8_t)c;
  }
  if (oracle_e4m3_value(best) == a) return sign | best;
  const double lo = oracle_e4m3_value(best), hi = oracle_e4m3_value((uint8_t)(best + 1));
  uint8_t pick;
  if (a - lo < hi - a) pick = best;
  else if (hi - a < a - lo) pick = (uint8_t)(best + 1);
  else pick = (best & 1) ? (uint8_t)(best + 1) : best;  /* tie: even mantissa */
  return sign | pick;
}

/* The E4M3 code of scale x element for every (E8M0 scale, FP4 code) pair:
 * an MXFP4 element only ever takes one of these 256 x 16 values. */
static void conversion_table(uint8_t table[256][16]) {
  for (int sc = 0; sc < 256; ++sc)
    for (int c = 0; c < 16; ++c)
      table[sc][c] = oracle_e4m3_encode(oracle_e8m0_value((uint8_t)sc) * oracle_fp4_value((uint8_t)c));
}

/* The conversion step: for each listed expert i (weights expert_ids[i] of
 * codes [*, N, K/2] and scales [*, N, K/32]) write the E4M3 codes of its
 * N x K weights (element k of row n: the FP4 code in nibble k % 2 of byte
 * k / 2, scaled by scale k / 32 of the row) into out[i] ([E, N, K] bytes). */
void oracle_mxfp4_to_fp8(const uint8_t *codes, const uint8_t *scales, const int32_t *expert_ids,
                         int32_t E, int32_t N, int32_t K, uint8_t *out) {
  static uint8_t table[256][16];
  conversion_table(table);
  for (int32_t i = 0; i < E; ++i) {
    const int64_t ex = expert_ids[i];
    const uint8_t *c = codes + ex * (int64_t)N * (K / 2);
    const uint8_t *s = scales + ex * (int64_t)N * (K / 32);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t k = 0; k < K; ++k) {
        const uint8_t byte = c[n * (K / 2) + k / 2];
        const uint8_t code = (k & 1) ? (byte >> 4) : (byte & 15);
        out[((int64_t)i * N + n) * K + k] = table[s[n * (K / 32) + k / 32]][code];
      }
  }
}

/* The expert product: token rows row_offsets[i] .. row_offsets[i+1]-1 of x
 * ([M, K] E4M3 codes) belong to listed expert i;
 *   y[r, n] = sum_k x[r, k] * w8_i[n, k]
 * with w8_i the E4M3 conversion of expert expert_ids[i]'s MXFP4 weights (as
 * oracle_mxfp4_to_fp8 writes it).  Double accumulation, fp32 result [M, N].
 * w8 is caller scratch of N * K bytes. */
void oracle_moe_gemm(const uint8_t *x, const int32_t *row_offsets, const int32_t *expert_ids,
                     int32_t E, const uint8_t *codes, const uint8_t *scales, int32_t N, int32_t K,
                     uint8_t *w8, float *y) {
  double e4m3[256];
  for (int c = 0; c < 256; ++c) e4m3[c] = oracle_e4m3_value((uint8_t)c);
  for (int32_t i = 0; i < E; ++i) {
    oracle_mxfp4_to_fp8(codes, scales, expert_ids + i, 1, N, K, w8);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t r = row_offsets[i]; r < row_offsets[i + 1]; ++r) {
      for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += e4m3[x[r * K + k]] * e4m3[w8[n * K + k]];
        y[r * N + n] = (float)acc;
      }
    }
  }
}
