/*
 * dsa_moe.h — C ABI of libdsa.so, MoE expert part: the expert matrix
 * product with 4-bit expert weights converted to 8-bit floating point just
 * before use, on AMD Instinct MI355X (gfx950).
 *
 * The method (web page "Day-0 Adaptation of Trillion-Parameter MoE Models on
 * Domestic GPUs", section 4 "Online Conversion of 4-Bit Expert Weights and
 * FP8 Workspace Reuse"; web page "Technical Path for Day-0 Adaptation of
 * Trillion-Parameter Models on Domestic GPUs", section 3.2 "Online
 * Conversion of Low-Precision Expert Weights"): expert weights stay in
 * MXFP4; right before an expert's product they are converted to FP8 and the
 * routed tokens are multiplied with them; no FP8 copy of all weights is ever
 * kept.  Three ways to run it:
 *   - dsa_moe_gemm_mxfp4: the conversion happens in registers inside the
 *     product kernel (the weights are read once, at 4.25 bits an element);
 *     no workspace at all; fastest on weights packed once, at load time,
 *     into the tiled layout (dsa_mxfp4_pack);
 *   - dsa_mxfp4_to_fp8 + dsa_moe_gemm_fp8: conversion into a caller's FP8
 *     workspace, then the product from it;
 *   - dsa_moe_gemm_staged: the pages' pipeline -- chunks of the listed
 *     experts are converted on a second stream into the two halves of one
 *     workspace that every layer reuses, each product waits (by event) for
 *     its chunk's conversion, each conversion waits (by event) until the
 *     product that last read that half has finished.
 * All three compute the same values.
 *
 * Formats (OCP Microscaling Formats (MX) v1.0):
 *   - weights of one layer, DSA_MXFP4_ROW_MAJOR: codes uint8 [num_experts,
 *     N, K/2], two FP4 E2M1 elements a byte (element 2i of a row in the low
 *     nibble, 2i+1 in the high nibble), and scales uint8 [num_experts, N,
 *     K/32], one E8M0 scale (2^(code-127); code 255 is NaN) for each 32
 *     consecutive elements (an MX block) of a row;
 *   - DSA_MXFP4_TILED (K a multiple of 256): the same bytes reordered so
 *     that what one 64-lane wave loads is contiguous.  Each expert's rows
 *     are cut into tiles of 16 (tile t = n / 16, r = n % 16) and each row
 *     into units of 256 elements (u = k / 256); unit (t, u) of expert e
 *     holds 2048 code bytes at ((e * N/16 + t) * K/256 + u) * 2048 and 128
 *     scale bytes at the same unit index * 128.  Inside a unit, MX block
 *     b = (k % 256) / 32 of row r belongs to lane L = 16 * (b / 2) + r and
 *     half h = b % 2: its 16 code bytes (same nibble order) sit at byte
 *     1024 h + 16 L and its scale at byte 2 L + h;
 *   - FP8 is E4M3 (the OCP "E4M3FN" encoding: bias 7, largest finite 448,
 *     S.1111.111 NaN).  The converted weight is the E4M3 number nearest to
 *     scale x element (ties to even mantissa), saturated to +-448 (a NaN
 *     scale gives 0x7f); the conversion is exact for scale codes 119..133;
 *   - the routed tokens x are E4M3 codes [M, K]; the result y is fp32
 *     [M, N]: y[r, n] = sum_k x[r, k] * w8_e[n, k] with the products exact
 *     and the sum accumulated in fp32 on the matrix cores.
 * Routing: listed expert i (0 <= i < n_act) is expert expert_ids[i] of the
 * layer, and the token rows routed to it are rows row_offsets[i] ..
 * row_offsets[i+1] - 1 of x and y (the caller groups tokens by expert);
 * expert_ids int32 [n_act], row_offsets int32 [n_act + 1], both device
 * arrays (device data: 0 <= expert_ids[i] < num_experts and 0 <=
 * row_offsets[i] <= row_offsets[i+1] <= M are not checked by release
 * builds; a debug build skips a bad expert or range and reports it through
 * dsa_check_device_errors).  Rows of y not covered by any range are left
 * untouched.  max_rows is the caller's bound on rows of one listed expert; it
 * only shapes the launch (any count is computed right; counts above it run
 * slower).
 * Shapes: K a multiple of 128, N a multiple of 16, 1 <= n_act <= 65535,
 * else DSA_ERR_UNSUPPORTED / DSA_ERR_SHAPE.  Pointers are device memory owned
 * by the caller, 16-byte aligned; work is enqueued on `stream`; arguments are
 * checked on the host before anything is launched (statuses of dsa.h).
 */
#ifndef DSA_MOE_H
#define DSA_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "dsa.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_MXFP4_ROW_MAJOR 0
#define DSA_MXFP4_TILED 1

/* One layer's MXFP4 expert weights (device pointers). */
typedef struct {
  const uint8_t *codes;   /* num_experts * N * K/2 FP4 E2M1 pairs  */
  const uint8_t *scales;  /* num_experts * N * K/32 E8M0 (4-byte aligned) */
  int32_t num_experts;
  int32_t N;              /* output features of each expert        */
  int32_t K;              /* input features                        */
  int32_t layout;         /* DSA_MXFP4_ROW_MAJOR or DSA_MXFP4_TILED */
} dsa_mxfp4_weights_t;

/* Reorders row-major weights (w->layout == DSA_MXFP4_ROW_MAJOR, K a
 * multiple of 256) into the tiled layout: codes_tiled and scales_tiled
 * receive the same number of bytes as w's arrays (no value changes; done
 * once when the weights are loaded).  DSA_ERR_SHAPE for tiled input. */
dsa_status_t dsa_mxfp4_pack(const dsa_mxfp4_weights_t *w, uint8_t *codes_tiled,
                            uint8_t *scales_tiled, hipStream_t stream);

/* Expert product with the MXFP4 -> FP8 conversion done in registers inside
 * the product kernel (page 2, section 3.2: conversion and product
 * pipelined).  x: E4M3 [M, K]; y: fp32 [M, N].  No workspace. */
dsa_status_t dsa_moe_gemm_mxfp4(const dsa_mxfp4_weights_t *w, const uint8_t *x,
                                const int32_t *expert_ids, const int32_t *row_offsets,
                                int32_t n_act, int32_t M, int32_t max_rows, float *y,
                                hipStream_t stream);

/* The conversion on its own (page 1, section 4: dequantise to 8-bit right
 * before the product): w8[i] ([n_act, N, K] E4M3 bytes, row-major whatever
 * w's layout) receives the converted weights of expert expert_ids[i]. */
dsa_status_t dsa_mxfp4_to_fp8(const dsa_mxfp4_weights_t *w, const int32_t *expert_ids,
                              int32_t n_act, uint8_t *w8, hipStream_t stream);

/* The product from converted weights: listed expert i's weights are w8[i]
 * ([n_act, N, K] E4M3), its rows row_offsets[i] .. row_offsets[i+1] - 1. */
dsa_status_t dsa_moe_gemm_fp8(const uint8_t *w8, int32_t N, int32_t K, const uint8_t *x,
                              const int32_t *row_offsets, int32_t n_act, int32_t M,
                              int32_t max_rows, float *y, hipStream_t stream);

/* Workspace bytes of dsa_moe_gemm_staged for chunks of chunk_experts
 * experts: two halves of chunk_experts * N * K bytes. */
size_t dsa_moe_staged_ws(int32_t N, int32_t K, int32_t chunk_experts);

/* The pages' staged pipeline (page 1, section 4, the pseudocode and the
 * synchronisation it asks for; page 2, section 3.2: one cross-layer FP8
 * workspace, chunked conversion).  The listed experts are split into
 * chunks of chunk = workspace_bytes / (2 N K) experts (at least 1, else
 * DSA_ERR_WORKSPACE); chunk c is converted on conv_stream into half c % 2
 * of the workspace and multiplied on `stream`.  Ordering, all by events:
 *   - at entry the call records events[4] on `stream` and conv_stream waits
 *     for it, so the conversions see everything enqueued on `stream` before
 *     the call (weights written there, the workspace's earlier users);
 *   - conversion c waits for events[2 + c % 2] ("half free"), recorded on
 *     `stream` after the product that last read that half -- in this call
 *     or an earlier one: the same workspace and events serve every layer;
 *   - product c waits for events[c % 2] ("half converted"), recorded on
 *     conv_stream after conversion c.
 * events: five caller-owned events (created with hipEventDisableTiming
 * preferably) that stay with this workspace for its lifetime; events never
 * recorded before count as complete.  With K a multiple of 256 the
 * workspace holds the converted weights in the tiled unit order (4096
 * bytes a unit).  conv_stream must differ from `stream`.  When the call
 * returns, everything is enqueued; y is complete once `stream` has reached
 * its end (every conversion precedes a product on it).  Results equal
 * dsa_moe_gemm_mxfp4's. */
dsa_status_t dsa_moe_gemm_staged(const dsa_mxfp4_weights_t *w, const uint8_t *x,
                                 const int32_t *expert_ids, const int32_t *row_offsets,
                                 int32_t n_act, int32_t M, int32_t max_rows, float *y,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream,
                                 hipStream_t conv_stream, hipEvent_t *events);

#ifdef __cplusplus
}
#endif

#endif /* DSA_MOE_H */
