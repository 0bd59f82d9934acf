// Host-side argument checks shared by the C-ABI entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "../../include/dsa.h"

namespace dsa {

// DSA_OK when the current device is a gfx950; the answer is cached per
// device id (a racy first fill is harmless: every writer stores the same).
inline dsa_status_t check_device() {
  static int cached[64] = {0};  // 0 unknown, 1 ok, 2 not ok
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DSA_ERR_DEVICE;
  if (dev < 64 && cached[dev]) return cached[dev] == 1 ? DSA_OK : DSA_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSA_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cached[dev] = ok ? 1 : 2;
  return ok ? DSA_OK : DSA_ERR_DEVICE;
}

inline dsa_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
}

// The kernels move 16-byte vectors: device buffers must start 16-byte
// aligned (every allocation of the HIP runtime and of torch is).
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Checks of the paged-cache description common to every call.
inline dsa_status_t check_cache_common(const dsa_paged_cache_t* c) {
  if (!c || !c->block_table) return DSA_ERR_NULL;
  if (c->n_seq < 1 || c->max_blocks_per_seq < 1 || c->num_blocks < 1 || c->block_size < 1)
    return DSA_ERR_SHAPE;
  return DSA_OK;
}

// Each translation unit's debug error word, read and cleared (0 in release
// builds; bit 31 set when reading failed).
__attribute__((visibility("hidden"))) uint32_t take_bounds_error_index_score(hipStream_t stream);
__attribute__((visibility("hidden"))) uint32_t take_bounds_error_topk(hipStream_t stream);
__attribute__((visibility("hidden"))) uint32_t take_bounds_error_cache_write(hipStream_t stream);
__attribute__((visibility("hidden"))) uint32_t take_bounds_error_moe(hipStream_t stream);

// The decode index score that also writes each 16-position group's two
// largest scores (the fused index + Top-K call), in index_score.hip.
__attribute__((visibility("hidden"))) dsa_status_t launch_index_score_decode_gmax(
    const dsa_paged_cache_t* c, const uint16_t* q_idx, const float* w, const int32_t* q_seq,
    const int32_t* q_pos, int n_q, int H_idx, float* scores, int64_t ld, float* gm1, float* gm2,
    int64_t ldg, hipStream_t stream);

}  // namespace dsa
