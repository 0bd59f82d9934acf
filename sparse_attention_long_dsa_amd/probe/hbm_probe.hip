// Achievable HBM read bandwidth of the device: a plain streaming read of a
// large buffer (far larger than the last-level cache), 16 bytes per lane per
// load, several independent loads in flight per lane, a persistent grid that
// covers every compute unit.  The measured rate is the practical ceiling the
// bandwidth-bound kernels are compared with, next to the 8 TB/s datasheet
// figure (web page "Day-0 Adaptation of Ultra-Large-Scale MoE Models on
// Heterogeneous AI Accelerators", section 5: record throughput baselines).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kInFlight = 8;  // 16-byte loads a lane keeps in flight

// Thread t of the grid reads the 16-byte vectors t, t + N, t + 2N, ... (N =
// all threads of the grid), kInFlight at a time, and folds them into one
// word that is stored once (so the loads cannot be dropped).
// NT: non-temporal loads (a hint not to keep the lines in the caches) for
// the bandwidth figure; ordinary loads when the read is meant to fill the
// caches with these (clean) lines.
template <bool NT>
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const u32x4* __restrict__ src,
                                                            int64_t n_vec, uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n_vec; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u)
      v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n_vec; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

// Chunked variant: workgroup b streams its own contiguous region (vectors
// b * per_block .. (b + 1) * per_block - 1, per_block a multiple of
// kThreads * kInFlight), each wave load one contiguous KB, kInFlight loads
// in flight per lane -- the pattern of a kernel whose workgroups each
// stream their own weight block.
__global__ __launch_bounds__(kThreads) void hbm_read_chunk_kernel(const u32x4* __restrict__ src,
                                                                  int64_t per_block,
                                                                  uint32_t* __restrict__ sink) {
  const u32x4* p = src + (int64_t)blockIdx.x * per_block + threadIdx.x;
  uint32_t acc = 0;
  for (int64_t i = 0; i < per_block; i += kThreads * kInFlight) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device buffer `src` once; `sink`
// receives one word per thread of the grid (grid_blocks * 256 words).
// nontemporal != 0: non-temporal loads; nontemporal == 2: the chunked
// pattern, each workgroup reading bytes / grid_blocks contiguous bytes
// (bytes must be a multiple of grid_blocks * 32768).  Returns 0, or 1 for
// bad arguments, 2 when the launch fails.
extern "C" int hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int grid_blocks,
                              int nontemporal, hipStream_t stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 != 0 || grid_blocks < 1) return 1;
  if (nontemporal == 2) {
    if (bytes % ((int64_t)grid_blocks * kThreads * kInFlight * 16) != 0) return 1;
    hipLaunchKernelGGL(hbm_read_chunk_kernel, dim3(grid_blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)src, bytes / 16 / grid_blocks, sink);
  } else if (nontemporal)
    hipLaunchKernelGGL(hbm_read_kernel<true>, dim3(grid_blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)src, bytes / 16, sink);
  else
    hipLaunchKernelGGL(hbm_read_kernel<false>, dim3(grid_blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
