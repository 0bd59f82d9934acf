// Paged cache write (web page "Day-0 Adaptation of Trillion-Parameter MoE
// Models on Domestic GPUs", section 3 item (2): the cache lives in
// non-contiguous blocks reached through an index table; web page "Day-0
// Adaptation of Ultra-Large-Scale MoE Models on Heterogeneous AI
// Accelerators", section 4: the layout a prefill writes must be the layout
// a decode reads).  New tokens' latent rows, value rows and indexer keys go
// to the physical slots their (sequence, position) map to through the one
// block table that every read call uses.
#include "common.h"
#include "host_util.h"

namespace dsa {
namespace {

constexpr int kTokensPerBlock = 4;                 // one wave per token
constexpr int kWriteThreads = kTokensPerBlock * kWave;

// Copies `chunks` 16-byte pieces of one row (one wave, 16 bytes a lane).
__device__ __forceinline__ void copy_row(uint16_t* __restrict__ dst, const uint16_t* __restrict__ src,
                                         int chunks, int lane) {
  for (int c = lane; c < chunks; c += kWave)
    *(u32x4*)(dst + 8 * c) = *(const u32x4*)(src + 8 * c);
}

// One wave per token, four tokens per workgroup.  Tokens whose sequence,
// position or physical block fall outside the cache description are
// skipped (no write).
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(
    uint16_t* __restrict__ kv, int64_t kv_stride, uint16_t* __restrict__ v, int64_t v_stride,
    uint16_t* __restrict__ k_idx, int64_t k_idx_stride, const int32_t* __restrict__ block_table,
    int n_seq, int max_blocks, int num_blocks, int bs, int d_qk, int d_v, int d_idx,
    const int32_t* __restrict__ seq, const int32_t* __restrict__ pos,
    const uint16_t* __restrict__ kv_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ k_idx_new, int n) {
  const int i = blockIdx.x * kTokensPerBlock + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (i >= n) return;
  const int b = seq[i], p = pos[i];
  if (b < 0 || b >= n_seq || p < 0 || p / bs >= max_blocks) return;
  const int blk = block_table[(int64_t)b * max_blocks + p / bs];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t row = (int64_t)blk * bs + p % bs;
  copy_row(kv + row * kv_stride, kv_new + (int64_t)i * d_qk, d_qk / 8, lane);
  if (v) copy_row(v + row * v_stride, v_new + (int64_t)i * d_v, d_v / 8, lane);
  copy_row(k_idx + row * k_idx_stride, k_idx_new + (int64_t)i * d_idx, d_idx / 8, lane);
}

}  // namespace

// Tokens outside the cache description are skipped by contract, so the
// cache write raises no debug error; its word stays 0.
uint32_t take_bounds_error_cache_write(hipStream_t stream) { return take_bounds_error(stream); }

}  // namespace dsa

extern "C" dsa_status_t dsa_cache_write(const dsa_paged_cache_t* cache, const int32_t* seq,
                                        const int32_t* pos, int32_t n, const uint16_t* kv_new,
                                        const uint16_t* v_new, const uint16_t* k_idx_new,
                                        hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_cache_common(cache);
  if (st != DSA_OK) return st;
  if (!cache->kv || !cache->k_idx || !seq || !pos || !kv_new || !k_idx_new) return DSA_ERR_NULL;
  if ((cache->v == nullptr) != (v_new == nullptr)) return DSA_ERR_NULL;
  if (n < 0) return DSA_ERR_SHAPE;
  if (cache->d_qk < 1 || cache->d_idx < 1 || (cache->v && cache->d_v < 1)) return DSA_ERR_SHAPE;
  if (cache->kv_row_stride < cache->d_qk || cache->k_idx_row_stride < cache->d_idx ||
      (cache->v && cache->v_row_stride < cache->d_v))
    return DSA_ERR_SHAPE;
  if (cache->d_qk % 8 || cache->d_idx % 8 || (cache->v && cache->d_v % 8) ||
      cache->kv_row_stride % 8 || cache->k_idx_row_stride % 8 || (cache->v && cache->v_row_stride % 8))
    return DSA_ERR_UNSUPPORTED;
  if (!aligned16(cache->kv) || !aligned16(cache->k_idx) || (cache->v && !aligned16(cache->v)) ||
      !aligned16(kv_new) || !aligned16(k_idx_new) || (v_new && !aligned16(v_new)))
    return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  if (n == 0) return DSA_OK;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)((n + kTokensPerBlock - 1) / kTokensPerBlock)),
                     dim3(kWriteThreads), 0, stream,
                     (uint16_t*)cache->kv, cache->kv_row_stride, (uint16_t*)cache->v,
                     cache->v_row_stride, (uint16_t*)cache->k_idx, cache->k_idx_row_stride,
                     cache->block_table, cache->n_seq, cache->max_blocks_per_seq,
                     cache->num_blocks, cache->block_size, cache->d_qk, cache->d_v, cache->d_idx,
                     seq, pos, kv_new, v_new, k_idx_new, n);
  return launch_status();
}
