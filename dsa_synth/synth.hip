// Seeded synthetic inputs for the DSA workloads: one counter-based generator,
// compiled once for the host and once for the device from the same source, so
// both sides of a parity test see bit-identical inputs.
//
// This file holds no part of the attention method: it only turns logical
// coordinates into pseudo-random values and stores them where a caller asks.
//
// Generator: every value is a pure function of (seed, tensor id, three
// logical coordinates).  The mixing step is the "lowbias32" integer hash
// published by C. Wellons (hash-prospector, 2018): xorshift 16, multiply by
// 0x7feb352d, xorshift 15, multiply by 0x846ca68b, xorshift 16.
//
// Value kinds
//   0  bf16 normal deviate: the top 16 hash bits index a 65536-entry table of
//      N(0,1) quantiles (bf16 bits) supplied by the caller;
//   1  bf16 holding an integer uniform on [lo, hi];
//   2  fp32 holding an integer uniform on [lo, hi].
// Integers use Lemire's multiply-shift reduction: lo + (h * (hi-lo+1)) >> 32.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__host__ __device__ inline uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__host__ __device__ inline uint32_t hash5(uint32_t seed, uint32_t tid, uint32_t a,
                                          uint32_t b, uint32_t c) {
  uint32_t h = mix32(seed * 0x9E3779B9u ^ (tid + 0x632BE5ABu));
  h = mix32(h ^ a);
  h = mix32(h + b * 0x85EBCA77u);
  h = mix32(h ^ (c * 0xC2B2AE3Du + 0x27D4EB2Fu));
  return h;
}

__host__ __device__ inline uint32_t int_in(uint32_t h, int lo, int hi) {
  uint64_t span = (uint64_t)(int64_t)(hi - lo + 1);
  return (uint32_t)(lo + (int64_t)(((uint64_t)h * span) >> 32));
}

// bf16 bits of a small integer (|v| < 256 is exact in bf16).
__host__ __device__ inline uint16_t int_to_bf16_bits(int v) {
  float f = (float)v;
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);  // exact: small integers have <= 8 significant bits
}

__host__ __device__ inline void store_value(void* out, int64_t off, int kind, uint32_t h,
                                            int lo, int hi, const uint16_t* table) {
  if (kind == 0) {
    ((uint16_t*)out)[off] = table[h >> 16];
  } else if (kind == 1) {
    ((uint16_t*)out)[off] = int_to_bf16_bits((int)int_in(h, lo, hi));
  } else {
    ((float*)out)[off] = (float)(int)int_in(h, lo, hi);
  }
}

// Physical row of logical position pos in a block-paged pool.
__host__ __device__ inline int64_t paged_row(const int32_t* bt_row, int bs, int64_t pos) {
  return (int64_t)bt_row[pos / bs] * bs + pos % bs;
}

__global__ void dense_kernel(void* out, int kind, uint32_t seed, uint32_t tid, int64_t a0,
                             int64_t na, int nb, int nc, int lo, int hi,
                             const uint16_t* table) {
  const int64_t total = na * nb * nc;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    int64_t c = e % nc, r = e / nc;
    int64_t b = r % nb, a = r / nb;
    uint32_t h = hash5(seed, tid, (uint32_t)(a0 + a), (uint32_t)b, (uint32_t)c);
    store_value(out, e, kind, h, lo, hi, table);
  }
}

__global__ void paged_kernel(void* pool, int64_t row_stride, int kind, uint32_t seed,
                             uint32_t tid, int seq, int64_t pos0, int64_t npos, int nc,
                             const int32_t* bt_row, int bs, int lo, int hi,
                             const uint16_t* table) {
  const int64_t total = npos * nc;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    int64_t c = e % nc, p = pos0 + e / nc;
    uint32_t h = hash5(seed, tid, (uint32_t)seq, (uint32_t)p, (uint32_t)c);
    store_value(pool, paged_row(bt_row, bs, p) * row_stride + c, kind, h, lo, hi, table);
  }
}

int grid_for(int64_t total) {
  int64_t g = (total + 255) / 256;
  return (int)(g < 65536 ? (g < 1 ? 1 : g) : 65536);
}

}  // namespace

extern "C" {

// One raw hash value, for tests of the generator itself.
uint32_t synth_hash(uint32_t seed, uint32_t tid, uint32_t a, uint32_t b, uint32_t c) {
  return hash5(seed, tid, a, b, c);
}

// out[(a-a0), b, c] for a in [a0, a0+na), b < nb, c < nc  (host memory).
int synth_dense_host(void* out, int kind, uint32_t seed, uint32_t tid, int64_t a0,
                     int64_t na, int nb, int nc, int lo, int hi, const uint16_t* table) {
  if (!out || na < 0 || nb < 0 || nc < 0 || (kind == 0 && !table)) return 1;
  int64_t e = 0;
  for (int64_t a = 0; a < na; ++a)
    for (int b = 0; b < nb; ++b)
      for (int c = 0; c < nc; ++c, ++e)
        store_value(out, e, kind, hash5(seed, tid, (uint32_t)(a0 + a), (uint32_t)b, (uint32_t)c),
                    lo, hi, table);
  return 0;
}

// Logical rows [pos0, pos0+npos) of sequence `seq`, nc columns each, stored at
// their physical rows of a paged pool (host memory).  bt_row is that
// sequence's block-table row.
int synth_paged_host(void* pool, int64_t row_stride, int kind, uint32_t seed, uint32_t tid,
                     int seq, int64_t pos0, int64_t npos, int nc, const int32_t* bt_row,
                     int bs, int lo, int hi, const uint16_t* table) {
  if (!pool || !bt_row || bs <= 0 || (kind == 0 && !table)) return 1;
  for (int64_t p = pos0; p < pos0 + npos; ++p) {
    int64_t base = paged_row(bt_row, bs, p) * row_stride;
    for (int c = 0; c < nc; ++c)
      store_value(pool, base + c, kind, hash5(seed, tid, (uint32_t)seq, (uint32_t)p, (uint32_t)c),
                  lo, hi, table);
  }
  return 0;
}

// Device twins of the two functions above; all pointers are device memory.
int synth_dense_device(void* out, int kind, uint32_t seed, uint32_t tid, int64_t a0,
                       int64_t na, int nb, int nc, int lo, int hi, const uint16_t* table,
                       hipStream_t stream) {
  if (!out || na < 0 || nb < 0 || nc < 0 || (kind == 0 && !table)) return 1;
  int64_t total = na * nb * nc;
  if (total == 0) return 0;
  hipLaunchKernelGGL(dense_kernel, dim3(grid_for(total)), dim3(256), 0, stream, out, kind, seed,
                     tid, a0, na, nb, nc, lo, hi, table);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

int synth_paged_device(void* pool, int64_t row_stride, int kind, uint32_t seed, uint32_t tid,
                       int seq, int64_t pos0, int64_t npos, int nc, const int32_t* bt_row,
                       int bs, int lo, int hi, const uint16_t* table, hipStream_t stream) {
  if (!pool || !bt_row || bs <= 0 || (kind == 0 && !table)) return 1;
  int64_t total = npos * nc;
  if (total == 0) return 0;
  hipLaunchKernelGGL(paged_kernel, dim3(grid_for(total)), dim3(256), 0, stream, pool,
                     row_stride, kind, seed, tid, seq, pos0, npos, nc, bt_row, bs, lo, hi, table);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Seeded Fisher-Yates shuffle of 0..n-1 (host).  Step i (from n-1 down to 1)
// swaps entry i with entry j = uniform integer on [0, i] from hash(seed, tid, i).
int synth_permutation(int32_t* out, int n, uint32_t seed, uint32_t tid) {
  if (!out || n < 0) return 1;
  for (int i = 0; i < n; ++i) out[i] = i;
  for (int i = n - 1; i >= 1; --i) {
    int j = (int)int_in(hash5(seed, tid, (uint32_t)i, 0, 0), 0, i);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
  return 0;
}

// n integers uniform on [lo, hi], entry i from hash(seed, tid, i)  (host).
int synth_uniform_ints(int32_t* out, int n, uint32_t seed, uint32_t tid, int lo, int hi) {
  if (!out || n < 0 || hi < lo) return 1;
  for (int i = 0; i < n; ++i) out[i] = (int32_t)int_in(hash5(seed, tid, (uint32_t)i, 0, 0), lo, hi);
  return 0;
}

}  // extern "C"
