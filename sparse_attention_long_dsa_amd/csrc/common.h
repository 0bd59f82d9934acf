// Shared device helpers for the gfx950 DSA kernels: bf16 <-> fp32, MFMA
// operand types, wave64 reductions and the paged-cache row lookup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even: one gfx950
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}
// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed fp16 pair, round to nearest even: one gfx950
// v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
}
// Eight bf16 (packed in pairs) -> eight fp16.  Exact for magnitudes in
// [2^-17, 65504]; smaller ones keep an absolute error below 2^-25.
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_f16x2(bf16_lo(v[i]), bf16_hi(v[i]));
  return as_f16x8(r);
}
__device__ __forceinline__ float f16_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// D = A(16x32) * B(32x16) + C on the gfx950 matrix cores, bf16 in, fp32 out.
// Operand layout (wave64): lane l holds row/column (l & 15) and the 8
// consecutive k-slots 8*(l >> 4) .. +7; the result lane l holds column
// (l & 15), rows 4*(l >> 4) .. +3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The same shape with fp16 operands.
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Direct global -> LDS load of 16 bytes a lane (lane l fills LDS bytes
// lds + 16 l .. + 15), written out so that the compiler does not track it:
// it would otherwise wait for every such load in flight before each LDS read,
// which serialises the loads of the next tile with the current tile's
// products.  Completion is awaited explicitly (s_waitcnt vmcnt) before the
// barrier that hands a tile to its readers.  M0 is saved and restored.
__device__ __forceinline__ void global_to_lds16(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}
// Checks of device data in debug builds (compiled with DSA_DEBUG_BOUNDS).
// The host never reads block-table entries, lengths, query positions or kept
// indices (that would need a synchronisation); a debug build checks each of
// them where a kernel reads it, replaces an out-of-range value by a safe one
// (block 0, nothing to score, a skipped index) and raises a bit of the
// translation unit's error word, which dsa_check_device_errors reads and
// clears.  Release builds compile the checks away.
#ifdef DSA_DEBUG_BOUNDS
constexpr bool kCheckBounds = true;
#else
constexpr bool kCheckBounds = false;
#endif
enum : uint32_t {
  kErrBlock = 1u,     // a block-table entry outside [0, num_blocks)
  kErrQuery = 2u,     // a query's sequence or position outside the cache description
  kErrIndex = 4u,     // a kept index at or past its row's candidate count
  kErrLength = 8u,    // a sequence length or candidate count out of range
};

namespace {
#ifdef DSA_DEBUG_BOUNDS
__device__ uint32_t g_bounds_error;  // one per translation unit
#endif
__device__ __forceinline__ void raise_error(uint32_t bits) {
#ifdef DSA_DEBUG_BOUNDS
  atomicOr(&g_bounds_error, bits);
#else
  (void)bits;
#endif
}
// Reads and clears this translation unit's error word (0 in release builds).
inline uint32_t take_bounds_error(hipStream_t stream) {
#ifdef DSA_DEBUG_BOUNDS
  uint32_t v = 0, zero = 0;
  if (hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_bounds_error), 4, 0, hipMemcpyDeviceToHost,
                               stream) != hipSuccess ||
      hipMemcpyToSymbolAsync(HIP_SYMBOL(g_bounds_error), &zero, 4, 0, hipMemcpyHostToDevice,
                             stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return 0x80000000u;
  return v;
#else
  (void)stream;
  return 0;
#endif
}
}  // namespace

// A block-table entry, checked in debug builds.
__device__ __forceinline__ int32_t checked_block(int32_t blk, int num_blocks) {
  if (kCheckBounds && (uint32_t)blk >= (uint32_t)num_blocks) {
    raise_error(kErrBlock);
    return 0;
  }
  return blk;
}

// Physical pool row of logical position `pos` of the sequence whose block
// table row is `bt_row`.
__device__ __forceinline__ int64_t paged_row(const int32_t* __restrict__ bt_row, int bs, int pos,
                                             int num_blocks) {
  return (int64_t)checked_block(bt_row[pos / bs], num_blocks) * bs + pos % bs;
}

// The gfx950 row swaps: after permlane16_swap(x, x) the first register holds
// rows (x0, x0, x2, x2) and the second (x1, x1, x3, x3) (a row is 16 lanes);
// after permlane32_swap(x, x) they hold halves (x_lo, x_lo) and (x_hi, x_hi).
// So op(first, second) is op(x, x of lane l ^ 16), resp. l ^ 32, in every
// lane, with no LDS round trip.
__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// max(x, 0) as one integer max on the bit pattern (negative floats have
// negative patterns), without the NaN canonicalisation fmaxf brings along.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Order-preserving map of fp32 onto uint32: larger float -> larger key.
// -0.0 is folded onto +0.0 so the two compare equal.
// Wave-wide scans and reductions on the DPP row shifts and row broadcasts:
// VALU operations, where a shuffle is an LDS round trip.  A lane whose DPP
// source does not exist (or whose row is masked off) reads `old`, the
// operation's identity.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes: within each row of 16 by shifts
// of 1, 2, 4, 8, then row 0's total into row 1 and row 2's into row 3, then
// lane 31's running total into rows 2 and 3.
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
  v += dpp<kRowShr1>(0u, v);
  v += dpp<kRowShr2>(0u, v);
  v += dpp<kRowShr4>(0u, v);
  v += dpp<kRowShr8>(0u, v);
  v += dpp<kRowBcast15, 0xa>(0u, v);
  v += dpp<kRowBcast31, 0xc>(0u, v);
  return v;
}
// Sum, AND and OR over the wave (the same steps; lane 63 holds the result).
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_incl_add(v), kWave - 1);
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  v &= dpp<kRowShr1>(~0u, v);
  v &= dpp<kRowShr2>(~0u, v);
  v &= dpp<kRowShr4>(~0u, v);
  v &= dpp<kRowShr8>(~0u, v);
  v &= dpp<kRowBcast15, 0xa>(~0u, v);
  v &= dpp<kRowBcast31, 0xc>(~0u, v);
  return __builtin_amdgcn_readlane(v, kWave - 1);
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  v |= dpp<kRowShr1>(0u, v);
  v |= dpp<kRowShr2>(0u, v);
  v |= dpp<kRowShr4>(0u, v);
  v |= dpp<kRowShr8>(0u, v);
  v |= dpp<kRowBcast15, 0xa>(0u, v);
  v |= dpp<kRowBcast31, 0xc>(0u, v);
  return __builtin_amdgcn_readlane(v, kWave - 1);
}

__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace dsa
