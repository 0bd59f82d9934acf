// MoE expert product with MXFP4 weights converted to FP8 E4M3 just before
// use (web page "Day-0 Adaptation of Trillion-Parameter MoE Models on
// Domestic GPUs", section 4; web page "Technical Path for Day-0 Adaptation
// of Trillion-Parameter Models on Domestic GPUs", section 3.2).
//
// gfx950 design.  The product runs on the scaled FP8/FP6/FP4 matrix cores
// (v_mfma_scale_f32_16x16x128_f8f6f4 with both operands E4M3 and unit
// scales): 16 token rows x 16 weight rows x 128 k a step.  Each lane feeds
// one weight row and 32 consecutive k -- exactly one MX block, so one scale
// byte a lane and step -- and the tokens' operand uses the same k order, so
// the sum runs over matching k whatever order the unit walks them in.
// The conversion of a lane's 32 FP4 codes to E4M3 bytes costs a few byte
// permutes: a 256-entry LDS table gives, for each scale code, the E4M3
// bytes of the eight FP4 magnitudes (two dwords) and the sign mask, so the
// magnitudes go through two v_perm_b32 lookups and the signs are OR-ed in.
// Decode-sized expert batches (a few tokens an expert) are bound by
// reading the weights from HBM: each wave streams its weight rows once, 64
// bytes of codes a lane ahead of use, and reads the (few) token rows
// through L2.
#include "common.h"
#include "host_util.h"

#include "../../include/dsa_moe.h"

namespace dsa {
namespace {

typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr int kMoeThreads = 256;  // four waves
constexpr int kMoeWaves = kMoeThreads / kWave;

// E4M3 byte of (FP4 magnitude code c in 0..7) x 2^(sc - 127), rounded to
// nearest even and saturated to 448; NaN scale -> 0x7f.  FP4 magnitude c:
// 0 -> 0, 1 -> 0.5, else (1 + (c & 1) / 2) * 2^((c >> 1) - 1).
__device__ uint32_t e4m3_of_scaled_fp4(int c, int sc) {
  if (sc == 255) return 0x7f;
  if (c == 0) return 0;
  const int ue = c == 1 ? -1 : (c >> 1) - 1;  // unbiased exponent of the element
  const int mh = c == 1 ? 0 : (c & 1);        // its mantissa half bit
  const int be = ue + sc - 120;               // E4M3 biased exponent (bias 7)
  if (be >= 16) return 0x7e;                  // beyond 2^9 > 448: saturate
  if (be >= 1) return (uint32_t)(be << 3 | mh << 2);
  // Subnormal: the value in units of 2^-9 is (2 + mh) * 2^(be + 1), an
  // integer for be >= -1, else rounded to nearest even.
  const int e2 = be + 1, v = 2 + mh;
  if (e2 >= 0) return (uint32_t)(v << e2);
  const int sh = -e2;
  if (sh >= 3) return 0;                      // at most 3/8 of the smallest step
  int q = v >> sh;
  const int r = v & ((1 << sh) - 1), half = 1 << (sh - 1);
  if (r > half || (r == half && (q & 1))) ++q;
  return (uint32_t)q;
}

// The conversion table of one scale code: E4M3 bytes of magnitudes 0..3
// and 4..7, and the mask that keeps the elements' sign bits (0 for the NaN
// scale, whose result is always 0x7f).
struct ScaleEntry {
  uint32_t lo, hi, sign, pad;
};

__device__ __forceinline__ void fill_scale_table(ScaleEntry* tab) {
  for (int sc = threadIdx.x; sc < 256; sc += blockDim.x) {
    uint32_t lo = 0, hi = 0;
    for (int c = 0; c < 4; ++c) {
      lo |= e4m3_of_scaled_fp4(c, sc) << (8 * c);
      hi |= e4m3_of_scaled_fp4(c + 4, sc) << (8 * c);
    }
    tab[sc] = ScaleEntry{lo, hi, sc == 255 ? 0u : 0x80808080u, 0u};
  }
}

// 8 FP4 codes (one dword, element 2i in the low nibble of byte i) -> 8 E4M3
// bytes in element order (two dwords).
__device__ __forceinline__ void convert8(uint32_t w, const ScaleEntry& t, uint32_t& o0,
                                         uint32_t& o1) {
  const uint32_t even = __builtin_amdgcn_perm(t.hi, t.lo, w & 0x07070707u) | ((w << 4) & t.sign);
  const uint32_t odd = __builtin_amdgcn_perm(t.hi, t.lo, (w >> 4) & 0x07070707u) | (w & t.sign);
  o0 = __builtin_amdgcn_perm(odd, even, 0x05010400u);
  o1 = __builtin_amdgcn_perm(odd, even, 0x07030602u);
}

// 32 FP4 codes (16 bytes) of one MX block -> the 32 E4M3 bytes of an MFMA
// operand.
__device__ __forceinline__ i32x8 convert_block(u32x4 raw, const ScaleEntry& t) {
  i32x8 b;
  uint32_t o0, o1;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    convert8(raw[d], t, o0, o1);
    b[2 * d] = (int32_t)o0;
    b[2 * d + 1] = (int32_t)o1;
  }
  return b;
}

__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 c) {
  // Format 0 (E4M3) for both operands, E8M0 scales 127 (= 1).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 join(u32x4 a, u32x4 b) {
  return (i32x8){(int32_t)a[0], (int32_t)a[1], (int32_t)a[2], (int32_t)a[3],
                 (int32_t)b[0], (int32_t)b[1], (int32_t)b[2], (int32_t)b[3]};
}

// The row range of listed expert i, checked in debug builds.
__device__ __forceinline__ void expert_rows(const int32_t* __restrict__ row_offsets, int i, int M,
                                            int& row0, int& count) {
  row0 = row_offsets[i];
  const int row1 = row_offsets[i + 1];
  count = row1 - row0;
  if (kCheckBounds && (row0 < 0 || row1 > M || count < 0)) {
    if (threadIdx.x == 0) raise_error(kErrLength);
    count = 0;
  }
}

// One super-step of a lane's weight bytes: kRaw 16-byte pieces of each of
// its NT rows, and (MXFP4) the S scale bytes of each.
template <int NT, int kRaw, int S, bool kFp4>
__device__ __forceinline__ void load_weights(u32x4 (&raw)[NT][kRaw], uint32_t (&sc)[NT],
                                             const uint8_t* const (&wrow)[NT],
                                             const uint8_t* const (&srow)[NT],
                                             const bool (&tile_ok)[NT], int step) {
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (!tile_ok[j]) continue;
    const u32x4* p = (const u32x4*)(wrow[j] + (int64_t)step * 64 * kRaw);  // 4 groups x 16 kRaw
#pragma unroll
    for (int q = 0; q < kRaw; ++q) raw[j][q] = __builtin_nontemporal_load(p + q);
    if constexpr (kFp4) {
      const uint8_t* sp = srow[j] + (int64_t)step * 4 * S;
      if constexpr (S == 4) sc[j] = *(const uint32_t*)sp;
      else if constexpr (S == 2) sc[j] = *(const uint16_t*)sp;
      else sc[j] = *sp;
    }
  }
}

// The product kernel.  Workgroup (b, i, z): listed expert i, weight rows
// n0 = 64 NT b .. +64 NT (wave w takes NT tiles of 16 rows), token rows in
// passes of 16 RT starting at pass z, stepping gridDim.z.  kFp4: weights
// are MXFP4 codes + scales of expert expert_ids[i]; else E4M3 bytes w8[i].
// The k loop runs in super-steps of 128 S: lane (row l & 15, group g = l >>
// 4) holds k = kk + 32 S g + 32 s .. +31 in step s, for the weights (16 S
// code bytes, S scale bytes, loaded one super-step ahead) and the tokens
// alike.
template <int NT, int RT, int S, bool kFp4>
__global__ __launch_bounds__(kMoeThreads) void moe_gemm_kernel(
    const uint8_t* __restrict__ wsrc, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ expert_ids, int num_experts, int N, int K,
    const uint8_t* __restrict__ x, const int32_t* __restrict__ row_offsets, int M,
    float* __restrict__ y) {
  __shared__ ScaleEntry tab[kFp4 ? 256 : 1];
  if constexpr (kFp4) {
    fill_scale_table(tab);
    __syncthreads();
  }
  const int i = blockIdx.y;
  int row0, count;
  expert_rows(row_offsets, i, M, row0, count);
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int r16 = lane & 15, g = lane >> 4;
  const int nbase = (blockIdx.x * kMoeWaves + w) * 16 * NT;
  if (nbase >= N) return;

  // This lane's weight rows (one per tile) and their byte sources.
  const uint8_t* wrow[NT];
  const uint8_t* srow[NT];
  bool tile_ok[NT];
  int64_t ex = i;
  if constexpr (kFp4) {
    ex = expert_ids[i];
    if (kCheckBounds && (ex < 0 || ex >= num_experts)) {
      if (lane == 0) raise_error(kErrIndex);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = nbase + 16 * j + r16;
    tile_ok[j] = nbase + 16 * j < N;
    const int64_t rowid = ex * N + (tile_ok[j] ? n : 0);
    if constexpr (kFp4) {
      wrow[j] = wsrc + rowid * (K / 2) + 16 * S * g;
      srow[j] = scales + rowid * (K / 32) + S * g;
    } else {
      wrow[j] = wsrc + rowid * K + 32 * S * g;
      srow[j] = nullptr;
    }
  }
  constexpr int kRaw = kFp4 ? S : 2 * S;  // 16-byte pieces a lane and super-step
  const int steps = K / (128 * S);

  for (int pass = blockIdx.z; pass * 16 * RT < count; pass += gridDim.z) {
    const int pbase = pass * 16 * RT;
    f32x4 acc[RT][NT];
    const uint8_t* xrow[RT];
    bool xok[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int r = pbase + 16 * t + r16;
      xok[t] = r < count;
      xrow[t] = x + (int64_t)(row0 + (xok[t] ? r : 0)) * K + 32 * S * g;
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[t][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    u32x4 raw[NT][kRaw];
    uint32_t sc[NT];
    load_weights<NT, kRaw, S, kFp4>(raw, sc, wrow, srow, tile_ok, 0);
    for (int st = 0; st < steps; ++st) {
      u32x4 cur[NT][kRaw];
      uint32_t csc[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        csc[j] = sc[j];
#pragma unroll
        for (int q = 0; q < kRaw; ++q) cur[j][q] = raw[j][q];
      }
      if (st + 1 < steps) load_weights<NT, kRaw, S, kFp4>(raw, sc, wrow, srow, tile_ok, st + 1);
#pragma unroll
      for (int s = 0; s < S; ++s) {
        i32x8 a[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          if (xok[t]) {
            const u32x4* xp = (const u32x4*)(xrow[t] + (int64_t)st * 128 * S + 32 * s);
            a[t] = join(xp[0], xp[1]);
          } else {
            a[t] = (i32x8){0, 0, 0, 0, 0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          i32x8 b;
          if constexpr (kFp4) {
            b = convert_block(cur[j][s], tab[(csc[j] >> (8 * s)) & 255]);
          } else {
            b = join(cur[j][2 * s], cur[j][2 * s + 1]);
          }
#pragma unroll
          for (int t = 0; t < RT; ++t) acc[t][j] = mfma_fp8(a[t], b, acc[t][j]);
        }
      }
    }
    // Result lane l holds weight row (l & 15) of each tile and token rows
    // 4 g .. 4 g + 3 of each 16-row tile.
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        if (!tile_ok[j]) continue;
        const int n = nbase + 16 * j + r16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = pbase + 16 * t + 4 * g + q;
          if (r < count) y[(int64_t)(row0 + r) * N + n] = acc[t][j][q];
        }
      }
  }
}

// Conversion to a workspace: thread-block rows of 128 elements (four MX
// blocks: 64 code bytes, four scale bytes) -> 128 E4M3 bytes.
__global__ __launch_bounds__(kMoeThreads) void mxfp4_to_fp8_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ expert_ids, int num_experts, int N, int K, int n_act,
    uint8_t* __restrict__ w8) {
  __shared__ ScaleEntry tab[256];
  fill_scale_table(tab);
  __syncthreads();
  const int per_row = K / 128;
  const int64_t per_expert = (int64_t)N * per_row;
  const int64_t total = per_expert * n_act;
  for (int64_t u = (int64_t)blockIdx.x * kMoeThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kMoeThreads) {
    const int i = (int)(u / per_expert);
    const int64_t rem = u - (int64_t)i * per_expert;
    const int64_t n = rem / per_row;
    const int q = (int)(rem - n * per_row);
    int64_t ex = expert_ids[i];
    if (kCheckBounds && (ex < 0 || ex >= num_experts)) {
      raise_error(kErrIndex);
      continue;
    }
    const int64_t rowid = ex * N + n;
    const u32x4* src = (const u32x4*)(codes + rowid * (K / 2) + 64 * q);
    const uint32_t sc = *(const uint32_t*)(scales + rowid * (K / 32) + 4 * q);
    u32x4* dst = (u32x4*)(w8 + ((int64_t)i * N + n) * K + 128 * q);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const u32x4 raw = __builtin_nontemporal_load(src + b);
      const ScaleEntry& t = tab[(sc >> (8 * b)) & 255];
      const i32x8 o = convert_block(raw, t);
      dst[2 * b] = (u32x4){(uint32_t)o[0], (uint32_t)o[1], (uint32_t)o[2], (uint32_t)o[3]};
      dst[2 * b + 1] = (u32x4){(uint32_t)o[4], (uint32_t)o[5], (uint32_t)o[6], (uint32_t)o[7]};
    }
  }
}

template <bool kFp4, int NT, int RT, int S>
void launch_moe(const uint8_t* wsrc, const uint8_t* scales, const int32_t* expert_ids,
                int num_experts, int N, int K, const uint8_t* x, const int32_t* row_offsets,
                int n_act, int M, int max_rows, float* y, hipStream_t stream) {
  const int nblocks = (N + 16 * NT * kMoeWaves - 1) / (16 * NT * kMoeWaves);
  const int passes = max_rows < 1 ? 1 : (max_rows + 16 * RT - 1) / (16 * RT);
  const dim3 grid((unsigned)nblocks, (unsigned)n_act, (unsigned)(passes > 65535 ? 65535 : passes));
  hipLaunchKernelGGL((moe_gemm_kernel<NT, RT, S, kFp4>), grid, dim3(kMoeThreads), 0, stream,
                     wsrc, scales, expert_ids, num_experts, N, K, x, row_offsets, M, y);
}

// Row-tile count and super-step by size: one 16-row tile for decode-sized
// batches (the weights are read once whatever the row count), up to four
// tiles (64 rows) a pass for larger ones.
template <bool kFp4>
void dispatch_moe(const uint8_t* wsrc, const uint8_t* scales, const int32_t* expert_ids,
                  int num_experts, int N, int K, const uint8_t* x, const int32_t* row_offsets,
                  int n_act, int M, int max_rows, float* y, hipStream_t stream) {
#define DSA_MOE_LAUNCH(NT, RT, S)                                                              \
  launch_moe<kFp4, NT, RT, S>(wsrc, scales, expert_ids, num_experts, N, K, x, row_offsets, \
                              n_act, M, max_rows, y, stream)
  const bool s4 = K % 512 == 0;
  if (max_rows <= 16) {
    if (s4) DSA_MOE_LAUNCH(2, 1, 4); else DSA_MOE_LAUNCH(2, 1, 1);
  } else if (max_rows <= 32) {
    if (s4) DSA_MOE_LAUNCH(2, 2, 4); else DSA_MOE_LAUNCH(2, 2, 1);
  } else {
    if (s4) DSA_MOE_LAUNCH(2, 4, 4); else DSA_MOE_LAUNCH(2, 4, 1);
  }
#undef DSA_MOE_LAUNCH
}

dsa_status_t check_moe_common(int N, int K, const uint8_t* x, const int32_t* row_offsets,
                              int n_act, int M, float* y) {
  if (!x || !row_offsets || !y) return DSA_ERR_NULL;
  if (N < 1 || K < 1 || M < 0 || n_act < 1 || n_act > 65535) return DSA_ERR_SHAPE;
  if (K % 128 || N % 16) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(y)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status_t check_weights(const dsa_mxfp4_weights_t* w, const int32_t* expert_ids) {
  if (!w || !w->codes || !w->scales || !expert_ids) return DSA_ERR_NULL;
  if (w->num_experts < 1 || w->N < 1 || w->K < 1) return DSA_ERR_SHAPE;
  if (w->K % 128 || w->N % 16) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(w->codes) || ((uintptr_t)w->scales & 3)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status_t convert_launch(const dsa_mxfp4_weights_t* w, const int32_t* expert_ids, int n_act,
                            uint8_t* w8, hipStream_t stream) {
  const int64_t units = (int64_t)n_act * w->N * (w->K / 128);
  const int64_t blocks = (units + kMoeThreads - 1) / kMoeThreads;
  const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
  hipLaunchKernelGGL(mxfp4_to_fp8_kernel, dim3(grid), dim3(kMoeThreads), 0, stream, w->codes,
                     w->scales, expert_ids, w->num_experts, w->N, w->K, n_act, w8);
  return launch_status();
}

}  // namespace

uint32_t take_bounds_error_moe(hipStream_t stream) { return take_bounds_error(stream); }

}  // namespace dsa

extern "C" dsa_status_t dsa_moe_gemm_mxfp4(const dsa_mxfp4_weights_t* w, const uint8_t* x,
                                           const int32_t* expert_ids, const int32_t* row_offsets,
                                           int32_t n_act, int32_t M, int32_t max_rows, float* y,
                                           hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_weights(w, expert_ids);
  if (st != DSA_OK) return st;
  st = check_moe_common(w->N, w->K, x, row_offsets, n_act, M, y);
  if (st != DSA_OK) return st;
  st = check_device();
  if (st != DSA_OK) return st;
  dispatch_moe<true>(w->codes, w->scales, expert_ids, w->num_experts, w->N, w->K, x, row_offsets,
                     n_act, M, max_rows, y, stream);
  return launch_status();
}

extern "C" dsa_status_t dsa_mxfp4_to_fp8(const dsa_mxfp4_weights_t* w, const int32_t* expert_ids,
                                         int32_t n_act, uint8_t* w8, hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_weights(w, expert_ids);
  if (st != DSA_OK) return st;
  if (!w8) return DSA_ERR_NULL;
  if (n_act < 1 || n_act > 65535) return DSA_ERR_SHAPE;
  if (!aligned16(w8)) return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  return convert_launch(w, expert_ids, n_act, w8, stream);
}

extern "C" dsa_status_t dsa_moe_gemm_fp8(const uint8_t* w8, int32_t N, int32_t K, const uint8_t* x,
                                         const int32_t* row_offsets, int32_t n_act, int32_t M,
                                         int32_t max_rows, float* y, hipStream_t stream) {
  using namespace dsa;
  if (!w8) return DSA_ERR_NULL;
  dsa_status_t st = check_moe_common(N, K, x, row_offsets, n_act, M, y);
  if (st != DSA_OK) return st;
  if (!aligned16(w8)) return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  dispatch_moe<false>(w8, nullptr, nullptr, n_act, N, K, x, row_offsets, n_act, M, max_rows, y,
                      stream);
  return launch_status();
}

extern "C" size_t dsa_moe_staged_ws(int32_t N, int32_t K, int32_t chunk_experts) {
  if (N < 1 || K < 1 || chunk_experts < 1) return 0;
  return 2 * (size_t)chunk_experts * (size_t)N * (size_t)K;
}

extern "C" dsa_status_t dsa_moe_gemm_staged(const dsa_mxfp4_weights_t* w, const uint8_t* x,
                                            const int32_t* expert_ids, const int32_t* row_offsets,
                                            int32_t n_act, int32_t M, int32_t max_rows, float* y,
                                            void* workspace, size_t workspace_bytes,
                                            hipStream_t stream, hipStream_t conv_stream,
                                            hipEvent_t* events) {
  using namespace dsa;
  dsa_status_t st = check_weights(w, expert_ids);
  if (st != DSA_OK) return st;
  st = check_moe_common(w->N, w->K, x, row_offsets, n_act, M, y);
  if (st != DSA_OK) return st;
  if (!workspace || !events || !events[0] || !events[1] || !events[2] || !events[3])
    return DSA_ERR_NULL;
  if (conv_stream == stream) return DSA_ERR_SHAPE;
  if (!aligned16(workspace)) return DSA_ERR_UNSUPPORTED;
  const size_t expert_bytes = (size_t)w->N * (size_t)w->K;
  const int64_t chunk64 = (int64_t)(workspace_bytes / (2 * expert_bytes));
  if (chunk64 < 1) return DSA_ERR_WORKSPACE;
  const int chunk = (int)(chunk64 < n_act ? chunk64 : n_act);
  st = check_device();
  if (st != DSA_OK) return st;
  uint8_t* half[2] = {(uint8_t*)workspace, (uint8_t*)workspace + (size_t)chunk * expert_bytes};
  hipEvent_t* ready = events;      // half h holds converted weights
  hipEvent_t* free_ = events + 2;  // the last product reading half h has finished
  for (int c0 = 0, c = 0; c0 < n_act; c0 += chunk, ++c) {
    const int h = c & 1, n = n_act - c0 < chunk ? n_act - c0 : chunk;
    if (hipStreamWaitEvent(conv_stream, free_[h], 0) != hipSuccess) return DSA_ERR_HIP;
    st = convert_launch(w, expert_ids + c0, n, half[h], conv_stream);
    if (st != DSA_OK) return st;
    if (hipEventRecord(ready[h], conv_stream) != hipSuccess ||
        hipStreamWaitEvent(stream, ready[h], 0) != hipSuccess)
      return DSA_ERR_HIP;
    dispatch_moe<false>(half[h], nullptr, nullptr, n, w->N, w->K, x, row_offsets + c0, n, M,
                        max_rows, y, stream);
    st = launch_status();
    if (st != DSA_OK) return st;
    if (hipEventRecord(free_[h], stream) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}
