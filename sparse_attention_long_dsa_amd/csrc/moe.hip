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
// reading the weights from HBM: each wave streams its weight rows once, one
// super-step ahead of use, and reads the (few) token rows through L2.
//
// Weight layouts.  Row-major MXFP4 ([E, N, K/2] codes) makes a wave's 16
// rows 16 separate 128-byte pieces per super-step, which streams at about
// half of HBM speed; the tiled layout (DSA_MXFP4_TILED, made once by
// dsa_mxfp4_pack, still 4.25 bits an element) stores each 16-row x 256-k
// unit as one 2 KB block in the order the lanes read it, so every wave load
// is one contiguous KB.  The staged pipeline's FP8 workspace uses the same
// unit order (4 KB a unit).  Lane (row r, group g) of a unit holds k =
// 64 g .. 64 g + 63 as two MX blocks (one per 128-k step), in both layouts
// and in both kernels, so every path sums the same products in the same
// order and gives the same bits.
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

constexpr int kUnitK = 256;  // k elements of one tiled unit

// Per-lane strides of the weight sources (bytes): a super-step advances by
// kStep, the 16-byte pieces of one super-step lie kPiece apart; scales
// advance by kScaleStep.
template <bool kFp4, bool kTiled, int S>
struct WeightStrides {
  static constexpr int kStep = kTiled ? (kFp4 ? 2048 : 4096) : (kFp4 ? 64 * S : 128 * S);
  static constexpr int kPiece = kTiled ? 1024 : 16;
  static constexpr int kScaleStep = kTiled ? 128 : 4 * S;
};

// Byte offsets of (row n, 32-k block kb) of one expert's codes / scales in
// a layout (the block's 16 code bytes are contiguous in both).
__device__ __forceinline__ int64_t code_offset(bool tiled, int64_t n, int64_t kb, int N, int K) {
  if (!tiled) return n * (K / 2) + 16 * kb;
  const int64_t unit = (n / 16) * (K / kUnitK) + kb / 8;
  const int lane = (int)((kb % 8) / 2) * 16 + (int)(n % 16);
  return unit * 2048 + (kb % 2) * 1024 + lane * 16;
}
__device__ __forceinline__ int64_t scale_offset(bool tiled, int64_t n, int64_t kb, int N, int K) {
  if (!tiled) return n * (K / 32) + kb;
  const int64_t unit = (n / 16) * (K / kUnitK) + kb / 8;
  const int lane = (int)((kb % 8) / 2) * 16 + (int)(n % 16);
  return unit * 128 + lane * 2 + kb % 2;
}

// One super-step of a lane's weight bytes: kRaw 16-byte pieces of each of
// its NT rows, and (MXFP4) the S scale bytes of each.  Loads are
// unconditional (rows past N read a clamped row), so the compiler's wait
// counts stay exact: waiting for an older super-step never waits for these.
template <int NT, int kRaw, int S, bool kFp4, bool kTiled>
__device__ __forceinline__ void load_weights(u32x4 (&raw)[NT][kRaw], uint32_t (&sc)[NT],
                                             const uint8_t* const (&wrow)[NT],
                                             const uint8_t* const (&srow)[NT], int step) {
  using St = WeightStrides<kFp4, kTiled, S>;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const uint8_t* p = wrow[j] + (int64_t)step * St::kStep;
#pragma unroll
    for (int q = 0; q < kRaw; ++q)
      raw[j][q] = __builtin_nontemporal_load((const u32x4*)(p + q * St::kPiece));
    if constexpr (kFp4) {
      const uint8_t* sp = srow[j] + (int64_t)step * St::kScaleStep;
      if constexpr (S == 4) sc[j] = *(const uint32_t*)sp;
      else if constexpr (S == 2) sc[j] = *(const uint16_t*)sp;
      else sc[j] = *sp;
    }
  }
}

// One super-step of a lane's token bytes: 32 S bytes of each of its RT rows
// (rows past the expert's count read a clamped row).
template <int RT, int S>
__device__ __forceinline__ void load_tokens(u32x4 (&xa)[RT][2 * S],
                                            const uint8_t* const (&xrow)[RT], int step) {
#pragma unroll
  for (int t = 0; t < RT; ++t) {
    const u32x4* p = (const u32x4*)(xrow[t] + (int64_t)step * 128 * S);
#pragma unroll
    for (int q = 0; q < 2 * S; ++q) xa[t][q] = p[q];
  }
}

// The products of one super-step.
template <int NT, int RT, int S, bool kFp4, int kRaw>
__device__ __forceinline__ void super_step(f32x4 (&acc)[RT][NT], const u32x4 (&w)[NT][kRaw],
                                           const uint32_t (&sc)[NT], const u32x4 (&xa)[RT][2 * S],
                                           const ScaleEntry* tab) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    // Lanes of rows past the expert's count hold a clamped row: row i of the
    // product depends on row i of the tokens only, and those rows are never
    // stored.
    i32x8 a[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) a[t] = join(xa[t][2 * s], xa[t][2 * s + 1]);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      i32x8 b;
      if constexpr (kFp4) {
        b = convert_block(w[j][s], tab[(sc[j] >> (8 * s)) & 255]);
      } else {
        b = join(w[j][2 * s], w[j][2 * s + 1]);
      }
#pragma unroll
      for (int t = 0; t < RT; ++t) acc[t][j] = mfma_fp8(a[t], b, acc[t][j]);
    }
  }
}

// The product kernel.  Workgroup (b, i, z): listed expert i, weight rows
// n0 = 64 NT b .. +64 NT (wave w takes NT tiles of 16 rows), token rows in
// passes of 16 RT starting at pass z, stepping gridDim.z.  kFp4: weights
// are MXFP4 codes + scales of expert expert_ids[i]; else E4M3 bytes of
// listed expert i.  kTiled: the weights are in unit order (then S = 2).
// The k loop runs in super-steps of 128 S: lane (row l & 15, group g = l >>
// 4) holds k = kk + 32 S g + 32 s .. +31 in step s, for the weights and the
// tokens alike.  Order of loads in a super-step: its token bytes, then the
// next super-step's weights, then the products -- so the products wait for
// nothing issued after the loads they use, and each wave keeps one
// super-step of weights in flight.
template <int NT, int RT, int S, bool kFp4, bool kTiled>
__global__ __launch_bounds__(kMoeThreads) void moe_gemm_kernel(
    const uint8_t* __restrict__ wsrc, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ expert_ids, int num_experts, int N, int K,
    const uint8_t* __restrict__ x, const int32_t* __restrict__ row_offsets, int M,
    float* __restrict__ y) {
  static_assert(!kTiled || S == 2, "a tiled unit is two 128-k steps");
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

  // This lane's weight sources (one per tile).
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
  const int64_t ebytes = (int64_t)N * K / (kFp4 ? 2 : 1);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tile_ok[j] = nbase + 16 * j < N;
    const int n = (tile_ok[j] ? nbase + 16 * j : nbase) + r16;
    if constexpr (kTiled) {
      const int64_t unit0 = (int64_t)(n / 16) * (K / kUnitK);
      wrow[j] = wsrc + ex * ebytes + unit0 * (kFp4 ? 2048 : 4096) + lane * 16;
      srow[j] = kFp4 ? scales + ex * ((int64_t)N * K / 32) + unit0 * 128 + lane * 2 : nullptr;
    } else if constexpr (kFp4) {
      wrow[j] = wsrc + (ex * N + n) * (K / 2) + 16 * S * g;
      srow[j] = scales + (ex * N + n) * (K / 32) + S * g;
    } else {
      wrow[j] = wsrc + (ex * N + n) * K + 32 * S * g;
      srow[j] = nullptr;
    }
  }
  constexpr int kRaw = kFp4 ? S : 2 * S;  // 16-byte pieces a lane and super-step
  const int steps = K / (128 * S);

  for (int pass = blockIdx.z; pass * 16 * RT < count; pass += gridDim.z) {
    const int pbase = pass * 16 * RT;
    f32x4 acc[RT][NT];
    const uint8_t* xrow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int r = pbase + 16 * t + r16;
      xrow[t] = x + (int64_t)(row0 + (r < count ? r : 0)) * K + 32 * S * g;
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[t][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    // Two weight buffers used in turn (a register copy of a buffer in
    // flight would wait for its loads).
    u32x4 wa[NT][kRaw], wb[NT][kRaw], xa[RT][2 * S];
    uint32_t sa[NT], sb[NT];
    load_weights<NT, kRaw, S, kFp4, kTiled>(wa, sa, wrow, srow, 0);
    int st = 0;
    for (; st + 2 < steps; st += 2) {
      load_tokens<RT, S>(xa, xrow, st);
      load_weights<NT, kRaw, S, kFp4, kTiled>(wb, sb, wrow, srow, st + 1);
      super_step<NT, RT, S, kFp4, kRaw>(acc, wa, sa, xa, tab);
      load_tokens<RT, S>(xa, xrow, st + 1);
      load_weights<NT, kRaw, S, kFp4, kTiled>(wa, sa, wrow, srow, st + 2);
      super_step<NT, RT, S, kFp4, kRaw>(acc, wb, sb, xa, tab);
    }
    load_tokens<RT, S>(xa, xrow, st);
    if (st + 1 < steps) {
      load_weights<NT, kRaw, S, kFp4, kTiled>(wb, sb, wrow, srow, st + 1);
      super_step<NT, RT, S, kFp4, kRaw>(acc, wa, sa, xa, tab);
      load_tokens<RT, S>(xa, xrow, st + 1);
      super_step<NT, RT, S, kFp4, kRaw>(acc, wb, sb, xa, tab);
    } else {
      super_step<NT, RT, S, kFp4, kRaw>(acc, wa, sa, xa, tab);
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

// The product kernel for larger expert batches (prefill: a few hundred
// rows an expert), bound by the matrix cores.  Workgroup (b, i, z) of eight
// waves (two per SIMD, so one wave's conversion overlaps the other's
// products): listed expert i, weight rows 256 b .. +256, and the token rows
// of pass z (the expert's rows cut into ceil(count / 256) equal passes of
// whole 16-row tiles, at most 16 tiles).  Wave w takes weight rows
// 64 (w % 4) .. +64 (four 16-row tiles, converted in its registers from the
// tiled layout) and token tiles w / 4, w / 4 + 2, ... (every other tile, so
// both waves on a SIMD get half of a short pass).  Token tiles go through
// LDS, double buffered, in MFMA operand order: each 1 KB block (tile t,
// step s, half h) is what one wave reads with one 16-byte load a lane.  One
// barrier a 256-k super-step.  Weights, scales and token rows are read
// through buffer resources with per-tile offsets in scalar registers, so no
// per-tile address occupies vector registers.
constexpr int kBigThreads = 512;
constexpr int kBigRows = 256;   // token rows a pass
constexpr int kBigTiles = kBigRows / 16;
constexpr int kBigNT = 4;       // 16-row weight tiles a wave
constexpr int kBigWaveTiles = kBigTiles / 2;  // token tiles a wave
constexpr int kBigN = 4 * kBigNT * 16;        // weight rows a workgroup
constexpr int kBigStage = kBigTiles * 16 * 16 / kBigThreads;  // staged pieces a thread
constexpr uint32_t kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Token staging of one super-step, half H (0 or 1): thread (tile group tg =
// tid / 256, row r = (tid / 16) % 16, chunk c = tid % 16) moves row r of
// tiles tg + 2 v, v = H WT / 2 .. (H + 1) WT / 2 - 1, bytes 16 c .. +15 of
// the super-step's 256 (16 threads read a row's 256 bytes: coalesced).
// Chunk c = 4 g + p is part p (step p / 2, half p % 2) of operand lane
// L = 16 g + r.  Inside each 1 KB LDS block (tile, part p) lane L's 16 bytes
// sit at slot L ^ ((4 p + g) & 15): the 16 lanes of a store group (one row,
// all (g, p)) and of a load group (one g, all rows) then fall on 16
// different bank groups.  The tile offset is uniform (a scalar operand);
// rows past the expert's count read as zeros (buffer bounds).
__device__ __forceinline__ int big_slot(int p, int L) { return L ^ ((4 * p + (L >> 4)) & 15); }

template <int WT, int H>
__device__ __forceinline__ void big_stage_load(u32x4 (&xr)[WT / 2], __amdgpu_buffer_rsrc_t xrsrc,
                                               int voff, int tb, int K, int st) {
#pragma unroll
  for (int v = 0; v < WT / 2; ++v) {
    const int t = tb + 2 * (H * (WT / 2) + v);
    xr[v] = buf_load16(xrsrc, voff, 16 * t * K + st * kUnitK);
  }
}
template <int WT, int H>
__device__ __forceinline__ void big_stage_store(u32x4* xs, const u32x4 (&xr)[WT / 2], int xoff,
                                                int tb) {
#pragma unroll
  for (int v = 0; v < WT / 2; ++v) {
    const int t = tb + 2 * (H * (WT / 2) + v);
    xs[t * 256 + xoff] = xr[v];
  }
}

// One step's weight pieces of the wave's four tiles (16 bytes a lane each)
// and a super-step's scale pairs.
__device__ __forceinline__ void big_load_w(u32x4 (&w)[kBigNT], __amdgpu_buffer_rsrc_t wr,
                                           int lane, int unit0, int units, int st, int s) {
#pragma unroll
  for (int j = 0; j < kBigNT; ++j)
    w[j] = buf_load16(wr, lane * 16, ((unit0 + j * units) + st) * 2048 + s * 1024);
}
__device__ __forceinline__ void big_load_s(uint32_t (&sc)[kBigNT], __amdgpu_buffer_rsrc_t sr,
                                           int lane, int unit0, int units, int st) {
#pragma unroll
  for (int j = 0; j < kBigNT; ++j)
    sc[j] = __builtin_amdgcn_raw_buffer_load_b16(sr, lane * 2, ((unit0 + j * units) + st) * 128, 0);
}

// Step s of a super-step: the wave's four weight tiles of step (st, s) are
// converted and their registers refilled at once with step (st + 1, s) --
// two steps ahead of use (nothing on the last super-step) -- then the
// converted tiles times the wave's WT token tiles (LDS reads one tile ahead
// of the products).
template <int WT, int s, bool kMore>
__device__ __forceinline__ void big_products(f32x4 (&acc)[WT][kBigNT], u32x4 (&w)[kBigNT],
                                             const uint32_t (&sc)[kBigNT],
                                             __amdgpu_buffer_rsrc_t wr, int unit0, int units,
                                             int st, const u32x4* xs, int tg, int lane,
                                             const ScaleEntry* tab) {
  i32x8 b[kBigNT];
#pragma unroll
  for (int j = 0; j < kBigNT; ++j) b[j] = convert_block(w[j], tab[(sc[j] >> (8 * s)) & 255]);
  if (kMore) big_load_w(w, wr, lane, unit0, units, st + 1, s);
  // tile tg, step s: parts 2 s and 2 s + 1 at this lane's slots
  const u32x4* src0 = xs + (tg * 4 + s * 2) * 64 + big_slot(2 * s, lane);
  const u32x4* src1 = xs + (tg * 4 + s * 2 + 1) * 64 + big_slot(2 * s + 1, lane);
  i32x8 a = join(src0[0], src1[0]);
#pragma unroll
  for (int t = 0; t < WT; ++t) {
    i32x8 an = a;
    if (t + 1 < WT) an = join(src0[(t + 1) * 512], src1[(t + 1) * 512]);  // tile tg + 2 (t + 1)
#pragma unroll
    for (int j = 0; j < kBigNT; ++j) acc[t][j] = mfma_fp8(a, b[j], acc[t][j]);
    a = an;
  }
}

// One super-step st: the first half of token tiles st + 1 is loaded during
// step 0's products and the second half (with the scales of st + 1) during
// step 1's; the staged halves go to the other LDS buffer; a barrier ends
// it.  kLast: the final super-step (no loads of st + 1).
template <int WT, bool kLast>
__device__ __forceinline__ void big_super_step(
    f32x4 (&acc)[WT][kBigNT], u32x4 (&w0)[kBigNT], u32x4 (&w1)[kBigNT], uint32_t (&sc)[kBigNT],
    uint32_t (&scn)[kBigNT], u32x4 (&xr)[WT / 2], __amdgpu_buffer_rsrc_t wr,
    __amdgpu_buffer_rsrc_t sr, __amdgpu_buffer_rsrc_t xrsrc, int unit0, int units, int xvoff,
    int xoff, int tg, int K, int st, int lane, const u32x4* xs_cur, u32x4* xs_next,
    const ScaleEntry* tab) {
  if (!kLast) big_stage_load<WT, 0>(xr, xrsrc, xvoff, tg, K, st + 1);
  big_products<WT, 0, !kLast>(acc, w0, sc, wr, unit0, units, st, xs_cur, tg, lane, tab);
  if (!kLast) {
    big_load_s(scn, sr, lane, unit0, units, st + 1);
    big_stage_store<WT, 0>(xs_next, xr, xoff, tg);
    big_stage_load<WT, 1>(xr, xrsrc, xvoff, tg, K, st + 1);
  }
  big_products<WT, 1, !kLast>(acc, w1, sc, wr, unit0, units, st, xs_cur, tg, lane, tab);
  if (!kLast) {
    big_stage_store<WT, 1>(xs_next, xr, xoff, tg);
    __syncthreads();
  }
}

// One pass of up to 2 WT token tiles (rows pbase .. pbase + prow - 1 of the
// expert), every product on all 2 WT tiles (rows past prow are zeros or the
// next pass's rows, never stored).
template <int WT>
__device__ __forceinline__ void big_pass(u32x4 (*xs)[kBigTiles * 4 * 64],
                                         __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                         __amdgpu_buffer_rsrc_t xrsrc, int unit0, int units,
                                         int K, int N, int pbase, int prow, int row0, int tid,
                                         int nbase, const bool (&tile_ok)[kBigNT],
                                         const ScaleEntry* tab, float* __restrict__ y) {
  // the wave index through readfirstlane: wave-uniform values derived from
  // it stay in scalar registers (buffer offsets need them there)
  const int lane = tid & (kWave - 1), w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r16 = lane & 15, g = lane >> 4;
  const int tg = w >> 2;  // token tiles tg, tg + 2, ... (products and staging)
  const int srow = (tid >> 4) & 15, chunk = tid & 15;
  const int xoff = (chunk & 3) * 64 + big_slot(chunk & 3, 16 * (chunk >> 2) + srow);
  const int xvoff = (pbase + srow) * K + 16 * chunk;
  const int steps = units;
  f32x4 acc[WT][kBigNT];
#pragma unroll
  for (int t = 0; t < WT; ++t)
#pragma unroll
    for (int j = 0; j < kBigNT; ++j) acc[t][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

  u32x4 w0[kBigNT], w1[kBigNT], xr[WT / 2];
  uint32_t sa[kBigNT], sb[kBigNT];
  big_load_w(w0, wr, lane, unit0, units, 0, 0);
  big_load_w(w1, wr, lane, unit0, units, 0, 1);
  big_stage_load<WT, 0>(xr, xrsrc, xvoff, tg, K, 0);
  big_stage_store<WT, 0>(xs[0], xr, xoff, tg);
  big_stage_load<WT, 1>(xr, xrsrc, xvoff, tg, K, 0);
  big_load_s(sa, sr, lane, unit0, units, 0);
  big_stage_store<WT, 1>(xs[0], xr, xoff, tg);
  __syncthreads();  // the scale table and the first token tiles
  int st = 0;
  for (; st + 2 < steps; st += 2) {
    big_super_step<WT, false>(acc, w0, w1, sa, sb, xr, wr, sr, xrsrc, unit0, units, xvoff, xoff, tg, K,
                              st, lane, xs[0], xs[1], tab);
    big_super_step<WT, false>(acc, w0, w1, sb, sa, xr, wr, sr, xrsrc, unit0, units, xvoff, xoff, tg, K,
                              st + 1, lane, xs[1], xs[0], tab);
  }
  if (st + 1 < steps) {
    big_super_step<WT, false>(acc, w0, w1, sa, sb, xr, wr, sr, xrsrc, unit0, units, xvoff, xoff, tg, K,
                              st, lane, xs[0], xs[1], tab);
    big_super_step<WT, true>(acc, w0, w1, sb, sa, xr, wr, sr, xrsrc, unit0, units, xvoff, xoff, tg, K,
                             st + 1, lane, xs[1], xs[0], tab);
  } else {
    big_super_step<WT, true>(acc, w0, w1, sa, sb, xr, wr, sr, xrsrc, unit0, units, xvoff, xoff, tg, K,
                             st, lane, xs[0], xs[1], tab);
  }
#pragma unroll
  for (int t = 0; t < WT; ++t) {
    const int tile = tg + 2 * t;
#pragma unroll
    for (int j = 0; j < kBigNT; ++j) {
      if (!tile_ok[j]) continue;
      const int n = nbase + 16 * j + r16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 16 * tile + 4 * g + q;
        if (r < prow) y[(int64_t)(row0 + pbase + r) * N + n] = acc[t][j][q];
      }
    }
  }
  __syncthreads();  // every wave is done with the LDS tiles before the next pass
}

__global__ __launch_bounds__(kBigThreads) void moe_gemm_big_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const int32_t* __restrict__ expert_ids, int num_experts, int N, int K,
    const uint8_t* __restrict__ x, const int32_t* __restrict__ row_offsets, int M,
    float* __restrict__ y) {
  __shared__ ScaleEntry tab[256];
  __shared__ u32x4 xs[2][kBigTiles * 4 * 64];  // [buffer][tile][s][h][lane]
  fill_scale_table(tab);
  const int i = blockIdx.y;
  int row0, count;
  expert_rows(row_offsets, i, M, row0, count);
  const int passes = (count + kBigRows - 1) / kBigRows;
  // Equal passes of whole 16-row tiles.
  const int per_pass = passes ? ((count + passes - 1) / passes + 15) / 16 * 16 : 0;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int nbase = blockIdx.x * kBigN + (w & 3) * kBigNT * 16;
  int64_t ex = expert_ids[i];
  if (kCheckBounds && (ex < 0 || ex >= num_experts)) {
    if (tid == 0) raise_error(kErrIndex);
    ex = -1;
  }
  if (ex < 0) return;  // uniform over the workgroup, before any barrier

  // Weight tiles past N repeat the expert's first tile (their products are
  // never stored).
  const int units = K / kUnitK;
  const int ntile = nbase < N ? nbase / 16 : 0;
  bool tile_ok[kBigNT];
#pragma unroll
  for (int j = 0; j < kBigNT; ++j) tile_ok[j] = nbase + 16 * j < N;
  const int unit0 = ntile * units;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(codes + ex * ((int64_t)N * K / 2)), (short)0, N * (K / 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + ex * ((int64_t)N * K / 32)), (short)0, N * (K / 32), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(x + (int64_t)row0 * K), (short)0, count * K, kRsrcWord3);

  for (int pz = blockIdx.z; pz < passes; pz += gridDim.z) {
    const int pbase = pz * per_pass;
    const int prow = min(per_pass, count - pbase);
    const int pairs = (prow + 31) / 32;  // tile pairs: each wave takes one tile of a pair
    if (pairs > 6)
      big_pass<8>(xs, wr, sr, xrsrc, unit0, units, K, N, pbase, prow, row0, tid, nbase, tile_ok, tab, y);
    else if (pairs > 4)
      big_pass<6>(xs, wr, sr, xrsrc, unit0, units, K, N, pbase, prow, row0, tid, nbase, tile_ok, tab, y);
    else if (pairs > 2)
      big_pass<4>(xs, wr, sr, xrsrc, unit0, units, K, N, pbase, prow, row0, tid, nbase, tile_ok, tab, y);
    else
      big_pass<2>(xs, wr, sr, xrsrc, unit0, units, K, N, pbase, prow, row0, tid, nbase, tile_ok, tab, y);
  }
}

// Conversion: one thread per MX block (32 elements: 16 code bytes, one
// scale) -> 32 E4M3 bytes.  The input is in either layout; the output is
// row-major ([n_act, N, K], blocks in row order) or in unit order (the
// staged pipeline's workspace: a block's 32 bytes are pieces 2 q and 2 q + 1
// of its lane in a 4 KB unit).  Threads walk the output in storage order.
template <bool kTiledOut>
__global__ __launch_bounds__(kMoeThreads) void mxfp4_to_fp8_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int tiled_in,
    const int32_t* __restrict__ expert_ids, int num_experts, int N, int K, int n_act,
    uint8_t* __restrict__ w8) {
  __shared__ ScaleEntry tab[256];
  fill_scale_table(tab);
  __syncthreads();
  const int kbs = K / 32;
  const int64_t per_expert = (int64_t)N * kbs;
  const int64_t total = per_expert * n_act;
  for (int64_t u = (int64_t)blockIdx.x * kMoeThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kMoeThreads) {
    const int i = (int)(u / per_expert);
    const int64_t rem = u - (int64_t)i * per_expert;
    int64_t n, kb, out;
    if constexpr (kTiledOut) {
      // rem = ((tile * units + unit) * 2 + q) * 64 + lane
      const int lane = (int)(rem % 64), q = (int)((rem / 64) % 2);
      const int64_t unit = rem / 128;  // tile * (K / 256) + unit within the tile
      n = (unit / (K / kUnitK)) * 16 + lane % 16;
      kb = (unit % (K / kUnitK)) * 8 + (lane / 16) * 2 + q;
      out = (int64_t)i * N * K + unit * 4096 + 2 * q * 1024 + lane * 16;
    } else {
      n = rem / kbs;
      kb = rem % kbs;
      out = ((int64_t)i * N + n) * K + 32 * kb;
    }
    const int64_t ex = expert_ids[i];
    if (kCheckBounds && (ex < 0 || ex >= num_experts)) {
      raise_error(kErrIndex);
      continue;
    }
    const u32x4 raw = __builtin_nontemporal_load(
        (const u32x4*)(codes + ex * (int64_t)N * (K / 2) + code_offset(tiled_in, n, kb, N, K)));
    const ScaleEntry& t =
        tab[scales[ex * (int64_t)N * (K / 32) + scale_offset(tiled_in, n, kb, N, K)]];
    const i32x8 o = convert_block(raw, t);
    const u32x4 lo = {(uint32_t)o[0], (uint32_t)o[1], (uint32_t)o[2], (uint32_t)o[3]};
    const u32x4 hi = {(uint32_t)o[4], (uint32_t)o[5], (uint32_t)o[6], (uint32_t)o[7]};
    *(u32x4*)(w8 + out) = lo;
    *(u32x4*)(w8 + out + (kTiledOut ? 1024 : 16)) = hi;
  }
}

// Row-major MXFP4 -> unit order (a byte permutation): one thread per MX
// block, walking the output in storage order.
__global__ __launch_bounds__(kMoeThreads) void mxfp4_pack_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int E, int N, int K,
    uint8_t* __restrict__ codes_out, uint8_t* __restrict__ scales_out) {
  const int64_t per_expert = (int64_t)N * (K / 32);
  const int64_t total = per_expert * E;
  for (int64_t u = (int64_t)blockIdx.x * kMoeThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kMoeThreads) {
    const int64_t e = u / per_expert, rem = u - e * per_expert;
    const int lane = (int)(rem % 64), q = (int)((rem / 64) % 2);
    const int64_t unit = rem / 128;
    const int64_t n = (unit / (K / kUnitK)) * 16 + lane % 16;
    const int64_t kb = (unit % (K / kUnitK)) * 8 + (lane / 16) * 2 + q;
    const int64_t cbase = e * N * (K / 2), sbase = e * N * (K / 32);
    *(u32x4*)(codes_out + cbase + code_offset(true, n, kb, N, K)) =
        *(const u32x4*)(codes + cbase + code_offset(false, n, kb, N, K));
    scales_out[sbase + scale_offset(true, n, kb, N, K)] =
        scales[sbase + scale_offset(false, n, kb, N, K)];
  }
}

template <bool kFp4, bool kTiled, int NT, int RT, int S>
void launch_moe(const uint8_t* wsrc, const uint8_t* scales, const int32_t* expert_ids,
                int num_experts, int N, int K, const uint8_t* x, const int32_t* row_offsets,
                int n_act, int M, int max_rows, float* y, hipStream_t stream) {
  const int nblocks = (N + 16 * NT * kMoeWaves - 1) / (16 * NT * kMoeWaves);
  const int passes = max_rows < 1 ? 1 : (max_rows + 16 * RT - 1) / (16 * RT);
  const dim3 grid((unsigned)nblocks, (unsigned)n_act, (unsigned)(passes > 65535 ? 65535 : passes));
  hipLaunchKernelGGL((moe_gemm_kernel<NT, RT, S, kFp4, kTiled>), grid, dim3(kMoeThreads), 0,
                     stream, wsrc, scales, expert_ids, num_experts, N, K, x, row_offsets, M, y);
}

void launch_moe_big(const uint8_t* wsrc, const uint8_t* scales, const int32_t* expert_ids,
                    int num_experts, int N, int K, const uint8_t* x, const int32_t* row_offsets,
                    int n_act, int M, int max_rows, float* y, hipStream_t stream) {
  const int nblocks = (N + kBigN - 1) / kBigN;
  const int passes = (max_rows + kBigRows - 1) / kBigRows;
  const dim3 grid((unsigned)nblocks, (unsigned)n_act, (unsigned)(passes > 65535 ? 65535 : passes));
  hipLaunchKernelGGL(moe_gemm_big_kernel, grid, dim3(kBigThreads), 0, stream, wsrc, scales,
                     expert_ids, num_experts, N, K, x, row_offsets, M, y);
}

// Row tiles a pass by size: one 16-row tile for decode-sized batches (the
// weights are read once whatever the row count), two up to 32 rows; larger
// batches on tiled MXFP4 weights take the LDS-staged kernel (256 rows a
// pass), others four tiles (64 rows) a pass.  Super-steps of 256 k (the tiled unit; row-major weights
// with K % 256 != 0 take 128).
template <bool kFp4, bool kTiled>
void dispatch_moe(const uint8_t* wsrc, const uint8_t* scales, const int32_t* expert_ids,
                  int num_experts, int N, int K, const uint8_t* x, const int32_t* row_offsets,
                  int n_act, int M, int max_rows, float* y, hipStream_t stream) {
#define DSA_MOE_LAUNCH(RT, S)                                                              \
  launch_moe<kFp4, kTiled, 2, RT, S>(wsrc, scales, expert_ids, num_experts, N, K, x,      \
                                     row_offsets, n_act, M, max_rows, y, stream)
  if (kTiled || K % kUnitK == 0) {
    if (max_rows <= 16) DSA_MOE_LAUNCH(1, 2);
    else if (max_rows <= 32) DSA_MOE_LAUNCH(2, 2);
    else if (kFp4 && kTiled && (int64_t)M * K <= INT32_MAX &&
             (int64_t)N * K / 2 <= INT32_MAX)
      launch_moe_big(wsrc, scales, expert_ids, num_experts, N, K, x, row_offsets, n_act, M,
                     max_rows, y, stream);
    else DSA_MOE_LAUNCH(4, 2);
  } else if constexpr (!kTiled) {
    if (max_rows <= 16) DSA_MOE_LAUNCH(1, 1);
    else if (max_rows <= 32) DSA_MOE_LAUNCH(2, 1);
    else DSA_MOE_LAUNCH(4, 1);
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

dsa_status_t check_weights(const dsa_mxfp4_weights_t* w) {
  if (!w || !w->codes || !w->scales) return DSA_ERR_NULL;
  if (w->num_experts < 1 || w->N < 1 || w->K < 1) return DSA_ERR_SHAPE;
  if (w->layout != DSA_MXFP4_ROW_MAJOR && w->layout != DSA_MXFP4_TILED) return DSA_ERR_SHAPE;
  if (w->K % 128 || w->N % 16 || (w->layout == DSA_MXFP4_TILED && w->K % kUnitK))
    return DSA_ERR_UNSUPPORTED;
  if (!aligned16(w->codes) || ((uintptr_t)w->scales & 3)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

unsigned grid_for(int64_t threads) {
  const int64_t blocks = (threads + kMoeThreads - 1) / kMoeThreads;
  return (unsigned)(blocks < 16384 ? blocks : 16384);
}

dsa_status_t convert_launch(const dsa_mxfp4_weights_t* w, const int32_t* expert_ids, int n_act,
                            uint8_t* w8, bool tiled_out, hipStream_t stream) {
  const unsigned grid = grid_for((int64_t)n_act * w->N * (w->K / 32));
  const int tiled_in = w->layout == DSA_MXFP4_TILED;
  if (tiled_out)
    hipLaunchKernelGGL(mxfp4_to_fp8_kernel<true>, dim3(grid), dim3(kMoeThreads), 0, stream,
                       w->codes, w->scales, tiled_in, expert_ids, w->num_experts, w->N, w->K,
                       n_act, w8);
  else
    hipLaunchKernelGGL(mxfp4_to_fp8_kernel<false>, dim3(grid), dim3(kMoeThreads), 0, stream,
                       w->codes, w->scales, tiled_in, expert_ids, w->num_experts, w->N, w->K,
                       n_act, w8);
  return launch_status();
}

}  // namespace

uint32_t take_bounds_error_moe(hipStream_t stream) { return take_bounds_error(stream); }

}  // namespace dsa

extern "C" dsa_status_t dsa_mxfp4_pack(const dsa_mxfp4_weights_t* w, uint8_t* codes_tiled,
                                       uint8_t* scales_tiled, hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_weights(w);
  if (st != DSA_OK) return st;
  if (!codes_tiled || !scales_tiled) return DSA_ERR_NULL;
  if (w->layout != DSA_MXFP4_ROW_MAJOR) return DSA_ERR_SHAPE;
  if (w->K % kUnitK || !aligned16(codes_tiled)) return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  const unsigned grid = grid_for((int64_t)w->num_experts * w->N * (w->K / 32));
  hipLaunchKernelGGL(mxfp4_pack_kernel, dim3(grid), dim3(kMoeThreads), 0, stream, w->codes,
                     w->scales, w->num_experts, w->N, w->K, codes_tiled, scales_tiled);
  return launch_status();
}

extern "C" dsa_status_t dsa_moe_gemm_mxfp4(const dsa_mxfp4_weights_t* w, const uint8_t* x,
                                           const int32_t* expert_ids, const int32_t* row_offsets,
                                           int32_t n_act, int32_t M, int32_t max_rows, float* y,
                                           hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_weights(w);
  if (st != DSA_OK) return st;
  if (!expert_ids) return DSA_ERR_NULL;
  st = check_moe_common(w->N, w->K, x, row_offsets, n_act, M, y);
  if (st != DSA_OK) return st;
  st = check_device();
  if (st != DSA_OK) return st;
  if (w->layout == DSA_MXFP4_TILED)
    dispatch_moe<true, true>(w->codes, w->scales, expert_ids, w->num_experts, w->N, w->K, x,
                             row_offsets, n_act, M, max_rows, y, stream);
  else
    dispatch_moe<true, false>(w->codes, w->scales, expert_ids, w->num_experts, w->N, w->K, x,
                              row_offsets, n_act, M, max_rows, y, stream);
  return launch_status();
}

extern "C" dsa_status_t dsa_mxfp4_to_fp8(const dsa_mxfp4_weights_t* w, const int32_t* expert_ids,
                                         int32_t n_act, uint8_t* w8, hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_weights(w);
  if (st != DSA_OK) return st;
  if (!w8 || !expert_ids) return DSA_ERR_NULL;
  if (n_act < 1 || n_act > 65535) return DSA_ERR_SHAPE;
  if (!aligned16(w8)) return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  return convert_launch(w, expert_ids, n_act, w8, false, stream);
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
  dispatch_moe<false, false>(w8, nullptr, nullptr, n_act, N, K, x, row_offsets, n_act, M,
                             max_rows, y, stream);
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
  dsa_status_t st = check_weights(w);
  if (st != DSA_OK) return st;
  if (!expert_ids) return DSA_ERR_NULL;
  st = check_moe_common(w->N, w->K, x, row_offsets, n_act, M, y);
  if (st != DSA_OK) return st;
  if (!workspace || !events || !events[0] || !events[1] || !events[2] || !events[3] ||
      !events[4])
    return DSA_ERR_NULL;
  if (conv_stream == stream) return DSA_ERR_SHAPE;
  if (!aligned16(workspace)) return DSA_ERR_UNSUPPORTED;
  const size_t expert_bytes = (size_t)w->N * (size_t)w->K;
  const int64_t chunk64 = (int64_t)(workspace_bytes / (2 * expert_bytes));
  if (chunk64 < 1) return DSA_ERR_WORKSPACE;
  const int chunk = (int)(chunk64 < n_act ? chunk64 : n_act);
  st = check_device();
  if (st != DSA_OK) return st;
  // The workspace holds converted weights in unit order whenever K allows.
  const bool tiled = w->K % kUnitK == 0;
  uint8_t* half[2] = {(uint8_t*)workspace, (uint8_t*)workspace + (size_t)chunk * expert_bytes};
  hipEvent_t* ready = events;      // half h holds converted weights
  hipEvent_t* free_ = events + 2;  // the last product reading half h has finished
  // The conversions come after everything enqueued on `stream` so far.
  if (hipEventRecord(events[4], stream) != hipSuccess ||
      hipStreamWaitEvent(conv_stream, events[4], 0) != hipSuccess)
    return DSA_ERR_HIP;
  for (int c0 = 0, c = 0; c0 < n_act; c0 += chunk, ++c) {
    const int h = c & 1, n = n_act - c0 < chunk ? n_act - c0 : chunk;
    if (hipStreamWaitEvent(conv_stream, free_[h], 0) != hipSuccess) return DSA_ERR_HIP;
    st = convert_launch(w, expert_ids + c0, n, half[h], tiled, conv_stream);
    if (st != DSA_OK) return st;
    if (hipEventRecord(ready[h], conv_stream) != hipSuccess ||
        hipStreamWaitEvent(stream, ready[h], 0) != hipSuccess)
      return DSA_ERR_HIP;
    if (tiled)
      dispatch_moe<false, true>(half[h], nullptr, nullptr, n, w->N, w->K, x, row_offsets + c0, n,
                                M, max_rows, y, stream);
    else
      dispatch_moe<false, false>(half[h], nullptr, nullptr, n, w->N, w->K, x, row_offsets + c0,
                                 n, M, max_rows, y, stream);
    st = launch_status();
    if (st != DSA_OK) return st;
    if (hipEventRecord(free_[h], stream) != hipSuccess) return DSA_ERR_HIP;
  }
  return DSA_OK;
}
