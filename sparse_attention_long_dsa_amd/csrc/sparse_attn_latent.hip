// Exact sparse attention for the latent row shape (web page "Day-0
// Adaptation of Trillion-Parameter MoE Models on Domestic GPUs", section 3:
// exact attention over the Top-K positions read through the paged index
// table; item (3) separate prefill and decode paths): 128 query heads share
// one 576-wide cached row whose first 512 columns are the value.
#include "attn_common.h"

namespace dsa {
namespace {

// ===================================================== latent rows (MLA shape)
//
// 128 heads share one 576-wide row (512 value/latent + 64 rope columns, V =
// the first 512).  One workgroup takes one query and all 128 heads: four
// waves, one per SIMD, each owning 32 heads, so every row a tile brings
// into LDS is read once per wave for S and once per wave for P V, and the
// kernel is bound by the matrix cores rather than by LDS.
//
// Per tile of 32 kept rows:
//   gather:  the rows go from HBM straight into LDS with the gfx950 direct
//            global->LDS load (16 bytes a lane, no registers); the next
//            tile's loads are in flight while this tile computes (two LDS
//            buffers);
//   S^T = K Q^T on MFMA 32x32x16 bf16 (A = K rows from LDS, B = q held in
//            registers for the whole kernel); the A rows are read in a
//            permuted order so that each result lane holds one head and 16
//            tokens laid out exactly as the P^T operand of P V needs them;
//   online softmax in the log2 domain, per head in one lane pair;
//   O^T += V^T P^T on MFMA 32x32x16 (A = V^T read with the LDS transpose
//            load from the same tile, B = P^T straight from registers, as
//            bf16 hi + lo).  O^T (512 x 32 fp32 per wave) lives in the
//            accumulation registers.
namespace latent {

constexpr int kDqk = 576, kDv = 512, kHeads = 128;
constexpr int kWaves = 4, kThreads = kWaves * kWave;
constexpr int kRowSlots = kDqk / 8 + 1;             // 72 16-byte chunks + 1 pad slot (LDS banks)
constexpr int kRowElems = kRowSlots * 8;            // LDS row stride (elements)
constexpr int kTileSlots = kTile * kRowSlots;       // 2336
constexpr int kLoadBlocks = (kTileSlots + kWave - 1) / kWave;  // 37 wave loads hold a tile
constexpr int kWaveBlocks = (kLoadBlocks + kWaves - 1) / kWaves;  // loads per wave (all equal)
constexpr int kBufSlots = kWaveBlocks * kWaves * kWave;  // slots past the tile take junk
constexpr int kBufs = 3;                            // tiles t, t + 1, t + 2 in flight
constexpr int kKS = kDqk / 16;                      // k-steps of S
constexpr int kDVB = kDv / 32;                      // 32-wide value blocks
constexpr int kMaxTiles = 2048 / kTile;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Direct global -> LDS load of 16 bytes a lane (lane l fills LDS bytes
// lds + 16 l .. + 15), written out so that the compiler does not track it:
// it would otherwise wait for every such load in flight before each LDS read,
// which serialises the loads of the tiles ahead with the current tile's
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

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product with the accumulator pinned to VGPRs.  O^T fills all 256
// accumulation registers, so S^T has to accumulate in ordinary VGPRs; the
// compiler picks the register file of an MFMA result by itself, hence the
// explicit form (the result must not share registers with the operands,
// hence the early clobber on the form that starts from zero).
__device__ __forceinline__ void mfma32_vgpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_vgpr_first(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
// Wait states between the last MFMA writing these VGPRs and VALU reads of
// them (16-pass MFMA results; 24 states is more than the hardware needs).
__device__ __forceinline__ void mfma_result_fence(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}
__device__ __forceinline__ void mfma_result_fence(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}

// Token held in accumulator slot v by a lane of half h (= lane / 32):
// 8 h + (v % 8) for v < 8, 16 + 8 h + (v % 8) for v >= 8.  Accumulator row
// m of the 32x32 result holds token perm(m), so the A operand reads row
// perm(m) for its row m.
__device__ __forceinline__ int acc_token(int v, int h) { return 16 * (v >> 3) + 8 * h + (v & 7); }
__device__ __forceinline__ int perm_row(int m) {
  const int b = m >> 3, h = (m >> 2) & 1, i = m & 3;
  return 16 * (b >> 1) + 8 * h + 4 * (b & 1) + i;
}

// A operand of O^T += V^T P^T for value block dvb and token half ks: lane l
// holds value column 32 dvb + l % 32 and tokens 16 ks + 8 (l / 32) .. + 7.
// Within each 16-lane group, lane i names V[t0 + i / 4][c0 + 4 (i % 4) ..]
// and the transpose load hands lane j the column c0 + j of 4 tokens.
__device__ __forceinline__ bf16x8 load_vt32(const uint16_t* tile, int dvb, int ks, int lane) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int g = lane >> 4, i = lane & 15;
  const int c0 = 32 * dvb + 16 * (g & 1);
  const int t0 = 16 * ks + 8 * (g >> 1);
  const uint16_t* p0 = tile + (t0 + (i >> 2)) * kRowElems + c0 + 4 * (i & 3);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * kRowElems));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return as_bf16x8(u32x4{ua.x, ua.y, ub.x, ub.y});
}

__global__ __launch_bounds__(kThreads, 1) void sparse_attn_latent_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, const uint16_t* __restrict__ q, const int32_t* __restrict__ idx,
    int n_q, int K, const int32_t* __restrict__ seq_lens, int prefill_seq, int pos0,
    int tiles_per_split, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int n_splits) {
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kBufs][kBufSlots * 8];
  __shared__ int32_t trows[kMaxTiles * kTile];

  // blocks of one query share an XCD (same block id modulo 8)
  const int b = blockIdx.x;
  const int j = b >> 3;
  const int qi = (j / n_splits) * 8 + (b & 7), split = j % n_splits;
  if (qi >= n_q) return;
  const bool decode = seq_lens != nullptr;
  const int seq = decode ? qi : prefill_seq;
  const int n_cand = decode ? seq_lens[qi] : pos0 + qi + 1;
  const int count = min(K, n_cand);
  const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
  const int32_t* sel = idx + (int64_t)qi * K;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar
  const int half = lane >> 5;
  const int head = 32 * wave + (lane & 31);  // this lane's head (B operand column, O^T column)

  const int n_tiles = (count + kTile - 1) / kTile;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);

  // physical rows of this block's kept positions; a padded slot repeats the
  // first kept row (finite data, weight 0)
  const int32_t row0 = count > 0 ? (int32_t)paged_row(bt_row, bs, sel[0]) : 0;
  for (int r = threadIdx.x; r < (t_end - t_begin) * kTile; r += kThreads) {
    const int g = t_begin * kTile + r;
    trows[r] = g < count ? (int32_t)paged_row(bt_row, bs, sel[g]) : row0;
  }

  // q as the B operand of S^T: head `head`, dims 16 ks + 8 half .. + 7
  bf16x8 qf[kKS];
  {
    const uint16_t* qrow = q + ((int64_t)qi * kHeads + head) * kDqk + 8 * half;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(qrow + 16 * ks));
  }
  __syncthreads();

  // Wave w issues the tile's 16-byte slots 64 b + lane for b = w, w + 4, ...
  // (its i-th block is b = w + 4 i; every wave issues kWaveBlocks, so the
  // per-wave count of loads in flight is known).  Slot s is chunk s % 73 of
  // tile row s / 73; the pad chunk and the tail slots past the tile load a
  // valid chunk that nothing reads.  The blocks of a tile are issued one by
  // one between the S products of the tile two places earlier.
  const int32_t* ld_tr = trows;
  int ld_buf = 0, ld_r = 0, ld_c = 0;
  auto load_begin = [&](int t, int buf) {
    ld_tr = trows + (t - t_begin) * kTile;
    ld_buf = buf;
    const int s0 = kWave * wave + lane;
    ld_r = s0 / kRowSlots;
    ld_c = s0 - ld_r * kRowSlots;
  };
  const uint32_t tiles_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)tiles;
  const uint64_t row_bytes = (uint64_t)kv_stride * 2;
  auto load_block = [&](int i) {
    const int blk = wave + kWaves * i;
    const int rr = ld_r < kTile ? ld_r : 0;
    const int cc = ld_c < kDqk / 8 ? ld_c : 0;
    const char* src = (const char*)kv + (uint64_t)(uint32_t)ld_tr[rr] * row_bytes + 16 * cc;
    global_to_lds16(src, tiles_lds + (uint32_t)(ld_buf * kBufSlots + kWave * blk) * 16u);
    // this wave's next block is 256 slots on
    constexpr int kStepRows = kWaves * kWave / kRowSlots;
    constexpr int kStepSlots = kWaves * kWave % kRowSlots;
    ld_c += kStepSlots;
    ld_r += kStepRows;
    if (ld_c >= kRowSlots) {
      ld_c -= kRowSlots;
      ++ld_r;
    }
  };

  // A operand rows of S^T: this lane reads tile row perm(lane % 32), dims
  // 16 ks + 8 half .. + 7
  const int a_off = perm_row(lane & 31) * kRowElems + 8 * half;

  // Softmax base: the exponent base of a head is its maximum over the first
  // tile and is never moved, so O^T is never rescaled inside the loop (its
  // 256 registers stay in the accumulation file).  Later tiles may give
  // weights above 1; fp32 and bf16 hold them exactly as well up to 2^kMaxExp.
  // If any head passes that, the block runs the tiles a second time with the
  // base set to the true maximum (rare: a logit 44 above the first tile's).
  constexpr float kMaxExp = 64.f;
  f32x16 o[kDVB];
  float m_base = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
  bool redo = false;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (!__syncthreads_or(redo)) break;
      m_base = m_seen;
    }
#pragma unroll
    for (int d = 0; d < kDVB; ++d) o[d] = f32x16{};
    l_run = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (t_begin + j < t_end) {
        load_begin(t_begin + j, j);
#pragma unroll
        for (int i = 0; i < kWaveBlocks; ++i) load_block(i);
      }
    }

    for (int t = t_begin; t < t_end; ++t) {
      const int buf = (t - t_begin) % kBufs;
      // this tile's rows have landed (the next tile's kWaveBlocks loads may
      // still fly) ...
      if (t + 1 < t_end)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaveBlocks) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // ... for every wave, and tile t - 1's buffer is free
      const bool next = t + 2 < t_end;
      if (next) load_begin(t + 2, (buf + 2) % kBufs);
      const uint16_t* tile = tiles[buf];

      // ---- S^T = K Q^T.  With one wave per SIMD nothing else hides LDS
      // latency, so the A operands are read kDepthS k-steps ahead into a
      // ring (a slot is refilled two products after its last use).
      constexpr int kDepthS = 4, kRingS = kDepthS + 2;
      f32x16 s, s_odd;
      bf16x8 ar[kRingS];
#pragma unroll
      for (int j = 0; j < kDepthS; ++j) ar[j] = as_bf16x8(*(const u32x4*)(tile + a_off + 16 * j));
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) {
        f32x16& acc = (ks & 1) ? s_odd : s;
        if (ks < 2)
          mfma32_vgpr_first(acc, ar[ks], qf[ks]);
        else
          mfma32_vgpr(acc, ar[ks % kRingS], qf[ks]);
        if (ks + kDepthS < kKS)
          ar[(ks + kDepthS) % kRingS] = as_bf16x8(*(const u32x4*)(tile + a_off + 16 * (ks + kDepthS)));
        if (next && ks % 3 == 1 && ks / 3 < kWaveBlocks) load_block(ks / 3);
      }
      mfma_result_fence(s, s_odd);
      s += s_odd;

      // ---- softmax weights, log2 domain; masked tokens (only in a range's
      // last tile) get weight 0
      const int g0 = t * kTile;
      const bool full = g0 + kTile <= count;
      float sv[16];
      float mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sv[v] = s[v];
        if (!full && g0 + acc_token(v, half) >= count) sv[v] = -INFINITY;
        mt = fmaxf(mt, sv[v]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
      if (m_base == -INFINITY) m_base = mt;  // first tile (every tile has a kept row)
      m_seen = fmaxf(m_seen, mt);
      redo |= mt > m_base + kMaxExp;
      // P = P_hi + P_lo as bf16 pairs; tokens 0..15 (ks = 0) now, tokens
      // 16..31 while the first half's products run
      float psum = 0.f;
      u32x4 ph[2], pl[2];
      auto make_p = [&](int ks, int w) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sv[8 * ks + 2 * w], scale_log2, -m_base));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sv[8 * ks + 2 * w + 1], scale_log2, -m_base));
        psum += p0 + p1;
        const uint32_t hi = pack_bf16x2(p0, p1);
        ph[ks][w] = hi;
        pl[ks][w] = pack_bf16x2(p0 - bf16_lo(hi), p1 - bf16_hi(hi));
      };
#pragma unroll
      for (int w = 0; w < 4; ++w) make_p(0, w);

      // ---- O^T += V^T P^T (P as bf16 hi + lo).  V^T operands are read
      // kDepthV value blocks ahead; the scheduling barriers keep the
      // compiler from sinking the reads back next to their products.
      constexpr int kDepthV = 3, kRingV = kDepthV + 2;
      bf16x8 vr[kRingV];
#pragma unroll
      for (int j = 0; j < kDepthV; ++j) vr[j] = load_vt32(tile, j % kDVB, j / kDVB, lane);
      // Product i (i = ks * kDVB + d) adds its bf16-hi part, then the lo part
      // of product i - 1, so consecutive MFMAs never share an accumulator.
#pragma unroll
      for (int i = 0; i <= 2 * kDVB; ++i) {
        if (i + kDepthV < 2 * kDVB) {
          const int n = i + kDepthV;
          vr[n % kRingV] = load_vt32(tile, n % kDVB, n / kDVB, lane);
        }
        if (i < 2 * kDVB) {
          const int ks = i / kDVB, d = i % kDVB;
          o[d] = mfma32(vr[i % kRingV], as_bf16x8(ph[ks]), o[d]);
        }
        if (i > 0) {
          const int ks = (i - 1) / kDVB, d = (i - 1) % kDVB;
          o[d] = mfma32(vr[(i - 1) % kRingV], as_bf16x8(pl[ks]), o[d]);
        }
        if (i >= 1 && i <= 4) make_p(1, i - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      l_run += psum + __shfl_xor(psum, 32);
    }
  }
  const float m_run = m_base;

  // ---- epilogue: lane holds head `head`, value columns
  // 32 d + 8 (v / 4) + 4 half + v % 4
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_val = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  if (n_splits == 1) {
    uint16_t* orow = out + ((int64_t)qi * kHeads + head) * kDv + 4 * half;
#pragma unroll
    for (int d = 0; d < kDVB; ++d)
#pragma unroll
      for (int bq = 0; bq < 4; ++bq) {
        const uint32_t lo = pack_bf16x2(o[d][4 * bq] * inv_l, o[d][4 * bq + 1] * inv_l);
        const uint32_t hi = pack_bf16x2(o[d][4 * bq + 2] * inv_l, o[d][4 * bq + 3] * inv_l);
        *(uint2*)(orow + 32 * d + 8 * bq) = make_uint2(lo, hi);
      }
    if (lse && half == 0) lse[(int64_t)qi * kHeads + head] = lse_val;
  } else {
    const int64_t pidx = ((int64_t)qi * n_splits + split) * kHeads + head;
    float* prow = part_o + pidx * kDv + 4 * half;
#pragma unroll
    for (int d = 0; d < kDVB; ++d)
#pragma unroll
      for (int bq = 0; bq < 4; ++bq)
        *(f32x4*)(prow + 32 * d + 8 * bq) =
            f32x4{o[d][4 * bq] * inv_l, o[d][4 * bq + 1] * inv_l, o[d][4 * bq + 2] * inv_l,
                  o[d][4 * bq + 3] * inv_l};
    if (half == 0) part_lse[pidx] = lse_val;
  }
}

}  // namespace latent
}  // namespace

void launch_latent(const dsa_paged_cache_t* c, const uint16_t* q, const int32_t* idx, int n_q,
                   int K, const int32_t* seq_lens, int seq, int pos0, float sm_scale,
                   uint16_t* out, float* lse, float* part_o, float* part_lse, SplitPlan plan,
                   hipStream_t stream) {
  const int64_t blocks = ((int64_t)n_q + 7) / 8 * 8 * plan.n_splits;
  hipLaunchKernelGGL(latent::sparse_attn_latent_kernel, dim3((unsigned)blocks),
                     dim3(latent::kThreads), 0, stream, c->kv, c->kv_row_stride, c->block_table,
                     c->max_blocks_per_seq, c->block_size, q, idx, n_q, K, seq_lens, seq, pos0,
                     plan.tiles_per_split, sm_scale * kLog2e, out, lse, part_o, part_lse,
                     plan.n_splits);
  if (plan.n_splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel<latent::kDv>, dim3(n_q * latent::kHeads), dim3(128), 0,
                       stream, part_o, part_lse, plan.n_splits, latent::kHeads, out, lse);
}

}  // namespace dsa
