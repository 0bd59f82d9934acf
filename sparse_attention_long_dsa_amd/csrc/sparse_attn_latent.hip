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
// the first 512).  One workgroup takes one query and all 128 heads with
// four waves, one per SIMD.  The two products split the work differently:
//   S^T = K Q^T by heads: wave w owns heads 32 w .. 32 w + 31 (its q stays
//        in registers for the whole kernel), MFMA 32x32x16 bf16 with the K
//        rows as the A operand read from LDS;
//   O^T += V^T P^T by value columns: wave w owns columns 128 w .. + 127 for
//        all 128 heads, so each V^T operand (the slow LDS transpose read) is
//        read by one wave only and serves 4 head blocks.  This product runs
//        in fp16 (MFMA 32x32x16 f16, fp32 accumulation): P carries 11
//        significant bits, and the bf16 values convert exactly for
//        magnitudes in [2^-17, 65504].  P goes through a small LDS buffer
//        from the wave that computed it to all four.
// Softmax statistics stay with the head owner; the exponent base of a head
// is its maximum over the first tile that holds a kept row and never moves
// (negative indices are skipped, so a tile can hold none), so O^T (128 heads x
// 128 columns fp32 per wave, in the accumulation registers) is never
// rescaled.  A block whose later logits pass that base by more than 2^15 in
// weight (the fp16 range) runs its tiles again with the true maximum as the
// base.
//
// Tiles of 32 kept rows go from HBM straight into LDS (gfx950 direct
// global->LDS loads, no registers), one tile ahead.  Iteration t computes
// S(t) and the softmax of tile t, then O += V P for tile t - 1: three tile
// buffers (t - 1 for V, t for K, t + 1 loading) and two P buffers, one
// barrier per tile.
namespace latent {

constexpr int kDqk = 576, kDv = 512, kHeads = 128;
constexpr int kWaves = 4, kThreads = kWaves * kWave;
// LDS tile: the 512 latent (value) columns of each row at a stride of 67
// 16-byte slots (the 16 rows an A-operand read touches land in 16 different
// bank groups, and the 4 rows of a transposed V read in disjoint ones),
// followed by the 64 rope columns of all 32 rows in 8-slot rows whose chunk
// index is XOR-swizzled by bits 1..3 of the row.
constexpr int kLatBytes = kDv * 2;                  // 1024
constexpr int kRowBytes = kLatBytes + 48;           // 1072
constexpr int kRowElems = kRowBytes / 2;            // LDS row stride (elements)
constexpr int kRopeChunks = (kDqk - kDv) / 8;       // 8
constexpr int kLatRegion = kTile * kRowBytes;       // bytes
constexpr int kBufBytes = kLatRegion + kTile * kRopeChunks * 16;
constexpr int kRopeElems = kLatRegion / 2;          // element offset of the rope rows
constexpr int kBufs = 3;
constexpr int kKS = kDqk / 16;                      // k-steps of S
constexpr int kKSLat = kDv / 16;                    // k-steps over the latent columns
constexpr int kDvWave = kDv / kWaves;               // value columns per wave
constexpr int kDVB = kDvWave / 32;                  // 32-wide value blocks per wave
constexpr int kHB = kHeads / 32;                    // 32-head blocks
constexpr int kPElems = kHeads * kTile;             // one P buffer (fp16)
constexpr int kMaxTiles = 2048 / kTile;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The same load with a wave-uniform 64-bit base in SGPRs and a per-lane
// 32-bit byte offset (no vector address arithmetic).
__device__ __forceinline__ void global_to_lds16_s(const void* base, uint32_t off, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds)
      : "memory");
}

__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

// op(x, x of lane l ^ 32) in every lane l, by the gfx950 swap of the two
// 32-lane halves of a register pair: after the swap the first register holds
// (x[0..31], x[0..31]) and the second (x[32..63], x[32..63]).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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

// P buffer layout: head x 4 chunks of 8 tokens; the chunk index is
// XOR-swizzled with bits 2..3 of the head so that 16 lanes reading 16 heads
// at one chunk hit 16 different bank groups.
__device__ __forceinline__ int p_offset(int head, int chunk) {
  return head * kTile + 8 * (chunk ^ ((head >> 2) & 3));
}

// A operand of O^T += V^T P^T for value columns c0 .. c0 + 31 and token
// half ks: lane l holds column c0 + l % 32 and tokens 16 ks + 8 (l / 32)
// .. + 7.  Within each 16-lane group, lane i names V[t0 + i / 4][c + 4 (i %
// 4) ..] and the transpose load hands lane j the column c + j of 4 tokens.
__device__ __forceinline__ u32x4 load_vt32(const uint16_t* tile, int c0, int ks, int lane) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int g = lane >> 4, i = lane & 15;
  const int c = c0 + 16 * (g & 1);
  const int t0 = 16 * ks + 8 * (g >> 1);
  const uint16_t* p0 = tile + (t0 + (i >> 2)) * kRowElems + c + 4 * (i & 3);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * kRowElems));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return u32x4{ua.x, ua.y, ub.x, ub.y};
}

__global__ __launch_bounds__(kThreads, 1) void sparse_attn_latent_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, const uint16_t* __restrict__ q, const int32_t* __restrict__ idx,
    int n_q, int K, AttnQuery aq, int tiles_per_split, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, int n_splits) {
  __shared__ __attribute__((aligned(16))) uint16_t tiles[kBufs][kBufBytes / 2];
  __shared__ __attribute__((aligned(16))) uint16_t pbuf[2][kPElems];
  __shared__ int32_t trows[kMaxTiles * kTile];
  __shared__ uint32_t tvalid[kMaxTiles];  // per tile: slots that hold a kept row
  __shared__ float head_l[kHeads], head_lse[kHeads];

  // blocks of one query share an XCD (same block id modulo 8)
  const int b = blockIdx.x;
  const int j = b >> 3;
  const bool decode = aq.decode();
  // prefill rows usually grow with the query index: the latest go first
  const int qraw = (j / n_splits) * 8 + (b & 7), split = j % n_splits;
  const int qi = decode ? qraw : n_q - 1 - qraw;
  if (qi >= n_q || qi < 0) return;
  const int seq = aq.seq(qi);
  const int n_cand = aq.count(qi);
  const int count = min(K, n_cand);
  const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
  const int32_t* sel = idx + (int64_t)qi * K;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform: scalar
  const int half = lane >> 5;
  const int head = 32 * wave + (lane & 31);  // head whose S row and statistics this lane holds

  const int n_tiles = (count + kTile - 1) / kTile;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);

  // Prologue loads, in the order that keeps the two dependent round trips
  // (kept positions, then their block-table entries) off the q transfer:
  // the index loads go first, then q (the B operand of S^T: head `head`,
  // dims 16 ks + 8 half .. + 7), then the block-table loads, which wait
  // only for the index loads (memory returns in issue order) while q is
  // still in flight.
  constexpr int kPer = kMaxTiles * kTile / kThreads;
  const int n_rows = (t_end - t_begin) * kTile;
  const int32_t row_safe = (int32_t)checked_block(bt_row[0], aq.num_blocks) * bs;
  int32_t pos_r[kPer], blk_r[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = (int)threadIdx.x + kThreads * i;
    const int g = t_begin * kTile + r;
    pos_r[i] = r < n_rows && g < count ? aq.kept(sel[g], n_cand) : -1;
  }
  bf16x8 qf[kKS];
  {
    const uint16_t* qrow = q + ((int64_t)qi * kHeads + head) * kDqk + 8 * half;
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(qrow + 16 * ks));
  }
  // Physical rows of this block's kept positions, and per tile a bit mask of
  // the slots that hold one (slot < count and index >= 0: negative indices
  // are skipped).  Other slots read the row of position 0 (always a cached
  // token: finite data) with weight 0.
  {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      blk_r[i] = pos_r[i] >= 0 ? checked_block(bt_row[pos_r[i] / bs], aq.num_blocks) : 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int r = (int)threadIdx.x + kThreads * i;
      const bool ok = pos_r[i] >= 0;
      if (r < n_rows) trows[r] = ok ? blk_r[i] * bs + pos_r[i] % bs : row_safe;
      // slots 64 w' .. 64 w' + 63 of this wave: two tiles' masks
      const uint64_t m = __ballot(ok);
      const int s0 = kThreads * i + kWave * wave;
      if (lane == 0 && s0 < n_rows) {
        tvalid[s0 / kTile] = (uint32_t)m;
        tvalid[s0 / kTile + 1] = (uint32_t)(m >> 32);
      }
    }
  }

  // Consume q here, so that the compiler waits for these loads before the
  // tile loop.  Otherwise it counts them as possibly in flight inside the
  // loop and its waits there (which also cover the direct-to-LDS tile loads
  // it does not see) would drain the next tile's loads every tile.
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks) asm volatile("" ::"v"(qf[ks]));
  __syncthreads();

  // Loads of a tile: wave w brings rows 8 w .. 8 w + 7, one wave load per
  // row for the 512 latent columns (lane l: bytes 16 l .. of the row, the
  // row address is wave-uniform and lives in SGPRs) and one wave load for the
  // rope columns of all 8 rows (lane l: row 8 w + l / 8, the chunk that the
  // swizzle puts at rope slot 64 w + l).
  constexpr int kWaveRows = kTile / kWaves;       // 8
  constexpr int kWaveBlocks = kWaveRows + 1;      // 9 wave loads a tile
  const int32_t* ld_tr = trows;
  int ld_buf = 0, ld_next = 0, ld_rope = 0;
  const int rope_row = kWaveRows * wave + (lane >> 3);
  const uint32_t rope_col = kLatBytes + 16u * (uint32_t)((lane & 7) ^ ((rope_row >> 1) & 7));
  auto load_begin = [&](int t, int buf) {
    ld_tr = trows + (t - t_begin) * kTile + kWaveRows * wave;
    ld_buf = buf;
    ld_next = ld_tr[0];
    ld_rope = ld_tr[lane >> 3];
  };
  const uint32_t tiles_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)tiles;
  const uint64_t row_bytes = (uint64_t)kv_stride * 2;
  const uint32_t lane16 = 16u * (uint32_t)lane;
  auto load_block = [&](int i) {
    const uint32_t buf_lds = tiles_lds + (uint32_t)(ld_buf * kBufBytes);
    if (i < kWaveRows) {
      const int row = __builtin_amdgcn_readfirstlane(ld_next);
      if (i + 1 < kWaveRows) ld_next = ld_tr[i + 1];
      const char* src = (const char*)kv + (uint64_t)(uint32_t)row * row_bytes;
      global_to_lds16_s(src, lane16, buf_lds + (uint32_t)((kWaveRows * wave + i) * kRowBytes));
    } else {
      const char* src = (const char*)kv + (uint64_t)(uint32_t)ld_rope * row_bytes + rope_col;
      global_to_lds16(src, buf_lds + (uint32_t)(kLatRegion + kWave * 16 * wave));
    }
  };

  // A operand rows of S^T: this lane reads tile row perm(lane % 32), dims
  // 16 ks + 8 half .. + 7
  const int a_row = perm_row(lane & 31);
  const int a_off = a_row * kRowElems + 8 * half;
  // rope columns of that row: chunk 2 kc + half sits at slot
  // 8 row + ((2 kc + half) ^ x), x = bits 1..3 of the row; the XOR with 2 kc
  // only touches bits 4..5 of the element offset
  const int a_rope = kRopeElems + 64 * a_row + 8 * (half ^ ((a_row >> 1) & 7));
  const int c_wave = kDvWave * wave;  // first value column of this wave
  auto a_operand = [&](const uint16_t* tile, int ks) {
    const int off = ks < kKSLat ? a_off + 16 * ks : a_rope ^ (16 * (ks - kKSLat));
    return as_bf16x8(*(const u32x4*)(tile + off));
  };

  f32x16 o[kHB][kDVB];
  float m_base = -INFINITY, m_seen = -INFINITY, l_run = 0.f;

  // weights of tokens 16 ks + 8 half .. + 7 of head `head` (fp16, packed)
  auto weights_half = [&](const f32x16& sv, int ks, float& psum) {
    // before the first kept row the base is still -inf: every weight is 0
    const float m_use = m_base == -INFINITY ? 0.f : m_base;
    u32x4 ph;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = __builtin_amdgcn_exp2f(sv[8 * ks + 2 * w] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(sv[8 * ks + 2 * w + 1] - m_use);
      psum += p0 + p1;
      ph[w] = pack_f16x2(p0, p1);
    }
    return ph;
  };
  // token half ks of head `head` is chunk 2 ks + half of its P row
  auto store_p = [&](uint16_t* pw, const u32x4& ph0, const u32x4& ph1) {
    *(u32x4*)(pw + p_offset(head, half)) = ph0;
    *(u32x4*)(pw + p_offset(head, 2 + half)) = ph1;
  };
  // O^T += V^T P^T for token half ks of a tile: this wave's 128 value
  // columns, all 128 heads, fp16 operands: bp holds the P^T operands of the
  // 4 head blocks; per value block one transposed V^T read, converted to
  // fp16, serves 4 products.
  auto pv_ops = [&](const uint16_t* tile, const f16x8* bp, int ks) {
    u32x4 va = load_vt32(tile, c_wave, ks, lane);
#pragma unroll
    for (int d = 0; d < kDVB; ++d) {
      const f16x8 vcur = bf16x8_to_f16x8(va);
      if (d + 1 < kDVB) va = load_vt32(tile, c_wave + 32 * (d + 1), ks, lane);
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) o[hb][d] = mfma32_f16(vcur, bp[hb], o[hb][d]);
    }
  };

  constexpr float kMaxExp = 15.f;  // weights stay below 2^15 (fp16 range)
  bool redo = false;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (!__syncthreads_or(redo)) break;
      m_base = m_seen;
    }
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb)
#pragma unroll
      for (int d = 0; d < kDVB; ++d) o[hb][d] = f32x16{};
    l_run = 0.f;
    if (t_begin < t_end) {
      load_begin(t_begin, 0);
#pragma unroll
      for (int i = 0; i < kWaveBlocks; ++i) load_block(i);
    }

    // The products of "tile t_begin - 1" read a zeroed V region and zeroed
    // weights (they add exactly 0), and the last iteration's weights come
    // from S = -inf and are dropped, so that the weights of tile t and the
    // products of tile t - 1 run as one block in every iteration.
    {
      uint32_t* zv = (uint32_t*)tiles[kBufs - 1];
      for (int i = threadIdx.x; i < kLatRegion / 4; i += kThreads) zv[i] = 0u;
      uint32_t* zp = (uint32_t*)pbuf[1];
      for (int i = threadIdx.x; i < kPElems / 2; i += kThreads) zp[i] = 0u;
    }
    for (int t = t_begin; t <= t_end && t_begin < t_end; ++t) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t has landed (this wave's part)
      __syncthreads();  // ... all of it; P(t - 1) is written; tile t - 2 and P(t - 2) are free
      const bool have_s = t < t_end;
      const bool next = t + 1 < t_end;
      if (next) load_begin(t + 1, (t + 1 - t_begin) % kBufs);

      f32x16 s;  // S^T of tile t: head `head`, tokens acc_token(v, half)
      if (have_s) {
        const uint16_t* tile = tiles[(t - t_begin) % kBufs];
        constexpr int kDepthS = 2, kRingS = kDepthS + 2;
        bf16x8 ar[kRingS];
#pragma unroll
        for (int jj = 0; jj < kDepthS; ++jj) ar[jj] = a_operand(tile, jj);
#pragma unroll
        for (int ks = 0; ks < kKS; ++ks) {
          if (ks == 0)
            mfma32_vgpr_first(s, ar[0], qf[0]);
          else
            mfma32_vgpr(s, ar[ks % kRingS], qf[ks]);
          if (ks + kDepthS < kKS)
            ar[(ks + kDepthS) % kRingS] = a_operand(tile, ks + kDepthS);
          if (next && ks < kWaveBlocks) load_block(ks);
        }
        mfma_result_fence(s);
        // logits in the exp2 domain before the maximum is taken, so that any
        // finite scale (zero and negative ones included) gives the true
        // maximum; masked slots become -inf after scaling (weight 0)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] *= scale_log2;
        const uint32_t vm = tvalid[t - t_begin];
        if (vm != 0xffffffffu) {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (!((vm >> acc_token(v, half)) & 1u)) s[v] = -INFINITY;
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[v] = -INFINITY;  // past the last tile: weights 0
      }
      float mt = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) mt = fmaxf(mt, s[v]);
      mt = halves_max(mt);
      if (have_s && m_base == -INFINITY) m_base = mt;
      if (have_s) m_seen = fmaxf(m_seen, mt);
      redo |= have_s && mt > m_base + kMaxExp;

      const uint16_t* v_tile = tiles[(t + kBufs - 1 - t_begin) % kBufs];
      const uint16_t* pr = pbuf[(t + 1 - t_begin) & 1];
      uint16_t* pw = pbuf[(t - t_begin) & 1];
      {
        // P(t - 1) operands are read, and this tile's weights stored, outside
        // the products, so that no LDS write sits between them
        f16x8 bp0[kHB], bp1[kHB];
#pragma unroll
        for (int hb = 0; hb < kHB; ++hb) {
          bp0[hb] = as_f16x8(*(const u32x4*)(pr + p_offset(32 * hb + (lane & 31), half)));
          bp1[hb] = as_f16x8(*(const u32x4*)(pr + p_offset(32 * hb + (lane & 31), 2 + half)));
        }
        float psum = 0.f;
        const u32x4 ph0 = weights_half(s, 0, psum);
        const u32x4 ph1 = weights_half(s, 1, psum);
        const float tsum = halves_sum(psum);
        if (have_s) l_run += tsum;
        pv_ops(v_tile, bp0, 0);
        pv_ops(v_tile, bp1, 1);
        store_p(pw, ph0, ph1);
      }
    }
  }

  // ---- epilogue.  Head statistics go through LDS from their owners to the
  // waves holding the value columns.
  const float lse_val = l_run > 0.f ? (m_base + __log2f(l_run)) * kLn2 : -INFINITY;
  if (half == 0) {
    head_l[head] = l_run;
    head_lse[head] = lse_val;
  }
  __syncthreads();
  // Lane holds head 32 hb + lane % 32 and value columns
  // c_wave + 32 d + 8 (v / 4) + 4 half + v % 4.  The normalised rows go out
  // through LDS (the tile buffers are free now), 64 heads at a time, so that
  // every global store writes whole 1 KB rows: written straight from the
  // accumulator layout, each store instruction would touch 32 rows with 16
  // bytes each.  The final output is bf16; split partials are fp16 (11
  // significant bits: half the bytes of fp32 to write here and to read in the
  // merge).
  const bool final_out = n_splits == 1;
  uint16_t* const dst = final_out
                            ? out + (int64_t)qi * kHeads * kDv
                            : part_o + ((int64_t)qi * n_splits + split) * kHeads * kDv;
  constexpr int kStageRow = kDv + 8;  // elements: 1040-byte rows
  constexpr int kStageHeads = 64;
  static_assert(kStageHeads * kStageRow * 2 <= kBufs * kBufBytes, "stage fits the tile buffers");
  uint16_t* const stage = &tiles[0][0];
  // a fresh copy of the thread index: otherwise the compiler keeps the
  // prologue's thread-index sums alive across the tile loop (spilled to
  // scratch, and reloaded between the stores below, each reload waiting for
  // every store before it)
  int tid = (int)threadIdx.x;
  asm volatile("" : "+v"(tid));
#pragma unroll
  for (int r = 0; r < kHeads / kStageHeads; ++r) {
    if (r > 0) __syncthreads();  // the previous round's rows have been read out
#pragma unroll
    for (int hh = 0; hh < kStageHeads / 32; ++hh) {
      const int hb = (kStageHeads / 32) * r + hh;
      const int h = 32 * hb + (lane & 31);
      const float lh = head_l[h];
      const float inv_l = lh > 0.f ? 1.f / lh : 0.f;
      uint16_t* srow = stage + (h - kStageHeads * r) * kStageRow + c_wave + 4 * half;
#pragma unroll
      for (int d = 0; d < kDVB; ++d)
#pragma unroll
        for (int bq = 0; bq < 4; ++bq) {
          const float x0 = o[hb][d][4 * bq] * inv_l, x1 = o[hb][d][4 * bq + 1] * inv_l;
          const float x2 = o[hb][d][4 * bq + 2] * inv_l, x3 = o[hb][d][4 * bq + 3] * inv_l;
          *(uint2*)(srow + 32 * d + 8 * bq) =
              final_out ? make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3))
                        : make_uint2(pack_f16x2(x0, x1), pack_f16x2(x2, x3));
        }
    }
    __syncthreads();
    constexpr int kChunks = kDv / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < kStageHeads * kChunks / kThreads; ++i) {
      const int flat = kThreads * i + tid;
      const int row = flat / kChunks, ch = flat % kChunks;
      const u32x4 val = *(const u32x4*)(stage + row * kStageRow + 8 * ch);
      *(u32x4*)(dst + (int64_t)(kStageHeads * r + row) * kDv + 8 * ch) = val;
    }
  }
  if (final_out) {
    if (lse && half == 0) lse[(int64_t)qi * kHeads + head] = lse_val;
  } else if (half == 0) {
    part_lse[((int64_t)qi * n_splits + split) * kHeads + head] = lse_val;
  }
}

// Log-sum-exp merge of the split partials (fp16 O, fp32 lse) for up to NS
// splits: one wave per (query, head), lane l owns value columns 8 l ..
// 8 l + 7 (one 16-byte load per split, one 16-byte bf16 store); every load
// of a wave is issued before the first use, so the merge of a head costs
// one memory round trip.
template <int NS>
__global__ __launch_bounds__(256) void latent_combine_kernel(const uint16_t* __restrict__ part_o,
                                                             const float* __restrict__ part_lse,
                                                             int n_splits, int n_qh,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
  static_assert(kDv == 8 * kWave, "a lane owns 8 value columns");
  const int qh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  if (qh >= n_qh) return;
  const int qi = qh / kHeads, head = qh % kHeads;
  const int lane = threadIdx.x & (kWave - 1);
  // unconditional loads (slots past n_splits repeat the last split and get
  // weight 0): no branch between the loads
  float l[NS];
  u32x4 v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int64_t p = ((int64_t)qi * n_splits + min(s, n_splits - 1)) * kHeads + head;
    l[s] = part_lse[p];
    v[s] = *(const u32x4*)(part_o + p * kDv + 8 * lane);
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) m = fmaxf(m, l[s]);
  float acc[8] = {}, wsum = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const float wgt = s >= n_splits || l[s] == -INFINITY ? 0.f : __expf(l[s] - m);
    wsum += wgt;
    const f16x8 x = as_f16x8(v[s]);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += wgt * (float)x[i];
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i] * inv, acc[2 * i + 1] * inv);
  *(u32x4*)(out + (int64_t)qh * kDv + 8 * lane) = o;
  if (lse && lane == 0) lse[qh] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

}  // namespace latent
}  // namespace

uint32_t take_bounds_error_latent(hipStream_t stream) { return take_bounds_error(stream); }

void launch_latent(const dsa_paged_cache_t* c, const uint16_t* q, const int32_t* idx, int n_q,
                   int K, AttnQuery aq, float sm_scale, uint16_t* out, float* lse,
                   uint16_t* part_o, float* part_lse, SplitPlan plan, hipStream_t stream) {
  const int64_t blocks = ((int64_t)n_q + 7) / 8 * 8 * plan.n_splits;
  hipLaunchKernelGGL(latent::sparse_attn_latent_kernel, dim3((unsigned)blocks),
                     dim3(latent::kThreads), 0, stream, c->kv, c->kv_row_stride, c->block_table,
                     c->max_blocks_per_seq, c->block_size, q, idx, n_q, K, aq,
                     plan.tiles_per_split, sm_scale * kLog2e, out, lse, part_o, part_lse,
                     plan.n_splits);
  if (plan.n_splits <= 1) return;
  const int n_qh = n_q * latent::kHeads;
  const dim3 grid((unsigned)((n_qh + 3) / 4)), block(256);
  if (plan.n_splits <= 4)
    hipLaunchKernelGGL(latent::latent_combine_kernel<4>, grid, block, 0, stream, part_o, part_lse,
                       plan.n_splits, n_qh, out, lse);
  else if (plan.n_splits <= 8)
    hipLaunchKernelGGL(latent::latent_combine_kernel<8>, grid, block, 0, stream, part_o, part_lse,
                       plan.n_splits, n_qh, out, lse);
  else if (plan.n_splits <= 16)
    hipLaunchKernelGGL(latent::latent_combine_kernel<16>, grid, block, 0, stream, part_o,
                       part_lse, plan.n_splits, n_qh, out, lse);
  else
    hipLaunchKernelGGL((attn_combine_kernel<latent::kDv, uint16_t>), dim3(n_qh), dim3(128), 0,
                       stream, part_o, part_lse, plan.n_splits, latent::kHeads, out, lse);
}

}  // namespace dsa
