// Exact softmax attention over the kept positions only, reading K/V rows
// from a block-paged cache through the block table (web page "Day-0
// Adaptation of Trillion-Parameter MoE Models on Domestic GPUs", section 3:
// exact attention over the Top-K positions, item (2) paged layout with an
// index table, item (3) separate prefill and decode paths).
//
// This file holds the kernel for small multi-query heads (heads sharing one
// K/V head with separate K and V pools, d = 64) and the entry points of both
// attention calls; rows of the 576-wide latent shape go to the kernel in
// sparse_attn_latent.hip.
//
// One workgroup takes one query and a group of 16*NW heads; all heads share
// one K/V head, so each gathered tile in LDS serves every head of the group.
// Per tile of 32 kept positions:
//   gather:  32 rows go from HBM into an LDS K tile [token][d_qk] (bf16);
//            the loads of tile t+1 are in flight in registers while tile t
//            computes;
//   S^T = K Q^T   on MFMA 16x16x32 (A = K rows from LDS, B = q in registers;
//                 the result lane holds one head and 8 tokens, so softmax
//                 statistics need only two cross-lane steps);
//   online softmax in the log2 domain with fp32 statistics;
//   O^T += V^T P^T on MFMA (A = V^T read straight from the row-major tile
//                 with the gfx950 LDS transpose load, B = P^T
//                 straight from the S^T accumulators, so P never leaves
//                 registers; O^T's lane layout matches the per-head
//                 statistics, so rescaling needs no data movement).
// P enters the product as two bf16 MFMAs, P = P_hi + P_lo, which carries
// 16 significant bits of each weight: the remaining error is the rounding of
// the output to bf16.
// Decode splits the kept positions of a query over several workgroups
// (split-K) and merges the partial results by log-sum-exp in a second
// kernel; prefill has enough queries to fill the chip without splitting.
#include <algorithm>

#include <cmath>
#include <mutex>

#include "attn_common.h"
#include "host_util.h"

namespace dsa {
namespace {

// A 16x32 bf16 operand of V^T (rows: 16 value columns from dv0, k: tokens
// 8*grp .. 8*grp+7) read from a row-major [token][column] LDS tile with two
// transpose loads.  Within each group of 16 lanes, lane i names the 4
// values V[t0 + i/4][dv0 + 4*(i%4) .. +3]; the hardware hands lane j the
// values V[t0 .. t0+3][dv0 + j], i.e. 4 consecutive tokens of one column.
__device__ __forceinline__ bf16x8 load_vt_operand(const uint16_t* tile, int row_elems, int dv0,
                                                  int col, int grp) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const uint16_t* p0 = tile + (8 * grp + (col >> 2)) * row_elems + dv0 + 4 * (col & 3);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * row_elems));
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  return as_bf16x8(u32x4{ua.x, ua.y, ub.x, ub.y});
}

template <int HB, int D_QK, int D_V, bool SEP_V>
struct AttnCfg {
  // HB blocks of 16 heads; two waves (a pair) per head block.
  static constexpr int kWaves = 2 * HB;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kRow = D_QK + 8;    // K tile row (elements): the 16-byte pad keeps
                                           // row reads and transpose loads conflict-free
  static constexpr int kVRow = D_V + 8;    // V tile row (separate V pool only)
  static constexpr int kKS = D_QK / 32;    // k-steps of S
  static constexpr int kDTH = D_V / 32;    // 16-wide output tiles per wave (half of d_v)
  static constexpr int kKch = D_QK / 8;    // 16-byte chunks per K row
  static constexpr int kVch = D_V / 8;     // 16-byte chunks per V row
  // Loading plan of one tile: 16-byte chunks, consecutive threads on
  // consecutive chunks of a row.
  static constexpr int kKChunks = kTile * kKch;
  static constexpr int kVChunks = SEP_V ? kTile * kVch : 0;
  static constexpr int kKC = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVC = SEP_V ? (kVChunks + kThreads - 1) / kThreads : 1;
  static constexpr int kMaxTiles = 2048 / kTile;  // K <= 2048
};

// Registers holding one tile's gathered chunks between the global loads and
// the LDS stores, so the loads of tile t+1 fly while tile t computes.
template <class C>
struct Staged {
  u32x4 k[C::kKC];
  u32x4 v[C::kVC];
};

// Work item of a workgroup: which query, head group and split.  Blocks are
// dealt to the 8 XCDs round-robin by block id; every block of one query
// gets the same block id modulo 8, so the K/V rows one head group pulls in
// are L2 hits for the other.
struct AttnItem {
  int qi, hg, split;
};
__device__ __forceinline__ AttnItem attn_item(int n_q, int head_groups, int n_splits) {
  const int per_query = head_groups * n_splits;
  const int b = blockIdx.x;
  const int xcd = b & 7, j = b >> 3;
  const int sub = j % per_query;
  return AttnItem{(j / per_query) * 8 + xcd, sub % head_groups, sub / head_groups};
}

// Work split inside a workgroup.  Wave w serves head block hb = w % HB and
// tile half h = w / HB.  For S the pair (hb, 0), (hb, 1) splits the 32
// tokens of a tile (16 each); the pair then swaps per-head maxima and its
// halves of P through LDS, and for O each wave of the pair takes one half
// of the d_v value columns with all 32 tokens.  Two waves per SIMD hide each
// other's LDS and barrier latency, and each wave holds only half of O.
template <int HB, int D_QK, int D_V, bool SEP_V>
__global__ __launch_bounds__(2 * HB * kWave) void sparse_attn_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_stride, const uint16_t* __restrict__ vpool,
    int64_t v_stride, const int32_t* __restrict__ block_table, int max_blocks, int bs,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, int n_q, int K, int H,
    int head_groups, AttnQuery aq, int tiles_per_split, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int n_splits) {
  using C = AttnCfg<HB, D_QK, D_V, SEP_V>;
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kTile * C::kRow];
  __shared__ __attribute__((aligned(16))) uint16_t vtile[SEP_V ? kTile * C::kVRow : 8];
  __shared__ int32_t trows[C::kMaxTiles * kTile];  // physical rows of this block's range
  __shared__ float xmax[HB][2][16];                 // per-head maximum of each half tile
  __shared__ u32x4 xp[HB][2][kWave];                // P of each half tile: bf16 hi, lo

  const AttnItem it = attn_item(n_q, head_groups, n_splits);
  if (it.qi >= n_q) return;
  const int qi = it.qi, split = it.split;
  const int head0 = it.hg * 16 * HB;
  const int seq = aq.seq(qi);
  const int n_cand = aq.count(qi);
  const int count = min(K, n_cand);
  const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
  const int32_t* sel = idx + (int64_t)qi * K;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int hb = wave % HB, half = wave / HB;
  const int col = lane & 15, grp = lane >> 4;
  const int head = head0 + 16 * hb + col;  // the head this lane's statistics belong to

  const int n_tiles = (count + kTile - 1) / kTile;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);

  // physical pool rows of every kept position of this block (-1: none)
  for (int r = threadIdx.x; r < (t_end - t_begin) * kTile; r += C::kThreads) {
    const int g = t_begin * kTile + r;
    const int pos = g < count ? aq.kept(sel[g], n_cand) : -1;
    trows[r] = pos >= 0 ? (int32_t)paged_row(bt_row, bs, pos, aq.num_blocks) : -1;
  }

  // q as the B operand of S^T: dims 32*ks + 8*grp .. +7 of this lane's head
  bf16x8 qf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (head < H) v = *(const u32x4*)(q + ((int64_t)qi * H + head) * D_QK + 32 * ks + 8 * grp);
    qf[ks] = as_bf16x8(v);
  }

  // Per-thread chunk coordinates (the same for every tile).
  int k_row[C::kKC], k_off[C::kKC], v_row[C::kVC], v_off[C::kVC];
#pragma unroll
  for (int c = 0; c < C::kKC; ++c) {
    const int i = threadIdx.x + c * C::kThreads;
    k_row[c] = i < C::kKChunks ? i / C::kKch : -1;
    k_off[c] = 8 * (i % C::kKch);
  }
#pragma unroll
  for (int c = 0; c < C::kVC; ++c) {
    const int i = threadIdx.x + c * C::kThreads;
    v_row[c] = SEP_V && i < C::kVChunks ? i / C::kVch : -1;
    v_off[c] = 8 * (i % C::kVch);
  }
  __syncthreads();

  // Gather loads are branch-free: a padded slot reads pool row 0 (always
  // present) and its data is replaced by zeros.
  Staged<C> st;
  auto load_tile = [&](int t) {
    const int32_t* tr = trows + (t - t_begin) * kTile;
#pragma unroll
    for (int c = 0; c < C::kKC; ++c) {
      const int row = k_row[c] >= 0 ? tr[k_row[c]] : -1;
      const u32x4 v = *(const u32x4*)(kv + (int64_t)max(row, 0) * kv_stride + k_off[c]);
      st.k[c] = row >= 0 ? v : u32x4{0u, 0u, 0u, 0u};
    }
    if (SEP_V) {
#pragma unroll
      for (int c = 0; c < C::kVC; ++c) {
        const int row = v_row[c] >= 0 ? tr[v_row[c]] : -1;
        const u32x4 v = *(const u32x4*)(vpool + (int64_t)max(row, 0) * v_stride + v_off[c]);
        st.v[c] = row >= 0 ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int c = 0; c < C::kKC; ++c)
      if (k_row[c] >= 0) *(u32x4*)(ktile + k_row[c] * C::kRow + k_off[c]) = st.k[c];
    if (SEP_V) {
#pragma unroll
      for (int c = 0; c < C::kVC; ++c)
        if (v_row[c] >= 0) *(u32x4*)(vtile + v_row[c] * C::kVRow + v_off[c]) = st.v[c];
    }
  };

  f32x4 o[C::kDTH];
#pragma unroll
  for (int dt = 0; dt < C::kDTH; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile();
  }
  __syncthreads();

  const uint16_t* vsrc = SEP_V ? vtile : ktile;
  constexpr int kVStride = SEP_V ? C::kVRow : C::kRow;
  for (int t = t_begin; t < t_end; ++t) {
    if (t + 1 < t_end) load_tile(t + 1);  // in flight while this tile computes
    const int32_t* tr = trows + (t - t_begin) * kTile;

    // ---- S^T = K Q^T over this wave's half of the tile: A row m reads
    // token 8*(m/4) + 4*half + m%4, so the result lane (head, grp) holds
    // tokens 8*grp + 4*half + i.
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    {
      const uint16_t* krow = ktile + (8 * (col >> 2) + 4 * half + (col & 3)) * C::kRow + 8 * grp;
      constexpr int kDepth = 4;  // LDS operands in flight
      u32x4 a[kDepth];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) a[d] = *(const u32x4*)(krow + 32 * d);
#pragma unroll
      for (int ks = 0; ks < C::kKS; ++ks) {
        const u32x4 x0 = a[ks % kDepth];
        if (ks + kDepth < C::kKS) a[ks % kDepth] = *(const u32x4*)(krow + 32 * (ks + kDepth));
        s = mfma16x16x32(as_bf16x8(x0), qf[ks], s);
      }
    }

    // ---- online softmax (log2 domain); masked tokens contribute nothing.
    // The pair agrees on each head's maximum through LDS.  The exponent base
    // m_run moves only when a maximum exceeds it by more than kRebase, so
    // weights stay <= 2^kRebase and the O rescale is rare.
    float x[4];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = tr[8 * grp + 4 * half + i] >= 0;
      x[i] = valid ? s[i] * scale_log2 : -INFINITY;
      mt = fmaxf(mt, x[i]);
    }
    mt = wave_max_xor_16_32(mt);
    if (grp == 0) xmax[hb][half][col] = mt;
    __syncthreads();
    mt = fmaxf(xmax[hb][0][col], xmax[hb][1][col]);
    constexpr float kRebase = 8.f;
    if (m_run == -INFINITY) {
      m_run = mt;  // first tile with a kept position: O and l are still 0
    } else if (mt > m_run + kRebase) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mt);
      l_run *= alpha;
      m_run = mt;
#pragma unroll
      for (int dt = 0; dt < C::kDTH; ++dt) o[dt] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    // P = P_hi + P_lo, both bf16: the pair carries 16 significant bits of
    // each weight, so the weights add no error worth counting next to the
    // bf16 output.
    uint32_t ph[2], pl[2];
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(x[i] - m_use);
      const float p1 = __builtin_amdgcn_exp2f(x[i + 1] - m_use);
      ph[i >> 1] = pack_bf16x2(p0, p1);
      pl[i >> 1] = pack_bf16x2(p0 - bf16_lo(ph[i >> 1]), p1 - bf16_hi(ph[i >> 1]));
    }
    xp[hb][half][lane] = u32x4{ph[0], ph[1], pl[0], pl[1]};
    __syncthreads();
    // k-slot j of the P^T operand is token 8*grp + j: slots 0..3 from the
    // first half tile, 4..7 from the second.
    const u32x4 p0 = xp[hb][0][lane], p1 = xp[hb][1][lane];
    float psum = 0.f;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      psum += bf16_lo(p0[w]) + bf16_hi(p0[w]) + bf16_lo(p0[w + 2]) + bf16_hi(p0[w + 2]);
      psum += bf16_lo(p1[w]) + bf16_hi(p1[w]) + bf16_lo(p1[w + 2]) + bf16_hi(p1[w + 2]);
    }
    l_run += wave_sum_xor_16_32(psum);
    const bf16x8 pf_hi = as_bf16x8(u32x4{p0[0], p0[1], p1[0], p1[1]});
    const bf16x8 pf_lo = as_bf16x8(u32x4{p0[2], p0[3], p1[2], p1[3]});

    // ---- O^T += V^T P^T over this wave's half of the value columns
#pragma unroll
    for (int dt = 0; dt < C::kDTH; ++dt) {
      const bf16x8 va =
          load_vt_operand(vsrc, kVStride, (D_V / 2) * half + 16 * dt, col, grp);
      o[dt] = mfma16x16x32(va, pf_hi, o[dt]);
      o[dt] = mfma16x16x32(va, pf_lo, o[dt]);
    }
    __syncthreads();
    if (t + 1 < t_end) store_tile();
    __syncthreads();
  }

  // ---- epilogue: lane holds head `head`, value dims
  // (D_V/2)*half + 16*dt + 4*grp + i
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_val = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  if (head < H) {
    if (n_splits == 1) {
      uint16_t* orow = out + ((int64_t)qi * H + head) * D_V + (D_V / 2) * half + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < C::kDTH; ++dt) {
        const uint32_t lo = pack_bf16x2(o[dt][0] * inv_l, o[dt][1] * inv_l);
        const uint32_t hi = pack_bf16x2(o[dt][2] * inv_l, o[dt][3] * inv_l);
        *(uint2*)(orow + 16 * dt) = make_uint2(lo, hi);
      }
      if (lse && grp == 0 && half == 0) lse[(int64_t)qi * H + head] = lse_val;
    } else {
      const int64_t pidx = ((int64_t)qi * n_splits + split) * H + head;
      float* prow = part_o + pidx * D_V + (D_V / 2) * half + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < C::kDTH; ++dt) *(f32x4*)(prow + 16 * dt) = o[dt] * inv_l;
      if (grp == 0 && half == 0) part_lse[pidx] = lse_val;
    }
  }
}

enum Family { kLatent, kSmall, kNone };

Family family_of(const dsa_paged_cache_t* c, int H) {
  if (H == 128 && c->d_qk == 576 && c->d_v == 512 && c->v == nullptr) return kLatent;
  if (H == 8 && c->d_qk == 64 && c->d_v == 64 && c->v != nullptr) return kSmall;
  return kNone;
}

dsa_status_t check_attn_args(const dsa_paged_cache_t* c, const uint16_t* q, const int32_t* idx,
                             int n_q, int H, int K, float sm_scale, const uint16_t* out,
                             Family* fam) {
  dsa_status_t st = check_cache_common(c);
  if (st != DSA_OK) return st;
  if (!c->kv || !q || !idx || !out) return DSA_ERR_NULL;
  if (n_q < 1 || H < 1 || K < 1 || K > 2048) return DSA_ERR_SHAPE;
  if (!std::isfinite(sm_scale)) return DSA_ERR_SHAPE;
  if (c->kv_row_stride < c->d_qk) return DSA_ERR_SHAPE;
  if (c->v && c->v_row_stride < c->d_v) return DSA_ERR_SHAPE;
  if (!c->v && c->d_v > c->d_qk) return DSA_ERR_SHAPE;
  *fam = family_of(c, H);
  if (*fam == kNone) return DSA_ERR_UNSUPPORTED;
  if (c->kv_row_stride % 8 != 0 || (c->v && c->v_row_stride % 8 != 0)) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(c->kv) || (c->v && !aligned16(c->v)) || !aligned16(q) || !aligned16(out))
    return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

template <int HB, int D_QK, int D_V, bool SEP_V>
void launch_attn(const dsa_paged_cache_t* c, const uint16_t* q, const int32_t* idx, int n_q, int H,
                 int K, AttnQuery aq, float sm_scale, uint16_t* out, float* lse, float* part_o,
                 float* part_lse, SplitPlan plan, hipStream_t stream) {
  const int head_groups = (H + 16 * HB - 1) / (16 * HB);
  const int64_t blocks = ((int64_t)n_q + 7) / 8 * 8 * head_groups * plan.n_splits;
  hipLaunchKernelGGL((sparse_attn_kernel<HB, D_QK, D_V, SEP_V>), dim3((unsigned)blocks),
                     dim3(2 * HB * kWave), 0, stream, c->kv, c->kv_row_stride, c->v,
                     c->v_row_stride, c->block_table, c->max_blocks_per_seq, c->block_size, q,
                     idx, n_q, K, H, head_groups, aq, plan.tiles_per_split,
                     sm_scale * kLog2e, out, lse, part_o, part_lse, plan.n_splits);
  if (plan.n_splits > 1)
    hipLaunchKernelGGL((attn_combine_kernel<D_V, float>), dim3(n_q * H), dim3(128), 0, stream, part_o,
                       part_lse, plan.n_splits, H, out, lse);
}

int head_groups_of(int H) { return H == 128 ? 2 : 1; }

// Split plan of the decode call (also what sizes its workspace).
bool latent_shape(int H, int d_v) { return H == 128 && d_v == 512; }

SplitPlan decode_plan(int B, int H, int K, int d_v) {
  return latent_shape(H, d_v) ? plan_splits_latent(B, K) : plan_splits(B, head_groups_of(H), K);
}

// Bytes of the partial outputs in the workspace (256-byte rounded): fp16 for
// the latent family, fp32 for the other.
size_t part_o_bytes(int B, int H, int d_v, SplitPlan p) {
  const size_t elems = (size_t)B * p.n_splits * H * d_v;
  return (elems * (latent_shape(H, d_v) ? 2 : 4) + 255) / 256 * 256;
}

AttnQuery attn_query(const dsa_paged_cache_t* c, const int32_t* seq_lens, const int32_t* q_seq,
                     const int32_t* q_pos) {
  return AttnQuery{seq_lens, q_seq, q_pos, c->n_seq,
                   (int)std::min<int64_t>((int64_t)c->max_blocks_per_seq * c->block_size,
                                          0x7fffffff),
                   c->num_blocks};
}

uint32_t take_bounds_error_small(hipStream_t stream) { return take_bounds_error(stream); }

// Scratch of the allocation-free decode entry point: the split partials live
// in this file-scope device array (one copy per GPU, held until the process
// ends).  Host code uses the per-device address from hipGetSymbolAddress,
// never the array's name (a host-side stand-in).
constexpr size_t kStaticScratchBytes = (size_t)48 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on the first call on
// that device (with it current).
dsa_status_t static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t K,
                                                         int32_t d_v) {
  using namespace dsa;
  if (B < 1 || H < 1 || K < 1 || d_v < 1) return 0;
  const SplitPlan p = decode_plan(B, H, K, d_v);
  if (p.n_splits == 1) return 0;
  return part_o_bytes(B, H, d_v, p) + (size_t)B * p.n_splits * H * 4;
}

extern "C" dsa_status_t dsa_sparse_attn_decode(const dsa_paged_cache_t* cache, const uint16_t* q,
                                               const int32_t* idx, int32_t B, int32_t H,
                                               int32_t K, float sm_scale, uint16_t* out,
                                               float* lse, void* workspace,
                                               size_t workspace_bytes, hipStream_t stream) {
  using namespace dsa;
  Family fam;
  dsa_status_t st = check_attn_args(cache, q, idx, B, H, K, sm_scale, out, &fam);
  if (st != DSA_OK) return st;
  if (!cache->seq_lens) return DSA_ERR_NULL;
  if (B != cache->n_seq) return DSA_ERR_SHAPE;
  const size_t need = dsa_sparse_attn_decode_workspace_size(B, H, K, cache->d_v);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  const SplitPlan plan = decode_plan(B, H, K, cache->d_v);
  float* part_lse =
      need ? (float*)((char*)workspace + part_o_bytes(B, H, cache->d_v, plan)) : nullptr;
  const AttnQuery aq = attn_query(cache, cache->seq_lens, nullptr, nullptr);
  if (fam == kLatent)
    launch_latent(cache, q, idx, B, K, aq, sm_scale, out, lse, (uint16_t*)workspace, part_lse,
                  plan, stream);
  else
    launch_attn<1, 64, 64, true>(cache, q, idx, B, H, K, aq, sm_scale, out, lse,
                                 (float*)workspace, part_lse, plan, stream);
  return launch_status();
}

extern "C" dsa_status_t dsa_sparse_attn_decode_static(const dsa_paged_cache_t* cache,
                                                      const uint16_t* q, const int32_t* idx,
                                                      int32_t B, int32_t H, int32_t K,
                                                      float sm_scale, uint16_t* out, float* lse,
                                                      hipStream_t stream) {
  using namespace dsa;
  Family fam;
  dsa_status_t st = check_attn_args(cache, q, idx, B, H, K, sm_scale, out, &fam);
  if (st != DSA_OK) return st;
  if (!cache->seq_lens) return DSA_ERR_NULL;
  if (B != cache->n_seq) return DSA_ERR_SHAPE;
  const size_t need = dsa_sparse_attn_decode_workspace_size(B, H, K, cache->d_v);
  if (need > kStaticScratchBytes) return DSA_ERR_WORKSPACE;
  st = check_device();
  if (st != DSA_OK) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = static_scratch(&ws);
    if (st != DSA_OK) return st;
  }
  // every split writes all of its partial result (zeros / -inf for an
  // empty split), so nothing in the scratch needs clearing
  return dsa_sparse_attn_decode(cache, q, idx, B, H, K, sm_scale, out, lse, ws, need, stream);
}

extern "C" dsa_status_t dsa_sparse_attn_prefill(const dsa_paged_cache_t* cache,
                                                const uint16_t* q, const int32_t* q_seq,
                                                const int32_t* q_pos, const int32_t* idx,
                                                int32_t T, int32_t H, int32_t K, float sm_scale,
                                                uint16_t* out, float* lse, hipStream_t stream) {
  using namespace dsa;
  Family fam;
  dsa_status_t st = check_attn_args(cache, q, idx, T, H, K, sm_scale, out, &fam);
  if (st != DSA_OK) return st;
  if (!q_seq || !q_pos) return DSA_ERR_NULL;
  st = check_device();
  if (st != DSA_OK) return st;
  const SplitPlan one{1, (K + kTile - 1) / kTile};
  const AttnQuery aq = attn_query(cache, nullptr, q_seq, q_pos);
  if (fam == kLatent)
    launch_latent(cache, q, idx, T, K, aq, sm_scale, out, lse, nullptr, nullptr, one, stream);
  else
    launch_attn<1, 64, 64, true>(cache, q, idx, T, H, K, aq, sm_scale, out, lse, nullptr,
                                 nullptr, one, stream);
  return launch_status();
}

extern "C" dsa_status_t dsa_check_device_errors(hipStream_t stream) {
  using namespace dsa;
  if (!kCheckBounds) return DSA_ERR_UNSUPPORTED;
  const uint32_t e = take_bounds_error_small(stream) | take_bounds_error_latent(stream) |
                     take_bounds_error_index_score(stream) | take_bounds_error_topk(stream) |
                     take_bounds_error_cache_write(stream) | take_bounds_error_moe(stream);
  if (e & 0x80000000u) return DSA_ERR_HIP;
  return e ? DSA_ERR_BOUNDS : DSA_OK;
}

extern "C" const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "a size or stride is out of range or inconsistent";
    case DSA_ERR_UNSUPPORTED: return "no kernel for this head count or width";
    case DSA_ERR_WORKSPACE: return "workspace is missing or smaller than required";
    case DSA_ERR_DEVICE: return "the current device is not a usable gfx950";
    case DSA_ERR_HIP: return "a HIP launch failed";
    case DSA_ERR_BOUNDS: return "device data out of range (block table, lengths, positions or indices)";
  }
  return "unknown status";
}
