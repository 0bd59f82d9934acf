// Exact softmax attention over the kept positions only, reading K/V rows
// from a block-paged cache through the block table (web page "Day-0
// Adaptation of Trillion-Parameter MoE Models on Domestic GPUs", section 3:
// exact attention over the Top-K positions, item (2) paged layout with an
// index table, item (3) separate prefill and decode paths).
//
// One workgroup takes one query and a group of 16*NW heads; all heads share
// one K/V head (MQA, or the shared latent row where V is the first d_v
// columns of K), so each gathered K/V tile in LDS serves every head of the
// group.  Per tile of 32 kept positions:
//   gather:  32 rows go from HBM into an LDS K tile [token][d_qk] and a
//            transposed fp16 LDS V tile [d_v][token]; each lane moves
//            16-byte pieces of 8 rows and transposes the value part in
//            registers;
//   S^T = K Q^T   on MFMA 16x16x32 (A = K rows from LDS, B = q in registers;
//                 the result lane holds one head and 8 tokens, so softmax
//                 statistics need only two cross-lane steps);
//   online softmax in the log2 domain with fp32 statistics;
//   O^T += V^T P^T on MFMA (A = V^T from LDS, B = P^T straight from the S^T
//                 accumulators, so P never leaves registers; O^T's lane
//                 layout matches the per-head statistics, so rescaling needs
//                 no data movement).
// The P.V product runs in fp16, not bf16: bf16 values convert to fp16
// exactly (|v| < 65504; magnitudes below 2^-24 flush to zero), and the
// softmax weights in [0, 1] keep 11 significant bits instead of 8.  The
// normaliser is the sum of the rounded weights, so one kept position
// returns its V row exactly.
// Decode splits the kept positions of a query over several workgroups
// (split-K) and merges the partial results by log-sum-exp in a second
// kernel; prefill has enough queries to fill the chip without splitting.
#include <algorithm>

#include "common.h"
#include "host_util.h"

namespace dsa {
namespace {

constexpr int kTile = 32;  // kept positions per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Transpose an 8x8 block of bf16 into fp16: in[r] holds 8 consecutive bf16
// columns of row r; out[c] receives column c of rows 0..7 as fp16.
__device__ __forceinline__ void transpose8x8_to_f16(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = in[2 * p][w], b = in[2 * p + 1][w];
      o[p] = (c & 1) ? pack_f16x2(bf16_hi(a), bf16_hi(b)) : pack_f16x2(bf16_lo(a), bf16_lo(b));
    }
    out[c] = u32x4{o[0], o[1], o[2], o[3]};
  }
}

template <int NW, int D_QK, int D_V, bool SEP_V>
struct AttnCfg {
  static constexpr int kThreads = NW * kWave;
  static constexpr int kRow = D_QK + 8;    // K tile row (elements)
  static constexpr int kVtRow = kTile + 8;  // V^T tile row (elements)
  static constexpr int kKS = D_QK / 32;    // k-steps of S
  static constexpr int kDT = D_V / 16;     // 16-wide output tiles
  static constexpr int kKch = D_QK / 8;    // 16-byte chunks per K row
  static constexpr int kVch = D_V / 8;     // 16-byte chunks per V row
};

template <int NW, int D_QK, int D_V, bool SEP_V>
__global__ __launch_bounds__(NW * kWave) void sparse_attn_kernel(
    const uint16_t* __restrict__ kv, int64_t kv_stride, const uint16_t* __restrict__ vpool,
    int64_t v_stride, const int32_t* __restrict__ block_table, int max_blocks, int bs,
    const uint16_t* __restrict__ q, const int32_t* __restrict__ idx, int K, int H,
    const int32_t* __restrict__ seq_lens, int prefill_seq, int pos0, int tiles_per_split,
    float scale_log2, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ part_o, float* __restrict__ part_lse, int n_splits) {
  using C = AttnCfg<NW, D_QK, D_V, SEP_V>;
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kTile * C::kRow];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D_V * C::kVtRow];
  __shared__ int32_t trow[kTile];

  const int split = blockIdx.x;
  const int head0 = blockIdx.y * 16 * NW;
  const int qi = blockIdx.z;
  const bool decode = seq_lens != nullptr;
  const int seq = decode ? qi : prefill_seq;
  const int n_cand = decode ? seq_lens[qi] : pos0 + qi + 1;
  const int count = min(K, n_cand);
  const int32_t* bt_row = block_table + (int64_t)seq * max_blocks;
  const int32_t* sel = idx + (int64_t)qi * K;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15, grp = lane >> 4;
  const int head = head0 + 16 * wave + col;  // the head this lane's statistics belong to

  // q as the B operand of S^T: dims 32*ks + 8*grp .. +7 of this lane's head
  bf16x8 qf[C::kKS];
#pragma unroll
  for (int ks = 0; ks < C::kKS; ++ks) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (head < H) v = *(const u32x4*)(q + ((int64_t)qi * H + head) * D_QK + 32 * ks + 8 * grp);
    qf[ks] = as_bf16x8(v);
  }

  f32x4 o[C::kDT];
#pragma unroll
  for (int dt = 0; dt < C::kDT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (count + kTile - 1) / kTile;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);

  for (int t = t_begin; t < t_end; ++t) {
    const int base = t * kTile;
    if (threadIdx.x < kTile) {
      const int r = base + threadIdx.x;
      const int pos = r < count ? sel[r] : -1;
      trow[threadIdx.x] = pos >= 0 ? (int32_t)paged_row(bt_row, bs, pos) : -1;
    }
    __syncthreads();

    // ---- gather the tile into LDS
    for (int u = threadIdx.x; u < 4 * C::kKch; u += C::kThreads) {
      const int oct = u / C::kKch, ch = u % C::kKch;
      u32x4 r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int row = trow[8 * oct + j];
        r[j] = row >= 0 ? *(const u32x4*)(kv + (int64_t)row * kv_stride + 8 * ch)
                        : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) *(u32x4*)(ktile + (8 * oct + j) * C::kRow + 8 * ch) = r[j];
      if (!SEP_V && ch < C::kVch) {
        u32x4 c8[8];
        transpose8x8_to_f16(r, c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) *(u32x4*)(vt + (8 * ch + e) * C::kVtRow + 8 * oct) = c8[e];
      }
    }
    if (SEP_V) {
      for (int u = threadIdx.x; u < 4 * C::kVch; u += C::kThreads) {
        const int oct = u / C::kVch, ch = u % C::kVch;
        u32x4 r[8], c8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int row = trow[8 * oct + j];
          r[j] = row >= 0 ? *(const u32x4*)(vpool + (int64_t)row * v_stride + 8 * ch)
                          : u32x4{0u, 0u, 0u, 0u};
        }
        transpose8x8_to_f16(r, c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) *(u32x4*)(vt + (8 * ch + e) * C::kVtRow + 8 * oct) = c8[e];
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T.  Tile tt, A row m reads token 8*(m/4) + 4*tt + m%4,
    // so the result lane (head, grp) holds tokens 8*grp + 4*tt + i.
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int tok = 8 * (col >> 2) + 4 * tt + (col & 3);
      const uint16_t* krow = ktile + tok * C::kRow + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < C::kKS; ++ks)
        s[tt] = mfma16x16x32(as_bf16x8(*(const u32x4*)(krow + 32 * ks)), qf[ks], s[tt]);
    }

    // ---- online softmax (log2 domain); masked tokens contribute nothing
    float x[8];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool valid = trow[8 * grp + j] >= 0;
      x[j] = valid ? s[j >> 2][j & 3] * scale_log2 : -INFINITY;
      mt = fmaxf(mt, x[j]);
    }
    mt = wave_max_xor_16_32(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      pk[j >> 1] = pack_f16x2(__builtin_amdgcn_exp2f(x[j] - m_use),
                              __builtin_amdgcn_exp2f(x[j + 1] - m_use));
      // normalise by the weights as they enter the product
      psum += f16_bits_to_float(pk[j >> 1] & 0xffffu) + f16_bits_to_float(pk[j >> 1] >> 16);
    }
    psum = wave_sum_xor_16_32(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    const f16x8 pf = as_f16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});

    // ---- O^T = alpha * O^T + V^T P^T
    const uint16_t* vrow = vt + col * C::kVtRow + 8 * grp;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
      o[dt] *= alpha;
      o[dt] = mfma16x16x32(as_f16x8(*(const u32x4*)(vrow + 16 * dt * C::kVtRow)), pf, o[dt]);
    }
    __syncthreads();
  }

  // ---- epilogue: lane holds head `head`, value dims 16*dt + 4*grp + i
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse_val = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
  if (head < H) {
    if (n_splits == 1) {
      uint16_t* orow = out + ((int64_t)qi * H + head) * D_V + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
        const uint32_t lo = pack_bf16x2(o[dt][0] * inv_l, o[dt][1] * inv_l);
        const uint32_t hi = pack_bf16x2(o[dt][2] * inv_l, o[dt][3] * inv_l);
        *(uint2*)(orow + 16 * dt) = make_uint2(lo, hi);
      }
      if (lse && grp == 0) lse[(int64_t)qi * H + head] = lse_val;
    } else {
      const int64_t pidx = ((int64_t)qi * n_splits + split) * H + head;
      float* prow = part_o + pidx * D_V + 4 * grp;
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt)
        *(f32x4*)(prow + 16 * dt) = o[dt] * inv_l;
      if (grp == 0) part_lse[pidx] = lse_val;
    }
  }
}

// Log-sum-exp merge of the split-K partial results: one workgroup per
// (query, head); each thread owns value dims.
template <int D_V>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           int n_splits, int H,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int qh = blockIdx.x;  // qi * H + head
  const int qi = qh / H, head = qh % H;
  float m = -INFINITY;
  for (int s = 0; s < n_splits; ++s)
    m = fmaxf(m, part_lse[((int64_t)qi * n_splits + s) * H + head]);
  float wsum = 0.f;
  float acc[D_V / 128 > 0 ? D_V / 128 : 1] = {};
  constexpr int kPer = D_V / 128 > 0 ? D_V / 128 : 1;
  for (int s = 0; s < n_splits; ++s) {
    const int64_t p = ((int64_t)qi * n_splits + s) * H + head;
    const float l = part_lse[p];
    const float wgt = l == -INFINITY ? 0.f : __expf(l - m);
    wsum += wgt;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int d = threadIdx.x + 128 * e;
      if (d < D_V) acc[e] += wgt * part_o[p * D_V + d];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int d = threadIdx.x + 128 * e;
    if (d < D_V) out[(int64_t)qh * D_V + d] = (uint16_t)f32_to_bf16_bits(acc[e] * inv);
  }
  if (lse && threadIdx.x == 0) lse[qh] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

// Split-K plan for decode: enough workgroups to cover the chip about twice.
struct SplitPlan {
  int n_splits, tiles_per_split;
};
inline SplitPlan plan_splits(int B, int head_groups, int K) {
  const int tiles = (K + kTile - 1) / kTile;
  int want = (512 + B * head_groups - 1) / (B * head_groups);
  want = std::max(1, std::min(want, tiles));
  const int tps = (tiles + want - 1) / want;
  return SplitPlan{(tiles + tps - 1) / tps, tps};
}

enum Family { kLatent, kSmall, kNone };

Family family_of(const dsa_paged_cache_t* c, int H) {
  if (H == 128 && c->d_qk == 576 && c->d_v == 512 && c->v == nullptr) return kLatent;
  if (H == 8 && c->d_qk == 64 && c->d_v == 64 && c->v != nullptr) return kSmall;
  return kNone;
}

dsa_status_t check_attn_args(const dsa_paged_cache_t* c, const uint16_t* q, const int32_t* idx,
                             int n_q, int H, int K, const uint16_t* out, Family* fam) {
  dsa_status_t st = check_cache_common(c);
  if (st != DSA_OK) return st;
  if (!c->kv || !q || !idx || !out) return DSA_ERR_NULL;
  if (n_q < 1 || H < 1 || K < 1 || K > 2048) return DSA_ERR_SHAPE;
  if (c->kv_row_stride < c->d_qk) return DSA_ERR_SHAPE;
  if (c->v && c->v_row_stride < c->d_v) return DSA_ERR_SHAPE;
  if (!c->v && c->d_v > c->d_qk) return DSA_ERR_SHAPE;
  *fam = family_of(c, H);
  if (*fam == kNone) return DSA_ERR_UNSUPPORTED;
  if (c->kv_row_stride % 8 != 0 || (c->v && c->v_row_stride % 8 != 0)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

template <int NW, int D_QK, int D_V, bool SEP_V>
void launch_attn(const dsa_paged_cache_t* c, const uint16_t* q, const int32_t* idx, int n_q, int H,
                 int K, const int32_t* seq_lens, int seq, int pos0, float sm_scale, uint16_t* out,
                 float* lse, float* part_o, float* part_lse, SplitPlan plan, hipStream_t stream) {
  const int head_groups = (H + 16 * NW - 1) / (16 * NW);
  hipLaunchKernelGGL((sparse_attn_kernel<NW, D_QK, D_V, SEP_V>),
                     dim3(plan.n_splits, head_groups, n_q), dim3(NW * kWave), 0, stream, c->kv,
                     c->kv_row_stride, c->v, c->v_row_stride, c->block_table,
                     c->max_blocks_per_seq, c->block_size, q, idx, K, H, seq_lens, seq, pos0,
                     plan.tiles_per_split, sm_scale * kLog2e, out, lse, part_o, part_lse,
                     plan.n_splits);
  if (plan.n_splits > 1)
    hipLaunchKernelGGL(attn_combine_kernel<D_V>, dim3(n_q * H), dim3(128), 0, stream, part_o,
                       part_lse, plan.n_splits, H, out, lse);
}

int head_groups_of(int H) { return H == 128 ? 2 : 1; }

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t K,
                                                         int32_t d_v) {
  using namespace dsa;
  if (B < 1 || H < 1 || K < 1 || d_v < 1) return 0;
  const SplitPlan p = plan_splits(B, head_groups_of(H), K);
  if (p.n_splits == 1) return 0;
  const size_t o = (size_t)B * p.n_splits * H * d_v * 4;
  return (o + 255) / 256 * 256 + (size_t)B * p.n_splits * H * 4;
}

extern "C" dsa_status_t dsa_sparse_attn_decode(const dsa_paged_cache_t* cache, const uint16_t* q,
                                               const int32_t* idx, int32_t B, int32_t H,
                                               int32_t K, float sm_scale, uint16_t* out,
                                               float* lse, void* workspace,
                                               size_t workspace_bytes, hipStream_t stream) {
  using namespace dsa;
  Family fam;
  dsa_status_t st = check_attn_args(cache, q, idx, B, H, K, out, &fam);
  if (st != DSA_OK) return st;
  if (!cache->seq_lens) return DSA_ERR_NULL;
  if (B != cache->n_seq) return DSA_ERR_SHAPE;
  const size_t need = dsa_sparse_attn_decode_workspace_size(B, H, K, cache->d_v);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  st = check_device();
  if (st != DSA_OK) return st;
  const SplitPlan plan = plan_splits(B, head_groups_of(H), K);
  float* part_o = (float*)workspace;
  float* part_lse = need ? (float*)((char*)workspace +
                                    ((size_t)B * plan.n_splits * H * cache->d_v * 4 + 255) / 256 * 256)
                         : nullptr;
  if (fam == kLatent)
    launch_attn<4, 576, 512, false>(cache, q, idx, B, H, K, cache->seq_lens, 0, 0, sm_scale, out,
                                    lse, part_o, part_lse, plan, stream);
  else
    launch_attn<1, 64, 64, true>(cache, q, idx, B, H, K, cache->seq_lens, 0, 0, sm_scale, out,
                                 lse, part_o, part_lse, plan, stream);
  return launch_status();
}

extern "C" dsa_status_t dsa_sparse_attn_prefill(const dsa_paged_cache_t* cache,
                                                const uint16_t* q, const int32_t* idx, int32_t T,
                                                int32_t H, int32_t K, int32_t seq, int32_t pos0,
                                                float sm_scale, uint16_t* out, float* lse,
                                                hipStream_t stream) {
  using namespace dsa;
  Family fam;
  dsa_status_t st = check_attn_args(cache, q, idx, T, H, K, out, &fam);
  if (st != DSA_OK) return st;
  if (seq < 0 || seq >= cache->n_seq || pos0 < 0) return DSA_ERR_SHAPE;
  if ((int64_t)pos0 + T > (int64_t)cache->max_blocks_per_seq * cache->block_size)
    return DSA_ERR_SHAPE;
  st = check_device();
  if (st != DSA_OK) return st;
  const SplitPlan one{1, (K + kTile - 1) / kTile};
  if (fam == kLatent)
    launch_attn<4, 576, 512, false>(cache, q, idx, T, H, K, nullptr, seq, pos0, sm_scale, out,
                                    lse, nullptr, nullptr, one, stream);
  else
    launch_attn<1, 64, 64, true>(cache, q, idx, T, H, K, nullptr, seq, pos0, sm_scale, out, lse,
                                 nullptr, nullptr, one, stream);
  return launch_status();
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
  }
  return "unknown status";
}
