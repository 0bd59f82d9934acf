// Internal pieces shared by the two attention kernels (the latent-row
// kernel and the small MQA kernel): tile size, constants, the split-K plan
// and the log-sum-exp merge of split partial results.
#pragma once

#include <algorithm>

#include "common.h"

namespace dsa {

constexpr int kTile = 32;  // kept positions per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4i16 __attribute__((ext_vector_type(4)));

// The queries of an attention call.  Decode: query i is the last cached
// token of sequence i (seq_lens[i] candidates).  Prefill: query i belongs to
// sequence q_seq[i] at position q_pos[i] (q_pos[i] + 1 candidates).  Debug
// builds check both against the cache description and give a query outside
// it no candidates.
struct AttnQuery {
  const int32_t* seq_lens;  // decode, else NULL
  const int32_t* q_seq;     // prefill, else NULL
  const int32_t* q_pos;     // prefill, else NULL
  int n_seq, max_pos, num_blocks;
  __device__ __forceinline__ bool decode() const { return seq_lens != nullptr; }
  __device__ __forceinline__ int seq(int i) const {
    const int b = q_seq ? q_seq[i] : i;
    if (kCheckBounds && (b < 0 || b >= n_seq)) return 0;
    return b;
  }
  __device__ __forceinline__ int count(int i) const {
    const int n = q_pos ? q_pos[i] + 1 : seq_lens[i];
    if (kCheckBounds) {
      const int b = q_seq ? q_seq[i] : i;
      if (b < 0 || b >= n_seq || n < 0 || n > max_pos) {
        raise_error(q_pos ? kErrQuery : kErrLength);
        return 0;
      }
    }
    return n;
  }
  // A kept index of a row with n candidates (debug builds: one at or past n
  // is skipped).
  __device__ __forceinline__ int kept(int pos, int n) const {
    if (kCheckBounds && pos >= n) {
      raise_error(kErrIndex);
      return -1;
    }
    return pos;
  }
};

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

// Latent rows: one workgroup per CU; split each query's kept rows so that
// about 256 workgroups run.
inline SplitPlan plan_splits_latent(int B, int K) {
  const int tiles = (K + kTile - 1) / kTile;
  // about one workgroup per CU, but at least 4 tiles a split: a split's
  // fixed cost (its q and row lookups, its partial result) is worth ~2 tiles
  int want = (256 + B - 1) / B;
  want = std::max(1, std::min(want, std::max(1, tiles / 4)));
  const int tps = (tiles + want - 1) / want;
  return SplitPlan{(tiles + tps - 1) / tps, tps};
}

namespace {

// Four consecutive partial values as fp32: from fp32 partials, or from fp16
// ones (8 bytes).
__device__ __forceinline__ f32x4 load_part4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load_part4(const uint16_t* p) {
  const uint2 u = *(const uint2*)p;
  const f16x2 a = __builtin_bit_cast(f16x2, u.x), b = __builtin_bit_cast(f16x2, u.y);
  return f32x4{(float)a[0], (float)a[1], (float)b[0], (float)b[1]};
}

// Log-sum-exp merge of the split-K partial results: one workgroup per
// (query, head); thread t owns value dims 4 t .. 4 t + 3 (16-byte loads of
// fp32 partials or 8-byte loads of fp16 ones, 8-byte stores), looping when
// D_V > 4 * 128.
template <int D_V, typename PT>
__global__ __launch_bounds__(128) void attn_combine_kernel(const PT* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           int n_splits, int H,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse) {
  static_assert(D_V % 4 == 0, "value width must be a multiple of 4");
  constexpr int kPer = (D_V / 4 + 127) / 128;
  const int qh = blockIdx.x;  // qi * H + head
  const int qi = qh / H, head = qh % H;
  float m = -INFINITY;
  float wsum = 0.f;
  f32x4 acc[kPer] = {};
  constexpr int kMaxS = 16;
  if (n_splits <= kMaxS) {
    // every load of the workgroup goes out at once: one memory round trip
    float l[kMaxS];
    f32x4 v[kMaxS][kPer];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      if (s < n_splits) {
        const int64_t p = ((int64_t)qi * n_splits + s) * H + head;
        l[s] = part_lse[p];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          const int d = 4 * (threadIdx.x + 128 * e);
          v[s][e] = d < D_V ? load_part4(part_o + p * D_V + d) : f32x4{};
        }
      }
    }
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      if (s < n_splits) m = fmaxf(m, l[s]);
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      if (s < n_splits) {
        const float wgt = l[s] == -INFINITY ? 0.f : __expf(l[s] - m);
        wsum += wgt;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] += wgt * v[s][e];
      }
    }
  } else {
    for (int s = 0; s < n_splits; ++s)
      m = fmaxf(m, part_lse[((int64_t)qi * n_splits + s) * H + head]);
    for (int s = 0; s < n_splits; ++s) {
      const int64_t p = ((int64_t)qi * n_splits + s) * H + head;
      const float l = part_lse[p];
      const float wgt = l == -INFINITY ? 0.f : __expf(l - m);
      wsum += wgt;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int d = 4 * (threadIdx.x + 128 * e);
        if (d < D_V) acc[e] += wgt * load_part4(part_o + p * D_V + d);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int d = 4 * (threadIdx.x + 128 * e);
    if (d < D_V)
      *(uint2*)(out + (int64_t)qh * D_V + d) =
          make_uint2(pack_bf16x2(acc[e][0] * inv, acc[e][1] * inv),
                     pack_bf16x2(acc[e][2] * inv, acc[e][3] * inv));
  }
  if (lse && threadIdx.x == 0) lse[qh] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

}  // namespace

// Launches the latent-row kernel (128 heads on a 576-wide row, V = its
// first 512 columns), and the split merge when plan.n_splits > 1.
__attribute__((visibility("hidden"))) void launch_latent(const dsa_paged_cache_t* c,
                                                        const uint16_t* q, const int32_t* idx,
                                                        int n_q, int K, AttnQuery aq,
                                                        float sm_scale, uint16_t* out, float* lse,
                                                        uint16_t* part_o, float* part_lse,
                                                        SplitPlan plan, hipStream_t stream);
__attribute__((visibility("hidden"))) uint32_t take_bounds_error_latent(hipStream_t stream);

}  // namespace dsa
