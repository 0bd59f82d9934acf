// Indexer scoring for DSA (web page "Day-0 Adaptation of Trillion-Parameter
// MoE Models on Domestic GPUs", section 3 item (1): a low-dimensional
// similarity score for every past position, ahead of Top-K filtering).
//
//   score(i, s) = sum_h w[i,h] * max(0, q_idx[i,h,:] . k_idx(s,:))
//
// The per-head dot products are a dense contraction and run on the gfx950
// matrix cores: one MFMA 16x16x32 (bf16 in, fp32 accumulate) takes 16 heads
// (rows, from the query) against 16 positions (columns, from the indexer-key
// cache).  The ReLU, head weight and head sum are a VALU epilogue on the
// accumulators followed by a two-step cross-lane sum.  With integer-valued
// inputs every partial sum is an integer below 2^24, so fp32 gives the exact
// score whatever the summation order.
//
// Decode (one query per sequence, item (3): bandwidth bound): each workgroup
// streams one chunk of one sequence's indexer keys straight from HBM into
// MFMA operand registers (a lane loads 16 contiguous bytes of one key row);
// the query stays in registers.  Prefill (item (3): compute bound): each
// workgroup stages a tile of keys in LDS once and reuses it for a block of
// queries; the query block keeps its queries in registers over a long run
// of key tiles.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "host_util.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------- decode

// Scores of positions [t0, t1) of sequence b by one workgroup: the query's
// 64x128 operand sits in registers; the indexer keys stream HBM -> MFMA
// operand registers with two register buffers, so one round's loads fly
// while the previous round's MFMAs and epilogue run.
// The two largest of the 16 values held by the lanes of each 16-lane row
// (as a multiset: a value held twice is both), in every lane of the row.
// Each step merges two disjoint sets of lanes: pairs (quad xor 1), quads
// (quad xor 2), half rows (lane i with 7 - i), halves (lane i with 15 - i).
__device__ __forceinline__ void row_top2(float& a1, float& a2) {
  auto step = [&](auto ctrl) {
    constexpr int c = decltype(ctrl)::value;
    const float b1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a1), c, 0xf, 0xf, false));
    const float b2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a2), c, 0xf, 0xf, false));
    const float lo = fminf(a1, b1);
    a1 = fmaxf(a1, b1);
    a2 = fmaxf(lo, fmaxf(a2, b2));
  };
  step(std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  step(std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  step(std::integral_constant<int, 0x141>{});  // row_half_mirror
  step(std::integral_constant<int, 0x140>{});  // row_mirror
}

// Group maxima written by the fused decode path: for group g (positions
// 16 g .. 16 g + 15 of a row) m1[g] is its largest score and m2[g] its
// second largest (NaN when the group holds a single position).
struct GroupMaxOut {
  float* m1;
  float* m2;
  int64_t ldg;  // row stride of both arrays
};

// With a staging buffer `stage` (LDS, room for t1 - t0 scores, t0 a multiple
// of 16), the scores are kept there and written out once the whole segment
// is scored: score stores interleaved with the key stream slow the stream
// far more than their bytes (about 14% for 1.6% of the traffic, measured
// with a streaming probe), and one burst per segment costs about half of
// that.  All waves of the workgroup call it together in that case (it holds
// workgroup barriers).
template <int H_IDX, int D_IDX, int UNROLL, bool GMAX>
__device__ __forceinline__ void score_segment(const uint16_t* __restrict__ k_idx, int64_t k_stride,
                                              const int32_t* __restrict__ bt_row, int bs,
                                              int num_blocks, const uint16_t* __restrict__ q_row,
                                              const float* __restrict__ w_row,
                                              float* __restrict__ out, float* __restrict__ gm1,
                                              float* __restrict__ gm2, int t0, int t1,
                                              float* __restrict__ stage = nullptr,
                                              float* __restrict__ gstage1 = nullptr,
                                              float* __restrict__ gstage2 = nullptr) {
  constexpr int HT = (H_IDX + 15) / 16;  // 16-head tiles
  constexpr int KS = D_IDX / 32;         // 32-wide k-steps
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15, grp = lane >> 4;

  // A operand: head row 16*ht + col, dims 32*ks + 8*grp .. +7.
  bf16x8 qa[HT][KS];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const int head = 16 * ht + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (head < H_IDX) v = *(const u32x4*)(q_row + head * D_IDX + 32 * ks + 8 * grp);
      qa[ht][ks] = as_bf16x8(v);
    }
  }
  // Head weights of the accumulator rows this lane holds: 16*ht + 4*grp + i.
  float wr[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = 16 * ht + 4 * grp + i;
      wr[ht][i] = head < H_IDX ? w_row[head] : 0.f;
    }

  constexpr int kStep = kWaves * 16 * UNROLL;  // tokens per workgroup per round
  // Rounds start on a multiple of 16, so a 16-position group never straddles
  // a cache block (block sizes are multiples of 16) and its block-table
  // entry is one scalar load.  Scalar loads wait on their own counter, so
  // looking up the next round's blocks never waits for key loads in flight.
  // Loads carry no branches (so the compiler can keep a whole buffer of them
  // in flight): a group starting at or past t1 reads the last group again,
  // and positions of a group outside [t0, t1) are read from the same
  // physical block; none of these are written.
  const int a0 = t0 & ~15;
  const int g_last = (t1 - 1) & ~15;
  auto load = [&](u32x4 (&kb)[UNROLL][KS], int base) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int g0 = __builtin_amdgcn_readfirstlane(min(base + 16 * u, g_last));
      const int64_t phys = checked_block(bt_row[g0 / bs], num_blocks);
      const uint16_t* row = k_idx + (phys * bs + g0 % bs + col) * k_stride + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[u][ks] = *(const u32x4*)(row + 32 * ks);
    }
  };
  auto compute = [&](const u32x4 (&kb)[UNROLL][KS], int base) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      f32x4 acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
          acc[ht] = mfma16x16x32(qa[ht][ks], as_bf16x8(kb[u][ks]), acc[ht]);
      float s = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) s += wr[ht][i] * relu(acc[ht][i]);
      s = wave_sum_xor_16_32(s);
      const int tok = base + 16 * u + col;
      if (grp == 0 && tok >= t0 && tok < t1) {
        if (stage)
          stage[tok - t0] = s;
        else
          out[tok] = s;
      }
      if constexpr (GMAX) {
        // t0 is a multiple of 16 here: the group lies in [t0, t1) up to its tail
        const int g0 = base + 16 * u;
        float a1 = tok < t1 ? s : -INFINITY, a2 = -INFINITY;
        row_top2(a1, a2);
        if (lane == 0 && g0 < t1) {
          const float b2 = t1 - g0 >= 2 ? a2 : __int_as_float(0x7fc00000);
          if (stage) {
            gstage1[(g0 - t0) >> 4] = a1;
            gstage2[(g0 - t0) >> 4] = b2;
          } else {
            gm1[g0 >> 4] = a1;
            gm2[g0 >> 4] = b2;
          }
        }
      }
    }
  };

  // The loop body has no branches either (a round past t1 re-reads the
  // last group and writes nothing), so the compiler's load counting stays
  // exact and each compute waits only for its own buffer.
  u32x4 ka[UNROLL][KS], kb[UNROLL][KS];
  int base = a0 + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) * 16 * UNROLL;
  if (base < t1) {
    load(ka, base);
    for (; base < t1; base += 2 * kStep) {
      load(kb, base + kStep);
      compute(ka, base);
      load(ka, base + 2 * kStep);
      compute(kb, base + kStep);
    }
  }
  if (stage) {
    __syncthreads();  // every wave's scores are staged
    const int n = t1 - t0;
    for (int i = 4 * (int)threadIdx.x; i < n; i += 4 * kThreads) {
      if (i + 4 <= n)
        *(float4*)(out + t0 + i) = *(const float4*)(stage + i);
      else
        for (int j = i; j < n; ++j) out[t0 + j] = stage[j];
    }
    if constexpr (GMAX) {
      for (int g = (int)threadIdx.x; 16 * g < n; g += kThreads) {
        gm1[(t0 >> 4) + g] = gstage1[g];
        gm2[(t0 >> 4) + g] = gstage2[g];
      }
    }
    __syncthreads();  // the buffers are free again
  }
}

constexpr int kUnroll = 4;      // 16-position groups per wave per register buffer
constexpr int kFlatMaxSeq = 1024;
constexpr int kStageScores = 16384;  // staged scores per workgroup (64 KB of LDS)

// Query i of a call: its sequence and its candidate count (positions
// 0 .. n - 1).  Without per-query arrays, query i is the last cached token
// of sequence i.  Debug builds check the description against the cache and
// score nothing for a query outside it.
struct QueryDesc {
  const int32_t* q_seq;     // [n_q] or NULL
  const int32_t* q_pos;     // [n_q] or NULL
  const int32_t* seq_lens;  // [n_seq], used when q_pos is NULL
  int n_seq, max_pos;       // max_pos = max_blocks_per_seq * block_size
  int64_t ld;
  __device__ __forceinline__ int seq(int i) const { return q_seq ? q_seq[i] : i; }
  __device__ __forceinline__ int count(int i) const {
    const int n = q_pos ? q_pos[i] + 1 : seq_lens[i];
    if (kCheckBounds) {
      const int b = seq(i);
      if (b < 0 || b >= n_seq || n < 0 || n > max_pos || n > ld) {
        raise_error(q_pos ? kErrQuery : kErrLength);
        return 0;
      }
    }
    return n;
  }
};

// Decode, token-balanced: the batch's positions are laid end to end and
// each workgroup of a persistent grid takes one equal slice, whatever the
// ragged lengths; the query is reloaded only where a slice crosses into the
// next sequence.  Needs n_seq <= kFlatMaxSeq (prefix sums sit in LDS).
template <int H_IDX, int D_IDX, bool GMAX>
__global__ __launch_bounds__(kThreads, 2) void index_score_decode_flat_kernel(
    const uint16_t* __restrict__ k_idx, int64_t k_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, int num_blocks, QueryDesc qd, int n_seq,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    float* __restrict__ scores, int64_t ld, GroupMaxOut gmo) {
  // prefix sums in 16-position groups: they fit 32 bits (2^31 groups would
  // be 8 TB of indexer keys)
  __shared__ int32_t cum[kFlatMaxSeq + 1];
  __shared__ int64_t wave_tot[kWaves];
  __shared__ __attribute__((aligned(16))) float stage[kStageScores];
  __shared__ __attribute__((aligned(16))) float gstage[2][kStageScores / 16];
  // exclusive prefix of the lengths in 16-position groups (slices start on
  // a group boundary, so each group is scored by one workgroup): per-thread
  // runs, a scan across each wave's lanes, then the four wave totals
  const int per = (n_seq + kThreads - 1) / kThreads;
  const int s0 = threadIdx.x * per, s1 = min(s0 + per, n_seq);
  int64_t run = 0;
  for (int i = s0; i < s1; ++i) run += (qd.count(i) + 15) >> 4;
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int64_t incl = run;
#pragma unroll
  for (int d = 1; d < kWave; d *= 2) {
    const int64_t o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_tot[wv] = incl;
  __syncthreads();
  int64_t base = 0, total_all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    base += i < wv ? wave_tot[i] : 0;
    total_all += wave_tot[i];
  }
  run = base + incl - run;  // exclusive prefix of this thread's run
  for (int i = s0; i < s1; ++i) {
    cum[i] = (int32_t)run;
    run += (qd.count(i) + 15) >> 4;
  }
  if (threadIdx.x == 0) cum[n_seq] = (int32_t)total_all;
  __syncthreads();
  const int64_t total = cum[n_seq];
  const int64_t lo = total * blockIdx.x / gridDim.x;
  const int64_t hi = total * (blockIdx.x + 1) / gridDim.x;
  if (lo >= hi) return;
  // first sequence whose range ends after lo
  int b0 = 0, b1 = n_seq - 1;
  while (b0 < b1) {
    const int mid = (b0 + b1) / 2;
    if (cum[mid + 1] <= lo) b0 = mid + 1; else b1 = mid;
  }
  for (int b = b0; b < n_seq && cum[b] < hi; ++b) {
    const int L = qd.count(b);
    const int t0 = 16 * (int)max<int64_t>(lo - cum[b], 0);
    const int t1 = (int)min<int64_t>(16 * (hi - cum[b]), L);
    if (t0 >= t1) continue;
    // the segment's scores go out in one burst when they fit the staging
    // buffer (uniform: t0, t1 come from LDS data and the block index)
    score_segment<H_IDX, D_IDX, kUnroll, GMAX>(
        k_idx, k_stride, block_table + (int64_t)qd.seq(b) * max_blocks, bs, num_blocks,
        q_idx + (int64_t)b * H_IDX * D_IDX, w + (int64_t)b * H_IDX, scores + (int64_t)b * ld,
        gmo.m1 + b * gmo.ldg, gmo.m2 + b * gmo.ldg, t0, t1,
        t1 - t0 <= kStageScores ? stage : nullptr, gstage[0], gstage[1]);
  }
}

// Decode, one (sequence, chunk) per workgroup: for batches too wide for the
// token-balanced kernel.
template <int H_IDX, int D_IDX, bool GMAX>
__global__ __launch_bounds__(kThreads) void index_score_decode_kernel(
    const uint16_t* __restrict__ k_idx, int64_t k_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, int num_blocks, QueryDesc qd,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
    float* __restrict__ scores, int64_t ld, int chunk, GroupMaxOut gmo) {
  const int b = blockIdx.y;
  const int L = qd.count(b);
  const int t0 = blockIdx.x * chunk;  // chunk is a multiple of 16
  if (t0 >= L) return;
  score_segment<H_IDX, D_IDX, kUnroll, GMAX>(
      k_idx, k_stride, block_table + (int64_t)qd.seq(b) * max_blocks, bs, num_blocks,
      q_idx + (int64_t)b * H_IDX * D_IDX, w + (int64_t)b * H_IDX, scores + (int64_t)b * ld,
      gmo.m1 + b * gmo.ldg, gmo.m2 + b * gmo.ldg, t0, min(t0 + chunk, L));
}

// ---------------------------------------------------------------- prefill
//
// Prefill queries come in blocks of consecutive queries that usually belong
// to one sequence (a causal prefill chunk).  A block whose queries span
// several sequences is handled one sequence at a time: the block stages that
// sequence's keys and only its queries score them.

// The sequences and positions of a block's queries, staged in LDS; `lead[g]`
// is true when query g is the first of the block with its sequence.
template <int QB>
struct BlockQueries {
  int32_t seq[QB], pos[QB];
  __device__ void stage(const QueryDesc& qd, int q0, int qend) {
    for (int g = threadIdx.x; g < QB; g += blockDim.x) {
      const int qi = q0 + g;
      int b = -1, p = -1;
      if (qi < qend) {
        b = qd.seq(qi);
        p = qd.count(qi) - 1;  // -1: nothing to score (count 0)
        if (p < 0) b = -1;
      }
      seq[g] = b;
      pos[g] = p;
    }
  }
  // Is query g the first of the block with its sequence?
  __device__ bool lead(int g) const {
    if (seq[g] < 0) return false;
    for (int h = 0; h < g; ++h)
      if (seq[h] == seq[g]) return false;
    return true;
  }
  // Largest position among the block's queries of sequence b.
  __device__ int last_pos(int b) const {
    int m = -1;
    for (int h = 0; h < QB; ++h)
      if (seq[h] == b) m = max(m, pos[h]);
    return m;
  }
};

template <int H_IDX, int D_IDX, int QB, int KB>
__global__ __launch_bounds__(kThreads) void index_score_prefill_tile_kernel(
    const uint16_t* __restrict__ k_idx, int64_t k_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, int num_blocks, QueryDesc qd, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, int n_q, float* __restrict__ scores, int64_t ld) {
  constexpr int HT = (H_IDX + 15) / 16;
  constexpr int KS = D_IDX / 32;
  constexpr int ROW = D_IDX + 8;  // padded LDS row (elements)
  constexpr int CH = D_IDX / 8;   // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) uint16_t ktile[KB * ROW];
  __shared__ BlockQueries<QB> bq;

  const int q0 = blockIdx.y * QB;
  const int qend = min(q0 + QB, n_q);
  const int k0 = blockIdx.x * KB;
  bq.stage(qd, q0, qend);
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int col = lane & 15, grp = lane >> 4;
  for (int lg = 0; lg < QB; ++lg) {
    if (!bq.lead(lg)) continue;  // uniform: LDS data
    const int b = bq.seq[lg];
    const int last_pos = bq.last_pos(b);
    if (k0 > last_pos) continue;
    const int kend = min(k0 + KB, last_pos + 1);
    const int32_t* bt_row = block_table + (int64_t)b * max_blocks;
    __syncthreads();  // the previous sequence's tile is no longer read
    for (int c = threadIdx.x; c < KB * CH; c += kThreads) {
      const int r = c / CH, ch = c % CH;
      const int pos = k0 + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (pos < kend)
        v = *(const u32x4*)(k_idx + paged_row(bt_row, bs, pos, num_blocks) * k_stride + 8 * ch);
      *(u32x4*)(ktile + r * ROW + 8 * ch) = v;
    }
    __syncthreads();

    for (int g = wave; g < qend - q0; g += kWaves) {
      if (bq.seq[g] != b) continue;
      const int qi = q0 + g;
      const int n = min(kend, bq.pos[g] + 1) - k0;  // keys of this tile the query sees
      if (n <= 0) continue;
      bf16x8 qa[HT][KS];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        const int head = 16 * ht + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 v = {0u, 0u, 0u, 0u};
          if (head < H_IDX)
            v = *(const u32x4*)(q_idx + ((int64_t)qi * H_IDX + head) * D_IDX + 32 * ks + 8 * grp);
          qa[ht][ks] = as_bf16x8(v);
        }
      }
      float wr[HT][4];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int head = 16 * ht + 4 * grp + i;
          wr[ht][i] = head < H_IDX ? w[(int64_t)qi * H_IDX + head] : 0.f;
        }
      float* out = scores + (int64_t)qi * ld + k0;
      for (int gg = 0; gg * 16 < n; ++gg) {
        f32x4 acc[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kb =
              as_bf16x8(*(const u32x4*)(ktile + (16 * gg + col) * ROW + 32 * ks + 8 * grp));
#pragma unroll
          for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16x16x32(qa[ht][ks], kb, acc[ht]);
        }
        float s = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int i = 0; i < 4; ++i) s += wr[ht][i] * relu(acc[ht][i]);
        s = wave_sum_xor_16_32(s);
        if (grp == 0 && 16 * gg + col < n) out[16 * gg + col] = s;
      }
    }
  }
}

// Wide indexer (H_IDX x 128 dims, H_IDX a multiple of 16): one workgroup
// takes 16 consecutive queries and a chunk of up to kChunk key tiles of 128
// positions.  Each of its 16 waves keeps one query in registers for the
// whole chunk, so a query is read once per chunk rather than once per key
// tile, and every key tile staged in LDS serves 16 queries; key tiles go
// from HBM straight into LDS (direct loads, one tile ahead, no registers).
// Four waves per SIMD hide the LDS latency and overlap one wave's
// ReLU-weight-sum epilogue with another's products.  A tile row's sixteen
// 16-byte chunks are XOR-swizzled by the row index, so the 16 lanes that
// read 16 rows at one chunk hit 16 different bank groups; the direct loads
// honour the same map.
namespace pf {
constexpr int kWaves = 16, kThreads = kWaves * kWave;
constexpr int kQB = kWaves;                           // queries per workgroup (one per wave)
constexpr int kKT = 128;                              // keys per tile
constexpr int kChunk = 64;                            // tiles per workgroup at most (8192 keys)
constexpr int kD = 128;
constexpr int kRowChunks = kD / 8;                    // 16-byte chunks per key row
constexpr int kTileBytes = kKT * kD * 2;              // 32 KB
constexpr int kLoads = kTileBytes / (16 * kThreads);  // wave loads per wave per tile

// LDS of one workgroup: two key tiles and the physical rows of the chunk.
struct Stage {
  __attribute__((aligned(16))) uint16_t ktile[2][kTileBytes / 2];
  int32_t prow[kChunk * kKT];
};

// This wave's query as the A operand (head 16 ht + col, dims 32 ks + 8 grp
// ..) and the weights of the heads in this lane's result rows.
template <int H_IDX>
struct QueryRegs {
  bf16x8 qa[H_IDX / 16][kD / 32];
  float wr[H_IDX / 16][4];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ q_idx,
                                       const float* __restrict__ w, int qr, int col, int grp) {
#pragma unroll
    for (int ht = 0; ht < H_IDX / 16; ++ht) {
#pragma unroll
      for (int ks = 0; ks < kD / 32; ++ks)
        qa[ht][ks] = as_bf16x8(*(const u32x4*)(q_idx + ((int64_t)qr * H_IDX + 16 * ht + col) * kD +
                                                32 * ks + 8 * grp));
#pragma unroll
      for (int i = 0; i < 4; ++i) wr[ht][i] = w[(int64_t)qr * H_IDX + 16 * ht + 4 * grp + i];
    }
  }
};

// Scores of one sequence's keys at positions k_begin .. k_end - 1 (at most
// kChunk tiles) against every wave's query: the wave whose query sits at
// position qpos of this sequence (-1: none) writes the score of position p
// (p <= qpos) to out[p].  All waves of the workgroup call it together (it
// holds workgroup barriers); on return the tiles may be overwritten.
template <int H_IDX>
__device__ __forceinline__ void score_sequence(
    Stage& st, const uint16_t* __restrict__ k_idx, uint64_t row_bytes,
    const int32_t* __restrict__ bt_row, int bs, int num_blocks, int k_begin, int k_end, int qpos,
    const QueryRegs<H_IDX>& q, float* __restrict__ out, int tid) {
  constexpr int HT = H_IDX / 16, KS = kD / 32;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15, grp = lane >> 4;
  const int n_tiles = (k_end - k_begin + kKT - 1) / kKT;
  __syncthreads();  // the previous sequence's tiles and rows are no longer read
  // physical rows of the chunk's keys; slots past k_end repeat the first
  // key (finite data, never stored)
  for (int r = tid; r < n_tiles * kKT; r += kThreads) {
    const int pos = k_begin + r;
    st.prow[r] = (int32_t)paged_row(bt_row, bs, pos < k_end ? pos : k_begin, num_blocks);
  }
  __syncthreads();  // prow

  const uint32_t kt_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)st.ktile;
  // Wave load i of this wave fills tile slots 64 (kLoads wave + i) + lane:
  // slot s holds chunk (s % 16) ^ (r % 16) of tile row r = s / 16.
  auto load_tile = [&](int j, int buf) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int blk = kLoads * wave + i;
      const int slot = kWave * blk + lane;
      const int r = slot / kRowChunks;
      const int c = (slot % kRowChunks) ^ (r % kRowChunks);
      const char* src =
          (const char*)k_idx + (uint64_t)(uint32_t)st.prow[j * kKT + r] * row_bytes + 16 * c;
      global_to_lds16(src, kt_lds + (uint32_t)(buf * kTileBytes + 16 * kWave * blk));
    }
  };
  load_tile(0, 0);

  for (int j = 0; j < n_tiles; ++j) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of tile j has landed
    __syncthreads();  // all of tile j; tile j - 1's buffer is no longer read
    if (j + 1 < n_tiles) load_tile(j + 1, (j + 1) & 1);
    const uint16_t* kt = st.ktile[j & 1];
    const int k0 = k_begin + j * kKT;
    const int n = min(kKT, max(0, qpos + 1 - k0));  // keys of this tile the query sees
    for (int g = 0; 16 * g < n; ++g) {
      f32x4 acc[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) acc[ht] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * g + col;  // B operand: key row r, dims 32 ks + 8 grp ..
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int slot = r * kRowChunks + ((4 * ks + grp) ^ (r % kRowChunks));
        const bf16x8 kb = as_bf16x8(*(const u32x4*)(kt + 8 * slot));
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) acc[ht] = mfma16x16x32(q.qa[ht][ks], kb, acc[ht]);
      }
      float sc = 0.f;
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc += q.wr[ht][i] * relu(acc[ht][i]);
      sc = wave_sum_xor_16_32(sc);
      if (grp == 0 && r < n) out[k0 + r] = sc;
    }
  }
}
}  // namespace pf

template <int H_IDX>
__global__ __launch_bounds__(pf::kThreads, 1) void index_score_prefill_kernel(
    const uint16_t* __restrict__ k_idx, int64_t k_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, int num_blocks, QueryDesc qd, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, int n_q, float* __restrict__ scores, int64_t ld) {
  using pf::kChunk, pf::kKT, pf::kQB;
  __shared__ pf::Stage st;
  __shared__ BlockQueries<kQB> bq;

  // the query blocks of the latest positions (usually the longest rows)
  // first, so that the short ones fill in behind them
  const int q0 = (gridDim.y - 1 - blockIdx.y) * kQB;
  const int qend = min(q0 + kQB, n_q);
  const int k_begin = blockIdx.x * (kChunk * kKT);
  bq.stage(qd, q0, qend);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int qi = q0 + wave;
  pf::QueryRegs<H_IDX> q;
  q.load(q_idx, w, qi < qend ? qi : q0, lane & 15, lane >> 4);
  __syncthreads();  // bq

  for (int lg = 0; lg < kQB; ++lg) {
    if (!bq.lead(lg)) continue;  // uniform: LDS data
    const int b = bq.seq[lg];
    const int last_pos = bq.last_pos(b);
    if (k_begin > last_pos) continue;
    // this wave's query position if it belongs to sequence b (wave-uniform)
    const int qpos = qi < qend && bq.seq[wave] == b ? bq.pos[wave] : -1;
    pf::score_sequence<H_IDX>(st, k_idx, (uint64_t)k_stride * 2,
                              block_table + (int64_t)b * max_blocks, bs, num_blocks, k_begin,
                              min(k_begin + kChunk * kKT, last_pos + 1), qpos, q,
                              scores + (int64_t)qi * ld, threadIdx.x);
  }
}

// ------------------------------------------------- prefill, fused with Top-K
//
// Index score and Top-K of prefill rows in one kernel, with no T x T score
// matrix (web page "Day-0 Adaptation of Trillion-Parameter MoE Models on
// Domestic GPUs", section 3 item (3): prefill fuses index selection into
// large-granularity operators).  A persistent grid, one workgroup per CU,
// walks blocks of 16 queries.  Per block: the queries with more than K
// candidates are scored exactly as by the prefill kernel above (a row with
// at most K candidates keeps all of them whatever its scores, so it is not
// scored), each wave's row of scores going to its row of the workgroup's
// 512 KB slot of a bounded scratch (the slots of all resident workgroups
// total 128 MB whatever the prefill length); then pairs of waves select:
// the two waves of a pair split a row in halves (64 keys a lane), find the
// exact K-th largest key by the bitwise search, each step's two counts
// exchanged through LDS at a workgroup barrier (once at most 512 keys are
// still open, each wave moves its open keys into an LDS list and counts
// only those), and write the kept positions ascending (equal scores: lower
// position first).  Rows hold at most 8192 candidates.
namespace ftk {
constexpr int kQ = pf::kQB;                     // queries per block (one per wave)
constexpr int kMaxKeys = pf::kChunk * pf::kKT;  // candidates per row at most (8192)
constexpr int kHalf = kMaxKeys / 2;             // keys of a row per wave of a pair
constexpr int kR = kHalf / kWave;               // keys per lane (64)
constexpr int kSlotFloats = kQ * kMaxKeys;      // scratch floats per workgroup (512 KB)
constexpr int kMaxGrid = 256;                   // scratch slots
constexpr int kOpen = 512;                      // open keys listed per wave (LDS)

// Counts exchanged between the two waves of a pair (indexed by wave).
struct PairCounts {
  uint32_t a[kQ], o[kQ], c[2][kQ], gt[kQ], eq[kQ], steps[kQ];
};
}  // namespace ftk

__device__ __forceinline__ uint64_t lanes_below(int lane) { return (1ull << lane) - 1ull; }

// Set bits of the wave mask m in the lanes below this one.
__device__ __forceinline__ uint32_t bits_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// A value every lane of the wave holds alike, made visibly wave-uniform (a
// scalar register) for the compiler: values read from LDS or passed to an
// out-of-line function otherwise count as per-lane.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
template <class T>
__device__ __forceinline__ T* uni_ptr(T* p) {
  const uint64_t u = (uint64_t)p;
  return (T*)(((uint64_t)uni((uint32_t)(u >> 32)) << 32) | uni((uint32_t)u));
}

// Exact Top-K of one row held by a pair of waves (waves 2p and 2p + 1):
// wave h of the pair holds the keys of candidates pos0 + 64 i + lane in k[i]
// (0 = no candidate; i < rounds) and writes its kept positions into out.
// Every wave of the workgroup calls this together: the barriers it holds
// are the same in number in every wave (2, one per search step of the pair
// with the most bits to decide, then 1).  `active` (the same in both waves of a pair)
// is false when the pair has no row with more than K candidates; such a
// pair only takes part in the barriers; n is the row's candidate count.
//
// The K-th largest key tau is found one bit at a time from the top; both
// waves track, as pair totals, A (keys whose bits above the current one
// exceed tau's: kept) and U (keys whose bits above it equal tau's: still
// open).  Once U <= kOpen, each wave moves its open keys into its own LDS
// list and the remaining bits count only those (at most 8 a lane).
__device__ __forceinline__ void pair_topk_row(const uint32_t (&k)[ftk::kR], int rounds,
                                              bool active, int n, int K, int pos0,
                                              int32_t* __restrict__ out, ftk::PairCounts& x,
                                              uint32_t* __restrict__ open_list) {
  using ftk::kOpen, ftk::kR;
  constexpr int kOL = kOpen / kWave;  // open keys per lane
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int mate = wave ^ 1;
  // keys >= c among k (chunks of 8: keys past `rounds` are 0 and never
  // reach c >= 1)
  auto count_ge = [&](uint32_t c) {
    uint32_t cnt = 0;
#pragma unroll
    for (int i0 = 0; i0 < kR; i0 += 8)
      if (i0 < rounds) {
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) cnt += (uint32_t)__popcll(__ballot(k[i] >= c));
      }
    return cnt;
  };
  // bits where the row's keys differ (AND / OR over both halves)
  uint32_t a = 0xffffffffu, o = 0u;
#pragma unroll
  for (int i = 0; i < kR; ++i)
    if (k[i]) {
      a &= k[i];
      o |= k[i];
    }
  a = wave_and(a);  // wave-uniform (read from lane 63)
  o = wave_or(o);
  if (lane == 0) {
    x.a[wave] = a;
    x.o[wave] = o;
  }
  __syncthreads();
  a &= uni(x.a[mate]);
  o |= uni(x.o[mate]);
  uint32_t tau = a;  // bits not in diff are those of every key
  const uint32_t diff = active ? a ^ o : 0u;
  // search steps: one per bit of diff, as many in every wave as the pair
  // with the most needs
  if (lane == 0) x.steps[wave] = (uint32_t)__popc(diff);
  __syncthreads();
  uint32_t n_steps = 0;
#pragma unroll
  for (int v = 0; v < ftk::kQ; ++v) n_steps = max(n_steps, uni(x.steps[v]));
  uint32_t kept = 0, open = (uint32_t)n;  // A and U (pair totals)
  // the lists hold the keys open when they were made: those kept since are
  // in them too, those kept before are not
  uint32_t kept_listed = 0;
  bool listed = false;  // the same in both waves of the pair
  uint32_t u[kOL];
#pragma unroll
  for (int j = 0; j < kOL; ++j) u[j] = 0u;
  int list_len = 0;
  uint32_t rest = diff;  // bits still to decide, highest first
  for (uint32_t step = 0; step < n_steps; ++step) {
    const int bit = rest ? 31 - __clz(rest) : 0;
    const uint32_t b = rest ? 1u << bit : 0u;
    rest &= ~b;
    const bool test = b != 0u;  // the same in both waves of the pair
    if (test && !listed && open <= (uint32_t)kOpen) {
      // this wave's open keys (bits above `bit` equal to tau's) into its
      // list; the order does not matter for counting
      listed = true;
      kept_listed = kept;
#pragma unroll
      for (int i0 = 0; i0 < kR; i0 += 8)
        if (i0 < rounds) {
#pragma unroll
          for (int i = i0; i < i0 + 8; ++i) {
            const bool op = k[i] != 0u && ((k[i] ^ tau) >> bit) <= 1u;
            const uint64_t m = __ballot(op);
            const int at = list_len + (int)bits_below(m);
            if (op && at < kOpen) open_list[at] = k[i];  // at < kOpen: open <= kOpen
            list_len += __popcll(m);
          }
        }
#pragma unroll
      for (int j = 0; j < kOL; ++j)
        u[j] = kWave * j + lane < list_len ? open_list[kWave * j + lane] : 0u;
    }
    // keys of this wave (of its list, once listed) >= tau | b: the kept
    // ones (since listing) and the open ones with bit b set
    uint32_t c = 0;
    if (test) {
      if (listed) {
#pragma unroll
        for (int j = 0; j < kOL; ++j)
          if (kWave * j < list_len) c += (uint32_t)__popcll(__ballot(u[j] >= (tau | b)));
      } else {
        c = count_ge(tau | b);
      }
    }
    if (lane == 0) x.c[step & 1][wave] = c;
    __syncthreads();
    if (test) {
      c += uni(x.c[step & 1][mate]);
      const uint32_t open1 = c - (kept - kept_listed);  // open keys with bit b set
      if (kept + open1 >= (uint32_t)K) {
        tau |= b;
        open = open1;
      } else {
        kept += open1;
        open -= open1;
      }
    }
  }
  // keys above tau and equal to tau in this half
  uint32_t gt = 0, eq = 0;
  if (active) {
#pragma unroll
    for (int i0 = 0; i0 < kR; i0 += 8)
      if (i0 < rounds) {
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i) {
          gt += (uint32_t)__popcll(__ballot(k[i] > tau));
          eq += (uint32_t)__popcll(__ballot(k[i] == tau));
        }
      }
  }
  if (lane == 0) {
    x.gt[wave] = gt;
    x.eq[wave] = eq;
  }
  __syncthreads();
  if (!active) return;
  const uint32_t gt_mate = uni(x.gt[mate]);
  const uint32_t need = (uint32_t)K - (gt + gt_mate);  // keys equal to tau to keep
  // the second half starts after everything the first half keeps
  uint32_t base = 0, eq_seen = 0;
  if (wave & 1) {
    eq_seen = uni(x.eq[mate]);
    base = gt_mate + min(need, eq_seen);
  }
#pragma unroll
  for (int i0 = 0; i0 < kR; i0 += 8)
    if (i0 < rounds) {
#pragma unroll
      for (int i = i0; i < i0 + 8; ++i) {
        const uint64_t meq = __ballot(k[i] == tau);
        const uint32_t eq_before = eq_seen + bits_below(meq);
        const bool sel = k[i] > tau || (k[i] == tau && eq_before < need);
        const uint64_t msel = __ballot(sel);
        const uint32_t slot = base + bits_below(msel);
        if (sel && slot < (uint32_t)K) out[slot] = pos0 + kWave * i + lane;
        base += (uint32_t)__popcll(msel);
        eq_seen += (uint32_t)__popcll(meq);
      }
    }
}

// One wave's half of a row for pair_topk_row: its `mine` scores (from
// `row`, positions pos0 ..) read back as keys, then the selection.  Kept
// out of line: its registers are allocated apart from the scoring loop's,
// which otherwise spills (and each reload waits for the tile prefetch).
__device__ __attribute__((noinline)) void select_pair_row(const float* row_arg, int mine_arg,
                                                          int active_arg, int n_arg, int K_arg,
                                                          int pos0_arg, int32_t* out_arg) {
  __shared__ ftk::PairCounts x;
  __shared__ uint32_t open_lists[ftk::kQ][ftk::kOpen];
  // every argument is the same in all lanes of the wave
  const float* row = uni_ptr(row_arg);
  int32_t* out = uni_ptr(out_arg);
  const int mine = (int)uni(mine_arg), n = (int)uni(n_arg), K = (int)uni(K_arg);
  const int pos0 = (int)uni(pos0_arg);
  const bool active = uni(active_arg) != 0u;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rounds = active ? (mine + kWave - 1) / kWave : 0;
  uint32_t k[ftk::kR];
  // the row through a buffer resource: the lane offset is one vector
  // register and each load's offset a scalar constant
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)row, (short)0, ftk::kHalf * 4, 0x00020000);
  // every load is issued (a conditional one would wait at its branch);
  // they stay inside the row's half, entries past `mine` are stale and
  // masked (0 = no candidate: float_key of a score is never 0)
  // (the raw bits land in k first, so all 64 loads fly at once)
#pragma unroll
  for (int i = 0; i < ftk::kR; ++i)
    k[i] = __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_raw_buffer_load_b32(rsrc, lane * 4, i * kWave * 4, 0));
#pragma unroll
  for (int i = 0; i < ftk::kR; ++i)
    k[i] = kWave * i + lane < mine ? float_key(__builtin_bit_cast(float, k[i])) : 0u;
  pair_topk_row(k, rounds, active, n, K, pos0, out, x, open_lists[wave]);
}

template <int H_IDX>
__global__ __launch_bounds__(pf::kThreads, 1) void index_topk_prefill_kernel(
    const uint16_t* __restrict__ k_idx, int64_t k_stride, const int32_t* __restrict__ block_table,
    int max_blocks, int bs, int num_blocks, QueryDesc qd, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w, int n_q, int K, int32_t* __restrict__ idx,
    float* __restrict__ scratch) {
  using ftk::kMaxKeys, ftk::kQ, ftk::kR;
  __shared__ pf::Stage st;
  __shared__ BlockQueries<kQ> bq;
  __shared__ int32_t cnt[kQ];  // candidates of each query of the block (0: none)

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  float* slot = scratch + (int64_t)blockIdx.x * ftk::kSlotFloats;
  const uint64_t row_bytes = (uint64_t)k_stride * 2;
  const int nqb = (n_q + kQ - 1) / kQ;

  // Blocks in serpentine order over the grid, latest positions (usually the
  // longest rows) first: round r gives workgroup x block t = r G + x for even
  // r and r G + G - 1 - x for odd r, counted from the last block, so the
  // workgroups that take a long block in one round take a short one in the
  // next.
  for (int r = 0;; ++r) {
    const int t = r * (int)gridDim.x +
                  ((r & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x);
    if (t >= nqb) break;
    const int q0 = (nqb - 1 - t) * kQ;
    const int qend = min(q0 + kQ, n_q);
    __syncthreads();  // the previous block's bq, counts and tiles are no longer read
    bq.stage(qd, q0, qend);
    __syncthreads();
    if (threadIdx.x < kQ) {
      int n = bq.pos[threadIdx.x] + 1;  // 0 for no query / nothing to score
      if (n > kMaxKeys) {
        if (kCheckBounds) raise_error(kErrQuery);
        n = kMaxKeys;
      }
      cnt[threadIdx.x] = n;
    }
    __syncthreads();
    bool any = false;  // uniform: LDS data
    for (int g = 0; g < kQ; ++g) any |= cnt[g] > K;
    const int qi = q0 + wave;

    if (!any) {
      // every row keeps all its candidates: 0 .. n - 1, then -1
      if (qi < qend) {
        const int n = cnt[wave];
        int32_t* out = idx + (int64_t)qi * K;
        for (int i = lane; i < K; i += kWave) out[i] = i < n ? i : -1;
      }
      continue;
    }

    // ---- scores of the rows with more than K candidates, into the slot
    {
      // the thread index passed through an opaque move: values derived from
      // it are then computed per block rather than kept live across the
      // whole loop (which would spill, and each reload would wait for the
      // tile prefetch)
      int tid = threadIdx.x;
      asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(tid));
      const int ln = tid & (kWave - 1);
      const int my_n = cnt[wave];
      const bool scored = my_n > K;  // wave-uniform
      pf::QueryRegs<H_IDX> q;
      q.load(q_idx, w, scored ? qi : q0, ln & 15, ln >> 4);
      for (int lg = 0; lg < kQ; ++lg) {
        if (!bq.lead(lg)) continue;  // uniform: LDS data
        const int b = bq.seq[lg];
        int last = -1;  // last position any scored query of sequence b sees
        for (int g = 0; g < kQ; ++g)
          if (bq.seq[g] == b && cnt[g] > K) last = max(last, cnt[g] - 1);
        if (last < 0) continue;
        const int qpos = scored && bq.seq[wave] == b ? my_n - 1 : -1;
        pf::score_sequence<H_IDX>(st, k_idx, row_bytes, block_table + (int64_t)b * max_blocks,
                                  bs, num_blocks, 0, last + 1, qpos, q, slot + wave * kMaxKeys,
                                  tid);
      }
    }
    __syncthreads();  // every wave's scores are in the slot

    // ---- selection: the pair of waves 2p, 2p + 1 takes rows 2p and 2p + 1
#pragma unroll 1
    for (int rr = 0; rr < 2; ++rr) {
      const int g = (wave & ~1) + rr;
      const int n = q0 + g < qend ? cnt[g] : 0;
      const bool active = n > K;  // the same in both waves of the pair
      int32_t* out = idx + (int64_t)(q0 + g) * K;
      if (!active && q0 + g < qend) {
        // all candidates kept; the pair shares the writes
        for (int i = 64 * (wave & 1) + lane; i < K; i += 128) out[i] = i < n ? i : -1;
      }
      // wave h of the pair holds positions h * half .. (half positions per
      // wave, a multiple of 64)
      const int half = (n + 127) / 128 * 64;
      const int pos0 = (wave & 1) * half;
      const int mine = max(0, min(half, n - pos0));
      select_pair_row(slot + g * kMaxKeys + pos0, mine, active ? 1 : 0, n, K, pos0, out);
    }
  }
}

template <int H_IDX, int D_IDX, bool GMAX>
dsa_status_t launch_index_score(const dsa_paged_cache_t* c, dsa_phase_t phase,
                                const uint16_t* q_idx, const float* w, const int32_t* q_seq,
                                const int32_t* q_pos, int n_q, float* scores, int64_t ld,
                                GroupMaxOut gmo, hipStream_t stream) {
  const QueryDesc qd{q_seq, q_pos, c->seq_lens, c->n_seq,
                     (int)std::min<int64_t>((int64_t)c->max_blocks_per_seq * c->block_size,
                                            0x7fffffff),
                     ld};
  if (phase == DSA_DECODE) {
    if (n_q <= kFlatMaxSeq) {
      // persistent grid: as many workgroups as fit on the device at once
      static int grid_cache[64] = {0};  // per device (one per GMAX instantiation)
      int dev = 0;
      (void)hipGetDevice(&dev);
      int grid = dev < 64 ? grid_cache[dev] : 0;
      if (grid == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, index_score_decode_flat_kernel<H_IDX, D_IDX, GMAX>, kThreads, 0) !=
                hipSuccess)
          return DSA_ERR_HIP;
        grid = std::max(1, cus * std::max(1, per_cu));
        if (dev < 64) grid_cache[dev] = grid;
      }
      hipLaunchKernelGGL((index_score_decode_flat_kernel<H_IDX, D_IDX, GMAX>), dim3(grid),
                         dim3(kThreads), 0, stream, c->k_idx, c->k_idx_row_stride, c->block_table,
                         c->max_blocks_per_seq, c->block_size, c->num_blocks, qd, n_q, q_idx, w,
                         scores, ld, gmo);
    } else {
      // Chunk so that about 4096 workgroups cover n_q * ld positions.
      int64_t per = (int64_t)n_q * ld / 4096;
      int chunk = 1024;  // below this the per-workgroup query load dominates
      while (chunk < 8192 && chunk * 2 <= per) chunk *= 2;
      const int64_t nchunks = (ld + chunk - 1) / chunk;
      if (nchunks > 0x7fffffff || n_q > 65535) return DSA_ERR_SHAPE;
      hipLaunchKernelGGL((index_score_decode_kernel<H_IDX, D_IDX, GMAX>),
                         dim3((unsigned)nchunks, (unsigned)n_q), dim3(kThreads), 0, stream,
                         c->k_idx, c->k_idx_row_stride, c->block_table, c->max_blocks_per_seq,
                         c->block_size, c->num_blocks, qd, q_idx, w, scores, ld, chunk, gmo);
    }
  } else if constexpr (GMAX) {
    return DSA_ERR_SHAPE;  // group maxima come from the decode kernels only
  } else if constexpr (D_IDX == pf::kD && H_IDX % 16 == 0) {
    // a workgroup covers up to 8192 keys of 16 queries: a whole row for
    // positions below 8192, so the per-workgroup start (block-table
    // lookups, q loads, first tile) is paid once per query block
    const int64_t nchunks = (ld + pf::kChunk * pf::kKT - 1) / (pf::kChunk * pf::kKT);
    const int64_t nqb = ((int64_t)n_q + pf::kQB - 1) / pf::kQB;
    if (nqb > 65535) return DSA_ERR_SHAPE;
    hipLaunchKernelGGL((index_score_prefill_kernel<H_IDX>), dim3((unsigned)nchunks, (unsigned)nqb),
                       dim3(pf::kThreads), 0, stream, c->k_idx, c->k_idx_row_stride,
                       c->block_table, c->max_blocks_per_seq, c->block_size, c->num_blocks, qd,
                       q_idx, w, n_q, scores, ld);
  } else {
    constexpr int QB = 64, KB = 128;
    const int64_t nkt = (ld + KB - 1) / KB;
    const int64_t nqb = ((int64_t)n_q + QB - 1) / QB;
    if (nqb > 65535 || nkt > 0x7fffffff) return DSA_ERR_SHAPE;
    hipLaunchKernelGGL((index_score_prefill_tile_kernel<H_IDX, D_IDX, QB, KB>),
                       dim3((unsigned)nkt, (unsigned)nqb), dim3(kThreads), 0, stream, c->k_idx,
                       c->k_idx_row_stride, c->block_table, c->max_blocks_per_seq, c->block_size,
                       c->num_blocks, qd, q_idx, w, n_q, scores, ld);
  }
  return launch_status();
}

}  // namespace

uint32_t take_bounds_error_index_score(hipStream_t stream) { return take_bounds_error(stream); }

dsa_status_t launch_index_score_decode_gmax(const dsa_paged_cache_t* c, const uint16_t* q_idx,
                                            const float* w, const int32_t* q_seq,
                                            const int32_t* q_pos, int n_q, int H_idx,
                                            float* scores, int64_t ld, float* gm1, float* gm2,
                                            int64_t ldg, hipStream_t stream) {
  const GroupMaxOut gmo{gm1, gm2, ldg};
  if (H_idx == 64 && c->d_idx == 128)
    return launch_index_score<64, 128, true>(c, DSA_DECODE, q_idx, w, q_seq, q_pos, n_q, scores,
                                             ld, gmo, stream);
  return launch_index_score<4, 32, true>(c, DSA_DECODE, q_idx, w, q_seq, q_pos, n_q, scores, ld,
                                         gmo, stream);
}

}  // namespace dsa

extern "C" size_t dsa_index_topk_prefill_ws(int32_t n_q) {
  if (n_q < 1) return 0;
  // one slot per workgroup of the persistent grid, which never exceeds the
  // number of 16-query blocks
  const int64_t slots = std::min<int64_t>(dsa::ftk::kMaxGrid, ((int64_t)n_q + 15) / 16);
  return (size_t)slots * dsa::ftk::kSlotFloats * sizeof(float);
}

extern "C" dsa_status_t dsa_index_topk_prefill(const dsa_paged_cache_t* cache,
                                               const uint16_t* q_idx, const float* w,
                                               const int32_t* q_seq, const int32_t* q_pos,
                                               int32_t n_q, int32_t H_idx, int32_t K, int32_t* idx,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_cache_common(cache);
  if (st != DSA_OK) return st;
  if (!cache->k_idx || !q_idx || !w || !q_seq || !q_pos || !idx || !workspace) return DSA_ERR_NULL;
  if (n_q < 1 || K < 1 || K > 2048 || cache->k_idx_row_stride < cache->d_idx) return DSA_ERR_SHAPE;
  if (workspace_bytes < dsa_index_topk_prefill_ws(n_q)) return DSA_ERR_WORKSPACE;
  if (H_idx != 64 || cache->d_idx != 128) return DSA_ERR_UNSUPPORTED;
  if (cache->k_idx_row_stride % 8 != 0 || cache->block_size % 16 != 0) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(cache->k_idx) || !aligned16(q_idx) || !aligned16(workspace))
    return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  static int grid_cache[64] = {0};  // per device: resident workgroups
  int dev = 0;
  (void)hipGetDevice(&dev);
  int grid = dev < 64 ? grid_cache[dev] : 0;
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, index_topk_prefill_kernel<64>,
                                                     pf::kThreads, 0) != hipSuccess)
      return DSA_ERR_HIP;
    grid = std::max(1, std::min(ftk::kMaxGrid, cus * std::max(1, per_cu)));
    if (dev < 64) grid_cache[dev] = grid;
  }
  const int nqb = (n_q + ftk::kQ - 1) / ftk::kQ;
  const QueryDesc qd{q_seq, q_pos, cache->seq_lens, cache->n_seq,
                     (int)std::min<int64_t>((int64_t)cache->max_blocks_per_seq * cache->block_size,
                                            0x7fffffff),
                     ftk::kMaxKeys};
  hipLaunchKernelGGL(index_topk_prefill_kernel<64>, dim3((unsigned)std::min(grid, nqb)),
                     dim3(pf::kThreads), 0, stream, cache->k_idx, cache->k_idx_row_stride,
                     cache->block_table, cache->max_blocks_per_seq, cache->block_size,
                     cache->num_blocks, qd, q_idx, w, n_q, K, idx, (float*)workspace);
  return launch_status();
}

extern "C" size_t dsa_index_score_ws(dsa_phase_t phase, int32_t n_q, int64_t ld) {
  (void)phase;
  (void)n_q;
  (void)ld;
  return 0;  // the index score needs no workspace
}

extern "C" dsa_status_t dsa_index_score(const dsa_paged_cache_t* cache, dsa_phase_t phase,
                                        const uint16_t* q_idx, const float* w,
                                        const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                                        int32_t H_idx, float* scores, int64_t ld, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  using namespace dsa;
  (void)workspace;
  (void)workspace_bytes;
  dsa_status_t st = check_cache_common(cache);
  if (st != DSA_OK) return st;
  if (!cache->k_idx || !q_idx || !w || !scores) return DSA_ERR_NULL;
  if (phase != DSA_DECODE && phase != DSA_PREFILL) return DSA_ERR_SHAPE;
  if (n_q < 1 || ld < 1 || cache->k_idx_row_stride < cache->d_idx) return DSA_ERR_SHAPE;
  if ((q_seq == nullptr) != (q_pos == nullptr)) return DSA_ERR_NULL;
  if (!q_seq) {
    // query i is the last cached token of sequence i
    if (phase == DSA_PREFILL) return DSA_ERR_NULL;
    if (!cache->seq_lens) return DSA_ERR_NULL;
    if (n_q != cache->n_seq) return DSA_ERR_SHAPE;
  }
  const bool big = H_idx == 64 && cache->d_idx == 128;
  const bool small = H_idx == 4 && cache->d_idx == 32;
  if (!big && !small) return DSA_ERR_UNSUPPORTED;
  if (cache->k_idx_row_stride % 8 != 0) return DSA_ERR_UNSUPPORTED;  // 16-byte row alignment
  if (!aligned16(cache->k_idx) || !aligned16(q_idx)) return DSA_ERR_UNSUPPORTED;
  if (cache->block_size % 16 != 0) return DSA_ERR_UNSUPPORTED;        // 16-position groups
  st = check_device();
  if (st != DSA_OK) return st;
  const GroupMaxOut none{nullptr, nullptr, 0};
  if (big)
    return launch_index_score<64, 128, false>(cache, phase, q_idx, w, q_seq, q_pos, n_q, scores,
                                              ld, none, stream);
  return launch_index_score<4, 32, false>(cache, phase, q_idx, w, q_seq, q_pos, n_q, scores, ld,
                                          none, stream);
}
