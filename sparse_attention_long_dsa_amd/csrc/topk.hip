// Top-K position selection for DSA (web page "Day-0 Adaptation of
// Trillion-Parameter MoE Models on Domestic GPUs", section 3 item (1): Top-K
// as block-wise scoring, intra-block reduction and cross-block merge, with
// bitmask techniques and no global sort).
//
// Contract: row i keeps the K largest of its n_i scores, equal scores taken
// lower position first, written as ascending positions and padded with -1
// when n_i < K.
//
// Method: fp32 scores map to order-preserving 32-bit keys.  A radix
// threshold search finds the key tau of the K-th largest score and how many
// of the keys equal to tau must be kept ("need"); every key above tau is
// kept, and of the keys equal to tau the `need` lowest positions are kept.
// Nothing is ever fully sorted.
//
//   block-wise scoring:    each workgroup histograms a digit of the keys of
//                          its block of positions in LDS;
//   intra-block reduction: per-wave counts are reduced inside the workgroup
//                          and the threshold digit is located by a suffix
//                          scan of the histogram;
//   cross-block merge:     block histograms are merged across workgroups,
//                          and kept positions are compacted in position
//                          order with wave64 ballot bitmasks and popcount
//                          ranks (short rows), or gathered and merged across
//                          blocks (long rows).
//
// Two paths, chosen by the row capacity `ld`:
//   ld <= 16384: one workgroup per row; the whole row sits in LDS, three
//                digit passes (12, 12, 8 bits) run there and an ordered
//                ballot compaction writes the result (prefill rows);
//   ld  > 16384: many workgroups per row (decode rows up to millions of
//                positions): two global digit histograms (12 + 12 bits), a
//                gather of the keys sharing tau's top 24 bits, and one
//                workgroup per row that resolves the last 8 bits and the
//                ties and writes the row in position order.
#include <algorithm>

#include "common.h"
#include "host_util.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kShortMax = 16384;   // longest row handled in LDS
constexpr int kChunk = 4096;       // positions per workgroup on the long path
constexpr int kBins = 4096;        // 12-bit digits

__device__ __forceinline__ int row_count(const int32_t* n_valid, int causal_base, int row) {
  return n_valid ? n_valid[row] : causal_base + row + 1;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Exclusive sum of v over all threads with a larger thread index (a suffix
// scan in descending thread order).  `sh` holds kWaves words.
__device__ __forceinline__ uint32_t block_suffix_excl(uint32_t v, uint32_t* sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t x = __shfl_down(incl, off);
    if (lane + off < kWave) incl += x;
  }
  if (lane == 0) sh[wave] = incl;  // lane 0 holds the wave total
  __syncthreads();
  uint32_t higher = 0;
  for (int w2 = wave + 1; w2 < kWaves; ++w2) higher += sh[w2];
  __syncthreads();
  return incl - v + higher;
}

// Exclusive sum of v over all threads with a smaller thread index.
__device__ __forceinline__ uint32_t block_prefix_excl(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t x = __shfl_up(incl, off);
    if (lane >= off) incl += x;
  }
  if (lane == kWave - 1) sh[wave] = incl;
  __syncthreads();
  uint32_t lower = 0, all = 0;
  for (int w2 = 0; w2 < kWaves; ++w2) {
    if (w2 < wave) lower += sh[w2];
    all += sh[w2];
  }
  __syncthreads();
  *total = all;
  return incl - v + lower;
}

struct Bucket {
  uint32_t bin;    // bin holding the need-th largest
  uint32_t above;  // keys in bins above it
};

// Descending search of a histogram (LDS or global) of `nbins` bins for the
// bin where the running count from the top reaches `need`.  Every thread of
// the block gets the answer.  `sh` needs kWaves + 2 words.
template <typename Hist>
__device__ Bucket find_bucket_desc(Hist hist, int nbins, uint32_t need, uint32_t* sh) {
  const int per = nbins / kThreads;  // nbins is a multiple of kThreads
  const int lo = threadIdx.x * per;
  uint32_t mine = 0;
  for (int b = 0; b < per; ++b) mine += hist[lo + b];
  uint32_t run = block_suffix_excl(mine, sh);
  if (run < need && run + mine >= need) {
    for (int b = lo + per - 1; b >= lo; --b) {
      const uint32_t h = hist[b];
      if (run + h >= need) {
        sh[kWaves] = (uint32_t)b;
        sh[kWaves + 1] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  Bucket r{sh[kWaves], sh[kWaves + 1]};
  __syncthreads();
  return r;
}

// Ascending twin: the bin where the running count from the bottom reaches need.
__device__ Bucket find_bucket_asc(const uint32_t* hist, int nbins, uint32_t need, uint32_t* sh) {
  const int per = nbins / kThreads;
  const int lo = threadIdx.x * per;
  uint32_t mine = 0;
  for (int b = 0; b < per; ++b) mine += hist[lo + b];
  uint32_t total;
  uint32_t run = block_prefix_excl(mine, sh, &total);
  if (run < need && run + mine >= need) {
    for (int b = lo; b < lo + per; ++b) {
      const uint32_t h = hist[b];
      if (run + h >= need) {
        sh[kWaves] = (uint32_t)b;
        sh[kWaves + 1] = run;
        break;
      }
      run += h;
    }
  }
  __syncthreads();
  Bucket r{sh[kWaves], sh[kWaves + 1]};
  __syncthreads();
  return r;
}

// LDS histogram increment with one round of wave aggregation: the lanes that
// share the first active lane's bin add together with one atomic, the rest
// add one by one (scores that tie or sit in a narrow range would otherwise
// serialise on a single LDS address).
__device__ __forceinline__ void hist_add(uint32_t* hist, bool active, uint32_t bin) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int leader = __ffsll((unsigned long long)act) - 1;
  const uint32_t lbin = __shfl(bin, leader);
  const bool same = active && bin == lbin;
  const uint64_t m = __ballot(same);
  if (lane == leader) atomicAdd(&hist[lbin], (uint32_t)__popcll(m));
  if (active && !same) atomicAdd(&hist[bin], 1u);
}

// ================================================================ short rows

template <int MAXN>
__global__ __launch_bounds__(kThreads) void topk_short_kernel(const float* __restrict__ scores,
                                                              int64_t ld,
                                                              const int32_t* __restrict__ n_valid,
                                                              int causal_base, int K,
                                                              int32_t* __restrict__ idx) {
  __shared__ uint32_t keys[MAXN];
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[kWaves + 2];
  const int row = blockIdx.x;
  const int n = row_count(n_valid, causal_base, row);
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    for (int r = threadIdx.x; r < K; r += kThreads) out[r] = r < n ? r : -1;
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  for (int s = threadIdx.x; s < n; s += kThreads) keys[s] = float_key(src[s]);

  // threshold search: digits [31:20], [19:8], [7:0]
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)K;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nbins = pass < 2 ? kBins : 256;
    for (int b = threadIdx.x; b < nbins; b += kThreads) hist[b] = 0;
    __syncthreads();
    const int rounds = (n + kThreads - 1) / kThreads;
    for (int r = 0; r < rounds; ++r) {
      const int s = r * kThreads + threadIdx.x;
      const uint32_t k = s < n ? keys[s] : 0u;
      hist_add(hist, s < n && (k & pmask) == prefix, (k >> shift) & (uint32_t)(nbins - 1));
    }
    __syncthreads();
    const Bucket bk = find_bucket_desc(hist, nbins, need, sh);
    prefix |= bk.bin << shift;
    pmask |= (uint32_t)(nbins - 1) << shift;
    need -= bk.above;
  }
  const uint32_t tau = prefix;

  // ordered compaction: rank = #kept at lower positions
  //                          = #(key > tau) before + min(#(key == tau) before, need)
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t gt_base = 0, eq_base = 0;
  const int rounds = (n + kThreads - 1) / kThreads;
  for (int r = 0; r < rounds; ++r) {
    const int s = r * kThreads + threadIdx.x;
    const uint32_t k = s < n ? keys[s] : 0u;
    const bool gt = s < n && k > tau;
    const bool eq = s < n && k == tau;
    // per-wave bitmasks and popcount ranks, then a block prefix of the counts
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    const uint32_t packed = (uint32_t)__popcll(mgt) | ((uint32_t)__popcll(meq) << 16);
    uint32_t tot;
    const uint32_t before = block_prefix_excl(lane == 0 ? packed : 0u, sh, &tot);
    const uint32_t wave_gt = (__shfl(before, 0) & 0xffffu) + (uint32_t)__popcll(mgt & lanemask_lt(lane));
    const uint32_t wave_eq = (__shfl(before, 0) >> 16) + (uint32_t)__popcll(meq & lanemask_lt(lane));
    const uint32_t eq_rank = eq_base + wave_eq;
    if (gt || (eq && eq_rank < need)) {
      const uint32_t pos = gt_base + wave_gt + min(eq_rank, need);
      out[pos] = s;
    }
    gt_base += tot & 0xffffu;
    eq_base += tot >> 16;
  }
}

// ================================================================ long rows

// Per-row counters of the long path.
struct RowState {
  uint32_t kept, ncand;  // outright keeps and candidates gathered
  uint32_t pad[14];
};
static_assert(sizeof(RowState) == 64, "RowState is one 64-byte slot");

struct LongWs {
  uint32_t* hist0;   // [n_q][kBins]
  uint32_t* hist1;   // [n_q][kBins]
  RowState* state;   // [n_q]
  int32_t* sel;      // [n_q][K]
  uint2* cand;       // [n_q][ld]: (key, position)
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline size_t long_ws_bytes(int n_q, int64_t ld, int K, LongWs* ws, void* base) {
  const size_t h = align_up((size_t)n_q * kBins * 4, 256);
  const size_t c = align_up((size_t)n_q * sizeof(RowState), 256);
  const size_t s = align_up((size_t)n_q * K * 4, 256);
  const size_t d = align_up((size_t)n_q * ld * 8, 256);
  if (ws) {
    char* p = (char*)base;
    ws->hist0 = (uint32_t*)p;
    ws->hist1 = (uint32_t*)(p + h);
    ws->state = (RowState*)(p + 2 * h);
    ws->sel = (int32_t*)(p + 2 * h + c);
    ws->cand = (uint2*)(p + 2 * h + c + s);
  }
  return 2 * h + c + s + d;
}

__global__ __launch_bounds__(kThreads) void topk_clear_kernel(uint32_t* p, size_t nwords) {
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nwords;
       i += (size_t)gridDim.x * kThreads)
    p[i] = 0;
}

// One 4096-position block of a row: its keys, loaded coalesced.
struct BlockKeys {
  uint32_t key[kChunk / kThreads];
  int s0, s1;
};
__device__ __forceinline__ void load_block(const float* src, int s0, int s1, BlockKeys& bk) {
  bk.s0 = s0;
  bk.s1 = s1;
#pragma unroll
  for (int i = 0; i < kChunk / kThreads; ++i) {
    const int s = s0 + threadIdx.x + i * kThreads;
    bk.key[i] = s < s1 ? float_key(src[s]) : 0u;
  }
}

// block-wise scoring of the top digit (key bits [31:20])
__global__ __launch_bounds__(kThreads) void topk_hist0_kernel(const float* __restrict__ scores,
                                                              int64_t ld,
                                                              const int32_t* __restrict__ n_valid,
                                                              int causal_base, int K, LongWs ws) {
  __shared__ uint32_t hist[kBins];
  const int row = blockIdx.y;
  const int n = row_count(n_valid, causal_base, row);
  const int s0 = blockIdx.x * kChunk;
  if (n <= K || s0 >= n) return;
  for (int b = threadIdx.x; b < kBins; b += kThreads) hist[b] = 0;
  BlockKeys bk;
  load_block(scores + (int64_t)row * ld, s0, min(s0 + kChunk, n), bk);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kChunk / kThreads; ++i)
    hist_add(hist, s0 + (int)threadIdx.x + i * kThreads < bk.s1, bk.key[i] >> 20);
  __syncthreads();
  uint32_t* g = ws.hist0 + (size_t)row * kBins;
  for (int b = threadIdx.x; b < kBins; b += kThreads)
    if (hist[b]) atomicAdd(&g[b], hist[b]);
}

// second digit (bits [19:8]) of the keys whose top digit is tau's; every
// workgroup locates that top digit itself from the merged histogram
__global__ __launch_bounds__(kThreads) void topk_hist1_kernel(const float* __restrict__ scores,
                                                              int64_t ld,
                                                              const int32_t* __restrict__ n_valid,
                                                              int causal_base, int K, LongWs ws) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t sh[kWaves + 2];
  const int row = blockIdx.y;
  const int n = row_count(n_valid, causal_base, row);
  const int s0 = blockIdx.x * kChunk;
  if (n <= K || s0 >= n) return;
  for (int b = threadIdx.x; b < kBins; b += kThreads) hist[b] = 0;
  BlockKeys bk;
  load_block(scores + (int64_t)row * ld, s0, min(s0 + kChunk, n), bk);
  const Bucket b0 = find_bucket_desc(ws.hist0 + (size_t)row * kBins, kBins, (uint32_t)K, sh);
#pragma unroll
  for (int i = 0; i < kChunk / kThreads; ++i)
    hist_add(hist, s0 + (int)threadIdx.x + i * kThreads < bk.s1 && (bk.key[i] >> 20) == b0.bin,
             (bk.key[i] >> 8) & (kBins - 1));
  __syncthreads();
  uint32_t* g = ws.hist1 + (size_t)row * kBins;
  for (int b = threadIdx.x; b < kBins; b += kThreads)
    if (hist[b]) atomicAdd(&g[b], hist[b]);
}

// Wave-aggregated append: lanes with `pred` get consecutive slots from *ctr.
__device__ __forceinline__ uint32_t wave_append(uint32_t* ctr, bool pred) {
  const uint64_t m = __ballot(pred);
  if (m == 0) return 0;
  const int lane = threadIdx.x & (kWave - 1);
  const int leader = __ffsll((unsigned long long)m) - 1;
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(ctr, (uint32_t)__popcll(m));
  base = __shfl(base, leader);
  return base + (uint32_t)__popcll(m & lanemask_lt(lane));
}

// Final step of a row: settle the last 8 key bits and the ties among the
// candidates, then write the kept positions in ascending order (an LDS
// bitonic network over <= 2048 positions).
__device__ void topk_finish_row(int K, uint32_t tau24, uint32_t need1, uint32_t kept,
                                uint32_t ncand, const int32_t* sel, const uint2* cand_g,
                                int32_t* out, uint32_t* hist, int32_t* list, uint2* cand_lds,
                                uint32_t cand_cap, uint32_t* sh, uint32_t* nlist) {
  const uint2* cand = cand_g;
  if (ncand <= cand_cap) {  // generic pointer: the passes below read LDS instead of global
    for (uint32_t c = threadIdx.x; c < ncand; c += kThreads) cand_lds[c] = cand_g[c];
    cand = cand_lds;
  }
  for (uint32_t r = threadIdx.x; r < kept; r += kThreads) list[r] = sel[r];
  if (threadIdx.x == 0) *nlist = kept;
  for (int b = threadIdx.x; b < 256; b += kThreads) hist[b] = 0;
  __syncthreads();

  // last digit (bits [7:0]) over the candidates
  for (uint32_t c = threadIdx.x; c - threadIdx.x < ncand; c += kThreads) {
    const bool ok = c < ncand;
    hist_add(hist, ok, (ok ? cand[c].x : 0u) & 255u);
  }
  __syncthreads();
  const Bucket b2 = find_bucket_desc(hist, 256, need1, sh);
  const uint32_t tau = (tau24 << 8) | b2.bin;
  const uint32_t need2 = need1 - b2.above;  // ties at tau to keep, lowest positions first
  const uint32_t nties = hist[b2.bin];
  __syncthreads();

  // lowest `need2` tie positions: an ascending radix search over position
  // bits [30:20], [19:10], [9:0]
  uint32_t pmax = 0xffffffffu;  // keep ties with position <= pmax
  if (need2 < nties) {
    uint32_t prefix = 0, pmask = 0, want = need2;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 10 : 0);
      const int nb = pass == 0 ? 2048 : 1024;
      for (int b = threadIdx.x; b < nb; b += kThreads) hist[b] = 0;
      __syncthreads();
      for (uint32_t c = threadIdx.x; c - threadIdx.x < ncand; c += kThreads) {
        const bool ok = c < ncand;
        const uint2 e = ok ? cand[c] : make_uint2(0u, 0u);
        const bool t = ok && e.x == tau && (e.y & pmask) == prefix;
        hist_add(hist, t, (e.y >> shift) & (uint32_t)(nb - 1));
      }
      __syncthreads();
      const Bucket bp = find_bucket_asc(hist, nb, want, sh);
      prefix |= bp.bin << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      want -= bp.above;
    }
    pmax = prefix;
  }

  // add the kept candidates to the outright ones
  for (uint32_t c = threadIdx.x; c - threadIdx.x < ncand; c += kThreads) {
    const bool ok = c < ncand;
    const uint2 e = ok ? cand[c] : make_uint2(0u, 0u);
    const bool take = ok && (e.x > tau || (e.x == tau && e.y <= pmax));
    const uint32_t a = wave_append(nlist, take);
    if (take) list[a] = (int32_t)e.y;
  }
  __syncthreads();
  // *nlist == K here; pad to a power of two and sort ascending
  int P = 1;
  while (P < K) P <<= 1;
  for (int r = K + threadIdx.x; r < P; r += kThreads) list[r] = 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < P / 2; t += kThreads) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const int32_t a = list[i], b = list[j];
        if ((a > b) == up) {
          list[i] = b;
          list[j] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int r = threadIdx.x; r < K; r += kThreads) out[r] = list[r];
}

// cross-block merge, part 1: keys above tau's 24-bit prefix are kept
// outright and keys sharing it are gathered as candidates; each workgroup
// counts its own and reserves its output ranges with one atomic per list.
__global__ __launch_bounds__(kThreads) void topk_collect_kernel(const float* __restrict__ scores,
                                                                int64_t ld,
                                                                const int32_t* __restrict__ n_valid,
                                                                int causal_base, int K, LongWs ws) {
  __shared__ uint32_t sh[kWaves + 2];
  __shared__ uint32_t base[2];
  const int row = blockIdx.y;
  const int n = row_count(n_valid, causal_base, row);
  const int s0 = blockIdx.x * kChunk;
  if (n <= K || s0 >= n) return;
  BlockKeys bk;
  load_block(scores + (int64_t)row * ld, s0, min(s0 + kChunk, n), bk);
  const Bucket b0 = find_bucket_desc(ws.hist0 + (size_t)row * kBins, kBins, (uint32_t)K, sh);
  const Bucket b1 =
      find_bucket_desc(ws.hist1 + (size_t)row * kBins, kBins, (uint32_t)K - b0.above, sh);
  const uint32_t p24 = (b0.bin << 12) | b1.bin;
  uint32_t nk = 0, nm = 0;
#pragma unroll
  for (int i = 0; i < kChunk / kThreads; ++i) {
    const bool ok = s0 + (int)threadIdx.x + i * kThreads < bk.s1;
    nk += (ok && (bk.key[i] >> 8) > p24) ? 1u : 0u;
    nm += (ok && (bk.key[i] >> 8) == p24) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t before = block_prefix_excl(nk | (nm << 16), sh, &tot);
  RowState* st = ws.state + row;
  if (threadIdx.x == 0) {
    base[0] = (tot & 0xffffu) ? atomicAdd(&st->kept, tot & 0xffffu) : 0u;
    base[1] = (tot >> 16) ? atomicAdd(&st->ncand, tot >> 16) : 0u;
  }
  __syncthreads();
  uint32_t ok_at = base[0] + (before & 0xffffu), om_at = base[1] + (before >> 16);
  int32_t* sel = ws.sel + (size_t)row * K;
  uint2* cand = ws.cand + (size_t)row * ld;
#pragma unroll
  for (int i = 0; i < kChunk / kThreads; ++i) {
    const int s = s0 + threadIdx.x + i * kThreads;
    if (s < bk.s1 && (bk.key[i] >> 8) > p24) sel[ok_at++] = s;
    if (s < bk.s1 && (bk.key[i] >> 8) == p24) cand[om_at++] = make_uint2(bk.key[i], (uint32_t)s);
  }
}

// cross-block merge, part 2: one workgroup per row finishes the row.
__global__ __launch_bounds__(kThreads) void topk_final_kernel(const int32_t* __restrict__ n_valid,
                                                              int causal_base, int K, int64_t ld,
                                                              LongWs ws,
                                                              int32_t* __restrict__ idx) {
  constexpr uint32_t kCandCap = 4096;  // candidates cached in LDS
  __shared__ uint32_t hist[2048];
  __shared__ int32_t list[2048];
  __shared__ uint2 cand_lds[kCandCap];
  __shared__ uint32_t sh[kWaves + 2];
  __shared__ uint32_t nlist;
  const int row = blockIdx.x;
  const int n = row_count(n_valid, causal_base, row);
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    for (int r = threadIdx.x; r < K; r += kThreads) out[r] = r < n ? r : -1;
    return;
  }
  const Bucket b0 = find_bucket_desc(ws.hist0 + (size_t)row * kBins, kBins, (uint32_t)K, sh);
  const uint32_t need0 = (uint32_t)K - b0.above;
  const Bucket b1 = find_bucket_desc(ws.hist1 + (size_t)row * kBins, kBins, need0, sh);
  const RowState* st = ws.state + row;
  topk_finish_row(K, (b0.bin << 12) | b1.bin, need0 - b1.above, st->kept, st->ncand,
                  ws.sel + (size_t)row * K, ws.cand + (size_t)row * ld, out, hist, list,
                  cand_lds, kCandCap, sh, &nlist);
}

}  // namespace
}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int32_t n_q, int64_t ld, int32_t K) {
  if (n_q < 1 || ld < 1 || K < 1) return 0;
  if (ld <= dsa::kShortMax) return 0;
  return dsa::long_ws_bytes(n_q, ld, K, nullptr, nullptr);
}

extern "C" dsa_status_t dsa_topk(const float* scores, int64_t ld, int32_t n_q, int32_t K,
                                 const int32_t* n_valid, int32_t causal_base, int32_t* idx,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace dsa;
  if (!scores || !idx) return DSA_ERR_NULL;
  if (n_q < 1 || ld < 1 || K < 1 || K > 2048) return DSA_ERR_SHAPE;
  if (ld > 0x7fffffff) return DSA_ERR_SHAPE;
  if (!n_valid && (causal_base < 0 || (int64_t)causal_base + n_q > ld)) return DSA_ERR_SHAPE;
  const size_t need = dsa_topk_workspace_size(n_q, ld, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  dsa_status_t st = check_device();
  if (st != DSA_OK) return st;
  if (ld <= kShortMax) {
    if (ld <= 4096)
      hipLaunchKernelGGL(topk_short_kernel<4096>, dim3(n_q), dim3(kThreads), 0, stream, scores,
                         ld, n_valid, causal_base, K, idx);
    else if (ld <= 8192)
      hipLaunchKernelGGL(topk_short_kernel<8192>, dim3(n_q), dim3(kThreads), 0, stream, scores,
                         ld, n_valid, causal_base, K, idx);
    else
      hipLaunchKernelGGL(topk_short_kernel<16384>, dim3(n_q), dim3(kThreads), 0, stream, scores,
                         ld, n_valid, causal_base, K, idx);
    return launch_status();
  }
  LongWs ws;
  long_ws_bytes(n_q, ld, K, &ws, workspace);
  // histograms and row states are contiguous at the start of the workspace
  const size_t zero_words = ((char*)ws.sel - (char*)ws.hist0) / 4;
  hipLaunchKernelGGL(topk_clear_kernel,
                     dim3((unsigned)std::min<size_t>(1024, (zero_words + 255) / 256)),
                     dim3(kThreads), 0, stream, ws.hist0, zero_words);
  const dim3 grid((unsigned)((ld + kChunk - 1) / kChunk), (unsigned)n_q);
  hipLaunchKernelGGL(topk_hist0_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_valid,
                     causal_base, K, ws);
  hipLaunchKernelGGL(topk_hist1_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_valid,
                     causal_base, K, ws);
  hipLaunchKernelGGL(topk_collect_kernel, grid, dim3(kThreads), 0, stream, scores, ld, n_valid,
                     causal_base, K, ws);
  hipLaunchKernelGGL(topk_final_kernel, dim3(n_q), dim3(kThreads), 0, stream, n_valid,
                     causal_base, K, ld, ws, idx);
  return launch_status();
}
