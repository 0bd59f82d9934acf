// Top-K position selection for DSA (web page "Day-0 Adaptation of
// Trillion-Parameter MoE Models on Domestic GPUs", section 3 item (1): Top-K
// as block-wise scoring, intra-block reduction and cross-block merge, with
// bitmask techniques and no global sort).
//
// Contract: row i keeps the K largest of its n_i scores, equal scores taken
// lower position first, written as ascending positions and padded with -1
// when n_i < K.
//
// Method: fp32 scores map to order-preserving 32-bit keys.  The key tau of
// the K-th largest score is found by a bitwise search: starting from the
// bits every key shares, each bit where keys differ is tried from the top,
// and kept when at least K keys are >= the candidate.  The count is made
// with wave64 ballot bitmasks and popcounts, so scores that crowd into a
// narrow range cost nothing extra.  The short candidate lists of the last
// step are searched by radix passes instead (8 bits a pass, a 256-bin LDS
// histogram per wave built with one atomic add per key): far fewer
// barriers than one per bit.  Every key above tau is kept, and of the keys
// equal to tau the `need` lowest positions; an ordered compaction
// (per-thread counts and one block prefix scan) writes the kept positions
// in ascending order.  Nothing is ever sorted.
//
// Two paths, chosen by the row capacity `ld`:
//   ld <= 16384: one workgroup per row holds the row (prefill rows);
//   ld  > 16384: decode rows of up to millions of positions, in three steps
//     block-wise scoring:    one workgroup per row searches a strided sample
//                            of 8192 keys for a lower bound that about
//                            2K + 16 n / 8192 keys clear (rows that fit in
//                            the final step's LDS list skip this: bound 0);
//     intra-block reduction: one workgroup per 4096-position chunk writes
//                            its keys at or above the bound, with their
//                            positions, in position order into the chunk's
//                            own slot (ordered ballot compaction);
//     cross-block merge:     one workgroup per row concatenates the chunk
//                            slots in chunk order and runs the exact search
//                            and ordered compaction on that short list.
//   The bound only prunes: if the list is too long for LDS, or shorter than
//   K (a sample that misled), the last step runs the same exact search over
//   the list or the whole row in global memory, so the result is always
//   exact; only the speed depends on the data.
#include <algorithm>

#include "common.h"
#include "host_util.h"

namespace dsa {
namespace {

constexpr int kShortMax = 16384;    // longest row of the one-workgroup path
constexpr int kShortThreads = 512;
constexpr int kChunk = 4096;        // positions per workgroup of the chunk step
constexpr int kChunkThreads = 256;
constexpr int kSampleThreads = 1024;  // sample step: one workgroup per row
constexpr int kRowThreads = 1024;   // merge step: one workgroup per row
constexpr int kListCap = 12288;     // list entries the merge step holds in LDS
constexpr int kSample = 8192;       // sampled keys per long row
constexpr int kMaxChunks = 4096;    // ld <= kMaxChunks * kChunk

__device__ __forceinline__ int row_count(const int32_t* n_valid, int causal_base, int row,
                                         int64_t ld) {
  const int n = n_valid ? n_valid[row] : causal_base + row + 1;
  if (kCheckBounds && (n < 0 || n > ld)) {  // device data: checked in debug builds
    raise_error(kErrLength);
    return 0;
  }
  return n;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Block-wide reductions over T threads through a double-buffered LDS area
// (`sh` holds kShWords words): one barrier per call, and two consecutive
// calls never touch the same words.
template <int T>
struct Block {
  static constexpr int kW = T / kWave;
  static constexpr int kShWords = 4 * kW;
  uint32_t* sh;
  int parity = 0;
  __device__ explicit Block(uint32_t* s) : sh(s) {}
  __device__ uint32_t* buf() {
    uint32_t* b = sh + parity * 2 * kW;
    parity ^= 1;
    return b;
  }
  // Sum of one value per wave (uniform within each wave).
  __device__ uint32_t sum_waves(uint32_t wave_value) {
    uint32_t* b = buf();
    if ((threadIdx.x & (kWave - 1)) == 0) b[threadIdx.x / kWave] = wave_value;
    __syncthreads();
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) s += b[w];
    return s;
  }
  __device__ uint32_t sum(uint32_t v) { return sum_waves(wave_sum(v)); }
  // AND and OR of one value per thread.
  __device__ void and_or(uint32_t& a, uint32_t& o) {
    a = wave_and(a);
    o = wave_or(o);
    uint32_t* b = buf();
    if ((threadIdx.x & (kWave - 1)) == 0) {
      b[threadIdx.x / kWave] = a;
      b[kW + threadIdx.x / kWave] = o;
    }
    __syncthreads();
    a = 0xffffffffu;
    o = 0u;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      a &= b[w];
      o |= b[kW + w];
    }
  }
  // Exclusive prefix sum in thread order, and the block total.
  __device__ uint32_t prefix_excl(uint32_t v, uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const uint32_t incl = wave_incl_add(v);
    uint32_t* b = buf();
    if (lane == kWave - 1) b[wave] = incl;
    __syncthreads();
    uint32_t lower = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      lower += w < wave ? b[w] : 0u;
      all += b[w];
    }
    *total = all;
    return incl - v + lower;
  }
};

// Keep every key above tau and the first `need` keys equal to tau.
struct Threshold {
  uint32_t tau, need;
};

// Exact K-th largest key (1 <= K <= number of keys) by the bitwise search.
// (a, o): this thread's AND and OR over its keys (all-ones / 0 for none);
// wave_ge(c): this wave's number of keys >= c (uniform in the wave).  Keys
// are never 0 (0 marks an empty slot), and every candidate is >= 1.
template <int T, class WaveGE>
__device__ Threshold select_tau(Block<T>& blk, uint32_t a, uint32_t o, WaveGE wave_ge,
                                uint32_t K) {
  blk.and_or(a, o);
  uint32_t prefix = a;      // bits every key has set
  uint32_t diff = a ^ o;    // bits where keys differ
  while (diff) {
    const uint32_t bit = 1u << (31 - __clz(diff));
    diff &= ~bit;
    if (blk.sum_waves(wave_ge(prefix | bit)) >= K) prefix |= bit;
  }
  const uint32_t gt = prefix == 0xffffffffu ? 0u : blk.sum_waves(wave_ge(prefix + 1u));
  return Threshold{prefix, K - gt};
}

// Wave total of (key >= c) over R register keys: one ballot per key.
template <int R>
struct RegCount {
  const uint32_t (&k)[R];
  __device__ uint32_t operator()(uint32_t c) const {
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < R; ++i) n += (uint32_t)__popcll(__ballot(k[i] >= c));
    return n;
  }
};

// The same threshold by radix passes: from the highest bit where the keys
// differ, 8 bits at a time, every thread adds its live keys (those equal to
// the prefix on every bit decided so far) to its wave's 256-bin histogram
// of the next digit in LDS (one atomic add per key), and a suffix sum over
// the bins picks the digit that holds the K-th largest; the keys of higher
// digits are counted as above every later candidate.  Thread t holds the
// keys k[i] of the slots where valid(i) (uniform; 0 marks an empty slot,
// never counted).  With stop > 0 the search ends as soon as at most `stop`
// keys reach the value decided so far (lower bits as in the prefix): that
// value, which at least K keys reach, is returned as tau (need is then
// meaningless).  `hist` holds 256 words per wave, `bc` 7 words; four
// barriers a pass.
// on_pass(prefix) runs (in every thread) after each pass with the value
// decided so far.
struct NoPass {
  __device__ void operator()(uint32_t) const {}
};
template <int T, int R, class Valid, class OnPass = NoPass>
__device__ Threshold radix_select_tau(Block<T>& blk, const uint32_t (&k)[R], Valid valid,
                                      uint32_t K, uint32_t stop, uint32_t* hist, uint32_t* bc,
                                      OnPass on_pass = OnPass()) {
  constexpr int W = T / kWave;
  static_assert(T >= 256, "one thread per bin");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t a = 0xffffffffu, o = 0u;
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (valid(i) && k[i]) {
      a &= k[i];
      o |= k[i];
    }
  blk.and_or(a, o);
  uint32_t prefix = a, diff = a ^ o, above = 0;
  while (diff) {
    const int hi = 31 - __clz(diff), lo = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (hi == 31 ? 0xffffffffu : (2u << hi) - 1u) & ~((1u << lo) - 1u);
    const uint32_t M = hi == 31 ? 0u : ~((2u << hi) - 1u);  // the bits decided
    const uint32_t pm = prefix & M;
    for (int j = threadIdx.x; j < 256 * W; j += T) hist[j] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (valid(i) && k[i] != 0u && (k[i] & M) == pm)
        atomicAdd(&hist[256 * wave + ((k[i] & dmask) >> lo)], 1u);
    __syncthreads();
    // thread t < 256 takes digit 255 - t: its keys, then (a prefix over the
    // threads) the keys of digits >= 255 - t, within the wave and then
    // across the four waves
    uint32_t tot = 0, suf = 0;
    if (threadIdx.x < 256) {
      const int b = 255 - (int)threadIdx.x;
#pragma unroll
      for (int w = 0; w < W; ++w) tot += hist[256 * w + b];
      suf = wave_incl_add(tot);
      if (lane == kWave - 1) bc[wave] = suf;  // wave total (digits 255 - 64 wave down)
    }
    __syncthreads();
    const uint32_t need = K - above;
    if (threadIdx.x < 256) {
      for (int w = 0; w < wave; ++w) suf += bc[w];
      // the digit: the largest whose keys and those above reach need
      if (suf >= need && suf - tot < need) {
        bc[4] = 255u - threadIdx.x;
        bc[5] = suf - tot;  // keys of higher digits
        bc[6] = suf;        // keys of this digit and higher ones
      }
    }
    __syncthreads();
    const uint32_t digit = bc[4], reach = above + bc[6];  // keys >= the new prefix
    above += bc[5];
    prefix = (prefix & ~dmask) | (digit << lo);
    diff &= ~dmask;
    __syncthreads();  // bc and hist are rewritten by the next pass
    on_pass(prefix);
    if (stop && reach <= stop) break;
  }
  return Threshold{prefix, K - above};
}

template <int R>
__device__ __forceinline__ void thread_and_or(const uint32_t (&k)[R], uint32_t& a, uint32_t& o) {
  a = 0xffffffffu;
  o = 0u;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (k[i]) {
      a &= k[i];
      o |= k[i];
    }
  }
}

// Ordered compaction of a list of m < 65536 entries (key, position) in
// list order: thread t takes the contiguous run t R .. t R + R - 1 (R odd,
// so the lanes' LDS reads spread over the banks), and one block prefix of
// the per-thread counts gives each run its output slots:
//   slot = #(key > tau) before + min(#(key == tau) before, need).
template <int T, class Entry>
__device__ __forceinline__ void ordered_compact(Block<T>& blk, uint32_t m, Threshold th,
                                                Entry entry, int32_t* __restrict__ out) {
  const uint32_t R = ((m + T - 1) / T) | 1u;
  const uint32_t first = threadIdx.x * R;
  uint32_t gt = 0, eq = 0;
  for (uint32_t i = 0; i < R; ++i) {
    const uint32_t e = first + i;
    if (e < m) {
      const uint32_t k = entry(e).x;
      gt += k > th.tau ? 1u : 0u;
      eq += k == th.tau ? 1u : 0u;
    }
  }
  uint32_t tot;
  const uint32_t before = blk.prefix_excl(gt | (eq << 16), &tot);
  uint32_t g = before & 0xffffu, q = before >> 16;
  for (uint32_t i = 0; i < R; ++i) {
    const uint32_t e = first + i;
    if (e < m) {
      const uint2 v = entry(e);
      if (v.x > th.tau) {
        out[g + min(q, th.need)] = (int32_t)v.y;
        ++g;
      } else if (v.x == th.tau) {
        if (q < th.need) out[g + q] = (int32_t)v.y;
        ++q;
      }
    }
  }
}

__device__ __forceinline__ void write_all(int n, int K, int32_t* __restrict__ out, int T) {
  for (int r = threadIdx.x; r < K; r += T) out[r] = r < n ? r : -1;
}

// ================================================================ short rows

template <int MAXN>
__global__ __launch_bounds__(kShortThreads) void topk_short_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_valid,
    int causal_base, int K, int32_t* __restrict__ idx) {
  constexpr int T = kShortThreads, R = MAXN / T;
  __shared__ uint32_t keys[MAXN];
  __shared__ uint32_t sh[Block<T>::kShWords];
  const int row = blockIdx.x;
  const int n = row_count(n_valid, causal_base, row, ld);
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    write_all(n, K, out, T);
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  // thread t holds positions t + T i (all loads in flight together)
  float v[R];
#pragma unroll
  for (int i = 0; i < R; ++i) v[i] = src[min((int)threadIdx.x + T * i, n - 1)];
  uint32_t k[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int p = threadIdx.x + T * i;
    k[i] = p < n ? float_key(v[i]) : 0u;
    if (p < n) keys[p] = k[i];
  }
  uint32_t a, o;
  thread_and_or(k, a, o);
  Block<T> blk(sh);
  const Threshold th =
      select_tau(blk, a, o, RegCount<R>{k}, (uint32_t)K);
  __syncthreads();
  ordered_compact(blk, (uint32_t)n, th, [&](uint32_t e) { return make_uint2(keys[e], e); }, out);
}

// ================================================================ long rows

struct LongWs {
  uint32_t* lower;   // [n_q] the sample's lower bound on the kept keys
  uint32_t* count;   // [n_q][n_chunks] list entries each chunk wrote
  uint2* list;       // [n_q][ld] chunk c's entries (key, position) from c * kChunk
  int n_chunks;
};

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline size_t long_ws_bytes(int n_q, int64_t ld, LongWs* ws, void* base) {
  const int n_chunks = (int)((ld + kChunk - 1) / kChunk);
  const size_t lo = align_up((size_t)n_q * 4, 256);
  const size_t c = align_up((size_t)n_q * n_chunks * 4, 256);
  const size_t l = align_up((size_t)n_q * ld * 8, 256);
  if (ws) {
    char* p = (char*)base;
    ws->lower = (uint32_t*)p;
    ws->count = (uint32_t*)(p + lo);
    ws->list = (uint2*)(p + lo + c);
    ws->n_chunks = n_chunks;
  }
  return lo + c + l;
}

// block-wise scoring: the lower bound of a row from a strided sample of its
// keys (2048 groups of four consecutive positions, group g starting at
// floor(4 g n / 8192)); about r = 2 K 8192 / n + 16 sampled keys clear it, so
// about n r / 8192 keys of the row do
__global__ __launch_bounds__(kSampleThreads) void topk_sample_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_valid,
    int causal_base, int K, LongWs ws) {
  constexpr int T = kSampleThreads, R = kSample / T;
  __shared__ uint32_t sh[Block<T>::kShWords];
  const int row = blockIdx.x;
  const int n = row_count(n_valid, causal_base, row, ld);
  if (n <= K) return;
  if (n <= kListCap) {  // the whole row fits the merge step's list
    if (threadIdx.x == 0) ws.lower[row] = 0u;
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  // kSample / 4 groups of four consecutive keys, group g from floor(4 g n / kSample)
  float v[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t g = threadIdx.x + T * (i >> 2);
    v[i] = src[g * 4 * n / kSample + (i & 3)];
  }
  uint32_t k[R];
#pragma unroll
  for (int i = 0; i < R; ++i) k[i] = float_key(v[i]);
  const int64_t expect = ((int64_t)kSample * K + n - 1) / n;
  const uint32_t r = (uint32_t)std::min<int64_t>(kSample, 2 * expect + 16);
  uint32_t a, o;
  thread_and_or(k, a, o);
  Block<T> blk(sh);
  const Threshold th = select_tau(blk, a, o, RegCount<R>{k}, r);
  if (threadIdx.x == 0) ws.lower[row] = th.tau;
}

// intra-block reduction: the chunk's keys at or above the row's bound, in
// position order, into the chunk's slot of the row's list.  Slot i = 4 j + e
// of thread t holds position s0 + 1024 j + 4 t + e, so each load instruction
// of a wave reads 1 KB of contiguous scores (16 bytes a lane when VEC) and
// (j, t, e) order is position order; loads carry no branches (an address
// past the row end is clamped and its key discarded).
template <bool VEC>
__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_valid,
    int causal_base, int K, LongWs ws) {
  constexpr int T = kChunkThreads;
  static_assert(kChunk == 16 * T, "chunk layout: 16 keys per thread");
  __shared__ uint32_t sh[Block<T>::kShWords];
  const int row = blockIdx.y;
  const int s0 = blockIdx.x * kChunk;
  const float* src = scores + (int64_t)row * ld;
  // the loads address only the row's ld slots, so they go out together with
  // the read of the row length instead of after it
  float v[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int p = s0 + 4 * T * j + 4 * (int)threadIdx.x;
    if (VEC) {  // ld % 4 == 0: p < ld implies p + 3 < ld
      const float4 x = *(const float4*)(src + (p < ld ? p : 0));
      v[4 * j] = x.x;
      v[4 * j + 1] = x.y;
      v[4 * j + 2] = x.z;
      v[4 * j + 3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = src[min((int64_t)(p + e), ld - 1)];
    }
  }
  const int n = row_count(n_valid, causal_base, row, ld);
  if (n <= K || s0 >= n) return;
  const int s1 = min(s0 + kChunk, n);
  const uint32_t lower = ws.lower[row];
  uint32_t key[16];
  uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = s0 + 4 * T * (i >> 2) + 4 * (int)threadIdx.x + (i & 3);
    key[i] = p < s1 ? float_key(v[i]) : 0u;
    const bool keep = p < s1 && key[i] >= lower;
    c[i >> 2] += keep ? 1u : 0u;
    if (!keep) key[i] = 0u;
  }
  // offsets in (j, t, e) order: two block scans of two 16-bit counts each
  Block<T> blk(sh);
  uint32_t t01, t23;
  const uint32_t b01 = blk.prefix_excl(c[0] | (c[1] << 16), &t01);
  const uint32_t b23 = blk.prefix_excl(c[2] | (c[3] << 16), &t23);
  const uint32_t r0 = t01 & 0xffffu, r1 = t01 >> 16, r2 = t23 & 0xffffu, r3 = t23 >> 16;
  const uint32_t start[4] = {b01 & 0xffffu, r0 + (b01 >> 16), r0 + r1 + (b23 & 0xffffu),
                             r0 + r1 + r2 + (b23 >> 16)};
  uint2* dst = ws.list + (size_t)row * ld + s0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t at = start[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * j + e;
      if (key[i]) {
        const int p = s0 + 4 * T * j + 4 * (int)threadIdx.x + e;
        dst[at++] = make_uint2(key[i], (uint32_t)p);
      }
    }
  }
  const uint32_t total = r0 + r1 + r2 + r3;
  if (threadIdx.x == 0) ws.count[(size_t)row * ws.n_chunks + blockIdx.x] = total;
}

// cross-block merge: one workgroup per row
__global__ __launch_bounds__(kRowThreads) void topk_merge_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ n_valid,
    int causal_base, int K, LongWs ws, int32_t* __restrict__ idx) {
  constexpr int T = kRowThreads, R = kListCap / T;
  __shared__ uint2 ent[kListCap];
  __shared__ uint32_t off[kMaxChunks + 1];  // list offset of each chunk, then the total
  __shared__ uint32_t sh[Block<T>::kShWords];
  __shared__ uint32_t bc[8];
  const int row = blockIdx.x;
  const int n = row_count(n_valid, causal_base, row, ld);
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    write_all(n, K, out, T);
    return;
  }
  Block<T> blk(sh);
  const int nch = (n + kChunk - 1) / kChunk;
  const uint32_t* cnt = ws.count + (size_t)row * ws.n_chunks;
  uint32_t m = 0;
  for (int c0 = 0; c0 < ws.n_chunks; c0 += T) {  // chunks past the row end count 0
    const int c = c0 + threadIdx.x;
    uint32_t total;
    const uint32_t v = c < ws.n_chunks ? cnt[c] : 0u;
    const uint32_t before = blk.prefix_excl(c < nch ? v : 0u, &total);
    if (c < nch) off[c] = m + before;
    m += total;
  }
  if (threadIdx.x == 0) off[nch] = m;
  __syncthreads();
  const uint2* list = ws.list + (size_t)row * ld;
  // list entry e: chunk c = the last with off[c] <= e (fixed-step binary search)
  auto list_index = [&](uint32_t e) -> size_t {
    int c = 0;
#pragma unroll
    for (int step = kMaxChunks / 2; step >= 1; step >>= 1)
      if (c + step < nch && off[c + step] <= e) c += step;
    return (size_t)c * kChunk + (e - off[c]);
  };

  if (m >= (uint32_t)K && m <= (uint32_t)kListCap) {
    // thread t gathers the contiguous run of entries t rr .. t rr + rr - 1:
    // one binary search for its first entry, then a walk over the chunks
    const uint32_t rr = (m + T - 1) / T, first = threadIdx.x * rr;
    int c = 0;
#pragma unroll
    for (int step = kMaxChunks / 2; step >= 1; step >>= 1)
      if (c + step < nch && off[c + step] <= first) c += step;
    size_t at[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t e = first + i;
      at[i] = 0;
      if ((uint32_t)i < rr && e < m) {
        while (off[c + 1] <= e) ++c;
        at[i] = (size_t)c * kChunk + (e - off[c]);
      }
    }
    uint2 g[R];
#pragma unroll
    for (int i = 0; i < R; ++i) g[i] = list[at[i]];  // all in flight together
    uint32_t k[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t e = first + i;
      const bool ok = (uint32_t)i < rr && e < m;
      k[i] = ok ? g[i].x : 0u;
      if (ok) ent[e] = g[i];
    }
    // the chunk offsets are no longer needed: their words hold the histograms
    __syncthreads();
    const Threshold th =
        radix_select_tau(blk, k, [&](int i) { return i < (int)rr; }, (uint32_t)K, 0u, off, bc);
    ordered_compact(blk, m, th, [&](uint32_t e) { return ent[e]; }, out);
    return;
  }

  // Fallback, straight from global memory: the list when it holds at least
  // K entries (every key >= the K-th largest is in it), else the whole row.
  const bool use_list = m >= (uint32_t)K;
  const uint32_t mm = use_list ? m : (uint32_t)n;
  const float* src = scores + (int64_t)row * ld;
  auto entry = [&](uint32_t e) -> uint2 {
    return use_list ? list[list_index(e)] : make_uint2(float_key(src[e]), e);
  };
  uint32_t a = 0xffffffffu, o = 0u;
  for (uint32_t e = threadIdx.x; e < mm; e += T) {
    const uint32_t k = entry(e).x;
    a &= k;
    o |= k;
  }
  auto wave_ge = [&](uint32_t c) {
    uint32_t n_ge = 0;
    for (uint32_t e = threadIdx.x; e < mm; e += T) n_ge += entry(e).x >= c ? 1u : 0u;
    return wave_sum(n_ge);
  };
  const Threshold th = select_tau(blk, a, o, wave_ge, (uint32_t)K);
  // ordered compaction in rounds of T entries (the list may exceed 65535)
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t gt_base = 0, eq_base = 0;
  for (uint32_t e0 = 0; e0 < mm; e0 += T) {
    const uint32_t e = e0 + threadIdx.x;
    const uint2 v = e < mm ? entry(e) : make_uint2(0u, 0u);
    const bool gt = e < mm && v.x > th.tau;
    const bool eq = e < mm && v.x == th.tau;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    const uint32_t packed = (uint32_t)__popcll(mgt) | ((uint32_t)__popcll(meq) << 16);
    uint32_t tot;
    const uint32_t before = blk.prefix_excl(lane == 0 ? packed : 0u, &tot);
    const uint32_t b0 = __builtin_amdgcn_readlane(before, 0);
    const uint32_t wave_gt = (b0 & 0xffffu) + (uint32_t)__popcll(mgt & lanemask_lt(lane));
    const uint32_t wave_eq = (b0 >> 16) + (uint32_t)__popcll(meq & lanemask_lt(lane));
    const uint32_t eq_rank = eq_base + wave_eq;
    if (gt || (eq && eq_rank < th.need)) out[gt_base + wave_gt + min(eq_rank, th.need)] = (int32_t)v.y;
    gt_base += tot & 0xffffu;
    eq_base += tot >> 16;
  }
}

// ================================================================ fused decode rows
//
// The Top-K half of dsa_index_topk_decode.  The index kernel has already
// done the block-wise scoring: for every 16-position group g of a row it
// wrote the group's largest score m1[g] and second largest m2[g].  One
// workgroup per row then
//   1. takes a value that at least K of the group maxima reach (the K-th
//      largest, found to within 25% of K candidates): the maxima are scores
//      of distinct positions, so at least K scores of the row reach it, it
//      bounds the row's K-th largest score from below, and every kept
//      position lies in a group whose maximum reaches it (intra-block
//      reduction).  Rows of fewer than 4 K groups use both m1 and m2;
//   2. lists, in position order, the groups that reach the bound, then the
//      scores of those groups that reach it (ordered compaction; a thread
//      reads whole groups, 64 bytes each, all of its loads in flight at once);
//   3. runs the exact threshold search (radix passes) and ordered
//      compaction on that list (cross-block merge).
// A hint (the row's K-th largest key of an earlier call, kept in the
// workspace) replaces step 1's search when at least K and at most 2 K of the
// group maxima reach it.  When a list would overflow LDS the row is selected
// exactly from global memory instead.  Rows of at most 16384 candidates are
// selected whole, in registers.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedList = 12288;    // list entries held in LDS
constexpr int kFusedGroups = 4096;   // candidate groups held in LDS
constexpr int kFusedShort = 16384;   // rows up to this are selected whole
constexpr int kMaxSlots = 16;        // group slots per thread (the largest RG)

struct GroupMaxIn {
  const float* m1;
  const float* m2;
  int64_t ldg;
  uint32_t* tau;  // [n_q] K-th largest key of each row (written; read as a hint when seeded)
  int seed;
};

__device__ __forceinline__ uint32_t key_or_empty(float f) {
  return f == f ? float_key(f) : 0u;  // NaN marks "no value"
}

// Exact selection of a row straight from global memory (the fallback).
template <int T>
__device__ uint32_t select_row_global(Block<T>& blk, const float* __restrict__ src, uint32_t n,
                                      uint32_t K, int32_t* __restrict__ out) {
  uint32_t a = 0xffffffffu, o = 0u;
  for (uint32_t e = threadIdx.x; e < n; e += T) {
    const uint32_t k = float_key(src[e]);
    a &= k;
    o |= k;
  }
  auto wave_ge = [&](uint32_t c) {
    uint32_t n_ge = 0;
    for (uint32_t e = threadIdx.x; e < n; e += T) n_ge += float_key(src[e]) >= c ? 1u : 0u;
    return wave_sum(n_ge);
  };
  const Threshold th = select_tau(blk, a, o, wave_ge, K);
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t gt_base = 0, eq_base = 0;
  for (uint32_t e0 = 0; e0 < n; e0 += T) {
    const uint32_t e = e0 + threadIdx.x;
    const uint32_t k = e < n ? float_key(src[e]) : 0u;
    const bool gt = e < n && k > th.tau;
    const bool eq = e < n && k == th.tau;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    const uint32_t packed = (uint32_t)__popcll(mgt) | ((uint32_t)__popcll(meq) << 16);
    uint32_t tot;
    const uint32_t before = blk.prefix_excl(lane == 0 ? packed : 0u, &tot);
    const uint32_t b0 = __builtin_amdgcn_readlane(before, 0);
    const uint32_t wave_gt = (b0 & 0xffffu) + (uint32_t)__popcll(mgt & lanemask_lt(lane));
    const uint32_t wave_eq = (b0 >> 16) + (uint32_t)__popcll(meq & lanemask_lt(lane));
    const uint32_t eq_rank = eq_base + wave_eq;
    if (gt || (eq && eq_rank < th.need)) out[gt_base + wave_gt + min(eq_rank, th.need)] = (int32_t)e;
    gt_base += tot & 0xffffu;
    eq_base += tot >> 16;
  }
  return th.tau;
}

// Offsets of an ordered compaction whose items are laid out slot-major:
// item (i, t) = slot i of thread t comes before (i, t + 1) and (i + 1, 0).
// c[i]: the entries item (i, this thread) contributes; off[i] receives its
// first entry's position; returns the total.  Slots i >= n_slots (uniform)
// are ignored.  `sc` holds R * kFusedWaves + 1 words; two barriers.
template <int R>
__device__ uint32_t slot_major_offsets(const uint32_t (&c)[R], int n_slots, uint32_t (&off)[R],
                                       uint32_t* sc) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t incl[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (i < n_slots) {
      incl[i] = wave_incl_add(c[i]);
      if (lane == kWave - 1) sc[i * kFusedWaves + wave] = incl[i];
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of the n_slots * 16 wave totals, in place
    const int n = n_slots * kFusedWaves;
    const int per = (n + kWave - 1) / kWave;
    uint32_t run = 0;
    for (int e = lane * per; e < min(n, lane * per + per); ++e) run += sc[e];
    const uint32_t x = wave_incl_add(run);
    uint32_t acc = x - run;
    for (int e = lane * per; e < min(n, lane * per + per); ++e) {
      const uint32_t v = sc[e];
      sc[e] = acc;
      acc += v;
    }
    if (lane == kWave - 1) sc[n] = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < R; ++i)
    if (i < n_slots) off[i] = sc[i * kFusedWaves + wave] + incl[i] - c[i];
  return sc[n_slots * kFusedWaves];
}

template <int RG>
__global__ __launch_bounds__(kFusedThreads) void topk_fused_kernel(
    const float* __restrict__ scores, int64_t ld, const int32_t* __restrict__ counts,
    int count_add, int K, GroupMaxIn gm, int32_t* __restrict__ idx) {
  constexpr int T = kFusedThreads;
  __shared__ uint2 ent[kFusedList];
  __shared__ uint32_t cg[kFusedGroups];
  __shared__ uint32_t sc[kMaxSlots * kFusedWaves + 1];
  __shared__ uint32_t sh[Block<T>::kShWords];
  const int row = blockIdx.x;
  // candidates 0 .. n - 1: the sequence length, or the query position + 1
  const int n = row_count(counts, 0, row, ld - count_add) + count_add;
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    write_all(n, K, out, T);
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  Block<T> blk(sh);

  if (n <= kFusedShort) {  // the whole row in registers, 16 keys a thread
    constexpr int R = kFusedShort / T;
    uint32_t* keys = (uint32_t*)ent;
    float v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) v[i] = src[min((int)threadIdx.x + T * i, n - 1)];
    uint32_t k[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int p = threadIdx.x + T * i;
      k[i] = p < n ? float_key(v[i]) : 0u;
      if (p < n) keys[p] = k[i];
    }
    uint32_t a, o;
    thread_and_or(k, a, o);
    const Threshold th = select_tau(blk, a, o, RegCount<R>{k}, (uint32_t)K);
    __syncthreads();
    ordered_compact(blk, (uint32_t)n, th, [&](uint32_t e) { return make_uint2(keys[e], e); },
                    out);
    if (threadIdx.x == 0) gm.tau[row] = th.tau;
    return;
  }

  // ---- 1. bound.  Group j = slot i * T + t of thread t (consecutive lanes
  // read consecutive groups; rows have at most RG * T groups).
  const int G = (n + 15) >> 4;
  const int n_slots = (G + T - 1) / T;  // uniform
  const bool two = G < 4 * K;           // both maxima of each group
  const float* m1 = gm.m1 + (int64_t)row * gm.ldg;
  const float* m2 = gm.m2 + (int64_t)row * gm.ldg;
  uint32_t k1[RG], k2[RG];
  {
    float a1[RG], a2[RG];  // unconditional loads from clamped addresses, masked afterwards
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int j = min(i * T + (int)threadIdx.x, G - 1);
      a1[i] = i < n_slots ? m1[j] : 0.f;
      a2[i] = i < n_slots && two ? m2[j] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const bool live = i < n_slots && i * T + (int)threadIdx.x < G;
      k1[i] = live ? key_or_empty(a1[i]) : 0u;
      k2[i] = live && two ? key_or_empty(a2[i]) : 0u;
    }
  }
  // keys >= c among the live slots (n_slots is uniform: no wasted ballots)
  auto count_ge = [&](uint32_t c) {
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < RG; ++i)
      if (i < n_slots)
        cnt += (uint32_t)__popcll(__ballot(k1[i] >= c)) + (uint32_t)__popcll(__ballot(k2[i] >= c));
    return cnt;
  };
  uint32_t bound = 0;
  bool have = false;
  // After the bound's first radix pass every candidate group has its
  // maximum at or above the value decided so far: one score of each such
  // group is loaded then, so that the expansion's loads find its lines in
  // cache.  The values are not used (an empty asm statement keeps the loads).
  float pfv[RG] = {};
  bool pf_done = false;
  if (gm.seed) {  // a hint: valid if at least K maxima reach it, useful if at most 2 K do
    const uint32_t hint = gm.tau[row];
    if (hint != 0u) {
      const uint32_t c = blk.sum_waves(count_ge(hint));
      if (c >= (uint32_t)K && c <= 2u * (uint32_t)K) {
        bound = hint;
        have = true;
      }
    }
  }
  if (!have) {
    // radix passes towards the K-th largest key, stopped once at most 5 K / 4
    // keys reach the value decided (any value that K keys reach is a valid
    // bound)
    uint32_t kk[2 * RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      kk[i] = k1[i];
      kk[RG + i] = k2[i];
    }
    auto touch = [&](uint32_t pre) {  // after the first pass only
      if (pf_done) return;
      pf_done = true;
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        const int j = i * T + (int)threadIdx.x;
        pfv[i] = i < n_slots && j < G && k1[i] != 0u && k1[i] >= pre ? src[16 * j] : 0.f;
      }
    };
    bound = radix_select_tau(blk, kk, [&](int i) { return (i % RG) < n_slots; }, (uint32_t)K,
                             (uint32_t)K + (uint32_t)K / 4, cg, sc, touch).tau;
  }

  // ---- 2a. candidate groups (maximum >= bound), in position order
  uint32_t off[RG], flag[RG];
#pragma unroll
  for (int i = 0; i < RG; ++i) flag[i] = i < n_slots && k1[i] >= bound && k1[i] != 0u ? 1u : 0u;
  const uint32_t m_g = slot_major_offsets(flag, n_slots, off, sc);
  const bool fit = m_g <= (uint32_t)kFusedGroups;
  if (fit) {
#pragma unroll
    for (int i = 0; i < RG; ++i)
      if (i < n_slots && flag[i]) cg[off[i]] = (uint32_t)(i * T + (int)threadIdx.x);
  }
  __syncthreads();

  // ---- 2c. the listed groups' scores that reach the bound: thread t takes
  // listed groups t, t + T, ... (16 positions each, four 16-byte loads), all
  // of its loads in flight together; a count, one ordered prefix, then the
  // write of the same registers.
  uint32_t m = 0;
  if (fit) {
    constexpr int R = kFusedGroups / T;  // rounds of T groups
    const int rounds = (int)((m_g + T - 1) / T);  // uniform
    float4 x[R][4];
    int p0[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rounds) {
        const uint32_t c = (uint32_t)(r * T) + threadIdx.x;
        p0[r] = c < m_g ? (int)cg[c] * 16 : n;
#pragma unroll
        for (int v = 0; v < 4; ++v)  // a quarter that starts below ld ends below it (ld % 4 == 0)
          x[r][v] = *(const float4*)(src + min(p0[r] + 4 * v, (int)ld - 4));
      }
    }
    // hit[r]: bit 4 v + q set when position p0 + 4 v + q is a candidate
    // (below n) whose key reaches the bound.  For a bound above the key of
    // +0 (scores above 0: the usual case) that is one signed compare of the
    // raw bits, bits >= bound - 2^31, exact for every bit pattern: negative
    // values, -0 and negative NaNs fall below, positive NaNs (keys above
    // every finite one) reach it.  Otherwise the keys are formed.
    const bool pos_bound = bound > 0x80000000u;  // uniform
    const int bits_min = (int)(bound - 0x80000000u);
    uint32_t hit[R], cnt[R], eoff[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      hit[r] = 0;
      if (r < rounds) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float xv[4] = {x[r][v].x, x[r][v].y, x[r][v].z, x[r][v].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool h = pos_bound ? __float_as_int(xv[q]) >= bits_min : float_key(xv[q]) >= bound;
            hit[r] |= h ? 1u << (4 * v + q) : 0u;
          }
        }
        const int valid = n - p0[r];  // candidates in the group (the last one may be short)
        if (valid < 16) hit[r] &= valid > 0 ? (1u << valid) - 1u : 0u;
      }
      cnt[r] = (uint32_t)__popc(hit[r]);
    }
#pragma unroll
    for (int i = 0; i < RG; ++i) asm volatile("" ::"v"(pfv[i]));  // the early loads (done by now)
    m = slot_major_offsets(cnt, rounds, eoff, sc);
    if (m <= (uint32_t)kFusedList) {
      // the hits of each group, lowest position first; a hit's score is
      // picked out of the group's 16 registers by the bits of its index
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r < rounds) {
          const float f[16] = {x[r][0].x, x[r][0].y, x[r][0].z, x[r][0].w,
                               x[r][1].x, x[r][1].y, x[r][1].z, x[r][1].w,
                               x[r][2].x, x[r][2].y, x[r][2].z, x[r][2].w,
                               x[r][3].x, x[r][3].y, x[r][3].z, x[r][3].w};
          uint32_t at = eoff[r], h = hit[r];
          while (h) {
            const int q = __builtin_ctz(h);
            h &= h - 1u;
            // (selects of values, not of array elements: a conditional of two
            // lvalues would select an address and keep f in scratch memory)
            float g[8], k4[4], k2[2];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float lo = f[i], hi = f[8 + i];
              g[i] = (q & 8) ? hi : lo;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float lo = g[i], hi = g[4 + i];
              k4[i] = (q & 4) ? hi : lo;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const float lo = k4[i], hi = k4[2 + i];
              k2[i] = (q & 2) ? hi : lo;
            }
            const float lo = k2[0], hi = k2[1];
            ent[at++] = make_uint2(float_key((q & 1) ? hi : lo), (uint32_t)(p0[r] + q));
          }
        }
      }
    }
  }
  if (!fit || m > (uint32_t)kFusedList) {
    const uint32_t tau = select_row_global(blk, src, (uint32_t)n, (uint32_t)K, out);
    if (threadIdx.x == 0) gm.tau[row] = tau;
    return;
  }
  __syncthreads();

  // ---- 3. exact search (radix passes) and ordered compaction over the list
  constexpr int RL = kFusedList / T;
  const int rl = (int)((m + T - 1) / T);  // uniform
  uint32_t kl[RL];
#pragma unroll
  for (int i = 0; i < RL; ++i) {
    const uint32_t e = (uint32_t)(i * T) + threadIdx.x;
    kl[i] = i < rl && e < m ? ent[e].x : 0u;
  }
  const Threshold th =
      radix_select_tau(blk, kl, [&](int i) { return i < rl; }, (uint32_t)K, 0u, cg, sc);
  ordered_compact(blk, m, th, [&](uint32_t e) { return ent[e]; }, out);
  if (threadIdx.x == 0) gm.tau[row] = th.tau;
}

// Workspace of dsa_index_topk_decode: the group maxima and the per-row keys.
struct FusedWs {
  float* m1;
  float* m2;
  uint32_t* tau;
  int64_t ldg;
};

size_t fused_ws_bytes(int n_q, int64_t ld, FusedWs* ws, void* base) {
  const int64_t ldg = (ld + 15) / 16;
  const size_t gm = align_up((size_t)n_q * ldg * 4, 256);
  const size_t t = align_up((size_t)n_q * 4, 256);
  if (ws) {
    char* p = (char*)base;
    ws->m1 = (float*)p;
    ws->m2 = (float*)(p + gm);
    ws->tau = (uint32_t*)(p + 2 * gm);
    ws->ldg = ldg;
  }
  return 2 * gm + t;
}

}  // namespace

uint32_t take_bounds_error_topk(hipStream_t stream) { return take_bounds_error(stream); }

}  // namespace dsa

extern "C" size_t dsa_topk_workspace_size(int32_t n_q, int64_t ld, int32_t K) {
  if (n_q < 1 || ld < 1 || K < 1) return 0;
  if (ld <= dsa::kShortMax) return 0;
  return dsa::long_ws_bytes(n_q, ld, nullptr, nullptr);
}

extern "C" dsa_status_t dsa_topk(const float* scores, int64_t ld, int32_t n_q, int32_t K,
                                 const int32_t* n_valid, int32_t causal_base, int32_t* idx,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace dsa;
  if (!scores || !idx) return DSA_ERR_NULL;
  if (n_q < 1 || ld < 1 || K < 1 || K > 2048) return DSA_ERR_SHAPE;
  if (ld > (int64_t)kMaxChunks * kChunk) return DSA_ERR_SHAPE;
  if (!n_valid && (causal_base < 0 || (int64_t)causal_base + n_q > ld)) return DSA_ERR_SHAPE;
  const size_t need = dsa_topk_workspace_size(n_q, ld, K);
  if (need > 0 && (!workspace || workspace_bytes < need)) return DSA_ERR_WORKSPACE;
  dsa_status_t st = check_device();
  if (st != DSA_OK) return st;
  if (ld <= kShortMax) {
    if (ld <= 4096)
      hipLaunchKernelGGL(topk_short_kernel<4096>, dim3(n_q), dim3(kShortThreads), 0, stream,
                         scores, ld, n_valid, causal_base, K, idx);
    else if (ld <= 8192)
      hipLaunchKernelGGL(topk_short_kernel<8192>, dim3(n_q), dim3(kShortThreads), 0, stream,
                         scores, ld, n_valid, causal_base, K, idx);
    else
      hipLaunchKernelGGL(topk_short_kernel<16384>, dim3(n_q), dim3(kShortThreads), 0, stream,
                         scores, ld, n_valid, causal_base, K, idx);
    return launch_status();
  }
  LongWs ws;
  long_ws_bytes(n_q, ld, &ws, workspace);
  // 16-byte score loads need 16-byte aligned rows
  const bool vec_ok = ld % 4 == 0 && ((uintptr_t)scores & 15u) == 0;
  hipLaunchKernelGGL(topk_sample_kernel, dim3(n_q), dim3(kSampleThreads), 0, stream, scores, ld,
                     n_valid, causal_base, K, ws);
  const dim3 grid((unsigned)ws.n_chunks, (unsigned)n_q);
  if (vec_ok)
    hipLaunchKernelGGL(topk_chunk_kernel<true>, grid, dim3(kChunkThreads), 0, stream, scores, ld,
                       n_valid, causal_base, K, ws);
  else
    hipLaunchKernelGGL(topk_chunk_kernel<false>, grid, dim3(kChunkThreads), 0, stream, scores,
                       ld, n_valid, causal_base, K, ws);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n_q), dim3(kRowThreads), 0, stream, scores, ld,
                     n_valid, causal_base, K, ws, idx);
  return launch_status();
}

namespace dsa {
namespace {
// Rows of more than this many positions are selected by the three-launch
// path (sample, chunks, merge), whose chunk step spreads a row over many
// workgroups; one workgroup per row is faster below it.
constexpr int64_t kFusedMaxLd = 262144;
}  // namespace
}  // namespace dsa

namespace dsa {
namespace {
// counts[i] = q_pos[i] + 1 (the long-row path's candidate counts)
__global__ void counts_from_positions_kernel(const int32_t* __restrict__ q_pos,
                                             int32_t* __restrict__ counts, int n_q) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n_q) counts[i] = q_pos[i] + 1;
}
size_t long_path_ws_bytes(int n_q, int64_t ld) {
  return long_ws_bytes(n_q, ld, nullptr, nullptr) + align_up((size_t)n_q * 4, 256);
}
}  // namespace
}  // namespace dsa

extern "C" size_t dsa_index_topk_decode_ws(int32_t n_q, int64_t ld, int32_t K) {
  if (n_q < 1 || ld < 1 || K < 1) return 0;
  if (ld > dsa::kFusedMaxLd) return dsa::long_path_ws_bytes(n_q, ld);
  return dsa::fused_ws_bytes(n_q, ld, nullptr, nullptr);
}

extern "C" dsa_status_t dsa_index_topk_decode(const dsa_paged_cache_t* cache, const uint16_t* q_idx,
                                              const float* w, const int32_t* q_seq,
                                              const int32_t* q_pos, int32_t n_q, int32_t H_idx,
                                              int32_t K, float* scores, int64_t ld, int32_t* idx,
                                              int32_t flags, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  using namespace dsa;
  dsa_status_t st = check_cache_common(cache);
  if (st != DSA_OK) return st;
  if (!cache->k_idx || !q_idx || !w || !scores || !idx) return DSA_ERR_NULL;
  if ((q_seq == nullptr) != (q_pos == nullptr)) return DSA_ERR_NULL;
  if (!q_seq && !cache->seq_lens) return DSA_ERR_NULL;
  if (n_q < 1 || ld < 1 || K < 1 || K > 2048) return DSA_ERR_SHAPE;
  if (!q_seq && n_q != cache->n_seq) return DSA_ERR_SHAPE;
  if (ld % 4 != 0 || ld > (int64_t)1 << 24 || cache->k_idx_row_stride < cache->d_idx)
    return DSA_ERR_SHAPE;
  if ((flags & ~(DSA_TOPK_SEED_PREVIOUS | DSA_INDEX_TOPK_SCORE_ONLY |
                 DSA_INDEX_TOPK_SELECT_ONLY)) != 0 ||
      (flags & DSA_INDEX_TOPK_SCORE_ONLY && flags & DSA_INDEX_TOPK_SELECT_ONLY))
    return DSA_ERR_SHAPE;
  const bool big = H_idx == 64 && cache->d_idx == 128;
  const bool small = H_idx == 4 && cache->d_idx == 32;
  if (!big && !small) return DSA_ERR_UNSUPPORTED;
  if (cache->k_idx_row_stride % 8 != 0 || cache->block_size % 16 != 0) return DSA_ERR_UNSUPPORTED;
  if (!aligned16(cache->k_idx) || !aligned16(q_idx) || !aligned16(scores))
    return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_index_topk_decode_ws(n_q, ld, K);
  if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DSA_ERR_UNSUPPORTED;
  st = check_device();
  if (st != DSA_OK) return st;
  if (ld > kFusedMaxLd) {
    // long rows: the plain index score, then the three-launch Top-K (the
    // per-row hint is not used on this path)
    const size_t topk_bytes = long_ws_bytes(n_q, ld, nullptr, nullptr);
    int32_t* counts = (int32_t*)((char*)workspace + topk_bytes);
    if (!(flags & DSA_INDEX_TOPK_SELECT_ONLY)) {
      st = dsa_index_score(cache, DSA_DECODE, q_idx, w, q_seq, q_pos, n_q, H_idx, scores, ld,
                           nullptr, 0, stream);
      if (st != DSA_OK || (flags & DSA_INDEX_TOPK_SCORE_ONLY)) return st;
    }
    if (q_pos) {
      hipLaunchKernelGGL(counts_from_positions_kernel, dim3((n_q + 255) / 256), dim3(256), 0,
                         stream, q_pos, counts, n_q);
      st = launch_status();
      if (st != DSA_OK) return st;
    }
    return dsa_topk(scores, ld, n_q, K, q_pos ? counts : cache->seq_lens, 0, idx, workspace,
                    topk_bytes, stream);
  }
  FusedWs ws;
  fused_ws_bytes(n_q, ld, &ws, workspace);
  if (!(flags & DSA_INDEX_TOPK_SELECT_ONLY)) {
    st = launch_index_score_decode_gmax(cache, q_idx, w, q_seq, q_pos, n_q, H_idx, scores, ld,
                                        ws.m1, ws.m2, ws.ldg, stream);
    if (st != DSA_OK || (flags & DSA_INDEX_TOPK_SCORE_ONLY)) return st;
  }
  // the rows' counts: q_pos + 1, else the sequence lengths (query i is then
  // the last token of sequence i); the index kernel scored 0 .. count - 1
  const int32_t* counts = q_pos ? q_pos : cache->seq_lens;
  const int count_add = q_pos ? 1 : 0;
  const GroupMaxIn gm{ws.m1, ws.m2, ws.ldg, ws.tau, (flags & DSA_TOPK_SEED_PREVIOUS) ? 1 : 0};
  const int64_t per_thread = (ws.ldg + kFusedThreads - 1) / kFusedThreads;
#define DSA_FUSED(RGV)                                                                         \
  hipLaunchKernelGGL(topk_fused_kernel<RGV>, dim3(n_q), dim3(kFusedThreads), 0, stream, scores, \
                     ld, counts, count_add, K, gm, idx)
  // group-maximum slots per thread: every row fits (ld <= 262144: at most
  // 16 * 1024 groups)
  if (per_thread <= 2) DSA_FUSED(2);
  else if (per_thread <= 4) DSA_FUSED(4);
  else if (per_thread <= 8) DSA_FUSED(8);
  else DSA_FUSED(16);
#undef DSA_FUSED
  return launch_status();
}
