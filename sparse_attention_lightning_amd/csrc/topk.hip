// Token selector ("LLM architecture survey", section 2.2: each query keeps the k = 2048
// highest-scoring tokens). Exact top-k on the order-preserving uint32 image of the fp32
// scores; equal scores go to the lower position; output ascending, -1 padded.
//
// Two implementations with identical results. For small calls (decode, long-context share
// groups) the chunked radix form (topk_radix.hip) keeps the chip busy; for large ones (prefill,
// multi-token verification) the sampled form below reads the scores about once instead of five
// times. Three launches:
//   sample   one workgroup per row reads a block-strided sample (whole 64-byte lines, one
//            16-score block in `stride`, stride <= k / 64 so that about 128 sampled scores are
//            expected above the threshold) and radix-selects in LDS the key tau that about 2k
//            of the row's scores are expected to reach.
//   gather   chunk workgroups over the whole row append (key, position) of every score >= tau
//            to the row's candidate list (wave-aggregated atomics; order is irrelevant).
//   finish   one workgroup per row. If the list holds between k and kTkCap candidates it
//            contains the exact top-k (all scores >= tau, and tau is at most the k-th
//            largest); the workgroup radix-selects the k-th largest key T among them, breaks
//            ties at T toward lower positions with a second radix select on the complemented
//            position, and emits the k kept positions in order through LDS bitmaps of windows
//            of positions. Otherwise (a sample that missed,
//            or a flood of equal scores) it falls back to an exact scan of the whole row:
//            three histogram passes for T, then an ordered block-scan compaction.
// Rows with p + 1 <= k keep every visible token. Results are deterministic: the kept set is
// defined by score and position alone, never by the order of the appends.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

namespace radix {
size_t workspace_bytes(int rows, int L_max);
hipError_t launch(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s);
}  // namespace radix

namespace sampled {

constexpr int kTkThreads = 256;
constexpr int kTkCap = 8192;               // candidates kept per row (4 x the largest k)
#ifndef DSA_TK_SAMPLE_BLOCKS
#define DSA_TK_SAMPLE_BLOCKS 1024
#endif
constexpr int kTkSampleBlocks = DSA_TK_SAMPLE_BLOCKS;   // sampled 16-score blocks per row
constexpr int kTkChunk = 4096;             // scores per gather workgroup (16 per thread)
constexpr int kTkWindow = 1 << 18;         // positions per bitmap window in the finish step (32 KB)
static_assert(kTkCap >= 2 * kMaxK, "room for about 2k candidates plus spread");

struct TkRow {
  uint32_t count;   // candidates appended (may exceed kTkCap: the excess was not stored)
  uint32_t tau;     // candidate threshold key
  uint32_t pad[62];
};
static_assert(sizeof(TkRow) == 256, "row state is 256 bytes");

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static size_t workspace_bytes(int rows) {
  return align256(sizeof(TkRow) * (size_t)rows) + align256((size_t)rows * kTkCap * sizeof(uint2));
}

struct TkWs {
  TkRow* rows;
  uint2* cand;      // [rows][kTkCap] (key, position)
};

static TkWs carve(void* ws, int rows) {
  TkWs t;
  t.rows = (TkRow*)ws;
  t.cand = (uint2*)((char*)ws + align256(sizeof(TkRow) * (size_t)rows));
  return t;
}

struct TkRowInfo {
  int n, m;
};

__device__ __forceinline__ TkRowInfo tk_row(const int32_t* seq_lens, const int32_t* q_pos, int Q, int in_Q, int L_max,
                                            int k, int row) {
  const int b = row / Q, j = row - b * Q;
  const int p = query_pos(seq_lens, q_pos, in_Q, b, j);
  TkRowInfo ri;
  ri.n = max(0, min(p + 1, L_max));
  ri.m = min(k, ri.n);
  return ri;
}

// Block-wide exclusive scan of one uint32 per thread (256 threads); returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* excl, uint32_t* lds4) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds4[wave] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = lds4[i];
    before += (i < wave) ? t : 0u;
    total += t;
  }
  __syncthreads();
  *excl = before + x - v;
  return total;
}

// Radix-select scratch shared by the helpers below (LDS).
struct TkLds {
  uint32_t hist[4096];
  uint32_t lds4[4];
  uint32_t res[2];
};

// The bin of hist[0..NB) holding the need-th largest element and how many are still needed
// from it. Every thread of the block must call it.
template <int NB>
__device__ __forceinline__ void find_bin(TkLds& L, int need, uint32_t& bin, int& rem) {
  constexpr int PER = NB / kTkThreads;
  if (threadIdx.x == 0) { L.res[0] = 0; L.res[1] = 0; }
  const int top = NB - PER * (int)threadIdx.x;
  uint32_t h[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    h[e] = L.hist[top - 1 - e];
    mine += h[e];
  }
  uint32_t above;
  block_exclusive_scan(mine, &above, L.lds4);
  uint32_t cum = above;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (cum < (uint32_t)need && (uint32_t)need <= cum + h[e]) {
      L.res[0] = (uint32_t)(top - 1 - e);
      L.res[1] = (uint32_t)(need - (int)cum);
    }
    cum += h[e];
  }
  __syncthreads();
  bin = L.res[0];
  rem = (int)L.res[1];
  __syncthreads();
}

__device__ __forceinline__ void zero_hist(TkLds& L, int nb) {
  for (int i = threadIdx.x; i < nb; i += kTkThreads) L.hist[i] = 0u;
  __syncthreads();
}

// Block-wide min and max of one uint32 per thread.
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, TkLds& L, uint32_t& out_lo, uint32_t& out_hi) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, d, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, d, 64));
  }
  const int wave = threadIdx.x >> 6;
  __shared__ uint32_t mm[8];
  if ((threadIdx.x & 63) == 0) { mm[wave] = lo; mm[4 + wave] = hi; }
  __syncthreads();
  out_lo = min(min(mm[0], mm[1]), min(mm[2], mm[3]));
  out_hi = max(max(mm[4], mm[5]), max(mm[6], mm[7]));
  __syncthreads();
}

// The need-th largest 32-bit key among key(i), i < n, and how many keys equal to it must be
// taken. The radix digits are taken from key - min over only the significant bits of the
// observed range (up to 11 bits per level), so even tightly clustered keys spread over the
// histogram instead of piling onto one or two LDS counters; equal keys need no level at all.
template <typename KeyFn>
__device__ void select_key(TkLds& L, int n, int need, KeyFn key, uint32_t& T, int& rem) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += kTkThreads) {
    const uint32_t u = key(i);
    lo = min(lo, u);
    hi = max(hi, u);
  }
  block_minmax(lo, hi, L, lo, hi);
  const uint32_t span = hi - lo;
  int bits = span ? 32 - __clz((int)span) : 0;
  uint32_t prefix = 0;                    // offset bits resolved so far (those above `bits`)
  int nd = need;
  while (bits > 0) {                      // block-uniform
    const int w = min(11, bits), shift = bits - w;
    zero_hist(L, 2048);
    for (int i = threadIdx.x; i < n; i += kTkThreads) {
      const uint32_t off = key(i) - lo;
      if ((uint32_t)((uint64_t)off >> bits) == prefix) atomicAdd(&L.hist[(off >> shift) & ((1u << w) - 1)], 1u);
    }
    __syncthreads();
    uint32_t b;
    int r;
    find_bin<2048>(L, nd, b, r);
    prefix = (prefix << w) | b;
    nd = r;
    bits = shift;
  }
  T = lo + prefix;
  rem = nd;
}

// The need-th largest 24-bit value v(i) among the i with use(i): two 12-bit levels.
template <typename ValFn, typename UseFn>
__device__ uint32_t select_24(TkLds& L, int n, int need, ValFn v, UseFn use) {
  uint32_t b1, b2;
  int r1, r2;
  zero_hist(L, 4096);
  for (int i = threadIdx.x; i < n; i += kTkThreads)
    if (use(i)) atomicAdd(&L.hist[v(i) >> 12], 1u);
  __syncthreads();
  find_bin<4096>(L, need, b1, r1);
  zero_hist(L, 4096);
  for (int i = threadIdx.x; i < n; i += kTkThreads)
    if (use(i) && (v(i) >> 12) == b1) atomicAdd(&L.hist[v(i) & 0xFFF], 1u);
  __syncthreads();
  find_bin<4096>(L, r1, b2, r2);
  return (b1 << 12) | b2;
}

// ------------------------------------------------------------------------------------------ sample
template <bool VEC>
__global__ __launch_bounds__(kTkThreads) void topk_sample_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, TkWs ws) {
  __shared__ uint32_t skey[kTkSampleBlocks * 16];
  __shared__ TkLds L;
  const int row = blockIdx.x;
  const TkRowInfo ri = tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  TkRow* st = ws.rows + row;
  if (ri.m == ri.n) {
    if (threadIdx.x == 0) { st->count = 0; st->tau = 0; }
    return;
  }
  if (ri.n <= kTkCap) {                                // the whole row fits the candidate list
    if (threadIdx.x == 0) { st->tau = 0u; st->count = 0; }
    return;
  }
  const float* srow = scores + (int64_t)row * L_max;
  const int n_blocks = (ri.n + 15) / 16;
  const int stride = max(max(1, k / 64), (n_blocks + kTkSampleBlocks - 1) / kTkSampleBlocks);
  const int s_blocks = (n_blocks + stride - 1) / stride;
  constexpr int kPer = kTkSampleBlocks * 4 / kTkThreads;                   // float4 slots per thread
  float f[kPer][4];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {                                         // all loads in flight at once
    const int v = (int)threadIdx.x + e * kTkThreads;
    const int i0 = (v >> 2) * stride * 16 + 4 * (v & 3);
    if (VEC && v < s_blocks * 4 && i0 + 3 < ri.n) {
      const float4 x = *(const float4*)(srow + i0);
      f[e][0] = x.x; f[e][1] = x.y; f[e][2] = x.z; f[e][3] = x.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) f[e][c] = (v < s_blocks * 4 && i0 + c < ri.n) ? srow[i0 + c] : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = (int)threadIdx.x + e * kTkThreads;
    const int i0 = (v >> 2) * stride * 16 + 4 * (v & 3);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (v < s_blocks * 4) skey[4 * v + c] = (i0 + c < ri.n) ? float_key(f[e][c]) : 0u;   // 0: below every score
  }
  __syncthreads();
  const int s = s_blocks * 16;
  const int r = max(1, min((2 * k + stride - 1) / stride, s));   // ~2k scores of the row should reach tau
  uint32_t T;
  int rem;
  select_key(L, s, r, [&](int i) { return skey[i]; }, T, rem);
  if (threadIdx.x == 0) { st->tau = T; st->count = 0; }
}

// ------------------------------------------------------------------------------------------ gather
template <bool VEC>
__global__ __launch_bounds__(kTkThreads) void topk_gather_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TkWs ws) {
  const int row = blockIdx.x / n_chunks, chunk = blockIdx.x - row * n_chunks;
  const TkRowInfo ri = tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  if (ri.m == ri.n) return;
  const int lo = chunk * kTkChunk, hi = min(lo + kTkChunk, ri.n);
  if (lo >= hi) return;
  TkRow* st = ws.rows + row;
  const uint32_t tau = st->tau;
  const float* srow = scores + (int64_t)row * L_max;
  const int lane = threadIdx.x & 63;
  uint32_t u[16];
  int pos[16];
  int mine = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int i0 = lo + 4 * (int)threadIdx.x + 1024 * v;
    float f[4];
    if (VEC && i0 + 3 < hi) {
      const float4 x = *(const float4*)(srow + i0);
      f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = (i0 + e < hi) ? srow[i0 + e] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = float_key(f[e]);
      if (i0 + e < hi && key >= tau) {
        u[mine] = key;
        pos[mine] = i0 + e;
        ++mine;
      }
    }
  }
  // one atomic per wave reserves room for the wave's candidates
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  if (total == 0) return;
  uint32_t base = 0;
  if (lane == 63) base = atomicAdd(&st->count, (uint32_t)total);
  base = __shfl(base, 63, 64) + (uint32_t)(incl - mine);
  uint2* cand = ws.cand + (int64_t)row * kTkCap;
  for (int c = 0; c < mine; ++c)
    if (base + c < (uint32_t)kTkCap) cand[base + c] = make_uint2(u[c], (uint32_t)pos[c]);
}

// ------------------------------------------------------------------------------------------ finish
// Exact top-k of a whole row by one workgroup (the fallback): three histogram passes over the
// row for T and the tie quota, then an ordered block-scan compaction in position order.
__device__ void finish_full_scan(const float* __restrict__ srow, int n, int k, int32_t* __restrict__ out, TkLds& L) {
  auto key_at = [&](int i) { return float_key(srow[i]); };
  uint32_t T;
  int rem;
  select_key(L, n, k, key_at, T, rem);
  int gt_carry = 0, eq_carry = 0;
  for (int base = 0; base < n; base += kTkThreads * 4) {
    const int i0 = base + 4 * (int)threadIdx.x;
    uint32_t fgt = 0, feq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e < n) {
        const uint32_t u = key_at(i0 + e);
        fgt |= (uint32_t)(u > T) << e;
        feq |= (uint32_t)(u == T) << e;
      }
    }
    const uint32_t packed = (uint32_t)__builtin_popcount(fgt) | ((uint32_t)__builtin_popcount(feq) << 16);
    uint32_t before;
    const uint32_t tot = block_exclusive_scan(packed, &before, L.lds4);
    int g_b = gt_carry + (int)(before & 0xFFFF);
    int q_b = eq_carry + (int)(before >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool g = (fgt >> e) & 1, q = (feq >> e) & 1;
      const int slot = g_b + min(q_b, rem);
      if ((g || (q && q_b < rem)) && slot < k) out[slot] = i0 + e;
      g_b += g;
      q_b += q;
    }
    gt_carry += (int)(tot & 0xFFFF);
    eq_carry += (int)(tot >> 16);
  }
}

__global__ __launch_bounds__(kTkThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, TkWs ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t ckey[kTkCap];
  __shared__ int cpos[kTkCap];
  __shared__ uint32_t bitmap[kTkWindow / 32];
  __shared__ TkLds L;
  const int row = blockIdx.x;
  const TkRowInfo ri = tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  int32_t* out = idx + (int64_t)row * k;
  for (int i = ri.m + (int)threadIdx.x; i < k; i += kTkThreads) out[i] = -1;
  if (ri.m == ri.n) {                                  // keep every visible token
    for (int i = threadIdx.x; i < ri.n; i += kTkThreads) out[i] = i;
    return;
  }
  const TkRow* st = ws.rows + row;
  const int cnt = (int)st->count;
  if (cnt < k || cnt > kTkCap) {                       // the sample missed: exact scan of the row
    finish_full_scan(scores + (int64_t)row * L_max, ri.n, k, out, L);
    return;
  }
  const uint2* cand = ws.cand + (int64_t)row * kTkCap;
  constexpr int kCPer = kTkCap / kTkThreads;
  uint2 c[kCPer];
#pragma unroll
  for (int e = 0; e < kCPer; ++e) {                                        // all loads in flight at once
    const int i = (int)threadIdx.x + e * kTkThreads;
    if (i < cnt) c[e] = cand[i];
  }
#pragma unroll
  for (int e = 0; e < kCPer; ++e) {
    const int i = (int)threadIdx.x + e * kTkThreads;
    if (i < cnt) { ckey[i] = c[e].x; cpos[i] = (int)c[e].y; }
  }
  __syncthreads();
  uint32_t T;
  int rem;
  select_key(L, cnt, k, [&](int i) { return ckey[i]; }, T, rem);
  // ties at T: all of them, or the rem lowest positions (largest complemented positions)
  uint32_t eq_local = 0;
  for (int i = threadIdx.x; i < cnt; i += kTkThreads) eq_local += ckey[i] == T;
  uint32_t dummy;
  const int n_eq = (int)block_exclusive_scan(eq_local, &dummy, L.lds4);
  uint32_t pos_cut = 0;                                // keep ties with (0xFFFFFF - pos) >= pos_cut
  if (n_eq > rem)
    pos_cut = select_24(L, cnt, rem, [&](int i) { return 0xFFFFFFu - (uint32_t)cpos[i]; },
                        [&](int i) { return ckey[i] == T; });
  // Emit the kept positions in ascending order through a bitmap of a window of positions at a
  // time: kept candidates set their bits, a block scan of popcounts places them.
  auto keep = [&](int i) {
    return ckey[i] > T || (ckey[i] == T && (0xFFFFFFu - (uint32_t)cpos[i]) >= pos_cut);
  };
  int emitted = 0;
  for (int base = 0; base < ri.n; base += kTkWindow) {
    for (int i = threadIdx.x; i < kTkWindow / 32; i += kTkThreads) bitmap[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < cnt; i += kTkThreads) {
      const int q = cpos[i] - base;
      if (q >= 0 && q < kTkWindow && keep(i)) atomicOr(&bitmap[q >> 5], 1u << (q & 31));
    }
    __syncthreads();
    constexpr int W = kTkWindow / 32 / kTkThreads;                 // words per thread
    uint32_t pc = 0;
#pragma unroll
    for (int e = 0; e < W; ++e) pc += __builtin_popcount(bitmap[threadIdx.x * W + e]);
    uint32_t at;
    const uint32_t tot = block_exclusive_scan(pc, &at, L.lds4);
    int slot = emitted + (int)at;
#pragma unroll
    for (int e = 0; e < W; ++e) {
      uint32_t m = bitmap[threadIdx.x * W + e];
      while (m) {
        const int bit = __builtin_ctz(m);
        m &= m - 1;
        if (slot < k) out[slot] = base + 32 * (threadIdx.x * W + e) + bit;
        ++slot;
      }
    }
    emitted += (int)tot;
    __syncthreads();
  }
}

template <bool VEC>
static void launch_all(const HostBatch& bt, const float* scores, int k, int32_t* idx, TkWs w, int rows,
                       hipStream_t s) {
  const int n_chunks = (bt.L_max + kTkChunk - 1) / kTkChunk;
  const dim3 block(kTkThreads);
  hipLaunchKernelGGL(topk_sample_kernel<VEC>, dim3(rows), block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, w);
  hipLaunchKernelGGL(topk_gather_kernel<VEC>, dim3((unsigned)rows * n_chunks), block, 0, s, scores, bt.seq_lens,
                     bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, w, idx);
}

hipError_t launch(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s) {
  const int rows = bt.B * bt.Q;
  TkWs w = carve(ws, rows);
  // 16-byte vector loads need every row to start 16-byte aligned
  if (bt.L_max % 4 == 0 && ((uintptr_t)scores & 15) == 0)
    launch_all<true>(bt, scores, k, idx, w, rows, s);
  else
    launch_all<false>(bt, scores, k, idx, w, rows, s);
  return hipGetLastError();
}

}  // namespace sampled

#ifndef DSA_TOPK_SAMPLED_MIN_SCORES
#define DSA_TOPK_SAMPLED_MIN_SCORES (1 << 23)
#endif

// The sampled form once a call holds more than 8M scores (rows x L_max); below that the chunked
// radix form's extra passes over the scores cost less than one workgroup per row in series.
static bool use_sampled(const HostBatch& bt) {
  return (int64_t)bt.B * bt.Q * bt.L_max > (int64_t)DSA_TOPK_SAMPLED_MIN_SCORES;
}

// Room for either form, so that any call with at most `rows` rows fits.
size_t topk_workspace_bytes(int rows, int L_max) {
  return std::max(radix::workspace_bytes(rows, L_max), sampled::workspace_bytes(rows));
}

hipError_t launch_topk(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s) {
  if (use_sampled(bt)) return sampled::launch(bt, scores, k, idx, ws, s);
  return radix::launch(bt, scores, k, idx, ws, s);
}

}  // namespace dsa
