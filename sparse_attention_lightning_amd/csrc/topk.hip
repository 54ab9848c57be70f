// Token selector ("LLM architecture survey", section 2.2: each query keeps the k = 2048
// highest-scoring tokens). Exact top-k on the order-preserving uint32 image of the fp32
// scores; equal scores go to the lower position; output ascending, -1 padded.
//
// Three implementations with identical results, chosen by shape (see auto_form): the row form
// (one workgroup per row, one launch; further below) for short rows or many rows, the sampled
// form below for few rows of up to 256K and for large calls of longer rows, and the chunked
// radix form (topk_radix.hip) for small calls of long rows. The sampled form takes three
// launches:
//   sample   one 1024-thread workgroup per row reads a block-strided sample (whole 64-byte
//            lines, up to 512 blocks of 16 scores, 1024 on rows above 128K) and radix-selects a
//            lower bound tau of the sample rank that about 2k (2.5k above 128K) of the row's
//            scores are expected to reach.
//   gather   chunk workgroups over the whole row append (key, position) of every score >= tau
//            to the row's candidate list (one atomic per workgroup reserves its room; order is
//            irrelevant).
//   finish   one 1024-thread workgroup per row. If the list holds between k and kTkCap
//            candidates it contains the exact top-k (all scores >= tau, and tau is at most the
//            k-th largest); holding them in registers, the workgroup radix-selects the k-th
//            largest key T, breaks ties at T toward lower positions with a second radix select
//            on the complemented position, and emits the k kept positions in order by a bucket
//            sort in LDS. Otherwise (a sample that missed, or a flood of
//            equal scores) it falls back to an exact scan of the whole row: histogram passes
//            for T, then an ordered block-scan compaction.
// Rows with p + 1 <= k keep every visible token. Results are deterministic: the kept set is
// defined by score and position alone, never by the order of the appends.
#include <algorithm>
#include <cstddef>
#include <cstdlib>
#include <cstring>

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
constexpr int kGatherChunk = 4096;         // scores per gather workgroup (16 per thread)
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

// Block-wide exclusive scan of one uint32 per thread (NT threads); returns the total.
template <int NT = kTkThreads>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* excl, uint32_t* wsum) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    const uint32_t t = wsum[i];
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
  uint32_t lds4[16];      // one partial sum per wave (up to 16 waves)
  uint32_t mm[32];        // block min / max partials
  uint32_t res[2];
};

// The bin of hist[0..NB) holding the need-th largest element and how many are still needed
// from it. Every thread of the block must call it.
template <int NB, int NT = kTkThreads>
__device__ __forceinline__ void find_bin(TkLds& L, int need, uint32_t& bin, int& rem) {
  constexpr int PER = NB / NT;
  static_assert(PER >= 1 && NB % NT == 0, "whole bins per thread");
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
  block_exclusive_scan<NT>(mine, &above, L.lds4);
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

template <int NT = kTkThreads>
__device__ __forceinline__ void zero_hist(TkLds& L, int nb) {
  for (int i = threadIdx.x; i < nb; i += NT) L.hist[i] = 0u;
  __syncthreads();
}

// Block-wide min and max of one uint32 per thread.
template <int NT = kTkThreads>
__device__ __forceinline__ void block_minmax(uint32_t lo, uint32_t hi, TkLds& L, uint32_t& out_lo, uint32_t& out_hi) {
  constexpr int NWV = NT / 64;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, d, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, d, 64));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { L.mm[wave] = lo; L.mm[16 + wave] = hi; }
  __syncthreads();
  out_lo = 0xFFFFFFFFu;
  out_hi = 0u;
#pragma unroll
  for (int i = 0; i < NWV; ++i) {
    out_lo = min(out_lo, L.mm[i]);
    out_hi = max(out_hi, L.mm[16 + i]);
  }
  __syncthreads();
}

// f(key) for the key of every score srow[i], i < n: 8 per thread and pass, their loads issued
// together (clamped into the row, masked after).
template <int NT, typename F>
__device__ __forceinline__ void for_each_key(const float* __restrict__ srow, int n, F f) {
  for (int base = 0; base < n; base += NT * 8) {
    const int i0 = base + 4 * (int)threadIdx.x, i1 = i0 + 4 * NT;
    const float4 a = load4_clamped<false>(srow, i0, n), b = load4_clamped<false>(srow, i1, n);
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((e < 4 ? i0 : i1) + (e & 3) < n) f(float_key(v[e]));
  }
}

// The need-th largest key among those of srow[0..n) (n >= 1), and how many keys equal to it
// must be taken. The radix digits are taken from key - min over only the significant bits of
// the observed range (up to 11 bits per level), so even tightly clustered keys spread over the
// histogram instead of piling onto one or two LDS counters; equal keys need no level at all.
template <int NT = kTkThreads>
__device__ void select_key(TkLds& L, const float* __restrict__ srow, int n, int need, uint32_t& T, int& rem) {
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for_each_key<NT>(srow, n, [&](uint32_t u) {
    lo = min(lo, u);
    hi = max(hi, u);
  });
  block_minmax<NT>(lo, hi, L, lo, hi);
  const uint32_t span = hi - lo;
  int bits = span ? 32 - __clz((int)span) : 0;
  uint32_t prefix = 0;                    // offset bits resolved so far (those above `bits`)
  int nd = need;
  while (bits > 0) {                      // block-uniform
    const int w = min(11, bits), shift = bits - w;
    zero_hist<NT>(L, 2048);
    for_each_key<NT>(srow, n, [&](uint32_t u) {
      const uint32_t off = u - lo;
      if ((uint32_t)((uint64_t)off >> bits) == prefix) atomicAdd(&L.hist[(off >> shift) & ((1u << w) - 1)], 1u);
    });
    __syncthreads();
    uint32_t b;
    int r;
    find_bin<2048, NT>(L, nd, b, r);
    prefix = (prefix << w) | b;
    nd = r;
    bits = shift;
  }
  T = lo + prefix;
  rem = nd;
}

// ------------------------------------------------------------------------------------------ gather
// One workgroup per chunk of kGatherChunk scores. Its score loads go out first, all at once and
// clamped into the row, so that their latency overlaps that of the row's length and tau. A
// first pass counts the thread's candidates, one atomic per workgroup reserves their room, and
// a second pass over the same registers writes them.
template <bool VEC>
__global__ __launch_bounds__(kTkThreads) void topk_gather_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TkWs ws) {
  constexpr int NV = kGatherChunk / (4 * kTkThreads);
  const int row = blockIdx.x / n_chunks, chunk = blockIdx.x - row * n_chunks;
  const int lo = chunk * kGatherChunk;
  const float* srow = scores + (int64_t)row * L_max;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4 x[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) x[v] = load4_clamped<VEC, true>(srow, lo + 4 * tid + 4 * kTkThreads * v, L_max);
  const TkRowInfo ri = tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  if (ri.m == ri.n) return;
  const int hi = min(lo + kGatherChunk, ri.n);
  if (lo >= hi) return;
  TkRow* st = ws.rows + row;
  const uint32_t tau = st->tau;
  uint32_t mine = 0;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = lo + 4 * tid + 4 * kTkThreads * v;
    const float f[4] = {x[v].x, x[v].y, x[v].z, x[v].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) mine += (i0 + e < hi && float_key(f[e]) >= tau) ? 1u : 0u;
  }
  // wave scans, then the four wave totals through LDS (the early returns above are
  // workgroup-uniform)
  __shared__ uint32_t wtot[kTkThreads / 64];
  __shared__ uint32_t wg_base;
  const uint32_t incl = wave_incl_scan(mine, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kTkThreads / 64; ++i) t += wtot[i];
    wg_base = t ? atomicAdd(&st->count, t) : 0u;
  }
  __syncthreads();
  uint32_t slot = wg_base;
#pragma unroll
  for (int i = 0; i < kTkThreads / 64; ++i) slot += i < wave ? wtot[i] : 0u;
  slot += incl - mine;
  if (!mine) return;
  uint2* cand = ws.cand + (int64_t)row * kTkCap;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int i0 = lo + 4 * tid + 4 * kTkThreads * v;
    const float f[4] = {x[v].x, x[v].y, x[v].z, x[v].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = float_key(f[e]);
      if (i0 + e < hi && key >= tau) {
        if (slot < (uint32_t)kTkCap) cand[slot] = make_uint2(key, (uint32_t)(i0 + e));
        ++slot;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------ finish
// Exact top-k of a whole row of n > k scores by one workgroup (the fallback): histogram passes
// over the row for T and the tie quota, then an ordered block-scan compaction in position order
// that stops once all k outputs are placed (the keys above T number k - the tie quota), so a
// row of ties ends after its first block.
template <int NT = kTkThreads>
__device__ void finish_full_scan(const float* __restrict__ srow, int n, int k, int32_t* __restrict__ out, TkLds& L) {
  uint32_t T;
  int rem;
  select_key<NT>(L, srow, n, k, T, rem);
  const int n_gt = k - rem;
  int gt_carry = 0, eq_carry = 0;
  for (int base = 0; base < n; base += NT * 4) {
    const int i0 = base + 4 * (int)threadIdx.x;
    const float4 x = load4_clamped<false>(srow, i0, n);
    const float v[4] = {x.x, x.y, x.z, x.w};
    uint32_t fgt = 0, feq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e < n) {
        const uint32_t u = float_key(v[e]);
        fgt |= (uint32_t)(u > T) << e;
        feq |= (uint32_t)(u == T) << e;
      }
    }
    const uint32_t packed = (uint32_t)__builtin_popcount(fgt) | ((uint32_t)__builtin_popcount(feq) << 16);
    uint32_t before;
    const uint32_t tot = block_exclusive_scan<NT>(packed, &before, L.lds4);
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
    if (gt_carry >= n_gt && eq_carry >= rem) break;    // block-uniform
  }
}

}  // namespace sampled

// ------------------------------------------------------------------------------------------ rowsel
// The same selection (sample -> tau -> candidates >= tau -> exact select -> ordered emission)
// by one workgroup of 512 threads per row in a single launch, with the candidate list in LDS
// instead of global memory. It reads the row once plus an 8192-score sample, so it suits calls
// with enough rows to fill the chip and rows short enough for one workgroup to stream. Being one
// long chain of block-wide steps, it keeps each step short: wave scans and reductions by DPP
// row shifts and broadcasts (no LDS round trip), one barrier per block scan, candidate keys held
// in registers across the radix levels, and a double-buffered gather that compares the floats
// against tau directly (float_key is monotone, so key >= tau is f >= the float of tau).
namespace rowsel {

constexpr int kRT = 512;                   // threads per row workgroup (two workgroups per CU)
constexpr int kRCap = 4096;                // candidates kept in LDS (2 x the largest k)
constexpr int kRSample = 512;              // sampled 16-score blocks (8192 scores) ...
constexpr int kRSampleLong = 1024;         // ... and for rows above kRLongRow scores
constexpr int kRLongRow = 1 << 17;
constexpr int kRUnroll = 2;                // float4 per thread per gather pass (double-buffered)
constexpr int kRBins = 4096;               // 12-bit radix levels
constexpr int kRCPer = kRCap / kRT;        // candidate slots per thread
static_assert(kRCap >= 2 * kMaxK, "room for about 1.5k candidates plus spread");

// LDS of the block-wide selection steps of an NT-thread workgroup (shared by the row form and
// the sampled form's per-row kernels).
template <int NT>
struct SelLds {
  static_assert(kRBins % NT == 0, "whole bins per thread");
  union {
    alignas(16) uint32_t hist[2][kRBins];  // radix levels alternate between two histograms
    sampled::TkLds full;                   // the exact full-row fallback
  } h;
  uint32_t wred[4][NT / 64];               // per-wave partials, rotated over the block steps
  uint32_t res[2];
  uint32_t count;
};

struct RowLds {
  uint32_t key[kRCap];                     // candidates: key and position
  int pos[kRCap];
  SelLds<kRT> s;
};

template <int NT>
struct Blk {
  static constexpr int kW = NT / 64;       // waves
  SelLds<NT>& S;
  int tid, lane, wave;
  int slot = 0;                            // wred slot of the next block step
  int cur = 0;                             // the histogram that is clean

  // Exclusive prefix sum over the threads in order (one barrier); *total gets the block sum.
  __device__ uint32_t scan(uint32_t v, uint32_t* total) {
    uint32_t* w = S.wred[slot];
    slot = (slot + 1) & 3;
    const uint32_t x = wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
    if (lane == 63) w[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      const uint32_t t = w[i];
      before += i < wave ? t : 0u;
      tot += t;
    }
    *total = tot;
    return before + x - v;
  }
  __device__ uint32_t sum(uint32_t v) {
    uint32_t t;
    scan(v, &t);
    return t;
  }
  // Block min and max (one barrier).
  __device__ void minmax(uint32_t lo, uint32_t hi, uint32_t& olo, uint32_t& ohi) {
    uint32_t* w = S.wred[slot];
    slot = (slot + 2) & 3;
    uint32_t* w2 = S.wred[(slot + 3) & 3];
    lo = wave_incl_scan(lo, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return min(a, b); });
    hi = wave_incl_scan(hi, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
    if (lane == 63) { w[wave] = lo; w2[wave] = hi; }
    __syncthreads();
    olo = 0xFFFFFFFFu;
    ohi = 0u;
#pragma unroll
    for (int i = 0; i < kW; ++i) {
      olo = min(olo, w[i]);
      ohi = max(ohi, w2[i]);
    }
  }
  // The bin of hist[cur] holding the need-th largest counted element, and how many are still
  // needed from it (two barriers). Thread t owns bins [kRBins - 4(t+1), kRBins - 4t).
  __device__ void find_bin(int need, uint32_t& bin, int& rem) {
    constexpr int PER = kRBins / NT;
    static_assert(PER % 4 == 0, "whole 16-byte reads of bins");
    const uint32_t* hist = S.h.hist[cur];
    const int top = kRBins - PER * tid;
    // 16-byte reads: the lanes' bins are PER words apart, which as single-word reads would fall
    // on a few LDS banks; as 16-byte reads of consecutive lanes they do not conflict
    uint32_t h[PER], mine = 0;
#pragma unroll
    for (int v = 0; v < PER / 4; ++v) {
      const uint4 x = *(const uint4*)&hist[top - 4 * (v + 1)];
      h[4 * v + 0] = x.w;
      h[4 * v + 1] = x.z;
      h[4 * v + 2] = x.y;
      h[4 * v + 3] = x.x;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) mine += h[e];
    uint32_t tot;
    uint32_t cum = scan(mine, &tot);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (cum < (uint32_t)need && (uint32_t)need <= cum + h[e]) {
        S.res[0] = (uint32_t)(top - 1 - e);
        S.res[1] = (uint32_t)(need - (int)cum);
      }
      cum += h[e];
    }
    __syncthreads();
    bin = S.res[0];
    rem = (int)S.res[1];
  }
  // Radix select over the keys k[i] with ok[i] of every thread: the need-th largest key (exact,
  // and then *rem = how many keys equal to it are needed), or after at most two 12-bit levels a
  // lower bound of it (the low edge of its bin). Digits come from key - min over the significant
  // bits of the observed range.
  template <int PER>
  __device__ uint32_t select(const uint32_t (&k)[PER], const bool (&ok)[PER], int need, bool exact, int* rem) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (ok[e]) { lo = min(lo, k[e]); hi = max(hi, k[e]); }
    minmax(lo, hi, lo, hi);
    const uint32_t span = hi - lo;
    int bits = span ? 32 - __clz((int)span) : 0;
    uint32_t prefix = 0;
    int nd = need;
    for (int level = 0; bits > 0; ++level) {           // block-uniform
      if (!exact && level == 2) break;
      const int w = min(12, bits), shift = bits - w;
      uint32_t* hist = S.h.hist[cur];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const uint32_t off = k[e] - lo;
        if (ok[e] && (uint32_t)((uint64_t)off >> bits) == prefix) atomicAdd(&hist[(off >> shift) & ((1u << w) - 1)], 1u);
      }
      uint32_t* other = S.h.hist[cur ^ 1];
      for (int i = tid; i < kRBins; i += NT) other[i] = 0u;
      __syncthreads();
      uint32_t b;
      int r;
      find_bin(nd, b, r);
      cur ^= 1;
      prefix = (prefix << w) | b;
      nd = r;
      bits = shift;
    }
    if (rem) *rem = nd;
    return lo + (uint32_t)((uint64_t)prefix << bits);
  }
};

__device__ __forceinline__ float key_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// tau (a key) for a row of n > 0 scores: a lower bound of the r-th largest of a block-strided
// sample of up to NS 16-score blocks, r chosen so that about `target` of the row's scores
// are expected to reach it. The histograms must be zero on entry; returns with them ready.
template <int NT, int NS, bool VEC>
__device__ uint32_t sample_tau(Blk<NT>& B, const float* __restrict__ srow, int n, int target) {
  const int tid = B.tid;
  const int n_blocks = (n + 15) / 16;
  const int stride = (n_blocks + NS - 1) / NS;
  const int s_blocks = (n_blocks + stride - 1) / stride;
  constexpr int kPer = NS * 4 / NT;                    // float4 slots per thread
  uint32_t sk[kPer * 4];
  bool sok[kPer * 4];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int v = tid + e * NT;
    const int i0 = (v >> 2) * stride * 16 + 4 * (v & 3);
    const float4 x = load4_clamped<VEC>(srow, i0, n);
    const float f[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sok[4 * e + c] = v < s_blocks * 4 && i0 + c < n;
      sk[4 * e + c] = float_key(f[c]);
    }
  }
  int ns_local = 0;
#pragma unroll
  for (int e = 0; e < kPer * 4; ++e) ns_local += sok[e];
  const int ns = (int)B.sum((uint32_t)ns_local);       // also orders the caller's zeroing before use
  const int r = max(1, min((target + stride - 1) / stride, ns));
  return B.select(sk, sok, r, false, nullptr);
}

// Exact top-k of the candidates held in registers (PER per thread; every score of the row that
// can be among the k largest is a candidate, cnt >= k of them) written to out[0..k) in
// ascending position order: the k-th largest key T, the ties at T by the lowest positions, then
// the k kept positions in order by a bucket sort in LDS. Bucket = position >> shift, with shift
// the least that puts every position of the row below kEmitBuckets: count, prefix-sum the counts
// into bucket offsets, scatter each position into its bucket, and give each position its rank
// inside its bucket by counting the smaller ones there. A bucket spans 2^shift positions (64 at
// 128K, 512 at 1M), so the rank loops are short, and nothing walks the n positions of the row.
// The caller lends an LDS region of WORDS words free by then (its first use comes after the
// select's last barrier).
constexpr int kEmitBuckets = 2048;

template <int NT, int PER, int WORDS>
__device__ void select_emit(Blk<NT>& B, const uint32_t (&ck)[PER], const int (&cp)[PER], const bool (&cok)[PER], int n,
                            int k, int32_t* __restrict__ out, uint32_t* __restrict__ lds) {
  constexpr int BPT = kEmitBuckets / NT;               // buckets per thread in the prefix sum
  static_assert(BPT >= 1 && kEmitBuckets % NT == 0, "whole buckets per thread");
  static_assert(WORDS >= 2 * kEmitBuckets + kMaxK, "counts, offsets and the scattered positions");
  const int tid = B.tid;
  int rem;
  const uint32_t T = B.select(ck, cok, k, true, &rem);
  uint32_t eq_local = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) eq_local += cok[e] && ck[e] == T;
  const int n_eq = (int)B.sum(eq_local);
  uint32_t pos_cut = 0;                                // keep ties with (0xFFFFFF - pos) >= pos_cut
  if (n_eq > rem) {
    uint32_t tk[PER];
    bool tok[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      tok[e] = cok[e] && ck[e] == T;
      tk[e] = 0xFFFFFFu - (uint32_t)cp[e];
    }
    pos_cut = B.select(tk, tok, rem, true, nullptr);
  }
  bool keep[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e)
    keep[e] = cok[e] && (ck[e] > T || (ck[e] == T && (0xFFFFFFu - (uint32_t)cp[e]) >= pos_cut));
  uint32_t* cnt = lds;                                 // [kEmitBuckets] counts, then cursors
  uint32_t* off = lds + kEmitBuckets;                  // [kEmitBuckets] first slot of each bucket
  int* srt = (int*)(lds + 2 * kEmitBuckets);           // [k] positions, grouped by bucket
  int shift = 0;
  while (((n - 1) >> shift) >= kEmitBuckets) ++shift;  // block-uniform
#pragma unroll
  for (int b = 0; b < BPT; ++b) cnt[tid * BPT + b] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (keep[e]) atomicAdd(&cnt[cp[e] >> shift], 1u);
  __syncthreads();
  uint32_t c[BPT], mine = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    c[b] = cnt[tid * BPT + b];
    mine += c[b];
  }
  uint32_t total;
  uint32_t at = B.scan(mine, &total);                  // the scan's barrier orders the reads above
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    off[tid * BPT + b] = at;
    at += c[b];
    cnt[tid * BPT + b] = 0u;
  }
  __syncthreads();
  int slot[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    slot[e] = -1;
    if (keep[e]) {
      const int bk = cp[e] >> shift;
      slot[e] = (int)(off[bk] + atomicAdd(&cnt[bk], 1u));
      srt[slot[e]] = cp[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (slot[e] >= 0) {
      const int bk = cp[e] >> shift;
      const int b0 = (int)off[bk], b1 = b0 + (int)cnt[bk];
      int r = b0;
      for (int i = b0; i < b1; ++i) r += srt[i] < cp[e];
      if (r < k) out[r] = cp[e];
    }
  }
}

template <bool VEC, int NS>
__global__ __launch_bounds__(kRT) void topk_row_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int32_t* __restrict__ idx) {
  __shared__ RowLds R;
  SelLds<kRT>& S = R.s;
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  Blk<kRT> B{S, tid, lane, tid >> 6};
  const sampled::TkRowInfo ri = sampled::tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  int32_t* out = idx + (int64_t)row * k;
  for (int i = ri.m + tid; i < k; i += kRT) out[i] = -1;
  if (ri.m == ri.n) {                                  // keep every visible token
    for (int i = tid; i < ri.n; i += kRT) out[i] = i;
    return;
  }
  const float* srow = scores + (int64_t)row * L_max;
  const int n = ri.n;
  for (int i = tid; i < 2 * kRBins; i += kRT) (&S.h.hist[0][0])[i] = 0u;
  if (tid == 0) S.count = 0u;

  // ---- tau: about 3k/2 of the row's scores are expected to reach it (rows that fit the list
  // keep every score)
  float tau_f = -INFINITY;
  if (n > kRCap)
    tau_f = key_float(sample_tau<kRT, NS, VEC>(B, srow, n, 3 * k / 2));
  else
    __syncthreads();

  // ---- candidates: every visible score >= tau, appended to LDS (one atomic per wave and pass)
  constexpr int kStep = kRT * 4 * kRUnroll;
  float4 cur[kRUnroll], nxt[kRUnroll];
  auto load = [&](float4 (&d)[kRUnroll], int base) {
#pragma unroll
    for (int u = 0; u < kRUnroll; ++u) {
      d[u] = load4_clamped<VEC, true>(srow, base + 4 * (tid + u * kRT), n);   // past n: masked below
    }
  };
  load(cur, 0);
  for (int base = 0; base < n; base += kStep) {
    load(nxt, base + kStep);                           // the last pass's are clamped and unused
    uint64_t bal[kRUnroll][4];
    uint32_t total = 0;
#pragma unroll
    for (int u = 0; u < kRUnroll; ++u) {
      const int i0 = base + 4 * (tid + u * kRT);
      const float f[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bal[u][c] = __ballot(i0 + c < n && f[c] >= tau_f);
        total += (uint32_t)__popcll(bal[u][c]);
      }
    }
    if (total) {                                       // wave-uniform
      uint32_t at = 0;
      if (lane == 0) at = atomicAdd(&S.count, total);
      at = __builtin_amdgcn_readfirstlane(at);
#pragma unroll
      for (int u = 0; u < kRUnroll; ++u) {
        const int i0 = base + 4 * (tid + u * kRT);
        const float f[4] = {cur[u].x, cur[u].y, cur[u].z, cur[u].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint64_t b = bal[u][c];
          if ((b >> lane) & 1ull) {
            const uint32_t slot =
                at + __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            if (slot < (uint32_t)kRCap) {
              R.key[slot] = float_key(f[c]);
              R.pos[slot] = i0 + c;
            }
          }
          at += (uint32_t)__popcll(b);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRUnroll; ++u) cur[u] = nxt[u];
  }
  __syncthreads();
  const int cnt = (int)S.count;
  if (cnt < k || cnt > kRCap) {                        // the sample missed: exact scan of the row
    sampled::finish_full_scan<kRT>(srow, n, k, out, S.h.full);
    return;
  }
  uint32_t ck[kRCPer];
  int cp[kRCPer];
  bool cok[kRCPer];
#pragma unroll
  for (int e = 0; e < kRCPer; ++e) {
    const int i = tid + e * kRT;
    cok[e] = i < cnt;
    ck[e] = cok[e] ? R.key[i] : 0u;
    cp[e] = cok[e] ? R.pos[i] : 0;
  }
  // the candidate arrays (key, then pos: 2 kRCap words) are free once read into registers: the
  // emission's bucket sort takes them
  static_assert(offsetof(RowLds, pos) == offsetof(RowLds, key) + kRCap * sizeof(uint32_t), "key, then pos");
  select_emit<kRT, kRCPer, 2 * kRCap>(B, ck, cp, cok, n, k, out, R.key);
}

template <bool VEC>
static void launch_vec(const HostBatch& bt, const float* scores, int k, int32_t* idx, hipStream_t s) {
  const int rows = bt.B * bt.Q;
  // The count of scores above tau spreads as sqrt(target x sampling stride): longer rows take a
  // denser sample so that the list still holds between k and kRCap of them nearly always.
  if (bt.L_max > kRLongRow)
    hipLaunchKernelGGL((topk_row_kernel<VEC, kRSampleLong>), dim3(rows), dim3(kRT), 0, s, scores, bt.seq_lens,
                       bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, idx);
  else
    hipLaunchKernelGGL((topk_row_kernel<VEC, kRSample>), dim3(rows), dim3(kRT), 0, s, scores, bt.seq_lens,
                       bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, idx);
}

hipError_t launch(const HostBatch& bt, const float* scores, int k, int32_t* idx, hipStream_t s) {
  if (bt.L_max % 4 == 0 && ((uintptr_t)scores & 15) == 0)
    launch_vec<true>(bt, scores, k, idx, s);
  else
    launch_vec<false>(bt, scores, k, idx, s);
  return hipGetLastError();
}

}  // namespace rowsel

namespace sampled {

constexpr int kST = 1024;                  // threads of the per-row sample and finish workgroups

// sample: one 1024-thread workgroup per row; tau for about `target` candidates (rows that fit
// the candidate list keep every score: tau = 0, below every key).
template <bool VEC, int NS>
__global__ __launch_bounds__(kST) void topk_sample_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int target, TkWs ws) {
  __shared__ rowsel::SelLds<kST> S;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const TkRowInfo ri = tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  TkRow* st = ws.rows + row;
  if (ri.m == ri.n || ri.n <= kTkCap) {
    if (tid == 0) { st->count = 0; st->tau = 0u; }
    return;
  }
  rowsel::Blk<kST> B{S, tid, tid & 63, tid >> 6};
  for (int i = tid; i < 2 * rowsel::kRBins; i += kST) (&S.h.hist[0][0])[i] = 0u;
  const uint32_t tau = rowsel::sample_tau<kST, NS, VEC>(B, scores + (int64_t)row * L_max, ri.n, target);
  if (tid == 0) { st->tau = tau; st->count = 0; }
}

// finish: one 1024-thread workgroup per row over its candidate list (held in registers), or the
// exact full-row scan when the list missed (fewer than k) or overflowed.
__global__ __launch_bounds__(kST) void topk_finish_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, TkWs ws, int32_t* __restrict__ idx) {
  constexpr int PER = kTkCap / kST;
  constexpr int kEmitWords = 2 * rowsel::kEmitBuckets + kMaxK;   // the emission's bucket sort
  __shared__ rowsel::SelLds<kST> S;
  __shared__ uint32_t emit_bits[kEmitWords];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const TkRowInfo ri = tk_row(seq_lens, q_pos, Q, in_Q, L_max, k, row);
  int32_t* out = idx + (int64_t)row * k;
  for (int i = ri.m + tid; i < k; i += kST) out[i] = -1;
  if (ri.m == ri.n) {                                  // keep every visible token
    for (int i = tid; i < ri.n; i += kST) out[i] = i;
    return;
  }
  rowsel::Blk<kST> B{S, tid, tid & 63, tid >> 6};
  // every slot of the list is loaded at once, before the count is known (slots past the count
  // hold stale values and are masked)
  const uint2* cand = ws.cand + (int64_t)row * kTkCap;
  uint2 c[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) c[e] = cand[tid + e * kST];
  const int cnt = (int)ws.rows[row].count;
  if (cnt < k || cnt > kTkCap) {                       // the sample missed: exact scan of the row
    finish_full_scan<kST>(scores + (int64_t)row * L_max, ri.n, k, out, S.h.full);
    return;
  }
  for (int i = tid; i < 2 * rowsel::kRBins; i += kST) (&S.h.hist[0][0])[i] = 0u;
  uint32_t ck[PER];
  int cp[PER];
  bool cok[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    cok[e] = tid + e * kST < cnt;
    ck[e] = cok[e] ? c[e].x : 0u;
    cp[e] = cok[e] ? (int)c[e].y : 0;
  }
  __syncthreads();                                     // the zeroed histograms before the first level
  rowsel::select_emit<kST, PER, kEmitWords>(B, ck, cp, cok, ri.n, k, out, emit_bits);
}

template <bool VEC>
static void launch_all(const HostBatch& bt, const float* scores, int k, int32_t* idx, TkWs w, int rows,
                       hipStream_t s) {
  const int n_chunks = (bt.L_max + kGatherChunk - 1) / kGatherChunk;
  // The candidate count spreads as sqrt(target x sampling stride). Rows above 128K scores take
  // a denser sample and aim at 2.5k, midway between the bounds k and kTkCap (4k at the largest
  // k), so that a sample miss (and the exact full-row scan it costs) stays rare at 1M scores
  // per row.
  if (bt.L_max > rowsel::kRLongRow)
    hipLaunchKernelGGL((topk_sample_kernel<VEC, rowsel::kRSampleLong>), dim3(rows), dim3(kST), 0, s, scores,
                       bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, 5 * k / 2, w);
  else
    hipLaunchKernelGGL((topk_sample_kernel<VEC, rowsel::kRSample>), dim3(rows), dim3(kST), 0, s, scores,
                       bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, 2 * k, w);
  hipLaunchKernelGGL(topk_gather_kernel<VEC>, dim3((unsigned)rows * n_chunks), dim3(kTkThreads), 0, s, scores,
                     bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(rows), dim3(kST), 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q,
                     bt.in_Q, bt.L_max, k, w, idx);
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

enum TopkForm { kFormAuto = 0, kFormRadix, kFormSampled, kFormRow };

// DSA_TOPK_FORM = radix | sampled | row pins one form (all give identical results); unset or
// anything else leaves the choice to the size rules below.
static TopkForm forced_form() {
  const char* e = getenv("DSA_TOPK_FORM");
  if (!e) return kFormAuto;
  if (!strcmp(e, "radix")) return kFormRadix;
  if (!strcmp(e, "sampled")) return kFormSampled;
  if (!strcmp(e, "row")) return kFormRow;
  return kFormAuto;
}

// One workgroup per row streams a row at a few GB/s, so the one-launch row form wins when rows
// are short (at most 32K scores) or many (128 rows or more up to 64K scores, 256 or more up to
// 256K: two workgroups per CU then keep the chip busy). Other rows up to 256K go to the sampled
// form, whose gather spreads each row over the chip; longer rows to the sampled form once a call
// holds 8M scores (rows x L_max) or more, else to the chunked radix form.
static TopkForm auto_form(const HostBatch& bt) {
  const int64_t rows = (int64_t)bt.B * bt.Q;
  const int64_t L = bt.L_max;
  if (L <= (1 << 18)) {
    if (L <= (1 << 15) || (L <= (1 << 16) && rows >= 128) || rows >= 256) return kFormRow;
    return kFormSampled;
  }
  if (rows * L >= (int64_t)(1 << 23)) return kFormSampled;
  return kFormRadix;
}

// Room for any form, so that any call with at most `rows` rows fits (the row form needs none).
size_t topk_workspace_bytes(int rows, int L_max) {
  return std::max(radix::workspace_bytes(rows, L_max), sampled::workspace_bytes(rows));
}

hipError_t launch_topk(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s) {
  TopkForm f = forced_form();
  if (f == kFormAuto) f = auto_form(bt);
  if (f == kFormRow) return rowsel::launch(bt, scores, k, idx, s);
  if (f == kFormSampled) return sampled::launch(bt, scores, k, idx, ws, s);
  return radix::launch(bt, scores, k, idx, ws, s);
}

}  // namespace dsa
