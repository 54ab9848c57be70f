// Token selector, chunked radix form ("LLM architecture survey", section 2.2: each query keeps
// the k = 2048 highest-scoring tokens). Exact top-k by radix select on the order-preserving
// uint32 image of the fp32 scores, ties to the lower position, output ascending. Used when there
// are few rows (decode, long-context share groups): every pass spreads each row over many
// workgroups, so a handful of rows still fills the chip.
//
// A row (one query token) is cut into chunks of kTopkChunk scores, one workgroup per chunk,
// so long rows (128K, 1M) spread over the whole chip. Passes, one launch each:
//   hist0       histogram of key bits [31:21] (LDS, then global atomics into the row's bins)
//   hist1       every workgroup first finds the level-0 threshold bin b1 (a block scan of the
//               finished level-0 histogram), then bins bits [20:10] of the keys inside b1
//   hist2       finds b2 the same way, then bins bits [9:0] of the keys whose top 22 bits match
//   count       finds b3: T = (b1, b2, b3) is the k-th largest key and `rem` the number of ties
//               at T to keep; counts keys > T and keys == T in its chunk
//   compact     the chunk's output offset is the number of keys kept by earlier chunks (ties are
//               taken in position order); ordered scan-based compaction of the kept positions;
//               chunk 0 writes the -1 padding
// Workgroups never wait on each other: a pass only reads what earlier launches finished, and
// kernel boundaries make it visible. The chunk-0 workgroup of each pass stores the bin it
// found so that later passes scan only the newest histogram.
// Rows with p + 1 <= k keep every visible token and skip the histogram passes.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace radix {

constexpr int kTopkThreads = 256;
constexpr int kTopkVec = 4;                                   // floats per load
constexpr int kTopkVpt = 4;                                   // vector loads per thread
constexpr int kTopkPer = kTopkVec * kTopkVpt;                 // scores per thread
constexpr int kTopkChunk = kTopkThreads * kTopkPer;           // scores per workgroup
constexpr int kNB1 = 2048, kNB2 = 2048, kNB3 = 1024;

struct TopkRow {
  uint32_t hist1[kNB1];
  uint32_t hist2[kNB2];
  uint32_t hist3[kNB3];
  uint32_t bin[3];       // threshold bin found at each level (written by chunk 0)
  int32_t rem[3];        // keys still needed from that bin
  uint32_t pad[58];
};
static_assert(sizeof(TopkRow) % 256 == 0, "row state is 256-byte aligned");
constexpr int kZeroWords = kNB1 + kNB2 + kNB3;

struct TopkWs {
  TopkRow* rows;
  int32_t* gt;       // [rows][n_chunks] keys > T per chunk
  int32_t* eq;       // [rows][n_chunks] keys == T per chunk
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes(int rows, int L_max) {
  const size_t n_chunks = (L_max + kTopkChunk - 1) / kTopkChunk;
  return align256(sizeof(TopkRow) * (size_t)rows) + 2 * align256(sizeof(int32_t) * rows * n_chunks);
}

static TopkWs carve(void* ws, int rows, int n_chunks) {
  char* p = (char*)ws;
  TopkWs t;
  t.rows = (TopkRow*)p;
  p += align256(sizeof(TopkRow) * (size_t)rows);
  const size_t a = align256(sizeof(int32_t) * (size_t)rows * n_chunks);
  t.gt = (int32_t*)p;
  t.eq = (int32_t*)(p + a);
  return t;
}

struct RowInfo {
  int row, chunk, n, m, lo, hi;
};

__device__ __forceinline__ RowInfo row_info(const int32_t* seq_lens, const int32_t* q_pos, int Q, int in_Q,
                                            int L_max, int k, int n_chunks) {
  RowInfo ri;
  ri.row = blockIdx.x / n_chunks;
  ri.chunk = blockIdx.x - ri.row * n_chunks;
  const int b = ri.row / Q, j = ri.row - b * Q;
  const int p = query_pos(seq_lens, q_pos, in_Q, b, j);
  ri.n = max(0, min(p + 1, L_max));
  ri.m = min(k, ri.n);
  ri.lo = ri.chunk * kTopkChunk;
  ri.hi = min(ri.lo + kTopkChunk, ri.n);
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

// The bin of a finished histogram that holds the need-th largest key, and how many keys are
// still needed from it. Bins are scanned from the top; thread 0 owns the highest bins.
// Every thread of the block must call it.
template <int NB>
__device__ __forceinline__ void find_bin(const uint32_t* __restrict__ gh, int need, uint32_t* lds4,
                                         uint32_t* out_bin, int* out_rem) {
  constexpr int PER = NB / kTopkThreads;
  __shared__ uint32_t res[2];
  if (threadIdx.x == 0) { res[0] = 0; res[1] = 0; }
  const int top = NB - PER * (int)threadIdx.x;
  uint32_t h[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    h[e] = gh[top - 1 - e];
    mine += h[e];
  }
  uint32_t above;
  block_exclusive_scan(mine, &above, lds4);
  uint32_t cum = above;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (cum < (uint32_t)need && (uint32_t)need <= cum + h[e]) {
      res[0] = (uint32_t)(top - 1 - e);
      res[1] = (uint32_t)(need - (int)cum);
    }
    cum += h[e];
  }
  __syncthreads();
  *out_bin = res[0];
  *out_rem = (int)res[1];
  __syncthreads();
}

// This thread's scores of the chunk as keys: vectors of 4 at lo + 4*tid + 1024*v, v < kTopkVpt
// (each vector load of a wave covers 1 KB contiguous). Bit e of `valid`: element e in [lo, hi).
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ srow, int lo, int hi, uint32_t (&u)[kTopkPer],
                                           uint64_t& valid) {
  valid = 0;
#pragma unroll
  for (int v = 0; v < kTopkVpt; ++v) {
    const int i0 = lo + kTopkVec * (int)threadIdx.x + kTopkThreads * kTopkVec * v;
    const float4 x = load4_clamped<VEC>(srow, i0, hi);
    const float f[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u[4 * v + e] = float_key(f[e]);
      valid |= (uint64_t)(i0 + e < hi) << (4 * v + e);
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_zero_kernel(TopkRow* rows) {
  uint32_t* base = (uint32_t*)(rows + blockIdx.x);
  for (int i = threadIdx.x; i < kZeroWords; i += kTopkThreads) base[i] = 0u;
}

// Radix level LEVEL over key bits [31:21], [20:10] or [9:0].
template <int LEVEL, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TopkWs ws) {
  constexpr int NB = LEVEL == 2 ? kNB3 : kNB1;
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t lds4[4];
  const RowInfo ri = row_info(seq_lens, q_pos, Q, in_Q, L_max, k, n_chunks);
  if (ri.m == ri.n) return;                       // every visible token is kept
  TopkRow* st = ws.rows + ri.row;
  const float* srow = scores + (int64_t)ri.row * L_max;

  uint32_t u[kTopkPer];
  uint64_t valid = 0;
  if (ri.lo < ri.hi) load_chunk<VEC>(srow, ri.lo, ri.hi, u, valid);

  uint32_t prefix = 0;
  if (LEVEL == 1) {
    uint32_t b1;
    int rem1;
    find_bin<kNB1>(st->hist1, ri.m, lds4, &b1, &rem1);
    if (ri.chunk == 0 && threadIdx.x == 0) { st->bin[0] = b1; st->rem[0] = rem1; }
    prefix = b1;
  } else if (LEVEL == 2) {
    uint32_t b2;
    int rem2;
    const uint32_t b1 = st->bin[0];
    find_bin<kNB2>(st->hist2, st->rem[0], lds4, &b2, &rem2);
    if (ri.chunk == 0 && threadIdx.x == 0) { st->bin[1] = b2; st->rem[1] = rem2; }
    prefix = (b1 << 11) | b2;
  }
  if (ri.lo >= ri.hi) return;                     // block-uniform; after the find's barriers

  for (int i = threadIdx.x; i < NB; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kTopkPer; ++e) {
    if (!((valid >> e) & 1)) continue;
    const uint32_t x = u[e];
    if (LEVEL == 0) atomicAdd(&hist[x >> 21], 1u);
    else if (LEVEL == 1) { if ((x >> 21) == prefix) atomicAdd(&hist[(x >> 10) & 0x7FF], 1u); }
    else { if ((x >> 10) == prefix) atomicAdd(&hist[x & 0x3FF], 1u); }
  }
  __syncthreads();
  uint32_t* gh = LEVEL == 0 ? st->hist1 : (LEVEL == 1 ? st->hist2 : st->hist3);
  for (int i = threadIdx.x; i < NB; i += kTopkThreads) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
}

// Finds T and the tie quota, then counts keys > T and == T in the chunk.
template <bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_count_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TopkWs ws) {
  __shared__ uint32_t lds4[4];
  const RowInfo ri = row_info(seq_lens, q_pos, Q, in_Q, L_max, k, n_chunks);
  if (ri.m == ri.n) return;
  TopkRow* st = ws.rows + ri.row;
  const float* srow = scores + (int64_t)ri.row * L_max;
  uint32_t u[kTopkPer];
  uint64_t valid = 0;
  if (ri.lo < ri.hi) load_chunk<VEC>(srow, ri.lo, ri.hi, u, valid);
  uint32_t b3;
  int rem3;
  find_bin<kNB3>(st->hist3, st->rem[1], lds4, &b3, &rem3);
  const uint32_t T = (st->bin[0] << 21) | (st->bin[1] << 10) | b3;
  if (ri.chunk == 0 && threadIdx.x == 0) { st->bin[2] = b3; st->rem[2] = rem3; }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < kTopkPer; ++e) {
    const bool ok = (valid >> e) & 1;
    gt += ok && u[e] > T;
    eq += ok && u[e] == T;
  }
  uint32_t dummy;
  static_assert(kTopkChunk < 65536, "per-chunk counts fit 16 bits");
  const uint32_t packed = block_exclusive_scan(gt | (eq << 16), &dummy, lds4);
  if (threadIdx.x == 0) {
    const int64_t c = (int64_t)ri.row * n_chunks + ri.chunk;
    ws.gt[c] = (int32_t)(packed & 0xFFFF);
    ws.eq[c] = (int32_t)(packed >> 16);
  }
}

// Ordered compaction of each chunk's kept positions into idx.
template <bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_compact_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TopkWs ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t lds4[4];
  const RowInfo ri = row_info(seq_lens, q_pos, Q, in_Q, L_max, k, n_chunks);
  int32_t* out = idx + (int64_t)ri.row * k;
  if (ri.chunk == 0)
    for (int i = ri.m + (int)threadIdx.x; i < k; i += kTopkThreads) out[i] = -1;
  if (ri.lo >= ri.hi) return;
  if (ri.m == ri.n) {                      // keep all visible: position i goes to slot i
    for (int i = ri.lo + (int)threadIdx.x; i < ri.hi; i += kTopkThreads) out[i] = i;
    return;
  }
  const TopkRow* st = ws.rows + ri.row;
  const uint32_t T = (st->bin[0] << 21) | (st->bin[1] << 10) | st->bin[2];
  const int rem = st->rem[2];
  uint32_t u[kTopkPer];
  uint64_t valid;
  load_chunk<VEC>(scores + (int64_t)ri.row * L_max, ri.lo, ri.hi, u, valid);

  // keys kept by earlier chunks of the row, and ties seen before this chunk
  const int64_t cbase = (int64_t)ri.row * n_chunks;
  uint32_t gt_b = 0, eq_b = 0;
  for (int c = threadIdx.x; c < ri.chunk; c += kTopkThreads) {
    gt_b += (uint32_t)ws.gt[cbase + c];
    eq_b += (uint32_t)ws.eq[cbase + c];
  }
  uint32_t dummy;
  const uint32_t gt_before = block_exclusive_scan(gt_b, &dummy, lds4);
  const uint32_t eq_before = block_exclusive_scan(eq_b, &dummy, lds4);
  const int quota = max(0, min((int)ws.eq[cbase + ri.chunk], rem - (int)eq_before));
  const int off = (int)gt_before + min((int)eq_before, rem);

  int gt_carry = 0, eq_carry = 0;
#pragma unroll
  for (int v = 0; v < kTopkVpt; ++v) {
    const int i0 = ri.lo + kTopkVec * (int)threadIdx.x + kTopkThreads * kTopkVec * v;
    uint32_t fgt = 0, feq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool ok = (valid >> (4 * v + e)) & 1;
      fgt |= (uint32_t)(ok && u[4 * v + e] > T) << e;
      feq |= (uint32_t)(ok && u[4 * v + e] == T) << e;
    }
    const uint32_t packed = (uint32_t)__builtin_popcount(fgt) | ((uint32_t)__builtin_popcount(feq) << 16);
    uint32_t before;
    const uint32_t tot = block_exclusive_scan(packed, &before, lds4);
    int g_b = gt_carry + (int)(before & 0xFFFF);
    int q_b = eq_carry + (int)(before >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool g = (fgt >> e) & 1, q = (feq >> e) & 1;
      const int slot = off + g_b + min(q_b, quota);
      if ((g || (q && q_b < quota)) && slot < k) out[slot] = i0 + e;
      g_b += g;
      q_b += q;
    }
    gt_carry += (int)(tot & 0xFFFF);
    eq_carry += (int)(tot >> 16);
  }
}

template <bool VEC>
static void launch_all(const HostBatch& bt, const float* scores, int k, int32_t* idx, TopkWs w, int rows,
                       int n_chunks, hipStream_t s) {
  const dim3 block(kTopkThreads), grid((unsigned)rows * n_chunks);
  hipLaunchKernelGGL(topk_zero_kernel, dim3(rows), block, 0, s, w.rows);
  hipLaunchKernelGGL((topk_hist_kernel<0, VEC>), grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL((topk_hist_kernel<1, VEC>), grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL((topk_hist_kernel<2, VEC>), grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_count_kernel<VEC>, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_compact_kernel<VEC>, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q,
                     bt.L_max, k, n_chunks, w, idx);
}

hipError_t launch(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s) {
  const int rows = bt.B * bt.Q;
  const int n_chunks = (bt.L_max + kTopkChunk - 1) / kTopkChunk;
  TopkWs w = carve(ws, rows, n_chunks);
  // 16-byte vector loads need every row to start 16-byte aligned
  if (bt.L_max % 4 == 0 && ((uintptr_t)scores & 15) == 0)
    launch_all<true>(bt, scores, k, idx, w, rows, n_chunks, s);
  else
    launch_all<false>(bt, scores, k, idx, w, rows, n_chunks, s);
  return hipGetLastError();
}

}  // namespace radix
}  // namespace dsa
