// Token selector ("LLM architecture survey", section 2.2: each query keeps the k = 2048
// highest-scoring tokens). Exact top-k by radix select on the order-preserving uint32 image
// of the fp32 scores, ties to the lower position, output ascending.
//
// A row (one query token) is cut into chunks of kChunk scores, one workgroup per chunk, so
// long rows (128K, 1M) spread over the whole chip. Passes, one launch each:
//   level 1..3  histogram of key bits [31:21], [20:10], [9:0] among the scores that match
//               the prefix found so far (LDS histogram, then global atomics per row); the
//               last workgroup to finish a row finds the bin holding the k-th largest key
//               and the number still needed from it -> after level 3 the exact threshold
//               key T and the number of ties at T to take.
//   count       per chunk: #keys > T and #keys == T; the last workgroup of the row turns
//               these into each chunk's output offset and its share of the ties (ties are
//               taken in position order, so earlier chunks take theirs first).
//   compact     per chunk, an ordered (scan-based) compaction of the selected positions
//               into idx at the chunk's offset; chunk 0 also writes the -1 padding.
// "Last workgroup" is decided by an atomic counter per row and pass: nobody waits on anyone.
// Rows with p + 1 <= k keep every visible token and skip the histogram passes.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTopkChunk = 4096;     // scores per workgroup
constexpr int kTopkThreads = 256;
constexpr int kNB1 = 2048, kNB2 = 2048, kNB3 = 1024;

struct TopkRow {
  uint32_t hist1[kNB1];
  uint32_t hist2[kNB2];
  uint32_t hist3[kNB3];
  uint32_t ctr[4];       // finished-workgroup counters: level 1, 2, 3, count
  uint32_t bin[3];       // threshold bin of each level
  int32_t rem[3];        // scores still needed from that bin
  uint32_t pad[54];
};
static_assert(sizeof(TopkRow) % 256 == 0, "row state is 256-byte aligned");
constexpr int kZeroWords = kNB1 + kNB2 + kNB3 + 4;

struct TopkWs {
  TopkRow* rows;
  int32_t* gt;       // [rows][n_chunks]
  int32_t* eq;
  int32_t* off;
  int32_t* quota;
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t topk_workspace_bytes(int rows, int L_max) {
  const size_t n_chunks = (L_max + kTopkChunk - 1) / kTopkChunk;
  return align256(sizeof(TopkRow) * (size_t)rows) + 4 * align256(sizeof(int32_t) * rows * n_chunks);
}

static TopkWs carve(void* ws, int rows, int n_chunks) {
  char* p = (char*)ws;
  TopkWs t;
  t.rows = (TopkRow*)p;
  p += align256(sizeof(TopkRow) * (size_t)rows);
  const size_t a = align256(sizeof(int32_t) * (size_t)rows * n_chunks);
  t.gt = (int32_t*)p; p += a;
  t.eq = (int32_t*)p; p += a;
  t.off = (int32_t*)p; p += a;
  t.quota = (int32_t*)p;
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
  int p = query_pos(seq_lens, q_pos, in_Q, b, j);
  ri.n = max(0, min(p + 1, L_max));
  ri.m = min(k, ri.n);
  ri.lo = ri.chunk * kTopkChunk;
  ri.hi = min(ri.lo + kTopkChunk, ri.n);
  return ri;
}

__device__ __forceinline__ uint32_t load_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive scan of one uint32 per thread (256 threads); returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* excl, uint32_t* lds4) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t y = __shfl_up(x, d, 64);
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

// Marks this workgroup done for counter `ctr`; true in the last workgroup of the row.
__device__ __forceinline__ bool last_block(uint32_t* ctr, uint32_t n_blocks, int* lds_flag) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (old == n_blocks - 1);
  }
  __syncthreads();
  const bool last = *lds_flag;
  if (last) __threadfence();
  return last;
}

__global__ __launch_bounds__(kTopkThreads) void topk_zero_kernel(TopkRow* rows) {
  uint32_t* base = (uint32_t*)(rows + blockIdx.x);
  for (int i = threadIdx.x; i < kZeroWords; i += kTopkThreads) base[i] = 0u;
}

// One radix level. LEVEL 0: bits [31:21]; 1: [20:10] of keys whose top 11 bits == bin[0];
// 2: [9:0] of keys whose top 22 bits == (bin[0], bin[1]).
template <int LEVEL>
__global__ __launch_bounds__(kTopkThreads) void topk_level_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TopkWs ws) {
  constexpr int NB = LEVEL == 2 ? kNB3 : kNB1;
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t lds4[4];
  __shared__ int flag;
  const RowInfo ri = row_info(seq_lens, q_pos, Q, in_Q, L_max, k, n_chunks);
  if (ri.m == ri.n) return;                       // every visible token is kept
  TopkRow* st = ws.rows + ri.row;
  uint32_t prefix = 0;
  if (LEVEL == 1) prefix = st->bin[0];
  if (LEVEL == 2) prefix = (st->bin[0] << 11) | st->bin[1];

  for (int i = threadIdx.x; i < NB; i += kTopkThreads) hist[i] = 0u;
  __syncthreads();
  const float* srow = scores + (int64_t)ri.row * L_max;
  for (int i = ri.lo + (int)threadIdx.x; i < ri.hi; i += kTopkThreads) {
    const uint32_t u = float_key(srow[i]);
    if (LEVEL == 0) {
      atomicAdd(&hist[u >> 21], 1u);
    } else if (LEVEL == 1) {
      if ((u >> 21) == prefix) atomicAdd(&hist[(u >> 10) & 0x7FF], 1u);
    } else {
      if ((u >> 10) == prefix) atomicAdd(&hist[u & 0x3FF], 1u);
    }
  }
  __syncthreads();
  uint32_t* gh = LEVEL == 0 ? st->hist1 : (LEVEL == 1 ? st->hist2 : st->hist3);
  for (int i = threadIdx.x; i < NB; i += kTopkThreads) {
    const uint32_t c = hist[i];
    if (c) atomicAdd(&gh[i], c);
  }
  if (!last_block(&st->ctr[LEVEL], n_chunks, &flag)) return;

  // last workgroup of this row: find the bin holding the rem-th largest key
  const int need = LEVEL == 0 ? ri.m : st->rem[LEVEL - 1];
  constexpr int PER = NB / kTopkThreads;          // bins per thread, highest bins to thread 0
  const int top = NB - PER * (int)threadIdx.x;    // this thread's bins: [top - PER, top)
  uint32_t h[PER];
  uint32_t mine = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    h[e] = load_relaxed(&gh[top - 1 - e]);
    mine += h[e];
  }
  uint32_t above;
  block_exclusive_scan(mine, &above, lds4);
  uint32_t cum = above;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (cum < (uint32_t)need && (uint32_t)need <= cum + h[e]) {
      st->bin[LEVEL] = (uint32_t)(top - 1 - e);
      st->rem[LEVEL] = need - (int)cum;
    }
    cum += h[e];
  }
}

__device__ __forceinline__ uint32_t threshold_key(const TopkRow* st) {
  return (st->bin[0] << 21) | (st->bin[1] << 10) | st->bin[2];
}

// Per chunk: #keys > T and #keys == T; the row's last workgroup derives offsets and tie quotas.
__global__ __launch_bounds__(kTopkThreads) void topk_count_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int L_max, int k, int n_chunks, TopkWs ws) {
  __shared__ uint32_t lds4[4];
  __shared__ int flag;
  __shared__ uint32_t carry[2];
  const RowInfo ri = row_info(seq_lens, q_pos, Q, in_Q, L_max, k, n_chunks);
  if (ri.m == ri.n) return;
  TopkRow* st = ws.rows + ri.row;
  const uint32_t T = threshold_key(st);
  const float* srow = scores + (int64_t)ri.row * L_max;
  uint32_t gt = 0, eq = 0;
  for (int i = ri.lo + (int)threadIdx.x; i < ri.hi; i += kTopkThreads) {
    const uint32_t u = float_key(srow[i]);
    gt += (u > T);
    eq += (u == T);
  }
  uint32_t dummy;
  const uint32_t gt_tot = block_exclusive_scan(gt, &dummy, lds4);
  const uint32_t eq_tot = block_exclusive_scan(eq, &dummy, lds4);
  const int64_t cbase = (int64_t)ri.row * n_chunks;
  if (threadIdx.x == 0) {
    ws.gt[cbase + ri.chunk] = (int32_t)gt_tot;
    ws.eq[cbase + ri.chunk] = (int32_t)eq_tot;
  }
  if (!last_block(&st->ctr[3], n_chunks, &flag)) return;

  // offsets and tie quotas, chunk order = position order
  const int rem = st->rem[2];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int c0 = 0; c0 < n_chunks; c0 += kTopkThreads) {
    const int c = c0 + (int)threadIdx.x;
    const bool in = c < n_chunks;
    const uint32_t e = in ? load_relaxed((const uint32_t*)&ws.eq[cbase + c]) : 0u;
    const uint32_t g = in ? load_relaxed((const uint32_t*)&ws.gt[cbase + c]) : 0u;
    uint32_t e_before;
    const uint32_t e_tot = block_exclusive_scan(e, &e_before, lds4);
    e_before += carry[1];
    const int left = max(0, rem - (int)e_before);
    const uint32_t quota = (uint32_t)min((int)e, left);
    uint32_t o_before;
    const uint32_t o_tot = block_exclusive_scan(g + quota, &o_before, lds4);
    if (in) {
      ws.off[cbase + c] = (int32_t)(o_before + carry[0]);
      ws.quota[cbase + c] = (int32_t)quota;
    }
    __syncthreads();
    if (threadIdx.x == 0) { carry[0] += o_tot; carry[1] += e_tot; }
    __syncthreads();
  }
}

// Ordered compaction of each chunk's selected positions into idx.
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
  const uint32_t T = threshold_key(st);
  const int64_t cidx = (int64_t)ri.row * n_chunks + ri.chunk;
  const int off = ws.off[cidx];
  const int quota = ws.quota[cidx];
  const float* srow = scores + (int64_t)ri.row * L_max;
  int gt_carry = 0, eq_carry = 0;
  constexpr int E = 4;                        // consecutive scores per thread
  for (int base = ri.lo; base < ri.hi; base += kTopkThreads * E) {
    const int i0 = base + E * (int)threadIdx.x;
    uint32_t fgt = 0, feq = 0;                // bit e: score i0+e is > T / == T
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i < ri.hi) {
        const uint32_t u = float_key(srow[i]);
        fgt |= (uint32_t)(u > T) << e;
        feq |= (uint32_t)(u == T) << e;
      }
    }
    const uint32_t packed = (uint32_t)__builtin_popcount(fgt) | ((uint32_t)__builtin_popcount(feq) << 16);
    uint32_t before;
    const uint32_t tot = block_exclusive_scan(packed, &before, lds4);
    int gt_b = gt_carry + (int)(before & 0xFFFF);
    int eq_b = eq_carry + (int)(before >> 16);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool g = (fgt >> e) & 1, q = (feq >> e) & 1;
      const int slot = off + gt_b + min(eq_b, quota);
      if ((g || (q && eq_b < quota)) && slot < k) out[slot] = i0 + e;
      gt_b += g;
      eq_b += q;
    }
    gt_carry += (int)(tot & 0xFFFF);
    eq_carry += (int)(tot >> 16);
  }
}

hipError_t launch_topk(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s) {
  const int rows = bt.B * bt.Q;
  const int n_chunks = (bt.L_max + kTopkChunk - 1) / kTopkChunk;
  TopkWs w = carve(ws, rows, n_chunks);
  const dim3 block(kTopkThreads), grid((unsigned)rows * n_chunks);
  hipLaunchKernelGGL(topk_zero_kernel, dim3(rows), block, 0, s, w.rows);
  hipLaunchKernelGGL(topk_level_kernel<0>, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_level_kernel<1>, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_level_kernel<2>, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_count_kernel, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w);
  hipLaunchKernelGGL(topk_compact_kernel, grid, block, 0, s, scores, bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, bt.L_max, k, n_chunks, w, idx);
  return hipGetLastError();
}

}  // namespace dsa
