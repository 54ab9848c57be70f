// HiSparse hot buffer ("GLM-5.2 inference deployment" page, HiSparse section: the full KV
// cache sits in pinned host memory and the GPU keeps a buffer of hot slots, one KV page per
// slot). After a step's top-k, the swap-in detects the selected pages the buffer misses,
// evicts the least recently used slots, updates the page table and pulls the missing latent
// pages from host memory. Three launches on one stream:
//   mark   one thread per selected position: the page's clock is set to this step; a page
//          that is resident refreshes its slot's clock (so it cannot be evicted this step).
//   plan   one 1024-thread workgroup per sequence: the missing pages in ascending page order
//          (with one index set per sequence in dsa_topk's order, an ordered compaction of the
//          first position of each page run in the set; otherwise an ordered block compaction
//          over the page clocks); the same number of victims,
//          the least recently used of the slots this step does not use, ties to the lower
//          slot (a 4-pass radix select of the threshold clock, then an ordered compaction
//          with a quota for the slots at that clock), listed in ascending slot order; then
//          the table updates, the i-th missing page into the i-th victim. The copy list
//          (page, slot) and its length go to the workspace.
//   copy   one workgroup per copy-list entry: the page's rows from the host pool into the
//          slot, 16 bytes per lane. The host pool is read in place over the host link (pinned,
//          device-mapped memory), so no host thread waits for the miss list.
// A slot's clock is the last step whose selected set held its page; never-used slots have
// clock -1 and go first; equal clocks go to the lower slot. Physical page b * n_slots + s is
// slot s of sequence b, so the page table is the block table of the latent cache that sparse
// MLA reads.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {
namespace hs {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanPages = 4;                          // pages per thread and pass of the miss scan (16 measured slower)
constexpr int kCopyThreads = 256;

struct PlanLds {
  uint32_t wsum[2][kPlanWaves];
  uint32_t hist[256];
  uint32_t res[2];
};

// Exclusive prefix sum of one value per thread over the 1024-thread block, in thread order;
// *total gets the block sum. Two barriers; the per-wave partials alternate between two
// arrays, so back-to-back calls need no extra barrier.
__device__ uint32_t block_scan(PlanLds& L, int parity, uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_incl_scan(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 63) L.wsum[parity][wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kPlanWaves; ++i) {
    const uint32_t t = L.wsum[parity][i];
    before += i < wave ? t : 0u;
    tot += t;
  }
  *total = tot;
  return before + incl - v;
}

__global__ __launch_bounds__(256) void hs_mark_kernel(const int32_t* __restrict__ idx, int n_sets, int k, int chunks,
                                                    int32_t step, int32_t* __restrict__ block_table,
                                                    int32_t* __restrict__ slot_clock, int32_t* __restrict__ page_clock,
                                                    int max_pages, int n_slots, int page_size) {
  const int per_seq = n_sets * chunks;
  const int b = blockIdx.x / per_seq;
  const int rest = blockIdx.x - b * per_seq;
  const int set = rest / chunks, i = (rest - set * chunks) * 256 + threadIdx.x;
  if (i >= k) return;
  const int pos = idx[((int64_t)b * n_sets + set) * k + i];
  if (pos < 0) return;
  const int page = pos / page_size;
  if (page >= max_pages) return;                        // outside the sequence's pages
  page_clock[(int64_t)b * max_pages + page] = step;    // every writer stores the same value
  const int phys = block_table[(int64_t)b * max_pages + page];
  const int s = phys - b * n_slots;
  if (phys >= 0 && s >= 0 && s < n_slots) slot_clock[(int64_t)b * n_slots + s] = step;
}

__global__ __launch_bounds__(kPlanThreads) void hs_plan_kernel(const int32_t* __restrict__ idx, int n_sets, int k,
                                                               int page_size, int32_t step,
                                                               int32_t* __restrict__ block_table,
                                                               int32_t* __restrict__ slot_page,
                                                               int32_t* __restrict__ slot_clock,
                                                               const int32_t* __restrict__ page_clock, int max_pages,
                                                               int n_slots, int cap, int32_t* __restrict__ miss_page,
                                                               int32_t* __restrict__ victim, int32_t* __restrict__ n_copy,
                                                               int32_t* __restrict__ copied) {
  __shared__ PlanLds L;
  const int b = blockIdx.x, tid = threadIdx.x;
  int32_t* bt = block_table + (int64_t)b * max_pages;
  const int32_t* pc = page_clock + (int64_t)b * max_pages;
  int32_t* sp = slot_page + (int64_t)b * n_slots;
  int32_t* sc = slot_clock + (int64_t)b * n_slots;
  int32_t* mp = miss_page + (int64_t)b * cap;
  int32_t* vs = victim + (int64_t)b * cap;
  int parity = 0;

  // ---- missing pages (selected this step, not resident), ascending.
  uint32_t n_miss = 0;
  bool listed = false;
  // One index set whose valid positions ascend, -1 only after them (as dsa_topk writes it):
  // pages ascend too and repeat only in runs, so the first position of each run names its page
  // once, in order. Positions i and i + kPlanThreads per thread (k <= 2 kPlanThreads).
  if (n_sets == 1) {
    const int32_t* ip = idx + (int64_t)b * k;
    int cur[2], prv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = tid + e * kPlanThreads;
      cur[e] = i < k ? ip[i] : -1;
      prv[e] = (i > 0 && i < k) ? ip[i - 1] : -1;
    }
    int bad = 0;
#pragma unroll
    for (int e = 0; e < 2; ++e)
      if (cur[e] >= 0 && tid + e * kPlanThreads > 0 && (prv[e] < 0 || prv[e] > cur[e])) bad = 1;
    if (!__syncthreads_or(bad)) {                        // workgroup-uniform
      int page[2], res[2];
      bool cand[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        page[e] = cur[e] >= 0 ? cur[e] / page_size : -1;
        const int pp = prv[e] >= 0 ? prv[e] / page_size : -1;
        cand[e] = cur[e] >= 0 && page[e] < max_pages && page[e] != pp;
        res[e] = bt[cand[e] ? page[e] : 0];              // both loads go out together
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {                      // positions [0, 1024), then [1024, 2048)
        const uint32_t flag = cand[e] && res[e] < 0;
        uint32_t tot;
        const uint32_t at = n_miss + block_scan(L, parity, flag, &tot);
        parity ^= 1;
        if (flag && at < (uint32_t)cap) mp[at] = page[e];
        n_miss += tot;
      }
      listed = true;
    }
  }
  // Otherwise every page clock: kPlanPages consecutive pages per thread and pass. Loads are
  // clamped into the sequence's pages (and masked) rather than branched, and the next pass's go
  // out before this pass's scan, so that the passes do not wait for memory one after another.
  int pc_cur[kPlanPages], bt_cur[kPlanPages], pc_nxt[kPlanPages], bt_nxt[kPlanPages];
  auto load_pages = [&](int base, int (&c)[kPlanPages], int (&t)[kPlanPages]) {
#pragma unroll
    for (int e = 0; e < kPlanPages; ++e) {
      const int p = min(base + kPlanPages * tid + e, max_pages - 1);
      c[e] = pc[p];
      t[e] = bt[p];
    }
  };
  if (!listed) load_pages(0, pc_cur, bt_cur);
  for (int base = 0; !listed && base < max_pages; base += kPlanPages * kPlanThreads) {
    load_pages(base + kPlanPages * kPlanThreads, pc_nxt, bt_nxt);
    uint32_t flags = 0;
#pragma unroll
    for (int e = 0; e < kPlanPages; ++e) {
      const int p = base + kPlanPages * tid + e;
      if (p < max_pages && pc_cur[e] == step && bt_cur[e] < 0) flags |= 1u << e;
    }
    uint32_t tot;
    uint32_t at = n_miss + block_scan(L, parity, (uint32_t)__builtin_popcount(flags), &tot);
    parity ^= 1;
#pragma unroll
    for (int e = 0; e < kPlanPages; ++e)
      if ((flags >> e) & 1) {
        if (at < (uint32_t)cap) mp[at] = base + kPlanPages * tid + e;
        ++at;
      }
    n_miss += tot;
#pragma unroll
    for (int e = 0; e < kPlanPages; ++e) {
      pc_cur[e] = pc_nxt[e];
      bt_cur[e] = bt_nxt[e];
    }
  }
  if (n_miss > (uint32_t)cap) n_miss = cap;             // the host check rules this out
  if (n_miss == 0) {                                     // workgroup-uniform
    if (tid == 0) {
      n_copy[b] = 0;
      if (copied) copied[b] = 0;
    }
    return;
  }

  // ---- victims: the n_miss smallest keys (clock + 1) among slots not used this step (clock
  // below the step), ties to the lower slot. Radix select of the threshold key T, 8 bits at a
  // time from the top. Slot clocks are read four per thread at once, clamped into the sequence's
  // slots and masked.
  uint32_t prefix = 0;
  int need = (int)n_miss;
  if (tid == 0) L.res[0] = L.res[1] = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    // every eligible key is at most `step`: levels above its top bit are all zero (bin 0 holds
    // every key, so the prefix gains a zero byte and `need` stays)
    if (shift > 0 && (step >> shift) == 0) {             // workgroup-uniform
      prefix <<= 8;
      continue;
    }
    for (int i = tid; i < 256; i += kPlanThreads) L.hist[i] = 0u;
    __syncthreads();
    for (int s0 = 0; s0 < n_slots; s0 += 4 * kPlanThreads) {
      int c[4];                                          // four clocks per thread, loaded together
#pragma unroll
      for (int e = 0; e < 4; ++e) c[e] = sc[min(s0 + e * kPlanThreads + tid, n_slots - 1)];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = (uint32_t)(c[e] + 1);
        const bool ok = s0 + e * kPlanThreads + tid < n_slots && c[e] < step;
        const bool match = shift == 24 || (key >> (shift + 8)) == prefix;
        if (ok && match) atomicAdd(&L.hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (tid < 64) {                                      // wave 0: the bin of the need-th smallest
      uint32_t h[4], mine = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = L.hist[4 * tid + e];
        mine += h[e];
      }
      const uint32_t incl = wave_incl_scan(mine, 0u, [](uint32_t a, uint32_t c) { return a + c; });
      uint32_t cum = incl - mine;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (cum < (uint32_t)need && (uint32_t)need <= cum + h[e]) {
          L.res[0] = 4 * tid + e;
          L.res[1] = (uint32_t)need - cum;
        }
        cum += h[e];
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | L.res[0];
    need = (int)L.res[1];
    __syncthreads();                                     // res is rewritten by the next pass
  }
  const uint32_t T = prefix;                             // keys < T all go; need of those == T
  // ordered compaction in slot order: keys below T, and the first `need` slots at T
  uint32_t taken = 0, eq_seen = 0;
  for (int base = 0; base < n_slots; base += 4 * kPlanThreads) {
    uint32_t lt = 0, eq = 0;
    int c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) c[e] = sc[min(base + 4 * tid + e, n_slots - 1)];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = (uint32_t)(c[e] + 1);
      const bool ok = base + 4 * tid + e < n_slots && c[e] < step;
      if (ok && key < T) lt |= 1u << e;
      if (ok && key == T) eq |= 1u << e;
    }
    uint32_t tot_eq;
    uint32_t eq_before = eq_seen + block_scan(L, parity, (uint32_t)__builtin_popcount(eq), &tot_eq);
    parity ^= 1;
    uint32_t take = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool q = (eq >> e) & 1;
      if (((lt >> e) & 1) || (q && eq_before < (uint32_t)need)) take |= 1u << e;
      eq_before += q;
    }
    uint32_t tot_take;
    uint32_t at = taken + block_scan(L, parity, (uint32_t)__builtin_popcount(take), &tot_take);
    parity ^= 1;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((take >> e) & 1) {
        if (at < n_miss) vs[at] = base + 4 * tid + e;
        ++at;
      }
    taken += tot_take;
    eq_seen += tot_eq;
  }
  // Every miss has a victim when the step selects at most n_slots pages and is later than
  // every step before it (the caller's contract); otherwise only the pairs that exist are made.
  const uint32_t n_pairs = min(n_miss, taken);
  if (tid == 0) {
    n_copy[b] = (int32_t)n_pairs;
    if (copied) copied[b] = (int32_t)n_pairs;
  }
  __syncthreads();                                       // the lists are complete

  // ---- table updates: the i-th missing page takes the i-th victim in slot order (old pages
  // leave; they are resident and not selected, the new ones are selected and not resident:
  // disjoint)
  for (uint32_t i = tid; i < n_pairs; i += kPlanThreads) {
    const int p = mp[i], s = vs[i];
    const int old = sp[s];
    if (old >= 0 && old < max_pages) bt[old] = -1;
    bt[p] = b * n_slots + s;
    sp[s] = p;
    sc[s] = step;
  }
}

__global__ __launch_bounds__(kCopyThreads) void hs_copy_kernel(const uint8_t* __restrict__ host_pool,
                                                             uint8_t* __restrict__ device_pool, int cap,
                                                             const int32_t* __restrict__ miss_page,
                                                             const int32_t* __restrict__ victim,
                                                             const int32_t* __restrict__ n_copy, int max_pages,
                                                             int n_slots, int page_size, int row_bytes) {
  const int b = blockIdx.x / cap, i = blockIdx.x - b * cap;
  if (i >= n_copy[b]) return;
  const int p = miss_page[(int64_t)b * cap + i], s = victim[(int64_t)b * cap + i];
  if (p < 0 || p >= max_pages || s < 0 || s >= n_slots) return;   // written by the plan; never so
  const int64_t page_bytes = (int64_t)page_size * row_bytes;
  const int64_t chunks = page_bytes / 16;                          // 16-byte chunks per page
  const v4i* src = (const v4i*)(host_pool + ((int64_t)b * max_pages + p) * page_bytes);
  v4i* dst = (v4i*)(device_pool + ((int64_t)b * n_slots + s) * page_bytes);
  for (int64_t c = threadIdx.x; c < chunks; c += kCopyThreads) dst[c] = src[c];
}

}  // namespace hs

size_t hisparse_workspace_bytes(int B, int cap) {
  const size_t list = ((size_t)B * cap * sizeof(int32_t) + 255) & ~(size_t)255;
  return 2 * list + (((size_t)B * sizeof(int32_t) + 255) & ~(size_t)255);
}

hipError_t launch_hisparse_swap_in(int B, const int32_t* idx, int n_sets, int k, int32_t step, const HostHotBuffer& hb,
                                   const void* host_pool, void* device_pool, int32_t* copied, void* ws,
                                   hipStream_t s) {
  const int cap = n_sets * k;
  const size_t list = ((size_t)B * cap * sizeof(int32_t) + 255) & ~(size_t)255;
  int32_t* miss_page = (int32_t*)ws;
  int32_t* victim = (int32_t*)((char*)ws + list);
  int32_t* n_copy = (int32_t*)((char*)ws + 2 * list);
  const int chunks = (k + 255) / 256;
  hipLaunchKernelGGL(hs::hs_mark_kernel, dim3((unsigned)(B * n_sets * chunks)), dim3(256), 0, s, idx, n_sets, k, chunks,
                     step, hb.block_table, hb.slot_clock, hb.page_clock, hb.max_pages, hb.n_slots, hb.page_size);
  static_assert(2 * hs::kPlanThreads >= 2048, "the one-set miss list reads two positions per thread");
  hipLaunchKernelGGL(hs::hs_plan_kernel, dim3(B), dim3(hs::kPlanThreads), 0, s, idx, n_sets, k, hb.page_size, step,
                     hb.block_table, hb.slot_page,
                     hb.slot_clock, hb.page_clock, hb.max_pages, hb.n_slots, cap, miss_page, victim, n_copy, copied);
  hipLaunchKernelGGL(hs::hs_copy_kernel, dim3((unsigned)(B * cap)), dim3(hs::kCopyThreads), 0, s,
                     (const uint8_t*)host_pool, (uint8_t*)device_pool, cap, miss_page, victim, n_copy, hb.max_pages,
                     hb.n_slots, hb.page_size, hb.row_bytes);
  return hipGetLastError();
}

}  // namespace dsa
