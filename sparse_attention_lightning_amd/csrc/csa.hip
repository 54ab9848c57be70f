// Compressed sparse attention ("LLM architecture survey", section 2.3 DeepSeek-V4: the KV cache
// compressed along the sequence by 4, DSA's top-k selection over the compressed entries, and a
// sliding window of the last 128 raw tokens; HCA compresses by 128 and attends densely).
//
// The path reuses the DSA kernels on the compressed caches and adds two small kernels:
//   csa_prep_kernel   per query token at raw position p: the position of its last visible
//                     compressed entry, (p + 1) / ratio - 1 (an entry is visible once its last
//                     raw token is; -1 when none is), and the window's index list
//                     max(0, p - window + 1) .. p, padded with -1;
//   (indexer scan, top-k and sparse MLA over the compressed caches with those positions;
//    sparse MLA over the raw latent cache with the window lists)
//   csa_merge_kernel  one softmax over both sets, from the two partial attentions by their
//                     log-sum-exp: lse = log(e^lse_c + e^lse_w),
//                     o = e^(lse_c - lse) o_c + e^(lse_w - lse) o_w.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

// idx_all (when k covers every compressed row a sequence can have): the selection keeps every
// visible entry whatever the scores, so it is written directly, 0 .. n_c - 1 then -1, and the
// scan and top-k are skipped.
__global__ __launch_bounds__(256) void csa_prep_kernel(const int32_t* __restrict__ seq_lens,
                                                       const int32_t* __restrict__ q_pos, int Q, int ratio,
                                                       int window, int k, int32_t* __restrict__ qpos_c,
                                                       int32_t* __restrict__ idx_w, int32_t* __restrict__ idx_all) {
  const int row = blockIdx.x;
  const int b = row / Q, j = row - b * Q;
  const int p = query_pos(seq_lens, q_pos, Q, b, j);
  if (threadIdx.x == 0 && qpos_c) qpos_c[row] = (p + 1) / ratio - 1;
  if (idx_all) {
    const int n_c = (p + 1) / ratio;
    for (int i = threadIdx.x; i < k; i += blockDim.x) idx_all[(int64_t)row * k + i] = i < n_c ? i : -1;
  }
  if (idx_w) {
    const int start = max(0, p - window + 1);
    const int cnt = p - start + 1;
    for (int i = threadIdx.x; i < window; i += blockDim.x) idx_w[(int64_t)row * window + i] = i < cnt ? start + i : -1;
  }
}

// In place: out holds the window's attention (o_w) on entry and the merged result on exit.
// One thread per 4 dims of one (query token, head).
__global__ __launch_bounds__(256) void csa_merge_kernel(const float* __restrict__ o_c, const float* __restrict__ lse_c,
                                                        const float* __restrict__ lse_w, float* __restrict__ out,
                                                        float* __restrict__ lse, int64_t n_heads) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t rh = t >> 7;                         // 128 threads x 4 dims per head
  if (rh >= n_heads) return;
  const float lc = lse_c[rh], lw = lse_w[rh];
  const float m = fmaxf(lc, lw);
  v4f r = {0.f, 0.f, 0.f, 0.f};
  float l = -INFINITY;
  if (m != -INFINITY) {
    const float wc = expf(lc - m), ww = expf(lw - m);
    const float inv = 1.f / (wc + ww);
    const v4f a = *(const v4f*)(o_c + t * 4), c = *(const v4f*)(out + t * 4);
    r = (wc * inv) * a + (ww * inv) * c;
    l = m + logf(wc + ww);
  }
  *(v4f*)(out + t * 4) = r;
  if (lse && (t & 127) == 0) lse[rh] = l;
}

static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct CsaWs {
  float* scores;
  void* topk;
  int32_t* qpos_c;
  int32_t* idx_w;
  float* o_c;
  float* lse_c;
  float* lse_w;
  void* mla;
};

static CsaWs csa_carve(void* ws, int rows, int Lc_max, int H, int k, int window, size_t* total) {
  CsaWs w{};
  char* p = (char*)ws;
  auto take = [&](size_t n) { char* q = p; p += a256(n); return (void*)q; };
  if (k > 0 && k < Lc_max) {                         // a selection that needs the scores
    w.scores = (float*)take((size_t)rows * Lc_max * sizeof(float));
    w.topk = take(topk_workspace_bytes(rows, Lc_max));
    w.qpos_c = (int32_t*)take((size_t)rows * sizeof(int32_t));
  }
  if (window > 0) w.idx_w = (int32_t*)take((size_t)rows * window * sizeof(int32_t));
  if (k > 0 && window > 0) {
    w.o_c = (float*)take((size_t)rows * H * kDv * sizeof(float));
    w.lse_c = (float*)take((size_t)rows * H * sizeof(float));
    w.lse_w = (float*)take((size_t)rows * H * sizeof(float));
  }
  size_t mla = 0;
  if (k > 0) mla = std::max(mla, sparse_mla_workspace_bytes(rows, H, k, 1));
  if (window > 0) mla = std::max(mla, sparse_mla_workspace_bytes(rows, H, window, 1));
  w.mla = mla ? take(mla) : nullptr;
  *total = (size_t)(p - (char*)ws);
  return w;
}

size_t csa_workspace_bytes(int B, int Q, int L_max, int H, int ratio, int k, int window) {
  size_t total = 0;
  const int Lc_max = (L_max + ratio - 1) / ratio;
  csa_carve(nullptr, B * Q, Lc_max, H, k, window, &total);
  return total;
}

hipError_t launch_csa(const HostBatch& bt, const uint8_t* q_e4m3, const float* w, int Hi, const HostCache& keys_c,
                      const HostCache& latent_c, const HostCache& latent, int ratio, int k, int window,
                      const uint16_t* q_bf16, int H, float scale, float* out, float* lse, int32_t* idx_out, void* ws,
                      hipStream_t s) {
  const int rows = bt.B * bt.Q;
  const int Lc_max = (bt.L_max + ratio - 1) / ratio;
  size_t total = 0;
  const CsaWs W = csa_carve(ws, rows, Lc_max, H, k, window, &total);
  const bool keep_all = k >= Lc_max;                 // e.g. HCA: every visible entry, no scores needed
  hipLaunchKernelGGL(csa_prep_kernel, dim3(rows), dim3(256), 0, s, bt.seq_lens, bt.q_pos, bt.Q, ratio, window, k,
                     W.qpos_c, W.idx_w, (k > 0 && keep_all) ? idx_out : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool both = k > 0 && window > 0;
  if (k > 0) {
    // the compressed caches, addressed like any cache of Lc_max rows per sequence, with each
    // query at its last visible compressed entry
    const HostBatch bc{bt.B, bt.Q, Lc_max, bt.seq_lens, W.qpos_c, bt.Q};
    if (!keep_all) {
      if ((e = launch_index_score(bc, q_e4m3, w, Hi, keys_c, W.scores, s)) != hipSuccess) return e;
      if ((e = launch_topk(bc, W.scores, k, idx_out, W.topk, s)) != hipSuccess) return e;
    }
    if ((e = launch_sparse_mla(bc, q_bf16, H, latent_c, idx_out, k, k, scale, both ? W.o_c : out,
                               both ? W.lse_c : lse, W.mla, s)) != hipSuccess)
      return e;
  }
  if (window > 0) {
    if ((e = launch_sparse_mla(bt, q_bf16, H, latent, W.idx_w, window, window, scale, out, both ? W.lse_w : lse,
                               W.mla, s)) != hipSuccess)
      return e;
  }
  if (both) {
    const int64_t n_heads = (int64_t)rows * H;
    const int64_t threads = n_heads * (kDv / 4);
    hipLaunchKernelGGL(csa_merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, W.o_c, W.lse_c,
                       W.lse_w, out, lse, n_heads);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsa
