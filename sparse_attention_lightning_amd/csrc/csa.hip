// Compressed sparse attention ("LLM architecture survey", section 2.3 DeepSeek-V4: the KV cache
// compressed along the sequence by 4, DSA's top-k selection over the compressed entries, and a
// sliding window of the last 128 raw tokens; HCA compresses by 128 and attends densely).
//
// The path reuses the DSA kernels on the compressed caches and adds one small kernel:
//   csa_prep_kernel   per query token at raw position p: the position of its last visible
//                     compressed entry, (p + 1) / ratio - 1 (an entry is visible once its last
//                     raw token is; -1 when none is), and the window's index list
//                     max(0, p - window + 1) .. p, padded with -1;
//   (indexer scan and top-k over the compressed keys with those positions; then one sparse MLA
//    launch over the union of the two lists, the selected compressed rows of the compressed
//    latent cache and the window's rows of the raw latent cache, in one softmax: its splits run
//    over the two lists one after the other, and its combine merges them)
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

static inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct CsaWs {
  float* scores;
  void* topk;
  int32_t* qpos_c;
  int32_t* idx_w;
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
  const size_t mla = sparse_mla_workspace_bytes(rows, H, k + window, 1);
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
  if (k == 0)                                        // the window alone
    return launch_sparse_mla(bt, q_bf16, H, latent, W.idx_w, window, window, scale, out, lse, W.mla, s);
  // the compressed caches, addressed like any cache of Lc_max rows per sequence, with each query
  // at its last visible compressed entry
  const HostBatch bc{bt.B, bt.Q, Lc_max, bt.seq_lens, W.qpos_c, bt.Q};
  if (!keep_all) {
    if ((e = launch_index_score(bc, q_e4m3, w, Hi, keys_c, W.scores, s)) != hipSuccess) return e;
    if ((e = launch_topk(bc, W.scores, k, idx_out, W.topk, s)) != hipSuccess) return e;
  }
  if (window == 0) return launch_sparse_mla(bc, q_bf16, H, latent_c, idx_out, k, k, scale, out, lse, W.mla, s);
  return launch_sparse_mla_union(bc, q_bf16, H, latent_c, idx_out, k, k, latent, bt.L_max, W.idx_w, window, window,
                                 scale, out, lse, W.mla, s);
}

}  // namespace dsa
