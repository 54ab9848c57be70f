// Internal launchers of the DSA kernels (host side). Arguments are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct HostCache {
  const void* base;
  const int32_t* table;
  int max_pages, page_size;
};

struct HostBatch {
  int B, Q, L_max;
  const int32_t* seq_lens;
  const int32_t* q_pos;
  int in_Q;   // query tokens per sequence in the inputs (q, w, q_pos rows); Q <= in_Q
};

// Lightning-indexer scores [B][Q][L_max].
hipError_t launch_index_score(const HostBatch& bt, const uint8_t* q, const float* w, int Hi,
                              const HostCache& keys, float* scores, hipStream_t s);

// Top-k selection. Workspace layout and size are owned by topk.hip.
size_t topk_workspace_bytes(int rows, int L_max);
hipError_t launch_topk(const HostBatch& bt, const float* scores, int k, int32_t* idx, void* ws, hipStream_t s);

// Sparse MLA (MQA mode). Workspace holds split partials. Layers that share one index set go up
// to kMlaMaxLayers per launch.
constexpr int kMlaMaxLayers = 8;
int sparse_mla_splits(int rows, int H, int k, int nl, bool f8);
size_t sparse_mla_workspace_bytes(int rows, int H, int k, int n_layers);
hipError_t launch_sparse_mla(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                             const int32_t* idx, int k, int idx_q_stride, float scale, float* out,
                             float* lse, void* ws, hipStream_t s);
// One softmax over the union of two index lists: idx (k entries per query token) over latent
// (bt.L_max rows per sequence) and idx2 (k2 entries) over latent2 (L_max2 rows per sequence).
hipError_t launch_sparse_mla_union(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                                   const int32_t* idx, int k, int idx_q_stride, const HostCache& latent2, int L_max2,
                                   const int32_t* idx2, int k2, int idx2_q_stride, float scale, float* out, float* lse,
                                   void* ws, hipStream_t s);
// FP8 latent rows: 576 OCP E4M3 codes per token, value = latent_scale x code (latent_scale > 0)
hipError_t launch_sparse_mla_fp8(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                                 float latent_scale, const int32_t* idx, int k, int idx_q_stride, float scale,
                                 float* out, float* lse, void* ws, hipStream_t s);
hipError_t launch_sparse_mla_layers(const HostBatch& bt, const uint16_t* const* q, int H, const HostCache* latents,
                                    const int32_t* idx, int k, int idx_q_stride, float scale, float* const* out,
                                    float* const* lse, int n_layers, void* ws, hipStream_t s);
// FP8 latent rows, one scale per layer's cache (layers sharing a scale are launched together)
hipError_t launch_sparse_mla_layers_fp8(const HostBatch& bt, const uint16_t* const* q, int H, const HostCache* latents,
                                        const float* latent_scales, const int32_t* idx, int k, int idx_q_stride,
                                        float scale, float* const* out, float* const* lse, int n_layers, void* ws,
                                        hipStream_t s);

// Compressed sparse attention: the DSA scan and top-k over compressed caches, then one attention
// over the selected compressed rows and a raw sliding window. Workspace layout owned by csa.hip.
size_t csa_workspace_bytes(int B, int Q, int L_max, int H, int ratio, int k, int window);
hipError_t launch_csa(const HostBatch& bt, const uint8_t* q_e4m3, const float* w, int Hi, const HostCache& keys_c,
                      const HostCache& latent_c, const HostCache& latent, int ratio, int k, int window,
                      const uint16_t* q_bf16, int H, float scale, float* out, float* lse, int32_t* idx_out, void* ws,
                      hipStream_t s);

// HiSparse hot buffer: top-k driven swap-in of latent pages from a host pool into per-sequence
// device slots. Workspace: the copy list (page, slot) of every sequence and its length.
struct HostHotBuffer {
  int32_t* block_table;
  int32_t* slot_page;
  int32_t* slot_clock;
  int32_t* page_clock;
  int max_pages, n_slots, page_size, row_bytes;
};
size_t hisparse_workspace_bytes(int B, int cap);
hipError_t launch_hisparse_swap_in(int B, const int32_t* idx, int n_sets, int k, int32_t step, const HostHotBuffer& hb,
                                   const void* host_pool, void* device_pool, int32_t* copied, void* ws,
                                   hipStream_t s);

}  // namespace dsa
