// C ABI of the DSA hot path: host-side validation, workspace sizing and launch order.
// Every check runs before any HIP call, so a rejected call touches neither the GPU nor
// the HIP runtime (this is what the CPU-only tests exercise). The one exception is the
// swap-in's last check, a pointer query on its host pool, after all the others.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/dsa.h"
#include "dsa_launch.h"

// Scratch of the allocation-free entry point (dsa_forward_shared_noalloc): every GPU the library
// runs on holds one copy of this array until the process ends. Host code never passes the name
// itself to a kernel or copy: in host code it is a stand-in, not a device address. The device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current.
constexpr size_t kScratchBytes = DSA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxTopK = 2048;

dsa_status check_batch(const dsa_batch_t* bt, const char* who) {
  if (!bt) return fail(DSA_ERR_INVALID_ARG, "%s: batch is NULL", who);
  if (bt->B < 1 || bt->Q < 1 || bt->L_max < 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: B=%d Q=%d L_max=%d must be >= 1", who, bt->B, bt->Q, bt->L_max);
  if (bt->Q > bt->L_max) return fail(DSA_ERR_INVALID_ARG, "%s: Q=%d exceeds L_max=%d", who, bt->Q, bt->L_max);
  if (!bt->seq_lens || !aligned(bt->seq_lens, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: seq_lens is NULL or misaligned", who);
  if (bt->q_pos && !aligned(bt->q_pos, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: q_pos misaligned", who);
  if ((int64_t)bt->B * bt->Q > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, "%s: B*Q=%lld too large", who, (long long)bt->B * bt->Q);
  if (bt->L_max > (1 << 24)) return fail(DSA_ERR_UNSUPPORTED, "%s: L_max=%d above 16M tokens", who, bt->L_max);
  return DSA_OK;
}

// Calls with a score matrix [B*Q][L_max]: at most 2^36 entries, which also keeps every grid of
// the scan and top-k kernels (one workgroup per 2048 or 4096 scores) within int range.
dsa_status check_score_matrix(const dsa_batch_t* bt, const char* who) {
  if ((int64_t)bt->B * bt->Q * bt->L_max > (int64_t(1) << 36))
    return fail(DSA_ERR_UNSUPPORTED, "%s: B*Q*L_max=%lld scores above 2^36", who,
                (long long)bt->B * bt->Q * bt->L_max);
  return DSA_OK;
}

dsa_status check_cache(const dsa_cache_t* c, int L_max, const char* who, const char* name) {
  if (!c) return fail(DSA_ERR_INVALID_ARG, "%s: %s cache is NULL", who, name);
  if (!c->base || !aligned(c->base, 16)) return fail(DSA_ERR_INVALID_ARG, "%s: %s base is NULL or not 16-byte aligned", who, name);
  if (c->block_table) {
    if (!aligned(c->block_table, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: %s block_table misaligned", who, name);
    if (c->page_size < 16 || c->page_size % 16)
      return fail(DSA_ERR_UNSUPPORTED, "%s: %s page_size=%d must be a positive multiple of 16", who, name, c->page_size);
    const int64_t need = ((int64_t)L_max + c->page_size - 1) / c->page_size;
    if (c->max_pages < need)
      return fail(DSA_ERR_INVALID_ARG, "%s: %s max_pages=%d < ceil(L_max/page_size)=%lld", who, name, c->max_pages, (long long)need);
  }
  return DSA_OK;
}

dsa_status check_ptr(const void* p, size_t a, const char* who, const char* name) {
  if (!p || !aligned(p, a)) return fail(DSA_ERR_INVALID_ARG, "%s: %s is NULL or not %zu-byte aligned", who, name, a);
  return DSA_OK;
}

dsa_status check_ws(void* ws, size_t have, size_t need, const char* who) {
  if (need == 0) return DSA_OK;
  if (!ws || !aligned(ws, 256)) return fail(DSA_ERR_WORKSPACE, "%s: workspace is NULL or not 256-byte aligned", who);
  if (have < need) return fail(DSA_ERR_WORKSPACE, "%s: workspace %zu bytes < required %zu", who, have, need);
  return DSA_OK;
}

dsa::HostBatch host_batch(const dsa_batch_t* bt) {
  return dsa::HostBatch{bt->B, bt->Q, bt->L_max, bt->seq_lens, bt->q_pos, bt->Q};
}
dsa::HostCache host_cache(const dsa_cache_t* c) {
  return dsa::HostCache{c->base, c->block_table, c->block_table ? c->max_pages : 0,
                        c->block_table ? c->page_size : 0};
}

dsa_status launched(hipError_t e, const char* who) {
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  return DSA_OK;
}

#define TRY(x)                      \
  do {                              \
    dsa_status _st = (x);           \
    if (_st != DSA_OK) return _st;  \
  } while (0)

size_t scores_bytes(int rows, int L_max) { return align256((size_t)rows * L_max * sizeof(float)); }

// Device address of `scratch` on the GPU that owns `stream` (the current device for the NULL
// stream), looked up once per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

dsa_status scratch_for_stream(hipStream_t stream, void** out, const char* who) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: device of the stream: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(DSA_ERR_UNSUPPORTED, "%s: device %d beyond %d", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(DSA_ERR_HIP, "%s: hipSetDevice(%d): %s", who, dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who, hipGetErrorString(e));
    if (e2 != hipSuccess) return fail(DSA_ERR_HIP, "%s: hipSetDevice(%d): %s", who, cur, hipGetErrorString(e2));
    if (!p || !aligned(p, 256)) return fail(DSA_ERR_HIP, "%s: scratch address %p not 256-byte aligned", who, p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_str(dsa_status s) {
  switch (s) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "DSA_UNKNOWN_STATUS";
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

size_t dsa_workspace_size(int op, const dsa_batch_t* bt, int Hi, int H, int k, int n_layers) {
  (void)Hi;
  if (!bt || bt->B < 1 || bt->Q < 1 || bt->L_max < 1 || k < 1) return 0;
  if ((int64_t)bt->B * bt->Q > (1 << 24) || bt->L_max > (1 << 24)) return 0;   // shapes every entry point rejects
  const int rows = bt->B * bt->Q;
  switch (op) {
    case DSA_OP_INDEX_SCORE: return 0;
    case DSA_OP_TOPK: return dsa::topk_workspace_bytes(rows, bt->L_max);
    case DSA_OP_SPARSE_MLA: return (H == 64 || H == 128) ? dsa::sparse_mla_workspace_bytes(rows, H, k, 1) : 0;
    case DSA_OP_HISPARSE_SWAP_IN: return dsa::hisparse_workspace_bytes(bt->B, bt->Q * k);
    case DSA_OP_FORWARD_SHARED: {
      // scores + top-k state for every query token (the largest case), then the MLA partials
      size_t a = scores_bytes(rows, bt->L_max) + align256(dsa::topk_workspace_bytes(rows, bt->L_max));
      size_t m = ((H == 64 || H == 128) && n_layers >= 1) ? dsa::sparse_mla_workspace_bytes(rows, H, k, n_layers) : 0;
      return a + align256(m);
    }
  }
  return 0;
}

dsa_status dsa_index_score(const dsa_batch_t* batch, const uint8_t* q, const float* w, int Hi,
                           const dsa_cache_t* keys, float* scores, void* stream) {
  const char* who = "dsa_index_score";
  TRY(check_batch(batch, who));
  TRY(check_score_matrix(batch, who));
  if (Hi != 32 && Hi != 64) return fail(DSA_ERR_UNSUPPORTED, "%s: Hi=%d (supported: 32, 64)", who, Hi);
  TRY(check_ptr(q, 16, who, "q"));
  TRY(check_ptr(w, 4, who, "w"));
  TRY(check_ptr(scores, 4, who, "scores"));
  TRY(check_cache(keys, batch->L_max, who, "keys"));
  g_last_error.clear();
  return launched(dsa::launch_index_score(host_batch(batch), q, w, Hi, host_cache(keys), scores, (hipStream_t)stream), who);
}

dsa_status dsa_topk(const dsa_batch_t* batch, const float* scores, int k, int32_t* idx, void* ws, size_t ws_bytes,
                    void* stream) {
  const char* who = "dsa_topk";
  TRY(check_batch(batch, who));
  TRY(check_score_matrix(batch, who));
  if (k < 1 || k > kMaxTopK) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [1, %d]", who, k, kMaxTopK);
  TRY(check_ptr(scores, 4, who, "scores"));
  TRY(check_ptr(idx, 4, who, "idx"));
  TRY(check_ws(ws, ws_bytes, dsa::topk_workspace_bytes(batch->B * batch->Q, batch->L_max), who));
  g_last_error.clear();
  return launched(dsa::launch_topk(host_batch(batch), scores, k, idx, ws, (hipStream_t)stream), who);
}

dsa_status dsa_sparse_mla_fwd(const dsa_batch_t* batch, const uint16_t* q, int H, const dsa_cache_t* latent,
                              const int32_t* idx, int k, int idx_q_stride, float softmax_scale, float* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
  const char* who = "dsa_sparse_mla_fwd";
  TRY(check_batch(batch, who));
  if (H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: H=%d (supported: 64, 128)", who, H);
  if (k < 1 || k > kMaxTopK) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [1, %d]", who, k, kMaxTopK);
  if (idx_q_stride != 0 && idx_q_stride != k)
    return fail(DSA_ERR_INVALID_ARG, "%s: idx_q_stride=%d must be 0 or k=%d", who, idx_q_stride, k);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(DSA_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0", who);
  TRY(check_ptr(q, 16, who, "q"));
  TRY(check_ptr(idx, 4, who, "idx"));
  TRY(check_ptr(out, 16, who, "out"));
  if (lse && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: lse misaligned", who);
  TRY(check_cache(latent, batch->L_max, who, "latent"));
  TRY(check_ws(ws, ws_bytes, dsa::sparse_mla_workspace_bytes(batch->B * batch->Q, H, k, 1), who));
  g_last_error.clear();
  return launched(dsa::launch_sparse_mla(host_batch(batch), q, H, host_cache(latent), idx, k, idx_q_stride,
                                         softmax_scale, out, lse, ws, (hipStream_t)stream),
                  who);
}

dsa_status dsa_sparse_mla_fwd_fp8(const dsa_batch_t* batch, const uint16_t* q, int H, const dsa_cache_t* latent,
                                  float latent_scale, const int32_t* idx, int k, int idx_q_stride,
                                  float softmax_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                                  void* stream) {
  const char* who = "dsa_sparse_mla_fwd_fp8";
  TRY(check_batch(batch, who));
  if (H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: H=%d (supported: 64, 128)", who, H);
  if (k < 1 || k > kMaxTopK) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [1, %d]", who, k, kMaxTopK);
  if (idx_q_stride != 0 && idx_q_stride != k)
    return fail(DSA_ERR_INVALID_ARG, "%s: idx_q_stride=%d must be 0 or k=%d", who, idx_q_stride, k);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(DSA_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0", who);
  if (!std::isfinite(latent_scale) || !(latent_scale > 0.f))
    return fail(DSA_ERR_INVALID_ARG, "%s: latent_scale must be finite and > 0", who);
  TRY(check_ptr(q, 16, who, "q"));
  TRY(check_ptr(idx, 4, who, "idx"));
  TRY(check_ptr(out, 16, who, "out"));
  if (lse && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: lse misaligned", who);
  TRY(check_cache(latent, batch->L_max, who, "latent"));
  TRY(check_ws(ws, ws_bytes, dsa::sparse_mla_workspace_bytes(batch->B * batch->Q, H, k, 1), who));
  g_last_error.clear();
  return launched(dsa::launch_sparse_mla_fp8(host_batch(batch), q, H, host_cache(latent), latent_scale, idx, k,
                                             idx_q_stride, softmax_scale, out, lse, ws, (hipStream_t)stream),
                  who);
}

}  // extern "C"

namespace {

// Argument checks of an IndexShare group call (everything but the workspace).
dsa_status check_forward_shared(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                                const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                                const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents,
                                float softmax_scale, float* const* out, float* const* lse, int32_t* idx_out,
                                const char* who) {
  TRY(check_batch(batch, who));
  TRY(check_score_matrix(batch, who));
  if (Hi != 32 && Hi != 64) return fail(DSA_ERR_UNSUPPORTED, "%s: Hi=%d (supported: 32, 64)", who, Hi);
  if (H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: H=%d (supported: 64, 128)", who, H);
  if (k < 1 || k > kMaxTopK) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [1, %d]", who, k, kMaxTopK);
  if (share_first_query != 0 && share_first_query != 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: share_first_query=%d must be 0 or 1", who, share_first_query);
  if (n_layers < 1 || n_layers > 64) return fail(DSA_ERR_INVALID_ARG, "%s: n_layers=%d outside [1, 64]", who, n_layers);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(DSA_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0", who);
  TRY(check_ptr(q_e4m3, 16, who, "q_e4m3"));
  TRY(check_ptr(w, 4, who, "w"));
  TRY(check_ptr(idx_out, 4, who, "idx_out"));
  TRY(check_cache(keys, batch->L_max, who, "keys"));
  if (!q_bf16 || !latents || !out) return fail(DSA_ERR_INVALID_ARG, "%s: per-layer arrays must not be NULL", who);
  for (int l = 0; l < n_layers; ++l) {
    TRY(check_ptr(q_bf16[l], 16, who, "q_bf16[layer]"));
    TRY(check_ptr(out[l], 16, who, "out[layer]"));
    TRY(check_cache(&latents[l], batch->L_max, who, "latent"));
    if (lse && lse[l] && !aligned(lse[l], 4)) return fail(DSA_ERR_INVALID_ARG, "%s: lse[%d] misaligned", who, l);
  }
  return DSA_OK;
}

// The launches of an IndexShare group call on a checked workspace of the required size.
dsa_status run_forward_shared(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                              const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                              const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents, float softmax_scale,
                              float* const* out, float* const* lse, int32_t* idx_out, void* ws, hipStream_t s,
                              const char* who, const float* latent_scales = nullptr) {
  const int rows_all = batch->B * batch->Q;
  dsa::HostBatch sel = host_batch(batch);          // the query tokens that get scores + top-k
  if (share_first_query) sel.Q = 1;                // token 0 of each sequence; inputs keep stride Q
  char* p = (char*)ws;
  float* scores = (float*)p;
  p += scores_bytes(rows_all, batch->L_max);
  void* topk_ws = p;
  p += align256(dsa::topk_workspace_bytes(rows_all, batch->L_max));
  void* mla_ws = p;

  TRY(launched(dsa::launch_index_score(sel, q_e4m3, w, Hi, host_cache(keys), scores, s), who));
  TRY(launched(dsa::launch_topk(sel, scores, k, idx_out, topk_ws, s), who));
  const int stride = share_first_query ? 0 : k;
  std::vector<dsa::HostCache> lat(n_layers);
  std::vector<float*> lse_l(n_layers);
  for (int l = 0; l < n_layers; ++l) {
    lat[l] = host_cache(&latents[l]);
    lse_l[l] = lse ? lse[l] : nullptr;
  }
  // all layers of the group in one launch (up to 8 at a time): they share the index set
  if (latent_scales)
    TRY(launched(dsa::launch_sparse_mla_layers_fp8(host_batch(batch), q_bf16, H, lat.data(), latent_scales, idx_out,
                                                   k, stride, softmax_scale, out, lse_l.data(), n_layers, mla_ws, s),
                 who));
  else
    TRY(launched(dsa::launch_sparse_mla_layers(host_batch(batch), q_bf16, H, lat.data(), idx_out, k, stride,
                                               softmax_scale, out, lse_l.data(), n_layers, mla_ws, s),
                 who));
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status dsa_forward_shared(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                              const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                              const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents, float softmax_scale,
                              float* const* out, float* const* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                              void* stream) {
  const char* who = "dsa_forward_shared";
  TRY(check_forward_shared(batch, q_e4m3, w, Hi, keys, k, share_first_query, n_layers, q_bf16, H, latents,
                           softmax_scale, out, lse, idx_out, who));
  const size_t need = dsa_workspace_size(DSA_OP_FORWARD_SHARED, batch, Hi, H, k, n_layers);
  TRY(check_ws(ws, ws_bytes, need, who));
  g_last_error.clear();
  return run_forward_shared(batch, q_e4m3, w, Hi, keys, k, share_first_query, n_layers, q_bf16, H, latents,
                            softmax_scale, out, lse, idx_out, ws, (hipStream_t)stream, who);
}

dsa_status dsa_forward_shared_fp8(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                                  const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                                  const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents,
                                  const float* latent_scales, float softmax_scale, float* const* out,
                                  float* const* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "dsa_forward_shared_fp8";
  TRY(check_forward_shared(batch, q_e4m3, w, Hi, keys, k, share_first_query, n_layers, q_bf16, H, latents,
                           softmax_scale, out, lse, idx_out, who));
  if (!latent_scales) return fail(DSA_ERR_INVALID_ARG, "%s: latent_scales is NULL", who);
  for (int l = 0; l < n_layers; ++l)
    if (!std::isfinite(latent_scales[l]) || !(latent_scales[l] > 0.f))
      return fail(DSA_ERR_INVALID_ARG, "%s: latent_scales[%d] must be finite and > 0", who, l);
  const size_t need = dsa_workspace_size(DSA_OP_FORWARD_SHARED, batch, Hi, H, k, n_layers);
  TRY(check_ws(ws, ws_bytes, need, who));
  g_last_error.clear();
  return run_forward_shared(batch, q_e4m3, w, Hi, keys, k, share_first_query, n_layers, q_bf16, H, latents,
                            softmax_scale, out, lse, idx_out, ws, (hipStream_t)stream, who, latent_scales);
}

dsa_status dsa_forward_shared_noalloc(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                                      const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                                      const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents,
                                      float softmax_scale, float* const* out, float* const* lse, int32_t* idx_out,
                                      void* stream) {
  const char* who = "dsa_forward_shared_noalloc";
  TRY(check_forward_shared(batch, q_e4m3, w, Hi, keys, k, share_first_query, n_layers, q_bf16, H, latents,
                           softmax_scale, out, lse, idx_out, who));
  const size_t need = dsa_workspace_size(DSA_OP_FORWARD_SHARED, batch, Hi, H, k, n_layers);
  if (need > kScratchBytes)
    return fail(DSA_ERR_UNSUPPORTED,
                "%s: this call needs %zu bytes of scratch, above the %zu bytes the library holds per device; "
                "call dsa_forward_shared with a workspace of dsa_workspace_size(DSA_OP_FORWARD_SHARED, ...) bytes",
                who, need, kScratchBytes);
  void* ws = nullptr;
  TRY(scratch_for_stream((hipStream_t)stream, &ws, who));
  g_last_error.clear();
  return run_forward_shared(batch, q_e4m3, w, Hi, keys, k, share_first_query, n_layers, q_bf16, H, latents,
                            softmax_scale, out, lse, idx_out, ws, (hipStream_t)stream, who);
}

size_t dsa_csa_workspace_size(const dsa_batch_t* bt, int H, int ratio, int k, int window) {
  if (!bt || bt->B < 1 || bt->Q < 1 || bt->L_max < 1 || (H != 64 && H != 128) || ratio < 1 || k < 0 || window < 0 ||
      k > kMaxTopK || window > kMaxTopK || (k == 0 && window == 0))
    return 0;
  return dsa::csa_workspace_bytes(bt->B, bt->Q, bt->L_max, H, ratio, k, window);
}

dsa_status dsa_csa_forward(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                           const dsa_cache_t* keys_c, const dsa_cache_t* latent_c, const dsa_cache_t* latent,
                           int ratio, int k, int window, const uint16_t* q_bf16, int H, float softmax_scale,
                           float* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "dsa_csa_forward";
  TRY(check_batch(batch, who));
  TRY(check_score_matrix(batch, who));
  if (H != 64 && H != 128) return fail(DSA_ERR_UNSUPPORTED, "%s: H=%d (supported: 64, 128)", who, H);
  if (ratio < 1 || ratio > batch->L_max) return fail(DSA_ERR_INVALID_ARG, "%s: ratio=%d outside [1, L_max]", who, ratio);
  if (k < 0 || k > kMaxTopK) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [0, %d]", who, k, kMaxTopK);
  if (window < 0 || window > kMaxTopK)
    return fail(DSA_ERR_UNSUPPORTED, "%s: window=%d outside [0, %d]", who, window, kMaxTopK);
  if (k == 0 && window == 0) return fail(DSA_ERR_INVALID_ARG, "%s: k and window are both 0: nothing to attend", who);
  if (!std::isfinite(softmax_scale) || softmax_scale < 0.f)
    return fail(DSA_ERR_INVALID_ARG, "%s: softmax_scale must be finite and >= 0", who);
  TRY(check_ptr(q_bf16, 16, who, "q_bf16"));
  TRY(check_ptr(out, 16, who, "out"));
  if (lse && !aligned(lse, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: lse misaligned", who);
  const int Lc_max = (batch->L_max + ratio - 1) / ratio;
  if (k > 0) {
    if (k < Lc_max) {                                // the selection reads the scores
      if (Hi != 32 && Hi != 64) return fail(DSA_ERR_UNSUPPORTED, "%s: Hi=%d (supported: 32, 64)", who, Hi);
      TRY(check_ptr(q_e4m3, 16, who, "q_e4m3"));
      TRY(check_ptr(w, 4, who, "w"));
      TRY(check_cache(keys_c, Lc_max, who, "compressed keys"));
    }
    TRY(check_ptr(idx_out, 4, who, "idx_out"));
    TRY(check_cache(latent_c, Lc_max, who, "compressed latent"));
  }
  if (window > 0) TRY(check_cache(latent, batch->L_max, who, "latent"));
  TRY(check_ws(ws, ws_bytes, dsa::csa_workspace_bytes(batch->B, batch->Q, batch->L_max, H, ratio, k, window), who));
  g_last_error.clear();
  const dsa::HostCache none{nullptr, nullptr, 0, 0};
  return launched(dsa::launch_csa(host_batch(batch), q_e4m3, w, Hi, (k > 0 && k < Lc_max) ? host_cache(keys_c) : none,
                                  k > 0 ? host_cache(latent_c) : none, window > 0 ? host_cache(latent) : none, ratio,
                                  k, window, q_bf16, H, softmax_scale, out, lse, idx_out, ws, (hipStream_t)stream),
                  who);
}

dsa_status dsa_hisparse_swap_in(int32_t B, const int32_t* idx, int32_t n_sets, int k, int32_t step,
                                const dsa_hot_buffer_t* hb, const void* host_pool, void* device_pool,
                                int32_t* copied, void* ws, size_t ws_bytes, void* stream) {
  const char* who = "dsa_hisparse_swap_in";
  if (B < 1 || n_sets < 1) return fail(DSA_ERR_INVALID_ARG, "%s: B=%d n_sets=%d must be >= 1", who, B, n_sets);
  if (k < 1 || k > kMaxTopK) return fail(DSA_ERR_UNSUPPORTED, "%s: k=%d outside [1, %d]", who, k, kMaxTopK);
  if (step < 0) return fail(DSA_ERR_INVALID_ARG, "%s: step=%d must be >= 0", who, step);
  if (!hb) return fail(DSA_ERR_INVALID_ARG, "%s: hot buffer is NULL", who);
  TRY(check_ptr(idx, 4, who, "idx"));
  TRY(check_ptr(hb->block_table, 4, who, "block_table"));
  TRY(check_ptr(hb->slot_page, 4, who, "slot_page"));
  TRY(check_ptr(hb->slot_clock, 4, who, "slot_clock"));
  TRY(check_ptr(hb->page_clock, 4, who, "page_clock"));
  if (hb->page_size < 16 || hb->page_size % 16)
    return fail(DSA_ERR_UNSUPPORTED, "%s: page_size=%d must be a positive multiple of 16", who, hb->page_size);
  if (hb->row_bytes != 2 * 576 && hb->row_bytes != 576)
    return fail(DSA_ERR_UNSUPPORTED, "%s: row_bytes=%d (supported: 1152, 576)", who, hb->row_bytes);
  if (hb->max_pages < 1 || hb->n_slots < 1)
    return fail(DSA_ERR_INVALID_ARG, "%s: max_pages=%d n_slots=%d must be >= 1", who, hb->max_pages, hb->n_slots);
  if ((int64_t)n_sets * k > hb->n_slots)
    return fail(DSA_ERR_UNSUPPORTED, "%s: a step selects up to n_sets*k=%lld pages, more than n_slots=%d", who,
                (long long)n_sets * k, hb->n_slots);
  if ((int64_t)B * hb->n_slots >= (1LL << 31) || (int64_t)B * n_sets * k >= (1LL << 31) ||
      (int64_t)hb->max_pages * hb->page_size > (1 << 24))
    return fail(DSA_ERR_UNSUPPORTED, "%s: sizes beyond the int32 page and position ranges", who);
  TRY(check_ptr(device_pool, 16, who, "device_pool"));
  TRY(check_ptr(host_pool, 16, who, "host_pool"));
  if (copied && !aligned(copied, 4)) return fail(DSA_ERR_INVALID_ARG, "%s: copied misaligned", who);
  TRY(check_ws(ws, ws_bytes, dsa::hisparse_workspace_bytes(B, n_sets * k), who));
  // The copy kernel reads host_pool in place: it must be memory the device can address.
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_pool) != hipSuccess) {
    (void)hipGetLastError();
    return fail(DSA_ERR_INVALID_ARG, "%s: host_pool is neither pinned host memory nor device memory", who);
  }
  const void* pool_dev = nullptr;
  if (attr.type == hipMemoryTypeHost && attr.devicePointer && attr.hostPointer)
    pool_dev = (const char*)attr.devicePointer + ((const char*)host_pool - (const char*)attr.hostPointer);
  else if (attr.type == hipMemoryTypeDevice)
    pool_dev = host_pool;
  if (!pool_dev)
    return fail(DSA_ERR_INVALID_ARG, "%s: host_pool is neither pinned, device-mapped host memory nor device memory", who);
  g_last_error.clear();
  const dsa::HostHotBuffer h{hb->block_table, hb->slot_page, hb->slot_clock, hb->page_clock,
                             hb->max_pages, hb->n_slots, hb->page_size, hb->row_bytes};
  return launched(dsa::launch_hisparse_swap_in(B, idx, n_sets, k, step, h, pool_dev, device_pool, copied, ws,
                                               (hipStream_t)stream),
                  who);
}

}  // extern "C"
