/*
 * dsa.h -- C ABI of the DeepSeek Sparse Attention (DSA) hot path on AMD MI355X (gfx950).
 *
 * The path has three stages and one reuse scheme ("LLM architecture survey" page,
 * section 2.2 DeepSeek-V3.2, and section 7.2 GLM-5.2 with Fig. 7-2):
 *   1. lightning indexer: a score for every preceding token, s_t = sum_h w_h * ReLU(q_h . k_t),
 *      Hi heads of dim 128 in FP8                                   -> dsa_index_score
 *   2. token selector: the k (= 2048) highest-scoring tokens per query -> dsa_topk
 *   3. MLA in MQA mode over only the selected latent rows (512 latent + 64 RoPE dims)
 *                                                                     -> dsa_sparse_mla_fwd
 *   4. IndexShare: one index set serves a group of consecutive layers, or all draft
 *      positions of a speculative step ("GLM-5.2 inference deployment" page, MTP
 *      draft + verify: indices computed at draft step 1 only)      -> dsa_forward_shared
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless marked (host). Every call is asynchronous on
 *     `stream` (a hipStream_t; NULL is the default stream) and launches no host sync.
 *   - The caller owns every buffer. The library never allocates, frees, or keeps a pointer
 *     after the call returns; scratch memory comes from the caller-provided workspace, sized
 *     by dsa_workspace_size().
 *   - Arguments are validated on the host before anything is launched; a failed check
 *     returns a status and launches nothing. Device-side contents (seq_lens, q_pos, block
 *     tables, indices) are trusted, not checked: 1 <= seq_lens[b] <= L_max,
 *     0 <= q_pos < seq_lens[b], page ids inside the pool for every page below seq_lens[b].
 *   - Results are bitwise reproducible run to run (fixed reduction orders, no float
 *     atomics). The library holds no global mutable state and is thread-safe; calls that
 *     share a workspace must not overlap in time.
 *   - Dtypes: "e4m3" = OCP FP8 E4M3FN codes in uint8 (torch.float8_e4m3fn); "bf16" =
 *     bfloat16 bits in uint16 (torch.bfloat16); float = IEEE binary32.
 *   - Fixed dims: indexer head dim 128; latent row 576 (512 latent + 64 RoPE) bf16; value
 *     = the first 512 dims of the row.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or stride            */
  DSA_ERR_UNSUPPORTED = 2,  /* a shape outside what the kernels are built for          */
  DSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than dsa_workspace_size()  */
  DSA_ERR_HIP = 4           /* a HIP launch error; text in dsa_last_error()            */
} dsa_status;

/* A token-major cache of one kind of row (indexer keys: 128 e4m3 bytes per token;
 * latent rows: 576 bf16 per token).
 *   contiguous (block_table == NULL): base is [B][L_max][D]; token t of sequence b is row b*L_max + t.
 *   paged: base is a pool [n_pages][page_size][D]; token t of sequence b is at
 *          page block_table[b*max_pages + t/page_size], row t % page_size.
 * The KV page / slot unit follows the GLM-5.2 inference page (HiSparse section: slot = KV page). */
typedef struct {
  const void* base;            /* device, 16-byte aligned                                   */
  const int32_t* block_table;  /* device [B][max_pages] physical page ids, or NULL            */
  int32_t max_pages;           /* row stride of block_table (>= ceil(L_max / page_size))      */
  int32_t page_size;           /* tokens per page, a positive multiple of 16 (paged only)     */
} dsa_cache_t;

/* A batch of B sequences with Q query tokens each. Query token j of sequence b sits at
 * position q_pos[b*Q + j], or at seq_lens[b] - Q + j when q_pos is NULL (the Q newest
 * cache entries). Causality is inclusive: the query at position p sees tokens 0..p.
 * Limits (DSA_ERR_UNSUPPORTED beyond them): B*Q <= 2^24 and L_max <= 2^24; a call that
 * writes or reads a score matrix (dsa_index_score, dsa_topk, dsa_forward_shared*,
 * dsa_csa_forward) also needs B*Q*L_max <= 2^36, i.e. at most 256 GiB of fp32 scores. */
typedef struct {
  int32_t B, Q, L_max;         /* (host) sizes; L_max is the row stride of scores and caches  */
  const int32_t* seq_lens;     /* device [B]                                                  */
  const int32_t* q_pos;        /* device [B][Q] or NULL                                       */
} dsa_batch_t;

/* Lightning indexer ("LLM architecture survey", section 2.2: 64 heads x 128, FP8, a scalar
 * relevance score for every preceding token; section 7.2: GLM-5.2 uses 32 heads).
 *   q       [B][Q][Hi][128] e4m3      w [B][Q][Hi] float (per query token, per head)
 *   keys    cache of 128-byte e4m3 rows
 *   scores  [B][Q][L_max] float, written in full: s_t for t <= p, -inf for t > p.
 * Hi must be 32 or 64. The dot products run on FP8 matrix cores with fp32 accumulation;
 * the head sum is fp32. Needs no workspace. */
dsa_status dsa_index_score(const dsa_batch_t* batch, const uint8_t* q, const float* w, int Hi,
                           const dsa_cache_t* keys, float* scores, void* stream);

/* Token selector ("LLM architecture survey", section 2.2: each query keeps the k = 2048
 * highest-scoring history tokens).
 *   scores  [B][Q][L_max] float; only entries 0..p of each row are read.
 *   idx     [B][Q][k] int32: the positions of the min(k, p+1) highest scores, ascending,
 *           then -1 up to k. Equal scores go to the lower position; -0 equals +0; NaN is
 *           not allowed in scores 0..p.
 * 1 <= k <= 2048. ws: dsa_workspace_size(DSA_OP_TOPK, ...) bytes, 256-byte aligned.
 * Three implementations give identical results; the library picks one by shape (one workgroup
 * per row for rows of at most 32768 scores, of at most 65536 with 128 rows or more, or of at
 * most 262144 with 256 rows or more; a sampled-threshold form for other rows up to 262144 and
 * for calls of longer rows holding 8M scores or more; else a chunked radix form). The environment variable DSA_TOPK_FORM =
 * radix | sampled | row, read at each call, pins one of them (for tests and measurements). */
dsa_status dsa_topk(const dsa_batch_t* batch, const float* scores, int k, int32_t* idx,
                    void* ws, size_t ws_bytes, void* stream);

/* Sparse MLA in MQA mode ("LLM architecture survey", section 2.1: the latent row is kv rank
 * 512 plus a 64-dim RoPE part; section 2.2: DSA runs on MLA's MQA mode and only the selected
 * tokens take the full attention path).
 * For query token (b, j) and head h over the selected rows c_i (entries -1 are skipped):
 *   z_i = softmax_scale * (q_h . c_i) over all 576 dims, o_h = sum_i softmax(z)_i c_i[0:512],
 *   lse_h = log(sum_i exp z_i) (natural log).
 *   q       [B][Q][H][576] bf16          latent  cache of 576-bf16 rows
 *   idx     row (b, j) at idx + b*(idx_q_stride ? Q*k : k) + j*idx_q_stride; idx_q_stride is
 *           k (one set per query token) or 0 (one set per sequence, shared by its Q tokens)
 *   out     [B][Q][H][512] float         lse [B][Q][H] float, or NULL
 * A query whose set has no valid entry gets out = 0 and lse = -inf.
 * H must be 64 or 128; 1 <= k <= 2048; softmax_scale finite and >= 0 (the kernel takes the
 * maximum of the raw logits and scales it, which needs a non-negative scale; a negative or
 * non-finite scale returns DSA_ERR_INVALID_ARG). QK and PV run on bf16 matrix cores with fp32
 * accumulation; softmax weights are rounded to bf16 for PV and the output is normalised by the
 * sum of the rounded weights (lse by the sum of the unrounded ones).
 * ws: dsa_workspace_size(DSA_OP_SPARSE_MLA, ...) bytes (split partials), 256-byte aligned. */
dsa_status dsa_sparse_mla_fwd(const dsa_batch_t* batch, const uint16_t* q, int H,
                              const dsa_cache_t* latent, const int32_t* idx, int k, int idx_q_stride,
                              float softmax_scale, float* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream);

/* Sparse MLA over an FP8 latent cache (the inference page's KV-cache precision option
 * fp8_e4m3; "MLA + KV FP8" compression in its HiSparse section). The pages give no scale
 * convention; here a latent row is 576 OCP E4M3FN codes (576 bytes, half a bf16 row) and one
 * scale serves the whole cache: the value of a code c is latent_scale x e4m3(c).
 * Everything else as dsa_sparse_mla_fwd, which it equals on the decoded values: every E4M3
 * value is exact in bf16, so the products and sums are those of a bf16 cache holding
 * latent_scale x e4m3(c) when latent_scale is a power of two (and differ only by the rounding
 * of that product otherwise). latent_scale must be finite and > 0. The workspace is that of
 * dsa_sparse_mla_fwd. */
dsa_status dsa_sparse_mla_fwd_fp8(const dsa_batch_t* batch, const uint16_t* q, int H,
                                  const dsa_cache_t* latent, float latent_scale, const int32_t* idx, int k,
                                  int idx_q_stride, float softmax_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, void* stream);

/* IndexShare group ("LLM architecture survey", section 7.2 and Fig. 7-2: every 4 sparse
 * layers share one indexer whose top-k indices the following layers reuse; "GLM-5.2
 * inference deployment", MTP draft + verify: draft steps reuse the step-1 indices).
 * Runs dsa_index_score + dsa_topk once, then dsa_sparse_mla_fwd for each of n_layers layers
 * with that layer's query and latent cache and the same indices.
 *   share_first_query = 0: one index set per query token, idx_out [B][Q][k];
 *   share_first_query = 1: the set of query token 0 of each sequence serves all its Q
 *                          tokens, idx_out [B][1][k] (scores computed for token 0 only).
 *   q_bf16, latents, out, lse: (host) arrays of n_layers device pointers / caches; lse may be
 *   NULL or hold NULL entries. Shapes per layer as in dsa_sparse_mla_fwd.
 * ws: dsa_workspace_size(DSA_OP_FORWARD_SHARED, ...) bytes; it holds the scores, so the
 * scores are not returned. */
dsa_status dsa_forward_shared(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                              const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                              const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents,
                              float softmax_scale, float* const* out, float* const* lse,
                              int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* dsa_forward_shared over FP8 latent caches (the inference page's fp8_e4m3 KV-cache option next
 * to IndexShare): latents[l] holds rows of 576 E4M3 codes whose values are latent_scales[l] x
 * e4m3(code), as in dsa_sparse_mla_fwd_fp8; each layer then equals dsa_sparse_mla_fwd_fp8 with
 * that scale, bit for bit. latent_scales: (host) [n_layers], each finite and > 0. Everything
 * else (workspace included) as dsa_forward_shared. */
dsa_status dsa_forward_shared_fp8(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                                  const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                                  const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents,
                                  const float* latent_scales, float softmax_scale, float* const* out,
                                  float* const* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* dsa_forward_shared for callers that cannot allocate device memory: code being captured into a
 * HIP graph, tight serving loops, and harnesses that forbid hipMalloc. Same arguments, results
 * and errors as dsa_forward_shared, without the workspace: the call uses a scratch array that the
 * library holds in device memory, DSA_NOALLOC_SCRATCH_BYTES (128 MiB) on each GPU it runs on,
 * from that GPU's first call until the process ends. It covers, for example, decode at B = 32
 * and 128K tokens (83 MiB), the 8-position verification batch at B = 64 and 32K (96 MiB) and
 * the 4-layer group at B = 8 and 1M tokens (97 MiB). A call whose dsa_workspace_size(
 * DSA_OP_FORWARD_SHARED, ...) exceeds it returns DSA_ERR_UNSUPPORTED and launches nothing.
 * The call itself allocates nothing and calls no allocating routine. Every call on one GPU
 * shares that GPU's scratch: calls that overlap in time on one GPU (on different streams, or from
 * different host threads) race and give undefined results; serialise them. The scratch keeps the
 * last call's contents; no result depends on them. The GPU is the one that owns `stream` (the
 * current device for the NULL stream). */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dsa_status dsa_forward_shared_noalloc(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                                      const dsa_cache_t* keys, int k, int share_first_query, int n_layers,
                                      const uint16_t* const* q_bf16, int H, const dsa_cache_t* latents,
                                      float softmax_scale, float* const* out, float* const* lse,
                                      int32_t* idx_out, void* stream);

/* Compressed sparse attention ("LLM architecture survey", section 2.3 DeepSeek-V4: CSA compresses
 * the KV cache along the sequence by 4, runs DSA's sparse selection over the compressed entries
 * (top-1024 in V4-Pro, top-512 in V4-Flash) and adds a sliding window of the last 128 raw tokens;
 * HCA compresses by 128 and attends densely, which is this call with k >= the visible entries and
 * window 0). The compression is a learned map of the model: the compressed caches are inputs.
 * For query token (b, j) at raw position p:
 *   - compressed entry c summarises raw tokens ratio*c .. ratio*c + ratio - 1 and is visible once
 *     its last raw token is: the first n_c = (p + 1) / ratio entries (none before a block is full);
 *   - lightning-indexer scores of the query (q_e4m3, w, Hi as in dsa_index_score) against those
 *     n_c compressed keys, and the k best of them as in dsa_topk -> idx_out [B][Q][k] (entry ids,
 *     ascending, -1 padded);
 *   - the window: raw tokens max(0, p - window + 1) .. p of the raw latent cache;
 *   - one MQA-mode softmax (as in dsa_sparse_mla_fwd: q_bf16 [B][Q][H][576], softmax_scale) over
 *     the selected compressed latent rows and the window's raw rows together; a raw token in the
 *     window and its compressed block both count. out [B][Q][H][512], lse [B][Q][H] or NULL.
 * Caches: keys_c (128-byte e4m3 rows) and latent_c (576-bf16 rows) hold L_c = ceil(L_max / ratio)
 * rows per sequence (contiguous [B][L_c][D] or paged with their own block table and max_pages >=
 * ceil(L_c / page_size)); latent is the raw latent cache of L_max rows per sequence. Only the
 * window's raw rows are read.
 * 1 <= ratio <= L_max; 0 <= k <= 2048; 0 <= window <= 2048, not both 0. With k = 0 (a sliding
 * window only) q_e4m3, w, keys_c, latent_c and idx_out are not read; with window = 0, latent is not.
 * With k >= L_c every visible entry is selected whatever its score, so the scores are not computed
 * (q_e4m3, w and keys_c are then not read; HCA).
 * ws: dsa_csa_workspace_size(batch, H, ratio, k, window) bytes, 256-byte aligned (0 when the
 * arguments are out of range). */
size_t dsa_csa_workspace_size(const dsa_batch_t* batch, int H, int ratio, int k, int window);
dsa_status dsa_csa_forward(const dsa_batch_t* batch, const uint8_t* q_e4m3, const float* w, int Hi,
                           const dsa_cache_t* keys_c, const dsa_cache_t* latent_c, const dsa_cache_t* latent,
                           int ratio, int k, int window, const uint16_t* q_bf16, int H, float softmax_scale,
                           float* out, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes, void* stream);

/* HiSparse hot buffer ("GLM-5.2 inference deployment" page, HiSparse section: a GPU hot
 * buffer over the KV cache kept whole in pinned host memory, driven by the step's top-K; one
 * slot per KV page; the page gives 4096-6144 device slots and 8-10x that in host memory).
 * Every sequence owns n_slots device slots of one page each; its whole latent cache stays in
 * host memory. State, in device memory owned by the caller and kept across steps (every entry
 * -1 before the first step):
 *   block_table [B][max_pages] int32  physical page b*n_slots + s of each resident logical
 *                                      page, else -1. {device_pool, block_table, max_pages,
 *                                      page_size} is then the latent cache for dsa_sparse_mla_fwd.
 *   slot_page   [B][n_slots]   int32  logical page held by each slot, else -1
 *   slot_clock  [B][n_slots]   int32  last step whose selected set used the slot, else -1
 *   page_clock  [B][max_pages] int32  last step whose selected set held the page, else -1 */
typedef struct {
  int32_t* block_table;
  int32_t* slot_page;
  int32_t* slot_clock;
  int32_t* page_clock;
  int32_t max_pages;           /* (host) logical pages per sequence                          */
  int32_t n_slots;             /* (host) device slots per sequence                           */
  int32_t page_size;           /* (host) tokens per page (= per slot), a positive multiple of 16 */
  int32_t row_bytes;           /* (host) bytes per token row in both pools: 1152 (bf16 latent rows)
                                  or 576 (E4M3 rows, for dsa_sparse_mla_fwd_fp8)               */
} dsa_hot_buffer_t;

/* One swap-in step, after dsa_topk of the step (page's three steps: top-K miss detection, LRU
 * eviction, page-table update with an asynchronous host-to-device pull).
 *   idx          [B][n_sets][k] int32 selected positions as dsa_topk writes them (-1 skipped)
 *   step         >= 0, larger than the step of every earlier call on the same state
 *   host_pool    [B][max_pages][page_size][row_bytes], every page of every sequence: pinned host
 *                memory mapped for the device (hipHostMalloc, torch pin_memory), or device
 *                memory. Checked with hipPointerGetAttributes: DSA_ERR_INVALID_ARG otherwise.
 *   device_pool  [B*n_slots][page_size][row_bytes] device memory
 *   copied       device [B] int32: pages copied for each sequence in this step, or NULL
 * Afterwards every page holding a selected position is resident. Hits refresh their slot's
 * clock. The missing pages evict as many of the slots this step does not use, least recently
 * used first (never-used slots have clock -1; equal clocks: lower slot first); the i-th missing
 * page in ascending page order takes the i-th of those slots in ascending slot order, is copied
 * from host_pool, and the page the slot held leaves block_table.
 * Requires n_sets*k <= n_slots (DSA_ERR_UNSUPPORTED otherwise), so a step's selected set fits.
 * The pages are read from host memory by the copy kernel itself: no host thread waits for the
 * miss list. ws: dsa_workspace_size(DSA_OP_HISPARSE_SWAP_IN, batch with B, Q = n_sets and any
 * L_max >= 1, 0, 0, k, 0) bytes, 256-byte aligned. */
dsa_status dsa_hisparse_swap_in(int32_t B, const int32_t* idx, int32_t n_sets, int k, int32_t step,
                                const dsa_hot_buffer_t* hb, const void* host_pool, void* device_pool,
                                int32_t* copied, void* ws, size_t ws_bytes, void* stream);

/* Workspace sizes, from host fields of `batch` only (B, Q, L_max); 0 for a shape outside the
 * batch limits above (which every entry point rejects). */
enum { DSA_OP_INDEX_SCORE = 0, DSA_OP_TOPK = 1, DSA_OP_SPARSE_MLA = 2, DSA_OP_FORWARD_SHARED = 3,
       DSA_OP_HISPARSE_SWAP_IN = 4 };
size_t dsa_workspace_size(int op, const dsa_batch_t* batch, int Hi, int H, int k, int n_layers);

const char* dsa_status_str(dsa_status s);
/* Thread-local text of the last failure on this thread; valid until the next call. */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
