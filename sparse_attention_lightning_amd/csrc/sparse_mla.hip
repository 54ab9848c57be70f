// Sparse MLA in MQA mode ("LLM architecture survey", section 2.1 DeepSeek-V3: one cached
// latent row per token, 512 latent dims + 64 RoPE dims, 128 query heads; section 2.2
// DeepSeek-V3.2: DSA runs on MLA's MQA mode and only the k selected tokens take the full
// attention path). Every head of a query attends the same gathered rows:
//   z_i = scale * q_h . c_i (576 dims), o_h = sum_i softmax(z)_i c_i[0:512], lse_h = log sum exp z.
//
// One workgroup = one query token x 64 heads (4 waves x 16 heads) x one split of the selected
// tokens. Per step of 32 tokens the workgroup gathers the 32 rows (1152 B each, through the
// index list and the block table) into a token-major LDS tile, then each wave runs
//   S^T[32 tok x 16 heads] = K_tile . Q^T      (bf16 16x16x32 matrix cores, K = 576)
// with its 16 query heads held in registers as the B operand. S^T's accumulator layout
// (lane = head, 4 tokens per register) is exactly the A-operand layout that P needs for
//   O[16 heads x 512] += P . V                 (bf16 16x16x32 matrix cores, K = 32 tokens)
// once the K order of V matches: V's B operand is read straight from the same token-major
// tile with the LDS transpose read (ds_read_b64_tr_b16), tokens permuted to P's order.
// The online softmax runs in the log2 domain in fp32; P is rounded to bf16 for PV.
// With several splits, each workgroup writes its normalised partial (o_s, lse_s) and a
// combine kernel merges them: lse = log sum_s exp lse_s, o = sum_s exp(lse_s - lse) o_s.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kMlaThreads = 256;
constexpr int kHeadsPerWg = 64;
constexpr int kTok = 32;                       // tokens per step
constexpr int kRowBytes = kDqk * 2;            // 1152
constexpr int kPitch = kRowBytes + 16;         // padded LDS row: 16 consecutive rows hit distinct banks
constexpr int kRowChunks = kRowBytes / 16;     // 72 16-byte chunks per row
constexpr int kStepChunks = kTok * kRowChunks; // 2304
constexpr int kChunksPerThread = kStepChunks / kMlaThreads;  // 9
static_assert(kStepChunks % kMlaThreads == 0, "even gather split");
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#ifndef DSA_MLA_TARGET_WGS
#define DSA_MLA_TARGET_WGS 256
#endif
#ifndef DSA_MLA_MIN_SPLIT
#define DSA_MLA_MIN_SPLIT 128
#endif

int sparse_mla_splits(int rows, int H, int k) {
  const int wgs = rows * (H / kHeadsPerWg);
  int s = 1;
  // aim for enough workgroups to fill the chip while each split keeps a minimum of tokens
  while (wgs * s < DSA_MLA_TARGET_WGS && (k + 2 * s - 1) / (2 * s) >= DSA_MLA_MIN_SPLIT && s < 16) s *= 2;
  return s;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t sparse_mla_workspace_bytes(int rows, int H, int k) {
  const int s = sparse_mla_splits(rows, H, k);
  if (s == 1) return 0;
  return align256((size_t)rows * s * H * kDv * sizeof(float)) + align256((size_t)rows * s * H * sizeof(float));
}

__device__ __forceinline__ v8bf load_v8bf(const void* p) { return *(const v8bf*)p; }

__device__ __forceinline__ v4bf lds_tr_read(const uint8_t* lds_byte_ptr) {
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(lds_byte_ptr));
}

template <bool SPLIT>
__global__ __launch_bounds__(kMlaThreads) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, CacheView lat, const int32_t* __restrict__ idx, int k, int idx_q_stride,
    int Q, int H, int splits, int split_len, float scale_log2,
    float* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ part_o, float* __restrict__ part_lse) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTok * kPitch];
  __shared__ int vflag[kTok];
  __shared__ int rowid[kMaxK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int hgroups = H / kHeadsPerWg;
  int item = blockIdx.x;
  const int split = item % splits; item /= splits;
  const int hg = item % hgroups;
  const int bq = item / hgroups;
  const int b = bq / Q, j = bq - b * Q;
  const int h0 = hg * kHeadsPerWg + wave * 16;          // this wave's first head

  const int32_t* irow = idx + (int64_t)b * (idx_q_stride ? (int64_t)Q * k : k) + (int64_t)j * idx_q_stride;
  const int tok_begin = split * split_len;
  const int tok_end = min(k, tok_begin + split_len);

  // query heads h0 + (l % 16) as the B operand of S^T = K . Q^T: 8 dims per lane per K step
  v8bf qb[kDqk / 32];
  const uint16_t* qrow = q + ((int64_t)bq * H + h0 + c16) * kDqk;
#pragma unroll
  for (int s = 0; s < kDqk / 32; ++s) qb[s] = load_v8bf(qrow + 32 * s + 8 * g);

  v4f o[kDv / 16];
#pragma unroll
  for (int nt = 0; nt < kDv / 16; ++nt) o[nt] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max (log2 domain) of head c16
  float l_run = 0.f;         // this lane's share of the softmax denominator

  // Row index (into the cache's rows) of every token of this split, resolved once through the
  // index list and the block table; -1 for masked tokens (index -1 or past k).
  for (int i = tid; i < tok_end - tok_begin; i += kMlaThreads) {
    const int pos = irow[tok_begin + i];
    int r = -1;
    if (pos >= 0)
      r = lat.table ? lat.table[(int64_t)b * lat.max_pages + pos / lat.page_size] * lat.page_size + pos % lat.page_size
                    : b * lat.L_max + pos;
    rowid[i] = r;
  }
  __syncthreads();
  // Gather: 8 threads per row (32 rows per step), thread (row tid/8, part) loads the 16-byte
  // chunks part + 8i, i < 9, of its row; rows are loaded one step before they are used.
  // Masked rows read a valid dummy row and are zeroed in LDS.
  const int grow = tid >> 3, gpart = tid & 7;
  auto row_of = [&](int tok0) -> int {
    const int i = tok0 - tok_begin + grow;
    return (tok0 + grow < tok_end) ? rowid[i] : -1;
  };
  v4i stage[kChunksPerThread];
  auto load_rows = [&](int r) {
    const uint8_t* src = lat.base + (r >= 0 ? (int64_t)r * kRowBytes : 0);
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) stage[i] = *(const v4i*)(src + 16 * (gpart + 8 * i));
  };
  int r_cur = row_of(tok_begin);
  load_rows(r_cur);
  for (int tok0 = tok_begin; tok0 < tok_end; tok0 += kTok) {
    __syncthreads();                           // previous step done with the tile
    const bool row_ok = r_cur >= 0;
    uint8_t* dst = tile + grow * kPitch + 16 * gpart;
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i)
      *(v4i*)(dst + 128 * i) = row_ok ? stage[i] : (v4i){0, 0, 0, 0};
    if (gpart == 0) vflag[grow] = row_ok;
    __syncthreads();
    if (tok0 + kTok < tok_end) {               // block-uniform
      r_cur = row_of(tok0 + kTok);
      load_rows(r_cur);
    }

    // ---- S^T = K_tile . Q^T : two 16-token tiles
    // four independent accumulator chains (2 token tiles x 2 halves of K) keep the matrix
    // pipe busy with one wave per SIMD
    v4f sacc[2], sacc2[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) sacc[mt] = sacc2[mt] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kDqk / 64; ++s)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const uint8_t* arow = tile + (16 * mt + c16) * kPitch + 16 * g;
        sacc[mt] = mfma_bf16(load_v8bf(arow + 64 * s), qb[s], sacc[mt]);
        sacc2[mt] = mfma_bf16(load_v8bf(arow + 64 * (s + kDqk / 64)), qb[s + kDqk / 64], sacc2[mt]);
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) sacc[mt] += sacc2[mt];
    // ---- online softmax for head c16 over tokens 16mt + 4g + r
    float z[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = vflag[16 * mt + 4 * g + r];
        z[mt][r] = ok ? sacc[mt][r] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, z[mt][r]);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float psum = 0.f;
    v8bf pa;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pv = exp2f(z[mt][r] - m_use);
        psum += pv;
        pa[4 * mt + r] = (__bf16)pv;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    // ---- rescale O: this lane's accumulators hold heads 4g + r
    if (__ballot(alpha != 1.f) != 0ull) {      // wave-uniform: skip when no head's max moved
      float al[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
      for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[nt][r] *= al[r];
    }
    // ---- O += P . V, V^T fragments by transpose reads: tokens 4g+e (e<4), 16+4g+(e-4) (e>=4)
    const uint8_t* v0 = tile + (4 * g + (c16 >> 2)) * kPitch + 8 * (c16 & 3);
    const uint8_t* v1 = v0 + 16 * kPitch;
#pragma unroll
    for (int nt = 0; nt < kDv / 16; ++nt) {
      const v4bf lo = lds_tr_read(v0 + 32 * nt);
      const v4bf hi = lds_tr_read(v1 + 32 * nt);
      const v8bf vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[nt] = mfma_bf16(pa, vb, o[nt]);
    }
  }

  // ---- finish: denominator of head c16, then per accumulator head 4g + r
  float l_tot = l_run + shfl_xor(l_run, 16);
  l_tot += shfl_xor(l_tot, 32);
  const float lse_h = (l_tot > 0.f) ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __shfl(l_tot, 4 * g + r, 64);
    inv[r] = lr > 0.f ? 1.f / lr : 0.f;
  }
  float* obase;
  if (SPLIT) {
    const int64_t ps = (int64_t)bq * splits + split;
    obase = part_o + (ps * H + h0) * kDv;
    if (g == 0) part_lse[ps * H + h0 + c16] = lse_h;
  } else {
    obase = out + ((int64_t)bq * H + h0) * kDv;
    if (g == 0 && lse_out) lse_out[(int64_t)bq * H + h0 + c16] = lse_h;
  }
#pragma unroll
  for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) obase[(4 * g + r) * kDv + 16 * nt + c16] = o[nt][r] * inv[r];
}

// Merge split partials: one workgroup per (query token, 2 heads), 128 threads x 4 dims per head.
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ part_o,
                                                          const float* __restrict__ part_lse, int H, int splits,
                                                          float* __restrict__ out, float* __restrict__ lse_out) {
  const int hl = threadIdx.x >> 7, t = threadIdx.x & 127;
  const int bq = blockIdx.x / (H / 2);
  const int h = (blockIdx.x - bq * (H / 2)) * 2 + hl;
  float mx = -INFINITY;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, part_lse[((int64_t)bq * splits + s) * H + h]);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const int64_t ps = (int64_t)bq * splits + s;
      const float wgt = expf(part_lse[ps * H + h] - mx);
      den += wgt;
      const v4f v = *(const v4f*)(part_o + (ps * H + h) * kDv + 4 * t);
      acc += wgt * v;
    }
    acc *= 1.f / den;
  }
  *(v4f*)(out + ((int64_t)bq * H + h) * kDv + 4 * t) = acc;
  if (t == 0 && lse_out) lse_out[(int64_t)bq * H + h] = (mx == -INFINITY) ? -INFINITY : mx + logf(den);
}

hipError_t launch_sparse_mla(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                             const int32_t* idx, int k, int idx_q_stride, float scale, float* out, float* lse,
                             void* ws, hipStream_t s) {
  CacheView lv{(const uint8_t*)latent.base, latent.table, latent.max_pages, latent.page_size, kRowBytes, bt.L_max};
  const int rows = bt.B * bt.Q;
  const int splits = sparse_mla_splits(rows, H, k);
  int split_len = (k + splits - 1) / splits;
  split_len = (split_len + kTok - 1) / kTok * kTok;
  const dim3 grid((unsigned)rows * (H / kHeadsPerWg) * splits), block(kMlaThreads);
  const float sl2 = scale * kLog2e;
  if (splits == 1) {
    hipLaunchKernelGGL(sparse_mla_kernel<false>, grid, block, 0, s, q, lv, idx, k, idx_q_stride, bt.Q, H, 1,
                       split_len, sl2, out, lse, nullptr, nullptr);
    return hipGetLastError();
  }
  float* part_o = (float*)ws;
  float* part_lse = (float*)((char*)ws + align256((size_t)rows * splits * H * kDv * sizeof(float)));
  hipLaunchKernelGGL(sparse_mla_kernel<true>, grid, block, 0, s, q, lv, idx, k, idx_q_stride, bt.Q, H, splits,
                     split_len, sl2, nullptr, nullptr, part_o, part_lse);
  hipLaunchKernelGGL(mla_combine_kernel, dim3((unsigned)rows * (H / 2)), dim3(256), 0, s, part_o, part_lse, H,
                     splits, out, lse);
  return hipGetLastError();
}

}  // namespace dsa
