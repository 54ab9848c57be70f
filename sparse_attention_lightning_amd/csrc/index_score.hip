// Lightning indexer ("LLM architecture survey", section 2.2 DeepSeek-V3.2): for a query token
// at position p, s_t = sum_h w_h * ReLU(q_h . k_t) for every t <= p; -inf after p.
//
// Decode form: one workgroup row per query token, the key range split across workgroups and
// waves. The contraction runs on the 16x16x128 FP8 matrix cores with the query's heads as the
// rows of A (held in registers for the whole scan) and 16 keys as the columns of B (streamed
// from HBM, 32 contiguous bytes per lane). The accumulator then holds 4 heads x 1 key per
// lane, so ReLU and the weighted head sum are in-register FMAs followed by a 3-shuffle
// reduce-scatter across the four 16-lane groups, which leaves lane l with the score of key
// t + l: one coalesced 256-byte store per 64 keys.
#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

#ifndef DSA_SCORE_CHUNK
#define DSA_SCORE_CHUNK 1024
#endif
#ifndef DSA_SCORE_PIPE
#define DSA_SCORE_PIPE 0
#endif
constexpr int kScoreChunk = DSA_SCORE_CHUNK;   // keys per workgroup (4 waves)
constexpr int kScoreWaveKeys = kScoreChunk / 4;
static_assert(kScoreWaveKeys / 16 + 1 <= 64, "a wave's pages fit in one register across lanes");

// XCD-aware work index: consecutive workgroup ids are dispatched round-robin over the 8 XCDs;
// remap so that each XCD walks a contiguous range of work items (items sharing keys share L2).
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int per = n >> 3;
  if ((n & 7) != 0 || per == 0) return id;
  return (id & 7) * per + (id >> 3);
}

template <int HI>
__global__ __launch_bounds__(256) void index_score_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, CacheView keys,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int n_chunks, int n_items, float* __restrict__ scores) {
  constexpr int MT = HI / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // work item = (b, chunk, j) with j fastest, so the Q queries reading the same keys run together
  const int item = xcd_remap(blockIdx.x, n_items);
  const int j = item % Q;
  const int rest = item / Q;
  const int chunk = rest % n_chunks;
  const int b = rest / n_chunks;
  const int bq = b * Q + j;          // score row
  const int bqi = b * in_Q + j;      // q / w row
  const int L_max = keys.L_max;
  int p = query_pos(seq_lens, q_pos, in_Q, b, j);
  p = min(p, L_max - 1);

  const int t_begin = chunk * kScoreChunk + wave * kScoreWaveKeys;
  const int t_end = min(t_begin + kScoreWaveKeys, L_max);
  float* srow = scores + (int64_t)bq * L_max;
  if (t_begin >= t_end) return;

  if (t_begin > p) {  // nothing visible in this wave's range
    for (int t = t_begin + lane; t < t_end; t += kWave) srow[t] = -INFINITY;
    return;
  }

  // Byte order along K shared by both operands: lane group g holds bytes [16g, 16g+16) and
  // [64+16g, 64+16g+16) of a 128-byte row, so each 16-byte load instruction of a wave covers
  // 16 whole 64-byte segments.
  // query operand: A rows = heads 16m + (l % 16)
  v8i qa[MT];
  const uint8_t* qrow = q + (int64_t)bqi * HI * kDi;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const uint8_t* hp = qrow + (16 * m + c16) * kDi;
    const v4i lo4 = *(const v4i*)(hp + 16 * g), hi4 = *(const v4i*)(hp + 64 + 16 * g);
    qa[m] = (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
  }
  // weights of the heads this lane's accumulators hold: head 16m + 4g + r
  float wr[MT][4];
  const float* wrow = w + (int64_t)bqi * HI;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[m][r] = wrow[16 * m + 4 * g + r];

  // Page ids of this wave's key range, one per lane, resolved once: the key loads then never
  // wait on a block-table load. Group t's page is read back with a wave-uniform readlane.
  const bool paged = keys.table != nullptr;
  int page0 = 0, my_page = 0;
  if (paged) {
    page0 = t_begin / keys.page_size;
    const int pg = page0 + lane;
    const int last = min(t_end - 1, p) / keys.page_size;
    if (pg <= last) my_page = keys.table[(int64_t)b * keys.max_pages + pg];
  }
  auto group_row = [&](int t16) -> const uint8_t* {   // row of key t16 (a multiple of 16)
    if (!paged) return keys.base + ((int64_t)b * L_max + t16) * kDi;
    const int page = __builtin_amdgcn_readlane(my_page, t16 / keys.page_size - page0);
    return keys.base + ((int64_t)page * keys.page_size + (t16 % keys.page_size)) * kDi;
  };
  // keys t .. t+63 as four B operands (16 keys each); keys after p are not read
  auto load_keys = [&](int t, v4i (&kb)[4][2]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int tk = t + 16 * c + c16;     // this lane's key (B column)
      if (t + 16 * c <= p && t + 16 * c < t_end) {
        const uint8_t* rowp = group_row(t + 16 * c) + (int64_t)c16 * kDi;  // 16 keys share a page
        kb[c][0] = tk <= p ? *(const v4i*)(rowp + 16 * g) : (v4i){0, 0, 0, 0};
        kb[c][1] = tk <= p ? *(const v4i*)(rowp + 64 + 16 * g) : (v4i){0, 0, 0, 0};
      } else {
        kb[c][0] = (v4i){0, 0, 0, 0};
        kb[c][1] = (v4i){0, 0, 0, 0};
      }
    }
  };
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  auto score_keys = [&](int t, const v4i (&kb)[4][2]) {
    if (t >= t_end) return;
    float part[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const v8i bk = {kb[c][0][0], kb[c][0][1], kb[c][0][2], kb[c][0][3],
                      kb[c][1][0], kb[c][1][1], kb[c][1][2], kb[c][1][3]};
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const v4f acc = mfma_fp8(qa[m], bk, zero);
#pragma unroll
        for (int r = 0; r < 4; ++r) s += wr[m][r] * fmaxf(acc[r], 0.f);
      }
      part[c] = s;
    }
    // reduce-scatter over the 4 lane groups: group g ends with the full score of key group c = g
    const bool lo = g < 2;
    const float r0 = shfl_xor(lo ? part[2] : part[0], 32);
    const float r1 = shfl_xor(lo ? part[3] : part[1], 32);
    const float x0 = (lo ? part[0] : part[2]) + r0;
    const float x1 = (lo ? part[1] : part[3]) + r1;
    const bool odd = g & 1;
    const float r2 = shfl_xor(odd ? x0 : x1, 16);
    const float v = (odd ? x1 : x0) + r2;
    const int tk = t + lane;
    if (tk < t_end) srow[tk] = (tk <= p) ? v : -INFINITY;
  };

#if DSA_SCORE_PIPE
  // two-stage pipeline: the next 64 keys are in flight while the current 64 are scored
  v4i ka[4][2], kb2[4][2];
  load_keys(t_begin, ka);
  for (int t = t_begin; t < t_end; t += 128) {
    load_keys(t + 64, kb2);
    score_keys(t, ka);
    load_keys(t + 128, ka);
    score_keys(t + 64, kb2);
  }
#else
  for (int t = t_begin; t < t_end; t += 64) {
    v4i ka[4][2];
    load_keys(t, ka);
    score_keys(t, ka);
  }
#endif
}

hipError_t launch_index_score(const HostBatch& bt, const uint8_t* q, const float* w, int Hi,
                              const HostCache& keys, float* scores, hipStream_t s) {
  CacheView kv{(const uint8_t*)keys.base, keys.table, keys.max_pages, keys.page_size, kDi, bt.L_max};
  const int n_chunks = (bt.L_max + kScoreChunk - 1) / kScoreChunk;
  const int n_items = bt.B * bt.Q * n_chunks;
  dim3 grid(n_items), block(256);
  if (Hi == 64)
    hipLaunchKernelGGL(index_score_decode_kernel<64>, grid, block, 0, s, q, w, kv, bt.seq_lens, bt.q_pos,
                       bt.Q, bt.in_Q, n_chunks, n_items, scores);
  else
    hipLaunchKernelGGL(index_score_decode_kernel<32>, grid, block, 0, s, q, w, kv, bt.seq_lens, bt.q_pos,
                       bt.Q, bt.in_Q, n_chunks, n_items, scores);
  return hipGetLastError();
}

}  // namespace dsa
