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
#define DSA_SCORE_CHUNK 2048
#endif
#ifndef DSA_SCORE_PIPE
#define DSA_SCORE_PIPE 0
#endif
#ifndef DSA_SCORE_NT
#define DSA_SCORE_NT 0
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
#if DSA_SCORE_NT
        kb[c][0] = tk <= p ? __builtin_nontemporal_load((const v4i*)(rowp + 16 * g)) : (v4i){0, 0, 0, 0};
        kb[c][1] = tk <= p ? __builtin_nontemporal_load((const v4i*)(rowp + 64 + 16 * g)) : (v4i){0, 0, 0, 0};
#else
        kb[c][0] = tk <= p ? *(const v4i*)(rowp + 16 * g) : (v4i){0, 0, 0, 0};
        kb[c][1] = tk <= p ? *(const v4i*)(rowp + 64 + 16 * g) : (v4i){0, 0, 0, 0};
#endif
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
        for (int r = 0; r < 4; ++r) s += wr[m][r] * relu(acc[r]);
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

// ------------------------------------------------------------------------------------------
// Multi-query form (prefill chunks, speculative verify): the query tokens of one sequence share
// every key, so a workgroup of 8 waves, one query token each, stages each tile of 256 keys once
// in LDS (direct-to-LDS loads into a 2-stage ring, rows XOR-swizzled by 16-byte chunk so the 16
// rows of one matrix-core operand fetch hit distinct banks). Each wave runs its 64 heads x 16
// keys per group through 4 FP8 matrix-core products, pipelined with the ReLU / weighted head
// sum of the previous group, and a 3-swap reduce-scatter leaves one key per lane for a
// coalesced store per 64 keys. Keys after the last query's position are neither loaded nor
// scored; scores after each query's own position are -inf.
//
// The kernel is bound by VALU issue: the epilogue costs 2 VALU operations per head x key (an
// integer max for the ReLU, a multiply-add), 8 per matrix-core product of 32 cycles, so every
// other VALU instruction comes straight out of the matrix-core rate. Tile loads therefore take
// wave-uniform (scalar) addresses and the reduce-scatter uses lane-swap instructions.
#ifndef DSA_MQ_TILE
#define DSA_MQ_TILE 256
#endif
#ifndef DSA_MQ_STAGES
#define DSA_MQ_STAGES 2
#endif
#ifndef DSA_MQ_CHUNK
#define DSA_MQ_CHUNK 4096
#endif
#ifndef DSA_MQ_SCHED
#define DSA_MQ_SCHED 0
#endif
constexpr int kMqTile = DSA_MQ_TILE;                 // keys per LDS tile
constexpr int kMqStages = DSA_MQ_STAGES;
constexpr int kMqChunk = DSA_MQ_CHUNK;               // keys per workgroup
constexpr int kMqDma = kMqTile / 8;                  // 1 KB direct-to-LDS loads per tile
constexpr int kMqWaves = 8;                          // query tokens per workgroup
static_assert(kMqChunk % kMqTile == 0 && kMqDma % kMqWaves == 0, "tile shape");

template <int VM>
__device__ __forceinline__ void mq_wait() {
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// p[c] holds, in lane 16g + j, the partial sum of lane group g for key j of group c. Returns in
// lane 16c + j the sum over the four lane groups of p[c]. Two half-wave swaps put p[0] (p[1])
// in the low and p[2] (p[3]) in the high half, each summed over g and g ^ 2; one swap of 16-lane
// rows then pairs g with g ^ 1.
__device__ __forceinline__ float reduce_scatter4(const float (&p)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
  const float x0 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float x1 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(x0), __float_as_uint(x1), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// How a tile load finds its 8 rows.
enum MqRows { kRowsContiguous = 0, kRowsPaged = 1, kRowsPerLane = 2 };

template <int HI, int ROWS>
__global__ __launch_bounds__(kMqWaves * 64) void index_score_multi_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, CacheView keys,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int n_qgroups, int n_chunks, float* __restrict__ scores) {
  constexpr int MT = HI / 16;
  constexpr int kG = kMqTile / 16;                    // 16-key groups per tile
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kMqStages][kMqTile * kDi];
  __shared__ int pmax_lds;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  // work item = (b, chunk, query group), query group fastest: groups sharing keys run together
  const int item = blockIdx.x;
  const int qg = item % n_qgroups;
  const int rest = item / n_qgroups;
  const int chunk = rest % n_chunks;
  const int b = rest / n_chunks;
  const int L_max = keys.L_max;
  const int t0 = chunk * kMqChunk;
  const int t1 = min(t0 + kMqChunk, L_max);

  const int jq = qg * kMqWaves + wave;
  const bool live = jq < Q;
  const int pq = live ? min(query_pos(seq_lens, q_pos, in_Q, b, jq), L_max - 1) : -1;
  if (threadIdx.x == 0) pmax_lds = -1;
  __syncthreads();
  if (lane == 0) atomicMax(&pmax_lds, pq);
  __syncthreads();
  const int pmax = __builtin_amdgcn_readfirstlane(pmax_lds);   // keys after it are never loaded
  const int t_load_end = min(t1, pmax + 1);
  const int n_tiles = t_load_end > t0 ? (t_load_end - t0 + kMqTile - 1) / kMqTile : 0;
  constexpr int my_dma = kMqDma / kMqWaves;

  // Load d covers rows 8d..8d+7 of the tile: lane l lands in row 8d + l/8, slot l%8, and fetches
  // the 16-byte chunk that the swizzle puts there. The row's swizzle term (row >> 1) & 7 equals
  // (4 (d & 1) + l / 16) & 7, so the lane's offset from the 8-row base is one of two constants
  // and the base is wave-uniform: the 8 rows lie in one page (page sizes are multiples of 16),
  // or inside the sequence when the cache is contiguous and L_max % 8 == 0; otherwise each lane
  // clamps its own row. Groups past the last visible key re-read the group that holds it.
  const uint32_t lane_off0 = (lane >> 3) * 128 + 16 * ((lane & 7) ^ ((lane >> 4) & 7));
  const uint32_t lane_off1 = (lane >> 3) * 128 + 16 * ((lane & 7) ^ ((4 + (lane >> 4)) & 7));
  const int last_group = pmax & ~7;
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)keys.table;     // read-only: scalar loads
  auto issue_tile = [&](int tt) {
    uint8_t* lds = ring[tt % kMqStages];
#pragma unroll
    for (int i = 0; i < my_dma; ++i) {
      const int d = wave + kMqWaves * i;
      const int tr = min(t0 + tt * kMqTile + 8 * d, last_group);
      const uint32_t off = (d & 1) ? lane_off1 : lane_off0;
      const uint8_t* src;
      if constexpr (ROWS == kRowsContiguous) {
        src = keys.base + ((int64_t)b * L_max + tr) * kDi + off;
      } else if constexpr (ROWS == kRowsPaged) {
        const int page = table[(int64_t)b * keys.max_pages + tr / keys.page_size];
        src = keys.base + ((int64_t)page * keys.page_size + tr % keys.page_size) * kDi + off;
      } else {
        const int t = min(tr + (lane >> 3), pmax);
        src = keys.base + ((int64_t)b * L_max + t) * kDi + (off & 127u);
      }
      __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(lds + d * 1024),
                                       16, 0, 0);
    }
  };

  // A operands: rows = heads 16m + c16, lane group g holds bytes [16g,+16) and [64+16g,+16);
  // weights of the heads 16m + 4g + r that the accumulator registers hold.
  v8i qa[MT];
  float wr[MT][4];
  {
    const int jj = live ? jq : 0;
    const uint8_t* qrow = q + ((int64_t)b * in_Q + jj) * HI * kDi;
    const float* wrow = w + ((int64_t)b * in_Q + jj) * HI;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint8_t* hp = qrow + (16 * m + c16) * kDi;
      const v4i lo4 = *(const v4i*)(hp + 16 * g), hi4 = *(const v4i*)(hp + 64 + 16 * g);
      qa[m] = (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[m][r] = wrow[16 * m + 4 * g + r];
    }
  }
  float* srow = scores + ((int64_t)b * Q + (live ? jq : 0)) * L_max;
  // scores of keys in this chunk that no tile covers (after pmax): -inf
  if (live)
    for (int t = max(t0, t_load_end) + lane; t < t1; t += kWave) srow[t] = -INFINITY;

  // prefetch distance: kMqStages - 1 tiles are in flight while one is computed
  constexpr int kAhead = kMqStages - 1;
  static_assert(kAhead >= 1, "at least two stages");
#pragma unroll
  for (int a = 0; a < kAhead; ++a)
    if (a < n_tiles) issue_tile(a);
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // per-lane B fragment offsets in a 16-row group (the swizzle repeats every 16 rows)
  const int b_lo = c16 * 128 + 16 * (g ^ ((c16 >> 1) & 7));
  const int b_hi = c16 * 128 + 16 * ((g + 4) ^ ((c16 >> 1) & 7));
  for (int tt = 0; tt < n_tiles; ++tt) {
    // tile tt has landed once only the later tiles' loads (at most kAhead - 1 tiles) are in flight
    const int later = min(kAhead - 1, n_tiles - 1 - tt) * my_dma;
    switch (later) {
      case 1: mq_wait<1>(); break;
      case 2: mq_wait<2>(); break;
      case 3: mq_wait<3>(); break;
      case 4: mq_wait<4>(); break;
      case 6: mq_wait<6>(); break;
      case 8: mq_wait<8>(); break;
      case 12: mq_wait<12>(); break;
      case 16: mq_wait<16>(); break;
      default: mq_wait<0>(); break;
    }
    __builtin_amdgcn_s_barrier();
    // the slot of tile tt + kAhead was last read in tile tt - 1, which every wave has finished
    if (tt + kAhead < n_tiles) issue_tile(tt + kAhead);
    const uint8_t* tile = ring[tt % kMqStages];
    const int tb = t0 + tt * kMqTile;
    auto frag = [&](int gi) {
      const uint8_t* gp = tile + gi * 16 * 128;
      const v4i lo4 = *(const v4i*)(gp + b_lo), hi4 = *(const v4i*)(gp + b_hi);
      return (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    };
    // Software pipeline over the tile's groups: the products of group gi + 1 share a scheduling
    // region with the epilogue of group gi (issued a full group earlier, so no epilogue
    // instruction waits on a product in flight), and B fragments are read two groups ahead.
    // Keys after pmax inside the last tile are computed on valid rows and stored as -inf.
    v4f acc[2][MT];
    v8i bk_next = frag(1);
    {
      const v8i bk0 = frag(0);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[0][m] = mfma_fp8(qa[m], bk0, zero);
    }
    float part[4];
#pragma unroll
    for (int gi = 0; gi < kG; ++gi) {
      __builtin_amdgcn_sched_barrier(0);
      if (gi + 1 < kG) {
        const v8i bk_after = frag(gi + 2 < kG ? gi + 2 : gi + 1);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[(gi + 1) & 1][m] = mfma_fp8(qa[m], bk_next, zero);
        bk_next = bk_after;
      }
      float sum = 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum += wr[m][r] * relu(acc[gi & 1][m][r]);
      part[gi & 3] = sum;
#if DSA_MQ_SCHED
      if (gi + 2 < kG) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // next-but-one fragment
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // one product
        __builtin_amdgcn_sched_group_barrier(0x002, DSA_MQ_SCHED, 0);         // then VALU
      }
#endif
      if ((gi & 3) == 3) {
        const float v = reduce_scatter4(part);        // lane 16c + j: key j of group c
        const int tk = tb + 64 * (gi >> 2) + lane;
        if (live && tk < t1) srow[tk] = (tk <= pq) ? v : -INFINITY;
      }
    }
  }
}

template <int HI, int ROWS>
static void launch_multi(const HostBatch& bt, const uint8_t* q, const float* w, const CacheView& kv, float* scores,
                         hipStream_t s) {
  const int qgroups = (bt.Q + kMqWaves - 1) / kMqWaves;
  const int n_chunks = (bt.L_max + kMqChunk - 1) / kMqChunk;
  const dim3 grid((unsigned)bt.B * n_chunks * qgroups), block(kMqWaves * 64);
  hipLaunchKernelGGL((index_score_multi_kernel<HI, ROWS>), grid, block, 0, s, q, w, kv, bt.seq_lens, bt.q_pos, bt.Q,
                     bt.in_Q, qgroups, n_chunks, scores);
}

template <int HI>
static void launch_multi_rows(const HostBatch& bt, const uint8_t* q, const float* w, const CacheView& kv,
                              float* scores, hipStream_t s) {
  if (kv.table != nullptr) launch_multi<HI, kRowsPaged>(bt, q, w, kv, scores, s);
  else if (bt.L_max % 8 == 0) launch_multi<HI, kRowsContiguous>(bt, q, w, kv, scores, s);
  else launch_multi<HI, kRowsPerLane>(bt, q, w, kv, scores, s);
}

hipError_t launch_index_score(const HostBatch& bt, const uint8_t* q, const float* w, int Hi,
                              const HostCache& keys, float* scores, hipStream_t s) {
  CacheView kv{(const uint8_t*)keys.base, keys.table, keys.max_pages, keys.page_size, kDi, bt.L_max};
  if (bt.Q >= 2) {
    if (Hi == 64) launch_multi_rows<64>(bt, q, w, kv, scores, s);
    else launch_multi_rows<32>(bt, q, w, kv, scores, s);
    return hipGetLastError();
  }
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
