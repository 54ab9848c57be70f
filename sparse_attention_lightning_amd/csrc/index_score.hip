// Lightning indexer ("LLM architecture survey", section 2.2 DeepSeek-V3.2): for a query token
// at position p, s_t = sum_h w_h * ReLU(q_h . k_t) for every t <= p; -inf after p.
//
// The contraction runs on the 16x16x128 FP8 matrix cores with the query's heads as the rows of
// A (held in registers) and 16 keys as the columns of B. The accumulator then holds 4 heads x
// 1 key per lane, so ReLU and the weighted head sum are in-register multiply-adds, and a 3-swap
// reduce-scatter across the four 16-lane groups leaves lane l with the score of key t + l: one
// coalesced 256-byte store per 64 keys. Keys reach LDS through direct-to-LDS loads of 8 whole
// rows (1 KB, wave-uniform base address) with rows XOR-swizzled by 16-byte chunk, so that the
// rows of one B operand read from LDS hit distinct banks (the LDS serves 16-byte reads eight
// lanes at a time over 32 banks; the swizzle by row & 7 spreads those eight rows).
//
// Two forms: decode (one query token per sequence: each wave streams its own key range through
// a private ring, HBM-bound) and multi-query (prefill chunks, speculative verify: 8 query tokens
// share each key tile, matrix-core / VALU-bound).
#include <type_traits>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kScoreChunk = 2048;              // keys per workgroup of the decode form ...
constexpr int kScoreChunkSmall = 256;          // ... and in a launch that would not fill the chip
constexpr int kChipCUs = 256;                   // compute units of the part
constexpr int kDecWaves = 4;                    // waves per workgroup

// XCD-aware work index: consecutive workgroup ids are dispatched round-robin over the 8 XCDs;
// remap so that each XCD walks a contiguous range of work items (items sharing keys share L2).
__device__ __forceinline__ int xcd_remap(int id, int n) {
  const int per = n >> 3;
  if ((n & 7) != 0 || per == 0) return id;
  return (id & 7) * per + (id >> 3);
}

// ------------------------------------------------------------------------------------------
// Multi-query form (prefill chunks, speculative verify): the query tokens of one sequence share
// every key, so a workgroup of 8 waves, one query token each, stages each tile of 256 keys once
// in LDS (direct-to-LDS loads into a 2-stage ring, rows XOR-swizzled by 16-byte chunk so the
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
constexpr int kMqTile = 256;                         // keys per LDS tile
constexpr int kMqStages = 2;
constexpr int kMqChunk = 4096;                       // keys per workgroup ...
constexpr int kMqChunkLarge = 8192;                  // ... in launches of many rounds (below)
constexpr int kMqAux = 0;                            // cache policy of the tile loads: default
constexpr int kMqDma = kMqTile / 8;                  // 1 KB direct-to-LDS loads per tile
constexpr int kMqWaves = 8;                          // query tokens per workgroup
static_assert(kMqChunk % kMqTile == 0 && kMqChunkLarge % kMqTile == 0 && kMqDma % kMqWaves == 0, "tile shape");

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

template <int HI, int ROWS, int CHUNK>
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
  // work item = (b, chunk, query group), query group fastest: groups sharing keys run together,
  // and on one XCD (each XCD walks a contiguous range of items), so they share its L2
  const int item = xcd_remap(blockIdx.x, (int)gridDim.x);
  const int qg = item % n_qgroups;
  const int rest = item / n_qgroups;
  const int chunk = rest % n_chunks;
  const int b = rest / n_chunks;
  const int L_max = keys.L_max;
  const int t0 = chunk * CHUNK;
  const int t1 = min(t0 + CHUNK, L_max);

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
  // the 16-byte chunk that the swizzle puts there. The row's swizzle term row & 7 equals l / 8,
  // so the lane's offset from the 8-row base is one constant and the base is wave-uniform: the
  // 8 rows lie in one page (page sizes are multiples of 16), or inside the sequence when the
  // cache is contiguous and L_max % 8 == 0; otherwise each lane clamps its own row. Groups past
  // the last visible key re-read the group that holds it.
  const uint32_t lane_off = (lane >> 3) * 128 + 16 * ((lane & 7) ^ (lane >> 3));
  const int last_group = pmax & ~7;
  const __attribute__((address_space(4))) int32_t* table =
      (const __attribute__((address_space(4))) int32_t*)keys.table;     // read-only: scalar loads
  auto issue_tile = [&](int tt) {
    uint8_t* lds = ring[tt % kMqStages];
#pragma unroll
    for (int i = 0; i < my_dma; ++i) {
      const int d = wave + kMqWaves * i;
      const int tr = min(t0 + tt * kMqTile + 8 * d, last_group);
      const uint32_t off = lane_off;
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
                                       16, 0, kMqAux);
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
  // per-lane B fragment offsets in a 16-row group (the swizzle repeats every 8 rows)
  const int b_lo = c16 * 128 + 16 * (g ^ (c16 & 7));
  const int b_hi = c16 * 128 + 16 * ((g + 4) ^ (c16 & 7));
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
    const int tb = t0 + tt * kMqTile;
    // Software pipeline over the tile's groups: the products of group gi + 1 share a scheduling
    // region with the epilogue of group gi (issued a full group earlier, so no epilogue
    // instruction waits on a product in flight), and B fragments are read two groups ahead.
    // Keys after pmax inside the last tile are computed on valid rows and stored as -inf.
    // An interior tile (every key at or before this wave's query and inside the chunk) stores its
    // scores with no bound checks, from a wave-uniform base; the tile's branch is taken once.
    auto run_tile = [&](auto interior_c, auto slot_c) {
      constexpr bool kInterior = decltype(interior_c)::value;
      const uint8_t* tile = ring[decltype(slot_c)::value];
      float* const stile = srow + tb + lane;
      auto frag = [&](int gi) {
        const uint8_t* gp = tile + gi * 16 * 128;
        const v4i lo4 = *(const v4i*)(gp + b_lo), hi4 = *(const v4i*)(gp + b_hi);
        return (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      };
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
        if ((gi & 3) == 3) {
          const float v = reduce_scatter4(part);      // lane 16c + j: key j of group c
          if constexpr (kInterior) {
            stile[64 * (gi >> 2)] = v;
          } else {
            const int tk = tb + 64 * (gi >> 2) + lane;
            if (live && tk < t1) srow[tk] = (tk <= pq) ? v : -INFINITY;
          }
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using Yes = std::true_type;
    using No = std::false_type;
    static_assert(kMqStages == 2, "two ring slots");
    const bool interior = tb + kMqTile - 1 <= pq && tb + kMqTile <= t1;     // wave-uniform
    if (tt & 1) {
      if (interior) run_tile(Yes{}, I1{});
      else run_tile(No{}, I1{});
    } else {
      if (interior) run_tile(Yes{}, I0{});
      else run_tile(No{}, I0{});
    }
  }
}

// A workgroup's key chunk: 8192 keys when the launch still holds 16 or more workgroups per CU at
// that size (the prefill chunk: 8192 workgroups), else 4096. Longer chunks halve the workgroups
// that fill and drain a tile pipeline (prefill scan 1.4% faster, scores identical); in launches
// of a round or two (the verification batch: 512 workgroups at 4096 keys) they leave CUs idle.
template <int HI, int ROWS>
static void launch_multi(const HostBatch& bt, const uint8_t* q, const float* w, const CacheView& kv, float* scores,
                         hipStream_t s) {
  const int qgroups = (bt.Q + kMqWaves - 1) / kMqWaves;
  auto go = [&](auto chunk_c) {
    constexpr int CH = decltype(chunk_c)::value;
    const int n_chunks = (bt.L_max + CH - 1) / CH;
    const dim3 grid((unsigned)bt.B * n_chunks * qgroups), block(kMqWaves * 64);
    hipLaunchKernelGGL((index_score_multi_kernel<HI, ROWS, CH>), grid, block, 0, s, q, w, kv, bt.seq_lens, bt.q_pos,
                       bt.Q, bt.in_Q, qgroups, n_chunks, scores);
  };
  const int64_t wgs_large = (int64_t)bt.B * ((bt.L_max + kMqChunkLarge - 1) / kMqChunkLarge) * qgroups;
  if (wgs_large >= 16 * kChipCUs) go(std::integral_constant<int, kMqChunkLarge>{});
  else go(std::integral_constant<int, kMqChunk>{});
}

template <int HI>
static void launch_multi_rows(const HostBatch& bt, const uint8_t* q, const float* w, const CacheView& kv,
                              float* scores, hipStream_t s) {
  if (kv.table != nullptr) launch_multi<HI, kRowsPaged>(bt, q, w, kv, scores, s);
  else if (bt.L_max % 8 == 0) launch_multi<HI, kRowsContiguous>(bt, q, w, kv, scores, s);
  else launch_multi<HI, kRowsPerLane>(bt, q, w, kv, scores, s);
}

// Decode form: each wave streams its own key range through a private ring of kDecStages tiles
// of 64 keys and waits on its own load counter only, so no workgroup barrier is involved. Two
// stages keep LDS at 64 KB per workgroup, two workgroups per CU; the tile loads are marked
// nontemporal (the keys are read once per step), which measured about 10% faster than cached.
constexpr int kDecStages = 2;
constexpr int kDecAux = 2;                           // cache policy of the tile loads: nontemporal
constexpr int kDecTile = 64;                         // keys per ring slot: one reduce-scatter

template <int VM>
__device__ __forceinline__ void dec_wait() {
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int HI, int ROWS, int CHUNK>
__global__ __launch_bounds__(kDecWaves * 64) void index_score_decode_kernel(
    const uint8_t* __restrict__ q, const float* __restrict__ w, CacheView keys,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ q_pos,
    int Q, int in_Q, int n_chunks, int n_items, float* __restrict__ scores) {
  constexpr int MT = HI / 16;
  constexpr int kWaveKeys = CHUNK / kDecWaves;
  static_assert(kWaveKeys / 16 + 1 <= 64, "a wave's pages fit in one register across lanes");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kDecWaves][kDecStages][kDecTile * kDi];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int j = item % Q;
  const int rest = item / Q;
  const int chunk = rest % n_chunks;
  const int b = rest / n_chunks;
  const int bq = b * Q + j;
  const int bqi = b * in_Q + j;
  const int L_max = keys.L_max;
  const int p = __builtin_amdgcn_readfirstlane(min(query_pos(seq_lens, q_pos, in_Q, b, j), L_max - 1));
  const int t_begin = chunk * CHUNK + wave * kWaveKeys;
  const int t_end = min(t_begin + kWaveKeys, L_max);
  float* srow = scores + (int64_t)bq * L_max;
  if (t_begin >= t_end) return;
  if (t_begin > p) {
    for (int t = t_begin + lane; t < t_end; t += kWave) srow[t] = -INFINITY;
    return;
  }
  const int t_vis = min(t_end, p + 1);                       // keys read: [t_begin, t_vis)
  for (int t = t_vis + lane; t < t_end; t += kWave) srow[t] = -INFINITY;
  const int n_tiles = (t_vis - t_begin + kDecTile - 1) / kDecTile;

  // page ids of the wave's range, one per lane, read back with a wave-uniform readlane
  int page0 = 0, my_page = 0;
  if constexpr (ROWS == kRowsPaged) {
    page0 = t_begin / keys.page_size;
    const int pg = page0 + lane;
    if (pg <= p / keys.page_size && pg * keys.page_size < t_end) my_page = keys.table[(int64_t)b * keys.max_pages + pg];
  }
  const uint32_t lane_off = (lane >> 3) * 128 + 16 * ((lane & 7) ^ (lane >> 3));
  const int last_group = p & ~7;
  auto issue_tile = [&](int tt) {
    uint8_t* lds = ring[wave][tt % kDecStages];
#pragma unroll
    for (int d = 0; d < kDecTile / 8; ++d) {
      const int tr = min(t_begin + tt * kDecTile + 8 * d, last_group);
      const uint32_t off = lane_off;
      const uint8_t* src;
      if constexpr (ROWS == kRowsContiguous) {
        src = keys.base + ((int64_t)b * L_max + tr) * kDi + off;
      } else if constexpr (ROWS == kRowsPaged) {
        const int page = __builtin_amdgcn_readlane(my_page, tr / keys.page_size - page0);
        src = keys.base + ((int64_t)page * keys.page_size + tr % keys.page_size) * kDi + off;
      } else {
        const int t = min(tr + (lane >> 3), p);
        src = keys.base + ((int64_t)b * L_max + t) * kDi + (off & 127u);
      }
      __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(lds + d * 1024),
                                       16, 0, kDecAux);
    }
  };
  v8i qa[MT];
  float wr[MT][4];
  {
    const uint8_t* qrow = q + (int64_t)bqi * HI * kDi;
    const float* wrow = w + (int64_t)bqi * HI;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint8_t* hp = qrow + (16 * m + c16) * kDi;
      const v4i lo4 = *(const v4i*)(hp + 16 * g), hi4 = *(const v4i*)(hp + 64 + 16 * g);
      qa[m] = (v8i){lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
      for (int r = 0; r < 4; ++r) wr[m][r] = wrow[16 * m + 4 * g + r];
    }
  }
  constexpr int kAhead = kDecStages - 1;
#pragma unroll
  for (int a = 0; a < kAhead; ++a)
    if (a < n_tiles) issue_tile(a);

  const int b_lo = c16 * 128 + 16 * (g ^ (c16 & 7));
  const int b_hi = c16 * 128 + 16 * ((g + 4) ^ (c16 & 7));
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  constexpr int my_dma = kDecTile / 8;
  for (int tt = 0; tt < n_tiles; ++tt) {
    // tile tt has landed once only the later tiles' loads are in flight
    const int later = min(kAhead - 1, n_tiles - 1 - tt) * my_dma;
    switch (later) {
      case 4: dec_wait<4>(); break;
      case 8: dec_wait<8>(); break;
      case 12: dec_wait<12>(); break;
      case 16: dec_wait<16>(); break;
      case 24: dec_wait<24>(); break;
      case 32: dec_wait<32>(); break;
      case 40: dec_wait<40>(); break;
      case 48: dec_wait<48>(); break;
      default: dec_wait<0>(); break;
    }
    if (tt + kAhead < n_tiles) issue_tile(tt + kAhead);
    const uint8_t* tile = ring[wave][tt % kDecStages];
    float part[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint8_t* gp = tile + c * 16 * 128;
      const v4i lo4 = *(const v4i*)(gp + b_lo), hi4 = *(const v4i*)(gp + b_hi);
      const v8i bk = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      float sum = 0.f;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const v4f acc = mfma_fp8(qa[m], bk, zero);
#pragma unroll
        for (int r = 0; r < 4; ++r) sum += wr[m][r] * relu(acc[r]);
      }
      part[c] = sum;
    }
    const float v = reduce_scatter4(part);
    const int tk = t_begin + tt * kDecTile + lane;
    if (tk < t_vis) srow[tk] = v;
  }
}

hipError_t launch_index_score(const HostBatch& bt, const uint8_t* q, const float* w, int Hi,
                              const HostCache& keys, float* scores, hipStream_t s) {
  CacheView kv{(const uint8_t*)keys.base, keys.table, keys.max_pages, keys.page_size, kDi, bt.L_max};
  if (bt.Q >= 2) {
    if (Hi == 64) launch_multi_rows<64>(bt, q, w, kv, scores, s);
    else launch_multi_rows<32>(bt, q, w, kv, scores, s);
    return hipGetLastError();
  }
  // Each wave streams its keys one tile after another, so a launch with fewer workgroups than
  // CUs (one short sequence) takes workgroups of 256 keys, one tile per wave: the scan is then
  // one memory round trip per wave instead of eight.
  const bool small = (int64_t)bt.B * bt.Q * ((bt.L_max + kScoreChunk - 1) / kScoreChunk) < kChipCUs;
  auto dec = [&](auto hi, auto chunk_c) {
    constexpr int HI = decltype(hi)::value;
    constexpr int CH = decltype(chunk_c)::value;
    const int n_chunks = (bt.L_max + CH - 1) / CH;
    const int n_items = bt.B * bt.Q * n_chunks;
    const dim3 grid(n_items), block(kDecWaves * 64);
    if (kv.table != nullptr)
      hipLaunchKernelGGL((index_score_decode_kernel<HI, kRowsPaged, CH>), grid, block, 0, s, q, w, kv, bt.seq_lens,
                         bt.q_pos, bt.Q, bt.in_Q, n_chunks, n_items, scores);
    else if (bt.L_max % 8 == 0)
      hipLaunchKernelGGL((index_score_decode_kernel<HI, kRowsContiguous, CH>), grid, block, 0, s, q, w, kv,
                         bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, n_chunks, n_items, scores);
    else
      hipLaunchKernelGGL((index_score_decode_kernel<HI, kRowsPerLane, CH>), grid, block, 0, s, q, w, kv,
                         bt.seq_lens, bt.q_pos, bt.Q, bt.in_Q, n_chunks, n_items, scores);
  };
  using Big = std::integral_constant<int, kScoreChunk>;
  using Small = std::integral_constant<int, kScoreChunkSmall>;
  auto by_chunk = [&](auto hi) {
    if (small) dec(hi, Small{});
    else dec(hi, Big{});
  };
  if (Hi == 64) by_chunk(std::integral_constant<int, 64>{});
  else by_chunk(std::integral_constant<int, 32>{});
  return hipGetLastError();
}

}  // namespace dsa
