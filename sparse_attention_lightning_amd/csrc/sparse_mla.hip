// Sparse MLA in MQA mode ("LLM architecture survey", section 2.1 DeepSeek-V3: one cached
// latent row per token, 512 latent dims + 64 RoPE dims, 128 query heads; section 2.2
// DeepSeek-V3.2: DSA runs on MLA's MQA mode and only the k selected tokens take the full
// attention path). Every head of a query attends the same gathered rows:
//   z_i = scale * q_h . c_i (576 dims), o_h = sum_i softmax(z)_i c_i[0:512], lse_h = log sum exp z.
//
// One workgroup = one query token x all H heads (4 waves, one per SIMD, 32 heads each at
// H = 128; or, in launches too small to fill half the chip, 64 of the 128 heads at 16 per
// wave) x one split of the selected tokens. Per step of 32 tokens the workgroup gathers the
// 32 rows (1152 B each, through the index list and the block table) into a token-major LDS
// tile, then each wave runs, for each of its 16-head tiles,
//   S^T[32 tok x 16 heads] = K_tile . Q^T      (bf16 16x16x32 matrix cores, K = 576)
// with its query heads held in registers as the B operands: every K fragment read from LDS
// feeds both head tiles. S^T's accumulator layout (lane = head, 4 tokens per register) is
// exactly the A-operand layout that P needs for
//   O[16 heads x 512] += P . V                 (bf16 16x16x32 matrix cores, K = 32 tokens)
// once the K order of V matches: V's B operand is read straight from the same token-major
// tile with the LDS transpose read (ds_read_b64_tr_b16), tokens permuted to P's order, and
// every V fragment also feeds both head tiles. The 32-head output accumulator (256 registers)
// lives in the matrix-core accumulator registers; it is only ever written by products, which
// is why the softmax keeps one reference per head instead of rescaling O (see the kernel).
// The softmax runs in the log2 domain in fp32; P is rounded to bf16 for PV, and the output is
// normalised by the sum of those rounded weights (lse by the sum of the fp32 ones).
// With several splits, each workgroup writes its partial in fp32 as it stands in the
// accumulators, with lse_s and the factor f_s that normalises it (1 / its weight sum, times the
// cache scale for E4M3 rows), and a combine kernel merges them: lse = log sum_s exp lse_s,
// o = sum_s exp(lse_s - lse) f_s o_s.
#include <algorithm>
#include <type_traits>

#include "dsa_device.h"
#include "dsa_launch.h"

namespace dsa {

constexpr int kTok = 32;                        // tokens per step
constexpr int kRowBytes = kDqk * 2;             // 1152
constexpr int kSegs = kRowBytes / 128;          // 9 segments of 128 B per row
constexpr int kTileBytes = kTok * kRowBytes;    // 36 KB per step
// FP8 latent rows (576 E4M3 codes): a step's 32 rows land in a staging buffer, 8 rows per
// wave in 4.5 loads of 1 KB (5 issued, the last half onto a dummy tail), and each wave turns
// its own rows into the bf16 tile of the next step.
constexpr int kRowBytes8 = kDqk;                // 576
constexpr int kChunks8Wave = 8 * kRowBytes8 / 16;   // 288 chunks of 16 B per wave and step
constexpr int kDma8 = (kChunks8Wave + 63) / 64;     // 5 loads per wave and step
constexpr int kWaveStage8 = kDma8 * 1024;           // 5 KB per wave
constexpr int kStageBytes8 = 4 * kWaveStage8;       // 20 KB per step
constexpr int kStages = 3;                      // LDS ring depth: rows land kStages - 1 steps ahead
constexpr int kFragBatch = 2;                   // LDS fragments per read batch (32 heads per wave) ...
constexpr int kFragBatchK16 = 4;                // ... and with 16 heads per wave: K fragments
constexpr int kFragBatchV16 = 4;                //                                  V fragments
constexpr float kRefHeadroom = 64.f;            // log2 headroom of P above the softmax reference
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Split partials: unnormalised outputs o_s, with lse_s and the normalising factor f_s, all fp32.
// (bf16 partials lose up to 2^-9 of |o_s|, which is more than 2e-2 once outputs reach about 10.)
typedef float part_t;

// The second index list of a union launch: compressed sparse attention attends, in one softmax,
// over the selected compressed rows (the first list, over the layer's cache) and the window's raw
// rows (this list, over its own cache). k = 0 in every other launch.
struct MlaSecond {
  CacheView lat;
  const int32_t* idx;
  int k, idx_q_stride;
};

// Per-layer arguments of a launch over up to kMlaMaxLayers layers that share one index set
// (IndexShare): blockIdx.y picks the layer.
struct MlaLayers {
  const uint16_t* q[kMlaMaxLayers];
  CacheView lat[kMlaMaxLayers];
  float* out[kMlaMaxLayers];
  float* lse[kMlaMaxLayers];
};

constexpr int kMaxSplits = 16;                  // splits per query token, at most

constexpr int kTargetWgs = 256;                 // workgroups a launch aims at (one per CU)
constexpr int kMinSplit = 128;                  // tokens per split, at least

// Splits per query token: enough workgroups to fill the chip while each split keeps a minimum
// of tokens. Workgroups are counted as the launch makes them, over all nl layers it holds: at
// H = 128, a launch that fills at most half the chip deals the 128 heads to two workgroups
// (below). At 32 query tokens (or 8 tokens x 4 layers) that gives 4 splits x 2 head groups
// rather than 8 (16) splits x 1: fewer fp32 partials to write and merge (measured at 32 tokens:
// MLA + combine 46.4 against 53.1 us). A group of layers may therefore split differently from
// a launch of one of its layers alone, and round differently within the tolerance.
// FP8 rows keep one head group per split (the count ignores head groups): two groups would each
// gather and convert the same E4M3 rows, and 8 splits x 32 heads per wave measured 62 us against
// 70 us for 4 x 2 at 32 decode rows.
int sparse_mla_splits(int rows, int H, int k, int nl, bool f8) {
  const int units = rows * nl;
  auto wgs = [&](int s) {
    return (!f8 && H == 128 && 2 * units * s <= kTargetWgs) ? 2 * units * s : units * s;
  };
  int s = 1;
  while (wgs(s) < kTargetWgs && (k + 2 * s - 1) / (2 * s) >= kMinSplit && s < kMaxSplits) s *= 2;
  while ((k + s - 1) / s > kMaxK && s < kMaxSplits) s *= 2;   // a split's row ids fit the LDS list
  return s;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split partials of one launch of nl layers: per layer [rows][splits][H][512] part_t, then
// [rows][splits][H] fp32 lse followed by [rows][splits][H] fp32 normalising factors.
static size_t part_o_layer(int rows, int splits, int H) { return align256((size_t)rows * splits * H * kDv * sizeof(part_t)); }
static size_t part_lse_layer(int rows, int splits, int H) { return align256(2 * (size_t)rows * splits * H * sizeof(float)); }
static size_t launch_ws_bytes(int rows, int H, int k, int nl, bool f8) {
  const int s = sparse_mla_splits(rows, H, k, nl, f8);
  if (s == 1) return 0;
  return (size_t)nl * (part_o_layer(rows, s, H) + part_lse_layer(rows, s, H));
}

size_t sparse_mla_workspace_bytes(int rows, int H, int k, int n_layers) {
  // layers go kMlaMaxLayers per launch; the last launch may hold fewer. One size serves bf16 and
  // FP8 rows, whose split counts may differ.
  size_t b = 0;
  for (const bool f8 : {false, true}) {
    b = std::max(b, launch_ws_bytes(rows, H, k, std::min(n_layers, kMlaMaxLayers), f8));
    if (n_layers > kMlaMaxLayers && n_layers % kMlaMaxLayers)
      b = std::max(b, launch_ws_bytes(rows, H, k, n_layers % kMlaMaxLayers, f8));
  }
  return b;
}

typedef const __attribute__((address_space(3))) uint8_t* lds_ptr;

__device__ __forceinline__ v8bf lds_v8bf(lds_ptr p) { return *(const __attribute__((address_space(3))) v8bf*)p; }

// An offset the compiler may not look through: fragment reads at (slot + offset) plus a constant
// then keep the constant in the instruction's offset field, instead of the compiler merging it
// into the XOR-swizzled offset (it turns the addition of disjoint bits into an OR, which the
// offset field cannot absorb) and computing a fresh address per fragment. Only the offset is
// hidden: the pointer keeps its LDS variable, which the wait analysis below relies on.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t a) {
  asm volatile("" : "+v"(a));
  return a;
}

__device__ __forceinline__ v4bf lds_tr_read(lds_ptr p) {
  typedef __attribute__((address_space(3))) v4bf lds_v4bf;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p));
}

// LDS tile layout of one step: 9 segments of [32 rows][128 B]; inside a row segment the eight
// 16-byte chunks are XOR-swizzled by (row & 7). The LDS serves a 16-byte-per-lane read eight
// lanes at a time over its 32 banks: the eight rows of a fragment read then hit eight distinct
// 16-byte bank groups, and so do the 4 tokens x 2 chunks of a transpose read (measured: no
// bank-conflict cycles, against 31% of LDS-busy cycles with a (row >> 1) swizzle).
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return (chunk >> 3) * (kTok * 128) + row * 128 + 16 * ((chunk & 7) ^ (row & 7));
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt
// [11:8]): wait until at most VM vector memory operations and LGKM LDS/scalar operations of
// this wave are outstanding. VM = 63 / LGKM = 15 mean "no wait" on that counter.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

template <int NW, int HT, bool SPLIT, bool F8>
__global__ __launch_bounds__(NW * 64, 1) void sparse_mla_kernel(
    MlaLayers layers, const int32_t* __restrict__ idx, int k, int idx_q_stride, MlaSecond sec, int Q, int H,
    int splits,
    int split_len, float scale_log2, float out_scale, part_t* __restrict__ part_o_all,
    float* __restrict__ part_lse_all, int64_t part_o_stride, int64_t part_lse_stride, int64_t nrm_off, int n_hg,
    int n_units, bool tok_xcd) {
  // layer blockIdx.y of the launch: its query, latent cache, outputs and partials
  const int layer = blockIdx.y;
  const uint16_t* __restrict__ q = layers.q[layer];
  const CacheView lat = layers.lat[layer];
  float* __restrict__ out = layers.out[layer];
  float* __restrict__ lse_out = layers.lse[layer];
  part_t* __restrict__ part_o = part_o_all + layer * part_o_stride;
  float* __restrict__ part_lse = part_lse_all + layer * part_lse_stride;
  // fragments per LDS read batch: a batch feeds FB x HT products, enough to cover the latency of
  // the next batch's reads
  constexpr int FBK = HT == 1 ? kFragBatchK16 : kFragBatch;
  constexpr int FBV = HT == 1 ? kFragBatchV16 : kFragBatch;
  // The ring of gathered tiles, as three LDS variables. While a direct-to-LDS load is in flight
  // the compiler makes every LDS read that may alias its destination wait for it (a wait on the
  // vector-memory counter, i.e. for every gather issued so far); reads and loads that name
  // different LDS variables are known not to alias. With the step loop unrolled by three, every
  // read and every load names its slot statically, so the gather of step st + 2 stays in flight
  // through step st.
  static_assert(kStages == 3, "three named ring slots");
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[F8 ? 1024 : kTileBytes];      // FP8: two slots
  __shared__ __attribute__((aligned(1024))) uint8_t stg0[F8 ? kStageBytes8 : 1024];      // FP8 staging
  __shared__ __attribute__((aligned(1024))) uint8_t stg1[F8 ? kStageBytes8 : 1024];
  auto ring_of = [&](auto slot) -> uint8_t* {
    constexpr int S = decltype(slot)::value;
    if constexpr (S == 0) return ring0;
    else if constexpr (S == 1) return ring1;
    else return ring2;
  };
  auto stg_of = [&](auto p) -> uint8_t* {
    if constexpr (decltype(p)::value == 0) return stg0;
    else return stg1;
  };
  __shared__ int rowid[kMaxK];
  __shared__ int redo_any;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  // Workgroups are dealt to the 8 XCDs in turn, so workgroup ids 8 apart share an XCD and its
  // L2. With at least 8 query tokens (tok_xcd), every workgroup of token bq (its splits x n_hg
  // head groups) gets an id congruent to bq mod 8: the head groups of a split gather the same
  // rows, and every split reads the token's query, from that one L2. With fewer tokens the
  // splits spread over the XCDs and only the head groups of a split share one (ids 8 apart).
  int bq, split, hg = 0;
  if (tok_xcd) {
    const int per_tok = splits * n_hg;
    const int r8 = blockIdx.x >> 3;
    bq = (r8 / per_tok) * 8 + (blockIdx.x & 7);
    const int w_tok = r8 - (r8 / per_tok) * per_tok;
    split = w_tok / n_hg;
    hg = w_tok - split * n_hg;
    if (bq * splits >= n_units) return;                // the grid is padded to whole groups of 8 tokens
  } else {
    int unit = blockIdx.x;
    if (n_hg > 1) {
      const int grp = blockIdx.x / (8 * n_hg), r = blockIdx.x - grp * 8 * n_hg;
      hg = r >> 3;
      unit = grp * 8 + (r & 7);
    }
    if (unit >= n_units) return;                       // the grid is padded to whole groups of 8
    split = unit % splits;
    bq = unit / splits;
  }
  const int b = bq / Q, j = bq - b * Q;
  const int h0 = (hg * NW + wave) * 16 * HT;           // this wave's heads: tile ht = h0 + 16 ht ..
  constexpr int my_dma = kSegs;                        // loads this wave issues per step

  // The split's tokens: positions tok_begin .. tok_end of the list, or of the two lists one after
  // the other in a union launch (token t >= k is entry t - k of the second list).
  const int32_t* irow = idx + (int64_t)b * (idx_q_stride ? (int64_t)Q * k : k) + (int64_t)j * idx_q_stride;
  const bool two = sec.k > 0;                          // launch-uniform
  const int32_t* irow2 =
      two ? sec.idx + (int64_t)b * (sec.idx_q_stride ? (int64_t)Q * sec.k : sec.k) + (int64_t)j * sec.idx_q_stride
          : nullptr;
  const int tok_begin = split * split_len;
  const int tok_end = min(k + sec.k, tok_begin + split_len);
  const int n_steps = tok_end > tok_begin ? (tok_end - tok_begin + kTok - 1) / kTok : 0;

  // Direct-to-LDS gather of step st: load d = (row group rg = d % 4, segment d / 4) lands rows
  // 8rg + l/8, slot l%8 of the segment, fetching the chunk that the swizzle puts there.
  // Loads are dealt round-robin over the waves; with 4 waves, wave w issues exactly the 9
  // segments of row group w, so one row id per lane serves all of its loads of a step.
  static_assert(NW == 4, "loads of a wave share one row group");
  const int my_row = 8 * wave + (lane >> 3);
  // Steps past the last one load row 0 into a slot that is read no more: every step issues the
  // same loads, so the number of loads in flight is the same on every path.
  auto step_row = [&](int st) { return st < n_steps ? rowid[st * kTok + my_row] : -1; };
  // row ids: r >= 0 a row of the layer's cache, r <= -2 row -2 - r of the second list's cache,
  // -1 a masked token (its loads read row 0, and its tile row is zeroed)
  auto row_base = [&](int r, int64_t row_bytes) -> const uint8_t* {
    if (r >= 0) return lat.base + (int64_t)r * row_bytes;
    if (r <= -2) return sec.lat.base + (int64_t)(-2 - r) * row_bytes;
    return lat.base;
  };
  auto row_src = [&](int r) -> const uint8_t* { return row_base(r, kRowBytes) + 16 * ((lane & 7) ^ (my_row & 7)); };
  auto step_src = [&](int st) { return row_src(step_row(st)); };
  auto issue_seg = [&](const uint8_t* src, auto slot, int sg) {
    uint8_t* base = ring_of(slot) + wave * 1024;
    __builtin_amdgcn_global_load_lds((const void*)(src + 128 * sg),
                                     (__attribute__((address_space(3))) void*)(base + sg * (kTok * 128)), 16, 0, 0);
  };
  auto issue_step = [&](int st, auto slot) {
    const uint8_t* src = step_src(st);
#pragma unroll
    for (int sg = 0; sg < kSegs; ++sg) issue_seg(src, slot, sg);
  };

  // Row index (into the cache's rows) of every token of the split, -1 for masked tokens. The
  // chain index -> block table -> gather is the kernel's start-up latency, so every index load
  // goes out at once, then every table load (unconditional, a masked token reading the
  // sequence's first entry, and in one branch, so that they issue as one batch), then the
  // query: the loads complete in order, and the query's latency then overlaps the table's.
  const int n_tok = n_steps * kTok;
  constexpr int kPerThread = kMaxK / (NW * 64);
  int pos_t[kPerThread], page_t[kPerThread] = {};
  const int32_t* trow = lat.table ? lat.table + (int64_t)b * lat.max_pages : nullptr;
  const int32_t* trow2 = two && sec.lat.table ? sec.lat.table + (int64_t)b * sec.lat.max_pages : nullptr;
  if (!two) {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int i = tid + e * NW * 64;
      pos_t[e] = (i < n_tok && tok_begin + i < tok_end) ? irow[tok_begin + i] : -1;
    }
    if (trow) {                                        // block-uniform
      const uint32_t ps = (uint32_t)lat.page_size;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) page_t[e] = trow[(uint32_t)max(pos_t[e], 0) / ps];
    }
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const int t = tok_begin + tid + e * NW * 64;
      const int32_t* src = t < k ? irow + t : irow2 + (t - k);
      pos_t[e] = (tid + e * NW * 64 < n_tok && t < tok_end) ? *src : -1;
    }
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const bool s2 = tok_begin + tid + e * NW * 64 >= k;
      const int32_t* tr = s2 ? trow2 : trow;
      const uint32_t ps = (uint32_t)(s2 ? sec.lat.page_size : lat.page_size);
      if (tr) page_t[e] = tr[(uint32_t)max(pos_t[e], 0) / ps];
    }
  }

  // query heads h0 + 16 ht + (l % 16) as the B operands of S^T = K . Q^T: 8 dims per lane per K step
  v8bf qb[HT][kDqk / 32];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const uint16_t* qrow = q + ((int64_t)bq * H + h0 + 16 * ht + c16) * kDqk;
#pragma unroll
    for (int s = 0; s < kDqk / 32; ++s) qb[ht][s] = *(const v8bf*)(qrow + 32 * s + 8 * g);
  }

  if (tid == 0) redo_any = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int i = tid + e * NW * 64;
    const int pos = pos_t[e];
    if (i < n_tok) {
      if (!two || tok_begin + i < k)
        rowid[i] = pos < 0 ? -1 : trow ? page_t[e] * lat.page_size + pos % lat.page_size : b * lat.L_max + pos;
      else
        rowid[i] = pos < 0 ? -1
                           : -2 - (trow2 ? page_t[e] * sec.lat.page_size + pos % sec.lat.page_size
                                         : b * sec.lat.L_max + pos);
    }
  }
  __syncthreads();

  // FP8 rows of step st into staging buffer p: chunk i = 64 d + lane of the wave's 288 is
  // 16 bytes of row 8 wave + i / 36; chunks past 288 (half of the last load) and rows of
  // masked tokens or of steps past the last read row 0 into places nothing reads.
  // load d of this wave's share of step st, into staging buffer p. The lane's chunk numbers
  // are recomputed at every load rather than kept across the loop, where they would cost
  // registers the step needs.
  auto issue_seg8 = [&](int st, auto p, int d) {
    uint8_t* base = stg_of(p) + wave * kWaveStage8;
    const int ln = (int)opaque_u32((uint32_t)lane);
    const int i = d * 64 + ln;
    const int rl = i / 36, c = i - 36 * (i / 36);
    const int r = (i < kChunks8Wave && st < n_steps) ? rowid[st * kTok + 8 * wave + rl] : -1;
    const uint8_t* src = row_base(r, kRowBytes8) + (r != -1 ? 16 * c : 0);
    __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(base + d * 1024),
                                     16, 0, 0);
  };
  auto issue_step8 = [&](int st, auto p) {
#pragma unroll
    for (int d = 0; d < kDma8; ++d) issue_seg8(st, p, d);
  };
  // this wave's 8 FP8 rows of step st, from staging buffer p into the bf16 tile of `slot`
  // (masked tokens become zero rows). E4M3 values are exact in bf16, and gfx950 converts two
  // codes to two packed bf16 in one instruction (scale 1: the same bits as the fp32 route,
  // whose upper half is the bf16 pattern, on every non-NaN code).
  auto convert8 = [&](int st, auto p, auto slot) {
    const uint8_t* sb = stg_of(p) + wave * kWaveStage8;
    uint8_t* tile = ring_of(slot);
    // two codes of x (bytes 0-1, or 2-3 when `upper`) as two packed bf16
    auto two = [](uint32_t x, bool upper) -> uint32_t {
      const v2bf r = upper ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true)
                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
      return __builtin_bit_cast(uint32_t, r);
    };
    const int ln = (int)opaque_u32((uint32_t)lane);
#pragma unroll 1
    for (int e = 0; e < kDma8; ++e) {                // one chunk at a time: few registers live
      const int i = e * 64 + ln;
      if (i < kChunks8Wave) {
        const int rl = i / 36, c = i - 36 * (i / 36);
        const int row = 8 * wave + rl;
        v4i lo = {0, 0, 0, 0}, hi = {0, 0, 0, 0};
        if (rowid[st * kTok + row] != -1) {
          const v4i x = *(const v4i*)(sb + 16 * i);      // dims 16c .. 16c + 15
          lo = (v4i){(int)two(x[0], false), (int)two(x[0], true), (int)two(x[1], false), (int)two(x[1], true)};
          hi = (v4i){(int)two(x[2], false), (int)two(x[2], true), (int)two(x[3], false), (int)two(x[3], true)};
        }
        *(v4i*)(tile + tile_off(row, 2 * c)) = lo;
        *(v4i*)(tile + tile_off(row, 2 * c + 1)) = hi;
      }
    }
  };

  // masked rows this wave landed: overwrite the dummy bytes with zeros
  auto zero_masked = [&](int st, auto slot) {
    if (rowid[st * kTok + my_row] != -1) return;
    uint8_t* base = ring_of(slot) + wave * 1024;
#pragma unroll
    for (int sg = 0; sg < kSegs; ++sg) *(v4i*)(base + sg * (kTok * 128) + 16 * lane) = (v4i){0, 0, 0, 0};
  };

  // Per-lane LDS offsets inside a tile. Chunk c of row r sits at segment c/8, slot
  // (c & 7) ^ (r & 7); for the fragments below the slot varies only in bits the XOR
  // immediates flip, so one base per row serves all of them:
  //   QK (token 16mt + c16, chunk 4s + g):   (qk_base[mt] ^ 64 (s & 1)) + (s / 2) * 4096
  //   PV (token row vrow_hf, dims 16nt..):   (pv_base[hf] ^ 32 (nt & 3)) + (nt / 4) * 4096
  int qk_base[2], pv_base[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) qk_base[mt] = tile_off(16 * mt + c16, g);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
    pv_base[hf] = tile_off(4 * g + (c16 >> 2) + 16 * hf, (c16 & 3) >> 1) + 8 * (c16 & 1);

  // Softmax reference. Every head keeps one reference m_ref (log2 domain) for the whole split:
  // the maximum of the first step that has a visible token. P = 2^(z - m_ref) may exceed 1
  // (fp32 and bf16 hold up to 2^127), so the accumulator O is never rescaled and is touched
  // only by matrix-core products. Should a later logit exceed m_ref by more than
  // kRefHeadroom, the split is computed again with m_ref = the exact maximum of its logits,
  // which the first pass records.
  v4f o[HT][kDv / 16];
  // l_run sums the fp32 weights (for lse); l_pv sums the bf16-rounded weights that PV multiplies,
  // so that the output's numerator and denominator use the same weights: a dominant token's
  // rounding then cancels instead of scaling the output by up to 1 +- 2^-9.
  float m_ref[HT], m_max[HT], l_run[HT], l_pv[HT];
  bool redo = false;
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) m_max[ht] = -INFINITY;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) {
      if (!redo_any) break;                            // workgroup-uniform
      __syncthreads();                                 // every wave is done with the ring
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
      for (int nt = 0; nt < kDv / 16; ++nt) o[ht][nt] = (v4f){0.f, 0.f, 0.f, 0.f};
      m_ref[ht] = pass == 0 ? -INFINITY : m_max[ht];
      l_run[ht] = 0.f;
      l_pv[ht] = 0.f;
    }
    constexpr int kAheadSteps = kStages - 1;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // QK, softmax and PV of step st on a landed bf16 tile
    // seg(sg) issues load segment sg of a later step. Issuing a direct-to-LDS load can hold the
    // wave for tens of cycles while the memory pipeline takes the previous ones; issued as one
    // block before the products, the 9 loads of a step took about a sixth of the step with the
    // matrix cores idle. The QK loop spreads them over its fragment batches instead, so that the
    // matrix cores run through those holds.
    auto compute = [&](int st, const uint8_t* tile, auto seg) {
      // one validity bit per token of the step (lanes 32..63 repeat lanes 0..31)
      const uint32_t valid = (uint32_t)__ballot(rowid[st * kTok + (lane & 31)] != -1);

      // LDS fragment reads go in batches of FBK, double-buffered: batch b + 1 is issued
      // right after an explicit wait for batch b and lands while batch b's products run. (While a
      // direct-to-LDS load is in flight the compiler waits for all LDS reads at every use, so
      // the distance between a read and its wait is set here, by the order of the code.)
      // ---- S^T = K_tile . Q^T over K = 576: each K fragment feeds HT products
      v4f sacc[HT][2];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) sacc[ht][mt] = (v4f){0.f, 0.f, 0.f, 0.f};
      {
        lds_ptr kb[2][2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int x = 0; x < 2; ++x) kb[mt][x] = (lds_ptr)tile + opaque_u32(qk_base[mt] ^ (64 * x));
        auto kfrag = [&](int i) {
          const int s2 = i >> 1, mt = i & 1;
          return lds_v8bf(kb[mt][s2 & 1] + (s2 >> 1) * (kTok * 128));
        };
        constexpr int NF = 2 * (kDqk / 32);
        static_assert(NF % FBK == 0, "whole batches of K fragments");
        v8bf kc[FBK], kn[FBK];
#pragma unroll
        for (int i = 0; i < FBK; ++i) kc[i] = kfrag(i);
#pragma unroll
        for (int bt = 0; bt < NF / FBK; ++bt) {
          wait_counts<63, 0>();
          __builtin_amdgcn_sched_barrier(0);
          if (bt + 1 < NF / FBK) {
#pragma unroll
            for (int i = 0; i < FBK; ++i) kn[i] = kfrag((bt + 1) * FBK + i);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < FBK; ++i) {
            const int f = bt * FBK + i;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) sacc[ht][f & 1] = mfma_bf16(kc[i], qb[ht][f >> 1], sacc[ht][f & 1]);
          }
          // the step's kSegs load segments, spread evenly over the NF / FBK batches
          constexpr int NB = NF / FBK;
#pragma unroll
          for (int sg = bt * kSegs / NB; sg < (bt + 1) * kSegs / NB; ++sg) seg(sg);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < FBK; ++i) kc[i] = kn[i];
        }
      }
      // V^T fragments by transpose reads, tokens 4g+e (e<4), 16+4g+(e-4) (e>=4); the first batch
      // is issued before the softmax, which has no LDS traffic of its own
      lds_ptr vb[2][4];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int x = 0; x < 4; ++x) vb[hf][x] = (lds_ptr)tile + opaque_u32(pv_base[hf] ^ (32 * x));
      auto vfrag = [&](int nt) {
        const v4bf lo = lds_tr_read(vb[0][nt & 3] + (nt >> 2) * (kTok * 128));
        const v4bf hi = lds_tr_read(vb[1][nt & 3] + (nt >> 2) * (kTok * 128));
        return (v8bf){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      v8bf vc[FBV], vn[FBV];
#pragma unroll
      for (int i = 0; i < FBV; ++i) vc[i] = vfrag(i);
      __builtin_amdgcn_sched_barrier(0);

      // ---- softmax weights of heads h0 + 16 ht + c16 over tokens 16mt + 4g + r. The maximum is
      // taken over the raw logits (the scale is positive, so it commutes with the maximum) and
      // the scale is folded into the exponent's multiply-add; masked tokens (only in a step
      // with -1 entries or past the end of the split) become -inf.
      const bool all_valid = valid == 0xffffffffu;     // wave-uniform
      v8bf pa[HT];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        float z[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = sacc[ht][i >> 2][i & 3];
        if (!all_valid) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (!((valid >> (16 * (i >> 2) + 4 * g + (i & 3))) & 1u)) z[i] = -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])), fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
        tmax = max_xor32(max_xor16(tmax)) * scale_log2;
        m_max[ht] = fmaxf(m_max[ht], tmax);
        if (m_ref[ht] == -INFINITY) m_ref[ht] = tmax;  // the first step with a visible token
        redo |= tmax > m_ref[ht] + kRefHeadroom;
        const float neg_m = (m_ref[ht] == -INFINITY) ? 0.f : -m_ref[ht];
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // v_exp_f32 directly: its flush of results below 2^-126 to 0 is harmless here
          const float pv = __builtin_amdgcn_exp2f(fmaf(z[i], scale_log2, neg_m));
          psum += pv;
          pa[ht][i] = (__bf16)pv;
        }
        l_run[ht] += psum;
        // the rounded weights, two per dot-product instruction (products by 1 are exact)
        const v2bf one2 = {(__bf16)1.f, (__bf16)1.f};
        float pbsum = l_pv[ht];
#pragma unroll
        for (int i = 0; i < 8; i += 2)
          pbsum = __builtin_amdgcn_fdot2_f32_bf16((v2bf){pa[ht][i], pa[ht][i + 1]}, one2, pbsum, false);
        l_pv[ht] = pbsum;
      }
      __builtin_amdgcn_sched_barrier(0);
      // ---- O += P . V; each V fragment feeds HT products
      {
        constexpr int NV = kDv / 16;
        static_assert(NV % FBV == 0, "whole batches of V fragments");
#pragma unroll
        for (int bt = 0; bt < NV / FBV; ++bt) {
          wait_counts<63, 0>();
          __builtin_amdgcn_sched_barrier(0);
          if (bt + 1 < NV / FBV) {
#pragma unroll
            for (int i = 0; i < FBV; ++i) vn[i] = vfrag((bt + 1) * FBV + i);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < FBV; ++i) {
            const int nt = bt * FBV + i;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) o[ht][nt] = mfma_bf16(pa[ht], vc[i], o[ht][nt]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < FBV; ++i) vc[i] = vn[i];
        }
      }
    };
    if constexpr (!F8) {
      issue_step(0, I0{});
      issue_step(1, I1{});
      // the row of step st + 2 is read from LDS a step early, so that its latency is not waited
      // for right before the loads that need it
      int row_ahead = step_row(kAheadSteps);
      // step st in ring slot S = st % 3
      auto step_body = [&](int st, auto slot) {
        constexpr int S = decltype(slot)::value;
        static_assert(kAheadSteps == 2, "one step of loads in flight behind the current one");
        wait_counts<my_dma, 15>();                     // this step's rows have landed
        zero_masked(st, slot);
        wait_counts<63, 0>();                          // LDS writes done before the barrier
        __builtin_amdgcn_s_barrier();
        // into step st - 1's slot, which every wave has finished reading
        const uint8_t* src = row_src(row_ahead);
        row_ahead = step_row(st + kAheadSteps + 1);
        using SN = std::integral_constant<int, (S + kAheadSteps) % kStages>;
        compute(st, ring_of(slot), [&](int sg) { issue_seg(src, SN{}, sg); });
      };
      // unrolled by the three ring slots, so that every step names its slots statically
      for (int st = 0; st < n_steps; st += kStages) {
        step_body(st, I0{});
        if (st + 1 < n_steps) step_body(st + 1, I1{});
        if (st + 2 < n_steps) step_body(st + 2, std::integral_constant<int, 2>{});
      }
    } else {
      // FP8: loads two steps ahead into two staging buffers; each wave converts its rows of step
      // st + 1 into the other bf16 slot while step st computes, so two bf16 slots suffice.
      issue_step8(0, I0{});
      issue_step8(1, I1{});
      wait_counts<kDma8, 15>();                        // step 0's rows (this wave's) have landed
      convert8(0, I0{}, I0{});
      auto step8 = [&](int st, auto p) {               // p = st % 2: staging and bf16 slot of st
        constexpr int P = decltype(p)::value;
        using Pn = std::integral_constant<int, 1 - P>;
        wait_counts<63, 0>();                          // conversion writes done before the barrier
        __builtin_amdgcn_s_barrier();
        // bf16 slot 1 - p held step st - 1, which every wave has finished reading
        if (st + 1 < n_steps) {                        // workgroup-uniform
          wait_counts<0, 15>();                        // step st + 1's rows have landed
          convert8(st + 1, Pn{}, Pn{});
        }
        // staging p held step st, which this wave converted a step ago: step st + 2's loads go
        // there, spread over the QK loop like the bf16 path's
        compute(st, ring_of(p), [&](int sg) {
          if (sg < kDma8) issue_seg8(st + 2, p, sg);
        });
      };
      for (int st = 0; st < n_steps; st += 2) {
        step8(st, I0{});
        if (st + 1 < n_steps) step8(st + 1, I1{});
      }
    }
    wait_counts<0, 15>();                              // the loads past the last step have landed
    if (pass == 0) {
      if (__ballot(redo) != 0ull && lane == 0) atomicOr(&redo_any, 1);
      __syncthreads();
    }
  }

  // ---- finish: denominators of heads h0 + 16 ht + c16, then per accumulator head h0 + 16 ht + 4g + r
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    const float l_tot = sum_xor32(sum_xor16(l_run[ht]));
    const float lpv_tot = sum_xor32(sum_xor16(l_pv[ht]));
    const float lse_h = (l_tot > 0.f) ? (m_ref[ht] + log2f(l_tot)) * kLn2 : -INFINITY;
    const int hb = h0 + 16 * ht;
    if (SPLIT) {
      // the partial as the accumulators hold it; the combine applies the factor
      const int64_t ps = (int64_t)bq * splits + split;
      part_t* pbase = part_o + (ps * H + hb) * kDv;
      if (g == 0) {
        float f = lpv_tot > 0.f ? 1.f / lpv_tot : 0.f;
        if constexpr (F8) f *= out_scale;             // the FP8 cache's scale on the values
        part_lse[ps * H + hb + c16] = lse_h;
        part_lse[nrm_off + ps * H + hb + c16] = f;
      }
#pragma unroll
      for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pbase[(4 * g + r) * kDv + 16 * nt + c16] = (part_t)o[ht][nt][r];
    } else {
      float inv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lr = __shfl(lpv_tot, 4 * g + r, 64);
        inv[r] = lr > 0.f ? 1.f / lr : 0.f;
        if constexpr (F8) inv[r] *= out_scale;       // the FP8 cache's scale on the values
      }
      float* obase = out + ((int64_t)bq * H + hb) * kDv;
      if (g == 0 && lse_out) lse_out[(int64_t)bq * H + hb + c16] = lse_h;
#pragma unroll
      for (int nt = 0; nt < kDv / 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) obase[(4 * g + r) * kDv + 16 * nt + c16] = o[ht][nt][r] * inv[r];
    }
  }
}

// Merge split partials: one workgroup per (query token, 4 heads), 64 threads x 8 dims per head
// (two 16-byte loads per split and thread); every split's lse and partial are loaded before the
// merge, so the loads overlap. S > 0 fixes the split count at S: registers for exactly that many
// partials, so that every workgroup of a decode-sized launch fits on the chip at once (at 4
// splits: 55 VGPRs and 8 waves per SIMD, against 175 VGPRs for the general form). S = 0 takes
// any count up to kMaxSplits from `splits_rt`; it serves 16 splits, where the fixed form's
// compiler schedule consumed each partial before loading the next and measured slower.
template <int S>
__global__ __launch_bounds__(256) void mla_combine_kernel(MlaLayers layers, const part_t* __restrict__ part_o_all,
                                                          const float* __restrict__ part_lse_all, int H, int n_rows,
                                                          int splits_rt,
                                                          int64_t part_o_stride, int64_t part_lse_stride,
                                                          int64_t nrm_off) {
  constexpr int N = S > 0 ? S : kMaxSplits;
  const int splits = S > 0 ? S : splits_rt;
  typedef part_t p8 __attribute__((ext_vector_type(8)));
  const int layer = blockIdx.y;
  const part_t* __restrict__ part_o = part_o_all + layer * part_o_stride;
  const float* __restrict__ part_lse = part_lse_all + layer * part_lse_stride;
  float* __restrict__ out = layers.out[layer];
  float* __restrict__ lse_out = layers.lse[layer];
  const int hl = threadIdx.x >> 6, t = threadIdx.x & 63;
  // with at least 8 query tokens, the workgroups of token bq get ids congruent to bq mod 8, like
  // the attention's that wrote its partials: one XCD
  int bq, h;
  if (n_rows >= 8) {
    const int r8 = blockIdx.x >> 3, per_tok = H / 4;
    bq = (r8 / per_tok) * 8 + (blockIdx.x & 7);
    if (bq >= n_rows) return;                          // the grid is padded to whole groups of 8 tokens
    h = (r8 - (r8 / per_tok) * per_tok) * 4 + hl;
  } else {
    bq = blockIdx.x / (H / 4);
    h = (blockIdx.x - bq * (H / 4)) * 4 + hl;
  }
  float ls[N], nr[N];
  p8 po[N];
#pragma unroll
  for (int s = 0; s < N; ++s) {
    const bool in = S > 0 || s < splits;
    const int64_t ps = (int64_t)bq * splits + s;
    ls[s] = in ? part_lse[ps * H + h] : -INFINITY;
    nr[s] = in ? part_lse[nrm_off + ps * H + h] : 0.f;
    if (in) po[s] = *(const p8*)(part_o + (ps * H + h) * kDv + 8 * t);
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < N; ++s) mx = fmaxf(mx, ls[s]);
  v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float den = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int s = 0; s < N; ++s) {
      if (S > 0 || s < splits) {
        const float wgt = expf(ls[s] - mx);
        den += wgt;
        const float c = wgt * nr[s];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e >> 2][e & 3] += c * (float)po[s][e];
      }
    }
    const float inv = 1.f / den;
    acc[0] *= inv;
    acc[1] *= inv;
  }
  float* orow = out + ((int64_t)bq * H + h) * kDv + 8 * t;
  *(v4f*)orow = acc[0];
  *(v4f*)(orow + 4) = acc[1];
  if (t == 0 && lse_out) lse_out[(int64_t)bq * H + h] = (mx == -INFINITY) ? -INFINITY : mx + logf(den);
}

template <int NW, int HT, bool F8>
static void launch_mla(int splits, dim3 grid, hipStream_t s, const MlaLayers& L, const int32_t* idx, int k,
                       int idx_q_stride, const MlaSecond& sec, int Q, int H, int split_len, float sl2,
                       float out_scale, part_t* part_o, float* part_lse, int64_t so, int64_t sl, int n_hg,
                       int units, bool tok_xcd) {
  const dim3 block(NW * 64);
  const int64_t nrm_off = (int64_t)units * H;          // the factors follow the units' lse
  if (splits == 1)
    hipLaunchKernelGGL((sparse_mla_kernel<NW, HT, false, F8>), grid, block, 0, s, L, idx, k, idx_q_stride, sec, Q,
                       H, 1, split_len, sl2, out_scale, nullptr, nullptr, (int64_t)0, (int64_t)0, (int64_t)0, n_hg,
                       units, tok_xcd);
  else
    hipLaunchKernelGGL((sparse_mla_kernel<NW, HT, true, F8>), grid, block, 0, s, L, idx, k, idx_q_stride, sec, Q,
                       H, splits, split_len, sl2, out_scale, part_o, part_lse, so, sl, nrm_off, n_hg, units, tok_xcd);
}

// The second list of a union launch (one layer), with its own cache of L_max rows per sequence.
struct HostSecond {
  HostCache latent;
  const int32_t* idx;
  int k, idx_q_stride, L_max;
};

// latent_scale > 0: FP8 latent rows (576 E4M3 codes, value = latent_scale x code); 0: bf16 rows
static hipError_t launch_layers(const HostBatch& bt, const uint16_t* const* q, int H, const HostCache* latents,
                                float latent_scale, const int32_t* idx, int k, int idx_q_stride, float scale,
                                float* const* out, float* const* lse, int n_layers, void* ws, hipStream_t s,
                                const HostSecond* second = nullptr) {
  const int rows = bt.B * bt.Q;
  const bool f8 = latent_scale > 0.f;
  const float sl2 = scale * (f8 ? latent_scale : 1.f) * kLog2e;
  MlaSecond sec{};
  if (second) {
    const HostCache& c = second->latent;
    sec.lat = CacheView{(const uint8_t*)c.base, c.table, c.max_pages, c.page_size, f8 ? kRowBytes8 : kRowBytes,
                        second->L_max};
    sec.idx = second->idx;
    sec.k = second->k;
    sec.idx_q_stride = second->idx_q_stride;
  }
  const int k_all = k + sec.k;
  for (int l0 = 0; l0 < n_layers; l0 += kMlaMaxLayers) {
    const int nl = std::min(kMlaMaxLayers, n_layers - l0);
    MlaLayers L{};
    for (int i = 0; i < nl; ++i) {
      const HostCache& c = latents[l0 + i];
      L.q[i] = q[l0 + i];
      L.lat[i] = CacheView{(const uint8_t*)c.base, c.table, c.max_pages, c.page_size, f8 ? kRowBytes8 : kRowBytes,
                           bt.L_max};
      L.out[i] = out[l0 + i];
      L.lse[i] = lse ? lse[l0 + i] : nullptr;
    }
    const int splits = sparse_mla_splits(rows, H, k_all, nl, f8);
    int split_len = (k_all + splits - 1) / splits;
    split_len = (split_len + kTok - 1) / kTok * kTok;
    part_t* part_o = nullptr;
    float* part_lse = nullptr;
    int64_t so = 0, sl = 0;
    if (splits > 1) {
      // every layer of the launch has its own partials
      so = (int64_t)(part_o_layer(rows, splits, H) / sizeof(part_t));
      sl = (int64_t)(part_lse_layer(rows, splits, H) / sizeof(float));
      part_o = (part_t*)ws;
      part_lse = (float*)((char*)ws + (size_t)nl * part_o_layer(rows, splits, H));
    }
    // one wave per SIMD: 4 waves x 32 heads (H = 128) or 4 waves x 16 heads (H = 64). When the
    // splits are already as short as they go and the launch still fills under half the chip, the
    // 128 heads are dealt to two workgroups of 4 x 16 heads instead (same splits, same results).
    const int units = rows * splits;
    const int n_hg = (H == 128 && 2 * units * nl <= kTargetWgs) ? 2 : 1;
    const bool tok_xcd = rows >= 8;
    const dim3 grid(tok_xcd ? (unsigned)((rows + 7) / 8 * 8 * splits * n_hg)
                            : (n_hg == 1 ? (unsigned)units : (unsigned)((units + 7) / 8 * 8 * n_hg)),
                    (unsigned)nl);
    const float os = f8 ? latent_scale : 1.f;
    if (f8 && H == 128 && n_hg == 1)
      launch_mla<4, 2, true>(splits, grid, s, L, idx, k, idx_q_stride, sec, bt.Q, H, split_len, sl2, os, part_o,
                             part_lse, so, sl, 1, units, tok_xcd);
    else if (f8)
      launch_mla<4, 1, true>(splits, grid, s, L, idx, k, idx_q_stride, sec, bt.Q, H, split_len, sl2, os, part_o,
                             part_lse, so, sl, n_hg, units, tok_xcd);
    else if (H == 128 && n_hg == 1)
      launch_mla<4, 2, false>(splits, grid, s, L, idx, k, idx_q_stride, sec, bt.Q, H, split_len, sl2, os, part_o,
                              part_lse, so, sl, 1, units, tok_xcd);
    else
      launch_mla<4, 1, false>(splits, grid, s, L, idx, k, idx_q_stride, sec, bt.Q, H, split_len, sl2, os, part_o,
                              part_lse, so, sl, n_hg, units, tok_xcd);
    if (splits > 1) {
      const dim3 cgrid((unsigned)(rows >= 8 ? (rows + 7) / 8 * 8 : rows) * (H / 4), (unsigned)nl), cblock(256);
      const int64_t nrm = (int64_t)units * H;
      switch (splits) {
        case 2:
          hipLaunchKernelGGL(mla_combine_kernel<2>, cgrid, cblock, 0, s, L, part_o, part_lse, H, rows, 2, so, sl, nrm);
          break;
        case 4:
          hipLaunchKernelGGL(mla_combine_kernel<4>, cgrid, cblock, 0, s, L, part_o, part_lse, H, rows, 4, so, sl, nrm);
          break;
        case 8:
          hipLaunchKernelGGL(mla_combine_kernel<8>, cgrid, cblock, 0, s, L, part_o, part_lse, H, rows, 8, so, sl, nrm);
          break;
        default:
          hipLaunchKernelGGL(mla_combine_kernel<0>, cgrid, cblock, 0, s, L, part_o, part_lse, H, rows, splits, so, sl, nrm);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_sparse_mla_layers(const HostBatch& bt, const uint16_t* const* q, int H, const HostCache* latents,
                                    const int32_t* idx, int k, int idx_q_stride, float scale, float* const* out,
                                    float* const* lse, int n_layers, void* ws, hipStream_t s) {
  return launch_layers(bt, q, H, latents, 0.f, idx, k, idx_q_stride, scale, out, lse, n_layers, ws, s);
}

hipError_t launch_sparse_mla_layers_fp8(const HostBatch& bt, const uint16_t* const* q, int H, const HostCache* latents,
                                        const float* latent_scales, const int32_t* idx, int k, int idx_q_stride,
                                        float scale, float* const* out, float* const* lse, int n_layers, void* ws,
                                        hipStream_t s) {
  // layers whose caches share a scale go together (the scale is an argument of the launch)
  for (int l0 = 0; l0 < n_layers;) {
    int l1 = l0 + 1;
    while (l1 < n_layers && latent_scales[l1] == latent_scales[l0]) ++l1;
    hipError_t e = launch_layers(bt, q + l0, H, latents + l0, latent_scales[l0], idx, k, idx_q_stride, scale, out + l0,
                                 lse ? lse + l0 : nullptr, l1 - l0, ws, s);
    if (e != hipSuccess) return e;
    l0 = l1;
  }
  return hipSuccess;
}

hipError_t launch_sparse_mla(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                             const int32_t* idx, int k, int idx_q_stride, float scale, float* out, float* lse,
                             void* ws, hipStream_t s) {
  float* lse_arr[1] = {lse};
  return launch_layers(bt, &q, H, &latent, 0.f, idx, k, idx_q_stride, scale, &out, lse ? lse_arr : nullptr, 1, ws, s);
}

hipError_t launch_sparse_mla_union(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                                   const int32_t* idx, int k, int idx_q_stride, const HostCache& latent2, int L_max2,
                                   const int32_t* idx2, int k2, int idx2_q_stride, float scale, float* out, float* lse,
                                   void* ws, hipStream_t s) {
  float* lse_arr[1] = {lse};
  const HostSecond second{latent2, idx2, k2, idx2_q_stride, L_max2};
  return launch_layers(bt, &q, H, &latent, 0.f, idx, k, idx_q_stride, scale, &out, lse ? lse_arr : nullptr, 1, ws, s,
                       k2 > 0 ? &second : nullptr);
}

hipError_t launch_sparse_mla_fp8(const HostBatch& bt, const uint16_t* q, int H, const HostCache& latent,
                                 float latent_scale, const int32_t* idx, int k, int idx_q_stride, float scale,
                                 float* out, float* lse, void* ws, hipStream_t s) {
  float* lse_arr[1] = {lse};
  return launch_layers(bt, &q, H, &latent, latent_scale, idx, k, idx_q_stride, scale, &out, lse ? lse_arr : nullptr,
                       1, ws, s);
}

}  // namespace dsa
