// Device-side helpers shared by the DSA kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kDi = 128;     // indexer head dim (bytes per e4m3 key row)
constexpr int kDqk = 576;    // latent row: 512 latent + 64 RoPE
constexpr int kDv = 512;     // value = first 512 dims of the latent row
constexpr int kMaxK = 2048;

// Row address of token t of sequence b in a token-major cache (contiguous or paged).
struct CacheView {
  const uint8_t* base;
  const int32_t* table;
  int max_pages, page_size;
  int64_t row_bytes;
  int L_max;
  __device__ __forceinline__ const uint8_t* row(int b, int t) const {
    if (table == nullptr) return base + ((int64_t)b * L_max + t) * row_bytes;
    int page = table[(int64_t)b * max_pages + t / page_size];
    return base + ((int64_t)page * page_size + (t % page_size)) * row_bytes;
  }
};

// Position of query token j of sequence b; in_Q = query tokens per sequence in the inputs.
__device__ __forceinline__ int query_pos(const int32_t* seq_lens, const int32_t* q_pos, int in_Q, int b, int j) {
  return q_pos ? q_pos[b * in_Q + j] : seq_lens[b] - in_Q + j;
}

// 16x16x128 FP8(E4M3) x FP8(E4M3) -> fp32 matrix-core product, accumulating into c.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, 32 bytes each; the two
// operands must use the same byte order along K. c[r] = C[4*(l/16) + r][l % 16].
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 matrix-core product: lane l supplies 8 bf16 of row (l % 16) of A and of
// column (l % 16) of B with one shared K order; c[r] = C[4*(l/16) + r][l % 16].
__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// All-reduce of x over the lane pairs (l, l ^ 16) and (l, l ^ 32) with gfx950's lane swaps
// (VALU, no LDS round trip). permlane16_swap(x, x) returns ([x0, x0, x2, x2], [x1, x1, x3, x3])
// in 16-lane rows, permlane32_swap(x, x) returns ([x.lo, x.lo], [x.hi, x.hi]); combining the
// two results of a swap pairs every lane with its partner. The operation is applied to the
// same two operands in every lane, so both lanes of a pair hold the identical result.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(x, 0) as one integer max on the bit pattern: every negative float (sign bit set) is a
// negative int32 and maps to +0; non-negative floats are unchanged. Unlike fmaxf it needs no
// NaN-quieting instruction in front.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Order-preserving map of an IEEE float to uint32 (larger float -> larger key); -0 -> +0.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Four consecutive fp32 values from i0 (a multiple of 4) of a row with `lim` >= 1 readable
// entries. With VEC the row starts 16-byte aligned inside an allocation that is a multiple of 4
// entries long, so the aligned vector holding entry lim - 1 is readable. The address is clamped
// into the row instead of guarded by a branch: a branch around each load makes the compiler wait
// at the join for every load before it, while clamped loads issue back to back. Entries at or
// past lim hold some in-row value; the caller masks them.
// NT: a nontemporal load (for passes that read each score once).
template <bool VEC, bool NT = false>
__device__ __forceinline__ float4 load4_clamped(const float* __restrict__ row, int i0, int lim) {
  if (VEC && NT) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 v = __builtin_nontemporal_load((const f4*)(row + min(i0, (lim - 1) & ~3)));
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  if (VEC) return *(const float4*)(row + min(i0, (lim - 1) & ~3));
  float4 x;
  x.x = row[min(i0 + 0, lim - 1)];
  x.y = row[min(i0 + 1, lim - 1)];
  x.z = row[min(i0 + 2, lim - 1)];
  x.w = row[min(i0 + 3, lim - 1)];
  return x;
}

// Wave-inclusive scans by DPP: row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast 15
// and 31 carry the row totals across rows (lanes shifted in from outside a row read `id`).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, CTRL, ROWMASK, 0xf, false);
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp_u32<0x111, 0xf>(x, id));
  x = op(x, dpp_u32<0x112, 0xf>(x, id));
  x = op(x, dpp_u32<0x114, 0xf>(x, id));
  x = op(x, dpp_u32<0x118, 0xf>(x, id));
  x = op(x, dpp_u32<0x142, 0xa>(x, id));
  x = op(x, dpp_u32<0x143, 0xc>(x, id));
  return x;
}

}  // namespace dsa
