// Device helpers shared by the gfx950 kernels: vector types, storage-dtype
// traits, MFMA wrappers and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kHeadDim = 128;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// 2^x on the transcendental unit (exact 0 for -inf).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) for x >= 1 (the only arguments used here: a running sum whose
// largest term is exp2(0) = 1).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Logit soft cap of a raw score s: cap_out * tanh(y), y = s * cap_in / (2 log2 e),
// with tanh(y) = 1 - 2 / (2^(2 y log2 e) + 1). Saturates to +-cap_out (2^x
// gives inf or 0); the absolute error of the tanh is a few ulp of 1.
__device__ __forceinline__ float soft_cap(float s, float cap_in, float cap_out) {
  const float e = fast_exp2(s * cap_in);
  return fmaf(-2.f * cap_out, __builtin_amdgcn_rcpf(e + 1.f), cap_out);
}

__device__ __forceinline__ u32x4 load_16B(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 load_16B_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Raw buffer resource over [base, base + num_bytes): loads at byte offsets
// at or past num_bytes return zero (the hardware range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num_bytes, 0x00020000);
}
// Cache policy of a buffer load (gfx950 encoding of the instruction's sc0 /
// nt / sc1 bits): kStream marks data read once (non-temporal), so a streamed
// KV cache does not displace reused data in the L2 and the Infinity Cache.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;
template <int POLICY = kCacheDefault>
__device__ __forceinline__ u32x4 buffer_load_16B(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, POLICY));
}

// ---------------------------------------------------------------------------
// storage dtypes
// ---------------------------------------------------------------------------
struct F16 {
  using elem = _Float16;
  static __device__ __forceinline__ f32x8 to_f32(u32x4 v) {
    return __builtin_convertvector(__builtin_bit_cast(f16x8, v), f32x8);
  }
  // Round-to-nearest-even fp32 -> fp16.
  static __device__ __forceinline__ elem from_f32(float x) { return static_cast<_Float16>(x); }
  // Two fp32 values rounded (nearest even) and packed, first in the low half.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
  }
  // acc + (sum of the two packed values), exact products, fp32 accumulate.
  static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed),
                                  f16x2{static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)},
                                  acc, false);
  }
  static __device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

struct BF16 {
  using elem = __bf16;
  static __device__ __forceinline__ f32x8 to_f32(u32x4 v) {
    f32x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = __uint_as_float(v[i] << 16);
      r[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
    return r;
  }
  // Round-to-nearest-even fp32 -> bf16.
  static __device__ __forceinline__ elem from_f32(float x) { return static_cast<__bf16>(x); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
  }
  static __device__ __forceinline__ float add_pair(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                           bf16x2{static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)},
                                           acc, false);
  }
  static __device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};

// Output element conversion (final outputs may be the storage dtype or fp32).
template <class OUT>
__device__ __forceinline__ OUT out_cast(float x) {
  return static_cast<OUT>(x);
}

// ---------------------------------------------------------------------------
// wave-level reductions across the four 16-lane rows (lanes l, l^16, l^32, l^48)
// v_permlane16_swap / v_permlane32_swap with both operands equal yield, in
// their two results, the lane's own value and its partner's (l^16 / l^32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_across_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_rows(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Same across the two 32-lane halves only (lanes l, l^32).
__device__ __forceinline__ float max_across_halves(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Across all 64 lanes (butterfly order: the same bits on every run).
__device__ __forceinline__ float wave_reduce_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_reduce_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Row mapping of a planned group to output rows: decode rows are the G query
// heads of one request; prefill rows are GQA-packed (row r of a request is
// query token r / G, head g*G + r % G).
struct RowMap {
  int32_t num_qo_heads;
  int32_t group;   // G
  bool prefill;
  // Returns the output row index (token_row * Hq + head) or -1 if the row is padding.
  __device__ __forceinline__ int64_t out_row(const int32_t* qo_indptr, int b, int tile, int g,
                                             int r, int rows_per_tile) const {
    if (!prefill) {
      if (r >= group) return -1;
      return static_cast<int64_t>(b) * num_qo_heads + g * group + r;
    }
    const int q0 = qo_indptr[b], q1 = qo_indptr[b + 1];
    const int packed = tile * rows_per_tile + r;
    if (packed >= (q1 - q0) * group) return -1;
    const int tok = packed / group, hh = packed - tok * group;
    return static_cast<int64_t>(q0 + tok) * num_qo_heads + g * group + hh;
  }
};

}  // namespace pkv
