// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA lane layouts used throughout (checked on an MI355X with an in-bounds probe
// against a CPU matmul; both 16-bit input types behave the same):
//   v_mfma_f32_16x16x32_{f16,bf16}  C[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l % 16][8*(l/16) + j], j = 0..7   (8 halves per lane)
//     B: lane l holds B[8*(l/16) + j][l % 16], j = 0..7
//     C: lane l holds C[4*(l/16) + i][l % 16], i = 0..3   (4 floats per lane)
//   v_mfma_f32_32x32x16_{f16,bf16}  C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[l % 32][8*(l/32) + j], j = 0..7
//     B: lane l holds B[8*(l/32) + j][l % 32], j = 0..7
//     C: lane l holds C[8*g + 4*(l/32) + i][l % 32] at element 4*g + i, g, i = 0..3
// The reduction index k only has to be enumerated the same way in A and B, so the
// kernels are free to permute it consistently (the P.V product relies on this).
//
// ds_read_b64_tr_b16 (LDS transpose read): inside each group of 16 lanes, lane r
// receives element (r % 4) of the 8-byte words addressed by lanes r/4, r/4 + 4,
// r/4 + 8 and r/4 + 12 of the group, in that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short2v __attribute__((ext_vector_type(2)));

constexpr int kPage = 64;          // tokens per KV page == KV tile width T
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct F16 {};
struct BF16 {};

// Eight 16-bit values reinterpreted as the MFMA operand type of the storage dtype.
template <typename T> struct Op;
template <> struct Op<F16> {
  typedef half8 vec;
  static __device__ __forceinline__ float4v mfma(const vec& a, const vec& b, const float4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float16v mfma32(const vec& a, const vec& b, const float16v& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // Round-to-nearest-even fp32 -> fp16 (v_cvt_f16_f32 under the default rounding mode).
  static __device__ __forceinline__ uint16_t from_float(float x) {
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  static __device__ __forceinline__ float to_float(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  // Two floats -> two fp16 (round to nearest even) in one dword, lo first (v_cvt_pk_f16_f32).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, half2v));
  }
  // acc + lo + hi of a packed pair, accumulated in fp32 (v_dot2c_f32_f16 against (1, 1)).
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, pair), half2v{1, 1}, acc, false);
  }
};
template <> struct Op<BF16> {
  typedef bf16x8 vec;
  static __device__ __forceinline__ float4v mfma(const vec& a, const vec& b, const float4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float16v mfma32(const vec& a, const vec& b, const float16v& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Round-to-nearest-even fp32 -> bf16 (gfx950 converts natively).
  static __device__ __forceinline__ uint16_t from_float(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
  static __device__ __forceinline__ float to_float(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
  // Two floats -> two bf16 (round to nearest even) in one dword, lo first (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2v{lo, hi}, bf16x2));
  }
  // acc + lo + hi of a packed pair, accumulated in fp32 (v_dot2c_f32_bf16 against (1, 1)).
  static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(short2v, pair),
                                          short2v{0x3F80, 0x3F80}, acc, false);
  }
};

template <typename T>
__device__ __forceinline__ typename Op<T>::vec as_op(const u32x4& r) {
  return __builtin_bit_cast(typename Op<T>::vec, r);
}

// Pack two floats into one dword of two 16-bit values (lo first), round to nearest even.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return Op<T>::pack(lo, hi);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// Max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows of a wave).
__device__ __forceinline__ float rows4_max(float x) { return wave_max_xor(wave_max_xor(x, 16), 32); }
__device__ __forceinline__ float rows4_sum(float x) { return wave_sum_xor(wave_sum_xor(x, 16), 32); }

// LDS transpose read of four 16-bit values (see the header comment).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  short4v r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) short4v*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace attn
