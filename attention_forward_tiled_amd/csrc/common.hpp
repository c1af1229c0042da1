// Device-side building blocks shared by the gfx950 attention kernels.
//
// MFMA lane layouts used throughout (checked on an MI355X with an in-bounds probe
// against a CPU matmul; both 16-bit input types behave the same):
//   v_mfma_f32_16x16x32_{f16,bf16}  C[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[l % 16][8*(l/16) + j], j = 0..7   (8 halves per lane)
//     B: lane l holds B[8*(l/16) + j][l % 16], j = 0..7
//     C: lane l holds C[4*(l/16) + i][l % 16], i = 0..3   (4 floats per lane)
//   v_mfma_f32_16x16x16_{f16,bf16}  C[16x16] += A[16x16] * B[16x16]
//     A: lane l holds A[l % 16][4*(l/16) + j], j = 0..3;  B: lane l holds B[4*(l/16) + j][l % 16]
//     C: as for 16x16x32
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
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
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
  // v_mfma_f32_16x16x16_f16 on four 16-bit values per lane held in two dwords.
  static __device__ __forceinline__ float4v mfma16k(const u32x2& a, const u32x2& b, const float4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4, a), __builtin_bit_cast(half4, b), c,
                                                0, 0, 0);
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
  // v_mfma_f32_16x16x16_bf16 on four 16-bit values per lane held in two dwords.
  static __device__ __forceinline__ float4v mfma16k(const u32x2& a, const u32x2& b, const float4v& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a),
                                                    __builtin_bit_cast(short4v, b), c, 0, 0, 0);
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

// fp32 -> bf16 bit pattern rounded to nearest with ties away from zero (mode 1) or
// toward zero (mode 2): add half a bf16 unit to the magnitude (mode 1) and truncate.
// NaN stays a quiet NaN; the magnitude add cannot carry into the sign bit.
__device__ __forceinline__ uint32_t bf16_bits_directed(float x, int mode) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return (u >> 16) | 0x0040u;
  return ((u & 0x80000000u) | (mode == 1 ? mag + 0x8000u : mag)) >> 16;
}

// Two fp32 values -> two bf16 in one dword (lo first) with output rounding `mode`
// (0 to nearest even, the hardware conversion; 1 ties away from zero; 2 toward zero).
__device__ __forceinline__ uint32_t pack_bf16_round(float lo, float hi, int mode) {
  if (mode == 0) return Op<BF16>::pack(lo, hi);
  return bf16_bits_directed(lo, mode) | (bf16_bits_directed(hi, mode) << 16);
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

constexpr unsigned kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters untouched

// s_waitcnt immediate that waits until at most n vector-memory operations are outstanding
// (vmcnt is split over bits 3:0 and 15:14 of the immediate).
constexpr unsigned wait_vm(unsigned n) { return kWaitVm0 | (n & 15u) | ((n >> 4) << 14); }

// 16 bytes of zeros in global memory: the source of every LDS row past a key length.
static __device__ __align__(16) const uint16_t kZeroChunk[8] = {0, 0, 0, 0, 0, 0, 0, 0};

// Byte address of a shared-memory location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)(p);
}

// Debug builds: fill BYTES of LDS with all-ones words (NaN as fp16, bf16 and fp32) and
// wait for every thread, before the kernel's first copy into LDS.
template <int BYTES>
__device__ __forceinline__ void poison_lds(void* lds) {
  uint32_t* w = static_cast<uint32_t*>(lds);
  for (int i = threadIdx.x; i < BYTES / 4; i += blockDim.x) w[i] = 0xFFFFFFFFu;
  __syncthreads();
}

// global_load_lds_dwordx4 with a per-lane 64-bit address: lane l's 16 bytes land at LDS
// byte lds + 16 * l. Issued from inline asm so that the compiler does not fence LDS reads
// of the other stage on it; completion is awaited explicitly (vmcnt) before the barrier
// that publishes the stage.
// Invariant: the asm sets m0 (the copy's LDS base) behind the compiler's back, since the
// compiler reserves m0 and cannot take it as a clobber. This is correct only while the
// generated code itself keeps nothing in m0 (no register-indexed moves, messages or GWS
// operations in these kernels). The build checks the gfx950 assembly of every source and
// fails if m0 appears anywhere but in the s_mov_b32 m0 / s_nop 0 / global_load_lds_dwordx4
// sequence below; the per-launch-form parity tests guard the copies' results.
// NT marks the load non-temporal: for data read once (the decode's K/V pages) it keeps
// the stream from displacing reusable lines in the caches, and the decode stream runs
// about 12% faster with it; the prefill's K/V tiles are re-read by other workgroups
// through L2 and keep the default policy.
template <bool NT = false>
__device__ __forceinline__ void dma16_v(const uint16_t* g, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// Same copy with a wave-uniform base in SGPRs and a per-lane 32-bit byte offset.
template <bool NT = false>
__device__ __forceinline__ void dma16_s(const uint16_t* base, uint32_t voff, uint32_t lds) {
  // readfirstlane returns a signed int: widen through uint32_t so the low word is not
  // sign-extended into the high one.
  const uint64_t b = (uint64_t)base;
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint64_t bs = ((uint64_t)hi << 32) | (uint64_t)lo;
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :: "v"(voff), "s"((const uint16_t*)bs), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
  else
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"((const uint16_t*)bs), "s"(__builtin_amdgcn_readfirstlane(lds))
                 : "memory");
}

// Read-only device int through the constant address space, so it becomes a scalar load.
__device__ __forceinline__ int scalar_load(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace attn
