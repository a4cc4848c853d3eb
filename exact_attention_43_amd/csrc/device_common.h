// Device-side helpers shared by the exattn kernels (gfx950 / CDNA4, wave64).
//
// Data move as raw 16-bit patterns in 16-byte vectors; they are reinterpreted as
// bf16x8 / f16x8 only at the MFMA call.  Accumulation is fp32 throughout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Element-type traits: MFMA on the 16-bit type, and the packed fp32 -> 16-bit
// conversion (round to nearest even; v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // 16x16x16: A lane l holds A[l%16][4(l/16)..+3], B lane l holds B[4(l/16)..+3][l%16].
  static __device__ __forceinline__ f32x4_t mfma16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
};

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x16_t mfma32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t mfma16x16x16(u32x2_t a, u32x2_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
};

// 2^x on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 on the hardware unit (v_log_f32).
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// tanh(y) = 1 - 2 / (exp(2y) + 1), with exp(2y) = 2^(2 y log2 e).  Saturates to
// +-1 (exp2 overflows to +inf or underflows to 0) instead of producing NaN.
__device__ __forceinline__ float tanh_exp2(float y) {
  float e = fast_exp2(y * (2.0f * kLog2e));
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// LDS transposing read (ds_read_b64_tr_b16): within each group of 16 lanes,
// output lane i element t is element (i & 3) of the 4 16-bit values that
// source lane (i >> 2) + 4 t addresses (8 bytes per lane).
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint8_t* lds) {
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)lds));
}

// Touch every 64-byte line of the kernel-argument block in one batch of scalar
// loads and wait once.  The compiler loads argument fields when first used,
// and the first use of each line would otherwise cost its own dependent round
// trip to memory before the kernel's first loads can go out.
template <int BYTES>
__device__ __forceinline__ void prefetch_kernargs() {
  const __attribute__((address_space(4))) uint32_t* ka =
      (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t acc = ka[BYTES / 4 - 1];
#pragma unroll
  for (int o = 0; o < BYTES; o += 64) acc ^= ka[o / 4];
  asm volatile("" ::"s"(acc));
}

// Swap values between the two 32-lane halves of the wave (lane i <-> lane i ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }

// Order this wave's LDS writes before its following LDS reads of other lanes'
// data (LDS operations of one wave complete in issue order once counted down).
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Transpose helper: from four 16-byte rows (8 x 16-bit each) take column t of
// every row and return those four 16-bit values packed (row 0 in the low half
// of the first word).  One v_perm_b32 per output word.
__device__ __forceinline__ u32x2_t column4(const u32x4_t& r0, const u32x4_t& r1,
                                           const u32x4_t& r2, const u32x4_t& r3, int t) {
  const int w = t >> 1;
  // v_perm_b32(s0, s1, sel): selector bytes 0-3 pick bytes of s1, 4-7 bytes of s0.
  const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
  u32x2_t out;
  out[0] = __builtin_amdgcn_perm(r1[w], r0[w], sel);
  out[1] = __builtin_amdgcn_perm(r3[w], r2[w], sel);
  return out;
}

}  // namespace exattn
