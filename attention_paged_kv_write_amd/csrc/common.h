// Device helpers shared by the kernels of the paged-attention library (gfx950).
//
// Wave64 throughout.  Cross-lane reductions use DPP inside a 16-lane row
// (quad_perm, row_half_mirror, row_mirror), ds_swizzle across the two rows of
// a 32-lane half, and ds_bpermute between the two halves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// Lazy rescaling: a softmax row keeps its running max until a tile's max
// exceeds it by more than this (log2 units), so unnormalised probabilities stay
// below 2^8; the result is unchanged (numerator and denominator share the max).
constexpr float kRescaleSlack = 8.f;

// ---------------------------------------------------------------------------
// bf16 <-> f32 on raw bit patterns
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// ---------------------------------------------------------------------------
// Cross-lane exchange
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                         CTRL, 0xf, 0xf, false));
}

// DPP controls (GFX9 encoding).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within 16

// Lane i <- lane i ^ 16 (inside each 32-lane half): ds_swizzle bit mode,
// and_mask 0x1f, or_mask 0, xor_mask 0x10.
__device__ __forceinline__ float swz_xor16(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

// Lane i <- lane i ^ 32.
__device__ __forceinline__ float xchg_xor32(float x) {
  const int src = (__lane_id() ^ 32) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, x)));
}

// Lane i <- lane i ^ m for any m in {1,...,32} (epilogue use).
__device__ __forceinline__ float xchg_xor(float x, int m) {
  const int src = (__lane_id() ^ m) << 2;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, x)));
}

struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// All-reduce over groups of W consecutive lanes (W in 1,2,4,8,16,32,64).
template <int W, class Op>
__device__ __forceinline__ float group_allreduce(float x, Op op) {
  if constexpr (W >= 2) x = op(x, dpp_f32<kDppXor1>(x));
  if constexpr (W >= 4) x = op(x, dpp_f32<kDppXor2>(x));
  if constexpr (W >= 8) x = op(x, dpp_f32<kDppRowHalfMirror>(x));
  if constexpr (W >= 16) x = op(x, dpp_f32<kDppRowMirror>(x));
  if constexpr (W >= 32) x = op(x, swz_xor16(x));
  if constexpr (W >= 64) x = op(x, xchg_xor32(x));
  return x;
}

// All-reduce across the four 16-lane rows (lanes l, l^16, l^32, l^48).
template <class Op>
__device__ __forceinline__ float across_rows(float x, Op op) {
  x = op(x, swz_xor16(x));
  x = op(x, xchg_xor32(x));
  return x;
}

// max(a, b, c) as one v_max3_f32, without the NaN-quieting copies the
// compiler puts in front of fmaxf on matrix-core results.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return fmaxf(a, fmaxf(b, c));
#endif
}

// Max over lanes l, l^16, l^32, l^48 (the four key quarters of a query column).
__device__ __forceinline__ float quarter_max(float x) {
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = vmax3(__uint_as_float(p16[0]), __uint_as_float(p16[1]), __uint_as_float(p16[1]));
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return vmax3(__uint_as_float(p32[0]), __uint_as_float(p32[1]), __uint_as_float(p32[1]));
}

// exp2 that treats a -inf argument exactly (hardware v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// 16 bytes per lane straight from global memory into LDS (no VGPRs): lane l's
// bytes land at lds_base + 16*l; lds_base must be wave-uniform.  Completion is
// counted by vmcnt.  (A plain device function: called inside a lambda, the
// builtin would also be instantiated for the host, where it does not exist.)
// AUX is the cache-policy immediate (2: non-temporal, for data read once).
template <int AUX = 0>
__device__ __forceinline__ void global_to_lds16(const void* src, void* lds_base) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  typedef __attribute__((address_space(1))) void* gbl_ptr;
  __builtin_amdgcn_global_load_lds((gbl_ptr)src, (lds_ptr)lds_base, 16, 0, AUX);
}

// 32-bit LDS byte address of a __shared__ object (for inline-asm DS operands).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const void* lds_cptr;
  return static_cast<uint32_t>((uintptr_t)((lds_cptr)p));
}

// ---------------------------------------------------------------------------
// Division by a per-pool scale s, correctly rounded.  The steps are those the
// compiler emits for an IEEE fp32 division (a reciprocal refined once, then
// two residual corrections), with the reciprocal built once per scale and
// without the operand scaling and result fix-up steps, which change nothing
// while |s| lies in [2^-30, 2^30] and the quotient is a normal number below
// 2^20.  A larger first product (an infinite numerator, an overflowing
// quotient) is kept as it is: the +-448 clamp that follows saturates it the
// same way.  The sign is taken from the first product, so a zero keeps its
// sign.  Other scales divide.
// ---------------------------------------------------------------------------
struct ScaleRcp {
  float s, r;
  bool fast;
};

__device__ __forceinline__ ScaleRcp scale_rcp(float s) {
  const float a = fabsf(s);
  const float r0 = __builtin_amdgcn_rcpf(s);
  return ScaleRcp{s, fmaf(fmaf(-s, r0, 1.f), r0, r0), a >= 0x1p-30f && a <= 0x1p30f};
}

__device__ __forceinline__ float div_by_scale(float x, const ScaleRcp& sr) {
  const float q0 = x * sr.r;
  float q = fmaf(fmaf(-sr.s, q0, x), sr.r, q0);
  q = fmaf(fmaf(-sr.s, q, x), sr.r, q);
  q = fabsf(q0) > 1.0e6f ? q0 : q;
  return copysignf(q, q0);
}

// ---------------------------------------------------------------------------
// E4M3 (OCP FP8) codes of 16 floats: the code nearest to x / scale (the
// correctly rounded fp32 quotient), ties to even.  The hardware convert rounds
// that way but turns magnitudes from 464 up into NaN, so the quotient is
// clamped to +-448 first (saturation); a NaN quotient becomes code 0x7F.  Byte
// i of the result holds element i.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 e4m3_codes16(const float* q16) {
  u32x4 out;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float y[4];
    uint32_t nan_mask = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float q = q16[4 * d + i];
      nan_mask |= (q != q) ? (0xFFu << (8 * i)) : 0u;
      y[i] = fminf(fmaxf(q, -448.f), 448.f);
    }
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
    out[d] = (static_cast<uint32_t>(r) & ~nan_mask) | (0x7F7F7F7Fu & nan_mask);
  }
  return out;
}

__device__ __forceinline__ u32x4 quantize16_e4m3(const float* x, const ScaleRcp& sr) {
  float q[16];
  if (sr.fast) {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = div_by_scale(x[i], sr);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = x[i] / sr.s;
  }
  return e4m3_codes16(q);
}

__device__ __forceinline__ u32x4 quantize16_e4m3(const float* x, float scale) {
  return quantize16_e4m3(x, scale_rcp(scale));
}

}  // namespace pa
