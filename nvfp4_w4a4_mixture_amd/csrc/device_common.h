// Device helpers shared by the gfx950 kernels: NVFP4 element encoders, the
// exact FP4 x E4M3 -> FP16 decode that feeds the 16-bit MFMA, and small
// wave-level utilities.
//
// Format facts used here ("K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card,
// "Quantization Setup": FP4 E2M1 values, group 16, FP8 E4M3 block scales):
//   E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7, bit 3 = sign);
//   E4M3-FN value 2^(e-7) * (1 + m/8), subnormal 2^-6 * m/8, max 448 (0x7E).
// A decoded element code * S has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in FP16 (normal range); the product of two
// decoded elements is exact in FP32, and the MFMA accumulates in FP32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace moe {

constexpr float kE2M1Max = 6.0f;
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// E4M3-FN round-to-nearest-even of a non-negative float, saturating at 448.
// Normal range: round the float32 mantissa to 3 bits in integer arithmetic
// (carry into the exponent is the correct rounding).  Below 2^-6 the E4M3
// grid is uniform with step 2^-9, so the code is rint(s * 512) (ties to even),
// and 8 there is the smallest normal code 0x08, which is also correct.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float s) {
  if (!(s < kE4M3Max)) return 0x7Eu;  // >= 448, +inf
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);
  uint32_t b = __float_as_uint(s);
  uint32_t t = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;  // biased exp << 3 | mant3, rounded
  uint32_t code = t - ((127u - 7u) << 3);
  return code > 0x7Eu ? 0x7Eu : code;
}

// Value of an E4M3 byte with sign bit 0 (block scales are never negative).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Eight E2M1 codes of v[0..7] in one dword (element 2j in the low nibble of
// byte j): round to nearest even on the value set {0, 0.5, 1, 1.5, 2, 3, 4,
// 6}, saturating at 6, sign from the sign bit of v (so a small negative value
// gives -0).  At a boundary the tie goes to the even code: 0.25 -> 0,
// 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0.
// As comparisons on a = |v|, the code magnitude is (a > 0.25) + (a >= 0.75) +
// (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5).  The hardware
// convert with scale 1.0 implements exactly this rule: it was compared with
// that expression on the device, in both operand slots, for every non-NaN
// float32.  The byte selector must be a literal, hence the four calls.
__device__ __forceinline__ uint32_t e2m1_encode8(const float* v) {
  uint32_t d = 0u;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[0], v[1], 1.0f, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[2], v[3], 1.0f, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[4], v[5], 1.0f, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[6], v[7], 1.0f, 3);
  return d;
}

// Quantize one block of 16 floats against global scale gs.  Returns the E4M3
// scale byte; writes 8 packed code bytes (element 2j in the low nibble) into
// lo (bytes 0..3) and hi (bytes 4..7).  Every step is one IEEE float32
// operation in the order s = (amax / 6) * gs, inv = gs / S, v = x * inv.
__device__ __forceinline__ uint32_t quantize_block16(const float* x, float gs, uint32_t& lo, uint32_t& hi) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(x[i]));
  float s = amax / kE2M1Max;
  s = s * gs;
  uint32_t sc = e4m3_encode_nonneg(s);
  float sd = e4m3_to_f32(sc);
  lo = 0;
  hi = 0;
  if (sd != 0.0f) {
    float inv = gs / sd;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = x[i] * inv;
    lo = e2m1_encode8(v);
    hi = e2m1_encode8(v + 8);
  }
  return sc;
}

// Decode 8 packed E2M1 codes (one dword, element 0 in bits 3:0) times the
// block scale S (given as FP16, exact) into 8 FP16 values for an MFMA
// operand.  The scaled convert applies only the exponent of its scale
// operand, so it converts with scale 1 and an exact packed FP16 multiply
// applies the full E4M3 value.
__device__ __forceinline__ half8_t decode8(uint32_t codes, half2_t s2) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// {S, S} in FP16 for byte k of a dword of four E4M3 scale bytes.  The FP8
// convert turns two E4M3 bytes into two FP16 values exactly (every E4M3 value,
// subnormals included, is an FP16 value; byte 0 -> low half, checked for all
// 127 finite codes on the device), and the broadcast of one half folds into the
// op_sel of the multiply that consumes it, so the four scales of a dword cost
// two converts.
__device__ __forceinline__ half2_t scale_pair(uint32_t scales4, int k) {
  const half2_t two = k >= 2 ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scales4, 1.0f, true)
                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(scales4, 1.0f, false);
  return (k & 1) ? two.yy : two.xx;
}

// silu(g) = g / (1 + e^-g) from the hardware base-2 exponential and reciprocal
// (about 1 ulp each); for very negative g, 2^x overflows to +inf and the
// result is -0.
__device__ __forceinline__ float silu(float g) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

// Pair rows are stored as FP16 values times a power of two 2^E per row, with E
// from a bound on |w_p f| that no operands can exceed: a decoded element
// (code times E4M3 scale) is at most 6 * 448 = 2688 in magnitude, so an FP32
// accumulator over K products is at most K * 2688^2 (to within its rounding)
// and |w_p f| <= |w_p| * K * 2688^2 * alpha.  E = floor(log2(bound)) - 14
// keeps every stored value below 2^15, inside FP16's finite range (largest
// 65504).  A loose bound costs no precision: FP16 keeps 11 significant bits
// over its normal range, which reaches 29 binades below 2^15.  E is clamped to
// [-126, 113], so that 2^E and 2^-E are normal floats; a finite bound never
// reaches the upper end, and below the lower one the values are too small to
// reach 2^15.  Returns 2^-E, the factor applied before the FP16 rounding, and
// sets scale = 2^E, the row's scale.
__device__ __forceinline__ float pair_row_scale(float wp, int64_t K, float alpha, float& scale) {
  const float bound = fabsf(wp) * ((float)K * 7225344.0f) * alpha;  // 2688^2 = 7225344
  const int eb = (int)((__float_as_uint(bound) >> 23) & 255u) - 127;  // floor(log2(bound)) when bound is normal
  const int E = min(max(eb - 14, -126), 113);
  scale = __uint_as_float((uint32_t)(127 + E) << 23);
  return __uint_as_float((uint32_t)(127 - E) << 23);
}

// Weight block scales are stored tiled: the 16 x 8 scale bytes of 16
// consecutive rows and 128 consecutive columns form one 128-byte block
// (row-major inside), blocks ordered by column within a 16-row tile and tiles
// by row.  Byte of (row, scale block b = column / 16) for K columns:
__host__ __device__ __forceinline__ int64_t tiled_scale_index(int64_t row, int64_t b, int64_t K) {
  return (row >> 4) * K + (b >> 3) * 128 + (row & 15) * 8 + (b & 7);
}

// global -> LDS DMA of 16 (4) bytes per lane: lane l's bytes land at lds + 16 l (4 l);
// lds must be wave-uniform
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

__device__ __forceinline__ void dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((glb_void_t*)g, (lds_void_t*)lds, 4, 0, 0);
}

// The same DMAs written as inline asm, in the SGPR-base form (wave-uniform
// 64-bit base, 32-bit lane offset).  The compiler then does not count them as
// outstanding LDS writes, so the LDS reads it issues itself get no blanket
// vmcnt(0); the caller orders every read of a DMA'd buffer with its own vmcnt
// wait and a barrier.  The instruction has no destination register (it
// writes LDS at M0 + 16 * lane, or 4 * lane), and M0 is declared as an output
// so the compiler knows the asm redefines it.  lds and sbase must be
// wave-uniform.
__device__ __forceinline__ void dma16_async(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t m0;
  asm volatile("s_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2"
               : "={m0}"(m0)
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4_async(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t m0;
  asm volatile("s_mov_b32 m0, %3\n\tglobal_load_lds_dword %1, %2"
               : "={m0}"(m0)
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory");
}

// Every LDS access this wave has issued has completed; then the workgroup barrier.
__device__ __forceinline__ void barrier_after_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N), leaving the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace moe
