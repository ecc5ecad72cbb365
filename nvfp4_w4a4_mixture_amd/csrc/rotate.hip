// Offline Hadamard rotation of the hidden dimension ("[NetsPresso AQ Deep
// Dive] How to Quantize the K-EXAONE-236B Model to 4-Bit (NVFP4)", "Offline
// Fusion of Multiple Quantization Algorithms": the weights' coordinate system
// is rotated before quantization so that outliers do not pile up in one block;
// the rotation is absorbed into the weights and nothing runs at inference).
//
//   dst[r, :] = bf16_rne( ((src[r, :] * signs) . blockdiag(H_b, ..., H_b)) / sqrt(b) )
//
// H_b is the Sylvester Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n,
// -H_n]]), applied as the fast transform: log2(b) butterfly stages
// (u, v) -> (u + v, u - v) over pairs `len` apart inside aligned blocks of b.
//
// Exactness: the butterflies run in FP64.  Inputs are BF16 (8 significant
// bits) times +-1 and every stage only adds or subtracts, so each partial sum
// is exact as long as the magnitudes in a block span less than about 2^44;
// then one FP64 division by sqrt(b) (correctly rounded, as is sqrt) and one
// rounding to BF16 (through FP32 with round-to-odd, which keeps the final
// round-to-nearest-even correct) give the correctly rounded BF16 of the exact
// rotation, independent of the summation order.
//
// One workgroup per row.  The log2(b) stages are split into passes: pass 0
// takes the first r0 = ((log2(b) - 1) % 3) + 1 stages (len 1 .. 2^(r0-1)) on 8
// consecutive elements read straight from HBM (16 bytes per thread); every
// later pass takes three stages, len = S, 2S, 4S with S = 2^r0, 8 * 2^r0, ...:
// a thread holds the 8 elements whose indices differ only in the three bits of
// S, 2S and 4S, and runs the stages in registers.  Since 8S <= b divides the
// row length, those 8 indices always lie in the row.  The row meets in LDS
// between passes.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kRotMaxCols = 16384;

// LDS slot of row element i: one FP64 of padding per 32 elements, so that the
// 8-element groups of neighbouring threads do not fall on the same banks
__device__ __forceinline__ int lds_slot(int i) { return i + (i >> 5); }
constexpr int lds_doubles(int cols) { return cols + cols / 32; }

__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  float f = (float)d;  // round to nearest even
  uint32_t u = __float_as_uint(f);
  if ((double)f != d) {  // inexact: truncate toward zero and set the sticky lowest bit (round to odd)
    if (__builtin_fabs((double)f) > __builtin_fabs(d)) u -= 1u;
    u |= 1u;
  }
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// the butterfly stages of one pass over v[0..7] (element j at index base + j * stride):
// stage sb of the pass (len = stride << sb) runs when len < limit
__device__ __forceinline__ void butterflies8(double (&v)[8], int stride, int limit) {
#pragma unroll
  for (int sb = 0; sb < 3; ++sb) {
    if ((stride << sb) < limit) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if ((j & (1 << sb)) == 0) {
          const double x = v[j], y = v[j + (1 << sb)];
          v[j] = x + y;
          v[j + (1 << sb)] = x - y;
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void hadamard_rotate_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                              int cols, const float* __restrict__ signs, int b,
                                                              double sqrtb, uint16_t* __restrict__ dst,
                                                              int64_t ld_dst) {
  extern __shared__ double row[];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* s = src + r * ld_src;
  const int groups = cols / 8;  // 8-element groups per pass
  const int log2b = 31 - __builtin_clz((unsigned)b);
  const int first = 1 << ((log2b - 1) % 3 + 1);  // pass 0 runs the stages with len < first
  // pass 0: stages len 1 .. first/2 on 8 consecutive elements loaded from HBM
  for (int m = tid; m < groups; m += 256) {
    const int c = 8 * m;
    const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(s + c);
    double v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = (double)__uint_as_float(raw[j] << 16);
      v[2 * j + 1] = (double)__uint_as_float(raw[j] & 0xFFFF0000u);
    }
    if (signs != nullptr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] *= (double)signs[c + j];
    }
    butterflies8(v, 1, first);
#pragma unroll
    for (int j = 0; j < 8; ++j) row[lds_slot(c + j)] = v[j];
  }
  // later passes: element j of group m sits at base(m) + j * stride, base(m) = m with 3 zero
  // bits inserted at bit log2(stride)
  for (int stride = first; stride < b; stride *= 8) {
    __syncthreads();
    for (int m = tid; m < groups; m += 256) {
      const int lo = m & (stride - 1);
      const int base = ((m - lo) << 3) | lo;
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = row[lds_slot(base + j * stride)];
      butterflies8(v, stride, b);
#pragma unroll
      for (int j = 0; j < 8; ++j) row[lds_slot(base + j * stride)] = v[j];
    }
  }
  __syncthreads();
  uint16_t* d = dst + r * ld_dst;
  for (int m = tid; m < groups; m += 256) {
    const int c = 8 * m;
    u32x4_t o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = f64_to_bf16_rne(row[lds_slot(c + 2 * j)] / sqrtb) |
             (f64_to_bf16_rne(row[lds_slot(c + 2 * j + 1)] / sqrtb) << 16);
    *reinterpret_cast<u32x4_t*>(d + c) = o;
  }
}

hipError_t launch_hadamard_rotate(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld_src, const float* signs,
                                  int64_t b, uint16_t* dst, int64_t ld_dst, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&hadamard_rotate_kernel),
                                         lds_doubles(kRotMaxCols) * (int)sizeof(double)))
    return e;
  const size_t lds = (size_t)lds_doubles((int)cols) * sizeof(double);
  hipLaunchKernelGGL(hadamard_rotate_kernel, dim3((unsigned)rows), dim3(256), lds, st, src,
                     ld_src, (int)cols, signs, (int)b, __builtin_sqrt((double)b), dst, ld_dst);
  return hipGetLastError();
}

int64_t hadamard_max_cols() { return kRotMaxCols; }

}  // namespace moe
