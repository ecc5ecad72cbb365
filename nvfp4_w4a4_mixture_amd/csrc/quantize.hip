// NVFP4 quantization kernels ("K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card,
// "Quantization Setup": E2M1 codes, one E4M3 scale per 16 elements, FP32
// global scale; activations dynamic against a calibrated global scale,
// weights round-to-nearest per expert Linear).
//
// One thread quantizes one 16-element block: it reads 32 contiguous bytes of
// BF16, writes 8 bytes of codes and 1 scale byte.  Activation scales are
// row-major [rows, cols/16]; weight scales go to the tiled layout the expert
// kernels read (16 rows x 128 columns = one 128-byte block, see
// tiled_scale_index).  Consecutive threads take
// consecutive blocks of a row, so a wave reads 2 KiB and writes 512 B + 64 B
// contiguously: the kernel streams HBM at its roofline (2.5625 B/element).
#include "device_common.h"
#include "launch.h"

namespace moe {

__global__ __launch_bounds__(256) void quantize_bf16_kernel(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t blocks_per_row, int64_t ld,
                                                            const float* __restrict__ gs, int64_t rows_per_gs,
                                                            uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                            int tiled) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= rows * blocks_per_row) return;
  const int64_t r = b / blocks_per_row;
  const int64_t c = b - r * blocks_per_row;
  const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + c * 16);
  const uint4 v0 = src[0];
  const uint4 v1 = src[1];
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  float f[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
  const float g = gs[r / rows_per_gs];
  uint32_t lo, hi;
  const uint32_t sc = quantize_block16(f, g, lo, hi);
  reinterpret_cast<uint2*>(codes)[b] = make_uint2(lo, hi);
  scales[tiled ? tiled_scale_index(r, c, blocks_per_row * 16) : b] = (uint8_t)sc;
}

// amax per matrix of a [batch, per_matrix] BF16 array, as float bits
// (non-negative floats order like unsigned integers).
__global__ __launch_bounds__(256) void amax_bf16_kernel(const uint16_t* __restrict__ w, int64_t per_matrix,
                                                        uint32_t* __restrict__ amax_bits) {
  const int64_t mat = blockIdx.y;
  const uint16_t* base = w + mat * per_matrix;
  uint32_t m = 0;
  const int64_t n8 = per_matrix / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
    const uint4 v = reinterpret_cast<const uint4*>(base)[i];
    const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = max(m, (q[j] & 0x7FFFu) << 16);
      m = max(m, ((q[j] >> 16) & 0x7FFFu) << 16);
    }
  }
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = max(max(part[0], part[1]), max(part[2], part[3]));
    atomicMax(&amax_bits[mat], r);
  }
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// gs = f32(2688 / amax), 1 when amax is 0 (in place over the amax bits).
__global__ void global_scale_kernel(float* gs, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float a = gs[i];
  gs[i] = (a == 0.0f) ? 1.0f : (kE4M3Max * kE2M1Max) / a;
}

hipError_t launch_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* gs,
                                int64_t rows_per_gs, uint8_t* codes, uint8_t* scales, bool tiled_scales,
                                hipStream_t stream) {
  const int64_t bpr = cols / 16;
  const int64_t n = rows * bpr;
  if (n == 0) return hipSuccess;
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(quantize_bf16_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, rows, bpr, ld, gs,
                     rows_per_gs, codes, scales, tiled_scales ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_weight_global_scales(const uint16_t* w, int64_t batch, int64_t per_matrix, float* gs,
                                       hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<uint32_t*>(gs), batch, 0u);
  int64_t per_block = 256 * 8 * 16;  // elements per workgroup pass
  int64_t gx = (per_matrix + per_block - 1) / per_block;
  if (gx > 1024) gx = 1024;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(amax_bf16_kernel, dim3((unsigned)gx, (unsigned)batch), dim3(256), 0, stream, w, per_matrix,
                     reinterpret_cast<uint32_t*>(gs));
  hipLaunchKernelGGL(global_scale_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, stream, gs, batch);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {

// One-time relayout of canonical NVFP4 weight scales ([R, K/16] row-major) into
// the tiled order the expert kernels read ([R/16, K/128, 16, 8]), and back.
// Thread t moves the 8 scale bytes of one (row, 128-column group): one 8-byte
// read and one 8-byte write.  Codes are kept in their canonical layout.
template <bool TO_TILED>
__global__ __launch_bounds__(256) void relayout_scales_kernel(const uint8_t* __restrict__ src, int64_t rows,
                                                              int64_t K, uint8_t* __restrict__ dst) {
  const int64_t groups = K / 128;  // 8-byte scale groups per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * groups) return;
  const int64_t r = i / groups, g = i - r * groups;
  const int64_t canon = r * (K / 16) + 8 * g;
  const int64_t tiled = tiled_scale_index(r, 8 * g, K);
  if (TO_TILED)
    *reinterpret_cast<uint2*>(dst + tiled) = *reinterpret_cast<const uint2*>(src + canon);
  else
    *reinterpret_cast<uint2*>(dst + canon) = *reinterpret_cast<const uint2*>(src + tiled);
}

hipError_t launch_relayout_scales(const uint8_t* src, int64_t rows, int64_t K, bool to_tiled, uint8_t* dst,
                                  hipStream_t st) {
  const int64_t n = rows * (K / 128);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (to_tiled) hipLaunchKernelGGL(relayout_scales_kernel<true>, dim3(grid), dim3(256), 0, st, src, rows, K, dst);
  else hipLaunchKernelGGL(relayout_scales_kernel<false>, dim3(grid), dim3(256), 0, st, src, rows, K, dst);
  return hipGetLastError();
}

}  // namespace moe
