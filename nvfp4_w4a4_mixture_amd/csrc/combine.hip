// Weighted combine and REAP saliency.
//
// combine ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning Setup":
// renormalized sigmoid routing weights): y[t] = sum_j pair row t*k + j, in
// j order, where the pair rows already carry w_{t,j}; for the block output the
// shared expert's FP32 row is added last.  A pair row is FP16 times its
// power-of-two scale, so each decoded value is exact in FP32.  HBM-bound:
// eight columns of y per thread, k (+1) 16-byte reads, issued eight at a time.
//
// REAP saliency (same card and section: mean(topk_weight * ||f_e(x)||_2) over
// routed tokens, routing weights including routed_scaling_factor): one
// workgroup per expert walks its pairs in sorted order; FP64 partial sums in
// a fixed thread/tree order make the result deterministic.
#include "device_common.h"
#include "launch.h"

namespace moe {

// y for columns 8 i .. 8 i + 7 of the [T, H] output (i < T * H / 8)
template <bool BF16_OUT>
__device__ __forceinline__ void combine_one(const uint16_t* __restrict__ pair_out, const float* __restrict__ pair_scale,
                                            const float* __restrict__ add, int64_t T, int k, int64_t H,
                                            void* __restrict__ y, int64_t i) {
  const int64_t h8 = H / 8;
  if (i >= T * h8) return;
  const int64_t t = i / h8, c = i - t * h8;
  const half8_t* src = reinterpret_cast<const half8_t*>(pair_out) + (t * k) * h8 + c;
  const float* scl = pair_scale + t * k;
  // the k rows in chunks of 8 loads issued together, summed in j order
  float s[8];
  for (int j0 = 0; j0 < k; j0 += 8) {
    const int n = k - j0 < 8 ? k - j0 : 8;
    half8_t v[8];
    float sc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < n) {
        v[u] = __builtin_nontemporal_load(src + (int64_t)(j0 + u) * h8);  // each pair row is read once
        sc[u] = scl[j0 + u];
      }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < n) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float d = (float)v[u][q] * sc[u];  // exact: FP16 value times a power of two
          s[q] = j0 + u == 0 ? d : s[q] + d;
        }
      }
    }
  }
  if (add != nullptr) {  // the block output: routed combine, then the shared expert
    const float4* a4 = reinterpret_cast<const float4*>(add) + 2 * i;
    const float4 v0 = a4[0], v1 = a4[1];
    s[0] += v0.x;
    s[1] += v0.y;
    s[2] += v0.z;
    s[3] += v0.w;
    s[4] += v1.x;
    s[5] += v1.y;
    s[6] += v1.z;
    s[7] += v1.w;
  }
  if (BF16_OUT) {
    auto rne = [](float f) -> uint32_t {
      const uint32_t u = __float_as_uint(f);
      return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    };
    uint4 o;
    o.x = rne(s[0]) | (rne(s[1]) << 16);
    o.y = rne(s[2]) | (rne(s[3]) << 16);
    o.z = rne(s[4]) | (rne(s[5]) << 16);
    o.w = rne(s[6]) | (rne(s[7]) << 16);
    reinterpret_cast<uint4*>(y)[i] = o;
  } else {
    float4* o = reinterpret_cast<float4*>(y) + 2 * i;
    o[0] = make_float4(s[0], s[1], s[2], s[3]);
    o[1] = make_float4(s[4], s[5], s[6], s[7]);
  }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ pair_out,
                                                      const float* __restrict__ pair_scale,
                                                      const float* __restrict__ add, int64_t T, int k, int64_t H,
                                                      void* __restrict__ y) {
  combine_one<BF16_OUT>(pair_out, pair_scale, add, T, k, H, y, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// saliency of expert e: its pairs walked in sorted order, FP64 sums in a fixed tree
__device__ __forceinline__ void reap_one(const float* __restrict__ sq, const float* __restrict__ topk_w,
                                         const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted,
                                         float* __restrict__ saliency, int e) {
  const int b = offsets[e], n = offsets[e + 1] - b;
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int p = sorted[b + i];
    s += (double)topk_w[p] * sqrt((double)sq[p]);
  }
  __shared__ double red[256];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) saliency[e] = n > 0 ? (float)(red[0] / (double)n) : 0.0f;
}

__global__ __launch_bounds__(256) void reap_kernel(const float* __restrict__ sq, const float* __restrict__ topk_w,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ sorted, float* __restrict__ saliency) {
  reap_one(sq, topk_w, offsets, sorted, saliency, blockIdx.x);
}

// combine and REAP in one launch: blocks [0, nb) combine, blocks [nb, nb + E) one expert each
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_reap_kernel(const uint16_t* __restrict__ pair_out,
                                                           const float* __restrict__ pair_scale, int64_t T, int k,
                                                           int64_t H, void* __restrict__ y, unsigned nb,
                                                           const float* __restrict__ sq,
                                                           const float* __restrict__ topk_w,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ sorted,
                                                           float* __restrict__ saliency) {
  if (blockIdx.x < nb)
    combine_one<BF16_OUT>(pair_out, pair_scale, nullptr, T, k, H, y, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  else
    reap_one(sq, topk_w, offsets, sorted, saliency, (int)(blockIdx.x - nb));
}

hipError_t launch_combine(const uint16_t* pair_out, const float* pair_scale, const float* add, int64_t T, int64_t k,
                          int64_t H, int out_dtype, void* y, hipStream_t st) {
  const int64_t n = T * (H / 8);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (out_dtype == 0)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, st, pair_out, pair_scale, add, T, (int)k, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, st, pair_out, pair_scale, add, T, (int)k, H,
                       y);
  return hipGetLastError();
}

hipError_t launch_reap(const float* sq, const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                       int64_t E, float* saliency, hipStream_t st) {
  hipLaunchKernelGGL(reap_kernel, dim3((unsigned)E), dim3(256), 0, st, sq, topk_w, offsets, sorted, saliency);
  return hipGetLastError();
}

hipError_t launch_combine_reap(const uint16_t* pair_out, const float* pair_scale, int64_t T, int64_t k, int64_t H,
                               int out_dtype, void* y, const float* sq, const float* topk_w, const int32_t* offsets,
                               const int32_t* sorted, int64_t E, float* saliency, hipStream_t st) {
  const unsigned nb = (unsigned)((T * (H / 8) + 255) / 256);
  const dim3 grid(nb + (unsigned)E);
  if (out_dtype == 0)
    hipLaunchKernelGGL(combine_reap_kernel<true>, grid, dim3(256), 0, st, pair_out, pair_scale, T, (int)k, H, y, nb, sq,
                       topk_w, offsets, sorted, saliency);
  else
    hipLaunchKernelGGL(combine_reap_kernel<false>, grid, dim3(256), 0, st, pair_out, pair_scale, T, (int)k, H, y, nb,
                       sq, topk_w, offsets, sorted, saliency);
  return hipGetLastError();
}

}  // namespace moe
