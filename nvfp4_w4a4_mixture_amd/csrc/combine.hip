// Weighted combine and REAP saliency.
//
// combine ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning Setup":
// renormalized sigmoid routing weights): y[t] = sum_j pair_out[t*k + j], in
// j order, where pair_out already carries w_{t,j}; for the block output the
// shared expert's FP32 row is added last.  HBM-bound: one float4 of y per
// thread, k (+1) float4 reads, issued eight at a time.
//
// REAP saliency (same card and section: mean(topk_weight * ||f_e(x)||_2) over
// routed tokens, routing weights including routed_scaling_factor): one
// workgroup per expert walks its pairs in sorted order; FP64 partial sums in
// a fixed thread/tree order make the result deterministic.
#include "device_common.h"
#include "launch.h"

namespace moe {

// y for one float4 column group i of the [T, H/4] output
template <bool BF16_OUT>
__device__ __forceinline__ void combine_one(const float* __restrict__ pair_out, const float* __restrict__ add,
                                            int64_t T, int k, int64_t H, void* __restrict__ y, int64_t i) {
  const int64_t h4 = H / 4;
  if (i >= T * h4) return;
  const int64_t t = i / h4, c = i - t * h4;
  const float4* src = reinterpret_cast<const float4*>(pair_out) + (t * k) * h4 + c;
  // the k rows in chunks of 8 loads issued together, summed in j order
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    const int n = k - j0 < 8 ? k - j0 : 8;
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < n) {
        // each pair row is read once: non-temporal
        const float4_t t = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(src + (int64_t)(j0 + u) * h4));
        v[u] = make_float4(t[0], t[1], t[2], t[3]);
      }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < n) {
        if (j0 + u == 0) {
          s = v[u];
        } else {
          s.x += v[u].x;
          s.y += v[u].y;
          s.z += v[u].z;
          s.w += v[u].w;
        }
      }
    }
  }
  if (add != nullptr) {  // the block output: routed combine, then the shared expert
    const float4 v = reinterpret_cast<const float4*>(add)[i];
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  if (BF16_OUT) {
    auto rne = [](float f) -> uint32_t {
      const uint32_t u = __float_as_uint(f);
      return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    };
    uint2 o;
    o.x = rne(s.x) | (rne(s.y) << 16);
    o.y = rne(s.z) | (rne(s.w) << 16);
    reinterpret_cast<uint2*>(y)[i] = o;
  } else {
    reinterpret_cast<float4*>(y)[i] = s;
  }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ pair_out,
                                                      const float* __restrict__ add, int64_t T, int k, int64_t H,
                                                      void* __restrict__ y) {
  combine_one<BF16_OUT>(pair_out, add, T, k, H, y, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
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
__global__ __launch_bounds__(256) void combine_reap_kernel(const float* __restrict__ pair_out, int64_t T, int k,
                                                           int64_t H, void* __restrict__ y, unsigned nb,
                                                           const float* __restrict__ sq,
                                                           const float* __restrict__ topk_w,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ sorted,
                                                           float* __restrict__ saliency) {
  if (blockIdx.x < nb)
    combine_one<BF16_OUT>(pair_out, nullptr, T, k, H, y, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  else
    reap_one(sq, topk_w, offsets, sorted, saliency, (int)(blockIdx.x - nb));
}

hipError_t launch_combine(const float* pair_out, const float* add, int64_t T, int64_t k, int64_t H, int out_dtype,
                          void* y, hipStream_t st) {
  const int64_t n = T * (H / 4);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (out_dtype == 0)
    hipLaunchKernelGGL(combine_kernel<true>, dim3(grid), dim3(256), 0, st, pair_out, add, T, (int)k, H, y);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3(grid), dim3(256), 0, st, pair_out, add, T, (int)k, H, y);
  return hipGetLastError();
}

hipError_t launch_reap(const float* sq, const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                       int64_t E, float* saliency, hipStream_t st) {
  hipLaunchKernelGGL(reap_kernel, dim3((unsigned)E), dim3(256), 0, st, sq, topk_w, offsets, sorted, saliency);
  return hipGetLastError();
}

hipError_t launch_combine_reap(const float* pair_out, int64_t T, int64_t k, int64_t H, int out_dtype, void* y,
                               const float* sq, const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                               int64_t E, float* saliency, hipStream_t st) {
  const unsigned nb = (unsigned)((T * (H / 4) + 255) / 256);
  const dim3 grid(nb + (unsigned)E);
  if (out_dtype == 0)
    hipLaunchKernelGGL(combine_reap_kernel<true>, grid, dim3(256), 0, st, pair_out, T, (int)k, H, y, nb, sq, topk_w,
                       offsets, sorted, saliency);
  else
    hipLaunchKernelGGL(combine_reap_kernel<false>, grid, dim3(256), 0, st, pair_out, T, (int)k, H, y, nb, sq, topk_w,
                       offsets, sorted, saliency);
  return hipGetLastError();
}

}  // namespace moe
