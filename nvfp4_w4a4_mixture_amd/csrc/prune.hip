// REAP one-shot expert pruning ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card,
// introduction and "Pruning Setup": the routed experts of lowest REAP saliency
// are removed, 128 -> 80 per layer, and the router's gate weight and
// e_score_correction_bias are sliced to the experts that remain).
//
// Selection: one workgroup, one thread per expert.  Each thread counts the
// experts ordered before it under (saliency descending, index ascending) --
// a strict total order, so the ranks are a permutation of 0..E-1 and exactly
// n_keep experts have rank < n_keep.  The kept flags are compacted in index
// order with a wave ballot and a 4-entry LDS scan, so keep_ids is ascending.
//
// Slicing: every per-expert tensor of the layer (codes, tiled scales, global
// scales, router rows, bias) is one contiguous byte block per expert, so the
// pruned layer is built by one block gather per tensor, HBM-bound: 16-byte
// loads and stores when sizes and pointers allow.
#include "device_common.h"
#include "launch.h"

namespace moe {

// Monotone map of a float onto uint32 (larger float -> larger key), with
// -0 and +0 mapped together so that equal values compare equal.
__device__ __forceinline__ uint32_t saliency_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(256) void prune_select_kernel(const float* __restrict__ saliency, int E, int n_keep,
                                                           int32_t* __restrict__ keep_ids) {
  __shared__ uint32_t key[256];
  __shared__ int wsum[4];
  const int e = threadIdx.x;
  if (e < E) key[e] = saliency_key(saliency[e]);
  __syncthreads();
  int kept = 0;
  if (e < E) {
    const uint32_t ke = key[e];
    int rank = 0;
    for (int j = 0; j < E; ++j) {
      const uint32_t kj = key[j];
      rank += (kj > ke) | ((kj == ke) & (j < e));
    }
    kept = rank < n_keep;
  }
  const uint64_t m = __ballot(kept);
  const int lane = e & 63, w = e >> 6;
  const int pre = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[w] = __popcll(m);
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  if (kept) keep_ids[base + pre] = e;
}

// dst block i = src block ids[i]; n_per elements of V per block.  An id
// outside [0, n_src) leaves its destination block unwritten.
template <typename V>
__global__ __launch_bounds__(256) void gather_blocks_kernel(const V* __restrict__ src, int64_t n_src,
                                                            V* __restrict__ dst, int64_t n_per,
                                                            const int32_t* __restrict__ ids) {
  const int64_t id = ids[blockIdx.y];
  if (id < 0 || id >= n_src) return;
  const V* s = src + id * n_per;
  V* d = dst + (int64_t)blockIdx.y * n_per;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  // four independent loads in flight per thread before their stores
  for (; c + 3 * stride < n_per; c += 4 * stride) {
    const V v0 = s[c], v1 = s[c + stride], v2 = s[c + 2 * stride], v3 = s[c + 3 * stride];
    d[c] = v0;
    d[c + stride] = v1;
    d[c + 2 * stride] = v2;
    d[c + 3 * stride] = v3;
  }
  for (; c < n_per; c += stride) d[c] = s[c];
}

hipError_t launch_prune_select(const float* saliency, int64_t E, int64_t n_keep, int32_t* keep_ids,
                               hipStream_t st) {
  hipLaunchKernelGGL(prune_select_kernel, dim3(1), dim3(256), 0, st, saliency, (int)E, (int)n_keep, keep_ids);
  return hipGetLastError();
}

template <typename V>
static hipError_t gather_as(const void* src, int64_t n_src, int64_t bytes, const int32_t* ids, int64_t n_ids,
                            void* dst, hipStream_t st) {
  const int64_t n_per = bytes / (int64_t)sizeof(V);
  // about 4096 workgroups in all, at most one per 256 elements of a block
  int64_t gx = (4096 + n_ids - 1) / n_ids;
  gx = gx < (n_per + 255) / 256 ? gx : (n_per + 255) / 256;
  gx = gx < 1 ? 1 : gx;
  hipLaunchKernelGGL(gather_blocks_kernel<V>, dim3((unsigned)gx, (unsigned)n_ids), dim3(256), 0, st,
                     static_cast<const V*>(src), n_src, static_cast<V*>(dst), n_per, ids);
  return hipGetLastError();
}

hipError_t launch_gather_blocks(const void* src, int64_t n_src, int64_t bytes, const int32_t* ids, int64_t n_ids,
                                void* dst, hipStream_t st) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) | (uintptr_t)bytes;
  if (a % 16 == 0) return gather_as<uint4>(src, n_src, bytes, ids, n_ids, dst, st);
  if (a % 4 == 0) return gather_as<uint32_t>(src, n_src, bytes, ids, n_ids, dst, st);
  return gather_as<uint8_t>(src, n_src, bytes, ids, n_ids, dst, st);
}

}  // namespace moe
