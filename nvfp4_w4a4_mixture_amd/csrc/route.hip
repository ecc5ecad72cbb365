// Routing: sigmoid + bias top-k, renormalized and scaled, and the stable
// expert permutation ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning
// Setup": renormalized sigmoid routing, e_score_correction_bias,
// routed_scaling_factor; the forum post "1x Spark GB10 ...", "Caveats":
// top-8 routing; "K-EXAONE-152B-A23B-REAP-80E-NVFP4", "Quantization Setup":
// the router stays BF16).
//
// route_logits_kernel: FP64 logit partials for a 64-token tile over one range
// of the hidden dimension, from BF16 x and W_r staged through LDS (every
// product and sum is FP64).  route_select_kernel: one wave per token sums the
// partials in a fixed order and selects the top-k with wave-wide argmax
// reductions.  Selection decides integers, so it runs in FP64 like the
// definition it follows; ties go to the lower expert index.
//
// The permutation is a stable counting sort in three passes over chunks of
// kPermChunk pairs: per-chunk histograms, a per-expert scan over chunks, and a
// per-chunk scatter that ranks equal experts by pair id with wave ballots.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kTok = 64;          // tokens per logits workgroup (4 per thread row)
constexpr int kHC = 32;           // hidden elements per LDS stage
constexpr int kPermChunk = 2048;  // pairs per permutation chunk
constexpr int kTargetWGs = 512;   // logits grid size to aim for (2 per CU)
constexpr int kMaxSplit = 32;     // bounds the partial sums each selecting lane reads

// H is split into `nsplit` ranges of `hlen` (a multiple of kHC) so that small
// token counts still spread over the whole chip; partial logits are summed in
// split order by the selection kernel (deterministic).
struct RouteSplit {
  int64_t nsplit, hlen;
};

static RouteSplit route_split(int64_t T, int64_t H) {
  const int64_t ntiles = (T + kTok - 1) / kTok;
  const int64_t nch = (H + kHC - 1) / kHC;
  int64_t ns = ntiles > 0 ? (kTargetWGs + ntiles - 1) / ntiles : 1;
  ns = ns < 1 ? 1 : (ns > kMaxSplit ? kMaxSplit : ns);
  ns = ns > nch ? nch : ns;
  const int64_t hlen = ((nch + ns - 1) / ns) * kHC;
  return {(H + hlen - 1) / hlen, hlen};
}

// Partial FP64 logits: part[split][t][e] = sum over the split's h range of
// x[t,h] * W_r[e,h].  BF16 values are converted once to FP64 in LDS; each
// thread holds a 4-token x JE-expert register tile (e = te + 16 j).
template <int JE>
__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t H,
                                                           int64_t ldx, const uint16_t* __restrict__ wr, int E,
                                                           int64_t hlen, double* __restrict__ part) {
  constexpr int kEP = 16 * JE;
  __shared__ __align__(16) double xs[kTok * kHC];
  __shared__ __align__(16) double ws[kEP * (kHC + 1)];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int64_t split = blockIdx.y;
  const int64_t hbeg = split * hlen;
  const int64_t hend = hbeg + hlen < H ? hbeg + hlen : H;
  const int te = tid & 15;  // expert lane
  const int tt = tid >> 4;  // tokens 4*tt .. 4*tt+3
  double acc[4][JE];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JE; ++j) acc[i][j] = 0.0;

  for (int64_t h0 = hbeg; h0 < hend; h0 += kHC) {
    for (int i = tid; i < kTok * kHC; i += 256) {
      const int r = i / kHC, c = i % kHC;
      const int64_t t = t0 + r, hh = h0 + c;
      xs[i] = (t < T && hh < hend) ? (double)bf16_to_f32(x[t * ldx + hh]) : 0.0;
    }
    for (int i = tid; i < kEP * kHC; i += 256) {
      const int r = i / kHC, c = i % kHC;
      const int64_t hh = h0 + c;
      ws[r * (kHC + 1) + c] = (r < E && hh < hend) ? (double)bf16_to_f32(wr[(int64_t)r * H + hh]) : 0.0;
    }
    __syncthreads();
#pragma unroll 2
    for (int c = 0; c < kHC; ++c) {
      double xv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = xs[(4 * tt + i) * kHC + c];
#pragma unroll
      for (int j = 0; j < JE; ++j) {
        const double w = ws[(te + 16 * j) * (kHC + 1) + c];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_fma(xv[i], w, acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t t = t0 + 4 * tt + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < JE; ++j) {
      const int e = te + 16 * j;
      if (e < E) part[(split * T + t) * E + e] = acc[i][j];
    }
  }
}

// One wave per token: logit = sum of the partials in split order; score =
// sigmoid(logit) + bias; k rounds of a wave-wide argmax under the total order
// (score descending, expert ascending); weights rsf * s_j / sum s.
__global__ __launch_bounds__(256) void route_select_kernel(const double* __restrict__ part, int64_t nsplit, int64_t T,
                                                           const float* __restrict__ bias, int E, int k, float rsf,
                                                           int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_w) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  double sc[4], sg[4];
  bool taken[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    taken[i] = (e >= E);
    sg[i] = 0.0;
    sc[i] = 0.0;
    if (e < E) {
      double z = 0.0;
#pragma unroll 8
      for (int64_t s = 0; s < nsplit; ++s) z += part[(s * T + t) * E + e];  // fixed order
      sg[i] = 1.0 / (1.0 + exp(-z));
      sc[i] = sg[i] + (double)bias[e];
    }
  }
  double ssum = 0.0;
  int my_e[4] = {0, 0, 0, 0};  // slot j is kept by lane j % 64 in my_e[j / 64]
  double my_s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int j = 0; j < k; ++j) {
    double bs = -__builtin_inf();
    int be = 0x7FFFFFFF;
    double bg = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!taken[i] && (sc[i] > bs || be == 0x7FFFFFFF)) {  // i ascending = expert ascending
        bs = sc[i];
        be = lane + 64 * i;
        bg = sg[i];
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double os = __shfl_xor(bs, off);
      const int oe = __shfl_xor(be, off);
      const double og = __shfl_xor(bg, off);
      if (os > bs || (os == bs && oe < be)) {
        bs = os;
        be = oe;
        bg = og;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == be) taken[i] = true;
    ssum += bg;  // every lane sums in the same order j = 0..k-1
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i == (j >> 6) && lane == (j & 63)) {
        my_e[i] = be;
        my_s[i] = bg;
      }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = lane + 64 * i;
    if (j < k) {
      topk_ids[t * k + j] = my_e[i];
      topk_w[t * k + j] = (float)((double)rsf * my_s[i] / ssum);
    }
  }
}

// Per-chunk expert histograms: counts[c][e] for chunk c of kPermChunk pairs.
__global__ __launch_bounds__(256) void perm_count_kernel(const int32_t* __restrict__ ids, int64_t npairs, int E,
                                                         int32_t* __restrict__ chunk_counts) {
  __shared__ int32_t hist[256];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)c * kPermChunk;
  for (int i = threadIdx.x; i < kPermChunk; i += 256) {
    const int64_t p = p0 + i;
    if (p < npairs) atomicAdd(&hist[ids[p]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)c * E + e] = hist[e];
}

// One thread per expert: totals over chunks, then the exclusive scan over
// experts, then each chunk's base offset for each expert.
__global__ __launch_bounds__(256) void perm_scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks, int E,
                                                        int32_t* __restrict__ chunk_base, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets) {
  __shared__ int32_t tot[256];
  __shared__ int32_t off[257];
  const int e = threadIdx.x;
  int32_t s = 0;
  if (e < E)
    for (int c = 0; c < nchunks; ++c) s += chunk_counts[(int64_t)c * E + e];
  tot[e] = (e < E) ? s : 0;
  __syncthreads();
  if (e == 0) {
    int32_t run = 0;
    for (int i = 0; i < E; ++i) {
      off[i] = run;
      run += tot[i];
    }
    off[E] = run;
  }
  __syncthreads();
  if (e < E) {
    counts[e] = tot[e];
    offsets[e] = off[e];
    int32_t run = off[e];
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(int64_t)c * E + e] = run;
      run += chunk_counts[(int64_t)c * E + e];
    }
  }
  if (e == 0) offsets[E] = off[E];
}

// Stable scatter of one chunk: pairs are taken in increasing id, 256 at a
// time; within a wave a lane's rank among equal experts comes from an 8-bit
// ballot match; across waves from per-wave counts in LDS.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ ids, int64_t npairs, int E,
                                                           const int32_t* __restrict__ chunk_base,
                                                           int32_t* __restrict__ sorted_pair_ids) {
  __shared__ int32_t run[256];
  __shared__ int32_t wave_cnt[4][256];
  const int c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) run[e] = chunk_base[(int64_t)c * E + e];
  const int64_t p0 = (int64_t)c * kPermChunk;
  for (int sub = 0; sub < kPermChunk; sub += 256) {
    for (int i = tid; i < 4 * 256; i += 256) (&wave_cnt[0][0])[i] = 0;
    __syncthreads();
    const int64_t p = p0 + sub + tid;
    const bool valid = p < npairs;
    const int e = valid ? ids[p] : -1;
    // lanes of this wave holding the same expert
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t b = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? b : ~b;
    }
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & lower);
    const bool last = valid && ((same >> lane) >> 1) == 0;  // highest lane of its expert
    if (last) wave_cnt[wave][e] = rank + 1;
    __syncthreads();
    if (valid) {
      int base = run[e];
      for (int w = 0; w < wave; ++w) base += wave_cnt[w][e];
      sorted_pair_ids[base + rank] = (int32_t)p;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += 256)
      run[ee] += wave_cnt[0][ee] + wave_cnt[1][ee] + wave_cnt[2][ee] + wave_cnt[3][ee];
    __syncthreads();
  }
}

static size_t align256(size_t v) { return (v + 255) / 256 * 256; }

size_t route_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t k) {
  const int64_t npairs = T * k;
  const int64_t nchunks = (npairs + kPermChunk - 1) / kPermChunk;
  const RouteSplit sp = route_split(T, H);
  return align256((size_t)(2 * nchunks * E * 4)) + (size_t)(sp.nsplit * T * E * 8);
}

template <int JE>
static void launch_logits(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, int E,
                          RouteSplit sp, double* part, hipStream_t st) {
  const dim3 grid((unsigned)((T + kTok - 1) / kTok), (unsigned)sp.nsplit);
  hipLaunchKernelGGL(route_logits_kernel<JE>, grid, dim3(256), 0, st, x, T, H, ldx, wr, E, sp.hlen, part);
}

hipError_t launch_route(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, const float* bias,
                        int64_t E, int64_t k, float rsf, int32_t* topk_ids, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, void* workspace, hipStream_t st) {
  const int e = (int)E, kk = (int)k;
  const int64_t npairs = T * k;
  const int nchunks = (int)((npairs + kPermChunk - 1) / kPermChunk);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_counts + (int64_t)nchunks * E;
  if (T == 0) {  // no pairs: zero counts and offsets only
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, 0, e, chunk_base, counts, offsets);
    return hipGetLastError();
  }
  const RouteSplit sp = route_split(T, H);
  double* part = reinterpret_cast<double*>(static_cast<unsigned char*>(workspace) +
                                           align256((size_t)(2 * nchunks * E * 4)));
  switch ((e + 15) / 16) {
#define LG(N) \
  case N: launch_logits<N>(x, T, H, ldx, wr, e, sp, part, st); break;
    LG(1) LG(2) LG(3) LG(4) LG(5) LG(6) LG(7) LG(8) LG(9) LG(10) LG(11) LG(12) LG(13) LG(14) LG(15) LG(16)
#undef LG
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(route_select_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, part, sp.nsplit, T, bias,
                     e, kk, rsf, topk_ids, topk_w);
  hipLaunchKernelGGL(perm_count_kernel, dim3(nchunks), dim3(256), 0, st, topk_ids, npairs, e, chunk_counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, nchunks, e, chunk_base, counts,
                     offsets);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(256), 0, st, topk_ids, npairs, e, chunk_base, sorted);
  return hipGetLastError();
}

}  // namespace moe
