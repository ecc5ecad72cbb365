// Routing: sigmoid + bias top-k, renormalized and scaled, and the stable
// expert permutation ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning
// Setup": renormalized sigmoid routing, e_score_correction_bias,
// routed_scaling_factor; the forum post "1x Spark GB10 ...", "Caveats":
// top-8 routing; "K-EXAONE-152B-A23B-REAP-80E-NVFP4", "Quantization Setup":
// the router stays BF16).
//
// route_select_kernel: one workgroup per 32 tokens.  The FP64 logit tile
// [32, E] is computed from BF16 x and W_r staged through LDS (each BF16 value
// converted once to FP64; every product and sum is FP64), kept in LDS, then
// each wave selects the top-k of 8 tokens with wave-wide argmax reductions.
// Selection decides integers, so it runs in FP64 like the reference
// definition; ties go to the lower expert index.
//
// The permutation is a stable counting sort in three passes over chunks of
// kPermChunk pairs: per-chunk histograms, a per-expert scan over chunks, and a
// per-chunk scatter that ranks equal experts by pair id with wave ballots.
#include "device_common.h"
#include "launch.h"

namespace moe {

constexpr int kTok = 32;        // tokens per routing workgroup
constexpr int kHC = 32;         // hidden elements per LDS stage
constexpr int kPermChunk = 2048;  // pairs per permutation chunk

template <int JE>  // experts per thread: e = te + 16 * j, j < JE (E <= 16 * JE)
__global__ __launch_bounds__(256) void route_select_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t H,
                                                           int64_t ldx, const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int E, int k, float rsf,
                                                           int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
  // LDS: x stage [kTok][kHC] f64, w stage [16*JE][kHC+1] f64; reused for logits [kTok][E] f64.
  constexpr int kEP = 16 * JE;
  constexpr int kStageBytes = (kTok * kHC + kEP * (kHC + 1)) * 8;
  constexpr int kLogitBytes = kTok * kEP * 8;
  constexpr int kLdsBytes = kStageBytes > kLogitBytes ? kStageBytes : kLogitBytes;
  __shared__ __align__(16) unsigned char smem[kLdsBytes];
  double* xs = reinterpret_cast<double*>(smem);
  double* ws = xs + kTok * kHC;
  double* logits = reinterpret_cast<double*>(smem);

  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int te = tid & 15;  // expert lane
  const int tt = tid >> 4;  // tokens tt*2, tt*2+1
  double acc[2][JE];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < JE; ++j) acc[i][j] = 0.0;

  for (int64_t h0 = 0; h0 < H; h0 += kHC) {
    // stage x: kTok * kHC values, 4 per thread
    for (int i = tid; i < kTok * kHC; i += 256) {
      const int r = i / kHC, c = i % kHC;
      const int64_t t = t0 + r;
      const int64_t hh = h0 + c;
      xs[i] = (t < T && hh < H) ? (double)bf16_to_f32(x[t * ldx + hh]) : 0.0;
    }
    for (int i = tid; i < kEP * kHC; i += 256) {
      const int r = i / kHC, c = i % kHC;
      const int64_t hh = h0 + c;
      ws[r * (kHC + 1) + c] = (r < E && hh < H) ? (double)bf16_to_f32(wr[(int64_t)r * H + hh]) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kHC; ++c) {
      const double xa = xs[(tt * 2) * kHC + c];
      const double xb = xs[(tt * 2 + 1) * kHC + c];
#pragma unroll
      for (int j = 0; j < JE; ++j) {
        const double w = ws[(te + 16 * j) * (kHC + 1) + c];
        acc[0][j] = __builtin_fma(xa, w, acc[0][j]);
        acc[1][j] = __builtin_fma(xb, w, acc[1][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < JE; ++j) logits[(tt * 2 + i) * kEP + te + 16 * j] = acc[i][j];
  __syncthreads();

  // selection: wave w handles tokens w*8 .. w*8+7
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int q = 0; q < kTok / 4; ++q) {
    const int r = wave * (kTok / 4) + q;
    const int64_t t = t0 + r;
    if (t >= T) break;
    // each lane owns experts lane, lane+64, lane+128, lane+192
    double sc[4], sg[4];
    bool taken[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      taken[i] = (e >= E);
      sg[i] = 0.0;
      sc[i] = 0.0;
      if (e < E) {
        const double z = logits[r * kEP + e];
        sg[i] = 1.0 / (1.0 + exp(-z));
        sc[i] = sg[i] + (double)bias[e];
      }
    }
    double ssum = 0.0;
    int my_e[4] = {0, 0, 0, 0};  // slot j is kept by lane j % 64 in my_e[j / 64]
    double my_s[4] = {0.0, 0.0, 0.0, 0.0};
    for (int j = 0; j < k; ++j) {
      // this lane's best remaining candidate: highest score, then lowest index
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
      // wave-wide argmax under the total order (score desc, index asc)
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

size_t route_workspace_bytes(int64_t T, int64_t E, int64_t k) {
  const int64_t npairs = T * k;
  const int64_t nchunks = (npairs + kPermChunk - 1) / kPermChunk;
  return (size_t)(2 * nchunks * E * 4);
}

template <int JE>
static void launch_select(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr,
                          const float* bias, int E, int k, float rsf, int32_t* ids, float* w, hipStream_t st) {
  const unsigned grid = (unsigned)((T + kTok - 1) / kTok);
  hipLaunchKernelGGL(route_select_kernel<JE>, dim3(grid), dim3(256), 0, st, x, T, H, ldx, wr, bias, E, k, rsf, ids,
                     w);
}

hipError_t launch_route(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, const float* bias,
                        int64_t E, int64_t k, float rsf, int32_t* topk_ids, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, void* workspace, hipStream_t st) {
  const int e = (int)E, kk = (int)k;
  const int je = (e + 15) / 16;
  const int64_t npairs = T * k;
  const int nchunks = (int)((npairs + kPermChunk - 1) / kPermChunk);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_counts + (int64_t)nchunks * E;
  if (T == 0) {  // no pairs: zero counts and offsets only
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, 0, e, chunk_base, counts, offsets);
    return hipGetLastError();
  }
  switch (je) {
#define SEL(N) \
  case N: launch_select<N>(x, T, H, ldx, wr, bias, e, kk, rsf, topk_ids, topk_w, st); break;
    SEL(1) SEL(2) SEL(3) SEL(4) SEL(5) SEL(6) SEL(7) SEL(8) SEL(9) SEL(10) SEL(11) SEL(12) SEL(13) SEL(14) SEL(15)
    SEL(16)
#undef SEL
    default: return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL(perm_count_kernel, dim3(nchunks), dim3(256), 0, st, topk_ids, npairs, e, chunk_counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, nchunks, e, chunk_base, counts,
                     offsets);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(256), 0, st, topk_ids, npairs, e, chunk_base, sorted);
  return hipGetLastError();
}

}  // namespace moe
