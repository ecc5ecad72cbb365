// Routing: sigmoid + bias top-k, renormalized and scaled, and the stable
// expert permutation ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning
// Setup": renormalized sigmoid routing, e_score_correction_bias,
// routed_scaling_factor; the forum post "1x Spark GB10 ...", "Caveats":
// top-8 routing; "K-EXAONE-152B-A23B-REAP-80E-NVFP4", "Quantization Setup":
// the router stays BF16).
//
// Logits: FP64 partial sums over ranges of H, on the FP64 matrix cores
// (route_logits_mfma_kernel) when rows are 16-byte aligned and H % 16 == 0,
// else on the vector units (route_logits_kernel for batches,
// route_logits_decode_kernel for T <= 16).  Every product of two BF16 values
// is exact in FP64.  The MFMA kernel can also write the NVFP4 quantization of
// x, which it holds in registers anyway (moe_route_quantize).
//
// Selection (route_select_kernel): one wave per token sums the partials in
// split order and ranks every expert under (score descending, expert
// ascending); rank < k is slot `rank` of the top-k.  Selection decides
// integers, so it runs in FP64 like the definition it follows; ties go to the
// lower expert index.
//
// Permutation: a stable counting sort, in one workgroup for up to 16 tokens
// (perm_small_kernel), else in three passes over chunks of kPermChunk
// pairs: per-chunk histograms, a per-expert scan over chunks, and a per-chunk
// scatter that ranks equal experts by pair id with wave ballots.
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

// Orders this wave's LDS writes before its later LDS reads (lanes read what
// other lanes of the same wave wrote).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Selection key of an FP64 score: a signed 64-bit integer in the order of the
// scores, with -0 equal to +0 and NaN below every number (below -inf).  Keys
// are totally ordered, so with ties going to the lower expert index every rank
// 0..E-1 is taken by exactly one expert, also when scores are NaN (a token
// whose x holds a NaN or an infinity, or a NaN bias).  This is the order of a
// stable sort of the scores, descending, with NaN last.
__device__ __forceinline__ long long score_key(double v) {
  if (v != v) return (long long)0x8000000000000000ull;  // NaN: the smallest key
  long long b = __double_as_longlong(v);
  if (b == (long long)0x8000000000000000ull) b = 0;  // -0 -> +0
  return b < 0 ? (b ^ 0x7FFFFFFFFFFFFFFFll) : b;      // negatives: larger magnitude, smaller key
}

// Top-k of one token by one wave from its scores.  Lane holds, for the
// experts e = lane + 64 i (i < NG, e < E), sg = sigmoid(logit) and
// sc = sg + bias.  The top-k are the experts whose rank under the total order
// (score key descending, expert ascending) is below k: each lane ranks its
// experts against every key, broadcast from the wave's LDS row `row` (>= E + 1
// doubles, 16-byte aligned; padded to an even length with the smallest key at
// index E, which outranks nothing), so slot j holds the j-th expert of that
// order.  The row is then reused for the selected sg; weights are
// rsf * s_j / sum s, the sum taken over j = 0..k-1 in order.  On return
// slot[i] = 1 + the slot of expert lane + 64 i (0: not chosen).
template <int NG>
__device__ __forceinline__ void rank_select(const double (&sg)[NG], const double (&sc)[NG], int64_t t, int E, int k,
                                            float rsf, int lane, double* row, int32_t* __restrict__ topk_ids,
                                            float* __restrict__ topk_w, int (&slot)[4]) {
  long long* krow = reinterpret_cast<long long*>(row);
  long long key[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    key[i] = score_key(sc[i]);
    if (lane + 64 * i < E) krow[lane + 64 * i] = key[i];
  }
  if (lane == 0 && (E & 1)) krow[E] = (long long)0x8000000000000000ull;
  wave_lds_sync();
  int rank[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) rank[i] = 0;
  const int npair = (E + 1) >> 1;
#pragma unroll 4
  for (int q = 0; q < npair; ++q) {
    const longlong2 v = reinterpret_cast<const longlong2*>(krow)[q];
    const int e0 = 2 * q;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const int e = lane + 64 * i;
      rank[i] += (int)(v.x > key[i]) | ((int)(v.x == key[i]) & (int)(e0 < e));
      rank[i] += (int)(v.y > key[i]) | ((int)(v.y == key[i]) & (int)(e0 + 1 < e));
    }
  }
  wave_lds_sync();  // every lane has read the keys; the row now takes sg by slot
#pragma unroll
  for (int i = 0; i < 4; ++i) slot[i] = 0;
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    const int e = lane + 64 * i;
    if (e < E && rank[i] < k) {
      slot[i] = rank[i] + 1;
      topk_ids[t * k + rank[i]] = e;
      row[rank[i]] = sg[i];
    }
  }
  wave_lds_sync();
  double ssum = 0.0;
  for (int j = 0; j < k; ++j) ssum += row[j];
  for (int j = lane; j < k; j += 64) topk_w[t * k + j] = (float)((double)rsf * row[j] / ssum);
  wave_lds_sync();  // the row is reused by the wave's next token
}

// General path: one wave per token sums the partials in split order (lanes
// past E read expert E-1 and ignore it, so every load is unconditional and
// the loads of several splits are in flight together), then rank_select.
template <int NG>
__device__ __forceinline__ void select_token_ng(const double* __restrict__ part, int64_t nsplit, int64_t T, int64_t t,
                                                const float* __restrict__ bias, int E, int k, float rsf, int lane,
                                                double* row, int32_t* __restrict__ topk_ids,
                                                float* __restrict__ topk_w, int (&slot)[4]) {
  int ec[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) ec[i] = lane + 64 * i < E ? lane + 64 * i : E - 1;
  double z[NG], b[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    z[i] = 0.0;
    b[i] = (double)bias[ec[i]];
  }
  const double* pt = part + t * E;
  const int64_t stride = T * E;
#pragma unroll 8
  for (int64_t s = 0; s < nsplit; ++s) {  // fixed order over splits
    const double* ps = pt + s * stride;
#pragma unroll
    for (int i = 0; i < NG; ++i) z[i] += ps[ec[i]];
  }
  double sg[NG], sc[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    sg[i] = 1.0 / (1.0 + exp(-z[i]));
    sc[i] = sg[i] + b[i];
  }
  rank_select<NG>(sg, sc, t, E, k, rsf, lane, row, topk_ids, topk_w, slot);
}

__global__ __launch_bounds__(256) void route_select_kernel(const double* __restrict__ part, int64_t nsplit, int64_t T,
                                                           const float* __restrict__ bias, int E, int k, float rsf,
                                                           int32_t* __restrict__ topk_ids,
                                                           float* __restrict__ topk_w) {
  __shared__ __align__(16) double rows[4][258];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 4 + wave;
  if (t >= T) return;
  int slot[4];
  double* row = rows[wave];
  switch ((E + 63) >> 6) {
    case 1: select_token_ng<1>(part, nsplit, T, t, bias, E, k, rsf, lane, row, topk_ids, topk_w, slot); break;
    case 2: select_token_ng<2>(part, nsplit, T, t, bias, E, k, rsf, lane, row, topk_ids, topk_w, slot); break;
    case 3: select_token_ng<3>(part, nsplit, T, t, bias, E, k, rsf, lane, row, topk_ids, topk_w, slot); break;
    default: select_token_ng<4>(part, nsplit, T, t, bias, E, k, rsf, lane, row, topk_ids, topk_w, slot); break;
  }
}

// FP64 matrix-core logits.  v_mfma_f64_16x16x4_f64 (16 tokens x 16 experts x 4
// h per instruction) with each lane's operands converted from BF16 in
// registers: lane l supplies token row l % 16 of A and expert column l % 16 of
// B for k = l / 16, and register i of the result is token (l / 16) + 4 i,
// expert l % 16 (layout checked by a probe on the device).  The sum over k is
// free to permute as long as A and B agree, so lane group g takes 16
// contiguous h of every 64-h chunk: two 16-byte loads per row and chunk, no
// LDS.  Every product of two BF16 values is exact in FP64.
//   batches (T > 16): a workgroup = 4 waves x 16 tokens over one H range;
//   decode (T <= 16): a workgroup = 16 tokens over 256 h, wave w takes the
//   w-th 64-h quarter, and the quarter sums are added in wave order in LDS.
// Requires H % 16 == 0, ldx % 8 == 0 and 16-byte aligned x and W_r.
typedef double double4_t __attribute__((ext_vector_type(4)));
constexpr int kMfmaChunk = 64;

struct MfmaSplit {
  int64_t nsplit, hlen;
};
// Batches: 16-token row blocks per wave.  Two blocks share each converted
// router value between two MFMAs (half the BF16 -> FP64 converts per MFMA);
// above 128 experts their accumulators would not fit, so one.
static inline int mfma_row_blocks(int nt) { return nt <= 8 ? 2 : 1; }

static MfmaSplit mfma_split(int64_t T, int64_t H, int nt) {
  if (T <= 16) return {(H + 255) / 256, 256};
  const int64_t blocks = (T + 64 * mfma_row_blocks(nt) - 1) / (64 * mfma_row_blocks(nt));
  const int64_t nch = (H + kMfmaChunk - 1) / kMfmaChunk;
  int64_t ns = (kTargetWGs + blocks - 1) / blocks;
  ns = ns < 1 ? 1 : (ns > kMaxSplit ? kMaxSplit : ns);
  ns = ns > nch ? nch : ns;
  const int64_t hlen = ((nch + ns - 1) / ns) * kMfmaChunk;
  return {(H + hlen - 1) / hlen, hlen};
}

__device__ __forceinline__ double bf16_pair_elem(const u32x4_t& lo, const u32x4_t& hi, int s) {
  const uint32_t w = (s < 8 ? lo : hi)[(s >> 1) & 3];
  return (double)__uint_as_float((s & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// QUANT: every lane also writes the NVFP4 quantization of its 16 x values (one
// block) to codes [T, H/2] and scales [T, H/16] against the global scale *qgs
// (the same steps as nvfp4_quantize_act); the grid covers each block once.
template <int NT, bool SPLIT_H, bool QUANT, int MB>
__global__ __launch_bounds__(256) void route_logits_mfma_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t H,
                                                                int64_t ldx, const uint16_t* __restrict__ wr, int E,
                                                                int64_t hlen, double* __restrict__ part,
                                                                const float* __restrict__ qgs,
                                                                uint8_t* __restrict__ qcodes,
                                                                uint8_t* __restrict__ qscales) {
  __shared__ double red[SPLIT_H ? 3 : 1][SPLIT_H ? NT : 1][64][4];
  const int lane = threadIdx.x & 63, r = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t split = blockIdx.y;
  static_assert(!SPLIT_H || MB == 1, "decode: one row block");
  // this wave's first token; its row blocks are t0 + 16 m, m < MB
  const int64_t t0 = SPLIT_H ? 0 : (int64_t)blockIdx.x * (64 * MB) + 16 * MB * wave;
  const int64_t hs = split * hlen;
  const int64_t he = hs + hlen < H ? hs + hlen : H;
  const int64_t hb = SPLIT_H ? hs + kMfmaChunk * wave : hs;
  const int64_t hend = SPLIT_H ? (hb + kMfmaChunk < he ? hb + kMfmaChunk : he) : he;
  // this lane's token rows and expert rows (clamped; their results are not stored)
  const uint16_t* xrow[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int64_t t = t0 + 16 * m + r;
    xrow[m] = x + (t < T ? t : T - 1) * ldx + 16 * g;
  }
  const uint16_t* wrow[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int e = 16 * n + r;
    wrow[n] = wr + (int64_t)(e < E ? e : E - 1) * H + 16 * g;
  }
  double4_t acc[MB][NT];
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = double4_t{0.0, 0.0, 0.0, 0.0};
  struct Chunk {
    u32x4_t a[MB][2];
    u32x4_t b[NT][2];
  };
  auto load = [&](int64_t h0, Chunk& d) {
    const bool in = h0 + 16 * g < hend;  // H % 16 == 0: a lane group's 16 h are all in or all out
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      d.a[m][0] = in ? *reinterpret_cast<const u32x4_t*>(xrow[m] + h0) : z;
      d.a[m][1] = in ? *reinterpret_cast<const u32x4_t*>(xrow[m] + h0 + 8) : z;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      d.b[n][0] = in ? *reinterpret_cast<const u32x4_t*>(wrow[n] + h0) : z;
      d.b[n][1] = in ? *reinterpret_cast<const u32x4_t*>(wrow[n] + h0 + 8) : z;
    }
  };
  const float gsq = QUANT ? qgs[0] : 0.0f;
  auto quantize = [&](int64_t h0, const Chunk& d) {
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int64_t t = t0 + 16 * m + r;
      if (t < T && h0 + 16 * g < hend) {
        float f[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w = d.a[m][i >> 2][i & 3];
          f[2 * i] = bf16_to_f32(w & 0xFFFFu);
          f[2 * i + 1] = bf16_to_f32(w >> 16);
        }
        uint32_t lo, hi;
        const uint32_t sc = quantize_block16(f, gsq, lo, hi);
        const int64_t hblk = h0 + 16 * g;
        *reinterpret_cast<uint2*>(qcodes + t * (H / 2) + hblk / 2) = make_uint2(lo, hi);
        qscales[t * (H / 16) + hblk / 16] = (uint8_t)sc;
      }
    }
  };
  auto compute = [&](const Chunk& d) {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      double av[MB];
#pragma unroll
      for (int m = 0; m < MB; ++m) av[m] = bf16_pair_elem(d.a[m][0], d.a[m][1], s);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const double bv = bf16_pair_elem(d.b[n][0], d.b[n][1], s);
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[m], bv, acc[m][n], 0, 0, 0);
      }
    }
  };
  if (hb < hend) {
    Chunk cur, nxt;
    load(hb, cur);
    for (int64_t h0 = hb; h0 < hend; h0 += kMfmaChunk) {
      if (h0 + kMfmaChunk < hend) load(h0 + kMfmaChunk, nxt);
      if (QUANT) quantize(h0, cur);
      compute(cur);
      cur = nxt;
    }
  }
  if (SPLIT_H) {
    if (wave > 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave - 1][n][lane][i] = acc[0][n][i];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[0][n][i] = ((acc[0][n][i] + red[0][n][lane][i]) + red[1][n][lane][i]) + red[2][n][lane][i];
  }
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const int e = 16 * n + r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tt = t0 + 16 * m + g + 4 * i;
        if (tt < T && e < E) part[(split * T + tt) * E + e] = acc[m][n][i];
      }
    }
}

template <int NT, bool SPLIT_H>
static void launch_logits_mfma(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, int E,
                               MfmaSplit sp, double* part, const float* qgs, uint8_t* qcodes, uint8_t* qscales,
                               hipStream_t st) {
  constexpr int MB = SPLIT_H ? 1 : (NT <= 8 ? 2 : 1);
  static_assert(SPLIT_H || MB == (NT <= 8 ? 2 : 1), "row blocks as mfma_row_blocks");
  const dim3 grid(SPLIT_H ? 1u : (unsigned)((T + 64 * MB - 1) / (64 * MB)), (unsigned)sp.nsplit);
  if (qcodes)
    hipLaunchKernelGGL((route_logits_mfma_kernel<NT, SPLIT_H, true, MB>), grid, dim3(256), 0, st, x, T, H, ldx, wr, E,
                       sp.hlen, part, qgs, qcodes, qscales);
  else
    hipLaunchKernelGGL((route_logits_mfma_kernel<NT, SPLIT_H, false, MB>), grid, dim3(256), 0, st, x, T, H, ldx, wr,
                       E, sp.hlen, part, qgs, qcodes, qscales);
}

// Smallest instantiated n-tile count covering E experts (E <= 256).
static int mfma_nt(int E) {
  const int need = (E + 15) / 16;
  return need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 5 ? 5 : need <= 8 ? 8 : 16;
}

// Decode batches (T <= kDecT).  Logits: each workgroup takes kDecH hidden
// elements for up to 64 experts; wave w takes the w-th quarter of that range,
// lane = expert, with the lane's 64 router weights in registers and the tokens'
// x values broadcast from LDS.  Quarter sums are added in wave order, so the
// partial for (split, t, e) is one fixed sum.  Requires 16-byte aligned x and
// W_r rows (ldx % 8 == 0, H % 8 == 0).
constexpr int kDecT = 16, kDecH = 256;
static inline int64_t dec_nsplit(int64_t H) { return (H + kDecH - 1) / kDecH; }

__global__ __launch_bounds__(256) void route_logits_decode_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t H,
                                                                  int64_t ldx, const uint16_t* __restrict__ wr,
                                                                  int E, double* __restrict__ part) {
  __shared__ __align__(16) double xs[kDecH][kDecT];
  __shared__ double red[3][kDecT][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t split = blockIdx.x;
  const int64_t h0 = split * kDecH;
  const int e = blockIdx.y * 64 + lane;
  // this lane's 64 router weights: row e, columns h0 + 64*wave ...
  u32x4_t wv[8];
  const int64_t hw = h0 + 64 * wave;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int64_t h = hw + 8 * c;
    wv[c] = (e < E && h < H) ? *reinterpret_cast<const u32x4_t*>(wr + (int64_t)e * H + h) : u32x4_t{0, 0, 0, 0};
  }
  // stage x[t][h0 .. h0+256) as FP64, transposed to xs[h][t]; zero past T and H
  {
    const int t = tid & 15, c0 = (tid >> 4) * 16;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c = c0 + 8 * half;
      const int64_t h = h0 + c;
      u32x4_t v = {0, 0, 0, 0};
      if (t < T && h < H) v = *reinterpret_cast<const u32x4_t*>(x + (int64_t)t * ldx + h);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xs[c + 2 * q][t] = (double)__uint_as_float(v[q] << 16);
        xs[c + 2 * q + 1][t] = (double)__uint_as_float(v[q] & 0xFFFF0000u);
      }
    }
  }
  __syncthreads();
  double acc[kDecT];
#pragma unroll
  for (int t = 0; t < kDecT; ++t) acc[t] = 0.0;
#pragma unroll 2
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t word = wv[c][q >> 1];
      const double w = (double)__uint_as_float((q & 1) ? (word & 0xFFFF0000u) : (word << 16));
      const double* xr = xs[64 * wave + 8 * c + q];
#pragma unroll
      for (int t = 0; t < kDecT; ++t) acc[t] = __builtin_fma(xr[t], w, acc[t]);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < kDecT; ++t) red[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave == 0 && e < E) {
    for (int t = 0; t < T; ++t) {
      const double z = ((acc[t] + red[0][t][lane]) + red[1][t][lane]) + red[2][t][lane];
      part[(split * T + t) * E + e] = z;
    }
  }
}

// Stable counting sort of a decode batch (T <= 16 tokens) in one workgroup,
// parallel over pairs p = t * k + j: each pair marks sel[t][e] and counts its
// expert (integer LDS atomics: order-free); an exclusive scan over experts
// gives the offsets; a pair's rank inside its expert is the number of earlier
// tokens that chose the same expert (a token never picks an expert twice),
// which is the order of pair ids.
constexpr int kSmallPermT = 16;
__global__ __launch_bounds__(256) void perm_small_kernel(const int32_t* __restrict__ ids, int T, int k, int E,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ sorted) {
  __shared__ uint32_t sel[kSmallPermT][256 / 4];  // bytes sel[t][e]
  __shared__ int32_t cnt[256];
  __shared__ int32_t base[256];
  __shared__ int32_t wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int npairs = T * k;
  for (int i = tid; i < kSmallPermT * 64; i += 256) (&sel[0][0])[i] = 0u;
  cnt[tid] = 0;
  __syncthreads();
  uint8_t* selb = reinterpret_cast<uint8_t*>(&sel[0][0]);
  for (int p = tid; p < npairs; p += 256) {
    const int e = ids[p];
    selb[(p / k) * 256 + e] = 1;
    atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  const int c = tid < E ? cnt[tid] : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int n = __shfl_up(incl, off);
    if (lane >= off) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = pre + incl - c;
    base[tid] = pre + incl - c;
  }
  if (tid == 0) offsets[E] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  for (int p = tid; p < npairs; p += 256) {
    const int e = ids[p], t = p / k;
    int r = 0;
    for (int t2 = 0; t2 < t; ++t2) r += selb[t2 * 256 + e];
    sorted[base[e] + r] = p;
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
  // unrolled so that the loads of several chunks are in flight together (integer sums: any order)
  if (e < E) {
#pragma unroll 16
    for (int c = 0; c < nchunks; ++c) s += chunk_counts[(int64_t)c * E + e];
  }
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
#pragma unroll 16
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
  int64_t nsplit = sp.nsplit;
  if (T <= kDecT && dec_nsplit(H) > nsplit) nsplit = dec_nsplit(H);
  if (mfma_split(T, H, mfma_nt((int)E)).nsplit > nsplit) nsplit = mfma_split(T, H, mfma_nt((int)E)).nsplit;
  return align256((size_t)(2 * nchunks * E * 4)) + (size_t)(nsplit * T * E * 8);
}

template <int JE>
static void launch_logits(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, int E,
                          RouteSplit sp, double* part, hipStream_t st) {
  const dim3 grid((unsigned)((T + kTok - 1) / kTok), (unsigned)sp.nsplit);
  hipLaunchKernelGGL(route_logits_kernel<JE>, grid, dim3(256), 0, st, x, T, H, ldx, wr, E, sp.hlen, part);
}

hipError_t launch_route(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, const float* bias,
                        int64_t E, int64_t k, float rsf, int32_t* topk_ids, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, void* workspace, const float* qgs, uint8_t* qcodes,
                        uint8_t* qscales, hipStream_t st) {
  const int e = (int)E, kk = (int)k;
  const int64_t npairs = T * k;
  const int nchunks = (int)((npairs + kPermChunk - 1) / kPermChunk);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(workspace);
  int32_t* chunk_base = chunk_counts + (int64_t)nchunks * E;
  if (T == 0) {  // no pairs: zero counts and offsets only
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, 0, e, chunk_base, counts, offsets);
    return hipGetLastError();
  }
  double* part = reinterpret_cast<double*>(static_cast<unsigned char*>(workspace) +
                                           align256((size_t)(2 * nchunks * E * 4)));
  const bool vec16 = (H % 8 == 0) && (ldx % 8 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)wr % 16 == 0);
  const int nt = mfma_nt(e);
  const bool mfma = vec16 && H % 16 == 0 && (T > kDecT || nt <= 8);
  int64_t nsplit = 0;
  if (mfma) {
    const MfmaSplit ms = mfma_split(T, H, nt);
    nsplit = ms.nsplit;
    const bool split_h = T <= kDecT;
#define LM(N)                                                                  \
  case N:                                                                      \
    if (split_h) launch_logits_mfma<N, true>(x, T, H, ldx, wr, e, ms, part, qgs, qcodes, qscales, st); \
    else launch_logits_mfma<N, false>(x, T, H, ldx, wr, e, ms, part, qgs, qcodes, qscales, st);        \
    break;
    switch (nt) {
      LM(1) LM(2) LM(4) LM(5) LM(8)
      case 16:  // only batches: decode batches with E > 128 take the register/LDS kernel (mfma is false there)
        launch_logits_mfma<16, false>(x, T, H, ldx, wr, e, ms, part, qgs, qcodes, qscales, st);
        break;
      default: return hipErrorInvalidValue;
    }
#undef LM
  } else {
    if (qcodes) {  // these logits kernels do not quantize: a separate pass
      const hipError_t err = launch_quantize_bf16(x, T, H, ldx, qgs, T, qcodes, qscales, false, st);
      if (err != hipSuccess) return err;
    }
    if (T <= kDecT && vec16) {
      nsplit = dec_nsplit(H);
      hipLaunchKernelGGL(route_logits_decode_kernel, dim3((unsigned)nsplit, (unsigned)((e + 63) / 64)), dim3(256), 0,
                         st, x, T, H, ldx, wr, e, part);
    } else {
      const RouteSplit sp = route_split(T, H);
      nsplit = sp.nsplit;
      switch ((e + 15) / 16) {
#define LG(N) \
  case N: launch_logits<N>(x, T, H, ldx, wr, e, sp, part, st); break;
        LG(1) LG(2) LG(3) LG(4) LG(5) LG(6) LG(7) LG(8) LG(9) LG(10) LG(11) LG(12) LG(13) LG(14) LG(15) LG(16)
#undef LG
        default: return hipErrorInvalidValue;
      }
    }
  }
  hipLaunchKernelGGL(route_select_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, part, nsplit, T, bias,
                     e, kk, rsf, topk_ids, topk_w);
  if (T <= kSmallPermT) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(256), 0, st, topk_ids, (int)T, kk, e, counts, offsets, sorted);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(perm_count_kernel, dim3(nchunks), dim3(256), 0, st, topk_ids, npairs, e, chunk_counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, st, chunk_counts, nchunks, e, chunk_base, counts,
                     offsets);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(nchunks), dim3(256), 0, st, topk_ids, npairs, e, chunk_base, sorted);
  return hipGetLastError();
}

}  // namespace moe
