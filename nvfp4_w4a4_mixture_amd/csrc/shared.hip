// The BF16 shared expert of the MoE block ("K-EXAONE-152B-A23B-REAP-80E-NVFP4"
// model card, "Quantization Setup": the shared experts stay BF16, only the
// routed experts are NVFP4; "K-EXAONE-152B-A23B-REAP-80E-BF16" model card,
// "Pruning Setup": the shared expert is kept whole).
//
//   stage 1 (gate_up): g, u = x . W_gate^T, x . W_up^T  (BF16 products, FP32
//                      accumulation); h = bf16_rne(silu(g) * u)
//   stage 2 (down):    s = h . W_down^T  (FP32 out, [T, H])
//
// Both operands are K-contiguous BF16 rows, the natural MFMA operand order.
// Two kernel families, chosen by T:
//  * dense_small_kernel (T <= 16): HBM-bound weight stream.  One workgroup per
//    (64 weight rows, 512 k); each wave takes 128 k of its 64 rows as 16
//    independent 16-byte loads per lane (nothing else in flight), 16x16x32
//    MFMA with the tokens as M; the four waves meet in LDS and the workgroup
//    writes one FP32 partial per K split.  A finalize pass sums the splits in
//    order (and applies SwiGLU + BF16 rounding for stage 1).
//  * dense_ring_kernel (T > 16): 256 x 256 tile per workgroup, 2 x 4 waves of
//    128 x 64, operand tiles streamed into a 4-stage LDS ring by DMA.  Stage
//    1's tile pairs 32 gate rows with the 32 up rows of the same h columns in
//    each wave, so SwiGLU is applied in registers.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

enum { kSharedGateUp = 0, kSharedDown = 1 };

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// small-T kernel

constexpr int kSmallKSplit = 512;  // k per workgroup: 4 waves x 128

// stage 1: tile = 32 h columns -> weight rows c0..c0+31 (gate) and I+c0.. (up);
// stage 2: tile = 64 output columns -> weight rows n0..n0+63.
// part: [S][T][R] FP32 with R = the weight's row count (2I or H).
template <int MODE>
__global__ __launch_bounds__(256) void dense_small_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                          const uint16_t* __restrict__ w, int64_t T, int64_t K,
                                                          int64_t I, int64_t R, float* __restrict__ part) {
  const int tile = blockIdx.x, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, q = lane >> 4;
  auto wrow = [&](int j) -> int64_t {
    if (MODE == kSharedGateUp) return (j < 2 ? 0 : I) + (int64_t)tile * 32 + 16 * (j & 1) + n16;
    return (int64_t)tile * 64 + 16 * j + n16;
  };
  float4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t k0 = (int64_t)s * kSmallKSplit + 128 * wave;
  if (k0 < K) {
    // MFMA step c covers k0 + 32c .. +31; lane group q supplies k0 + 32c + 8q .. +7
    const int64_t t = n16 < T ? n16 : T - 1;  // rows past T repeat the last token; never stored
    const u32x4_t* ap = reinterpret_cast<const u32x4_t*>(a + t * lda + k0 + 8 * q);
    u32x4_t av[4], bv[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4_t* bp = reinterpret_cast<const u32x4_t*>(w + wrow(j) * K + k0 + 8 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[j][c] = bp[4 * c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) av[c] = ap[4 * c];
    // all 20 loads are issued before the first MFMA waits on one of them
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[c]), as_bf16x8(bv[j][c]), acc[j], 0, 0, 0);
  }
  // acc[j][i]: token 4q + i, weight row wrow(j) (lane n16)
  __shared__ float red[4][4][16][16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][j][4 * q + i][n16] = acc[j][i];
  __syncthreads();
  const int m = tid >> 4, n = tid & 15;
  if (m < T) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = ((red[0][j][m][n] + red[1][j][m][n]) + red[2][j][m][n]) + red[3][j][m][n];
      int64_t row;
      if (MODE == kSharedGateUp) row = (j < 2 ? 0 : I) + (int64_t)tile * 32 + 16 * (j & 1) + n;
      else row = (int64_t)tile * 64 + 16 * j + n;
      part[((int64_t)s * T + m) * R + row] = v;
    }
  }
}

// h[t, c] = bf16(silu(g) * u), g and u summed over the S splits in order
__global__ __launch_bounds__(256) void dense_gate_finalize_kernel(const float* __restrict__ part, int S, int64_t T,
                                                                  int64_t I, uint16_t* __restrict__ h) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * I) return;
  const int64_t t = i / I, c = i - t * I;
  float g = 0.0f, u = 0.0f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float* p = part + ((int64_t)s * T + t) * 2 * I;
    g += p[c];
    u += p[I + c];
  }
  h[i] = (uint16_t)f32_to_bf16_rne(silu(g) * u);
}

__global__ __launch_bounds__(256) void dense_sum_finalize_kernel(const float* __restrict__ part, int S, int64_t n,
                                                                 float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) v += part[(int64_t)s * n + i];
  out[i] = v;
}

// ---------------------------------------------------------------------------
// tiled kernel with a DMA ring (the production path for T > 16)
//
// 256 x 256 workgroup tile, eight waves in 2 (M) x 4 (N), each owning 128 x 64
// (4 x 2 accumulators of 32 x 32), two waves per SIMD so that one wave's LDS
// reads overlap the other's MFMAs.  Operand tiles go from HBM straight into a
// 4-stage LDS ring (global_load_lds, 32 k per stage: 64 B per row in four
// 16-byte slots, chunk c of row r in slot c ^ ((r >> 2) & 3)); each wave reads
// its fragments of a stage in one asm block that waits only for LDS, so the
// DMA of later stages stays in flight.

namespace dr {
constexpr int BM = 256, BN = 256, NS = 4;
constexpr int kTile = BM * 64;           // one operand's stage: 256 rows x 32 k x 2 B
constexpr int kStage = 2 * kTile;        // A then B
constexpr int kLds = NS * kStage;        // 128 KiB
constexpr int kLoadsPerStage = 2 + 2;    // 16-byte DMA per wave and stage: A, B
}  // namespace dr

template <int MODE>
__global__ __launch_bounds__(512) void dense_ring_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                         const uint16_t* __restrict__ w, int64_t T, int64_t K,
                                                         int64_t I, uint16_t* __restrict__ h, int64_t ldh,
                                                         float* __restrict__ out, int64_t ldo) {
  using namespace dr;
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int64_t m0 = (int64_t)mt * BM;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 31, g = lane >> 5;

  // B tile row n -> weight row.  Stage 1: N wave n / 64 owns h columns nt*128 + 32*(n/64) + 0..31,
  // as gate rows (n % 64 < 32) and as up rows.
  auto b_row = [&](int n) -> int64_t {
    if (MODE == kSharedGateUp) {
      const int wv = n >> 6, j = (n >> 5) & 1, cc = n & 31;
      return (j ? I : 0) + (int64_t)nt * 128 + 32 * wv + cc;
    }
    return (int64_t)nt * BN + n;
  };
  // 16-byte DMA i (0, 1) of this wave: rows 16 q .. 16 q + 15, q = 8 i + wave; lane -> row 16 q + lane / 4,
  // LDS slot lane % 4 holding chunk slot ^ ((row >> 2) & 3)
  uint32_t a_off[2], b_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 16 * (8 * i + wave) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    const int64_t t = m0 + row < T ? m0 + row : T - 1;  // rows past T repeat the last token; never stored
    a_off[i] = (uint32_t)(t * lda * 2) + 16 * chunk;
    b_off[i] = (uint32_t)(b_row(row) * K * 2) + 16 * chunk;
  }
  float16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const uint32_t a_lane = (uint32_t)(wm * 128 + r) * 64u;
  const uint32_t b_lane = (uint32_t)kTile + (uint32_t)(wn * 64 + r) * 64u;
  // k-step s (0, 1) of a stage: chunk 2 s + g; rows 32 apart share (r >> 2) & 3
  const uint32_t slot0 = 16u * (uint32_t)((2 * 0 + g) ^ ((r >> 2) & 3));
  const uint32_t slot1 = 16u * (uint32_t)((2 * 1 + g) ^ ((r >> 2) & 3));

  // Pipelined ring, as in the FFN tile kernel: the DMA is inline asm (so the
  // compiler's own LDS reads get no blanket vmcnt(0)), one barrier per stage
  // between its two k-steps, and each k-step's fragments are read while the
  // previous k-step's MFMAs run.  The prologue fills all NS slots; at the
  // mid-stage barrier of stage st every wave has read slot st % NS
  // (lgkmcnt(0) before the barrier) and waited for stage st + 1, so stage
  // st + NS is issued into slot st % NS right after it.
  const int64_t nst = K / 32;  // >= 4 (K % 128 == 0)
  constexpr int L = kLoadsPerStage;
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane((uint32_t)wave);
  auto issue = [&](int64_t st) {
    const uint32_t sb = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(st % NS) * (uint32_t)kStage);
    const unsigned char* ag = reinterpret_cast<const unsigned char*>(a) + st * 64;
    const unsigned char* bg = reinterpret_cast<const unsigned char*>(w) + st * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_async(ag, a_off[i], sb + (8 * i + wave_u) * 1024u);
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_async(bg, b_off[i], sb + (uint32_t)kTile + (8 * i + wave_u) * 1024u);
  };
  auto load_k = [&](int64_t st, uint32_t slot, u32x4_t* fa, u32x4_t* fb) {
    const uint32_t sb = (uint32_t)(st % NS) * (uint32_t)kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const u32x4_t*>(smem + sb + a_lane + slot + 2048u * i);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const u32x4_t*>(smem + sb + b_lane + slot + 2048u * j);
  };
  auto mfma8 = [&](const u32x4_t* fa, const u32x4_t* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i][j], 0, 0, 0);
    // each MFMA followed by one of the 6 LDS reads issued before it in program order
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (m < 6) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
  };

#pragma unroll
  for (int p = 0; p < NS; ++p) issue(p);
  wait_vmcnt<3 * L>();  // stage 0 has landed (nst >= NS)
  barrier_after_lds();
  u32x4_t f0a[4], f0b[2];
  load_k(0, slot0, f0a, f0b);
  auto stage = [&](int64_t st, auto more_c, auto issue_c) {
    constexpr bool kMore = decltype(more_c)::value, kIssue = decltype(issue_c)::value;
    u32x4_t f1a[4], f1b[2], n0a[4], n0b[2];
    __builtin_amdgcn_sched_barrier(0);
    load_k(st, slot1, f1a, f1b);
    mfma8(f0a, f0b);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kMore) {
      // stage st + 1 has landed; the stages issued after it may stay in flight
      const int64_t ahead = nst - 2 - st;
      if (kIssue || ahead >= NS - 2) wait_vmcnt<(NS - 2) * L>();
      else if (ahead == 1) wait_vmcnt<L>();
      else wait_vmcnt<0>();
      barrier_after_lds();
      if constexpr (kIssue) issue(st + NS);
      load_k(st + 1, slot0, n0a, n0b);
    }
    mfma8(f1a, f1b);
    if constexpr (kMore) {
#pragma unroll
      for (int i = 0; i < 4; ++i) f0a[i] = n0a[i];
#pragma unroll
      for (int j = 0; j < 2; ++j) f0b[j] = n0b[j];
    }
  };
  int64_t st = 0;
  for (; st + NS < nst; ++st) stage(st, std::true_type{}, std::true_type{});
  for (; st + 1 < nst; ++st) stage(st, std::true_type{}, std::false_type{});
  stage(st, std::false_type{}, std::false_type{});
  wait_vmcnt<0>();  // nothing is in flight here

  // ---- epilogues.  acc[i][j][e]: row wm*128 + 32 i + 8 (e/4) + 4 g + e%4, column r of B fragment j
  if (MODE == kSharedGateUp) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t t = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
        if (t < T) {
          const int64_t c = (int64_t)nt * 128 + wn * 32 + r;
          h[t * ldh + c] = (uint16_t)f32_to_bf16_rne(silu(acc[i][0][e]) * acc[i][1][e]);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
          if (t < T) out[t * ldo + (int64_t)nt * BN + wn * 64 + 32 * j + r] = acc[i][j][e];
        }
  }
}

// ---------------------------------------------------------------------------
// launchers


static int small_splits(int64_t K) { return (int)((K + kSmallKSplit - 1) / kSmallKSplit); }

bool shared_use_small(int64_t T) { return T <= 16; }

size_t shared_part_bytes(int64_t T, int64_t H, int64_t I) {
  if (!shared_use_small(T)) return 0;
  const size_t g = (size_t)small_splits(H) * (size_t)T * (size_t)(2 * I);
  const size_t d = (size_t)small_splits(I) * (size_t)T * (size_t)H;
  return (g > d ? g : d) * sizeof(float);
}

hipError_t launch_shared_stage(int mode, const uint16_t* a, int64_t lda, const uint16_t* w, int64_t T, int64_t H,
                               int64_t I, uint16_t* h, float* out, float* part, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t K = mode == kSharedGateUp ? H : I;
  if (shared_use_small(T)) {
    const int S = small_splits(K);
    const int64_t R = mode == kSharedGateUp ? 2 * I : H;
    if (mode == kSharedGateUp) {
      hipLaunchKernelGGL(dense_small_kernel<kSharedGateUp>, dim3((unsigned)(I / 32), (unsigned)S), dim3(256), 0, st,
                         a, lda, w, T, K, I, R, part);
      const int64_t n = T * I;
      hipLaunchKernelGGL(dense_gate_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, S, T,
                         I, h);
    } else {
      hipLaunchKernelGGL(dense_small_kernel<kSharedDown>, dim3((unsigned)(H / 64), (unsigned)S), dim3(256), 0, st, a,
                         lda, w, T, K, I, R, part);
      const int64_t n = T * H;
      hipLaunchKernelGGL(dense_sum_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, S, n,
                         out);
    }
    return hipGetLastError();
  }
  const unsigned mtiles = (unsigned)((T + dr::BM - 1) / dr::BM);
  if (mode == kSharedGateUp) {
    if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&dense_ring_kernel<kSharedGateUp>), dr::kLds))
      return e;
    hipLaunchKernelGGL(dense_ring_kernel<kSharedGateUp>, dim3((unsigned)(I / 128), mtiles), dim3(512), dr::kLds, st, a,
                       lda, w, T, K, I, h, I, (float*)nullptr, (int64_t)0);
  } else {
    if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&dense_ring_kernel<kSharedDown>), dr::kLds))
      return e;
    hipLaunchKernelGGL(dense_ring_kernel<kSharedDown>, dim3((unsigned)(H / dr::BN), mtiles), dim3(512), dr::kLds, st, a,
                       lda, w, T, K, I, (uint16_t*)nullptr, (int64_t)0, out, H);
  }
  return hipGetLastError();
}

}  // namespace moe
