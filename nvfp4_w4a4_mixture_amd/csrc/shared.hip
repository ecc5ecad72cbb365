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
//  * dense_tiled_kernel (T > 16): MFMA-bound.  256 x 256 tile per workgroup,
//    2 x 2 waves of 128 x 128 (16 32x32x16 accumulators each), 64-k stages in
//    an LDS double buffer filled from registers (the next stage's global loads
//    are in flight while the current one is multiplied), 16-byte chunks
//    swizzled by row so that fragment reads and stores are bank-conflict
//    free.  Stage 1's tile pairs 64 gate rows with the 64 up rows of the same
//    h columns in each wave, so SwiGLU is applied in registers.
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
// tiled kernel

constexpr int kDBM = 256, kDBN = 256, kDBK = 64;
constexpr int kDTileBytes = kDBM * kDBK * 2;        // one operand's stage: 256 rows x 128 B
constexpr int kDStage = 2 * kDTileBytes;            // A then B
constexpr int kDLds = 2 * kDStage;                  // double buffer, 128 KB

// 16-byte chunk c of row r is stored in slot c ^ ((r >> 1) & 7): the 16 rows a
// fragment read touches at one chunk, and the 2 rows of 8 chunks a store
// group writes, land in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int dslot(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int MODE>
__global__ __launch_bounds__(256) void dense_tiled_kernel(const uint16_t* __restrict__ a, int64_t lda,
                                                          const uint16_t* __restrict__ w, int64_t T, int64_t K,
                                                          int64_t I, uint16_t* __restrict__ h, int64_t ldh,
                                                          float* __restrict__ out, int64_t ldo) {
  const int nt = blockIdx.x, mt = blockIdx.y;
  const int64_t m0 = (int64_t)mt * kDBM;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;

  // B tile row n -> weight row.  Stage 1: wave wn's 128 rows are h columns
  // nt*128 + wn*64 + 0..63 as gate rows (n % 128 < 64) then as up rows.
  auto b_row = [&](int n) -> int64_t {
    if (MODE == kSharedGateUp) {
      const int wv = n >> 7, j = (n & 127) >> 5, cc = n & 31;
      return (j < 2 ? 0 : I) + (int64_t)nt * 128 + wv * 64 + 32 * (j & 1) + cc;
    }
    return (int64_t)nt * kDBN + n;
  };
  // global -> register loads: load i of a thread covers row 32 i + tid / 8, chunk tid % 8
  const int lrow = tid >> 3, lchunk = tid & 7;
  const uint16_t* ag[8];
  const uint16_t* bg[8];
  uint32_t lds_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 32 * i + lrow;
    const int64_t t = m0 + row < T ? m0 + row : T - 1;  // rows past T repeat the last token; never stored
    ag[i] = a + t * lda + 8 * lchunk;
    bg[i] = w + b_row(row) * K + 8 * lchunk;
    lds_off[i] = (uint32_t)(row * 128 + 16 * dslot(row, lchunk));
  }
  u32x4_t ra[8], rb[8];
  auto gload = [&](int64_t st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(ag[i] + st * kDBK);
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(bg[i] + st * kDBK);
  };
  auto lstore = [&](int buf) {
    unsigned char* base = smem + buf * kDStage;
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(base + lds_off[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4_t*>(base + kDTileBytes + lds_off[i]) = rb[i];
  };

  float16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // fragment i of this wave: rows wm*128 + 32 i + r (A), wn*128 + 32 j + r (B);
  // k-step s of a stage: chunk 2 s + g.  (32 i + r) >> 1 & 7 == (r >> 1) & 7.
  const int arow = wm * 128 + r, brow = wn * 128 + r;
  auto frag = [&](const unsigned char* base, int row, int s) -> bf16x8_t {
    return as_bf16x8(*reinterpret_cast<const u32x4_t*>(base + row * 128 + 16 * dslot(r, 2 * s + g)));
  };

  const int64_t nst = K / kDBK;
  gload(0);
  lstore(0);
  if (nst > 1) gload(1);
  for (int64_t st = 0; st < nst; ++st) {
    __syncthreads();  // stage st is in buffer st & 1 for every wave; buffer (st + 1) & 1 is free
    const unsigned char* base = smem + (int)(st & 1) * kDStage;
    bf16x8_t fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = frag(base, arow + 32 * i, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[0][j] = frag(base + kDTileBytes, brow + 32 * j, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int cur = s & 1;
      if (s + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[cur ^ 1][i] = frag(base, arow + 32 * i, s + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[cur ^ 1][j] = frag(base + kDTileBytes, brow + 32 * j, s + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < nst) {
      lstore((int)((st + 1) & 1));
      if (st + 2 < nst) gload(st + 2);
    }
  }

  // ---- epilogues.  acc[i][j][e]: row wm*128 + 32 i + 8 (e/4) + 4 g + e%4, column r of tile j
  if (MODE == kSharedGateUp) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
          if (t < T) {
            const int64_t c = (int64_t)nt * 128 + wn * 64 + 32 * j + r;
            h[t * ldh + c] = (uint16_t)f32_to_bf16_rne(silu(acc[i][j][e]) * acc[i][j + 2][e]);
          }
        }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t t = m0 + wm * 128 + 32 * i + 8 * (e >> 2) + 4 * g + (e & 3);
          if (t < T) out[t * ldo + (int64_t)nt * kDBN + wn * 128 + 32 * j + r] = acc[i][j][e];
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
  const unsigned mtiles = (unsigned)((T + kDBM - 1) / kDBM);
  if (mode == kSharedGateUp) {
    if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&dense_tiled_kernel<kSharedGateUp>), kDLds))
      return e;
    hipLaunchKernelGGL(dense_tiled_kernel<kSharedGateUp>, dim3((unsigned)(I / 128), mtiles), dim3(256), kDLds, st, a,
                       lda, w, T, K, I, h, I, (float*)nullptr, (int64_t)0);
  } else {
    if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&dense_tiled_kernel<kSharedDown>), kDLds))
      return e;
    hipLaunchKernelGGL(dense_tiled_kernel<kSharedDown>, dim3((unsigned)(H / kDBN), mtiles), dim3(256), kDLds, st, a,
                       lda, w, T, K, I, (uint16_t*)nullptr, (int64_t)0, out, H);
  }
  return hipGetLastError();
}

}  // namespace moe
