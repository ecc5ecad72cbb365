// Grouped NVFP4 W4A4 expert FFN on gfx950 ("K-EXAONE-152B-A23B-REAP-80E-NVFP4"
// model card, "Quantization Setup": every routed expert Linear is NVFP4 W4A4
// with its own scales; the BF16 parent's experts are SwiGLU MLPs).
//
//   stage 1 (gate_up): g, u = xhat . W_gate^T, xhat . W_up^T ; h = silu(g) * u,
//                       h re-quantized to NVFP4 with the expert's calibrated gs_h
//   stage 2 (down):    f = hhat . W_down^T ; pair_out[p] = w_p * f (FP16 times a
//                       power-of-two scale per pair row) ; sum f^2
//
// Both operands stay FP4 in memory.  Each lane decodes its MFMA operand in
// registers: 8 E2M1 codes (one dword) -> 8 FP16 values times the E4M3 block
// scale, exact (see device_common.h), then the 16-bit MFMA accumulates exact
// products in FP32.  The global scales are applied once in the epilogue
// (alpha = 1 / (gs_act * gs_weight)).
//
// K permutation: an MFMA sums over its K slice, so the assignment of logical
// k to (k-step, lane group) is free as long as A and B lanes of the same group
// agree.  Each lane group takes a contiguous run of logical k, so a lane reads
// 16 contiguous bytes (32 codes, 4 k-steps) and one scale dword at a time.
//
// Two kernels:
//  * ffn_small_kernel (decode batches, every expert has <= 16 pairs): one
//    workgroup per (expert, 64-row weight tile); the four waves take
//    256-element K iterations in turn (a full 128-byte line per weight row),
//    each prefetching its next iteration into registers; weights
//    go straight from HBM to registers (each weight byte is used once),
//    16x16x32 MFMA; the waves' partial sums meet in LDS.
//  * ffn_tiled_kernel (any M): one workgroup per (m-tile of an expert's
//    pairs, n-tile of weight rows); A and B FP4 tiles go from HBM straight
//    into a 4-stage ring of LDS stages (global_load_lds, no register staging);
//    32x32x16 MFMA, 2x2 waves of 128x128 each (16 accumulator tiles per wave:
//    8 decoded fragments feed 16 MFMAs per k-step).  One barrier per stage,
//    mid-stage; the fragment reads of the next half-stage and the FP4 decode
//    of the next k-step run beside the current k-step's MFMAs.  An expert's
//    last m-tile with at most 128 pair rows runs wide instead: 128 rows
//    against two n-tiles, 1x4 waves, a 3-stage ring.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace moe {

enum { kGateUp = 0, kDown = 1 };

// ---------------------------------------------------------------------------
// small-M kernel

constexpr int kSmallRows = 16;  // pairs per expert handled (M_e <= 16)

// Per-lane operand data of one K iteration (KB logical k per row; each lane
// group of 16 lanes takes KB/4 contiguous k: KB/8 code bytes, KB/64 scales).
template <int KB>
struct SmallIter {
  static constexpr int kDw = KB / 32;  // code dwords per lane = MFMA k-steps
  u32x4_t ac[kDw / 4];
  uint32_t as;
  u32x4_t bc[4][kDw / 4];
  uint32_t bs[4];
};

#ifndef MOE_SMALL_NT
#define MOE_SMALL_NT 0  // plain loads measured faster than non-temporal ones for this stream
#endif
// the decode kernel's weight stream: each byte is read once
__device__ __forceinline__ u32x4_t load_stream(const u32x4_t* p) {
#if MOE_SMALL_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <int KB>
__device__ __forceinline__ uint32_t load_scales(const uint8_t* p) {
  if (KB == 256) return *reinterpret_cast<const uint32_t*>(p);
  return *reinterpret_cast<const uint16_t*>(p);
}

#ifndef MOE_SMALL_WAVES_PER_EU
#define MOE_SMALL_WAVES_PER_EU 3
#endif
template <int MODE, int KB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(MOE_SMALL_WAVES_PER_EU)))
void ffn_small_kernel(FfnArgs a) {
  using It = SmallIter<KB>;
  constexpr int kDw = It::kDw;
  const int tile = blockIdx.x;
  const int e = blockIdx.y;
  const int off = a.offsets[e];
  const int Me = a.offsets[e + 1] - off;
  if (Me <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int64_t K = a.K;
  const int64_t kbytes = K / 2, kscales = K / 16;

  // Every load is a wave-uniform base that advances with the K iteration
  // plus a 32-bit lane offset fixed for the whole kernel.
  // A row (pair c of this expert); rows past M_e read row off's data and take
  // a zero scale, so they decode to zeros without a branch.
  const bool a_valid = c < Me;
  const int cc = a_valid ? c : 0;
  const int64_t arow = (MODE == kGateUp) ? (int64_t)(a.sorted[off + cc] / a.k) : (int64_t)(off + cc);
  const uint32_t a_off = (uint32_t)(arow * kbytes) + g * (KB / 8);
  const uint32_t as_off = (uint32_t)(arow * kscales) + g * (KB / 64);
  // B: the tile's first row, then rows 16 j + c of the 4 n-subtiles (gate_up:
  // gate rows for h columns tile*32 + 0..31, then the matching up rows)
  const int64_t brow0 = (MODE == kGateUp) ? (int64_t)e * 2 * a.I + (int64_t)tile * 32
                                          : (int64_t)e * a.H + (int64_t)tile * 64;
  const uint8_t* b_code_base = a.b_codes + brow0 * kbytes;
  const uint8_t* b_scale_base = a.b_scales + (brow0 >> 4) * K;  // tiled scales, brow0 % 16 == 0
  uint32_t b_off[4], bs_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t r = (MODE == kGateUp ? (j < 2 ? 0 : a.I) + 16 * (j & 1) : 16 * j) + c;
    b_off[j] = (uint32_t)(r * kbytes) + g * (KB / 8);
    // a K iteration of a 16-row tile is KB contiguous scale bytes (KB / 128 blocks)
    bs_off[j] = (uint32_t)((r >> 4) * K + (r & 15) * 8) + (KB == 256 ? (g >> 1) * 128 + 4 * (g & 1) : 2 * g);
  }

  // down epilogue: the output row of thread tid (pair tid / 16) and its weight,
  // loaded now so that the epilogue does not wait for them
  const int erow = tid >> 4;
  const int64_t ep_pair = (MODE == kDown && erow < Me) ? (int64_t)a.sorted[off + erow] : 0;
  const float ep_w = (MODE == kDown && erow < Me) ? a.topk_w[ep_pair] : 0.0f;

  auto load = [&](int it, It& d) {
    const uint8_t* ab = a.a_codes + (int64_t)it * (KB / 2);
    const uint8_t* asb = a.a_scales + (int64_t)it * (KB / 16);
    const uint8_t* bb = b_code_base + (int64_t)it * (KB / 2);
    const uint8_t* bsb = b_scale_base + (int64_t)it * KB;
#pragma unroll
    for (int q = 0; q < kDw / 4; ++q) d.ac[q] = *reinterpret_cast<const u32x4_t*>(ab + a_off + 16 * q);
    const uint32_t asv = load_scales<KB>(asb + as_off);
    d.as = a_valid ? asv : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < kDw / 4; ++q)
        d.bc[j][q] = load_stream(reinterpret_cast<const u32x4_t*>(bb + b_off[j] + 16 * q));
      d.bs[j] = load_scales<KB>(bsb + bs_off[j]);
    }
  };

  float4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const It& d) {
#pragma unroll
    for (int s = 0; s < kDw; ++s) {
      const int sbyte = s >> 1;  // two dwords (16 codes) per scale block
      const half8_t af = decode8(d.ac[s >> 2][s & 3], scale_pair(d.as, sbyte));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t bf = decode8(d.bc[j][s >> 2][s & 3], scale_pair(d.bs[j], sbyte));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[j], 0, 0, 0);
      }
    }
  };

  // wave w takes K iterations w, w + 4, ...: at any time the four waves read
  // neighbouring lines of each weight row; the next iteration's loads are in
  // flight while the current one is decoded and multiplied
  const int nit = (int)(K / KB);
  if (wave < nit) {
    // Two buffers in turn, no copy between them (a copy of registers a load
    // is still writing waits for that load), and the last iteration on a path
    // of its own: every compute that has a prefetch in flight behind it waits
    // only for its own loads.
    It b0, b1;
    load(wave, b0);
    for (int it = wave;;) {
      if (it + 4 >= nit) {
        compute(b0);
        break;
      }
      load(it + 4, b1);
      compute(b0);
      it += 4;
      if (it + 4 >= nit) {
        compute(b1);
        break;
      }
      load(it + 4, b0);
      compute(b1);
      it += 4;
    }
  }

  // reduce the four waves' partial tiles in a fixed order
  __shared__ float part[4][4][64][4];  // [wave][subtile][lane][reg]
  __shared__ float tilebuf[16][64 + 4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][j][lane][r] = acc[j][r];
  __syncthreads();
  {
    const int j = tid >> 6, l = tid & 63;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = ((part[0][j][l][r] + part[1][j][l][r]) + part[2][j][l][r]) + part[3][j][l][r];
      tilebuf[4 * (l >> 4) + r][16 * j + (l & 15)] = v;  // row = pair, col = subtile column
    }
  }
  __syncthreads();

  if (MODE == kGateUp) {
    // 16 rows x 2 blocks of 16 h columns; tilebuf cols 0..31 = gate, 32..63 = up
    if (tid < 32) {
      const int row = tid >> 1, blk = tid & 1;
      if (row < Me) {
        const float alpha_g = 1.0f / (a.a_gs[0] * a.b_gs[2 * e]);
        const float alpha_u = 1.0f / (a.a_gs[0] * a.b_gs[2 * e + 1]);
        float h[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float gv = tilebuf[row][16 * blk + i] * alpha_g;
          const float uv = tilebuf[row][32 + 16 * blk + i] * alpha_u;
          h[i] = silu(gv) * uv;
        }
        uint32_t lo, hi;
        const uint32_t sc = quantize_block16(h, a.h_gs[e], lo, hi);
        const int64_t hrow = off + row;
        const int64_t hcol = (int64_t)tile * 32 + 16 * blk;
        *reinterpret_cast<uint2*>(a.h_codes + hrow * (a.I / 2) + hcol / 2) = make_uint2(lo, hi);
        a.h_scales[hrow * (a.I / 16) + hcol / 16] = (uint8_t)sc;
      }
    }
  } else {
    const int q = tid & 15;  // 4 consecutive columns per thread, row erow
    const float alpha = 1.0f / (a.a_gs[e] * a.b_gs[e]);
    float f[4];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = tilebuf[erow][4 * q + i] * alpha;
      ss += f[i] * f[i];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 16);
    if (erow < Me) {
      float sc;
      const float m = ep_w * pair_row_scale(ep_w, a.K, alpha, sc);  // w_p 2^-E, exact
      half4_t out;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = (_Float16)(m * f[i]);
      *reinterpret_cast<half4_t*>(reinterpret_cast<_Float16*>(a.pair_out) + ep_pair * a.H + (int64_t)tile * 64 + 4 * q) =
          out;
      if (tile == 0 && q == 0) a.pair_scale[ep_pair] = sc;
      if (a.sq_part != nullptr && q == 0) a.sq_part[ep_pair * a.n_part + tile] = ss;
    }
  }
}

// ---------------------------------------------------------------------------
// tiled kernel
//
// Four waves, each owning a 128 x 128 block of 16 accumulator tiles.  A full
// tile is 256 pair rows x 256 weight rows (waves 2 x 2).  An expert's last
// m-tile with at most 128 rows is run wide instead: 128 pair rows x 512 weight
// rows (n-tile nt and a partner n-tile, waves 1 x 4 over the weight rows), and
// the workgroups of the partner n-tiles exit, so no MFMA work goes to the
// empty half; one of at most 64 rows runs as a half tile, 64 x 512, with half
// the MFMA work.  Workgroups go to the 8 XCDs in turn by linear id; the partner
// is chosen so that the working workgroups stay spread over all XCDs: with the
// XCD-aware tile order (a multiple of 8 n-tiles) it is the n-tile half a
// quarter away inside the same XCD's quarter, otherwise nt + gx / 2.

// SHAPE 0: full tile, 256 pair rows x 256 weight rows (waves 2 x 2 of 128 x 128);
// 1: wide, 128 x 512 (waves 1 x 4 of 128 x 128); 2: half, 64 x 512 (waves
// 1 x 4 of 64 x 128, half the MFMA work of the others).
template <int SHAPE>
struct TileShape {
  static constexpr bool kWide = SHAPE != 0;                             // two n-tiles
  static constexpr int kARows = SHAPE == 0 ? 256 : SHAPE == 1 ? 128 : 64;  // pair rows (A)
  static constexpr int kBRows = SHAPE == 0 ? 256 : 512;                 // weight rows (B)
  static constexpr int NA = (SHAPE == 0 ? kARows / 2 : kARows) / 32;   // A fragments per wave: 4, 4, 2
  static constexpr int NS = SHAPE == 0 ? 4 : 3;                         // ring stages of 128 k
  // codes: [row][4 slots of 16 B], chunk c of row r in slot c ^ ((r >> 2) & 3):
  // 16 lanes reading one chunk of 16 consecutive rows, and the 16 lanes of a
  // DMA group writing the 4 chunks of 4 consecutive rows, each touch 16
  // distinct 16-byte bank groups (64 banks); scales: [row][8 B]
  static constexpr int kACodeBytes = kARows * 64;
  static constexpr int kAScaleBytes = kARows * 8;
  static constexpr int kBCodeBytes = kBRows * 64;
  static constexpr int kBScaleBytes = kBRows * 8;
  static constexpr int kStage = kACodeBytes + kAScaleBytes + kBCodeBytes + kBScaleBytes;
  static constexpr int kHcols = kBRows / 2;     // gate_up: h columns per tile
  static constexpr int kHStride = kHcols + 4;   // floats per LDS row of h
  static constexpr int kHBytes = kARows * kHStride * 4;
  static constexpr int kBody = NS * kStage > kHBytes ? NS * kStage : kHBytes;
  // down epilogue: pair ids and weights, then the per-lane row sums of f^2 (4 waves x 32 lanes for wide tiles,
  // 2 x 32 for full ones), rows padded to kARows + 4 floats
  static constexpr int kSqLdsBytes = 2 * kARows * 4 + (kWide ? 4 : 2) * 32 * (kARows + 4) * 4;
  static_assert(kSqLdsBytes <= kBody, "down epilogue LDS");
  // DMA instructions per wave per stage: 16-byte code loads cover 16 rows,
  // 4-byte scale loads cover 32 rows.  The half tile's 64 rows of A scales
  // are two such loads; waves w and w + 2 both issue the one for rows
  // 32 (w % 2) .., writing the same bytes, so every wave issues as many
  // loads as the others.
  static constexpr int kACodeOps = kARows / 64, kAScaleOps = kARows >= 128 ? kARows / 128 : 1;
  static constexpr int kBCodeOps = kBRows / 64, kBScaleOps = kBRows / 128;
  static constexpr int kLoadsPerStage = kACodeOps + kAScaleOps + kBCodeOps + kBScaleOps;
};
constexpr int max3(int x, int y, int z) { return x > y ? (x > z ? x : z) : (y > z ? y : z); }
struct Tiled {
  static constexpr int BM = 256, BN = 256, kHcols = 128;  // the full tile: m-tile height, n-tile width
  static constexpr int kLds = max3(TileShape<0>::kBody, TileShape<1>::kBody, TileShape<2>::kBody);
};
static_assert(TileShape<0>::kHcols == Tiled::kHcols && TileShape<0>::kBRows == Tiled::BN &&
                  TileShape<0>::kARows == Tiled::BM, "full tile shape");
static_assert(Tiled::kLds <= 160 * 1024, "LDS");

// One tile: expert e's pair rows off + row0 .. off + row0 + rows_here - 1
// (rows of the expert-sorted pair order) against n-tile nt (and nt2 when WIDE).
template <int MODE, int SHAPE>
__device__ __forceinline__ void tiled_tile(const FfnArgs& a, int nt, int nt2, int e, int row0, int off,
                                           int rows_here) {
  using S = TileShape<SHAPE>;
  constexpr bool WIDE = S::kWide;
  constexpr int NS = S::NS, NA = S::NA;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: kept in scalar registers
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  // this wave's first A row and first B row inside the tile
  const int a_row0 = WIDE ? 0 : 128 * wm;
  const int b_row0 = WIDE ? 256 * wm + 128 * wn : 128 * wn;
  const int64_t K = a.K, kbytes = K / 2, kscales = K / 16;

  // ---- per-lane DMA sources.  Rows past rows_here read the tile's first row:
  // their MFMA output rows are never stored.
  auto a_row = [&](int m) -> int64_t {
    const int mm = m < rows_here ? m : 0;
    return (MODE == kGateUp) ? (int64_t)(a.sorted[off + row0 + mm] / a.k) : (int64_t)(off + row0 + mm);
  };
  // B rows 0..255 belong to n-tile nt, rows 256..511 (WIDE) to n-tile nt2.
  // gate_up: each 128-row wave block holds 64 gate rows then the 64 up rows of
  // the same h columns (so SwiGLU pairs meet in one wave's registers)
  auto b_row = [&](int n) -> int64_t {
    const int64_t ntile = n < 256 ? nt : nt2;
    const int nl = n % 256;
    if (MODE == kGateUp) {
      const int wv = nl / 128, j = (nl % 128) / 32, cc = nl % 32;
      const int64_t col = ntile * Tiled::kHcols + wv * 64 + 32 * (j % 2) + cc;
      return (int64_t)e * 2 * a.I + (j < 2 ? 0 : a.I) + col;
    } else {
      return (int64_t)e * a.H + ntile * Tiled::BN + nl;
    }
  };
  // DMA sources: a wave-uniform base per operand that advances with the stage
  // plus a 32-bit lane offset fixed for the kernel (B offsets are relative to
  // the expert's first row).
  // 16-byte code DMA i of this wave: rows 16 q .. 16 q + 15 with q = 4 i + wave;
  // lane -> row 16 q + lane / 4, LDS slot lane % 4 holding chunk slot ^ ((row >> 2) & 3)
  const int64_t erow0 = MODE == kGateUp ? (int64_t)e * 2 * a.I : (int64_t)e * a.H;  // expert's first B row
  const uint8_t* b_code_expert = a.b_codes + erow0 * kbytes;
  const uint8_t* b_scale_expert = a.b_scales + (erow0 >> 4) * K;  // tiled scales; erow0 % 16 == 0
  uint32_t a_code_off[S::kACodeOps], b_code_off[S::kBCodeOps];
#pragma unroll
  for (int i = 0; i < S::kACodeOps; ++i) {
    const int row = 16 * (4 * i + wave) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    a_code_off[i] = (uint32_t)(a_row(row) * kbytes) + 16 * chunk;
  }
#pragma unroll
  for (int i = 0; i < S::kBCodeOps; ++i) {
    const int row = 16 * (4 * i + wave) + (lane >> 2);
    const int chunk = (lane & 3) ^ ((row >> 2) & 3);
    b_code_off[i] = (uint32_t)((b_row(row) - erow0) * kbytes) + 16 * chunk;
  }
  // 4-byte scale DMA i of this wave: rows 32 q .. 32 q + 31, q = 4 i + wave (A of the half tile: q = wave % 2);
  // lane -> row 32 q + lane / 2, dword lane % 2
  auto a_scale_block = [&](int i) -> int {  // the 32-row block of A-scale DMA i
    if constexpr (S::kARows >= 128) return 4 * i + wave;
    else return (4 * i + wave) % (S::kARows / 32);
  };
  uint32_t a_scale_off[S::kAScaleOps], b_scale_off[S::kBScaleOps];
#pragma unroll
  for (int i = 0; i < S::kAScaleOps; ++i) {
    const int row = 32 * a_scale_block(i) + (lane >> 1);
    a_scale_off[i] = (uint32_t)(a_row(row) * kscales) + 4 * (lane & 1);
  }
#pragma unroll
  for (int i = 0; i < S::kBScaleOps; ++i) {
    const int64_t br = b_row(32 * (4 * i + wave) + (lane >> 1)) - erow0;
    b_scale_off[i] = (uint32_t)tiled_scale_index(br, 0, K) + 4 * (lane & 1);  // tiled: 128 B per stage
  }

  float16_t acc[NA][4];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  // this lane's LDS byte offsets inside a stage
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const uint32_t a_lane = (uint32_t)(a_row0 + r) * 64u;
  const uint32_t b_lane = (uint32_t)(S::kACodeBytes + S::kAScaleBytes) + (uint32_t)(b_row0 + r) * 64u;
  const uint32_t as_lane = (uint32_t)S::kACodeBytes + (uint32_t)(a_row0 + r) * 8u + 4u * g;
  const uint32_t bs_lane =
      (uint32_t)(S::kACodeBytes + S::kAScaleBytes + S::kBCodeBytes) + (uint32_t)(b_row0 + r) * 8u + 4u * g;
  // rows read by this lane are r + multiples of 32, so (row >> 2) & 3 == (r >> 2) & 3
  const uint32_t slot_q0 = (uint32_t)((2 * g) ^ ((r >> 2) & 3)), slot_q1 = (uint32_t)((2 * g + 1) ^ ((r >> 2) & 3));

  // Pipelined ring.  The DMA is issued as inline asm, so the compiler issues
  // the fragment reads itself, with per-read lgkmcnt waits, and never drains
  // the DMA still in flight.  Each 128-k stage is two halves of four 16-k
  // sub-steps: the second half's code words are read during the first half,
  // and after the one barrier per stage (mid-stage) the next stage's
  // first-half words and scales are read during the second half.  The decode
  // of sub-step n + 1 runs beside the 16 MFMAs of sub-step n throughout,
  // across stage boundaries too.
  //
  // Ring: the prologue fills all NS slots.  At the mid-stage barrier of stage
  // st every wave has finished its reads of slot st % NS (lgkmcnt(0) before
  // the barrier) and waited for its DMA of stage st + 1, so stage st + NS can
  // go into slot st % NS from then on.  Its DMA is spread over the four
  // sub-steps of the second half, a quarter each, between the MFMAs: issued
  // in one block after the barrier, the DMA of all four waves queued in the
  // address unit at once and held up every wave's MFMAs (gate_up 4.6% slower).
  const int64_t nst = K / 128;
  constexpr int L = S::kLoadsPerStage;
  static_assert((NS - 1) * L < 64, "vmcnt range");
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane((uint32_t)wave);
  // DMA ops lo .. hi - 1 of stage st, in the order A codes, A scales, B codes,
  // B scales (L ops in all)
  auto issue_ops = [&](int64_t st, auto lo_c, auto hi_c) {
    constexpr int lo = decltype(lo_c)::value, hi = decltype(hi_c)::value;
    constexpr int o1 = S::kACodeOps, o2 = o1 + S::kAScaleOps, o3 = o2 + S::kBCodeOps;
    const uint32_t sb = __builtin_amdgcn_readfirstlane(lds_base + (uint32_t)(st % NS) * (uint32_t)S::kStage);
    const uint8_t* ac = a.a_codes + st * 64;  // 128 k per stage
    const uint8_t* as = a.a_scales + st * 8;
    const uint8_t* bc = b_code_expert + st * 64;
    const uint8_t* bs = b_scale_expert + st * 128;
#pragma unroll
    for (int o = lo; o < hi; ++o) {
      if (o < o1) {
        dma16_async(ac, a_code_off[o], sb + (4 * o + wave_u) * 1024u);
      } else if (o < o2) {
        const uint32_t blk = S::kARows >= 128 ? 4u * (uint32_t)(o - o1) + wave_u : wave_u % (uint32_t)(S::kARows / 32);
        dma4_async(as, a_scale_off[o - o1], sb + (uint32_t)S::kACodeBytes + blk * 256u);
      } else if (o < o3) {
        dma16_async(bc, b_code_off[o - o2],
                    sb + (uint32_t)(S::kACodeBytes + S::kAScaleBytes) + (4 * (o - o2) + wave_u) * 1024u);
      } else {
        dma4_async(bs, b_scale_off[o - o3],
                   sb + (uint32_t)(S::kACodeBytes + S::kAScaleBytes + S::kBCodeBytes) + (4 * (o - o3) + wave_u) * 256u);
      }
    }
  };
  using std::integral_constant;
  auto issue_async = [&](int64_t st) { issue_ops(st, integral_constant<int, 0>{}, integral_constant<int, L>{}); };
  // this lane's fragment words of one half (fragment i of a row block sits
  // 2048 B = 32 rows after fragment i-1) and its scale words (256 B apart)
  auto load_half = [&](int64_t st, uint32_t slot, u32x4_t* fa, u32x4_t* fb) {
    const uint32_t sb = (uint32_t)(st % NS) * (uint32_t)S::kStage;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      fa[i] = *reinterpret_cast<const u32x4_t*>(smem + sb + a_lane + 16u * slot + 2048u * i);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j] = *reinterpret_cast<const u32x4_t*>(smem + sb + b_lane + 16u * slot + 2048u * j);
  };
  auto load_scales = [&](int64_t st, uint32_t* sa, uint32_t* sbv) {
    const uint32_t sb = (uint32_t)(st % NS) * (uint32_t)S::kStage;
#pragma unroll
    for (int i = 0; i < NA; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(smem + sb + as_lane + 256u * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) sbv[j] = *reinterpret_cast<const uint32_t*>(smem + sb + bs_lane + 256u * j);
  };
  // sub-step ss (q = ss / 4 half, dword ss % 4) uses scale byte 2 q + (ss % 4) / 2 of the lane's word
  half8_t da[2][NA], db[2][4];
  auto decode = [&](int buf, const u32x4_t* fa, const u32x4_t* fb, int w, const uint32_t* sa, const uint32_t* sbv,
                    int sbyte) {
#pragma unroll
    for (int i = 0; i < NA; ++i) da[buf][i] = decode8(fa[i][w], scale_pair(sa[i], sbyte));
#pragma unroll
    for (int j = 0; j < 4; ++j) db[buf][j] = decode8(fb[j][w], scale_pair(sbv[j], sbyte));
  };
  // the 16 MFMAs of a sub-step, each followed by a slice of the next
  // sub-step's decode and, for the first n_ds, by one of the LDS reads just
  // issued in program order (so they go out early instead of just before use)
  // (the half tile: 8 MFMAs per sub-step beside 6 decoded fragments, so 7 VALU slots each)
  constexpr int kValuSlots = NA == 4 ? 6 : 7;
  auto mfma16 = [&](int buf, int n_ds) {
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(da[buf][i], db[buf][j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int m = 0; m < 4 * NA; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      if (m < n_ds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      __builtin_amdgcn_sched_group_barrier(0x002, kValuSlots, 0);  // VALU
    }
  };

#pragma unroll
  for (int p = 0; p < NS; ++p)
    if (p < nst) issue_async(p);
  // stage 0 has landed; up to NS - 1 later stages may stay in flight
  {
    const int64_t later = nst - 1 < NS - 1 ? nst - 1 : NS - 1;
    if (later >= 3) wait_vmcnt<3 * L>();
    else if (later == 2) wait_vmcnt<2 * L>();
    else if (later == 1) wait_vmcnt<L>();
    else wait_vmcnt<0>();
  }
  barrier_after_lds();
  u32x4_t c0a[NA], c0b[4];
  uint32_t sa[NA], sbv[4];
  load_half(0, slot_q0, c0a, c0b);
  load_scales(0, sa, sbv);
  decode(0, c0a, c0b, 0, sa, sbv, 0);
  // One stage; MORE: a stage follows, ISSUE: stage st + NS exists.  The
  // loop is peeled on both so the steady-state body has no branch, and the
  // compiler's LDS wait counts stay exact.
  auto stage = [&](int64_t st, auto more_c, auto issue_c) {
    constexpr bool kMore = decltype(more_c)::value, kIssue = decltype(issue_c)::value;
    // Each sub-step is its own scheduling region (sched_barrier), so no
    // decode, and no scale convert in particular, is hoisted next to the
    // LDS read it depends on; the reads are issued at the top of a half.
    u32x4_t c1a[NA], c1b[4];
    __builtin_amdgcn_sched_barrier(0);
    load_half(st, slot_q1, c1a, c1b);
#pragma unroll
    for (int ss = 0; ss < 4; ++ss) {
      if (ss > 0) __builtin_amdgcn_sched_barrier(0);
      if (ss < 3) decode((ss + 1) & 1, c0a, c0b, ss + 1, sa, sbv, (ss + 1) >> 1);
      else decode(0, c1a, c1b, 0, sa, sbv, 2);
      mfma16(ss & 1, ss == 0 ? (NA + 4 < 8 ? NA + 4 : 8) : 0);
    }
    u32x4_t n0a[NA], n0b[4];
    uint32_t nsa[NA], nsb[4];
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kMore) {
      // stage st + 1 has landed; the stages issued after it (up to NS - 2) may stay in flight
      const int64_t ahead = nst - 2 - st;
      if (kIssue || ahead >= NS - 2) wait_vmcnt<(NS - 2) * L>();
      else if (ahead == 1) wait_vmcnt<L>();
      else wait_vmcnt<0>();
      barrier_after_lds();
      load_half(st + 1, slot_q0, n0a, n0b);
      load_scales(st + 1, nsa, nsb);
    }
#pragma unroll
    for (int ss = 4; ss < 8; ++ss) {
      if (ss > 4) __builtin_amdgcn_sched_barrier(0);
      if constexpr (kIssue) {
        if (ss == 4) issue_ops(st + NS, integral_constant<int, 0>{}, integral_constant<int, L / 4>{});
        else if (ss == 5) issue_ops(st + NS, integral_constant<int, L / 4>{}, integral_constant<int, L / 2>{});
        else if (ss == 6) issue_ops(st + NS, integral_constant<int, L / 2>{}, integral_constant<int, 3 * L / 4>{});
        else issue_ops(st + NS, integral_constant<int, 3 * L / 4>{}, integral_constant<int, L>{});
      }
      if (ss < 7) {
        decode((ss + 1) & 1, c1a, c1b, (ss + 1) & 3, sa, sbv, 2 + (((ss + 1) & 3) >> 1));
      } else if (kMore) {
        // Pin the next stage's words here: instruction selection would
        // otherwise place their (pure) converts right after the reads, and
        // the wave would wait for the LDS there.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < NA) asm volatile("" : "+v"(nsa[i]));
          asm volatile("" : "+v"(nsb[i]));
          if (i < NA) asm volatile("" : "+v"(n0a[i]));
          asm volatile("" : "+v"(n0b[i]));
        }
        decode(0, n0a, n0b, 0, nsa, nsb, 0);
      }
      mfma16(ss & 1, (kMore && ss == 4) ? 12 : 0);
    }
    if constexpr (kMore) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i < NA) c0a[i] = n0a[i];
        c0b[i] = n0b[i];
        if (i < NA) sa[i] = nsa[i];
        sbv[i] = nsb[i];
      }
    }
  };
  int64_t st = 0;
  for (; st + NS < nst; ++st) stage(st, std::true_type{}, std::true_type{});
  for (; st + 1 < nst; ++st) stage(st, std::true_type{}, std::false_type{});
  stage(st, std::false_type{}, std::false_type{});
  wait_vmcnt<0>();  // nothing is in flight here; the epilogue's barrier does not know of the asm DMA
  __syncthreads();  // every wave is done with the ring before the epilogue reuses the LDS

  // ---- epilogues.  acc[i][j][q]: tile row a_row0 + 32 i + 8 (q/4) + 4 g + q%4,
  // tile column b_row0 + 32 j + r
  if (MODE == kGateUp) {
    float* hbuf = reinterpret_cast<float*>(smem);
    const float alpha_g = 1.0f / (a.a_gs[0] * a.b_gs[2 * e]);
    const float alpha_u = 1.0f / (a.a_gs[0] * a.b_gs[2 * e + 1]);
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = a_row0 + 32 * i + 8 * (q >> 2) + 4 * g + (q & 3);
          const int hc = b_row0 / 2 + 32 * j + r;  // h column inside the tile
          const float gv = acc[i][j][q] * alpha_g;
          const float uv = acc[i][j + 2][q] * alpha_u;
          hbuf[row * S::kHStride + hc] = silu(gv) * uv;
        }
    __syncthreads();
    const float gsh = a.h_gs[e];
    constexpr int kBlkPerRow = S::kHcols / 16;
    // 8 independent blocks per thread, unrolled so that one block's LDS reads
    // overlap another's arithmetic (one wave per SIMD)
#pragma unroll 4
    for (int b = tid; b < S::kARows * kBlkPerRow; b += 256) {
      const int row = b / kBlkPerRow, cb = b % kBlkPerRow;
      if (row >= rows_here) continue;
      float h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = hbuf[row * S::kHStride + 16 * cb + i];
      uint32_t lo, hi;
      const uint32_t sc = quantize_block16(h, gsh, lo, hi);
      const int64_t hrow = off + row0 + row;
      // h columns 0..127 of the tile belong to n-tile nt, 128..255 (WIDE) to nt2
      const int64_t hcol = (int64_t)(cb < 8 ? nt : nt2) * Tiled::kHcols + 16 * (cb % 8);
      *reinterpret_cast<uint2*>(a.h_codes + hrow * (a.I / 2) + hcol / 2) = make_uint2(lo, hi);
      a.h_scales[hrow * (a.I / 16) + hcol / 16] = (uint8_t)sc;
    }
  } else {
    // The lane's column r and row half g again, from the hardware lane id:
    // values derived from threadIdx.x at the top would be held across the loop.
    const int lane_e = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int r = lane_e & 31, g = lane_e >> 5;
    // the tile's pair ids and weights w_p 2^-E (E: the row's scale exponent), staged once in the (now free)
    // ring; the workgroup of n-tile 0 writes the rows' scales 2^E
    const float alpha = 1.0f / (a.a_gs[e] * a.b_gs[e]);
    int32_t* prow = reinterpret_cast<int32_t*>(smem);
    float* wrow = reinterpret_cast<float*>(smem + S::kARows * 4);
    for (int t = tid; t < S::kARows; t += 256) {
      const int32_t p = t < rows_here ? a.sorted[off + row0 + t] : 0;
      prow[t] = p;
      float m = 0.0f;
      if (t < rows_here) {
        const float wp = a.topk_w[p];
        float sc;
        m = wp * pair_row_scale(wp, a.K, alpha, sc);
        if (nt == 0) a.pair_scale[p] = sc;
      }
      wrow[t] = m;
    }
    // Each lane's sums of f^2 over its 4 columns, by row: sql[slot][r][row],
    // slot = wn (full tiles; wm picks the rows) or the wave (wide tiles: wm is
    // the n-tile), rows padded to a stride of kARows + 4 floats so that the
    // 16-byte writes of 16 consecutive lanes cover all 64 banks.  After the
    // barrier thread t adds up its row's partials in a fixed order.
    constexpr int kSqStride = S::kARows + 4;
    float* sql = reinterpret_cast<float*>(smem + 2 * S::kARows * 4);
    float* sqw = sql + ((WIDE ? wave : wn) * 32 + r) * kSqStride;
    __syncthreads();
    const int64_t col0 = (int64_t)((WIDE && wm) ? nt2 : nt) * Tiled::BN + 128 * wn;  // this wave's first column
#pragma unroll
    for (int i = 0; i < NA; ++i) {
#pragma unroll
      for (int qh = 0; qh < 4; ++qh) {
        // rows rb .. rb + 3 (q = 4 qh .. 4 qh + 3): their pair ids and scaled weights in one read each
        const int rb = a_row0 + 32 * i + 8 * qh + 4 * g;
        const int4 p4 = *reinterpret_cast<const int4*>(prow + rb);
        const float4 w4 = *reinterpret_cast<const float4*>(wrow + rb);
        float4 ss4;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int q = 4 * qh + qq, row = rb + qq;
          const int64_t p = qq == 0 ? p4.x : qq == 1 ? p4.y : qq == 2 ? p4.z : p4.w;
          const float wp = qq == 0 ? w4.x : qq == 1 ? w4.y : qq == 2 ? w4.z : w4.w;  // w_p 2^-E
          // one bounds branch per row around its four stores (a branch per
          // store made the compiler copy every accumulator out of the AGPRs
          // ahead of the first one, and spill)
          _Float16* dst = reinterpret_cast<_Float16*>(a.pair_out) + p * a.H + col0 + r;
          float ss = 0.0f, fv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            fv[j] = acc[i][j][q] * alpha;
            ss += fv[j] * fv[j];
          }
          if (row < rows_here) {
            // written once and read once by the combine: non-temporal, so the
            // weighted rows do not push the operand tiles out of L2
#pragma unroll
            for (int j = 0; j < 4; ++j) __builtin_nontemporal_store((_Float16)(wp * fv[j]), dst + 32 * j);
          }
          if (qq == 0) ss4.x = ss;
          else if (qq == 1) ss4.y = ss;
          else if (qq == 2) ss4.z = ss;
          else ss4.w = ss;
        }
        *reinterpret_cast<float4*>(sqw + rb) = ss4;
      }
    }
    __syncthreads();
    if (a.sq_part != nullptr) {
      // row t's sum: the 32 column lanes of each of its two waves in order, then the two waves
      auto row_sum = [&](int slot0, int row) -> float {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll 8
        for (int c = 0; c < 32; ++c) {
          s0 += sql[(slot0 * 32 + c) * kSqStride + row];
          s1 += sql[((slot0 + 1) * 32 + c) * kSqStride + row];
        }
        return s0 + s1;
      };
      if (WIDE) {
        const int h = tid / S::kARows, row = tid % S::kARows;  // 2 n-tiles x kARows rows (of 256 threads)
        if (h < 2 && row < rows_here) a.sq_part[(int64_t)prow[row] * a.n_part + (h ? nt2 : nt)] = row_sum(2 * h, row);
      } else if (tid < rows_here) {
        a.sq_part[(int64_t)prow[tid] * a.n_part + nt] = row_sum(0, tid);
      }
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(256) void ffn_tiled_kernel(FfnArgs a) {
  const int gx = (int)gridDim.x;  // n-tiles; gridDim.y = m-tile slots (even)
  int nt, mt, half;
  if ((gx & 7) == 0) {
    // Workgroups go to the 8 XCDs in turn by linear id L, and each XCD starts
    // its own in increasing order: XCD c = L % 8 runs its s-th workgroup
    // s = L / 8.  (c, s) maps to m-tile 2 (s / q) + c / 4 and n-tile
    // (c % 4) q + s % q, q = gx / 4: XCD c takes every other m-tile and one
    // quarter of the n-tiles, so each m-tile's activations are fetched by 4
    // of the 8 L2s instead of all 8, and each weight n-tile by 2 instead of 1.
    const int L = (int)blockIdx.x + gx * (int)blockIdx.y;
    const int c = L & 7, s = L >> 3, q = gx >> 2;
    const int mi = s / q, nn = s - mi * q;
    mt = 2 * mi + (c >> 2);
    nt = (c & 3) * q + nn;
    // a half-empty m-tile pairs n-tiles inside the XCD's quarter
    half = nn < (q >> 1) ? (q >> 1) : -(q >> 1);
  } else {  // fewer than 8 n-tiles, or not a multiple of 8: the launch order
    nt = (int)blockIdx.x;
    mt = (int)blockIdx.y;
    half = nt < (gx >> 1) ? (gx >> 1) : -(gx >> 1);
  }
  // one load for the tile's expert, first pair row and row count
  const int4 ti = reinterpret_cast<const int4*>(a.tile_info)[mt];
  const int rows_here = ti.z;
  if (rows_here <= 0) return;  // past the last m-tile
  const int e = ti.x, row0 = 0, off = ti.y;
  // A half-empty m-tile runs wide over n-tile nt and its partner nt + half (the
  // lower one of each pair works, the upper one exits), as 128 rows or, with
  // at most 64 rows, as the half tile.  The n-tile count (or the quarter q) is
  // even whenever this applies.
  const bool wide = rows_here <= 128 && (gx & 1) == 0;
  if (wide) {
    if (half < 0) return;
    if (rows_here <= 64) tiled_tile<MODE, 2>(a, nt, nt + half, e, row0, off, rows_here);
    else tiled_tile<MODE, 1>(a, nt, nt + half, e, row0, off, rows_here);
  } else {
    tiled_tile<MODE, 0>(a, nt, nt, e, row0, off, rows_here);
  }
}

// ---------------------------------------------------------------------------
// schedule + final reduction kernels

// m-tile schedule from the device-side expert offsets: slot i of the first
// sum_e ceil(n_e / BM) holds {expert, first pair row, rows (<= BM), 0} in
// expert order, the remaining slots up to n_slots hold rows 0.
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E, int BM,
                                                          int n_slots, int32_t* __restrict__ tile_info) {
  __shared__ int32_t base[257];
  const int e = threadIdx.x;
  const int cnt = (e < E) ? (offsets[e + 1] - offsets[e]) : 0;
  const int nt = (cnt + BM - 1) / BM;
  base[e] = nt;
  __syncthreads();
  if (e == 0) {
    int run = 0;
    for (int i = 0; i < E; ++i) {
      const int v = base[i];
      base[i] = run;
      run += v;
    }
    base[E] = run;
  }
  __syncthreads();
  int4* info = reinterpret_cast<int4*>(tile_info);
  if (e < E)
    for (int i = 0; i < nt; ++i) {
      const int rows = cnt - i * BM < BM ? cnt - i * BM : BM;
      info[base[e] + i] = make_int4(e, offsets[e] + i * BM, rows, 0);
    }
  for (int i = base[E] + e; i < n_slots; i += 256) info[i] = make_int4(0, 0, 0, 0);
}

__global__ void sq_reduce_kernel(const float* __restrict__ part, int64_t npairs, int n_part, float* __restrict__ out) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= npairs) return;
  float s = 0.0f;
#pragma unroll 8
  for (int i = 0; i < n_part; ++i) s += part[p * n_part + i];  // fixed order
  out[p] = s;
}

// ---------------------------------------------------------------------------
// host side

// m-tile slots: an upper bound on sum_e ceil(n_e / BM), rounded up to even (the XCD-aware tile order pairs them)
int64_t ffn_max_tiles(int64_t T, int64_t k, int64_t E) {
  const int64_t n = (T * k + Tiled::BM - 1) / Tiled::BM + E;
  return n + (n & 1);
}
int ffn_sq_parts(int64_t H) { return (int)(H / 64); }  // small kernel: 64-column tiles (the finest split)
bool ffn_use_small(int64_t T) { return T <= kSmallRows; }

hipError_t launch_ffn_stage(int mode, FfnArgs a, int64_t T, int64_t E, bool build_schedule, hipStream_t st) {
  if (ffn_use_small(T)) {
    const bool k256 = (a.K % 256) == 0;  // else K % 128 == 0
    const dim3 grid = mode == kGateUp ? dim3((unsigned)(a.I / 32), (unsigned)E) : dim3((unsigned)(a.H / 64), (unsigned)E);
    if (mode == kGateUp) {
      if (k256) hipLaunchKernelGGL((ffn_small_kernel<kGateUp, 256>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((ffn_small_kernel<kGateUp, 128>), grid, dim3(256), 0, st, a);
    } else {
      if (k256) hipLaunchKernelGGL((ffn_small_kernel<kDown, 256>), grid, dim3(256), 0, st, a);
      else hipLaunchKernelGGL((ffn_small_kernel<kDown, 128>), grid, dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  if (build_schedule) {
    // m-tile schedule from the device-side expert offsets (no host readback)
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, st, a.offsets, (int)E, Tiled::BM,
                       (int)ffn_max_tiles(T, a.k, E), const_cast<int32_t*>(a.tile_info));
  }
  const unsigned gy = (unsigned)ffn_max_tiles(T, a.k, E);
  // the tiles need more than the default 64 KiB of dynamic LDS
  if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&ffn_tiled_kernel<kGateUp>), Tiled::kLds))
    return e;
  if (hipError_t e = set_max_dynamic_lds(reinterpret_cast<const void*>(&ffn_tiled_kernel<kDown>), Tiled::kLds))
    return e;
  if (mode == kGateUp) {
    const unsigned gx = (unsigned)(a.I / Tiled::kHcols);
    hipLaunchKernelGGL(ffn_tiled_kernel<kGateUp>, dim3(gx, gy), dim3(256), Tiled::kLds, st, a);
  } else {
    const unsigned gx = (unsigned)(a.H / Tiled::BN);
    hipLaunchKernelGGL(ffn_tiled_kernel<kDown>, dim3(gx, gy), dim3(256), Tiled::kLds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_sq_reduce(const float* part, int64_t npairs, int n_part, float* out, hipStream_t st) {
  if (npairs == 0) return hipSuccess;
  hipLaunchKernelGGL(sq_reduce_kernel, dim3((unsigned)((npairs + 255) / 256)), dim3(256), 0, st, part, npairs, n_part,
                     out);
  return hipGetLastError();
}

int ffn_tiled_bm() { return Tiled::BM; }
int ffn_tiled_hcols() { return Tiled::kHcols; }
int ffn_tiled_bn() { return Tiled::BN; }

}  // namespace moe
