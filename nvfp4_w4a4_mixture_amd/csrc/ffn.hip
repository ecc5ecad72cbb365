// Grouped NVFP4 W4A4 expert FFN on gfx950 ("K-EXAONE-152B-A23B-REAP-80E-NVFP4"
// model card, "Quantization Setup": every routed expert Linear is NVFP4 W4A4
// with its own scales; the BF16 parent's experts are SwiGLU MLPs).
//
//   stage 1 (gate_up): g, u = xhat . W_gate^T, xhat . W_up^T ; h = silu(g) * u,
//                       h re-quantized to NVFP4 with the expert's calibrated gs_h
//   stage 2 (down):    f = hhat . W_down^T ; pair_out[p] = w_p * f ; sum f^2
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
//    workgroup per (expert, 64-row weight tile); each of the four waves takes
//    a contiguous quarter of K in 256-element iterations (a full 128-byte line
//    per weight row), prefetching the next iteration into registers; weights
//    go straight from HBM to registers (each weight byte is used once),
//    16x16x32 MFMA; the waves' partial sums meet in LDS.
//  * ffn_tiled_kernel (any M): one workgroup per (m-tile of an expert's
//    pairs, n-tile of weight rows); A and B FP4 tiles staged through
//    double-buffered LDS, 32x32x16 MFMA, 2x2 waves.
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

template <int KB>
__device__ __forceinline__ uint32_t load_scales(const uint8_t* p) {
  if (KB == 256) return *reinterpret_cast<const uint32_t*>(p);
  return *reinterpret_cast<const uint16_t*>(p);
}

template <int MODE, int KB>
__global__ __launch_bounds__(256) void ffn_small_kernel(FfnArgs a) {
  using It = SmallIter<KB>;
  constexpr int kDw = It::kDw;
  const int tile = blockIdx.x;
  const int e = blockIdx.y;
  const int off = a.offsets[e];
  const int Me = a.offsets[e + 1] - off;
  if (Me <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int64_t K = a.K;
  const int64_t kbytes = K / 2, kscales = K / 16;

  // A row (pair c of this expert)
  const bool a_valid = c < Me;
  int64_t arow = 0;
  if (a_valid) arow = (MODE == kGateUp) ? (int64_t)(a.sorted[off + c] / a.k) : (int64_t)(off + c);
  const uint8_t* a_code_row = a.a_codes + arow * kbytes + g * (KB / 8);
  const uint8_t* a_scale_row = a.a_scales + arow * kscales + g * (KB / 64);
  // B rows for the 4 n-subtiles of 16 rows
  const uint8_t* b_code_row[4];
  const uint8_t* b_scale_row[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t brow;
    if (MODE == kGateUp) {
      const int64_t col = (int64_t)tile * 32 + 16 * (j & 1) + c;  // h column
      brow = (int64_t)e * 2 * a.I + (j < 2 ? 0 : a.I) + col;
    } else {
      brow = (int64_t)e * a.H + (int64_t)tile * 64 + 16 * j + c;
    }
    b_code_row[j] = a.b_codes + brow * kbytes + g * (KB / 8);
    b_scale_row[j] = a.b_scales + brow * kscales + g * (KB / 64);
  }

  auto load = [&](int64_t it, It& d) {
    const int64_t cb = it * (KB / 2), sb = it * (KB / 16);
#pragma unroll
    for (int q = 0; q < kDw / 4; ++q)
      d.ac[q] = a_valid ? *reinterpret_cast<const u32x4_t*>(a_code_row + cb + 16 * q) : u32x4_t{0, 0, 0, 0};
    d.as = a_valid ? load_scales<KB>(a_scale_row + sb) : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < kDw / 4; ++q)
        d.bc[j][q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(b_code_row[j] + cb + 16 * q));
      d.bs[j] = load_scales<KB>(b_scale_row[j] + sb);
    }
  };

  float4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = float4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const It& d) {
#pragma unroll
    for (int s = 0; s < kDw; ++s) {
      const int sbyte = s >> 1;  // two dwords (16 codes) per scale block
      const half8_t af = decode8(d.ac[s >> 2][s & 3], scale_pair((d.as >> (8 * sbyte)) & 0xFFu));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t bf = decode8(d.bc[j][s >> 2][s & 3], scale_pair((d.bs[j] >> (8 * sbyte)) & 0xFFu));
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf, acc[j], 0, 0, 0);
      }
    }
  };

  // each wave takes a contiguous range of K iterations; the next iteration's
  // loads are in flight while the current one is decoded and multiplied
  const int64_t nit = K / KB;
  const int64_t it0 = (wave * nit) / 4, it1 = ((wave + 1) * nit) / 4;
  if (it0 < it1) {
    It cur, nxt;
    load(it0, cur);
    for (int64_t it = it0; it < it1; ++it) {
      if (it + 1 < it1) load(it + 1, nxt);
      compute(cur);
      cur = nxt;
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
    const int row = tid >> 4, q = tid & 15;  // 4 consecutive columns per thread
    const float alpha = 1.0f / (a.a_gs[e] * a.b_gs[e]);
    float f[4];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = tilebuf[row][4 * q + i] * alpha;
      ss += f[i] * f[i];
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 16);
    if (row < Me) {
      const int64_t p = a.sorted[off + row];
      const float wp = a.topk_w[p];
      float4 out = make_float4(wp * f[0], wp * f[1], wp * f[2], wp * f[3]);
      *reinterpret_cast<float4*>(a.pair_out + p * a.H + (int64_t)tile * 64 + 4 * q) = out;
      if (a.sq_part != nullptr && q == 0) a.sq_part[p * a.n_part + tile] = ss;
    }
  }
}

// ---------------------------------------------------------------------------
// tiled kernel

template <int WM, int WN>
struct TiledShape {
  static constexpr int BM = 64 * WM;  // 2 waves in M, WM 32-row MFMA tiles each
  static constexpr int BN = 64 * WN;  // 2 waves in N, WN 32-col MFMA tiles each
  static constexpr int kACodeBytes = 4 * BM * 16;  // [chunk 4][row][16 B]
  static constexpr int kAScaleBytes = 2 * BM * 4;  // [group 2][row][4 B]
  static constexpr int kBCodeBytes = 4 * BN * 16;
  static constexpr int kBScaleBytes = 2 * BN * 4;
  static constexpr int kStage = kACodeBytes + kAScaleBytes + kBCodeBytes + kBScaleBytes;
  static constexpr int kHcols = BN / 2;             // gate_up: h columns per tile
  static constexpr int kHStride = kHcols + 4;       // floats per LDS row of h
  static constexpr int kHBytes = BM * kHStride * 4;
  static constexpr int kLds = (2 * kStage > kHBytes ? 2 * kStage : kHBytes) + 2 * BM * 4;
};

template <int MODE, int WM, int WN>
__global__ __launch_bounds__(256) void ffn_tiled_kernel(FfnArgs a) {
  using S = TiledShape<WM, WN>;
  constexpr int BM = S::BM, BN = S::BN;
  const int nt = blockIdx.x;
  const int mt = blockIdx.y;
  if (mt >= a.num_tiles[0]) return;
  const int e = a.tile_expert[mt];
  const int row0 = a.tile_row0[mt];
  const int off = a.offsets[e];
  const int rows_here = min(BM, a.offsets[e + 1] - off - row0);

  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, g = lane >> 5;
  const int64_t K = a.K, kbytes = K / 2, kscales = K / 16;

  // ---- per-thread global sources
  // A codes: row = (tid >> 2) + 64 * i, chunk = tid & 3
  constexpr int kARowsPerThread = BM / 64;
  const uint8_t* a_code_src[kARowsPerThread];
  bool a_ok[kARowsPerThread];
#pragma unroll
  for (int i = 0; i < kARowsPerThread; ++i) {
    const int m = (tid >> 2) + 64 * i;
    a_ok[i] = m < rows_here;
    int64_t arow = 0;
    if (a_ok[i]) arow = (MODE == kGateUp) ? (int64_t)(a.sorted[off + row0 + m] / a.k) : (int64_t)(off + row0 + m);
    a_code_src[i] = a.a_codes + arow * kbytes + 16 * (tid & 3);
  }
  // A scales: row = (tid >> 1) + 128 * i, dword = tid & 1
  constexpr int kAScalePerThread = (BM * 2 + 255) / 256;
  const uint8_t* a_scale_src[kAScalePerThread];
  bool as_ok[kAScalePerThread];
#pragma unroll
  for (int i = 0; i < kAScalePerThread; ++i) {
    const int m = (tid >> 1) + 128 * i;
    as_ok[i] = m < rows_here && m < BM;
    int64_t arow = 0;
    if (as_ok[i]) arow = (MODE == kGateUp) ? (int64_t)(a.sorted[off + row0 + m] / a.k) : (int64_t)(off + row0 + m);
    a_scale_src[i] = a.a_scales + arow * kscales + 4 * (tid & 1);
  }
  // B rows
  auto b_row = [&](int n) -> int64_t {
    if (MODE == kGateUp) {
      const int wv = n / (32 * WN), j = (n % (32 * WN)) / 32, cc = n % 32;
      const int64_t col = (int64_t)nt * S::kHcols + wv * 16 * WN + 32 * (j % (WN / 2)) + cc;
      return (int64_t)e * 2 * a.I + (j < WN / 2 ? 0 : a.I) + col;
    } else {
      return (int64_t)e * a.H + (int64_t)nt * BN + n;
    }
  };
  constexpr int kBRowsPerThread = BN / 64;
  const uint8_t* b_code_src[kBRowsPerThread];
#pragma unroll
  for (int i = 0; i < kBRowsPerThread; ++i) b_code_src[i] = a.b_codes + b_row((tid >> 2) + 64 * i) * kbytes + 16 * (tid & 3);
  constexpr int kBScalePerThread = (BN * 2 + 255) / 256;
  const uint8_t* b_scale_src[kBScalePerThread];
  bool bs_ok[kBScalePerThread];
#pragma unroll
  for (int i = 0; i < kBScalePerThread; ++i) {
    const int n = (tid >> 1) + 128 * i;
    bs_ok[i] = n < BN;
    b_scale_src[i] = a.b_scales + b_row(bs_ok[i] ? n : 0) * kscales + 4 * (tid & 1);
  }

  uint4 ra[kARowsPerThread], rb[kBRowsPerThread];
  uint32_t ras[kAScalePerThread], rbs[kBScalePerThread];
  auto gload = [&](int64_t k0) {
    const int64_t cbo = k0 / 2, sbo = k0 / 16;
#pragma unroll
    for (int i = 0; i < kARowsPerThread; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_code_src[i] + cbo) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kAScalePerThread; ++i)
      ras[i] = as_ok[i] ? *reinterpret_cast<const uint32_t*>(a_scale_src[i] + sbo) : 0u;
#pragma unroll
    for (int i = 0; i < kBRowsPerThread; ++i) rb[i] = *reinterpret_cast<const uint4*>(b_code_src[i] + cbo);
#pragma unroll
    for (int i = 0; i < kBScalePerThread; ++i)
      rbs[i] = bs_ok[i] ? *reinterpret_cast<const uint32_t*>(b_scale_src[i] + sbo) : 0u;
  };
  auto lstore = [&](int buf) {
    unsigned char* base = smem + buf * S::kStage;
    uint4* ac = reinterpret_cast<uint4*>(base);
    uint32_t* as = reinterpret_cast<uint32_t*>(base + S::kACodeBytes);
    uint4* bc = reinterpret_cast<uint4*>(base + S::kACodeBytes + S::kAScaleBytes);
    uint32_t* bsc = reinterpret_cast<uint32_t*>(base + S::kACodeBytes + S::kAScaleBytes + S::kBCodeBytes);
#pragma unroll
    for (int i = 0; i < kARowsPerThread; ++i) ac[(tid & 3) * BM + (tid >> 2) + 64 * i] = ra[i];
#pragma unroll
    for (int i = 0; i < kAScalePerThread; ++i)
      if ((tid >> 1) + 128 * i < BM) as[(tid & 1) * BM + (tid >> 1) + 128 * i] = ras[i];
#pragma unroll
    for (int i = 0; i < kBRowsPerThread; ++i) bc[(tid & 3) * BN + (tid >> 2) + 64 * i] = rb[i];
#pragma unroll
    for (int i = 0; i < kBScalePerThread; ++i)
      if (bs_ok[i]) bsc[(tid & 1) * BN + (tid >> 1) + 128 * i] = rbs[i];
  };

  float16_t acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int64_t nst = K / 128;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t st = 0; st < nst; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nst) gload((st + 1) * 128);
    const unsigned char* base = smem + buf * S::kStage;
    const uint4* ac = reinterpret_cast<const uint4*>(base);
    const uint32_t* as = reinterpret_cast<const uint32_t*>(base + S::kACodeBytes);
    const uint4* bc = reinterpret_cast<const uint4*>(base + S::kACodeBytes + S::kAScaleBytes);
    const uint32_t* bsc = reinterpret_cast<const uint32_t*>(base + S::kACodeBytes + S::kAScaleBytes + S::kBCodeBytes);
    uint32_t sa[WM], sbv[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) sa[i] = as[g * BM + wm * 32 * WM + 32 * i + r];
#pragma unroll
    for (int j = 0; j < WN; ++j) sbv[j] = bsc[g * BN + wn * 32 * WN + 32 * j + r];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint4 ca[WM], cbq[WN];
#pragma unroll
      for (int i = 0; i < WM; ++i) ca[i] = ac[(2 * g + q) * BM + wm * 32 * WM + 32 * i + r];
#pragma unroll
      for (int j = 0; j < WN; ++j) cbq[j] = bc[(2 * g + q) * BN + wn * 32 * WN + 32 * j + r];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int sbyte = 2 * q + (s >> 1);
        half8_t af[WM], bf[WN];
#pragma unroll
        for (int i = 0; i < WM; ++i) {
          const uint32_t w = s == 0 ? ca[i].x : s == 1 ? ca[i].y : s == 2 ? ca[i].z : ca[i].w;
          af[i] = decode8(w, scale_pair((sa[i] >> (8 * sbyte)) & 0xFFu));
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const uint32_t w = s == 0 ? cbq[j].x : s == 1 ? cbq[j].y : s == 2 ? cbq[j].z : cbq[j].w;
          bf[j] = decode8(w, scale_pair((sbv[j] >> (8 * sbyte)) & 0xFFu));
        }
#pragma unroll
        for (int i = 0; i < WM; ++i)
#pragma unroll
          for (int j = 0; j < WN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    if (st + 1 < nst) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogues.  acc[i][j][q]: row = wm*32*WM + 32 i + 8 (q/4) + 4 g + q%4, col = r
  if (MODE == kGateUp) {
    float* hbuf = reinterpret_cast<float*>(smem);
    const float alpha_g = 1.0f / (a.a_gs[0] * a.b_gs[2 * e]);
    const float alpha_u = 1.0f / (a.a_gs[0] * a.b_gs[2 * e + 1]);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN / 2; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = wm * 32 * WM + 32 * i + 8 * (q >> 2) + 4 * g + (q & 3);
          const int hc = wn * 16 * WN + 32 * j + r;
          const float gv = acc[i][j][q] * alpha_g;
          const float uv = acc[i][j + WN / 2][q] * alpha_u;
          hbuf[row * S::kHStride + hc] = silu(gv) * uv;
        }
    __syncthreads();
    const float gsh = a.h_gs[e];
    constexpr int kBlkPerRow = S::kHcols / 16;
    for (int b = tid; b < BM * kBlkPerRow; b += 256) {
      const int row = b / kBlkPerRow, cb = b % kBlkPerRow;
      if (row >= rows_here) continue;
      float h[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) h[i] = hbuf[row * S::kHStride + 16 * cb + i];
      uint32_t lo, hi;
      const uint32_t sc = quantize_block16(h, gsh, lo, hi);
      const int64_t hrow = off + row0 + row;
      const int64_t hcol = (int64_t)nt * S::kHcols + 16 * cb;
      *reinterpret_cast<uint2*>(a.h_codes + hrow * (a.I / 2) + hcol / 2) = make_uint2(lo, hi);
      a.h_scales[hrow * (a.I / 16) + hcol / 16] = (uint8_t)sc;
    }
  } else {
    float* sqbuf = reinterpret_cast<float*>(smem + (S::kLds - 2 * BM * 4));
    const float alpha = 1.0f / (a.a_gs[e] * a.b_gs[e]);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = wm * 32 * WM + 32 * i + 8 * (q >> 2) + 4 * g + (q & 3);
        float ss = 0.0f;
        int64_t p = 0;
        float wp = 0.0f;
        const bool ok = row < rows_here;
        if (ok) {
          p = a.sorted[off + row0 + row];
          wp = a.topk_w[p];
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          const float f = acc[i][j][q] * alpha;
          ss += f * f;
          if (ok) a.pair_out[p * a.H + (int64_t)nt * BN + wn * 32 * WN + 32 * j + r] = wp * f;
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 32);
        if (r == 0) sqbuf[wn * BM + row] = ss;
      }
    }
    __syncthreads();
    if (a.sq_part != nullptr && tid < BM && tid < rows_here) {
      const int64_t p = a.sorted[off + row0 + tid];
      a.sq_part[p * a.n_part + nt] = sqbuf[tid] + sqbuf[BM + tid];
    }
  }
}

// ---------------------------------------------------------------------------
// schedule + final reduction kernels

// m-tiles of every expert, in expert order: tile i -> (expert, first row).
__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets, int E, int BM,
                                                          int32_t* __restrict__ tile_expert,
                                                          int32_t* __restrict__ tile_row0,
                                                          int32_t* __restrict__ num_tiles) {
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
    num_tiles[0] = run;
  }
  __syncthreads();
  if (e < E)
    for (int i = 0; i < nt; ++i) {
      tile_expert[base[e] + i] = e;
      tile_row0[base[e] + i] = i * BM;
    }
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

constexpr int kTiledWM = 2, kTiledWN = 2;
using Tiled = TiledShape<kTiledWM, kTiledWN>;

int64_t ffn_max_tiles(int64_t T, int64_t k, int64_t E) { return (T * k + Tiled::BM - 1) / Tiled::BM + E; }
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
                       const_cast<int32_t*>(a.tile_expert), const_cast<int32_t*>(a.tile_row0),
                       const_cast<int32_t*>(a.num_tiles));
  }
  const unsigned gy = (unsigned)ffn_max_tiles(T, a.k, E);
  if (mode == kGateUp) {
    const unsigned gx = (unsigned)(a.I / Tiled::kHcols);
    hipLaunchKernelGGL((ffn_tiled_kernel<kGateUp, kTiledWM, kTiledWN>), dim3(gx, gy), dim3(256), Tiled::kLds, st, a);
  } else {
    const unsigned gx = (unsigned)(a.H / Tiled::BN);
    hipLaunchKernelGGL((ffn_tiled_kernel<kDown, kTiledWM, kTiledWN>), dim3(gx, gy), dim3(256), Tiled::kLds, st, a);
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
