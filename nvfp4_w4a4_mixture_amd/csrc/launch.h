// Internal launcher interface between the C-ABI host code (api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <utility>
#include <vector>

namespace moe {

// Raise a kernel's dynamic LDS limit above the default 64 KiB (gfx950 has 160 KiB
// per CU), once per (kernel, device); later calls for the same pair return at once.
inline hipError_t set_max_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::vector<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  for (const auto& d : done)
    if (d.first == kernel && d.second == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.emplace_back(kernel, dev);
  return e;
}

// Arguments of one FFN stage (gate_up: A = x, B = w13; down: A = h, B = w2).
struct FfnArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* a_gs;  // gate_up: x_gs [1]; down: h_gs [E]
  const float* b_gs;  // gate_up: w13_gs [E, 2]; down: w2_gs [E]
  const float* h_gs;  // gate_up: h_gs [E]
  int64_t K;          // reduction length (H or I)
  int64_t I;
  int64_t H;
  int k;
  const int32_t* offsets;
  const int32_t* sorted;
  const float* topk_w;
  // tiled schedule (workspace): per m-tile slot {expert, first pair row, rows, 0};
  // rows 0 marks a slot past the last m-tile
  const int32_t* tile_info;
  uint8_t* h_codes;  // gate_up output
  uint8_t* h_scales;
  uint16_t* pair_out;  // down outputs: FP16 [T*k, H], value = pair_out * pair_scale[row]
  float* pair_scale;   // [T*k] powers of two
  float* sq_part;   // [T*k, n_part] partial sums of f^2, or null
  int n_part;
};

hipError_t launch_quantize_bf16(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const float* gs,
                                int64_t rows_per_gs, uint8_t* codes, uint8_t* scales, bool tiled_scales,
                                hipStream_t stream);
// canonical [rows, K/16] scales <-> tiled [rows/16, K/128, 16, 8] (rows % 16 == 0, K % 128 == 0)
hipError_t launch_relayout_scales(const uint8_t* src, int64_t rows, int64_t K, bool to_tiled, uint8_t* dst,
                                  hipStream_t st);
hipError_t launch_weight_global_scales(const uint16_t* w, int64_t batch, int64_t per_matrix, float* gs,
                                       hipStream_t stream);

size_t route_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t k);
hipError_t launch_route(const uint16_t* x, int64_t T, int64_t H, int64_t ldx, const uint16_t* wr, const float* bias,
                        int64_t E, int64_t k, float rsf, int32_t* topk_ids, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* sorted, void* workspace, const float* qgs, uint8_t* qcodes,
                        uint8_t* qscales, hipStream_t st);

int64_t ffn_max_tiles(int64_t T, int64_t k, int64_t E);
int ffn_sq_parts(int64_t H);
bool ffn_use_small(int64_t T);
int ffn_tiled_bm();
int ffn_tiled_hcols();
int ffn_tiled_bn();
// build_schedule: (re)build the tiled kernel's m-tile schedule in the workspace
// from expert_offsets before launching; a second stage of the same call may reuse it.
hipError_t launch_ffn_stage(int mode, FfnArgs a, int64_t T, int64_t E, bool build_schedule, hipStream_t st);
hipError_t launch_sq_reduce(const float* part, int64_t npairs, int n_part, float* out, hipStream_t st);

// y = sum_j pair_out[t*k + j] * pair_scale[t*k + j] (+ add[t] if add != null)
hipError_t launch_combine(const uint16_t* pair_out, const float* pair_scale, const float* add, int64_t T, int64_t k,
                          int64_t H, int out_dtype, void* y, hipStream_t st);
hipError_t launch_reap(const float* sq, const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                       int64_t E, float* saliency, hipStream_t st);
hipError_t launch_combine_reap(const uint16_t* pair_out, const float* pair_scale, int64_t T, int64_t k, int64_t H, int out_dtype, void* y,
                               const float* sq, const float* topk_w, const int32_t* offsets, const int32_t* sorted,
                               int64_t E, float* saliency, hipStream_t st);
hipError_t launch_prune_select(const float* saliency, int64_t E, int64_t n_keep, int32_t* keep_ids, hipStream_t st);
hipError_t launch_gather_blocks(const void* src, int64_t n_src, int64_t bytes, const int32_t* ids, int64_t n_ids,
                                void* dst, hipStream_t st);

// BF16 shared expert: mode 0 = gate_up (a = x, writes h), 1 = down (a = h, writes out)
bool shared_use_small(int64_t T);
size_t shared_part_bytes(int64_t T, int64_t H, int64_t I);
hipError_t launch_shared_stage(int mode, const uint16_t* a, int64_t lda, const uint16_t* w, int64_t T, int64_t H,
                               int64_t I, uint16_t* h, float* out, float* part, hipStream_t st);

// dst = bf16((src * signs) . blockdiag(H_b) / sqrt(b)), row by row
int64_t hadamard_max_cols();
hipError_t launch_hadamard_rotate(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld_src, const float* signs,
                                  int64_t b, uint16_t* dst, int64_t ld_dst, hipStream_t st);

}  // namespace moe
