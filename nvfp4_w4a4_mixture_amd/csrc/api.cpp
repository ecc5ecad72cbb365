// C ABI of libmoe_nvfp4.so (declared in include/moe_nvfp4.h).
//
// Every entry point validates its arguments on the host before making any HIP
// call, so a rejected call enqueues nothing and touches no output.  Kernel
// launches are asynchronous on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/moe_nvfp4.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// The current device must be gfx950; checked once per device id.
moe_status check_device() {
  static std::mutex mu;
  static int ok_state[64] = {0};  // 0 unknown, 1 ok, -1 bad
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(MOE_ERR_DEVICE, "no current HIP device");
  std::lock_guard<std::mutex> lk(mu);
  if (ok_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed");
    ok_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (ok_state[dev] < 0) {
      char msg[300];
      snprintf(msg, sizeof(msg), "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
      g_last_error = msg;
    }
  }
  if (ok_state[dev] < 0) return MOE_ERR_DEVICE;
  return MOE_OK;
}

moe_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// ---- FFN workspace layout
struct FfnWs {
  size_t tile_info, sq_part, h_codes, h_scales, total_stage, total_full;
};

FfnWs ffn_ws_layout(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I) {
  FfnWs w{};
  const int64_t tiles = moe::ffn_max_tiles(T, k, E);
  size_t o = 0;
  w.tile_info = o;
  o = round_up(o + (size_t)tiles * 16, 256);
  w.sq_part = o;
  o = round_up(o + (size_t)(T * k) * (size_t)moe::ffn_sq_parts(H) * 4, 256);
  w.total_stage = o;
  w.h_codes = o;
  o = round_up(o + (size_t)(T * k) * (size_t)(I / 2), 256);
  w.h_scales = o;
  o = round_up(o + (size_t)(T * k) * (size_t)(I / 16), 256);
  w.total_full = o;
  return w;
}

moe_status check_ffn_shapes(int64_t T, int64_t H, int64_t E, int64_t I, int64_t k) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "T must be >= 0 (got %lld)", (long long)T);
  if (H <= 0 || H % 256 != 0) return fail(MOE_ERR_SHAPE, "H must be a positive multiple of 256 (got %lld)", (long long)H);
  if (I <= 0 || I % 128 != 0) return fail(MOE_ERR_SHAPE, "I must be a positive multiple of 128 (got %lld)", (long long)I);
  if (k < 1 || E < k || E > 256) return fail(MOE_ERR_SHAPE, "need 1 <= k <= E <= 256 (k=%lld, E=%lld)", (long long)k, (long long)E);
  if (T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "T*k must be < 2^31");
  // The expert kernels address each operand with 32-bit byte offsets from a
  // wave-uniform base: x codes by token (T*H/2 bytes), the h codes by sorted
  // pair row (T*k*I/2 bytes), and each expert's weight codes from the expert's
  // first row (I*H bytes for w13); the tile grid's y dimension is limited too.
  const uint64_t lim = (uint64_t)1 << 32;
  if ((uint64_t)T * (uint64_t)(H / 2) >= lim)
    return fail(MOE_ERR_SHAPE, "x codes (T*H/2 = %llu bytes) must be under 4 GiB",
                (unsigned long long)((uint64_t)T * (uint64_t)(H / 2)));
  if ((uint64_t)(T * k) * (uint64_t)(I / 2) >= lim)
    return fail(MOE_ERR_SHAPE, "h codes (T*k*I/2 = %llu bytes) must be under 4 GiB",
                (unsigned long long)((uint64_t)(T * k) * (uint64_t)(I / 2)));
  if ((uint64_t)I * (uint64_t)H >= lim) return fail(MOE_ERR_SHAPE, "one expert's w13 codes (I*H bytes) must be under 4 GiB");
  if (moe::ffn_max_tiles(T, k, E) > 65535)
    return fail(MOE_ERR_SHAPE, "too many m-tiles (%lld > 65535) for one launch", (long long)moe::ffn_max_tiles(T, k, E));
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_abi_version(void) { return MOE_NVFP4_ABI_VERSION; }

size_t moe_route_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t k) {
  if (T < 0 || H < 1 || E < 1 || k < 1) return 0;
  return moe::route_workspace_bytes(T, H, E, k);
}

// Shared body of moe_route and moe_route_quantize (qcodes == NULL: no quantization).
static moe_status route_impl(const char* fn, const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx,
                             const uint16_t* w_router_bf16, const float* bias, int64_t E, int64_t k, float rsf,
                             const float* x_gs, uint8_t* x_codes, uint8_t* x_scales, int32_t* topk_ids, float* topk_w,
                             int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_pair_ids,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!w_router_bf16 || !bias || !expert_counts || !expert_offsets ||
      (T > 0 && (!x_bf16 || !topk_ids || !topk_w || !sorted_pair_ids)))
    return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (T < 0 || H < 1 || ldx < H) return fail(MOE_ERR_SHAPE, "%s: need T >= 0, H >= 1, ldx >= H", fn);
  if (k < 1 || E < k || E > 256) return fail(MOE_ERR_SHAPE, "%s: need 1 <= k <= E <= 256", fn);
  if (T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "%s: T*k must be < 2^31", fn);
  if (!(rsf > 0.0f)) return fail(MOE_ERR_SHAPE, "%s: routed_scaling_factor must be > 0", fn);
  if (x_codes) {
    if (H % 16 != 0) return fail(MOE_ERR_SHAPE, "%s: H must be a multiple of 16 to quantize x", fn);
    if (T > 0 && (!x_gs || !x_scales)) return fail(MOE_ERR_NULL, "%s: x_gs and x_scales are required", fn);
    if (T > 0 && (ldx % 8 != 0 || !aligned(x_bf16, 16) || !aligned(x_codes, 8)))
      return fail(MOE_ERR_ALIGN, "%s: x must be 16-byte aligned with ldx %% 8 == 0; x_codes 8-byte aligned", fn);
  }
  const size_t need = moe::route_workspace_bytes(T, H, E, k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  if (need > 0 && !aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  if (moe_status s = check_device()) return s;
  // T == 0 still writes zero counts and offsets.
  return launched(moe::launch_route(x_bf16, T, H, ldx, w_router_bf16, bias, E, k, rsf, topk_ids, topk_w,
                                    expert_counts, expert_offsets, sorted_pair_ids, workspace, x_gs,
                                    T > 0 ? x_codes : nullptr, x_scales, (hipStream_t)stream),
                  fn);
}

moe_status moe_route(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx, const uint16_t* w_router_bf16,
                     const float* bias, int64_t E, int64_t k, float routed_scaling_factor, int32_t* topk_ids,
                     float* topk_w, int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_pair_ids,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return route_impl("moe_route", x_bf16, T, H, ldx, w_router_bf16, bias, E, k, routed_scaling_factor, nullptr,
                    nullptr, nullptr, topk_ids, topk_w, expert_counts, expert_offsets, sorted_pair_ids, workspace,
                    workspace_bytes, stream);
}

moe_status moe_route_quantize(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx,
                              const uint16_t* w_router_bf16, const float* bias, int64_t E, int64_t k,
                              float routed_scaling_factor, const float* x_gs, uint8_t* x_codes, uint8_t* x_scales,
                              int32_t* topk_ids, float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_pair_ids, void* workspace, size_t workspace_bytes, void* stream) {
  if (T > 0 && !x_codes) return fail(MOE_ERR_NULL, "moe_route_quantize: x_codes is NULL");
  return route_impl("moe_route_quantize", x_bf16, T, H, ldx, w_router_bf16, bias, E, k, routed_scaling_factor, x_gs,
                    T > 0 ? x_codes : nullptr, x_scales, topk_ids, topk_w, expert_counts, expert_offsets,
                    sorted_pair_ids, workspace, workspace_bytes, stream);
}

moe_status nvfp4_quantize_act(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                              const float* global_scale, uint8_t* codes, uint8_t* scales_e4m3, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || ld < cols)
    return fail(MOE_ERR_SHAPE, "nvfp4_quantize_act: need rows >= 0, cols a positive multiple of 16, ld >= cols");
  if (rows == 0) return MOE_OK;
  if (!x_bf16 || !global_scale || !codes || !scales_e4m3)
    return fail(MOE_ERR_NULL, "nvfp4_quantize_act: a required pointer is NULL");
  if (ld % 8 != 0 || !aligned(x_bf16, 16) || !aligned(codes, 8))
    return fail(MOE_ERR_ALIGN, "nvfp4_quantize_act: x must be 16-byte aligned with ld %% 8 == 0; codes 8-byte aligned");
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_quantize_bf16(x_bf16, rows, cols, ld, global_scale, rows, codes, scales_e4m3, false,
                                            (hipStream_t)stream),
                  "nvfp4_quantize_act");
}

moe_status nvfp4_quantize_weights(const uint16_t* w_bf16, int64_t batch, int64_t rows, int64_t cols, uint8_t* codes,
                                  uint8_t* scales_e4m3, float* global_scales, void* stream) {
  if (batch < 0 || rows <= 0 || rows % 16 != 0 || cols <= 0 || cols % 128 != 0)
    return fail(MOE_ERR_SHAPE,
                "nvfp4_quantize_weights: need batch >= 0, rows a positive multiple of 16, cols a positive multiple of 128");
  if (batch == 0) return MOE_OK;
  if (!w_bf16 || !codes || !scales_e4m3 || !global_scales)
    return fail(MOE_ERR_NULL, "nvfp4_quantize_weights: a required pointer is NULL");
  if (!aligned(w_bf16, 16) || !aligned(codes, 8))
    return fail(MOE_ERR_ALIGN, "nvfp4_quantize_weights: w must be 16-byte aligned, codes 8-byte aligned");
  if (moe_status s = check_device()) return s;
  hipStream_t st = (hipStream_t)stream;
  if (moe_status s = launched(moe::launch_weight_global_scales(w_bf16, batch, rows * cols, global_scales, st),
                              "nvfp4_quantize_weights (global scales)"))
    return s;
  return launched(moe::launch_quantize_bf16(w_bf16, batch * rows, cols, cols, global_scales, rows, codes, scales_e4m3,
                                            true, st),
                  "nvfp4_quantize_weights");
}

size_t moe_ffn_stage_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I) {
  if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return 0;
  return ffn_ws_layout(T, k, E, H, I).total_stage;
}

size_t moe_ffn_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I) {
  if (T < 0 || k < 1 || E < 1 || H < 1 || I < 1) return 0;
  return ffn_ws_layout(T, k, E, H, I).total_full;
}

static moe_status gate_up_impl(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T,
                               int64_t H, const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
                               const float* h_gs, int64_t E, int64_t I, int64_t k, const int32_t* expert_offsets,
                               const int32_t* sorted_pair_ids, uint8_t* h_codes, uint8_t* h_scales,
                               unsigned char* ws, hipStream_t st) {
  const FfnWs L = ffn_ws_layout(T, k, E, H, I);
  moe::FfnArgs a{};
  a.a_codes = x_codes;
  a.a_scales = x_scales;
  a.b_codes = w13_codes;
  a.b_scales = w13_scales;
  a.a_gs = x_gs;
  a.b_gs = w13_gs;
  a.h_gs = h_gs;
  a.K = H;
  a.I = I;
  a.H = H;
  a.k = (int)k;
  a.offsets = expert_offsets;
  a.sorted = sorted_pair_ids;
  a.tile_info = reinterpret_cast<const int32_t*>(ws + L.tile_info);
  a.h_codes = h_codes;
  a.h_scales = h_scales;
  return launched(moe::launch_ffn_stage(0, a, T, E, /*build_schedule=*/true, st), "moe_nvfp4_gate_up_swiglu");
}

static moe_status down_impl(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs, int64_t T, int64_t H,
                            const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs, int64_t E,
                            int64_t I, int64_t k, const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                            const float* topk_w, uint16_t* pair_out, float* pair_scale, float* pair_sqnorm,
                            unsigned char* ws, bool build_schedule, hipStream_t st) {
  const FfnWs L = ffn_ws_layout(T, k, E, H, I);
  moe::FfnArgs a{};
  a.a_codes = h_codes;
  a.a_scales = h_scales;
  a.b_codes = w2_codes;
  a.b_scales = w2_scales;
  a.a_gs = h_gs;
  a.b_gs = w2_gs;
  a.K = I;
  a.I = I;
  a.H = H;
  a.k = (int)k;
  a.offsets = expert_offsets;
  a.sorted = sorted_pair_ids;
  a.topk_w = topk_w;
  a.tile_info = reinterpret_cast<const int32_t*>(ws + L.tile_info);
  a.pair_out = pair_out;
  a.pair_scale = pair_scale;
  a.sq_part = pair_sqnorm ? reinterpret_cast<float*>(ws + L.sq_part) : nullptr;
  a.n_part = moe::ffn_use_small(T) ? (int)(H / 64) : (int)(H / moe::ffn_tiled_bn());
  if (moe_status s = launched(moe::launch_ffn_stage(1, a, T, E, build_schedule, st), "moe_nvfp4_down_scatter"))
    return s;
  if (pair_sqnorm)
    return launched(moe::launch_sq_reduce(a.sq_part, T * k, a.n_part, pair_sqnorm, st), "moe_nvfp4_down_scatter (sq)");
  return MOE_OK;
}

moe_status moe_nvfp4_gate_up_swiglu(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T,
                                    int64_t H, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                    const float* w13_gs, const float* h_gs, int64_t E, int64_t I, int64_t k,
                                    const int32_t* expert_offsets, const int32_t* sorted_pair_ids, uint8_t* h_codes,
                                    uint8_t* h_scales, void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status s = check_ffn_shapes(T, H, E, I, k)) return s;
  if (T == 0) return MOE_OK;  // zero-size arrays may be NULL
  if (!x_codes || !x_scales || !x_gs || !w13_codes || !w13_scales || !w13_gs || !h_gs || !expert_offsets ||
      !sorted_pair_ids || !h_codes || !h_scales)
    return fail(MOE_ERR_NULL, "moe_nvfp4_gate_up_swiglu: a required pointer is NULL");
  if (!aligned(x_codes, 16) || !aligned(w13_codes, 16) || !aligned(h_codes, 16) || !aligned(x_scales, 16) ||
      !aligned(h_scales, 16) || !aligned(w13_scales, 4))
    return fail(MOE_ERR_ALIGN,
                "moe_nvfp4_gate_up_swiglu: code and activation-scale arrays must be 16-byte, weight scales 4-byte aligned");
  const size_t need = ffn_ws_layout(T, k, E, H, I).total_stage;
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_nvfp4_gate_up_swiglu: workspace needs %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (moe_status s = check_device()) return s;
  return gate_up_impl(x_codes, x_scales, x_gs, T, H, w13_codes, w13_scales, w13_gs, h_gs, E, I, k, expert_offsets,
                      sorted_pair_ids, h_codes, h_scales, static_cast<unsigned char*>(workspace), (hipStream_t)stream);
}

moe_status moe_nvfp4_down_scatter(const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs, int64_t T,
                                  int64_t H, const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                                  int64_t E, int64_t I, int64_t k, const int32_t* expert_offsets,
                                  const int32_t* sorted_pair_ids, const float* topk_w, uint16_t* pair_out,
                                  float* pair_scale, float* pair_sqnorm, void* workspace, size_t workspace_bytes, void* stream) {
  if (moe_status s = check_ffn_shapes(T, H, E, I, k)) return s;
  if (T == 0) return MOE_OK;  // zero-size arrays may be NULL
  if (!h_codes || !h_scales || !h_gs || !w2_codes || !w2_scales || !w2_gs || !expert_offsets || !sorted_pair_ids ||
      !topk_w || !pair_out || !pair_scale)
    return fail(MOE_ERR_NULL, "moe_nvfp4_down_scatter: a required pointer is NULL");
  if (!aligned(h_codes, 16) || !aligned(w2_codes, 16) || !aligned(pair_out, 16) || !aligned(h_scales, 16) ||
      !aligned(w2_scales, 4) || !aligned(pair_scale, 4))
    return fail(MOE_ERR_ALIGN, "moe_nvfp4_down_scatter: code arrays, h_scales and pair_out must be 16-byte, weight "
                               "scales and pair_scale 4-byte aligned");
  const size_t need = ffn_ws_layout(T, k, E, H, I).total_stage;
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "moe_nvfp4_down_scatter: workspace needs %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (moe_status s = check_device()) return s;
  return down_impl(h_codes, h_scales, h_gs, T, H, w2_codes, w2_scales, w2_gs, E, I, k, expert_offsets,
                   sorted_pair_ids, topk_w, pair_out, pair_scale, pair_sqnorm, static_cast<unsigned char*>(workspace),
                   /*build_schedule=*/true, (hipStream_t)stream);
}

// Validation shared by moe_nvfp4_grouped_ffn and its static-scratch variant.
static moe_status check_grouped_ffn(const char* fn, const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                    int64_t T, int64_t H, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                    const float* w13_gs, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                    const float* w2_gs, const float* h_gs, int64_t E, int64_t I, int64_t k,
                                    const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                                    const float* topk_w, const uint16_t* pair_out, const float* pair_scale) {
  if (moe_status s = check_ffn_shapes(T, H, E, I, k)) return s;
  if (T == 0) return MOE_OK;  // zero-size arrays may be NULL
  if (!x_codes || !x_scales || !x_gs || !w13_codes || !w13_scales || !w13_gs || !w2_codes || !w2_scales || !w2_gs ||
      !h_gs || !expert_offsets || !sorted_pair_ids || !topk_w || !pair_out || !pair_scale)
    return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(x_codes, 16) || !aligned(w13_codes, 16) || !aligned(w2_codes, 16) || !aligned(pair_out, 16) ||
      !aligned(x_scales, 16) || !aligned(w13_scales, 4) || !aligned(w2_scales, 4) || !aligned(pair_scale, 4))
    return fail(MOE_ERR_ALIGN,
                "%s: code arrays, x_scales and pair_out must be 16-byte, weight scales and pair_scale 4-byte aligned",
                fn);
  return MOE_OK;
}

// Both stages in one workspace `ws` of at least ffn_ws_layout(...).total_full bytes.
static moe_status grouped_ffn_impl(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T,
                                   int64_t H, const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
                                   const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                                   const float* h_gs, int64_t E, int64_t I, int64_t k, const int32_t* expert_offsets,
                                   const int32_t* sorted_pair_ids, const float* topk_w, uint16_t* pair_out,
                                   float* pair_scale, float* pair_sqnorm, unsigned char* ws, hipStream_t st) {
  const FfnWs L = ffn_ws_layout(T, k, E, H, I);
  uint8_t* h_codes = ws + L.h_codes;
  uint8_t* h_scales = ws + L.h_scales;
  if (moe_status s = gate_up_impl(x_codes, x_scales, x_gs, T, H, w13_codes, w13_scales, w13_gs, h_gs, E, I, k,
                                  expert_offsets, sorted_pair_ids, h_codes, h_scales, ws, st))
    return s;
  // stage 2 reuses the schedule stage 1 built in the same workspace
  return down_impl(h_codes, h_scales, h_gs, T, H, w2_codes, w2_scales, w2_gs, E, I, k, expert_offsets,
                   sorted_pair_ids, topk_w, pair_out, pair_scale, pair_sqnorm, ws, /*build_schedule=*/false, st);
}

moe_status moe_nvfp4_grouped_ffn(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T,
                                 int64_t H, const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
                                 const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
                                 const float* h_gs, int64_t E, int64_t I, int64_t k, const int32_t* expert_offsets,
                                 const int32_t* sorted_pair_ids, const float* topk_w, uint16_t* pair_out,
                                 float* pair_scale, float* pair_sqnorm, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  const char* fn = "moe_nvfp4_grouped_ffn";
  if (moe_status s = check_grouped_ffn(fn, x_codes, x_scales, x_gs, T, H, w13_codes, w13_scales, w13_gs, w2_codes,
                                       w2_scales, w2_gs, h_gs, E, I, k, expert_offsets, sorted_pair_ids, topk_w,
                                       pair_out, pair_scale))
    return s;
  if (T == 0) return MOE_OK;
  const FfnWs L = ffn_ws_layout(T, k, E, H, I);
  if (!workspace || workspace_bytes < L.total_full)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, L.total_full);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (moe_status s = check_device()) return s;
  return grouped_ffn_impl(x_codes, x_scales, x_gs, T, H, w13_codes, w13_scales, w13_gs, w2_codes, w2_scales, w2_gs,
                          h_gs, E, I, k, expert_offsets, sorted_pair_ids, topk_w, pair_out, pair_scale, pair_sqnorm,
                          static_cast<unsigned char*>(workspace), (hipStream_t)stream);
}

// ---- the grouped FFN on a static scratch array: allocates nothing

}  // extern "C"

namespace {

// The FFN workspace of the no-allocation entry point: one array per device,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: only its device address, from
// hipGetSymbolAddress, is ever passed to a kernel.
constexpr size_t kStaticScratchBytes = MOE_NVFP4_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};  // device address of `scratch` per device id

// The current device's copy of `scratch`, looked up once per device with that device current.
moe_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(MOE_ERR_DEVICE, "no current HIP device");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_nvfp4_grouped_ffn_noalloc(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs,
                                         int64_t T, int64_t H, const uint8_t* w13_codes, const uint8_t* w13_scales,
                                         const float* w13_gs, const uint8_t* w2_codes, const uint8_t* w2_scales,
                                         const float* w2_gs, const float* h_gs, int64_t E, int64_t I, int64_t k,
                                         const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                                         const float* topk_w, uint16_t* pair_out, float* pair_scale,
                                         float* pair_sqnorm, void* stream) {
  const char* fn = "moe_nvfp4_grouped_ffn_noalloc";
  if (moe_status s = check_grouped_ffn(fn, x_codes, x_scales, x_gs, T, H, w13_codes, w13_scales, w13_gs, w2_codes,
                                       w2_scales, w2_gs, h_gs, E, I, k, expert_offsets, sorted_pair_ids, topk_w,
                                       pair_out, pair_scale))
    return s;
  if (T == 0) return MOE_OK;
  const FfnWs L = ffn_ws_layout(T, k, E, H, I);
  if (L.total_full > kStaticScratchBytes)
    return fail(MOE_ERR_SHAPE, "%s: this shape needs %zu bytes of scratch; the static scratch holds %zu", fn,
                L.total_full, kStaticScratchBytes);
  if (moe_status s = check_device()) return s;
  void* ws = nullptr;
  if (moe_status s = static_scratch(&ws)) return s;
  // nothing in the workspace needs to start at zero: the schedule is rebuilt and
  // every h row and partial sum is written before it is read
  return grouped_ffn_impl(x_codes, x_scales, x_gs, T, H, w13_codes, w13_scales, w13_gs, w2_codes, w2_scales, w2_gs,
                          h_gs, E, I, k, expert_offsets, sorted_pair_ids, topk_w, pair_out, pair_scale, pair_sqnorm,
                          static_cast<unsigned char*>(ws), (hipStream_t)stream);
}

moe_status moe_combine(const uint16_t* pair_out, const float* pair_scale, int64_t T, int64_t k, int64_t H,
                       int32_t out_dtype, void* y, void* stream) {
  if (T < 0 || k < 1 || H <= 0 || H % 8 != 0 || (out_dtype != 0 && out_dtype != 1))
    return fail(MOE_ERR_SHAPE, "moe_combine: need T >= 0, k >= 1, H a positive multiple of 8, out_dtype 0 or 1");
  if (T == 0) return MOE_OK;
  if (!pair_out || !pair_scale || !y) return fail(MOE_ERR_NULL, "moe_combine: a required pointer is NULL");
  if (!aligned(pair_out, 16) || !aligned(y, 16) || !aligned(pair_scale, 4))
    return fail(MOE_ERR_ALIGN, "moe_combine: pair_out and y must be 16-byte, pair_scale 4-byte aligned");
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_combine(pair_out, pair_scale, nullptr, T, k, H, out_dtype, y, (hipStream_t)stream),
                  "moe_combine");
}

moe_status reap_saliency(const float* pair_sqnorm, const float* topk_w, const int32_t* expert_offsets,
                         const int32_t* sorted_pair_ids, int64_t T, int64_t k, int64_t E, float* saliency,
                         void* stream) {
  if (!expert_offsets || !saliency || (T > 0 && (!pair_sqnorm || !topk_w || !sorted_pair_ids)))
    return fail(MOE_ERR_NULL, "reap_saliency: a required pointer is NULL");
  if (T < 0 || k < 1 || E < 1 || E > 256 || T * k >= (int64_t)1 << 31)
    return fail(MOE_ERR_SHAPE, "reap_saliency: need T >= 0, k >= 1, 1 <= E <= 256");
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_reap(pair_sqnorm, topk_w, expert_offsets, sorted_pair_ids, E, saliency,
                                   (hipStream_t)stream),
                  "reap_saliency");
}

moe_status moe_combine_reap(const uint16_t* pair_out, const float* pair_scale, int64_t T, int64_t k, int64_t H,
                            int32_t out_dtype, void* y, const float* pair_sqnorm, const float* topk_w, const int32_t* expert_offsets,
                            const int32_t* sorted_pair_ids, int64_t E, float* saliency, void* stream) {
  const char* fn = "moe_combine_reap";
  if (T < 0 || k < 1 || H <= 0 || H % 8 != 0 || (out_dtype != 0 && out_dtype != 1))
    return fail(MOE_ERR_SHAPE, "%s: need T >= 0, k >= 1, H a positive multiple of 8, out_dtype 0 or 1", fn);
  if (E < 1 || E > 256 || T * k >= (int64_t)1 << 31) return fail(MOE_ERR_SHAPE, "%s: need 1 <= E <= 256", fn);
  if (!expert_offsets || !saliency ||
      (T > 0 && (!pair_out || !pair_scale || !y || !pair_sqnorm || !topk_w || !sorted_pair_ids)))
    return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (T > 0 && (!aligned(pair_out, 16) || !aligned(y, 16) || !aligned(pair_scale, 4)))
    return fail(MOE_ERR_ALIGN, "%s: pair_out and y must be 16-byte, pair_scale 4-byte aligned", fn);
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_combine_reap(pair_out, pair_scale, T, k, H, out_dtype, y, pair_sqnorm, topk_w,
                                           expert_offsets, sorted_pair_ids, E, saliency, (hipStream_t)stream),
                  fn);
}

moe_status reap_prune_select(const float* saliency, int64_t E, int64_t n_keep, int32_t* keep_ids, void* stream) {
  if (E < 1 || E > 256 || n_keep < 1 || n_keep > E)
    return fail(MOE_ERR_SHAPE, "reap_prune_select: need 1 <= n_keep <= E <= 256 (n_keep=%lld, E=%lld)",
                (long long)n_keep, (long long)E);
  if (!saliency || !keep_ids) return fail(MOE_ERR_NULL, "reap_prune_select: a required pointer is NULL");
  if (!aligned(saliency, 4) || !aligned(keep_ids, 4))
    return fail(MOE_ERR_ALIGN, "reap_prune_select: 4-byte alignment required");
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_prune_select(saliency, E, n_keep, keep_ids, (hipStream_t)stream), "reap_prune_select");
}

moe_status moe_gather_experts(const void* src, int64_t E_src, int64_t bytes_per_expert, const int32_t* keep_ids,
                              int64_t n_keep, void* dst, void* stream) {
  if (E_src < 1 || bytes_per_expert < 1 || n_keep < 1 || n_keep > 65535)
    return fail(MOE_ERR_SHAPE, "moe_gather_experts: need E_src >= 1, bytes_per_expert >= 1, 1 <= n_keep <= 65535");
  if (E_src > INT64_MAX / bytes_per_expert || n_keep > INT64_MAX / bytes_per_expert)
    return fail(MOE_ERR_SHAPE, "moe_gather_experts: total size overflows");
  if (!src || !dst || !keep_ids) return fail(MOE_ERR_NULL, "moe_gather_experts: a required pointer is NULL");
  if (!aligned(keep_ids, 4)) return fail(MOE_ERR_ALIGN, "moe_gather_experts: keep_ids must be 4-byte aligned");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t s1 = s0 + (uintptr_t)(E_src * bytes_per_expert), d1 = d0 + (uintptr_t)(n_keep * bytes_per_expert);
  if (s0 < d1 && d0 < s1) return fail(MOE_ERR_SHAPE, "moe_gather_experts: src and dst overlap");
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_gather_blocks(src, E_src, bytes_per_expert, keep_ids, n_keep, dst, (hipStream_t)stream),
                  "moe_gather_experts");
}

// ---- BF16 shared expert and the block output

size_t moe_shared_workspace_bytes(int64_t T, int64_t H, int64_t I) {
  if (T < 0 || H < 1 || I < 1) return 0;
  return round_up((size_t)T * (size_t)I * 2, 256) + round_up(moe::shared_part_bytes(T, H, I), 256);
}

namespace {

constexpr uint64_t kOffsetLimit = (uint64_t)1 << 32;  // kernels address each operand with 32-bit byte offsets

moe_status check_shared(const char* fn, int64_t T, int64_t H, int64_t I) {
  if (T < 0) return fail(MOE_ERR_SHAPE, "%s: T must be >= 0", fn);
  if (H <= 0 || H % 256 != 0) return fail(MOE_ERR_SHAPE, "%s: H must be a positive multiple of 256", fn);
  if (I <= 0 || I % 128 != 0) return fail(MOE_ERR_SHAPE, "%s: I must be a positive multiple of 128", fn);
  if ((uint64_t)(2 * I) * (uint64_t)H * 2 >= kOffsetLimit)
    return fail(MOE_ERR_SHAPE, "%s: each weight matrix must be under 4 GiB", fn);
  return MOE_OK;
}

moe_status shared_ws(const char* fn, int64_t T, int64_t H, int64_t I, void* workspace, size_t workspace_bytes,
                     float** part) {
  const size_t need = round_up(moe::shared_part_bytes(T, H, I), 256);
  *part = nullptr;
  if (need == 0) return MOE_OK;
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  *part = reinterpret_cast<float*>(workspace);
  return MOE_OK;
}

}  // namespace

moe_status moe_shared_gate_up(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx, const uint16_t* w13_bf16,
                              int64_t I, uint16_t* h_bf16, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_shared_gate_up";
  if (moe_status s = check_shared(fn, T, H, I)) return s;
  if (ldx < H || ldx % 8 != 0) return fail(MOE_ERR_SHAPE, "%s: ldx must be >= H and a multiple of 8", fn);
  if (T == 0) return MOE_OK;
  if ((uint64_t)T * (uint64_t)ldx * 2 >= kOffsetLimit || (uint64_t)T * (uint64_t)I * 2 >= kOffsetLimit)
    return fail(MOE_ERR_SHAPE, "%s: x and h must each be under 4 GiB", fn);
  if (!x_bf16 || !w13_bf16 || !h_bf16) return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(x_bf16, 16) || !aligned(w13_bf16, 16) || !aligned(h_bf16, 16))
    return fail(MOE_ERR_ALIGN, "%s: x, w13 and h must be 16-byte aligned", fn);
  float* part;
  if (moe_status s = shared_ws(fn, T, H, I, workspace, workspace_bytes, &part)) return s;
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_shared_stage(0, x_bf16, ldx, w13_bf16, T, H, I, h_bf16, nullptr, part,
                                           (hipStream_t)stream), fn);
}

moe_status moe_shared_down(const uint16_t* h_bf16, int64_t T, int64_t I, const uint16_t* w2_bf16, int64_t H,
                           float* shared_out, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "moe_shared_down";
  if (moe_status s = check_shared(fn, T, H, I)) return s;
  if (T == 0) return MOE_OK;
  if ((uint64_t)T * (uint64_t)I * 2 >= kOffsetLimit) return fail(MOE_ERR_SHAPE, "%s: h must be under 4 GiB", fn);
  if (!h_bf16 || !w2_bf16 || !shared_out) return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(h_bf16, 16) || !aligned(w2_bf16, 16) || !aligned(shared_out, 16))
    return fail(MOE_ERR_ALIGN, "%s: h, w2 and shared_out must be 16-byte aligned", fn);
  float* part;
  if (moe_status s = shared_ws(fn, T, H, I, workspace, workspace_bytes, &part)) return s;
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_shared_stage(1, h_bf16, I, w2_bf16, T, H, I, nullptr, shared_out, part,
                                           (hipStream_t)stream), fn);
}

moe_status moe_shared_expert(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx, const uint16_t* w13_bf16,
                             const uint16_t* w2_bf16, int64_t I, float* shared_out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const char* fn = "moe_shared_expert";
  if (moe_status s = check_shared(fn, T, H, I)) return s;
  if (ldx < H || ldx % 8 != 0) return fail(MOE_ERR_SHAPE, "%s: ldx must be >= H and a multiple of 8", fn);
  if (T == 0) return MOE_OK;
  const size_t hbytes = round_up((size_t)T * (size_t)I * 2, 256);
  const size_t need = moe_shared_workspace_bytes(T, H, I);
  if (!workspace || workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed", fn, need);
  if (!aligned(workspace, 256)) return fail(MOE_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  uint16_t* h = reinterpret_cast<uint16_t*>(workspace);
  void* rest = static_cast<unsigned char*>(workspace) + hbytes;
  if (moe_status s = moe_shared_gate_up(x_bf16, T, H, ldx, w13_bf16, I, h, rest, workspace_bytes - hbytes, stream))
    return s;
  return moe_shared_down(h, T, I, w2_bf16, H, shared_out, rest, workspace_bytes - hbytes, stream);
}

moe_status moe_combine_block(const uint16_t* pair_out, const float* pair_scale, const float* shared_out, int64_t T,
                             int64_t k, int64_t H, int32_t out_dtype, void* y, void* stream) {
  if (T < 0 || k < 1 || H <= 0 || H % 8 != 0 || (out_dtype != 0 && out_dtype != 1))
    return fail(MOE_ERR_SHAPE, "moe_combine_block: need T >= 0, k >= 1, H a positive multiple of 8, out_dtype 0 or 1");
  if (T == 0) return MOE_OK;
  if (!pair_out || !pair_scale || !shared_out || !y)
    return fail(MOE_ERR_NULL, "moe_combine_block: a required pointer is NULL");
  if (!aligned(pair_out, 16) || !aligned(shared_out, 16) || !aligned(y, 16) || !aligned(pair_scale, 4))
    return fail(MOE_ERR_ALIGN, "moe_combine_block: pair_out, shared_out and y must be 16-byte, pair_scale 4-byte aligned");
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_combine(pair_out, pair_scale, shared_out, T, k, H, out_dtype, y, (hipStream_t)stream),
                  "moe_combine_block");
}

// ---- offline Hadamard rotation

moe_status hadamard_rotate_bf16(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld_src, const float* signs,
                                int64_t block, uint16_t* dst, int64_t ld_dst, void* stream) {
  const char* fn = "hadamard_rotate_bf16";
  if (rows < 0 || rows > INT32_MAX) return fail(MOE_ERR_SHAPE, "%s: need 0 <= rows < 2^31", fn);
  if (cols < 8 || cols % 8 != 0 || cols > moe::hadamard_max_cols())
    return fail(MOE_ERR_SHAPE, "%s: cols must be a multiple of 8 in [8, %lld]", fn, (long long)moe::hadamard_max_cols());
  if (block < 2 || (block & (block - 1)) != 0 || block > cols || cols % block != 0)
    return fail(MOE_ERR_SHAPE, "%s: block must be a power of two >= 2 that divides cols", fn);
  if (ld_src < cols || ld_dst < cols || ld_src % 8 != 0 || ld_dst % 8 != 0)
    return fail(MOE_ERR_SHAPE, "%s: leading dimensions must be >= cols and multiples of 8", fn);
  if (rows == 0) return MOE_OK;
  if (!src || !dst) return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(src, 16) || !aligned(dst, 16) || !aligned(signs, 4))
    return fail(MOE_ERR_ALIGN, "%s: src and dst must be 16-byte aligned, signs 4-byte aligned", fn);
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t s1 = s0 + (uintptr_t)(((rows - 1) * ld_src + cols) * 2);
  const uintptr_t d1 = d0 + (uintptr_t)(((rows - 1) * ld_dst + cols) * 2);
  const bool in_place = s0 == d0 && ld_src == ld_dst;
  if (!in_place && s0 < d1 && d0 < s1)
    return fail(MOE_ERR_SHAPE, "%s: src and dst overlap (only the exact in-place call is allowed)", fn);
  if (moe_status s = check_device()) return s;
  return launched(moe::launch_hadamard_rotate(src, rows, cols, ld_src, signs, block, dst, ld_dst, (hipStream_t)stream),
                  fn);
}

// ---- one-time weight prepack (canonical -> kernel layout) and its inverse

static moe_status relayout_weights(const char* fn, const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N,
                                   int64_t K, int32_t kind, uint8_t* out_codes, uint8_t* out_scales, bool to_tiled,
                                   void* stream) {
  if (kind != 0 && kind != 1) return fail(MOE_ERR_SHAPE, "%s: kind must be 0 (w13) or 1 (w2)", fn);
  if (E < 0 || N <= 0 || K <= 0 || N % 16 != 0 || K % 128 != 0)
    return fail(MOE_ERR_SHAPE, "%s: need E >= 0, N a positive multiple of 16, K a positive multiple of 128", fn);
  if (kind == 0 && N % 2 != 0) return fail(MOE_ERR_SHAPE, "%s: w13 has 2I rows", fn);
  if (E == 0) return MOE_OK;
  if (!codes || !scales || !out_codes || !out_scales) return fail(MOE_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (!aligned(scales, 8) || !aligned(out_scales, 8)) return fail(MOE_ERR_ALIGN, "%s: scale arrays must be 8-byte aligned", fn);
  const int64_t rows = E * N;
  const size_t scale_bytes = (size_t)rows * (size_t)(K / 16);
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(scales), b0 = reinterpret_cast<uintptr_t>(out_scales);
  if (a0 < b0 + scale_bytes && b0 < a0 + scale_bytes)
    return fail(MOE_ERR_SHAPE, "%s: the scale arrays must not overlap", fn);
  if (moe_status s = check_device()) return s;
  hipStream_t st = (hipStream_t)stream;
  if (out_codes != codes) {
    const hipError_t e = hipMemcpyAsync(out_codes, codes, (size_t)rows * (size_t)(K / 2), hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return fail(MOE_ERR_LAUNCH, "%s: code copy: %s", fn, hipGetErrorString(e));
  }
  return launched(moe::launch_relayout_scales(scales, rows, K, to_tiled, out_scales, st), fn);
}

moe_status moe_nvfp4_prepack_weights(const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N, int64_t K,
                                     int32_t kind, uint8_t* packed_codes, uint8_t* packed_scales, void* stream) {
  return relayout_weights("moe_nvfp4_prepack_weights", codes, scales, E, N, K, kind, packed_codes, packed_scales, true,
                          stream);
}

moe_status moe_nvfp4_unpack_weights(const uint8_t* packed_codes, const uint8_t* packed_scales, int64_t E, int64_t N,
                                    int64_t K, int32_t kind, uint8_t* codes, uint8_t* scales, void* stream) {
  return relayout_weights("moe_nvfp4_unpack_weights", packed_codes, packed_scales, E, N, K, kind, codes, scales, false,
                          stream);
}

}  // extern "C"
