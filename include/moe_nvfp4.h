/*
 * moe_nvfp4.h -- C ABI of libmoe_nvfp4.so: the routed-expert MoE layer with
 * NVFP4 W4A4 experts, on one AMD Instinct MI355X (gfx950).
 *
 * The layer (what the pages state):
 *   - "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card, "Quantization Setup":
 *     NVFP4 W4A4 -- FP4 E2M1 values, one FP8 E4M3 block scale per 16
 *     elements, activations quantized dynamically against calibrated global
 *     scales, round-to-nearest, per-expert Linear modules; the router
 *     (mlp.gate) stays BF16.
 *   - NetsPresso AQ blog, "The Standard NVFP4 Serving Spec": the double-scale
 *     structure (an FP32 global scale times the E4M3 block scale).
 *   - "K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning Setup":
 *     renormalized sigmoid routing with e_score_correction_bias,
 *     routed_scaling_factor, and the REAP saliency
 *     mean(topk_weight * ||f_e(x)||_2) over routed tokens.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Pointers   Every array pointer is a DEVICE pointer, allocated and owned by
 *             the caller.  The library allocates and frees no device memory,
 *             keeps no pointer after returning, and the caller keeps every
 *             buffer alive until the enqueued work completes.
 *  Streams    `stream` is a hipStream_t (NULL = the default stream).  Every
 *             call only enqueues work and returns without synchronizing.
 *  Sizes      int64_t element counts.  T = tokens, H = hidden size,
 *             I = expert intermediate size, E = routed experts, k = top-k.
 *             A pair is one (token t, slot j); its id is p = t*k + j.
 *  NVFP4      A matrix [rows, cols] is stored as codes [rows, cols/2] (two
 *             E2M1 codes per byte, element 2j in bits 3:0, element 2j+1 in
 *             bits 7:4, bit 3 of a code = sign) plus scales [rows, cols/16]
 *             (one E4M3-FN byte per 16 consecutive elements of a row) plus an
 *             FP32 global scale gs.  value = e2m1(code) * e4m3(scale) / gs.
 *             Quantization: s = f32(f32(amax16 / 6) * gs); S = E4M3 RNE,
 *             saturating at 448; a zero S gives 16 zero codes; otherwise
 *             code = E2M1 RNE-even(f32(x * f32(gs / S))), saturating at 6,
 *             sign bit = sign bit of that product.
 *  Weights    w13 codes [E, 2I, H/2], scales tiled over the 2I*E rows,
 *             gs [E, 2]: rows 0..I-1 of an expert are the gate projection,
 *             rows I..2I-1 the up projection, each with its own global scale.
 *             w2 codes [E, H, I/2], scales tiled over the E*H rows, gs [E].
 *             Tiled scales (weights only): the same bytes as a row-major
 *             [R, K/16] array (R rows, K columns, R % 16 == 0, K % 128 == 0),
 *             reordered so that the 8 scales of 16 consecutive rows r and
 *             128 consecutive columns form one 128-byte block:
 *               byte of (row r, block b = column / 16) =
 *                 (r / 16) * K + (b / 8) * 128 + (r % 16) * 8 + b % 8,
 *             i.e. an array [R/16, K/128, 16, 8].  A K-step of an expert
 *             kernel then reads its 16 rows' scales as one contiguous run.
 *  Pair rows  The weighted expert output of pair p, w_p * f, as FP16 values
 *             pair_out [T*k, H] (IEEE binary16 bits) times a power of two
 *             pair_scale [T*k] (FP32): value = fp16(pair_out[p, c]) *
 *             pair_scale[p], which is exact in FP32 (above FP32's subnormal
 *             range).  pair_scale[p] = 2^E with E = floor(log2(B)) - 14,
 *             clamped to [-126, 113], for the bound, with e the expert of pair p,
 *             B = |w_p| * (I * 2688^2) * (1 / (h_gs[e] * w2_gs[e])) (FP32
 *             operations in that order) that no FP4 operands can exceed
 *             (2688 = 6 * 448, the largest decoded element); every stored
 *             value is then below 2^15 in magnitude, and pair_out[p, c] =
 *             fp16_rne(f32(w_p * 2^-E) * f[c]).  For values above 2^-29 * B
 *             (FP16's normal range) that rounding is within 2^-11 relative,
 *             well below the BF16 rounding of the output.
 *  Errors     Arguments are validated on the host before anything is
 *             enqueued.  A failed check returns its status, enqueues nothing
 *             and writes no output.  T == 0 (rows == 0) is a successful no-op
 *             (moe_route still writes zero counts and offsets, reap_saliency
 *             zero saliencies); pointers to zero-size arrays may be NULL.
 *             A failed launch returns MOE_ERR_LAUNCH.  Faults inside a kernel
 *             surface at the caller's next synchronization.  The message of
 *             the last non-OK status of the calling thread is available from
 *             moe_last_error().  No C++ exception crosses this interface.
 *  Threads    Calls are stateless apart from the thread-local error message
 *             and may be made from several host threads.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: pair rows FP16 with a per-row pair_scale (2: tiled weight block scales) */
#define MOE_NVFP4_ABI_VERSION 3

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_NULL 1      /* a required pointer is NULL                                  */
#define MOE_ERR_SHAPE 2     /* a size is out of range or inconsistent                      */
#define MOE_ERR_ALIGN 3     /* a pointer or leading dimension is not aligned as required    */
#define MOE_ERR_WORKSPACE 4 /* the workspace is NULL or smaller than the size query says    */
#define MOE_ERR_DEVICE 5    /* no usable gfx950 device is current, or a HIP query failed    */
#define MOE_ERR_LAUNCH 6    /* a kernel launch failed                                       */

/* Message describing the last non-OK status returned on this host thread. */
const char* moe_last_error(void);
/* MOE_NVFP4_ABI_VERSION of the loaded library. */
int32_t moe_abi_version(void);

/* ------------------------------------------------------------------------ */
/* Routing: sigmoid + bias top-k, renormalized and scaled, and the stable
 * expert permutation ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card,
 * "Pruning Setup"; "K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card,
 * "Quantization Setup": the router is BF16).
 *
 *   logit[t,e] = sum_h x[t,h] * w_router[e,h]   (BF16 products, FP64 sums)
 *   s = sigmoid(logit) (FP64); score = s + bias[e]
 *   topk_ids[t, 0..k-1]: the k largest scores, descending; equal scores go to
 *     the lower expert index, -0 equals +0, and a NaN score ranks below every
 *     number (so a token whose x holds a NaN or an infinity, or a NaN bias,
 *     still gets k distinct ids: those of a stable descending sort, NaN last)
 *   topk_w[t,j] = rsf * s_j / sum_{selected} s   (FP64, stored FP32; the
 *     bias selects, it does not enter the weights)
 *   expert_counts[e] = number of pairs routed to e
 *   expert_offsets[0..E] = exclusive prefix sum of the counts
 *   sorted_pair_ids[offsets[e] .. offsets[e+1]) = the pair ids p routed to e,
 *     in increasing order (a stable sort by expert)
 *
 * x_bf16 [T, ldx] (row-major, ldx >= H); w_router_bf16 [E, H]; bias [E]
 * FP32; 1 <= k <= E <= 256; T * k < 2^31; routed_scaling_factor > 0.
 * workspace: at least moe_route_workspace_bytes(T, H, E, k) bytes, 256-byte
 * aligned, device memory; its contents on entry do not matter. */
size_t moe_route_workspace_bytes(int64_t T, int64_t H, int64_t E, int64_t k);
moe_status moe_route(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx,
                     const uint16_t* w_router_bf16, const float* bias, int64_t E, int64_t k,
                     float routed_scaling_factor, int32_t* topk_ids, float* topk_w,
                     int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_pair_ids,
                     void* workspace, size_t workspace_bytes, void* stream);

/* moe_route and nvfp4_quantize_act(x, T, H, ldx, x_gs, x_codes, x_scales) in
 * one call: the routing pass that reads x also writes its NVFP4 codes
 * [T, H/2] and scales [T, H/16] (bit-identical to nvfp4_quantize_act).
 * Requirements of both calls apply (H % 16 == 0, ldx % 8 == 0, x 16-byte
 * aligned, x_codes 8-byte aligned); same workspace as moe_route. */
moe_status moe_route_quantize(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx,
                              const uint16_t* w_router_bf16, const float* bias, int64_t E, int64_t k,
                              float routed_scaling_factor, const float* x_gs, uint8_t* x_codes,
                              uint8_t* x_scales, int32_t* topk_ids, float* topk_w, int32_t* expert_counts,
                              int32_t* expert_offsets, int32_t* sorted_pair_ids, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Dynamic NVFP4 quantization of BF16 activations against a calibrated,
 * static global scale ("K-EXAONE-152B-A23B-REAP-80E-NVFP4" model card,
 * "Quantization Setup"; the double scale of the NetsPresso AQ blog,
 * "The Standard NVFP4 Serving Spec").
 *
 * x_bf16 [rows, ld] with ld >= cols, ld % 8 == 0, 16-byte aligned;
 * cols % 16 == 0; global_scale: device pointer to one FP32 (gs > 0).
 * codes [rows, cols/2] and scales [rows, cols/16] are written densely
 * (codes 8-byte aligned).  Bit-exact with the rule in the header comment. */
moe_status nvfp4_quantize_act(const uint16_t* x_bf16, int64_t rows, int64_t cols, int64_t ld,
                              const float* global_scale, uint8_t* codes, uint8_t* scales_e4m3,
                              void* stream);

/* Offline round-to-nearest quantization of `batch` BF16 weight matrices
 * [batch, rows, cols] (contiguous), each with its own global scale
 * gs[b] = f32(2688 / amax(|W_b|)) (1 when W_b is all zero), written to
 * global_scales [batch].  codes [batch, rows, cols/2]; scales tiled over the
 * batch*rows rows (layout in the header comment, K = cols).  For w13 pass
 * batch = 2E, rows = I (gate and up are separate Linear modules,
 * "per-expert Linear granularity"); for w2 pass batch = E, rows = H.
 * rows % 16 == 0, cols % 128 == 0; w_bf16 16-byte aligned. */
moe_status nvfp4_quantize_weights(const uint16_t* w_bf16, int64_t batch, int64_t rows, int64_t cols,
                                  uint8_t* codes, uint8_t* scales_e4m3, float* global_scales,
                                  void* stream);

/* One-time prepack of canonical NVFP4 expert weights into the layout the
 * FFN calls read, and its exact inverse (forum post "1x Spark GB10: 236B
 * unpruned K-EXAONE-236B-A23B serving ...", the serving instructions that open
 * it: the server's cold start is spent mostly on a one-time aligned repack of
 * the loaded weights; here the repack is this call, run once per weight set).  Canonical: codes [E, N, K/2] and
 * scales [E, N, K/16], both row-major (the form nvfp4_quantize_act writes and
 * an NVFP4 checkpoint stores).  Packed: codes unchanged, scales in the tiled
 * order of the header comment over the E*N rows.  Bit-preserving, so
 * unpack(prepack(w)) == w.  kind 0 = w13 (N = 2I rows, K = H), 1 = w2
 * (N = H, K = I).  Requires N % 16 == 0, K % 128 == 0; scale arrays 8-byte
 * aligned and not overlapping; the code arrays may be the same (no copy). */
moe_status moe_nvfp4_prepack_weights(const uint8_t* codes, const uint8_t* scales, int64_t E, int64_t N,
                                     int64_t K, int32_t kind, uint8_t* packed_codes,
                                     uint8_t* packed_scales, void* stream);
moe_status moe_nvfp4_unpack_weights(const uint8_t* packed_codes, const uint8_t* packed_scales, int64_t E,
                                    int64_t N, int64_t K, int32_t kind, uint8_t* codes, uint8_t* scales,
                                    void* stream);

/* ------------------------------------------------------------------------ */
/* The grouped NVFP4 W4A4 expert FFN ("K-EXAONE-152B-A23B-REAP-80E-NVFP4"
 * model card, "Quantization Setup": every routed expert Linear is W4A4):
 *
 *   for each expert e and each pair p in sorted_pair_ids[offsets[e]..):
 *     t = p / k;  xhat = dequant(x_codes[t], x_scales[t], x_gs)
 *     g = xhat . W_gate[e]^T, u = xhat . W_up[e]^T   (exact FP16 products of
 *         the decoded values, FP32 accumulation)
 *     h = silu(g) * u in FP32, quantized to NVFP4 with h_gs[e]
 *     f = hhat . W_down[e]^T                          (same arithmetic)
 *     pair row p = topk_w[p] * f     (pair_out and pair_scale, see "Pair rows")
 *     pair_sqnorm[p] = sum_h f[h]^2 (unweighted FP32 f; only if pair_sqnorm != NULL)
 *
 * x_codes [T, H/2], x_scales [T, H/16] (from nvfp4_quantize_act), x_gs
 * device FP32 [1]; weights in the layout of the header comment; h_gs [E]
 * FP32 (calibrated); expert_offsets [E+1] and sorted_pair_ids [T*k] from
 * moe_route; topk_w [T*k].  Requires H % 256 == 0, I % 128 == 0,
 * 1 <= k <= E <= 256; the kernels address operands with 32-bit byte offsets,
 * so x codes (T*H/2 bytes), h codes (T*k*I/2 bytes) and one expert's w13 codes
 * (I*H bytes) must each be under 4 GiB, and ceil(T*k/256) + E <= 65535
 * (MOE_ERR_SHAPE otherwise).  workspace: moe_ffn_workspace_bytes(...) bytes,
 * 256-byte aligned; it holds the re-quantized h, the tile schedule and the
 * per-tile partial sums of f^2.
 * Code arrays, activation scale arrays (x_scales, h_scales) and pair_out
 * must be 16-byte aligned, weight scale arrays and pair_scale 4-byte aligned.
 * Pairs not listed in sorted_pair_ids are not written. */
size_t moe_ffn_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I);
moe_status moe_nvfp4_grouped_ffn(
    const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T, int64_t H,
    const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
    const float* h_gs, int64_t E, int64_t I, int64_t k,
    const int32_t* expert_offsets, const int32_t* sorted_pair_ids, const float* topk_w,
    uint16_t* pair_out, float* pair_scale, float* pair_sqnorm,
    void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of moe_nvfp4_grouped_ffn as separate calls, with the
 * re-quantized hidden state in caller memory: h_codes [T*k, I/2] and
 * h_scales [T*k, I/16], row r = the r-th entry of sorted_pair_ids (grouped
 * by expert).  Same requirements as above; their workspace is
 * moe_ffn_stage_workspace_bytes(...) bytes. */
size_t moe_ffn_stage_workspace_bytes(int64_t T, int64_t k, int64_t E, int64_t H, int64_t I);
moe_status moe_nvfp4_gate_up_swiglu(
    const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T, int64_t H,
    const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
    const float* h_gs, int64_t E, int64_t I, int64_t k,
    const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
    uint8_t* h_codes, uint8_t* h_scales, void* workspace, size_t workspace_bytes, void* stream);
moe_status moe_nvfp4_down_scatter(
    const uint8_t* h_codes, const uint8_t* h_scales, const float* h_gs, int64_t T, int64_t H,
    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs, int64_t E, int64_t I,
    int64_t k, const int32_t* expert_offsets, const int32_t* sorted_pair_ids, const float* topk_w,
    uint16_t* pair_out, float* pair_scale, float* pair_sqnorm, void* workspace, size_t workspace_bytes,
    void* stream);

/* moe_nvfp4_grouped_ffn for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and requirements
 * as moe_nvfp4_grouped_ffn, without the workspace: the library's own static
 * scratch array of MOE_NVFP4_STATIC_SCRATCH_BYTES per device (held until the
 * process ends) takes its place, and the call allocates nothing.  Shapes whose
 * moe_ffn_workspace_bytes(T, k, E, H, I) exceeds that size are rejected with
 * MOE_ERR_SHAPE (at H 6144, I 2048, top-8: up to about 2,700 tokens).  Every
 * call on one device shares that device's array: calls that overlap in time on
 * one device (other streams, other host threads) race and must not be made. */
#define MOE_NVFP4_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
moe_status moe_nvfp4_grouped_ffn_noalloc(
    const uint8_t* x_codes, const uint8_t* x_scales, const float* x_gs, int64_t T, int64_t H,
    const uint8_t* w13_codes, const uint8_t* w13_scales, const float* w13_gs,
    const uint8_t* w2_codes, const uint8_t* w2_scales, const float* w2_gs,
    const float* h_gs, int64_t E, int64_t I, int64_t k,
    const int32_t* expert_offsets, const int32_t* sorted_pair_ids, const float* topk_w,
    uint16_t* pair_out, float* pair_scale, float* pair_sqnorm, void* stream);

/* ------------------------------------------------------------------------ */
/* Weighted combine: y[t, :] = sum_{j=0..k-1} pair row t*k + j (see "Pair
 * rows": fp16(pair_out) * pair_scale, exact in FP32), summed in FP32 in j
 * order (deterministic).  The pair rows already carry the routing weight
 * ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning Setup":
 * renormalized sigmoid routing weights).  out_dtype 0 writes BF16
 * (round-to-nearest-even), 1 writes FP32.  H % 8 == 0; pair_out and y 16-byte,
 * pair_scale 4-byte aligned. */
moe_status moe_combine(const uint16_t* pair_out, const float* pair_scale, int64_t T, int64_t k, int64_t H,
                       int32_t out_dtype, void* y, void* stream);

/* ------------------------------------------------------------------------ */
/* REAP saliency ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card, "Pruning
 * Setup": mean(topk_weight * ||f_e(x)||_2) over routed tokens, with the
 * model's sigmoid-and-bias routing weights including routed_scaling_factor):
 *   saliency[e] = (sum over p routed to e of topk_w[p] * sqrt(pair_sqnorm[p]))
 *                 / counts[e],   0 when no pair is routed to e.
 * Summed in sorted_pair_ids order in FP64 (deterministic); written FP32. */
moe_status reap_saliency(const float* pair_sqnorm, const float* topk_w,
                         const int32_t* expert_offsets, const int32_t* sorted_pair_ids,
                         int64_t T, int64_t k, int64_t E, float* saliency, void* stream);

/* moe_combine and reap_saliency in one launch (the same results): y from
 * the pair rows as moe_combine writes it, and saliency [E] as reap_saliency
 * writes it.  Same arguments and requirements as the two calls. */
moe_status moe_combine_reap(const uint16_t* pair_out, const float* pair_scale, int64_t T, int64_t k, int64_t H,
                            int32_t out_dtype, void* y, const float* pair_sqnorm, const float* topk_w,
                            const int32_t* expert_offsets, const int32_t* sorted_pair_ids, int64_t E,
                            float* saliency, void* stream);

/* ------------------------------------------------------------------------ */
/* REAP one-shot pruning ("K-EXAONE-152B-A23B-REAP-80E-BF16" model card,
 * introduction and "Pruning Setup": the routed experts of lowest REAP
 * saliency are removed, 128 -> 80 per layer; the router's gate weight and
 * e_score_correction_bias are sliced to the experts that remain and the
 * renormalized sigmoid routing is kept).
 *
 * reap_prune_select: keep_ids [n_keep] INT32 receives the n_keep experts of
 * highest saliency, in ascending index order.  Experts are ranked by
 * (saliency descending, index ascending): among equal saliencies the lower
 * index is kept, and -0 equals +0.  saliency [E] FP32 (from reap_saliency;
 * an expert never routed to has saliency 0 and is removed first).  For a NaN
 * saliency the result is still n_keep distinct ascending ids (NaN orders by
 * its bits), but which ones is unspecified.  1 <= n_keep <= E <= 256;
 * 4-byte aligned pointers. */
moe_status reap_prune_select(const float* saliency, int64_t E, int64_t n_keep, int32_t* keep_ids,
                             void* stream);

/* moe_gather_experts: slices one per-expert tensor of a layer to the kept
 * experts -- dst block i (bytes_per_expert bytes) = src block keep_ids[i].
 * Every per-expert tensor of the layer is such a sequence of contiguous
 * blocks: w13/w2 codes (2I*H/2 and H*I/2 bytes), their tiled scales (2I*H/16
 * and H*I/16 bytes), w13_gs (8), w2_gs (4), h_gs (4), router rows (2H) and
 * bias (4).  src holds E_src blocks, dst n_keep blocks; the two must not
 * overlap.  A keep_ids entry outside [0, E_src) leaves its dst block
 * unwritten.  1 <= n_keep <= 65535; keep_ids 4-byte aligned.  16-byte loads
 * and stores are used when src, dst and bytes_per_expert are multiples of 16. */
moe_status moe_gather_experts(const void* src, int64_t E_src, int64_t bytes_per_expert,
                              const int32_t* keep_ids, int64_t n_keep, void* dst, void* stream);

/* ------------------------------------------------------------------------ */
/* BF16 shared expert and the MoE block output.  "K-EXAONE-152B-A23B-REAP-
 * 80E-NVFP4" model card, "Quantization Setup": the shared experts are kept in
 * BF16 (only the routed experts are NVFP4); "K-EXAONE-152B-A23B-REAP-80E-BF16"
 * model card, "Pruning Setup": the shared expert is kept whole.  Every token
 * passes through it, with no routing weight:
 *
 *   g = x . W_gate^T, u = x . W_up^T      (BF16 products, FP32 accumulation)
 *   h = bf16_rne(silu(g) * u)             (the input of the BF16 down Linear)
 *   shared_out = h . W_down^T             (FP32, [T, H])
 *   block y[t] = sum_j pair row t*k + j + shared_out[t]
 *
 * x [T, H] BF16 with row stride ldx (ldx >= H, ldx % 8 == 0); w13 [2I, H]
 * BF16, gate rows 0..I-1 then up rows I..2I-1; w2 [H, I] BF16; h [T, I] BF16.
 * Requires H % 256 == 0, I % 128 == 0, and x, h and each weight matrix under
 * 4 GiB.  x, w13, w2, h and shared_out must be 16-byte aligned; workspace
 * 256-byte aligned, of moe_shared_workspace_bytes(T, H, I) bytes (the stage
 * calls need less; the same size serves them).  For T <= 16 the K dimension
 * is split across workgroups and the FP32 partial sums are added in a fixed
 * order, so results are deterministic for every T. */
size_t moe_shared_workspace_bytes(int64_t T, int64_t H, int64_t I);
moe_status moe_shared_expert(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx,
                             const uint16_t* w13_bf16, const uint16_t* w2_bf16, int64_t I,
                             float* shared_out, void* workspace, size_t workspace_bytes, void* stream);
/* The two stages of moe_shared_expert, with h in caller memory. */
moe_status moe_shared_gate_up(const uint16_t* x_bf16, int64_t T, int64_t H, int64_t ldx,
                              const uint16_t* w13_bf16, int64_t I, uint16_t* h_bf16, void* workspace,
                              size_t workspace_bytes, void* stream);
moe_status moe_shared_down(const uint16_t* h_bf16, int64_t T, int64_t I, const uint16_t* w2_bf16,
                           int64_t H, float* shared_out, void* workspace, size_t workspace_bytes,
                           void* stream);
/* moe_combine with the shared expert's row added after the k routed rows:
 * y[t] = (sum_j pair row t*k + j) + shared_out[t], FP32, then written as in
 * moe_combine.  shared_out [T, H] FP32, 16-byte aligned. */
moe_status moe_combine_block(const uint16_t* pair_out, const float* pair_scale, const float* shared_out,
                             int64_t T, int64_t k, int64_t H, int32_t out_dtype, void* y, void* stream);

/* ------------------------------------------------------------------------ */
/* Offline Hadamard rotation of the hidden dimension ("[NetsPresso AQ Deep
 * Dive] How to Quantize the K-EXAONE-236B Model to 4-Bit (NVFP4)", "Offline
 * Fusion of Multiple Quantization Algorithms": the weights' coordinates are
 * rotated before NVFP4 quantization so that outliers do not pile up in one
 * block; the rotation is absorbed into the weights).  Row by row:
 *
 *   dst[r, :] = bf16_rne( (src[r, :] * signs) . blockdiag(H_b, ..., H_b) / sqrt(b) )
 *
 * H_b is the +-1 Sylvester Hadamard matrix of size b = block (a power of two,
 * 2 <= b <= cols, cols % b == 0); signs [cols] FP32 +-1 (NULL = all +1).
 * Rotating x and each row of W_gate, W_up and the router by the same R keeps
 * x W^T unchanged in exact arithmetic.  src/dst [rows, cols] BF16 with row
 * strides ld_src/ld_dst (>= cols, multiples of 8); cols a multiple of 8, at
 * most 16384; src and dst 16-byte aligned and either identical (in place, same
 * stride) or not overlapping.  FP64 butterflies in a fixed order (the ±1 sums of
 * BF16 values are exact), one FP64 division by sqrt(b), then one rounding to
 * BF16: the correctly rounded rotation. */
moe_status hadamard_rotate_bf16(const uint16_t* src, int64_t rows, int64_t cols, int64_t ld_src,
                                const float* signs, int64_t block, uint16_t* dst, int64_t ld_dst,
                                void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
