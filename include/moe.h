/*
 * moe.h -- C ABI of the MI355X (gfx950) grouped expert MLP library (libmoe.so).
 *
 * The library implements the hot path of a mixture-of-experts feed-forward
 * layer on one GPU:
 *   token permutation by expert with per-expert counts (split_sizes),
 *   a grouped gate-up GEMM (H -> 2I) over all local experts in one launch,
 *   ScaledSwiGLU with the routing probability folded in,
 *   a grouped down GEMM (I -> H),
 *   the top-k un-permute / combine,
 * in BF16 and in MXFP8 (E4M3 elements with one E8M0 scale per 32 consecutive
 * values along the GEMM's K), forward and backward, and a forward in
 * per-tensor-scaled FP8 (E4M3 with one fp32 scale per operand tensor).
 *
 * Source of the method: page "BioNeMo Uses Grouped Kernels and MXFP8" --
 * Figure 1 (top-k router, outputs combined as a weighted sum), Grouping
 * fragmented expert workloads (split_sizes, separate per-expert weights,
 * gate-up out_features = 2 * intermediate_size, no bias), Reducing memory
 * pressure with MXFP8 and Figure 3 (E4M3 + E8M0 per 32 values), Fusing
 * precision conversion and expert computation and Figure 4 (quantize ->
 * fused gate-up + ScaledSwiGLU -> down projection); page "How BioNeMo cuts
 * overhead", How MXFP8 reduces memory use (16-bit master weights converted
 * for each low-precision GEMM).
 *
 * Conventions shared by every entry point
 *   - Every tensor argument is device memory owned by the caller, dense and
 *     row-major.  Weight pointer tables (w1, w2, dw1, dw2) are HOST arrays of
 *     E device pointers; the library copies them into kernel arguments.
 *   - The library never allocates device memory and never synchronizes the
 *     stream: all work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream).  split_sizes never leaves the device.
 *   - Host-detectable argument errors return a status before anything is
 *     enqueued.  An out-of-range expert id in topk_idx is detected on the
 *     device: the (token, slot) pair is dropped (row_id_map = -1) and a flag
 *     is raised in the first 4 bytes of the workspace; moe_read_device_error
 *     reads it.
 *   - Results are deterministic: identical inputs give identical bits (no
 *     floating-point atomics anywhere).
 *   - Calls are reentrant; concurrent calls must use distinct workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, non-positive or inconsistent size */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (shape alignment, dtype combination) */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the size query returned */
  MOE_ERR_HIP = 4           /* a HIP runtime call failed (launch error) */
} moe_status;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_MXFP8_E4M3 = 2,       /* E4M3FN bytes + E8M0 scale bytes, one per 32 values */
  MOE_FP8_E4M3 = 3          /* E4M3FN bytes + one fp32 scale per tensor (forward only) */
} moe_dtype;

/* Largest supported expert count and experts per token. */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16

/* Version of this ABI (bumped on any incompatible change). */
int moe_abi_version(void);

/* ------------------------------------------------------------------------
 * mxfp8_quantize -- OCP MXFP8 block quantization (the standalone Quantize
 * step of Figure 4's unfused flow).
 *
 * x        [rows, cols] in x_dtype (MOE_F32 or MOE_BF16).
 * axis 0:  blocks of 32 consecutive values along cols (row-wise).
 *          cols % 32 == 0.  q: [rows, cols] bytes; scales: [rows, cols/32].
 * axis 1:  blocks of 32 consecutive values along rows (column-wise), the
 *          rows being split into num_groups segments by the device array
 *          group_offsets [num_groups+1] (exclusive prefix, group_offsets[0]
 *          = 0, last = rows).  Blocks restart at every segment start and a
 *          segment's last block is zero-padded.  The output is TRANSPOSED
 *          so that the token axis is contiguous: segment g occupies columns
 *          [P_g, P_g + ceil(M_g/32)*32) of q [cols, rows_pad] and columns
 *          [P_g/32, ...) of scales [cols, rows_pad/32], where P_g is the
 *          prefix sum of the padded segment sizes and rows_pad =
 *          ceil(rows/32)*32 + 32*num_groups (an upper bound; the caller
 *          allocates it).
 *          Padding codes are 0x00; the columns past the last segment, up to
 *          rows_pad, are written as padding too (codes 0x00, scale bytes
 *          0x00).  cols % 32 == 0.  Offsets outside [0, rows]
 *          or decreasing are clamped on the device (the result is then not
 *          meaningful, but no access leaves the buffers described here).
 * Element rule: s = floor(log2(amax)) - 8 clamped to [-127, 127] (amax = 0
 * gives s = -127), scale byte = s + 127, code = E4M3FN(v / 2^s) rounded to
 * nearest even and saturated to +-448; the sign of a zero result is kept.
 * ------------------------------------------------------------------------ */
moe_status mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int axis,
                          const int32_t* group_offsets, int num_groups,
                          uint8_t* q, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------
 * mxfp8_quantize_weights -- OCP MXFP8 of a table of E bf16 weight matrices in
 * one launch, the conversion of the 16-bit master weights for each
 * low-precision GEMM (page "How BioNeMo cuts overhead", How MXFP8 reduces
 * memory use; blocks of 32 values with one E8M0 scale as in page "BioNeMo
 * Uses Grouped Kernels and MXFP8", Reducing memory pressure with MXFP8).
 * moe_grouped_mlp_fwd (axis 0) and moe_grouped_mlp_bwd (axis 1) run the same
 * kernels on every call unless their cached-weight arguments are given; this
 * entry point produces those cached arguments.
 *
 * w        HOST array of E device pointers, each a bf16 matrix [rows, cols].
 * axis 0:  row-wise, blocks along cols (cols % 32 == 0): q [E, rows, cols],
 *          scales [E, rows, cols/32] -- the forward GEMMs' B operands (W1_e
 *          along H, W2_e along I).
 * axis 1:  column-wise, blocks along rows (rows % 32 == 0), output transposed:
 *          q [E, cols, rows], scales [E, cols, rows/32] -- the backward dgrad
 *          GEMMs' B operands (W2_e^T along H, W1_e^T along 2I).  cols % 32 == 0.
 * skip     optional device int32 [E] (e.g. split_sizes): matrices with
 *          skip[e] == 0 are not quantized and their q / scales slots are left
 *          untouched.  NULL quantizes every matrix.
 * q, scales device, caller-owned.  1 <= E <= 256.  Element and scale rule as
 * mxfp8_quantize.
 * ------------------------------------------------------------------------ */
moe_status mxfp8_quantize_weights(const void* const* w, int E, int64_t rows, int64_t cols, int axis,
                                  const int32_t* skip, uint8_t* q, uint8_t* scales, void* stream);

/* ------------------------------------------------------------------------
 * fp8_tensor_quantize -- per-tensor-scaled FP8 (page "BioNeMo Uses Grouped
 * Kernels and MXFP8", Reducing memory pressure with MXFP8: FP8 and MXFP8 use
 * 8-bit values and differ in the granularity of their scaling; FP8 here has
 * one scale per tensor), current scaling.
 *
 * x        [rows, cols] in x_dtype (MOE_F32 or MOE_BF16), device.
 * Tensors: the row segments [group_offsets[g], group_offsets[g+1]) of x for
 *          g < num_groups (device int32 [num_groups+1], an exclusive prefix,
 *          last = rows; empty segments allowed), or, with group_offsets NULL
 *          and num_groups == 1, all of x.  Offsets outside [0, rows] or
 *          decreasing are clamped on the device (no access leaves the buffers).
 * Per tensor: amax = max |v|; s = 448 / amax as an fp32 division rounded to
 *          nearest (s = 1 when amax == 0; the largest finite float when the
 *          quotient overflows); code = E4M3FN(fp32(v * s)) rounded to nearest
 *          even, saturated to +-448, the sign of a zero result kept.  The
 *          value a code stands for is decode(code) / s.
 * q        [rows, cols] code bytes; scales [num_groups] fp32 s (s = 1 for an
 *          empty segment), device.
 * workspace: fp8_tensor_quantize_workspace(num_groups) bytes of device
 *          memory (amax partials), caller-owned.
 * cols % 8 == 0, else MOE_ERR_UNSUPPORTED; 1 <= num_groups <= 256.
 * ------------------------------------------------------------------------ */
size_t fp8_tensor_quantize_workspace(int num_groups);
moe_status fp8_tensor_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols,
                               const int32_t* group_offsets, int num_groups, uint8_t* q, float* scales,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute -- histogram, prefix sum and stable scatter of the (token,
 * slot) pairs by expert (the gather of each expert's tokens before the
 * grouped GEMM; split_sizes as in the grouped linear's interface).
 *
 * Source: page "BioNeMo Uses Grouped Kernels and MXFP8", Grouping fragmented
 * expert workloads -- the grouped linear takes one contiguous group of tokens
 * per expert plus split_sizes, the per-expert token counts, which absorb
 * uneven routing; Figure 1 -- the top-k router sends each token to k experts.
 *
 * x          [T, H] in x_dtype (MOE_F32 or MOE_BF16).
 * topk_idx   [T, k] int32 expert ids in [0, E).
 * topk_prob  [T, k] float32 routing probabilities (may be NULL if prob_perm is NULL).
 * perm_dtype MOE_BF16: x_perm is [T*k, H] bf16 (x rounded to nearest even);
 *            MOE_MXFP8_E4M3: x_perm is [T*k, H] E4M3 bytes and x_perm_scales
 *            [T*k, H/32] E8M0 bytes (H % 32 == 0); x_perm may be NULL to
 *            produce only the index outputs.
 * Outputs (device): split_sizes [E], offsets [E+1] (exclusive prefix sum),
 *   row_id_map [T*k] ((t*k + j) -> permuted row), src_index [T*k] (row ->
 *   t*k + j), prob_perm [T*k] (may be NULL).
 * Row order inside an expert's group is ascending t*k + j (stable).
 * workspace: at least moe_permute_workspace_size(T, k, E) bytes.
 * ------------------------------------------------------------------------ */
size_t moe_permute_workspace_size(int64_t T, int k, int E);
moe_status moe_permute(const void* x, int x_dtype, int64_t T, int64_t H,
                       const int32_t* topk_idx, const float* topk_prob, int k, int E,
                       int perm_dtype, void* x_perm, uint8_t* x_perm_scales,
                       int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                       int32_t* src_index, float* prob_perm,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same outputs, bit for bit, with no workspace
 * argument.  Its index scratch (error flag, per-block expert counts and
 * bases) is a fixed device array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends; nothing is
 * allocated by this call (no hipMalloc, no library allocation).
 *
 * Arguments as moe_permute, without workspace / workspace_bytes, plus
 * error_flag: optional device int32 that receives the bad-expert-id flag (0
 * or 1); NULL leaves it in the shared scratch only.
 * Limit: moe_permute_workspace_size(T, k, E) <= MOE_NOALLOC_SCRATCH_BYTES
 * (e.g. T <= 130752 tokens at E = 256, T <= 520k at E = 64), else
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  `stream` must belong to
 * the current device (else MOE_ERR_INVALID_ARG).
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams, or host threads) race and must be
 * serialized by the caller.  Each call writes every scratch word it reads, so
 * nothing needs clearing between calls.
 * ------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
moe_status moe_permute_noalloc(const void* x, int x_dtype, int64_t T, int64_t H,
                               const int32_t* topk_idx, const float* topk_prob, int k, int E,
                               int perm_dtype, void* x_perm, uint8_t* x_perm_scales,
                               int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                               int32_t* src_index, float* prob_perm, int32_t* error_flag, void* stream);

/* ------------------------------------------------------------------------
 * moe_route_topk -- the top-k router ahead of the permutation (page "BioNeMo
 * Uses Grouped Kernels and MXFP8", Figure 1: each token goes to k experts
 * whose outputs are combined with the routing weights).
 *
 * logits     [T, E] in logits_dtype (MOE_F32 or MOE_BF16), device.
 * topk_idx   [T, k] int32 out: the k largest logits of each token in
 *            descending order, equal logits -> lower expert id first.
 * topk_prob  [T, k] float32 out: softmax over all E experts renormalised over
 *            the k selected (= softmax of the k selected logits), fp32.
 * 1 <= k <= min(E, 16), E <= 256.  A token whose logits are all -inf (or
 * NaN) is outside the contract.
 * ------------------------------------------------------------------------ */
moe_status moe_route_topk(const void* logits, int logits_dtype, int64_t T, int E, int k,
                          int32_t* topk_idx, float* topk_prob, void* stream);

/* ------------------------------------------------------------------------
 * moe_route_permute -- moe_route_topk fused with moe_permute: the router
 * kernel also writes the expert histogram the permutation's prefix sum reads,
 * so the permutation's histogram pass over topk_idx is skipped.  Arguments as
 * the two calls; topk_idx / topk_prob are outputs here.  workspace: at least
 * moe_permute_workspace_size(T, k, E) bytes.
 * ------------------------------------------------------------------------ */
moe_status moe_route_permute(const void* logits, int logits_dtype, const void* x, int x_dtype,
                             int64_t T, int64_t H, int E, int k, int perm_dtype,
                             int32_t* topk_idx, float* topk_prob, void* x_perm, uint8_t* x_perm_scales,
                             int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                             int32_t* src_index, float* prob_perm,
                             void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_fwd -- the whole expert MLP forward.
 *
 * Source: page "BioNeMo Uses Grouped Kernels and MXFP8", Grouping fragmented
 * expert workloads and Figure 2 (all local experts' GEMMs of a projection in
 * one grouped submission instead of a loop of per-expert launches, gate-up
 * out_features = 2 * intermediate_size, no bias); Fusing precision
 * conversion and expert computation and Figure 4 (quantize, then one fused
 * kernel for gate-up + ScaledSwiGLU with the routing probabilities, then the
 * down projection); page "How BioNeMo cuts overhead", Why fused operations
 * matter (intermediates not materialized).
 *
 *   permute -> [MXFP8: quantize W1, W2] -> FC1 grouped GEMM with the
 *   ScaledSwiGLU * prob epilogue (writes h directly in the FC2 operand
 *   format; the 2I-wide gate-up output is never written unless saved_gu is
 *   given) -> FC2 grouped GEMM -> combine.
 *
 *   h[r, i]  = silu(g[r, i]) * u[r, i] * prob_perm[r],  silu(v) = v * sigmoid(v)
 *   g, u     = columns [0, I) and [I, 2I) of x_perm[r] . W1_e^T
 *   z[r]     = h[r] . W2_e^T            (rounded to io_dtype)
 *   out[t]   = sum_j z[row_id_map[t*k + j]]   (fp32 sum, rounded to io_dtype)
 *
 * Shapes: x, out [T, H] io_dtype (MOE_F32 or MOE_BF16); w1[e] [2I, H] bf16
 * (rows [0, I) gate, [I, 2I) up); w2[e] [H, I] bf16.
 * compute: MOE_BF16, MOE_MXFP8_E4M3 or MOE_FP8_E4M3 (both grouped GEMMs;
 * weights are quantized from the bf16 masters on every call).  MOE_FP8_E4M3
 * quantizes each GEMM operand tensor as fp8_tensor_quantize does: every W1_e
 * and W2_e, and each expert's rows of X_perm (bf16) and of h (rounded to bf16
 * first, since its scale needs the amax of the expert's whole h); it is
 * forward only (saved_* must be NULL, else MOE_ERR_UNSUPPORTED) and is not
 * offered by moe_grouped_mlp_fwd_loop.
 * Alignment: H % 64 == 0 and I % 64 == 0 (BF16); H % 128 == 0 and
 * I % 128 == 0 (MXFP8, FP8).  Any token counts per expert, including zero.
 * Permutation outputs are always written (caller buffers, device).
 * saved_*: optional (all NULL for inference, all set for training): bf16
 * copies kept for the backward -- x_perm [R, H], gu [R, 2I] (gate-up
 * output), h [R, I] (before MXFP8 quantization).  R = T*k.
 * w1q, w1s, w2q, w2s: optional pre-quantized MXFP8 weights (MXFP8 compute
 * only; all four or none): the row-wise mxfp8_quantize (axis 0) of every
 * W1_e and W2_e, stacked -- w1q [E, 2I, H] and w1s [E, 2I, H/32], w2q [E, H,
 * I] and w2s [E, H, I/32], device.  When given, the per-call weight
 * quantization is skipped (weights quantized once and cached by the caller)
 * and the workspace is smaller; w1 / w2 are then not read.
 * w1q, w1_scale, w2q, w2_scale: the same for MOE_FP8_E4M3 (all four or none;
 * w1s / w2s then NULL): fp8_tensor_quantize of every W1_e and W2_e as one
 * tensor each, stacked -- w1q [E, 2I, H] and w2q [E, H, I] codes, w1_scale
 * and w2_scale [E] fp32 scales s, device (ABI version 3).  Any other mix of
 * the six cached-weight fields is MOE_ERR_INVALID_ARG.
 * error_flag: optional device int32 that receives the permutation's flag for
 * out-of-range expert ids (0 or 1) instead of the first 4 bytes of the
 * workspace, so that it stays readable after later calls reuse the workspace
 * (moe_read_device_error accepts either address).
 * h_codes, h_scales: optional (MXFP8 compute only; both or neither, else
 * MOE_ERR_INVALID_ARG): caller buffers [R, I] and [R, I/32] that receive the
 * E4M3 codes and E8M0 scales of h which the FC1 epilogue's fused quantizer
 * writes and FC2 reads, in place of workspace buffers (the workspace is then
 * smaller).  Rows are in permuted order, quantized along I.
 * h_f32: optional [R, I] fp32, any compute: the epilogue also stores h =
 * silu(g) * u * p in fp32 exactly as it computed it, before rounding it to
 * bf16 or quantizing it -- the input of the fused quantizer, so that its
 * bytes can be checked against mxfp8_quantize's rule.  NULL in production.
 * w1tq_out, w1ts_out, w2tq_out, w2ts_out: optional (ABI version 6; MXFP8
 * compute with per-call weight quantization only -- not with w1q..w2s --
 * all four or none, else MOE_ERR_INVALID_ARG): caller buffers [E, H, 2I],
 * [E, H, 2I/32], [E, I, H], [E, I, H/32] that receive the weights quantized
 * along the backward's K as well, the very bytes mxfp8_quantize_weights
 * (axis 1) gives and moe_grouped_mlp_bwd's w1tq..w2ts take: the per-call
 * quantization then reads each bf16 weight once for both orientations (page
 * "How BioNeMo cuts overhead", How MXFP8 reduces memory use: the masters are
 * converted for each low-precision GEMM, forward and backward).  Experts
 * without tokens are skipped, as in the forward's own copy.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t T, H, I;
  int32_t E, k;
  int32_t compute;              /* moe_dtype: MOE_BF16, MOE_MXFP8_E4M3 or MOE_FP8_E4M3 */
  int32_t io_dtype;             /* moe_dtype: MOE_F32 or MOE_BF16 */
  const void* x;                /* [T, H] */
  const int32_t* topk_idx;      /* [T, k] */
  const float* topk_prob;       /* [T, k] */
  const void* const* w1;        /* host array of E device pointers, [2I, H] bf16 each */
  const void* const* w2;        /* host array of E device pointers, [H, I] bf16 each */
  void* out;                    /* [T, H] */
  int32_t* split_sizes;         /* [E]   */
  int32_t* offsets;             /* [E+1] */
  int32_t* row_id_map;          /* [R]   */
  int32_t* src_index;           /* [R]   */
  float* prob_perm;             /* [R]   */
  void* saved_x_perm;           /* [R, H]  bf16, or NULL */
  void* saved_gu;               /* [R, 2I] bf16, or NULL */
  void* saved_h;                /* [R, I]  bf16, or NULL */
  void* workspace;
  size_t workspace_bytes;
  const uint8_t* w1q;           /* [E, 2I, H]    E4M3, or NULL (ABI version 2) */
  const uint8_t* w1s;           /* [E, 2I, H/32] E8M0 */
  const uint8_t* w2q;           /* [E, H, I]     E4M3 */
  const uint8_t* w2s;           /* [E, H, I/32]  E8M0 */
  const float* w1_scale;        /* [E] fp32 per-tensor FP8 scales, or NULL (ABI version 3) */
  const float* w2_scale;        /* [E] */
  int32_t* error_flag;          /* device int32, or NULL (ABI version 4) */
  uint8_t* h_codes;             /* [R, I]    E4M3, or NULL (ABI version 4) */
  uint8_t* h_scales;            /* [R, I/32] E8M0 */
  float* h_f32;                 /* [R, I]    fp32, or NULL (ABI version 4) */
  uint8_t* w1tq_out;            /* [E, H, 2I]    E4M3, or NULL (ABI version 6) */
  uint8_t* w1ts_out;            /* [E, H, 2I/32] E8M0 */
  uint8_t* w2tq_out;            /* [E, I, H]     E4M3 */
  uint8_t* w2ts_out;            /* [E, I, H/32]  E8M0 */
} moe_mlp_fwd_args;

size_t moe_grouped_mlp_fwd_workspace(const moe_mlp_fwd_args* a);
moe_status moe_grouped_mlp_fwd(const moe_mlp_fwd_args* a, void* stream);

/* Same as moe_grouped_mlp_fwd, and additionally records events[i] (caller-
 * created hipEvent_t handles, moe_fwd_phase_count() + 1 of them) on `stream`
 * before phase i and after the last phase, without synchronizing, so a caller
 * can time each phase with hipEventElapsedTime.  Phases that do not apply to
 * the chosen precision are empty (their two events are adjacent).  Under
 * MOE_FP8_E4M3, permute_rows includes the quantization of X_perm and
 * fc1_gateup_swiglu that of h.
 * events == NULL behaves exactly like moe_grouped_mlp_fwd. */
moe_status moe_grouped_mlp_fwd_ex(const moe_mlp_fwd_args* a, void* stream, void* const* events);
int moe_fwd_phase_count(void);
const char* moe_fwd_phase_name(int i);   /* NULL when out of range */

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_bwd -- the matching fused backward.
 *
 * Source: page "BioNeMo Uses Grouped Kernels and MXFP8", Fusing precision
 * conversion and expert computation (MXFP8 enabled for forward and backward;
 * the fused forward has a corresponding fused backward operation); page "How
 * BioNeMo cuts overhead", Why fused operations matter (a fused operation for
 * the forward pass and a matching one for the backward pass).  The gradients
 * are those of the forward above; the grouped wgrad with K = split_sizes[e]
 * and the ScaledSwiGLU backward fused into the FC2 dgrad epilogue are this
 * library's design.
 *
 * Gradients of sum(out * dy):
 *   dz[r]     = dy[token of r]
 *   dh        = dz . W2_e                              (FC2 dgrad)
 *   a = silu(g) u;  dprob_perm[r] = sum_i dh[r,i] a[r,i]
 *   du = dh p silu(g);  dg = dh p u silu'(g),  silu'(g) = s (1 + g (1 - s)), s = sigmoid(g)
 *   dgu = [dg | du] rounded to bf16                    (FC2 dgrad epilogue)
 *   dW2_e = dz_e^T . h_e ;  dW1_e = dgu_e^T . x_perm_e  (variable-K wgrad; zero-token experts get 0)
 *   dx_perm = dgu . W1_e (rounded to io_dtype);  dx[t] = sum_j dx_perm[row_id_map[t*k+j]]
 *   dprob[t, j] = dprob_perm[row_id_map[t*k+j]]
 * Under MXFP8 every GEMM operand is quantized along that GEMM's own K
 * (token-axis blocks restart per expert).  dw1/dw2 are overwritten.
 * g, u, h and x_perm are the bf16 tensors saved by the forward.
 * w1tq, w1ts, w2tq, w2ts: optional (MXFP8 only; all four or none, else
 * MOE_ERR_INVALID_ARG): the transposed weights of the dgrad GEMMs quantized
 * once by the caller -- mxfp8_quantize_weights(w1, E, 2I, H, axis 1) and
 * mxfp8_quantize_weights(w2, E, H, I, axis 1).  Without them the backward
 * quantizes them itself on every call (one launch per weight table, experts
 * without tokens skipped).
 * Under MXFP8 the FC2 dgrad epilogue quantizes dgu itself (page "BioNeMo Uses
 * Grouped Kernels and MXFP8", Fusing precision conversion and expert
 * computation, Figure 4: the precision conversion fused into the expert
 * computation), from its bf16 values, both ways: row-wise along 2I for the
 * FC1 dgrad and along each expert's tokens for the FC1 wgrad; the bf16 dgu
 * itself is not written.  The optional debug outputs (MXFP8 only; all five or
 * none, else MOE_ERR_INVALID_ARG) receive, in the caller's buffers:
 *   dgu_bf16      [R, 2I] bf16, the values that are quantized;
 *   dgu_codes     [R, 2I] E4M3 and dgu_scales [R, 2I/32] E8M0 (row-wise);
 *   dgu_t_codes   [2I, rows_pad] E4M3 and dgu_t_scales [2I, rows_pad/32] E8M0,
 *                 transposed, with rows_pad = ceil(R/128)*128 + 128*E rounded
 *                 up to a multiple of 512 (ABI version 7; 6: not rounded): expert
 *                 e's tokens at columns [P_e, P_e + M_e) where P_e is the sum of
 *                 the earlier experts' counts each rounded up to 128; 32-token
 *                 blocks restart at P_e, the columns up to the next multiple of
 *                 128 are padding (codes 0), and the scale bytes past the last
 *                 padded segment are 0.  Other columns are not written.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t T, H, I;
  int32_t E, k;
  int32_t compute;              /* as in the forward */
  int32_t io_dtype;             /* dtype of dy and dx */
  int32_t dw_dtype;             /* MOE_F32 or MOE_BF16 */
  const void* dy;               /* [T, H] */
  const void* const* w1;        /* host array of E device pointers [2I, H] bf16 */
  const void* const* w2;        /* host array of E device pointers [H, I] bf16 */
  const int32_t* split_sizes;   /* from the forward */
  const int32_t* offsets;
  const int32_t* row_id_map;
  const int32_t* src_index;
  const float* prob_perm;
  const void* saved_x_perm;     /* [R, H]  bf16 */
  const void* saved_gu;         /* [R, 2I] bf16 */
  const void* saved_h;          /* [R, I]  bf16 */
  void* dx;                     /* [T, H] io_dtype */
  float* dprob;                 /* [T, k] */
  void* const* dw1;             /* host array of E device pointers [2I, H] dw_dtype */
  void* const* dw2;             /* host array of E device pointers [H, I] dw_dtype */
  void* workspace;
  size_t workspace_bytes;
  const uint8_t* w1tq;          /* [E, H, 2I]    E4M3, or NULL (ABI version 4) */
  const uint8_t* w1ts;          /* [E, H, 2I/32] E8M0 */
  const uint8_t* w2tq;          /* [E, I, H]     E4M3 */
  const uint8_t* w2ts;          /* [E, I, H/32]  E8M0 */
  uint16_t* dgu_bf16;           /* [R, 2I] bf16, or NULL (ABI version 5; MXFP8 debug) */
  uint8_t* dgu_codes;           /* [R, 2I]        E4M3 */
  uint8_t* dgu_scales;          /* [R, 2I/32]     E8M0 */
  uint8_t* dgu_t_codes;         /* [2I, rows_pad] E4M3 */
  uint8_t* dgu_t_scales;        /* [2I, rows_pad/32] E8M0 */
} moe_mlp_bwd_args;

size_t moe_grouped_mlp_bwd_workspace(const moe_mlp_bwd_args* a);
moe_status moe_grouped_mlp_bwd(const moe_mlp_bwd_args* a, void* stream);

/* Backward with per-phase events, as moe_grouped_mlp_fwd_ex (moe_bwd_phase_count() + 1
 * caller-created hipEvent_t handles; NULL behaves like moe_grouped_mlp_bwd). */
moe_status moe_grouped_mlp_bwd_ex(const moe_mlp_bwd_args* a, void* stream, void* const* events);
int moe_bwd_phase_count(void);
const char* moe_bwd_phase_name(int i);   /* NULL when out of range */

/* ------------------------------------------------------------------------
 * moe_grouped_mlp_fwd_loop -- the same layer as moe_grouped_mlp_fwd, but as a
 * per-expert loop: the permutation, then for each expert with tokens its own
 * launches (MXFP8: quantize W1_e, W2_e; FC1_e with the ScaledSwiGLU*prob
 * epilogue; FC2_e), then the combine.  This is the execution the pages
 * contrast with grouping (page "BioNeMo Uses Grouped Kernels and MXFP8",
 * Grouping fragmented expert workloads, Figure 2), kept as a baseline.
 *
 * Arguments as moe_grouped_mlp_fwd (same workspace size), plus
 * split_sizes_host: HOST array [E] of the per-expert token counts of topk_idx
 * (the caller obtains them, e.g. from a previous permutation; they must equal
 * the counts the device computes, which is the caller's responsibility; their
 * sum must be T*k).  Results equal moe_grouped_mlp_fwd's up to fp32
 * accumulation order.  The transposed-weight outputs (w1tq_out ..) are not
 * offered here (MOE_ERR_UNSUPPORTED).
 * ------------------------------------------------------------------------ */
moe_status moe_grouped_mlp_fwd_loop(const moe_mlp_fwd_args* a, const int32_t* split_sizes_host, void* stream);

/* Synchronizes `stream`, then returns the device error flag kept in the first
 * 4 bytes of `workspace` by the last moe_permute / moe_grouped_mlp_fwd call
 * that used it (0 = none, 1 = an expert id was out of range; every such call
 * rewrites the flag).  Returns -1 if the HIP calls fail. */
int moe_read_device_error(void* workspace, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostic for callers measuring the grouped GEMMs, not for production.
 * moe_set_tile_stats(buf, bytes) with a device buffer of at least
 * moe_tile_stats_bytes() bytes makes every later grouped-GEMM launch of
 * moe_grouped_mlp_fwd / _bwd (and their _ex forms; not the per-expert loop)
 * record, per wave, shader-clock cycle counts (s_memtime) into its slot of
 * buf; NULL turns it off (the default).  Slots, each 256 workgroups x 4 waves
 * x 4 uint32 words {main-loop cycles, epilogue cycles, work items, 0x7153}:
 * 0 FC1, 1 FC2 (main pass), 2 FC2 dgrad, 3 FC2 wgrad, 4 FC1 dgrad (main
 * pass), 5 FC1 wgrad.  A launch rewrites its slot; words of waves with no work
 * item are still written.  Outputs are unchanged.  The setting is process-wide
 * and not synchronized: set it while no call is being made.
 * MOE_ERR_INVALID_ARG if buf is not NULL and bytes is too small. */
size_t moe_tile_stats_bytes(void);
moe_status moe_set_tile_stats(uint32_t* device_buf, size_t bytes);

/* ------------------------------------------------------------------------
 * Diagnostic, not for production: the matrix-core issue-rate ceiling that the
 * grouped GEMMs' main loops are measured against.  moe_mfma_probe launches
 * moe_probe_workgroups() (256) workgroups of 4 waves on `stream`; every wave
 * issues `iters` rounds of 16 MFMAs into 16 independent 32 x 32 fp32
 * accumulators (the GEMM tiles' instruction and accumulator count), operands
 * in registers, no memory traffic.  kind: 0 MFMA-scale 32x32x64 E4M3 with
 * per-lane E8M0 scale registers, 1 the same with constant scales, 2 MFMA
 * 32x32x16 bf16 -- one operand pair, few distinct values; 3 (bf16) and 4
 * (E4M3, scale registers) cycle through 4 A and 4 B fragments of
 * pseudo-random values as a GEMM tile does, so that the operands change with
 * every MFMA.  cycles (device, 1024 uint64 = workgroups x 4 waves) receives
 * each wave's shader-clock cycles (s_memtime) of its MFMA loop; sink (device,
 * 256 x 256 floats) receives the accumulator sums, so that nothing is folded
 * away.  Both buffers belong to the caller.  Asynchronous: time it with events
 * on `stream`.  MOE_ERR_INVALID_ARG for kind outside [0, 4], iters outside
 * [1, 2^20] or a NULL buffer; MOE_ERR_HIP if the launch fails. */
int moe_probe_workgroups(void);
moe_status moe_mfma_probe(int kind, int iters, float* sink, uint64_t* cycles, void* stream);

/* Diagnostic, not for production: the rate at which the GEMMs' direct-to-LDS
 * loads fill LDS.  moe_load_probe launches 256 workgroups (one per CU) on
 * `stream`; each loads 64 KB per stage into LDS (16-byte lanes, the GEMMs'
 * load instruction), two stages in flight, a barrier per stage, for `stages`
 * stages, from the region of its XCD (workgroup b on XCD b % 8) in `buf`.
 * pattern: 0 every workgroup its own 64 KB chunks of a 2 MB region (L2
 * resident); 1 the same over 64 MB (streamed from HBM); 2 eight workgroups
 * per XCD sharing each chunk at the same stage (64 MB); 3 that sharing with
 * the GEMM operands' access, 512 rows of 4 KB of which each stage reads one
 * 128-byte slice per row.  buf (device, caller-owned, at least
 * moe_load_probe_bytes() = 512 MiB; its contents are never used) is only
 * read; cycles (device, 256 uint64) receives each workgroup's shader-clock
 * cycles.  MOE_ERR_INVALID_ARG for a pattern outside [0, 3], stages outside
 * [1, 65536], a NULL pointer or a short buffer; MOE_ERR_HIP if the launch
 * fails. */
size_t moe_load_probe_bytes(void);
moe_status moe_load_probe(int pattern, int stages, const void* buf, size_t bytes, uint64_t* cycles, void* stream);

/* Human-readable name of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
