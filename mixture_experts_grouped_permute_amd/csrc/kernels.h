// Kernel launchers shared between the C-ABI layer and the .hip sources.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kPermTokens = 64;    // tokens (k (token, slot) ids each) per histogram / scatter block
constexpr int kMaxTopK = 16;
constexpr int kGemmGrid = 256;     // persistent GEMM workgroups: one per CU, a multiple of the 8 XCDs

// ---- permutation (permute.hip)
// Number of permutation blocks (histogram chunks) for T tokens.
inline int perm_blocks(int64_t T) {
  const int64_t nb = (T + kPermTokens - 1) / kPermTokens;
  return nb < 1 ? 1 : (int)nb;
}
// block_counts: [nb][E] per-block expert counts followed by nb "bad id" flags.  With
// counts_ready the histogram pass is skipped (the router already wrote block_counts).
hipError_t launch_permute_indices(const int32_t* idx, const float* prob, int64_t T, int k, int E,
                                  int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                                  int32_t* src_index, float* prob_perm, int32_t* err_flag, int32_t* block_counts,
                                  int32_t* block_base, hipStream_t st, bool counts_ready = false);
// ---- fused router (router.hip): top-k of the logits [T, E] (f32 or bf16), renormalised
// softmax weights, and (block_counts != nullptr) the permutation's per-block histogram.
hipError_t launch_router(const void* logits, bool f32, int64_t T, int E, int k, int32_t* idx, float* prob,
                         int32_t* block_counts, hipStream_t st);
hipError_t launch_permute_rows(const void* x, bool x_f32, int64_t T, int64_t H, int k, const int32_t* row_id_map,
                               void* out, uint8_t* out_scales, bool mx, hipStream_t st);

// ---- quantization (quant.hip)
hipError_t launch_mx_quant_rows(const void* x, bool x_f32, int64_t rows, int64_t cols, uint8_t* q,
                                uint8_t* scales, hipStream_t st);
// Row-wise MXFP8 of E bf16 weight matrices [rows, cols] given by a host pointer table; experts with
// skip_if_empty != nullptr && skip_if_empty[e] == 0 are skipped (their codes are never read).
hipError_t launch_mx_quant_weights(const void* const* w, int E, int64_t rows, int64_t cols, uint8_t* q,
                                   uint8_t* scales, const int32_t* skip_if_empty, hipStream_t st);
// Column-wise MXFP8 of E bf16 weight matrices [rows, cols] (rows % 32 == 0) of a host pointer table
// in one launch, transposed: matrix e's codes [cols, rows] at q + e * cols * rows, its scales
// [cols, rows / 32] at scales + e * cols * rows / 32; skip_if_empty as launch_mx_quant_weights.
// With q_rows / s_rows the same read also gives the row-wise codes [rows, cols] and scales
// [rows, cols / 32] of every matrix (launch_mx_quant_weights' output), for cols % 32 == 0.
hipError_t launch_mx_quant_weights_t(const void* const* w, int E, int64_t rows, int64_t cols, uint8_t* q,
                                     uint8_t* scales, const int32_t* skip_if_empty, hipStream_t st,
                                     uint8_t* q_rows = nullptr, uint8_t* s_rows = nullptr);
// Column-wise (blocks along rows, restarted per segment, transposed output); see mxfp8_quantize axis 1.
// seg_align: segments are padded to a multiple of seg_align rows (32 for the C ABI; 128 when the
// result feeds the variable-K wgrad GEMM, whose K steps are 128 values).
// src_index != nullptr: segmented row r is row src_index[r] / src_k of x (x holds token rows; rows is
// the number of segmented rows).
hipError_t launch_mx_quant_cols(const void* x, bool x_f32, int64_t rows, int64_t cols,
                                const int32_t* group_offsets, int num_groups, int64_t rows_pad, uint8_t* q,
                                uint8_t* scales, hipStream_t st, int seg_align = 32,
                                const int32_t* src_index = nullptr, int src_k = 1);

// Per-tensor FP8 (one fp32 scale per tensor): the row segments [offsets[g], offsets[g+1]) of x
// [rows, cols] (offsets == nullptr: one segment of all rows), or each of E bf16 weight matrices
// [rows, cols] of a host pointer table (codes stacked [E, rows, cols]).  scales[g] = s,
// inv[g] = 1 / s (inv may be nullptr); part: pt_part_floats(G) floats of amax partials.
// cols % 8 == 0.
int pt_blocks(int G);
size_t pt_part_floats(int G);
// amax_in: per-tensor amax as float bits, already known (the amax pass is skipped); nullptr:
// computed here into part.
hipError_t launch_pt_quant(const void* x, bool x_f32, int64_t rows, int64_t cols, const int32_t* offsets, int G,
                           uint8_t* q, float* scales, float* inv, float* part, hipStream_t st,
                           const uint32_t* amax_in = nullptr);
hipError_t launch_pt_quant_weights(const void* const* w, int E, int64_t rows, int64_t cols, uint8_t* q,
                                   float* scales, float* inv, float* part, hipStream_t st);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);

// ---- combine / gather (combine.hip)
hipError_t launch_combine(const void* z, bool z_f32, int64_t T, int64_t H, int k, const int32_t* row_id_map,
                          void* out, bool out_f32, hipStream_t st);
// out[r] = bf16(x[src_index[r] / k]), r < offsets[E]
hipError_t launch_gather_rows(const void* x, bool f32, int64_t R, int64_t H, int k, const int32_t* src_index,
                              const int32_t* offsets, int E, void* out, hipStream_t st);
hipError_t launch_dprob_reduce(const float* partial, int64_t R, int parts, const int32_t* row_id_map,
                               int64_t T, int k, float* dprob, hipStream_t st);

// ---- grouped GEMMs (gemm.hip)
struct FwdGemm {
  // A operand: permuted rows [R, K] (bf16, or E4M3 codes + [R, K/32] scales)
  const void* a;
  const uint8_t* a_scales;
  // B operand per expert: bf16 table (w_tab) or contiguous MXFP8 codes/scales with strides
  const void* const* w_tab;          // host table of E device pointers (bf16 path)
  const uint8_t* wq;                 // MXFP8 codes base, expert e at wq + e * wq_stride
  int64_t wq_stride;
  const uint8_t* ws;                 // MXFP8 scales base
  int64_t ws_stride;
  int64_t K, N;                      // FC1: K = H, N = I (h columns); FC2: K = I, N = H
  int E;
  const int32_t* split_sizes;
  const float* prob_perm;            // FC1
  void* out;                         // FC1: h (bf16 or E4M3 codes) [R, I]; FC2: z [R, H]
  uint8_t* out_scales;               // FC1 MXFP8: [R, I/32]
  uint16_t* save_gu;                 // FC1 training: [R, 2I] bf16
  uint16_t* save_h;                  // FC1 MXFP8 training: [R, I] bf16 h
  bool out_f32;                      // FC2
  float* part;                       // FC2: kGemmGrid x 65536 fp32 for split tiles (nullptr: no split)
  // per-tensor FP8 (MXFP8 instance with every block scale 1, i.e. a_scales / ws point at 0x7F
  // bytes and ws_stride = 0): per expert the scale s of its A rows and of its weight; the products
  // are multiplied by (1 / s_a)(1 / s_b), and FC1 writes bf16 h to save_h instead of E4M3 codes.
  // nullptr: MXFP8.
  const float* pt_s_a;
  const float* pt_s_b;
  // per-tensor FP8, FC1: per expert max |bf16 h| as float bits, raised with an integer atomic max
  // (order-free, so deterministic); zeroed by the caller before the launch
  uint32_t* pt_amax_out;
  // FC1: optional fp32 copy of h = silu(g) u p [R, I] as the epilogue computes it, before it is
  // rounded to bf16 or quantized (the input of the fused quantizer); nullptr: not written
  float* h_f32;
  // diagnostic: kGemmGrid x 4 waves x kTileStatWords words of per-wave cycle counts (null: off)
  uint32_t* tstat = nullptr;
};
// Per-wave cycle counts of a grouped GEMM launch (diagnostic, moe_set_tile_stats): words
// {main-loop cycles, epilogue cycles, work items, kTileStatTag} per wave of each workgroup.
constexpr int kTileStatWords = 4;
constexpr uint32_t kTileStatTag = 0x7153u;
constexpr size_t kTileStatLaunchWords = (size_t)kGemmGrid * 4 * kTileStatWords;
// Slots of the launches that record them.
enum : int { kStatFc1 = 0, kStatFc2, kStatDgradFc2, kStatWgradFc2, kStatDgradFc1, kStatWgradFc1, kStatSlots };
// The caller's diagnostic buffer (kStatSlots x kTileStatLaunchWords words), or null.
uint32_t* tile_stat_slot(int slot);

// Workspace of the FC2 split-tile partials (bytes).
constexpr size_t kFc2PartBytes = (size_t)kGemmGrid * 65536 * sizeof(float);
hipError_t launch_fc1(const FwdGemm& g, bool mx, hipStream_t st);
hipError_t launch_fc2(const FwdGemm& g, bool mx, hipStream_t st);
// Sums the S fp32 K-part tiles of the split 256-row tiles of the last round (tile list of
// ceil(M_e / 256) x ceil(N / 256) tiles per expert, parts as written by a split GEMM pass) into
// out ([rows, N], bf16 or fp32).  kU: K units of 128 bytes of the GEMM.
hipError_t launch_split_fixup(const int32_t* split_sizes, int E, int64_t N, float* part, void* out, bool out_f32,
                              int kU, hipStream_t st);

// ---- backward grouped GEMMs (gemm_bwd.hip); byte strides throughout
struct BwdGemm {
  const void* a;            // dgrad: permuted rows (K-major); wgrad bf16: token-major rows; wgrad MXFP8: A^T [M][Rpad]
  int64_t lda;
  const uint8_t* a_scales;
  int64_t ldas;
  const void* b;            // wgrad bf16: token-major rows; MXFP8: transposed quantized operand
  int64_t ldb;
  int64_t b_stride;
  const uint8_t* b_scales;
  int64_t ldbs;
  int64_t bs_stride;
  const void* const* tab;   // bf16 dgrad: E weight pointers; wgrad: E dW output pointers
  int64_t M, N, K;
  int E;
  int pad;                  // MXFP8 wgrad: token segments padded to this many rows
  const int32_t* split_sizes;
  const uint16_t* gu;
  const float* prob_perm;
  uint16_t* dgu;            // bf16 dGU (BF16; MXFP8 only when asked for, as a debug output)
  float* dprob_part;
  int64_t I;
  // MXFP8 FC2 dgrad: dGU quantized in the epilogue, along 2I (row-wise, [R, 2I] + [R, 2I/32]) and
  // along each expert's tokens (transposed [2I, rows_pad] + [2I, rows_pad/32], segments padded to
  // 128 tokens)
  uint8_t *dgu_q, *dgu_s, *dgu_tq, *dgu_ts;
  int64_t rows_pad;
  void* out;
  bool out_f32;
  float* part;              // FC1 dgrad: split-tile partials (kFc2PartBytes), or null for no split
  uint32_t* tstat = nullptr;  // diagnostic per-wave cycle counts (kTileStatLaunchWords words), or null
};
hipError_t launch_bwd_dgrad_fc2(const BwdGemm& g, bool mx, hipStream_t st);
hipError_t launch_bwd_dgrad_fc1(const BwdGemm& g, bool mx, hipStream_t st);
hipError_t launch_bwd_wgrad(const BwdGemm& g, bool mx, hipStream_t st);
// zero the scale bytes of the transposed operand past its last 128-padded segment ([rows, ld])
hipError_t launch_scale_tail_zero(uint8_t* scales, int64_t rows, int64_t ld, const int32_t* split_sizes, int E,
                                  hipStream_t st);
int bwd_dprob_parts(int64_t I);

}  // namespace moe
