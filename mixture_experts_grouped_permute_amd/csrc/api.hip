// C-ABI entry points of libmoe.so: argument validation, workspace carving and
// launch sequencing.  Everything is enqueued on the caller's stream; nothing
// here allocates device memory or synchronizes (except moe_read_device_error).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe.h"
#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sequential carve-out of a caller-provided workspace (or a dry run to size it).
struct Carver {
  uint8_t* base;
  size_t used = 0;
  explicit Carver(void* b) : base(reinterpret_cast<uint8_t*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used = align_up(used + bytes);
    return p;
  }
};

inline bool io_ok(int d) { return d == MOE_F32 || d == MOE_BF16; }
inline size_t io_size(int d) { return d == MOE_F32 ? 4 : 2; }

struct PermWs {
  int32_t* err;
  int32_t* block_counts;
  int32_t* block_base;
};

PermWs carve_perm(Carver& c, int64_t T, int E) {
  PermWs w;
  const int nb = perm_blocks(T);
  w.err = reinterpret_cast<int32_t*>(c.take(kAlign));
  w.block_counts = reinterpret_cast<int32_t*>(c.take(sizeof(int32_t) * (size_t)nb * (E + 1)));
  w.block_base = reinterpret_cast<int32_t*>(c.take(sizeof(int32_t) * (size_t)nb * E));
  return w;
}

#define MOE_CHECK(cond, code) \
  do {                        \
    if (!(cond)) return (code); \
  } while (0)

#define HIP_TRY(expr)                         \
  do {                                        \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

moe_status check_common(int64_t T, int64_t H, int E, int k) {
  if (T <= 0 || H <= 0 || E <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || k > E) return MOE_ERR_INVALID_ARG;
  if (T * (int64_t)k > (int64_t)INT32_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Forward workspace plan (pointers are null on a dry run).
struct FwdPlan {
  PermWs perm;
  void* x_op;          // bf16 [R,H] or E4M3 [R,H]
  uint8_t* x_sc;       // [R,H/32]
  void* h_op;          // bf16 [R,I] or E4M3 [R,I]
  uint8_t* h_sc;       // [R,I/32]
  void* z;             // [R,H] io dtype
  float* part;         // FC2 split-tile partials
  uint8_t* w1q; uint8_t* w1s; uint8_t* w2q; uint8_t* w2s;
  // per-tensor FP8: bf16 X_perm and h ahead of their quantization, per-expert scales s and 1 / s
  // (X_perm rows, W1, h rows, W2), amax partials, and the 0x7F block scales the GEMMs read
  void* x_bf; void* h_bf;
  float *sx, *sw1, *sh, *sw2;
  float* pt_part;
  uint32_t* h_amax;    // per expert max |bf16 h| (float bits), raised by FC1's epilogue
  uint8_t* unit;
  int64_t unit_bytes;
  size_t bytes;
};

FwdPlan plan_fwd(const moe_mlp_fwd_args* a, void* ws) {
  FwdPlan p{};
  Carver c(ws);
  const int64_t R = a->T * a->k, H = a->H, I = a->I;
  const int E = a->E;
  const bool mx = a->compute == MOE_MXFP8_E4M3;
  p.perm = carve_perm(c, a->T, E);
  if (a->compute == MOE_FP8_E4M3) {
    auto f = [&](size_t n) { return reinterpret_cast<float*>(c.take(n * sizeof(float))); };
    p.x_bf = c.take((size_t)(R * H * 2));
    p.x_op = c.take((size_t)(R * H));
    p.h_bf = c.take((size_t)(R * I * 2));
    p.h_op = c.take((size_t)(R * I));
    if (a->w1q) {   // per-tensor FP8 weights cached by the caller: codes and fp32 scales
      p.w1q = const_cast<uint8_t*>(a->w1q);
      p.w2q = const_cast<uint8_t*>(a->w2q);
      p.sw1 = const_cast<float*>(a->w1_scale);
      p.sw2 = const_cast<float*>(a->w2_scale);
    } else {
      p.w1q = reinterpret_cast<uint8_t*>(c.take((size_t)(E * 2 * I * H)));
      p.w2q = reinterpret_cast<uint8_t*>(c.take((size_t)(E * H * I)));
      p.sw1 = f(E);
      p.sw2 = f(E);
    }
    p.sx = f(E);
    p.sh = f(E);
    p.pt_part = f(pt_part_floats(E));
    p.h_amax = reinterpret_cast<uint32_t*>(c.take((size_t)E * sizeof(uint32_t)));
    // unit block scales: the FC1 GEMM reads rows [0, max(R, 2I)) of H/32 bytes, FC2 rows
    // [0, max(R, H)) of I/32 bytes (the weight scales with expert stride 0)
    const int64_t u1 = (R > 2 * I ? R : 2 * I) * (H / 32), u2 = (R > H ? R : H) * (I / 32);
    p.unit_bytes = ((u1 > u2 ? u1 : u2) + 3) / 4 * 4;
    p.unit = reinterpret_cast<uint8_t*>(c.take((size_t)p.unit_bytes));
  } else if (mx) {
    p.x_op = c.take((size_t)(R * H));
    p.x_sc = reinterpret_cast<uint8_t*>(c.take((size_t)(R * H / 32)));
    if (a->h_codes) {   // h's codes and scales go to the caller's buffers
      p.h_op = a->h_codes;
      p.h_sc = a->h_scales;
    } else {
      p.h_op = c.take((size_t)(R * I));
      p.h_sc = reinterpret_cast<uint8_t*>(c.take((size_t)(R * I / 32)));
    }
    if (a->w1q) {   // quantized weights cached by the caller
      p.w1q = const_cast<uint8_t*>(a->w1q);
      p.w1s = const_cast<uint8_t*>(a->w1s);
      p.w2q = const_cast<uint8_t*>(a->w2q);
      p.w2s = const_cast<uint8_t*>(a->w2s);
    } else {
      p.w1q = reinterpret_cast<uint8_t*>(c.take((size_t)(E * 2 * I * H)));
      p.w1s = reinterpret_cast<uint8_t*>(c.take((size_t)(E * 2 * I * H / 32)));
      p.w2q = reinterpret_cast<uint8_t*>(c.take((size_t)(E * H * I)));
      p.w2s = reinterpret_cast<uint8_t*>(c.take((size_t)(E * H * I / 32)));
    }
  } else {
    if (!a->saved_x_perm) p.x_op = c.take((size_t)(R * H * 2));
    else p.x_op = a->saved_x_perm;
    if (!a->saved_h) p.h_op = c.take((size_t)(R * I * 2));
    else p.h_op = a->saved_h;
  }
  p.z = c.take((size_t)(R * H) * io_size(a->io_dtype));
  p.part = reinterpret_cast<float*>(c.take(kFc2PartBytes));
  p.bytes = c.used;
  if (a->error_flag) p.perm.err = a->error_flag;
  return p;
}

moe_status validate_fwd(const moe_mlp_fwd_args* a) {
  if (!a) return MOE_ERR_INVALID_ARG;
  moe_status s = check_common(a->T, a->H, a->E, a->k);
  if (s != MOE_OK) return s;
  if (a->I <= 0) return MOE_ERR_INVALID_ARG;
  if (!io_ok(a->io_dtype)) return MOE_ERR_INVALID_ARG;
  if (a->compute != MOE_BF16 && a->compute != MOE_MXFP8_E4M3 && a->compute != MOE_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  const int64_t align = a->compute == MOE_BF16 ? 64 : 128;
  if (a->H % align || a->I % align) return MOE_ERR_UNSUPPORTED;
  if (!a->x || !a->topk_idx || !a->topk_prob || !a->out) return MOE_ERR_INVALID_ARG;
  if (!a->w1q && (!a->w1 || !a->w2)) return MOE_ERR_INVALID_ARG;
  if (!a->split_sizes || !a->offsets || !a->row_id_map || !a->src_index || !a->prob_perm)
    return MOE_ERR_INVALID_ARG;
  if (!a->w1q)
    for (int e = 0; e < a->E; ++e)
      if (!a->w1[e] || !a->w2[e]) return MOE_ERR_INVALID_ARG;
  // cached weights: MXFP8 codes with E8M0 scales (w1s, w2s), or per-tensor FP8 codes with fp32
  // scales (w1_scale, w2_scale) -- all four of the precision's fields, or none of the six
  const bool any_q = a->w1q || a->w1s || a->w2q || a->w2s || a->w1_scale || a->w2_scale;
  const bool mx_q = a->w1q && a->w1s && a->w2q && a->w2s && !a->w1_scale && !a->w2_scale;
  const bool f8_q = a->w1q && a->w2q && a->w1_scale && a->w2_scale && !a->w1s && !a->w2s;
  if (any_q && !((mx_q && a->compute == MOE_MXFP8_E4M3) || (f8_q && a->compute == MOE_FP8_E4M3)))
    return MOE_ERR_INVALID_ARG;
  const bool any_saved = a->saved_x_perm || a->saved_gu || a->saved_h;
  const bool all_saved = a->saved_x_perm && a->saved_gu && a->saved_h;
  if (any_saved && !all_saved) return MOE_ERR_INVALID_ARG;
  if (any_saved && a->compute == MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;   // forward only
  if ((a->h_codes != nullptr) != (a->h_scales != nullptr)) return MOE_ERR_INVALID_ARG;
  const bool any_wt = a->w1tq_out || a->w1ts_out || a->w2tq_out || a->w2ts_out;
  const bool all_wt = a->w1tq_out && a->w1ts_out && a->w2tq_out && a->w2ts_out;
  if (any_wt && (!all_wt || a->compute != MOE_MXFP8_E4M3 || any_q)) return MOE_ERR_INVALID_ARG;
  if (a->h_codes && a->compute != MOE_MXFP8_E4M3) return MOE_ERR_INVALID_ARG;
  // 32-bit buffer ranges inside the GEMMs: every descriptor spans one 256-row tile of an
  // activation or one expert's weight matrix, so the limit is on an expert's weights (in bf16),
  // not on the number of tokens
  if (2 * a->I * a->H * 2 >= (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct BwdPlan {
  uint16_t* dz;         // [R, H] bf16
  uint16_t* dgu;        // [R, 2I] bf16
  float* dprob_part;    // [R, parts]
  void* dx_perm;        // [R, H] io dtype
  float* part;          // FC1 dgrad split-tile partials
  // MXFP8 operands, each quantized along its GEMM's K
  uint8_t *dzq, *dzs, *w2tq, *w2ts, *dzT, *dzTs, *hT, *hTs;
  uint8_t *dguq, *dgus, *w1tq, *w1ts, *dguT, *dguTs, *xT, *xTs;
  int64_t rows_pad;
  size_t bytes;
};

BwdPlan plan_bwd(const moe_mlp_bwd_args* a, void* ws) {
  BwdPlan p{};
  Carver c(ws);
  const int64_t R = a->T * a->k, H = a->H, I = a->I;
  const int E = a->E;
  const bool mx = a->compute == MOE_MXFP8_E4M3;
  p.dz = reinterpret_cast<uint16_t*>(c.take((size_t)(R * H * 2)));
  // MXFP8: the FC2 dgrad epilogue quantizes dgu itself; bf16 dgu only into the caller's debug buffer
  p.dgu = mx ? a->dgu_bf16 : reinterpret_cast<uint16_t*>(c.take((size_t)(R * 2 * I * 2)));
  p.dprob_part = reinterpret_cast<float*>(c.take((size_t)(R * bwd_dprob_parts(I) * 4)));
  p.dx_perm = c.take((size_t)(R * H) * io_size(a->io_dtype));
  p.part = reinterpret_cast<float*>(c.take(kFc2PartBytes));
  if (mx) {
    // the token-padded layout's rows: every segment padded to 128 tokens, the row length to 512
    // (whole 16-byte E8M0 groups per row for the weight gradients' scale loads)
    const int64_t Rp = ((R + 127) / 128 * 128 + 128 * (int64_t)E + 511) / 512 * 512;
    p.rows_pad = Rp;
    auto take8 = [&](int64_t n) { return reinterpret_cast<uint8_t*>(c.take((size_t)n)); };
    p.dzq = take8(R * H); p.dzs = take8(R * H / 32);
    if (a->w2tq) {
      p.w2tq = const_cast<uint8_t*>(a->w2tq); p.w2ts = const_cast<uint8_t*>(a->w2ts);
    } else {
      p.w2tq = take8((int64_t)E * I * H); p.w2ts = take8((int64_t)E * I * H / 32);
    }
    p.dzT = take8(H * Rp); p.dzTs = take8(H * Rp / 32);
    p.hT = take8(I * Rp); p.hTs = take8(I * Rp / 32);
    if (a->dgu_codes) {
      p.dguq = a->dgu_codes; p.dgus = a->dgu_scales;
    } else {
      p.dguq = take8(R * 2 * I); p.dgus = take8(R * 2 * I / 32);
    }
    if (a->w1tq) {
      p.w1tq = const_cast<uint8_t*>(a->w1tq); p.w1ts = const_cast<uint8_t*>(a->w1ts);
    } else {
      p.w1tq = take8((int64_t)E * H * 2 * I); p.w1ts = take8((int64_t)E * H * 2 * I / 32);
    }
    if (a->dgu_t_codes) {
      p.dguT = a->dgu_t_codes; p.dguTs = a->dgu_t_scales;
    } else {
      p.dguT = take8(2 * I * Rp); p.dguTs = take8(2 * I * Rp / 32);
    }
    p.xT = take8(H * Rp); p.xTs = take8(H * Rp / 32);
  }
  p.bytes = c.used;
  return p;
}

moe_status validate_bwd(const moe_mlp_bwd_args* a) {
  if (!a) return MOE_ERR_INVALID_ARG;
  moe_status s = check_common(a->T, a->H, a->E, a->k);
  if (s != MOE_OK) return s;
  if (a->I <= 0) return MOE_ERR_INVALID_ARG;
  if (!io_ok(a->io_dtype) || !io_ok(a->dw_dtype)) return MOE_ERR_INVALID_ARG;
  if (a->compute == MOE_FP8_E4M3) return MOE_ERR_UNSUPPORTED;   // the per-tensor FP8 variant is forward only
  if (a->compute != MOE_BF16 && a->compute != MOE_MXFP8_E4M3) return MOE_ERR_INVALID_ARG;
  const int64_t align = a->compute == MOE_BF16 ? 64 : 128;
  if (a->H % align || a->I % align) return MOE_ERR_UNSUPPORTED;
  if (!a->dy || !a->w1 || !a->w2 || !a->dx || !a->dprob || !a->dw1 || !a->dw2) return MOE_ERR_INVALID_ARG;
  if (!a->split_sizes || !a->offsets || !a->row_id_map || !a->src_index || !a->prob_perm) return MOE_ERR_INVALID_ARG;
  if (!a->saved_x_perm || !a->saved_gu || !a->saved_h) return MOE_ERR_INVALID_ARG;
  const bool any_wt = a->w1tq || a->w1ts || a->w2tq || a->w2ts;
  const bool all_wt = a->w1tq && a->w1ts && a->w2tq && a->w2ts;
  if (any_wt && (!all_wt || a->compute != MOE_MXFP8_E4M3)) return MOE_ERR_INVALID_ARG;
  const bool any_dbg = a->dgu_bf16 || a->dgu_codes || a->dgu_scales || a->dgu_t_codes || a->dgu_t_scales;
  const bool all_dbg = a->dgu_bf16 && a->dgu_codes && a->dgu_scales && a->dgu_t_codes && a->dgu_t_scales;
  if (any_dbg && (!all_dbg || a->compute != MOE_MXFP8_E4M3)) return MOE_ERR_INVALID_ARG;
  for (int e = 0; e < a->E; ++e)
    if (!a->w1[e] || !a->w2[e] || !a->dw1[e] || !a->dw2[e]) return MOE_ERR_INVALID_ARG;
  // 32-bit buffer ranges inside the GEMMs: per tile of an activation (the BF16 wgrad's token
  // segments get one descriptor per 64-token stage), per expert of the weights and of dW in fp32,
  // and, for the MXFP8 wgrad, per 256 rows of the token-contiguous operands
  const int64_t R = a->T * a->k;
  if (2 * a->I * a->H * 4 >= (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (a->compute == MOE_MXFP8_E4M3) {
    const int64_t Rp = (R + 127) / 128 * 128 + 128 * (int64_t)a->E;
    if (256 * Rp >= (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

// Per-tensor FP8 forward after the index pass: X_perm (bf16, then quantized per expert
// segment), the weights (per expert tensor), FC1 on unit-scaled codes writing bf16 h and each
// expert's amax of it, h quantized per expert segment, FC2, combine.  Every tensor's scale
// comes from its own amax.
template <typename Mark>
moe_status fwd_fp8_tail(const moe_mlp_fwd_args* a, const FwdPlan& p, hipStream_t st, Mark& mark) {
  const int64_t T = a->T, H = a->H, I = a->I, R = T * a->k;
  const int E = a->E, k = a->k;
  const bool x_f32 = a->io_dtype == MOE_F32;
  HIP_TRY(launch_permute_rows(a->x, x_f32, T, H, k, a->row_id_map, p.x_bf, nullptr, false, st));
  HIP_TRY(launch_pt_quant(p.x_bf, false, R, H, a->offsets, E, reinterpret_cast<uint8_t*>(p.x_op), p.sx, nullptr,
                          p.pt_part, st));
  MOE_CHECK(mark(2), MOE_ERR_HIP);
  HIP_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(p.unit), p.unit_bytes / 4, 0x7F7F7F7Fu, st));
  HIP_TRY(launch_fill_u32(p.h_amax, E, 0u, st));
  if (!a->w1q) HIP_TRY(launch_pt_quant_weights(a->w1, E, 2 * I, H, p.w1q, p.sw1, nullptr, p.pt_part, st));
  MOE_CHECK(mark(3), MOE_ERR_HIP);
  if (!a->w1q) HIP_TRY(launch_pt_quant_weights(a->w2, E, H, I, p.w2q, p.sw2, nullptr, p.pt_part, st));
  MOE_CHECK(mark(4), MOE_ERR_HIP);

  FwdGemm g1{};
  g1.a = p.x_op;
  g1.a_scales = p.unit;
  g1.wq = p.w1q;
  g1.wq_stride = 2 * I * H;
  g1.ws = p.unit;
  g1.ws_stride = 0;
  g1.K = H;
  g1.N = I;
  g1.E = E;
  g1.split_sizes = a->split_sizes;
  g1.prob_perm = a->prob_perm;
  g1.out = p.h_bf;
  g1.save_h = reinterpret_cast<uint16_t*>(p.h_bf);
  g1.pt_s_a = p.sx;
  g1.pt_s_b = p.sw1;
  g1.pt_amax_out = p.h_amax;
  g1.h_f32 = a->h_f32;
  g1.tstat = tile_stat_slot(kStatFc1);
  HIP_TRY(launch_fc1(g1, true, st));
  HIP_TRY(launch_pt_quant(p.h_bf, false, R, I, a->offsets, E, reinterpret_cast<uint8_t*>(p.h_op), p.sh, nullptr,
                          p.pt_part, st, p.h_amax));
  MOE_CHECK(mark(5), MOE_ERR_HIP);

  FwdGemm g2{};
  g2.a = p.h_op;
  g2.a_scales = p.unit;
  g2.wq = p.w2q;
  g2.wq_stride = H * I;
  g2.ws = p.unit;
  g2.ws_stride = 0;
  g2.K = I;
  g2.N = H;
  g2.E = E;
  g2.split_sizes = a->split_sizes;
  g2.out = p.z;
  g2.part = p.part;
  g2.out_f32 = x_f32;
  g2.pt_s_a = p.sh;
  g2.pt_s_b = p.sw2;
  g2.tstat = tile_stat_slot(kStatFc2);
  HIP_TRY(launch_fc2(g2, true, st));
  MOE_CHECK(mark(6), MOE_ERR_HIP);

  HIP_TRY(launch_combine(p.z, x_f32, T, H, k, a->row_id_map, a->out, x_f32, st));
  MOE_CHECK(mark(7), MOE_ERR_HIP);
  return MOE_OK;
}

// Host-side checks of a permutation call (nothing enqueued).
moe_status check_permute(const void* x, int x_dtype, int64_t T, int64_t H, const int32_t* topk_idx,
                         const float* topk_prob, int k, int E, int perm_dtype, const void* x_perm,
                         const uint8_t* x_perm_scales, const int32_t* split_sizes, const int32_t* offsets,
                         const int32_t* row_id_map, const int32_t* src_index, const float* prob_perm) {
  moe_status s = check_common(T, x_perm ? H : 1, E, k);
  if (s != MOE_OK) return s;
  MOE_CHECK(topk_idx && split_sizes && offsets && row_id_map && src_index, MOE_ERR_INVALID_ARG);
  MOE_CHECK(!prob_perm || topk_prob, MOE_ERR_INVALID_ARG);
  MOE_CHECK(perm_dtype == MOE_BF16 || perm_dtype == MOE_MXFP8_E4M3, MOE_ERR_INVALID_ARG);
  if (x_perm) {
    MOE_CHECK(x && io_ok(x_dtype), MOE_ERR_INVALID_ARG);
    MOE_CHECK(H % 32 == 0, MOE_ERR_UNSUPPORTED);
    if (perm_dtype == MOE_MXFP8_E4M3) MOE_CHECK(x_perm_scales != nullptr, MOE_ERR_INVALID_ARG);
  }
  return MOE_OK;
}

// The permutation's launches with the index scratch carved from `ws` (error_flag: where the
// bad-id flag goes instead of the scratch's first word, or nullptr).
moe_status permute_launch(const void* x, int x_dtype, int64_t T, int64_t H, const int32_t* topk_idx,
                          const float* topk_prob, int k, int E, int perm_dtype, void* x_perm,
                          uint8_t* x_perm_scales, int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                          int32_t* src_index, float* prob_perm, void* ws, int32_t* error_flag, hipStream_t st) {
  Carver c(ws);
  PermWs w = carve_perm(c, T, E);
  if (error_flag) w.err = error_flag;
  HIP_TRY(launch_permute_indices(topk_idx, topk_prob, T, k, E, split_sizes, offsets, row_id_map, src_index,
                                 prob_perm, w.err, w.block_counts, w.block_base, st));
  if (x_perm)
    HIP_TRY(launch_permute_rows(x, x_dtype == MOE_F32, T, H, k, row_id_map, x_perm, x_perm_scales,
                                perm_dtype == MOE_MXFP8_E4M3, st));
  return MOE_OK;
}

constexpr int kMaxDevices = 64;

// diagnostic per-wave cycle counts of the grouped GEMMs (moe_set_tile_stats), or null
uint32_t* g_tile_stats = nullptr;

}  // namespace

uint32_t* moe::tile_stat_slot(int slot) {
  return g_tile_stats ? g_tile_stats + (size_t)slot * kTileStatLaunchWords : nullptr;
}

extern "C" {

int moe_abi_version(void) { return 7; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

moe_status mxfp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int axis,
                          const int32_t* group_offsets, int num_groups, uint8_t* q, uint8_t* scales,
                          void* stream) {
  MOE_CHECK(x && q && scales, MOE_ERR_INVALID_ARG);
  MOE_CHECK(rows > 0 && cols > 0 && io_ok(x_dtype), MOE_ERR_INVALID_ARG);
  MOE_CHECK(cols % 32 == 0 || axis == 1, MOE_ERR_UNSUPPORTED);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (axis == 0) {
    HIP_TRY(launch_mx_quant_rows(x, x_dtype == MOE_F32, rows, cols, q, scales, st));
    return MOE_OK;
  }
  if (axis == 1) {
    MOE_CHECK(group_offsets && num_groups >= 1 && num_groups <= MOE_MAX_EXPERTS, MOE_ERR_INVALID_ARG);
    MOE_CHECK(cols % 32 == 0, MOE_ERR_UNSUPPORTED);
    const int64_t rows_pad = (rows + 31) / 32 * 32 + 32 * (int64_t)num_groups;
    HIP_TRY(launch_mx_quant_cols(x, x_dtype == MOE_F32, rows, cols, group_offsets, num_groups, rows_pad, q, scales,
                                 st));
    return MOE_OK;
  }
  return MOE_ERR_INVALID_ARG;
}

moe_status mxfp8_quantize_weights(const void* const* w, int E, int64_t rows, int64_t cols, int axis,
                                  const int32_t* skip, uint8_t* q, uint8_t* scales, void* stream) {
  MOE_CHECK(w && q && scales, MOE_ERR_INVALID_ARG);
  MOE_CHECK(E >= 1 && E <= MOE_MAX_EXPERTS && rows > 0 && cols > 0, MOE_ERR_INVALID_ARG);
  MOE_CHECK(axis == 0 || axis == 1, MOE_ERR_INVALID_ARG);
  for (int e = 0; e < E; ++e) MOE_CHECK(w[e] != nullptr, MOE_ERR_INVALID_ARG);
  MOE_CHECK(cols % 32 == 0 && (axis == 0 || rows % 32 == 0), MOE_ERR_UNSUPPORTED);
  MOE_CHECK(rows < (int64_t)INT32_MAX && cols < (int64_t)INT32_MAX, MOE_ERR_UNSUPPORTED);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (axis == 0) HIP_TRY(launch_mx_quant_weights(w, E, rows, cols, q, scales, skip, st));
  else HIP_TRY(launch_mx_quant_weights_t(w, E, rows, cols, q, scales, skip, st));
  return MOE_OK;
}

size_t fp8_tensor_quantize_workspace(int num_groups) {
  if (num_groups < 1 || num_groups > MOE_MAX_EXPERTS) return 0;
  return align_up(pt_part_floats(num_groups) * sizeof(float));
}

moe_status fp8_tensor_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, const int32_t* group_offsets,
                               int num_groups, uint8_t* q, float* scales, void* workspace, size_t workspace_bytes,
                               void* stream) {
  MOE_CHECK(x && q && scales, MOE_ERR_INVALID_ARG);
  MOE_CHECK(rows > 0 && cols > 0 && io_ok(x_dtype), MOE_ERR_INVALID_ARG);
  MOE_CHECK(num_groups >= 1 && num_groups <= MOE_MAX_EXPERTS, MOE_ERR_INVALID_ARG);
  MOE_CHECK(group_offsets || num_groups == 1, MOE_ERR_INVALID_ARG);
  MOE_CHECK(cols % 8 == 0, MOE_ERR_UNSUPPORTED);
  const size_t need = fp8_tensor_quantize_workspace(num_groups);
  MOE_CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE);
  HIP_TRY(launch_pt_quant(x, x_dtype == MOE_F32, rows, cols, group_offsets, num_groups, q, scales, nullptr,
                          reinterpret_cast<float*>(workspace), reinterpret_cast<hipStream_t>(stream)));
  return MOE_OK;
}

size_t moe_permute_workspace_size(int64_t T, int k, int E) {
  if (T <= 0 || k <= 0 || E <= 0) return 0;
  Carver c(nullptr);
  carve_perm(c, T, E);
  return c.used;
}

moe_status moe_permute(const void* x, int x_dtype, int64_t T, int64_t H, const int32_t* topk_idx,
                       const float* topk_prob, int k, int E, int perm_dtype, void* x_perm,
                       uint8_t* x_perm_scales, int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                       int32_t* src_index, float* prob_perm, void* workspace, size_t workspace_bytes,
                       void* stream) {
  moe_status s = check_permute(x, x_dtype, T, H, topk_idx, topk_prob, k, E, perm_dtype, x_perm, x_perm_scales,
                               split_sizes, offsets, row_id_map, src_index, prob_perm);
  if (s != MOE_OK) return s;
  const size_t need = moe_permute_workspace_size(T, k, E);
  MOE_CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE);
  return permute_launch(x, x_dtype, T, H, topk_idx, topk_prob, k, E, perm_dtype, x_perm, x_perm_scales,
                        split_sizes, offsets, row_id_map, src_index, prob_perm, workspace, nullptr,
                        reinterpret_cast<hipStream_t>(stream));
}

// ---- the allocation-free permutation: its index scratch (the error flag, per-block expert
// counts and bases) is this file-scope device array instead of a workspace.  Every GPU the
// library runs on holds its own copy until the process ends; host code never passes the array's
// name to a kernel (on the host it only stands in for the symbol) but the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (nullptr on failure).
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

moe_status moe_permute_noalloc(const void* x, int x_dtype, int64_t T, int64_t H, const int32_t* topk_idx,
                               const float* topk_prob, int k, int E, int perm_dtype, void* x_perm,
                               uint8_t* x_perm_scales, int32_t* split_sizes, int32_t* offsets,
                               int32_t* row_id_map, int32_t* src_index, float* prob_perm, int32_t* error_flag,
                               void* stream) {
  moe_status s = check_permute(x, x_dtype, T, H, topk_idx, topk_prob, k, E, perm_dtype, x_perm, x_perm_scales,
                               split_sizes, offsets, row_id_map, src_index, prob_perm);
  if (s != MOE_OK) return s;
  // the scratch holds a fixed number of bytes: larger index problems are refused up front
  MOE_CHECK(moe_permute_workspace_size(T, k, E) <= (size_t)MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_UNSUPPORTED);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int dev = -1, sdev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (st) {
    HIP_TRY(hipStreamGetDevice(st, &sdev));
    MOE_CHECK(sdev == dev, MOE_ERR_INVALID_ARG);   // the stream must belong to the current device
  }
  void* ws = scratch_ptr(dev);
  MOE_CHECK(ws != nullptr, MOE_ERR_HIP);
  return permute_launch(x, x_dtype, T, H, topk_idx, topk_prob, k, E, perm_dtype, x_perm, x_perm_scales,
                        split_sizes, offsets, row_id_map, src_index, prob_perm, ws, error_flag, st);
}

moe_status moe_route_topk(const void* logits, int logits_dtype, int64_t T, int E, int k, int32_t* topk_idx,
                          float* topk_prob, void* stream) {
  moe_status s = check_common(T, 1, E, k);
  if (s != MOE_OK) return s;
  MOE_CHECK(logits && io_ok(logits_dtype) && topk_idx && topk_prob, MOE_ERR_INVALID_ARG);
  HIP_TRY(launch_router(logits, logits_dtype == MOE_F32, T, E, k, topk_idx, topk_prob, nullptr,
                        reinterpret_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_route_permute(const void* logits, int logits_dtype, const void* x, int x_dtype, int64_t T,
                             int64_t H, int E, int k, int perm_dtype, int32_t* topk_idx, float* topk_prob,
                             void* x_perm, uint8_t* x_perm_scales, int32_t* split_sizes, int32_t* offsets,
                             int32_t* row_id_map, int32_t* src_index, float* prob_perm, void* workspace,
                             size_t workspace_bytes, void* stream) {
  moe_status s = check_common(T, x_perm ? H : 1, E, k);
  if (s != MOE_OK) return s;
  MOE_CHECK(logits && io_ok(logits_dtype) && topk_idx && topk_prob, MOE_ERR_INVALID_ARG);
  MOE_CHECK(split_sizes && offsets && row_id_map && src_index, MOE_ERR_INVALID_ARG);
  MOE_CHECK(perm_dtype == MOE_BF16 || perm_dtype == MOE_MXFP8_E4M3, MOE_ERR_INVALID_ARG);
  if (x_perm) {
    MOE_CHECK(x && io_ok(x_dtype), MOE_ERR_INVALID_ARG);
    MOE_CHECK(H % 32 == 0, MOE_ERR_UNSUPPORTED);
    if (perm_dtype == MOE_MXFP8_E4M3) MOE_CHECK(x_perm_scales != nullptr, MOE_ERR_INVALID_ARG);
  }
  const size_t need = moe_permute_workspace_size(T, k, E);
  MOE_CHECK(workspace && workspace_bytes >= need, MOE_ERR_WORKSPACE);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Carver c(workspace);
  PermWs w = carve_perm(c, T, E);
  HIP_TRY(launch_router(logits, logits_dtype == MOE_F32, T, E, k, topk_idx, topk_prob, w.block_counts, st));
  HIP_TRY(launch_permute_indices(topk_idx, topk_prob, T, k, E, split_sizes, offsets, row_id_map, src_index,
                                 prob_perm, w.err, w.block_counts, w.block_base, st, /*counts_ready=*/true));
  if (x_perm)
    HIP_TRY(launch_permute_rows(x, x_dtype == MOE_F32, T, H, k, row_id_map, x_perm, x_perm_scales,
                                perm_dtype == MOE_MXFP8_E4M3, st));
  return MOE_OK;
}

size_t moe_grouped_mlp_fwd_workspace(const moe_mlp_fwd_args* a) {
  if (validate_fwd(a) != MOE_OK) return 0;
  return plan_fwd(a, nullptr).bytes;
}

static const char* const kFwdPhases[] = {"permute_index", "permute_rows", "quant_w1", "quant_w2",
                                         "fc1_gateup_swiglu", "fc2_down", "combine"};
constexpr int kNumFwdPhases = 7;

int moe_fwd_phase_count(void) { return kNumFwdPhases; }
const char* moe_fwd_phase_name(int i) { return (i >= 0 && i < kNumFwdPhases) ? kFwdPhases[i] : nullptr; }

moe_status moe_grouped_mlp_fwd(const moe_mlp_fwd_args* a, void* stream) {
  return moe_grouped_mlp_fwd_ex(a, stream, nullptr);
}

moe_status moe_grouped_mlp_fwd_ex(const moe_mlp_fwd_args* a, void* stream, void* const* events) {
  moe_status s = validate_fwd(a);
  if (s != MOE_OK) return s;
  const size_t need = plan_fwd(a, nullptr).bytes;
  MOE_CHECK(a->workspace && a->workspace_bytes >= need, MOE_ERR_WORKSPACE);
  FwdPlan p = plan_fwd(a, a->workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t T = a->T, H = a->H, I = a->I;
  const int E = a->E, k = a->k;
  const bool mx = a->compute == MOE_MXFP8_E4M3;
  const bool x_f32 = a->io_dtype == MOE_F32;
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), st) == hipSuccess;
  };

  MOE_CHECK(mark(0), MOE_ERR_HIP);
  HIP_TRY(launch_permute_indices(a->topk_idx, a->topk_prob, T, k, a->E, a->split_sizes, a->offsets, a->row_id_map,
                                 a->src_index, a->prob_perm, p.perm.err, p.perm.block_counts, p.perm.block_base,
                                 st));
  MOE_CHECK(mark(1), MOE_ERR_HIP);
  if (a->compute == MOE_FP8_E4M3) return fwd_fp8_tail(a, p, st, mark);
  if (mx) {
    HIP_TRY(launch_permute_rows(a->x, x_f32, T, H, k, a->row_id_map, p.x_op, p.x_sc, true, st));
    if (a->saved_x_perm)
      HIP_TRY(launch_permute_rows(a->x, x_f32, T, H, k, a->row_id_map, a->saved_x_perm, nullptr, false, st));
    MOE_CHECK(mark(2), MOE_ERR_HIP);
    // per-call weight quantization; with the backward's transposed copies requested, one read of
    // each bf16 weight gives both
    if (!a->w1q && a->w1tq_out)
      HIP_TRY(launch_mx_quant_weights_t(a->w1, E, 2 * I, H, a->w1tq_out, a->w1ts_out, a->split_sizes, st, p.w1q, p.w1s));
    else if (!a->w1q)
      HIP_TRY(launch_mx_quant_weights(a->w1, E, 2 * I, H, p.w1q, p.w1s, a->split_sizes, st));
    MOE_CHECK(mark(3), MOE_ERR_HIP);
    if (!a->w1q && a->w2tq_out)
      HIP_TRY(launch_mx_quant_weights_t(a->w2, E, H, I, a->w2tq_out, a->w2ts_out, a->split_sizes, st, p.w2q, p.w2s));
    else if (!a->w1q)
      HIP_TRY(launch_mx_quant_weights(a->w2, E, H, I, p.w2q, p.w2s, a->split_sizes, st));
  } else {
    HIP_TRY(launch_permute_rows(a->x, x_f32, T, H, k, a->row_id_map, p.x_op, nullptr, false, st));
    MOE_CHECK(mark(2), MOE_ERR_HIP);
    MOE_CHECK(mark(3), MOE_ERR_HIP);
  }
  MOE_CHECK(mark(4), MOE_ERR_HIP);

  FwdGemm g1{};
  g1.a = p.x_op;
  g1.a_scales = p.x_sc;
  g1.w_tab = a->w1;
  g1.wq = p.w1q;
  g1.wq_stride = 2 * I * H;
  g1.ws = p.w1s;
  g1.ws_stride = 2 * I * H / 32;
  g1.K = H;
  g1.N = I;
  g1.E = E;
  g1.split_sizes = a->split_sizes;
  g1.prob_perm = a->prob_perm;
  g1.out = p.h_op;
  g1.out_scales = p.h_sc;
  g1.save_gu = reinterpret_cast<uint16_t*>(a->saved_gu);
  g1.save_h = mx ? reinterpret_cast<uint16_t*>(a->saved_h) : nullptr;
  g1.h_f32 = a->h_f32;
  g1.tstat = tile_stat_slot(kStatFc1);
  HIP_TRY(launch_fc1(g1, mx, st));
  MOE_CHECK(mark(5), MOE_ERR_HIP);

  FwdGemm g2{};
  g2.a = p.h_op;
  g2.a_scales = p.h_sc;
  g2.w_tab = a->w2;
  g2.wq = p.w2q;
  g2.wq_stride = H * I;
  g2.ws = p.w2s;
  g2.ws_stride = H * I / 32;
  g2.K = I;
  g2.N = H;
  g2.E = E;
  g2.split_sizes = a->split_sizes;
  g2.out = p.z;
  g2.part = p.part;
  g2.out_f32 = x_f32;
  g2.tstat = tile_stat_slot(kStatFc2);
  HIP_TRY(launch_fc2(g2, mx, st));
  MOE_CHECK(mark(6), MOE_ERR_HIP);

  HIP_TRY(launch_combine(p.z, x_f32, T, H, k, a->row_id_map, a->out, x_f32, st));
  MOE_CHECK(mark(7), MOE_ERR_HIP);
  return MOE_OK;
}

moe_status moe_grouped_mlp_fwd_loop(const moe_mlp_fwd_args* a, const int32_t* split_sizes_host, void* stream) {
  moe_status s = validate_fwd(a);
  if (s != MOE_OK) return s;
  MOE_CHECK(split_sizes_host != nullptr, MOE_ERR_INVALID_ARG);
  MOE_CHECK(a->compute != MOE_FP8_E4M3, MOE_ERR_UNSUPPORTED);
  MOE_CHECK(!a->w1tq_out, MOE_ERR_UNSUPPORTED);   // the baseline quantizes the forward's copy only
  int64_t sum = 0;
  for (int e = 0; e < a->E; ++e) {
    MOE_CHECK(split_sizes_host[e] >= 0, MOE_ERR_INVALID_ARG);
    sum += split_sizes_host[e];
  }
  MOE_CHECK(sum == a->T * a->k, MOE_ERR_INVALID_ARG);
  const size_t need = plan_fwd(a, nullptr).bytes;
  MOE_CHECK(a->workspace && a->workspace_bytes >= need, MOE_ERR_WORKSPACE);
  FwdPlan p = plan_fwd(a, a->workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t T = a->T, H = a->H, I = a->I;
  const int E = a->E, k = a->k;
  const bool mx = a->compute == MOE_MXFP8_E4M3;
  const bool x_f32 = a->io_dtype == MOE_F32;
  const int64_t esz = mx ? 1 : 2;

  HIP_TRY(launch_permute_indices(a->topk_idx, a->topk_prob, T, k, E, a->split_sizes, a->offsets, a->row_id_map,
                                 a->src_index, a->prob_perm, p.perm.err, p.perm.block_counts, p.perm.block_base,
                                 st));
  HIP_TRY(launch_permute_rows(a->x, x_f32, T, H, k, a->row_id_map, p.x_op, p.x_sc, mx, st));
  if (mx && a->saved_x_perm)
    HIP_TRY(launch_permute_rows(a->x, x_f32, T, H, k, a->row_id_map, a->saved_x_perm, nullptr, false, st));
  int64_t row0 = 0;
  for (int e = 0; e < E; ++e) {
    const int64_t Me = split_sizes_host[e];
    if (Me == 0) continue;
    uint8_t* xo = reinterpret_cast<uint8_t*>(p.x_op) + row0 * H * esz;
    uint8_t* ho = reinterpret_cast<uint8_t*>(p.h_op) + row0 * I * esz;
    // MXFP8 weights of expert e: cached by the caller, or quantized here into slot 0
    const uint8_t* w1q_e = a->w1q ? a->w1q + e * 2 * I * H : p.w1q;
    const uint8_t* w1s_e = a->w1q ? a->w1s + e * 2 * I * H / 32 : p.w1s;
    const uint8_t* w2q_e = a->w1q ? a->w2q + e * H * I : p.w2q;
    const uint8_t* w2s_e = a->w1q ? a->w2s + e * H * I / 32 : p.w2s;
    if (mx && !a->w1q) {
      HIP_TRY(launch_mx_quant_weights(a->w1 + e, 1, 2 * I, H, p.w1q, p.w1s, nullptr, st));
      HIP_TRY(launch_mx_quant_weights(a->w2 + e, 1, H, I, p.w2q, p.w2s, nullptr, st));
    }
    FwdGemm g1{};
    g1.a = xo;
    g1.a_scales = mx ? p.x_sc + row0 * (H / 32) : nullptr;
    g1.w_tab = a->w1 ? a->w1 + e : nullptr;
    g1.wq = w1q_e;
    g1.ws = w1s_e;
    g1.K = H;
    g1.N = I;
    g1.E = 1;
    g1.split_sizes = a->split_sizes + e;   // the expert's own count, on the device
    g1.prob_perm = a->prob_perm + row0;
    g1.out = ho;
    g1.out_scales = mx ? p.h_sc + row0 * (I / 32) : nullptr;
    g1.save_gu = a->saved_gu ? reinterpret_cast<uint16_t*>(a->saved_gu) + row0 * 2 * I : nullptr;
    g1.save_h = (mx && a->saved_h) ? reinterpret_cast<uint16_t*>(a->saved_h) + row0 * I : nullptr;
    g1.h_f32 = a->h_f32 ? a->h_f32 + row0 * I : nullptr;
    HIP_TRY(launch_fc1(g1, mx, st));
    FwdGemm g2{};
    g2.a = ho;
    g2.a_scales = g1.out_scales;
    g2.w_tab = a->w2 ? a->w2 + e : nullptr;
    g2.wq = w2q_e;
    g2.ws = w2s_e;
    g2.K = I;
    g2.N = H;
    g2.E = 1;
    g2.split_sizes = a->split_sizes + e;
    g2.out = reinterpret_cast<uint8_t*>(p.z) + row0 * H * io_size(a->io_dtype);
    g2.part = nullptr;
    g2.out_f32 = x_f32;
    HIP_TRY(launch_fc2(g2, mx, st));
    row0 += Me;
  }
  HIP_TRY(launch_combine(p.z, x_f32, T, H, k, a->row_id_map, a->out, x_f32, st));
  return MOE_OK;
}

size_t moe_grouped_mlp_bwd_workspace(const moe_mlp_bwd_args* a) {
  if (validate_bwd(a) != MOE_OK) return 0;
  return plan_bwd(a, nullptr).bytes;
}

static const char* const kBwdPhases[] = {"gather_dy", "quant_dgrad_fc2", "dgrad_fc2_swiglu_bwd",
                                         "quant_wgrad_fc2", "wgrad_fc2", "quant_dgrad_fc1", "dgrad_fc1",
                                         "quant_wgrad_fc1", "wgrad_fc1", "unpermute_dx_dprob"};
constexpr int kNumBwdPhases = 10;

int moe_bwd_phase_count(void) { return kNumBwdPhases; }
const char* moe_bwd_phase_name(int i) { return (i >= 0 && i < kNumBwdPhases) ? kBwdPhases[i] : nullptr; }

moe_status moe_grouped_mlp_bwd(const moe_mlp_bwd_args* a, void* stream) {
  return moe_grouped_mlp_bwd_ex(a, stream, nullptr);
}

moe_status moe_grouped_mlp_bwd_ex(const moe_mlp_bwd_args* a, void* stream, void* const* events) {
  moe_status s = validate_bwd(a);
  if (s != MOE_OK) return s;
  const size_t need = plan_bwd(a, nullptr).bytes;
  MOE_CHECK(a->workspace && a->workspace_bytes >= need, MOE_ERR_WORKSPACE);
  BwdPlan p = plan_bwd(a, a->workspace);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t T = a->T, H = a->H, I = a->I, R = T * a->k;
  const int E = a->E, k = a->k;
  const bool mx = a->compute == MOE_MXFP8_E4M3;
  const bool io_f32 = a->io_dtype == MOE_F32;
  const bool dw_f32 = a->dw_dtype == MOE_F32;
  const int parts = bwd_dprob_parts(I);
  auto mark = [&](int i) -> bool {
    return !events || hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), st) == hipSuccess;
  };

  // dz = bf16(dy) gathered into expert order.  MXFP8 with bf16 dy needs dz only as the two
  // quantized operands, which are made from dy directly (below): no gather.
  const bool dz_direct = mx && !io_f32;
  MOE_CHECK(mark(0), MOE_ERR_HIP);
  if (!dz_direct) HIP_TRY(launch_gather_rows(a->dy, io_f32, R, H, k, a->src_index, a->offsets, E, p.dz, st));
  MOE_CHECK(mark(1), MOE_ERR_HIP);

  // ---- FC2 dgrad with the ScaledSwiGLU backward epilogue -> dgu, dprob partials
  BwdGemm d2{};
  d2.M = 0; d2.N = I; d2.K = H; d2.E = E;
  d2.split_sizes = a->split_sizes;
  d2.gu = reinterpret_cast<const uint16_t*>(a->saved_gu);
  d2.prob_perm = a->prob_perm;
  d2.dgu = reinterpret_cast<uint16_t*>(p.dgu);
  d2.dprob_part = p.dprob_part;
  d2.I = I;
  if (mx) {
    d2.dgu_q = p.dguq; d2.dgu_s = p.dgus;
    d2.dgu_tq = p.dguT; d2.dgu_ts = p.dguTs;
    d2.rows_pad = p.rows_pad;
  }
  if (mx) {
    // dz along H: each token's dy row quantized once and written to its k permuted rows
    if (dz_direct) HIP_TRY(launch_permute_rows(a->dy, false, T, H, k, a->row_id_map, p.dzq, p.dzs, true, st));
    else HIP_TRY(launch_mx_quant_rows(p.dz, false, R, H, p.dzq, p.dzs, st));
    // W2_e^T along H for every expert with tokens, one launch (unless cached by the caller)
    if (!a->w2tq) HIP_TRY(launch_mx_quant_weights_t(a->w2, E, H, I, p.w2tq, p.w2ts, a->split_sizes, st));
    d2.a = p.dzq; d2.lda = H; d2.a_scales = p.dzs; d2.ldas = H / 32;
    d2.b = p.w2tq; d2.ldb = H; d2.b_stride = I * H; d2.b_scales = p.w2ts; d2.ldbs = H / 32;
    d2.bs_stride = I * (H / 32);
  } else {
    d2.a = p.dz; d2.lda = H * 2;
    d2.tab = a->w2; d2.ldb = I * 2;
  }
  MOE_CHECK(mark(2), MOE_ERR_HIP);
  d2.tstat = tile_stat_slot(kStatDgradFc2);
  HIP_TRY(launch_bwd_dgrad_fc2(d2, mx, st));
  // the token-axis scale bytes past the last padded segment: a wgrad scale-group load may read them
  if (mx) HIP_TRY(launch_scale_tail_zero(p.dguTs, 2 * I, p.rows_pad / 32, a->split_sizes, E, st));
  MOE_CHECK(mark(3), MOE_ERR_HIP);

  // ---- FC2 wgrad: dW2_e = dz_e^T h_e
  BwdGemm w2{};
  w2.M = H; w2.N = I; w2.E = E; w2.split_sizes = a->split_sizes;
  w2.tab = reinterpret_cast<const void* const*>(a->dw2);
  w2.out_f32 = dw_f32;
  if (mx) {
    const int64_t Rp = p.rows_pad;
    // dz along tokens, per expert segment (dy rows through src_index when dz was not gathered)
    if (dz_direct)
      HIP_TRY(launch_mx_quant_cols(a->dy, false, R, H, a->offsets, E, Rp, p.dzT, p.dzTs, st, 128, a->src_index, k));
    else
      HIP_TRY(launch_mx_quant_cols(p.dz, false, R, H, a->offsets, E, Rp, p.dzT, p.dzTs, st, 128));
    HIP_TRY(launch_mx_quant_cols(a->saved_h, false, R, I, a->offsets, E, Rp, p.hT, p.hTs, st, 128));
    w2.a = p.dzT; w2.lda = Rp; w2.a_scales = p.dzTs; w2.ldas = Rp / 32;
    w2.b = p.hT; w2.ldb = Rp; w2.b_scales = p.hTs; w2.ldbs = Rp / 32;
    w2.pad = 128;
  } else {
    w2.a = p.dz; w2.lda = H * 2;
    w2.b = a->saved_h; w2.ldb = I * 2;
  }
  MOE_CHECK(mark(4), MOE_ERR_HIP);
  w2.tstat = tile_stat_slot(kStatWgradFc2);
  HIP_TRY(launch_bwd_wgrad(w2, mx, st));
  MOE_CHECK(mark(5), MOE_ERR_HIP);

  // ---- FC1 dgrad: dx_perm = dgu . W1_e
  BwdGemm d1{};
  d1.N = H; d1.K = 2 * I; d1.E = E; d1.split_sizes = a->split_sizes;
  d1.out = p.dx_perm; d1.out_f32 = io_f32; d1.part = p.part;
  if (mx) {
    // dgu along 2I: quantized by the FC2 dgrad epilogue
    // W1_e^T along 2I for every expert with tokens, one launch (unless cached by the caller)
    if (!a->w1tq) HIP_TRY(launch_mx_quant_weights_t(a->w1, E, 2 * I, H, p.w1tq, p.w1ts, a->split_sizes, st));
    d1.a = p.dguq; d1.lda = 2 * I; d1.a_scales = p.dgus; d1.ldas = 2 * I / 32;
    d1.b = p.w1tq; d1.ldb = 2 * I; d1.b_stride = H * 2 * I; d1.b_scales = p.w1ts; d1.ldbs = 2 * I / 32;
    d1.bs_stride = H * (2 * I / 32);
  } else {
    d1.a = p.dgu; d1.lda = 2 * I * 2;
    d1.tab = a->w1; d1.ldb = H * 2;
  }
  MOE_CHECK(mark(6), MOE_ERR_HIP);
  d1.tstat = tile_stat_slot(kStatDgradFc1);
  HIP_TRY(launch_bwd_dgrad_fc1(d1, mx, st));
  MOE_CHECK(mark(7), MOE_ERR_HIP);

  // ---- FC1 wgrad: dW1_e = dgu_e^T x_perm_e
  BwdGemm w1{};
  w1.M = 2 * I; w1.N = H; w1.E = E; w1.split_sizes = a->split_sizes;
  w1.tab = reinterpret_cast<const void* const*>(a->dw1);
  w1.out_f32 = dw_f32;
  if (mx) {
    const int64_t Rp = p.rows_pad;
    // dgu along tokens: quantized by the FC2 dgrad epilogue
    HIP_TRY(launch_mx_quant_cols(a->saved_x_perm, false, R, H, a->offsets, E, Rp, p.xT, p.xTs, st, 128));
    w1.a = p.dguT; w1.lda = Rp; w1.a_scales = p.dguTs; w1.ldas = Rp / 32;
    w1.b = p.xT; w1.ldb = Rp; w1.b_scales = p.xTs; w1.ldbs = Rp / 32;
    w1.pad = 128;
  } else {
    w1.a = p.dgu; w1.lda = 2 * I * 2;
    w1.b = a->saved_x_perm; w1.ldb = H * 2;
  }
  MOE_CHECK(mark(8), MOE_ERR_HIP);
  w1.tstat = tile_stat_slot(kStatWgradFc1);
  HIP_TRY(launch_bwd_wgrad(w1, mx, st));
  MOE_CHECK(mark(9), MOE_ERR_HIP);

  // ---- un-permute: dx[t] = sum_j dx_perm[row(t, j)]; dprob[t, j] = sum of the row's partials
  HIP_TRY(launch_combine(p.dx_perm, io_f32, T, H, k, a->row_id_map, a->dx, io_f32, st));
  HIP_TRY(launch_dprob_reduce(p.dprob_part, R, parts, a->row_id_map, T, k, a->dprob, st));
  MOE_CHECK(mark(10), MOE_ERR_HIP);
  return MOE_OK;
}

size_t moe_tile_stats_bytes(void) { return (size_t)kStatSlots * kTileStatLaunchWords * sizeof(uint32_t); }

moe_status moe_set_tile_stats(uint32_t* device_buf, size_t bytes) {
  if (device_buf && bytes < moe_tile_stats_bytes()) return MOE_ERR_INVALID_ARG;
  g_tile_stats = device_buf;
  return MOE_OK;
}

int moe_read_device_error(void* workspace, void* stream) {
  if (!workspace) return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return -1;
  int32_t flag = 0;
  if (hipMemcpy(&flag, workspace, sizeof(flag), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return flag;
}

}  // extern "C"
