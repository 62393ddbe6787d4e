// Backward grouped GEMMs for gfx950 (the matching fused backward of the
// grouped expert MLP, page "BioNeMo Uses Grouped Kernels and MXFP8", Fusing
// precision conversion and expert computation; page "How BioNeMo cuts
// overhead", Why fused operations matter).
//
//   FC2 dgrad  dh = dz . W2_e           (M = tokens of e, N = I, K = H)
//              epilogue: ScaledSwiGLU backward -> dGU = [dg | du] (bf16) and a
//              per-(row, N-tile) partial of dprob = sum_i dh * silu(g) * u
//   FC1 dgrad  dX_perm = dGU . W1_e     (M = tokens of e, N = H, K = 2I)
//   wgrad      dW_e = A_e^T . B_e       (M, N fixed, K = tokens of e; an expert
//              with no tokens gets an all-zero dW_e)
//
// BF16 operands whose contiguous dimension is M or N (the weights in dgrad,
// both token-major activations in wgrad) are staged in LDS as they are stored
// (mnswz layout) and read with gfx950's transposing LDS load
// (ds_read_b64_tr_b16), which delivers the MFMA's K-major operand layout.
// MXFP8 operands arrive already quantized along each GEMM's K in K-major
// layout.  The main loop is the forward's interleaved stage schedule, the last
// stage of a tile loads the first stage of the next one, and the epilogues read
// the accumulators block by block and store whole 128-byte rows through a small
// LDS slot per wave (stage_rows32).
#include "gemm_core.h"

namespace moe {
namespace {
using namespace gemm;

enum : int { kRoleDgradFc2 = 0, kRoleDgradFc1 = 1, kRoleWgrad = 2 };

struct BwdKArgs {
  const uint8_t* a;
  int64_t lda;              // bytes between A rows (K-major) or between k-rows (MN-major)
  const uint8_t* as;        // MXFP8 A scales
  int64_t ldas;
  const uint8_t* b;         // B base when it is not a weight table entry
  int64_t ldb;
  int64_t b_stride;         // MXFP8 dgrad: per-expert stride of the transposed quantized weights
  const uint8_t* bs;
  int64_t ldbs;
  int64_t bs_stride;
  int64_t M, N, K;          // dgrad: N, K fixed (M = tokens of e); wgrad: M, N fixed (K = tokens of e)
  int E, nM, nN, pad;
  const int32_t* split_sizes;
  const uint16_t* gu;       // FC2 dgrad: saved gate-up output [R, 2I]
  const float* prob_perm;
  uint16_t* dgu;            // FC2 dgrad: [R, 2I]
  float* dprob_part;        // FC2 dgrad: [R, nN]
  int64_t I;
  uint8_t* out;             // FC1 dgrad: dx_perm [R, N]
  float* part;              // FC1 dgrad split parts: kGemmGrid x 64K floats
  uint32_t* tstat;          // per-wave cycle counts (diagnostic), or null
  int split;                // FC1 dgrad: 0 every tile; 1 tiles before the split ones; 2 the split parts
  uint8_t *dgu_q, *dgu_s;   // MXFP8 FC2 dgrad: dGU quantized along 2I, [R, 2I] + [R, 2I / 32]
  uint8_t *dgu_tq, *dgu_ts; // and along tokens, [2I, rows_pad] + [2I, rows_pad / 32]
  int64_t rows_pad;
  const uint8_t* tab[kMaxExperts];   // BF16 dgrad: W_e; wgrad: dW_e
};

__device__ __forceinline__ const uint8_t* bwd_table(int e) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint8_t* const* tab = reinterpret_cast<const uint8_t* const*>(
      reinterpret_cast<const char*>(__builtin_amdgcn_kernarg_segment_ptr()) + offsetof(BwdKArgs, tab));
  return tab[e];
#else
  (void)e;
  return nullptr;
#endif
}

// One work item of the backward kernel: a 256 x 256 output tile and its K extent.
struct BwdItem {
  int t, e, mt, nt, row0, mrows, ncols, kT, Me;
  int poff;                 // MXFP8 FC2 dgrad: the expert's first column in the token-padded layout
  int kz;                   // stages with data: loads of stages kz .. kT-1 read zeros (deep wgrad)
  int part, u0;             // K part of a split tile (-1: whole K) and its first stage
  int gs;                   // deep MXFP8 wgrad: stage of the item's first stage within its 16-byte scale group
  int64_t koff;
};

// kDeep (MXFP8): the forward's deep MXFP8 pipeline -- the stage barrier between the two MX
// substeps, stage loads issued two stages ahead, and the E8M0 bytes of four stages loaded together.
//   * one 16-byte scale load per row per group of four stages.  In dgrad (K % 512 == 0) the groups
//     start at K = 0.  In wgrad the groups are the token-padded layout's own 512-token (16-byte)
//     ones -- its row length is a multiple of 512 -- and an expert's segment, which starts at a
//     multiple of 128 tokens, enters its first group at stage gs = (start / 128) % 4; the bytes of
//     a group outside the segment belong to its neighbours and are never read back.
//     Every wgrad item runs at least two stages, as the pipeline needs: the stages past an
//     expert's tokens (an expert with at most 128 tokens, or none) load zeros, which add nothing.
template <int kRole, bool kMx, bool kOutF32, bool kDeep = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_gemm_kernel(const BwdKArgs p) {
  constexpr bool kWg = kRole == kRoleWgrad;
  constexpr bool kAMN = kWg && !kMx;   // bf16 wgrad: A is token-major
  constexpr bool kBMN = !kMx;          // bf16: B is N-contiguous (weights in dgrad, activations in wgrad)
  constexpr bool kD2 = kRole == kRoleDgradFc2;
  static_assert(!kDeep || kMx, "deep pipeline: MXFP8 only");
  // two stages of A + B (64 KB each), the MXFP8 scales (2 x 2 KB of one word per row per stage, or
  // in the deep pipeline 2 x 8 KB of 16 bytes per row per group of four stages), and for the FC2
  // dgrad the routing probabilities of the tile's rows (2 x 1 KB, by work item) and the per-row
  // dprob partials of the two wave columns (2 x 1 KB)
  constexpr int kScOff = 2 * kStageBytes;
  constexpr int kScBuf = kDeep ? 8192 : 2048;
  constexpr int kXOff = kScOff + (kMx ? 2 * kScBuf : 0);
  // MXFP8 FC2 dgrad: a 32 x 32 bf16 block per wave (2 KB each) for the transposes of the
  // token-axis quantization
  constexpr bool kQ = kD2 && kMx;
  constexpr int kTOff = kXOff + 4096;
  // BF16 FC2 dgrad: a 32 x 128-byte staging slot per wave (4 KB each) for full-line dG / dU stores
  constexpr bool kStage = kD2 && !kMx;
  constexpr int kSOff = kXOff + 4096;
  // the other roles' outputs (weight gradients, FC1 dgrad and its split parts): a 16 x 128-byte
  // slot per wave (2 KB each) for full-line stores
  constexpr bool kStageF = !kD2;
  constexpr int kFOff = kXOff + 16;
  __shared__ __attribute__((aligned(16)))
  uint8_t smem[kXOff + (kD2 ? 4096 : 16) + (kQ ? 4 * 2048 : 0) + (kStage ? 4 * 4096 : 0) + (kStageF ? 4 * 2048 : 0)];
  __shared__ Sched sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = p.E;
  build_sched(sched, p.split_sizes, E, p.nN, kWg ? (kMx ? p.pad : 1) : 0);
  // wgrad: every expert has the same nM x nN tiles, of K = its token count.  The tile space takes
  // the experts in decreasing K (ties by index), and a round's 256 consecutive tiles are dealt to
  // the workgroups forwards in even rounds and backwards in odd ones, so that a workgroup's long
  // tiles of one round meet short ones of the next -- with skewed routing, a plain deal leaves
  // some workgroups a sum of K well above the mean (64-expert FC2 wgrad: slowest wave 1.3-1.4x
  // the mean).  Each round's tiles still go to the XCDs 32 consecutive ones at a time.
  __shared__ int16_t worder[kWg ? kMaxExperts : 1];
  if constexpr (kWg) {
    if (tid < E) {
      const int c = sched.cnt[tid];
      int rank = 0;
      for (int e2 = 0; e2 < E; ++e2) {
        const int c2 = sched.cnt[e2];
        rank += (c2 > c || (c2 == c && e2 < tid)) ? 1 : 0;
      }
      worder[rank] = (int16_t)tid;
    }
    __syncthreads();
  }
  const int total = kWg ? E * p.nM * p.nN : __builtin_amdgcn_readfirstlane(sched.tile[E]);
  const int G = gridDim.x, per = G >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  constexpr int kKStep = kMx ? 128 : 64;                  // K values per LDS stage
  const int kU = kWg ? 0 : (int)(p.K * (kMx ? 1 : 2) / kRowBytes);   // dgrad K units of 128 bytes

  // FC1 dgrad balances its last round like the forward down projection: the rem = total % G tiles
  // of the last round are split into S parts along K; pass 1 runs tiles [0, full), pass 2 (the
  // fp32 instance) the parts, which store fp32 tiles to p.part for the fixup kernel to sum.
  int full = total, S = 1;
  if (kRole == kRoleDgradFc1 && p.split) split_policy(total, G, kU, full, S);
  const int lo = p.split == 2 ? full : 0;
  const int hi = p.split == 0 ? total : (p.split == 1 ? full : (S > 1 ? full + (total - full) * S : full));

  auto decode = [&](int round, BwdItem& it) {
    const int pos = xcd * per + slot;
    it.t = lo + round * G + ((kWg && (round & 1)) ? G - 1 - pos : pos);
    it.kT = 0;
    it.kz = 0;
    it.u0 = 0;
    it.gs = 0;
    it.part = -1;
    if (it.t >= hi) return;
    if constexpr (kWg) {
      const int pe = p.nM * p.nN;
      const int rank = it.t / pe;
      it.e = __builtin_amdgcn_readfirstlane((int)worder[rank]);
      const int local = it.t - rank * pe;
      // groups of 4 M-tiles when an expert's dW has few of them (FC2's H / 256 = 16): measured
      // 10 % faster for that wgrad than groups of 8, the same for FC1's 2I / 256 = 112
      tile_coords(local, p.nM, p.nN, it.mt, it.nt, p.nM <= 16 ? 4 : kGroupM);
      it.Me = __builtin_amdgcn_readfirstlane(sched.cnt[it.e]);
      it.koff = kMx ? __builtin_amdgcn_readfirstlane(sched.tile[it.e]) : __builtin_amdgcn_readfirstlane(sched.off[it.e]);
      it.kT = (it.Me + kKStep - 1) / kKStep;
      it.kz = it.kT;
      if (kDeep) it.gs = (int)((it.koff / 128) & 3);
      if (kDeep && it.kT < 2) it.kT = 2;
      it.row0 = it.mt * kBM;
      it.mrows = (int)min((int64_t)kBM, p.M - it.row0);
    } else {
      int tile = it.t;
      if (kOutF32 && p.split == 2) {
        tile = full + (it.t - full) / S;
        it.part = (it.t - full) % S;
      }
      it.e = __builtin_amdgcn_readfirstlane(find_expert(sched, E, tile));
      it.Me = __builtin_amdgcn_readfirstlane(sched.cnt[it.e]);
      if constexpr (kQ) {
        int po = 0;
        for (int e2 = 0; e2 < it.e; ++e2) po += (sched.cnt[e2] + 127) / 128 * 128;
        it.poff = __builtin_amdgcn_readfirstlane(po);
      }
      const int nMe = (it.Me + kBM - 1) / kBM;
      const int local = tile - __builtin_amdgcn_readfirstlane(sched.tile[it.e]);
      tile_coords(local, nMe, p.nN, it.mt, it.nt);
      it.row0 = __builtin_amdgcn_readfirstlane(sched.off[it.e]) + it.mt * kBM;
      it.mrows = min(kBM, it.Me - it.mt * kBM);
      it.koff = 0;
      it.u0 = it.part < 0 ? 0 : it.part * kU / S;
      it.kT = (it.part < 0 ? kU : (it.part + 1) * kU / S) - it.u0;
      it.kz = it.u0 + it.kT;
    }
    it.ncols = (int)min((int64_t)kBN, p.N - (int64_t)it.nt * kBN);
  };

  // ---- operands: two LDS stages of A and B (32 KB each) filled by direct-to-LDS loads
  // (buffer_load_dwordx4 ... lds, lane L's 16 bytes to slot L of a contiguous 1 KB block).
  //   K-major operand: 256 rows x 128 bytes of K in the swz layout; load q of wave w fills row
  //     pairs j = 4 (8w + q) + L / 16, slot s = L % 16 holding (row parity, chunk) = s ^ hs(j).
  //   MN-major operand (bf16, K rows of 256 contiguous columns): 64 K rows x 512 bytes in the
  //     mnswz layout; load q of wave w fills rows 2 (8w + q) + L / 32, physical chunk L % 32.
  //     In dgrad the K row advance is carried in the per-lane offset.  In wgrad (the token-major
  //     activations, whose token segment may span more than 4 GB) each stage gets descriptors
  //     based at its first token row, ending at the segment's end: rows past a ragged segment read
  //     zero, and no offset leaves 32 bits.
  //   MXFP8 operands are K-major, with one 4-byte E8M0 word per row per stage.
  // Invalid items and items without K stages get zero-range descriptors: their loads touch no
  // memory.
  struct Desc {
    i32x4 va, vb, vas, vbs;
    const uint8_t *pa, *pb;   // BF16 wgrad: operand bases of the item's first token row
    int64_t ea, eb;           // and the bytes from there to the segment's end
  };
  auto descs = [&](const BwdItem& it, Desc& d) {
    d.pa = p.a;
    d.pb = p.a;
    d.ea = 0;
    d.eb = 0;
    if (it.t >= hi || it.kT == 0) {
      d.va = make_vsharp(p.a, 0); d.vb = d.va; d.vas = d.va; d.vbs = d.va;
      return;
    }
    const int64_t n0 = (int64_t)it.nt * kBN;
    const int64_t m0w = (int64_t)it.mt * kBM;
    int64_t a_base_off, b_base_off;
    uint32_t a_range, b_range;
    const uint8_t* bbase;
    if constexpr (kAMN) {            // bf16 wgrad: A^T = token-major rows [tok][M]
      a_base_off = it.koff * p.lda + m0w * 2; a_range = (uint32_t)max((int64_t)0, it.Me * p.lda - m0w * 2);
    } else if constexpr (kWg) {      // MXFP8 wgrad: A^T quantized [M][Rpad], segment at koff
      a_base_off = m0w * p.lda + it.koff; a_range = (uint32_t)(it.mrows * p.lda - it.koff);
    } else {
      a_base_off = (int64_t)it.row0 * p.lda; a_range = (uint32_t)(it.mrows * p.lda);
    }
    if constexpr (kBMN) {
      if constexpr (kWg) {           // bf16 wgrad: token-major rows [tok][N]
        bbase = p.b; b_base_off = it.koff * p.ldb + n0 * 2; b_range = (uint32_t)max((int64_t)0, it.Me * p.ldb - n0 * 2);
      } else {                       // bf16 dgrad: W_e [K][N]
        bbase = bwd_table(it.e); b_base_off = n0 * 2; b_range = (uint32_t)(p.K * p.ldb - n0 * 2);
      }
    } else if constexpr (kWg) {      // MXFP8 wgrad: B^T quantized [N][Rpad]
      bbase = p.b; b_base_off = n0 * p.ldb + it.koff; b_range = (uint32_t)(it.ncols * p.ldb - it.koff);
    } else {                         // MXFP8 dgrad: W^T quantized [N][K] per expert
      bbase = p.b + (int64_t)it.e * p.b_stride; b_base_off = n0 * p.ldb; b_range = (uint32_t)(it.ncols * p.ldb);
    }
    if constexpr (kWg && !kMx) {
      d.pa = p.a + a_base_off;
      d.ea = max((int64_t)0, it.Me * p.lda - m0w * 2);
      d.pb = bbase + b_base_off;
      d.eb = max((int64_t)0, it.Me * p.ldb - n0 * 2);
      a_range = 0;
      b_range = 0;
    }
    d.va = make_vsharp(p.a + a_base_off, a_range);
    d.vb = make_vsharp(bbase + b_base_off, b_range);
    if constexpr (kMx) {
      if constexpr (kWg) {
        // ranges end at the scale arrays' ends: a group of scale bytes read past the last segment
        // (padding scales up to rows_pad) reads zeros beyond it
        // based at the 16-byte group holding the segment's first scale bytes (the deep pipeline's
        // groups are the layout's own)
        const int64_t s0 = kDeep ? it.koff / 32 - 4 * it.gs : it.koff / 32;
        d.vas = make_vsharp(p.as + m0w * p.ldas + s0, (uint32_t)(it.mrows * p.ldas - s0));
        d.vbs = make_vsharp(p.bs + n0 * p.ldbs + s0, (uint32_t)(it.ncols * p.ldbs - s0));
      } else {
        d.vas = make_vsharp(p.as + (int64_t)it.row0 * p.ldas, (uint32_t)(it.mrows * p.ldas));
        d.vbs = make_vsharp(p.bs + (int64_t)it.e * p.bs_stride + n0 * p.ldbs, (uint32_t)(it.ncols * p.ldbs));
      }
    } else {
      d.vas = d.va;
      d.vbs = d.vb;
    }
  };

  uint32_t a_vo[8], b_vo[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    // K-major slot mapping
    const int j = (wave * 8 + q) * 4 + (lane >> 4);
    const uint32_t hs = (uint32_t)((j & 7) | ((j & 4) << 1));
    const uint32_t sl = (uint32_t)(lane & 15) ^ hs;
    const int rk = 2 * j + (int)(sl >> 3);
    const uint32_t ck = sl & 7u;
    // MN-major slot mapping
    const int rm = 2 * (wave * 8 + q) + (lane >> 5);
    const uint32_t cm = (uint32_t)(lane & 31) ^ (((uint32_t)rm & 3u) << 2);
    a_vo[q] = kAMN ? (uint32_t)(rm * p.lda) + cm * 16 : (uint32_t)(rk * p.lda) + ck * 16;
    b_vo[q] = kBMN ? (uint32_t)(rm * p.ldb) + cm * 16 : (uint32_t)(rk * p.ldb) + ck * 16;
  }
  // per-stage advance of the offsets: K-major along the row (128 bytes), MN-major 64 rows down
  const uint32_t a_step = kAMN ? (uint32_t)(64 * p.lda) : (uint32_t)kRowBytes;
  const uint32_t b_step = kBMN ? (uint32_t)(64 * p.ldb) : (uint32_t)kRowBytes;
  uint32_t as_vo = 0, bs_vo = 0;
  uint32_t as4[1] = {0}, bs4[1] = {0};   // deep: scale group offsets
  if constexpr (kMx) {
    const int r = wave * 64 + lane;
    as_vo = (uint32_t)(r * p.ldas);
    bs_vo = (uint32_t)(r * p.ldbs);
    // group loads: row r's 16 bytes at r * 16 of the buffer
    as4[0] = (uint32_t)(r * p.ldas);
    bs4[0] = (uint32_t)(r * p.ldbs);
  }
  const i32x4 zdesc = make_vsharp(p.a, 0);   // zero range: loads read no memory and deliver zeros
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)(wave * 8) * 1024u);
  const uint32_t lds_sc = __builtin_amdgcn_readfirstlane(lds_addr(smem + kScOff) + (uint32_t)wave * (kDeep ? 1024u : 256u));
  // BF16 wgrad: descriptors of stage kt, based at its first token row (64 rows per stage), the
  // range clipped to the segment's end (and to 32 bits)
  auto stage_vs = [&](const uint8_t* base, int64_t ext, int kt, int64_t ld) -> i32x4 {
    const int64_t o = (int64_t)kt * 64 * ld;
    const int64_t r = ext - o;
    return make_vsharp(base + o, (uint32_t)(r <= 0 ? 0 : (r > (int64_t)0xFFFFFFFF ? (int64_t)0xFFFFFFFF : r)));
  };
  i32x4 sva = zdesc, svb = zdesc;
  // q runs 0..7 in order within a stage (unrolled), so the stage's descriptors are formed at q == 0
  auto dma_a = [&](const Desc& d, int b, int kt, int q, bool on = true) {
    if constexpr (kWg && !kMx) {
      if (q == 0) sva = stage_vs(d.pa, d.ea, kt, p.lda);
      dma16(sva, lds0 + (uint32_t)b * (uint32_t)kStageBytes + q * 1024u, a_vo[q], 0);
    } else {
      dma16(on ? d.va : zdesc, lds0 + (uint32_t)b * (uint32_t)kStageBytes + q * 1024u,
            a_vo[q] + (uint32_t)kt * a_step, 0);
    }
  };
  auto dma_b = [&](const Desc& d, int b, int kt, int q, bool on = true) {
    if constexpr (kWg && !kMx) {
      if (q == 0) svb = stage_vs(d.pb, d.eb, kt, p.ldb);
      dma16(svb, lds0 + (uint32_t)b * (uint32_t)kStageBytes + kTileBytes + q * 1024u, b_vo[q], 0);
    } else {
      dma16(on ? d.vb : zdesc, lds0 + (uint32_t)b * (uint32_t)kStageBytes + kTileBytes + q * 1024u,
            b_vo[q] + (uint32_t)kt * b_step, 0);
    }
  };
  auto dma_s = [&](const Desc& d, int b, int kt) {
    if constexpr (kMx && !kDeep) {
      const uint32_t ss = lds_sc + (uint32_t)b * 2048u;
      dma4(d.vas, ss, as_vo + (uint32_t)kt * 4u, 0);
      dma4(d.vbs, ss + 1024u, bs_vo + (uint32_t)kt * 4u, 0);
    }
  };
  // deep pipeline: the scales of stage group g (stages 4 g .. 4 g + 3) into scale buffer sb, row r's
  // 16 bytes at r * 16 (A rows, then B rows at 4096); predicated by the descriptor (off: no memory
  // read, zeros written to the buffer, which no pending stage uses)
  auto dma_sg = [&](const Desc& d, bool on, int sb, int g) {
    if constexpr (kDeep) {
      const uint32_t ss = lds_sc + (uint32_t)sb * (uint32_t)kScBuf;
      dma16(on ? d.vas : zdesc, ss, as4[0], (uint32_t)g * 16u);
      dma16(on ? d.vbs : zdesc, ss + 4096u, bs4[0], (uint32_t)g * 16u);
    }
  };

  BwdItem cur, nxt;
  Desc dc, dn;
  decode(0, cur);
  descs(cur, dc);
  int par = 0;             // buffer of the current item's first stage
  bool issued = false;     // the current item's first stage was loaded by the previous item
  int sbc = 0, sbn = 0;    // deep pipeline: scale buffers of the current and the next stage
  if constexpr (kDeep) {
    // the first item's first two stages (every item has at least two)
    if (cur.t < hi) {
      const bool on0 = cur.u0 < cur.kz, on1 = cur.u0 + 1 < cur.kz;
#pragma unroll
      for (int q = 0; q < 8; ++q) { dma_a(dc, 0, cur.u0, q, on0); dma_b(dc, 0, cur.u0, q, on0); }
      dma_sg(dc, true, 0, (cur.u0 + cur.gs) >> 2);
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) { dma_a(dc, 1, cur.u0 + 1, q, on1); dma_b(dc, 1, cur.u0 + 1, q, on1); }
      const bool ng = ((cur.u0 + 1 + cur.gs) & 3) == 0;
      sbn = ng ? 1 : 0;
      dma_sg(dc, ng, 1, (cur.u0 + 1 + cur.gs) >> 2);
    }
  }
  // diagnostic (p.tstat): shader-clock cycles of the main loops and of the epilogues of this wave
  const bool tst = p.tstat != nullptr;
  uint64_t tc_main = 0, tc_epi = 0, tc_t = 0;
  uint32_t n_items = 0;
  for (int round = 0; cur.t < hi; ++round) {
    if (tst) tc_t = __builtin_amdgcn_s_memtime();
    decode(round + 1, nxt);
    descs(nxt, dn);
    const int ipar = round & 1;
    if constexpr (kD2) {
      const float pr = tid < cur.mrows ? p.prob_perm[cur.row0 + tid] : 0.f;
      reinterpret_cast<float*>(smem + kXOff)[ipar * 256 + tid] = pr;
    }
    TileCore<kMx, false> core;
    core.zero();
    if constexpr (kDeep) {
      // as the forward's deep MXFP8 loop: stage s in buffer (par + s) & 1, the loads of the stage
      // after next (this item's, or the next item's first two) issued during stage s's second
      // substep into the buffer stage s just freed; a new scale group goes to the scale buffer
      // the next stage does not use
      const int n = cur.kT;
      StepFrag<true> f0;
      read_first<true, false, false, false, 16>(f0, smem + par * kStageBytes,
                                                smem + kScOff + sbc * kScBuf + ((cur.u0 + cur.gs) & 3) * 4, wm, wn,
                                                lane);
#pragma unroll 1
      for (int s = 0; s < n; ++s) {
        const int kt = cur.u0 + s, b = (par + s) & 1, bn = b ^ 1;
        const int kn = s + 1 < n ? kt + 1 : nxt.u0;
        const bool in2 = s + 2 < n;
        const Desc& dt = in2 ? dc : dn;
        const int k2 = in2 ? kt + 2 : nxt.u0 + (s + 2 - n);
        // stage positions within the 16-byte scale groups (shifted by each item's gs)
        const int gt = kt + cur.gs, gn = kn + (s + 1 < n ? cur.gs : nxt.gs), g2 = k2 + (in2 ? cur.gs : nxt.gs);
        const bool ng = (!in2 && s + 2 == n) || (g2 & 3) == 0;
        const int sbd = ng ? (sbn ^ 1) : sbn;
        const bool on = !kWg || k2 < (in2 ? cur.kz : nxt.kz);   // the stage holds data (wgrad)
        auto sync = [&]() {
          wait_vmcnt<0>();
          __syncthreads();
        };
        mma_stage_mx_deep<false>(core, f0, smem + b * kStageBytes, smem + kScOff + sbc * kScBuf + (gt & 3) * 4,
                                 smem + bn * kStageBytes, smem + kScOff + sbn * kScBuf + (gn & 3) * 4, wm, wn, lane,
                                 [&](int q) { dma_a(dt, b, k2, q, on); }, [&](int q) { dma_b(dt, b, k2, q, on); },
                                 [&]() { dma_sg(dt, ng, sbn ^ 1, g2 >> 2); }, sync);
        sbc = sbn;
        sbn = sbd;
      }
      par = (par + n) & 1;
    } else {
    if (!issued && cur.kT > 0) {
#pragma unroll
      for (int q = 0; q < 8; ++q) { dma_a(dc, par, cur.u0, q); dma_b(dc, par, cur.u0, q); }
      dma_s(dc, par, cur.u0);
    }
    // the last stage loads the next item's first one, if it has any stage
    const bool chain = nxt.t < hi && nxt.kT > 0;
#pragma unroll 1
    for (int s = 0; s < cur.kT; ++s) {
      const int b = (par + s) & 1;
      // stage s landed (own loads + barrier); every wave finished reading the other buffer, which
      // takes the next stage while this one is multiplied
      wait_vmcnt<0>();
      __syncthreads();
      const bool last = s + 1 == cur.kT;
      const Desc& dd = last ? dn : dc;
      const int kn = last ? nxt.u0 : cur.u0 + s + 1;
      const int bn = b ^ 1;
      const uint8_t* sA = smem + b * kStageBytes;
      const uint8_t* sS = smem + kScOff + b * 2048;
      mma_stage<kMx, false, kAMN, kBMN, 4>(
          core, sA, sS, wm, wn, lane, [&](int q) { dma_a(dd, bn, kn, q); }, [&](int q) { dma_b(dd, bn, kn, q); },
          [&]() { dma_s(dd, bn, kn); });
    }
    issued = cur.kT > 0 && chain;
    par = (par + cur.kT) & 1;
    }

    if (tst) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
      tc_main += t - tc_t;
      tc_t = t;
    }
    // ---- epilogue straight from the accumulators: acc[i][j][4 q + c] of lane l is output row
    // wm*128 + 32 i + l % 32 of the tile and column wn*128 + 32 j + 8 q + 4 (l / 32) + c.  Loads and
    // stores go through buffer descriptors that end at the tile's last valid row.
    int elane = lane;
    asm volatile("" : "+v"(elane));
    const int r32 = elane & 31, ch = (elane >> 5) * 4;
    const int64_t n0 = (int64_t)cur.nt * kBN;
    if constexpr (kD2) {
      // ScaledSwiGLU backward per element (dh = this tile, g / u = the saved gate-up output,
      // p = the routing probability of the row):
      //   dG = dh p u s (1 + g (1 - s)), dU = dh p g s, s = sigmoid(g); dprob partial = sum dh g s u.
      // The saved g / u of the next 32 x 32 block are loaded while this one is computed.  Each lane
      // first trades half of its accumulator runs with lane l ^ 32 (v_permlane32_swap), so that it
      // holds 8 consecutive columns 16 pp + 8 hh + [0, 8) (pp < 2, hh = l / 32) of its row: g / u are
      // then read and dG / dU written 16 bytes per lane, half the accesses of the accumulators'
      // 8-byte runs, with 32 contiguous bytes per row per access.
      const int64_t I = p.I;
      const uint32_t I32 = (uint32_t)I;
      const float* prs = reinterpret_cast<const float*>(smem + kXOff) + ipar * 256;
      float* red = reinterpret_cast<float*>(smem + kXOff + 2048);
      const uint32_t mr = (uint32_t)cur.mrows;
      const rsrc_t rgu = make_rsrc(p.gu + (int64_t)cur.row0 * 2 * I, mr * I32 * 4);
      const rsrc_t rdg = make_rsrc(p.dgu + (int64_t)cur.row0 * 2 * I, mr * I32 * 4);
      const int hh = elane >> 5;
      u32x4 gl[2][2], ul[2][2];                      // [buffer][pp]: 8 bf16 each
      auto boff = [&](int blk, int pp) -> uint32_t {  // byte offset of the lane's 8 gate columns
        const int i = blk >> 2, j = blk & 3;
        const uint32_t m = (uint32_t)(wm * 128 + i * 32 + r32);
        return (2 * m * I32 + (uint32_t)n0 + (uint32_t)(wn * 128 + j * 32 + 16 * pp + 8 * hh)) * 2u;
      };
      auto load = [&](int blk, int bf) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint32_t o = boff(blk, pp);
          gl[bf][pp] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rgu, o, 0, 0));
          ul[bf][pp] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rgu, o + I32 * 2u, 0, 0));
        }
      };
      // MXFP8: dGU quantized here, from its bf16 values (the operand the unfused path would quantize),
      // by the OCP rule of the row-wise quantizer:
      //   * along 2I (FC1 dgrad's K): a row's 32-column block lies in lanes l and l ^ 32, 16
      //     values each -- codes go out 8 bytes per run, the scale byte from the lane holding the
      //     block's first columns;
      //   * along the expert's tokens (FC1 wgrad's K), into the transposed layout whose segments
      //     are padded to 128 tokens: the wave writes the bf16 block to its LDS slot row by row and
      //     reads it back with transposing reads, lane l getting column l % 32 at rows
      //     16 (l / 32) + [0, 16); the column's 32-row block lies in lanes l and l ^ 32.  Blocks
      //     past the segment's padded end are left alone (they belong to the next segment); rows
      //     past the expert's tokens inside it are zero.
      [[maybe_unused]] const uint32_t I2 = 2u * I32;
      // (the row-wise outputs' descriptors end at the tile's last row; null-based with no range in BF16)
      [[maybe_unused]] const rsrc_t rq = make_rsrc(kQ ? p.dgu_q + (int64_t)cur.row0 * 2 * I : nullptr, kQ ? mr * I2 : 0u);
      [[maybe_unused]] const rsrc_t rqs =
          make_rsrc(kQ ? p.dgu_s + (int64_t)cur.row0 * (2 * I / 32) : nullptr, kQ ? mr * (I2 / 32) : 0u);
      // one 32-column block of dG (half 0) or dU (half 1): w0 / w1 its runs pp = 0 / 1.  The scale
      // bytes are collected into words, so that they leave as 4-byte stores: a row's bytes of the
      // wave's 4 column blocks (rword, byte j), and a column's bytes of the wave's 4 row blocks
      // (cword, byte i) -- both 4-byte aligned, as I % 128 == 0 and segments start at multiples of 128.
      // Along 2I (quant_rows): codes and scale from the lane's runs.  The codes of run pp (8 bytes,
      // columns 16 pp + 8 hh) are traded with lane l ^ 32 (v_permlane32_swap) so that the lane holds
      // the block row's 16-byte chunk hh; the 4 blocks of a row block then leave through the LDS
      // slot as whole 128-byte rows per half (stage_rows32), instead of 16-byte pieces of 32 rows.
      auto quant_rows = [&](const u32x4 w0, const u32x4 w1, int j, uint32_t& rword, u32x4& chunk) {
        // the bf16 values stay packed: amax on the bit patterns, codes by the scaled conversion
        const uint32_t wv[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
        const int sx = mx_shared_exp(max_xor32(bf16_amax<8>(wv)));
        const uint32_t c0[2] = {mx_pack4_bf16(w0[0], w0[1], sx), mx_pack4_bf16(w0[2], w0[3], sx)};
        const uint32_t c1[2] = {mx_pack4_bf16(w1[0], w1[1], sx), mx_pack4_bf16(w1[2], w1[3], sx)};
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const auto sw = __builtin_amdgcn_permlane32_swap(c0[k], c1[k], false, false);
          chunk[k] = sw[0];
          chunk[2 + k] = sw[1];
        }
        rword |= (uint32_t)(sx + 127) << (8 * j);
      };
      // Along the tokens: the block goes through the wave's 2 KB slot (row r at r * 64 bytes) and
      // comes back by transposing reads (tcols_read), which the row-wise work of both halves then
      // hides; tcols_quant encodes lane l's column l % 32, rows 16 (l / 32) + [0, 16).  The LDS unit
      // runs one wave's operations in issue order, so the second half's writes to the slot cannot
      // overtake the first half's reads.
      const uint32_t trd = (uint32_t)(16 * ((elane >> 4) >> 1) + (elane & 15) / 4) * 64u +
                           (uint32_t)(16 * ((elane >> 4) & 1) + 4 * (elane & 3)) * 2u;
      auto tcols_read = [&](const u32x4 w0, const u32x4 w1, uint32_t (&tw)[8]) {
        uint8_t* lt = smem + kTOff + wave * 2048;
        *reinterpret_cast<u32x4*>(lt + r32 * 64 + (8 * (elane >> 5)) * 2) = w0;
        *reinterpret_cast<u32x4*>(lt + r32 * 64 + (16 + 8 * (elane >> 5)) * 2) = w1;
        asm volatile("" ::: "memory");
        typedef __attribute__((address_space(3))) bf16x4_t lds_v4;
        const auto base = (__attribute__((address_space(3))) uint8_t*)(lt);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(base + trd + q * 256u));
          const u32x2 rw = __builtin_bit_cast(u32x2, r);
          tw[2 * q] = rw[0];
          tw[2 * q + 1] = rw[1];
        }
        asm volatile("" ::: "memory");
      };
      auto tcols_quant = [&](const uint32_t (&tw)[8], int half, int i, int j, uint32_t& cword) {
        const int srel = cur.mt * kBM + wm * 128 + i * 32;                   // block's first segment row
        const uint32_t colg = (half ? I32 : 0u) + (uint32_t)n0 + (uint32_t)(wn * 128 + j * 32);
        const int st = mx_shared_exp(max_xor32(bf16_amax<8>(tw)));
        const u32x4 c{mx_pack4_bf16(tw[0], tw[1], st), mx_pack4_bf16(tw[2], tw[3], st),
                      mx_pack4_bf16(tw[4], tw[5], st), mx_pack4_bf16(tw[6], tw[7], st)};
        // through descriptors over the block's 32 transposed rows: a split_sizes array that does
        // not match rows_pad cannot take the stores outside the buffers
        const uint32_t rp = (uint32_t)p.rows_pad, prow = (uint32_t)(cur.poff + srel);
        const rsrc_t rt = make_rsrc(p.dgu_tq + (int64_t)colg * p.rows_pad, 32u * rp);
        __builtin_amdgcn_raw_buffer_store_b128(c, rt, (uint32_t)(elane & 31) * rp + prow + 16u * (uint32_t)(elane >> 5), 0, 0);
        cword |= (uint32_t)(st + 127) << (8 * i);
      };
      [[maybe_unused]] uint32_t rsw[2] = {0u, 0u};                    // row scale words (current i)
      [[maybe_unused]] u32x4 rcode[2][4];                             // row codes (current i), by half, j
      [[maybe_unused]] uint32_t csw[4][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}, {0u, 0u}};   // column ones, by j
      // BF16: dG (then dU) of the two column blocks j, j + 1 of a row block, staged row by row in the
      // wave's slot (16-byte chunk c of row r at chunk c ^ (r & 7): conflict-free reads, 2-way
      // writes) and stored 8 whole 128-byte rows per instruction -- the direct stores wrote 32-byte
      // pieces of 32 rows each, and their partial lines cost the write path several times their
      // bytes.  e / o: the even / odd block's runs pp = 0, 1; colbyte: the pair's first column in the
      // dGU row, in bytes.
      [[maybe_unused]] auto flush_pair = [&](const u32x4 (&e)[2], const u32x4 (&o)[2], uint32_t colbyte, int i) {
        uint8_t* sl = smem + kSOff + wave * 4096;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            const uint32_t c = (uint32_t)(jj * 4 + 2 * pp + (elane >> 5));
            *reinterpret_cast<u32x4*>(sl + r32 * 128 + ((c ^ (uint32_t)(r32 & 7)) << 4)) = jj ? o[pp] : e[pp];
          }
        // the LDS unit runs one wave's operations in issue order: the reads below see these writes,
        // and the next pair's writes cannot overtake them, so no counter wait is needed -- the
        // empty asm only keeps the compiler from moving LDS accesses across it
        asm volatile("" ::: "memory");
        u32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 8 * q + (elane >> 3), ch = elane & 7;
          v[q] = *reinterpret_cast<const u32x4*>(sl + row * 128 + ((ch ^ (row & 7)) << 4));
        }
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t m = (uint32_t)(wm * 128 + i * 32 + 8 * q + (elane >> 3));
          __builtin_amdgcn_raw_buffer_store_b128(v[q], rdg, 2u * m * I32 * 2u + colbyte + (uint32_t)(elane & 7) * 16u, 0, 0);
        }
      };
      [[maybe_unused]] u32x4 gk[2], uk[2];   // BF16: the even block's dG, dU, kept for its pair
      float part[4] = {0.f, 0.f, 0.f, 0.f};
      load(0, 0);
#pragma unroll
      for (int blk = 0; blk < 16; ++blk) {
        const int i = blk >> 2, j = blk & 3, bf = blk & 1;
        if (blk + 1 < 16) load(blk + 1, bf ^ 1);
        const bool cv = n0 + wn * 128 + j * 32 < I;                 // wave-uniform
        if (cv) {
          const float pr = prs[wm * 128 + i * 32 + r32];
          float dh[16];
          agpr_read16(core.acc[i][j], dh);
          // dh[4 q + c] is column 8 q + 4 hh + c; after the swaps dh[8 pp + x] is column 16 pp + 8 hh + x
#pragma unroll
          for (int pp = 0; pp < 2; ++pp)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, dh[8 * pp + c]),
                                                              __builtin_bit_cast(uint32_t, dh[8 * pp + 4 + c]), false, false);
              dh[8 * pp + c] = __builtin_bit_cast(float, (uint32_t)r[0]);
              dh[8 * pp + 4 + c] = __builtin_bit_cast(float, (uint32_t)r[1]);
            }
          u32x4 gb[2], ub[2];   // dG, dU in bf16: 8 consecutive columns 16 pp + 8 hh + [0, 8) each
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            float dgv[8], duv[8];
#pragma unroll
            for (int x = 0; x < 8; ++x) {
              const uint32_t gw = gl[bf][pp][x >> 1], uw = ul[bf][pp][x >> 1];
              const float g = bf16_to_f32((uint16_t)((x & 1) ? (gw >> 16) : (gw & 0xFFFF)));
              const float uu = bf16_to_f32((uint16_t)((x & 1) ? (uw >> 16) : (uw & 0xFFFF)));
              const float d = dh[8 * pp + x];
              const float sg = sigmoid_f(g);
              const float sl = g * sg;
              part[i] += d * (sl * uu);
              const float da = d * pr;
              duv[x] = da * sl;
              dgv[x] = da * uu * (sg * (1.0f + g * (1.0f - sg)));
            }
            gb[pp] = u32x4{pack_bf16x2(dgv[0], dgv[1]), pack_bf16x2(dgv[2], dgv[3]), pack_bf16x2(dgv[4], dgv[5]),
                           pack_bf16x2(dgv[6], dgv[7])};
            ub[pp] = u32x4{pack_bf16x2(duv[0], duv[1]), pack_bf16x2(duv[2], duv[3]), pack_bf16x2(duv[4], duv[5]),
                           pack_bf16x2(duv[6], duv[7])};
            if (kQ && p.dgu) {   // MXFP8 debug output: the bf16 dGU, stored directly
              const uint32_t o = boff(blk, pp);
              __builtin_amdgcn_raw_buffer_store_b128(gb[pp], rdg, o, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b128(ub[pp], rdg, o + I32 * 2u, 0, 0);
            }
          }
          if constexpr (kStage) {
            if ((j & 1) == 0) {
              gk[0] = gb[0]; gk[1] = gb[1]; uk[0] = ub[0]; uk[1] = ub[1];
            } else {
              const uint32_t c0 = (uint32_t)n0 + (uint32_t)(wn * 128 + (j - 1) * 32);   // the pair's first column
              flush_pair(gk, gb, c0 * 2u, i);
              flush_pair(uk, ub, (I32 + c0) * 2u, i);
            }
          }
          if constexpr (kQ) {
            // blocks past the segment's padded end get no token-axis codes (they belong to the next
            // segment); rows past the expert's tokens inside it are zero
            const int srel = cur.mt * kBM + wm * 128 + i * 32;
            if (srel < (cur.Me + 127) / 128 * 128) {                    // wave-uniform
              uint32_t twg[8], twu[8];
              tcols_read(gb[0], gb[1], twg);
              quant_rows(gb[0], gb[1], j, rsw[0], rcode[0][j]);
              tcols_read(ub[0], ub[1], twu);
              quant_rows(ub[0], ub[1], j, rsw[1], rcode[1][j]);
              tcols_quant(twg, 0, i, j, csw[j][0]);
              tcols_quant(twu, 1, i, j, csw[j][1]);
            } else {
              quant_rows(gb[0], gb[1], j, rsw[0], rcode[0][j]);
              quant_rows(ub[0], ub[1], j, rsw[1], rcode[1][j]);
            }
            if (j == 3) {
              // the row block's codes of the wave's 4 column blocks (128 bytes per row and half), and
              // the rows' scale words, dG then dU (I % 128 == 0: the 4 blocks are all valid)
              const uint32_t m = (uint32_t)(wm * 128 + i * 32 + r32);
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                uint32_t lo[8], hi[8];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  lo[k] = rcode[half][0][k];
                  lo[4 + k] = rcode[half][1][k];
                  hi[k] = rcode[half][2][k];
                  hi[4 + k] = rcode[half][3][k];
                }
                u32x4 v[4];
                stage_rows32(smem + kTOff + wave * 2048, lo, hi, elane, v);
                const uint32_t c0 = (half ? I32 : 0u) + (uint32_t)n0 + (uint32_t)(wn * 128);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                  const uint32_t mm = (uint32_t)(wm * 128 + i * 32 + 8 * t + (elane >> 3));
                  __builtin_amdgcn_raw_buffer_store_b128(v[t], rq, mm * I2 + c0 + ((uint32_t)elane & 7u) * 16u, 0, 0);
                }
                const uint32_t so = (elane >> 5) == 0 ? m * (I2 / 32) + c0 / 32 : 0xFFFFFFF0u;
                __builtin_amdgcn_raw_buffer_store_b32(rsw[half], rqs, so, 0, 0);
                rsw[half] = 0;
              }
            }
          }
        }
      }
      if constexpr (kQ) {
        // a column's scale words of the wave's 4 row blocks: the wave's 128 rows lie wholly inside
        // the expert's 128-padded segment or wholly past it
        const int srel = cur.mt * kBM + wm * 128;
        if (srel < (cur.Me + 127) / 128 * 128) {
          const uint32_t rp = (uint32_t)p.rows_pad, prow = (uint32_t)(cur.poff + srel);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (n0 + wn * 128 + j * 32 >= I) continue;   // wave-uniform
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const uint32_t colg = (half ? I32 : 0u) + (uint32_t)n0 + (uint32_t)(wn * 128 + j * 32);
              const rsrc_t rts = make_rsrc(p.dgu_ts + (int64_t)colg * (p.rows_pad / 32), 32u * (rp / 32));
              const uint32_t tso = (elane >> 5) == 0 ? (uint32_t)(elane & 31) * (rp / 32) + prow / 32 : 0xFFFFFFF0u;
              __builtin_amdgcn_raw_buffer_store_b32(csw[j][half], rts, tso, 0, 0);
            }
          }
        }
      }
      // per-row partial over the tile's 256 columns: the lane pair (l, l ^ 32) holds a row's 128
      // columns of this wave, the two waves of a row block the two halves -- fixed-order sums
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = part[i] + __shfl_xor(part[i], 32, 64);
        if (ch == 0) red[wn * 256 + wm * 128 + i * 32 + r32] = s;
      }
      __syncthreads();
      if (tid < cur.mrows) p.dprob_part[(int64_t)(cur.row0 + tid) * p.nN + cur.nt] = red[tid] + red[256 + tid];
    } else {
      // FC1 dgrad: dx_perm rows of the tile (a split part: its whole fp32 tile, row-major
      // [256][256], to its slot of p.part); wgrad: rows m0w.. of dW_e
      const bool sp = kOutF32 && cur.part >= 0;
      const uint32_t N32 = sp ? 256u : (uint32_t)p.N;
      const uint32_t es = kOutF32 ? 4u : 2u;
      const int64_t r0 = kWg ? (int64_t)cur.mt * kBM : (int64_t)cur.row0;
      uint8_t* obase = kWg ? const_cast<uint8_t*>(bwd_table(cur.e)) : p.out;
      const rsrc_t ro = sp ? make_rsrc(p.part + (size_t)(cur.t - full) * 65536, 65536u * 4u)
                           : make_rsrc(obase + r0 * p.N * es, (uint32_t)cur.mrows * N32 * es);
      const int64_t cbase = sp ? 0 : n0;                             // tile's first column in the destination
      // A row of a 32 x 32 fp32 block, or of a pair of bf16 blocks j = 2 jp, 2 jp + 1, is 128 bytes,
      // which lanes l and l + 32 hold as 16-byte chunks 2 q + l / 32: it goes through the wave's
      // LDS slot (stage_rows32) and out 8 whole rows per store, each unit's stores issued after the
      // next unit's LDS round trip.  A unit past N (a ragged last N tile; N is a multiple of 64)
      // gets offsets past the descriptor's range, so its stores are dropped.  Weight gradients are
      // written once and never re-read here: non-temporal stores.
      constexpr int kStoreAux = kWg ? 2 : 0;
      constexpr int kUnits = kOutF32 ? 16 : 8;
      uint8_t* sl = smem + kFOff + wave * 2048;
      u32x4 pend[4];               // the previous unit's rows 8 t + l / 8, t < 4
      uint32_t pend_off = 0;
#pragma unroll
      for (int u = 0; u < kUnits; ++u) {
        const int i = kOutF32 ? u >> 2 : u >> 1;
        const int j0 = kOutF32 ? (u & 3) : 2 * (u & 1);   // the unit's first block
        uint32_t lo[8], hi[8];
        if constexpr (kOutF32) {
          float a[16];
          agpr_read16(core.acc[i][j0], a);
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            lo[k] = __builtin_bit_cast(uint32_t, a[k]);
            hi[k] = __builtin_bit_cast(uint32_t, a[8 + k]);
          }
        } else {
          float a0[16], a1[16];
          agpr_read16(core.acc[i][j0], a0);
          agpr_read16(core.acc[i][j0 + 1], a1);
          u32x4 e[2], o[2];   // the lane-paired bf16 runs: chunks 2 pp + l / 32 of each block's 64 bytes
          pack_bf16_runs8(a0, e);
          pack_bf16_runs8(a1, o);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            lo[k] = e[0][k];
            lo[4 + k] = e[1][k];
            hi[k] = o[0][k];
            hi[4 + k] = o[1][k];
          }
        }
        u32x4 v[4];
        stage_rows32(sl, lo, hi, elane, v);
        if (u > 0) {
#pragma unroll
          for (int t = 0; t < 4; ++t) __builtin_amdgcn_raw_buffer_store_b128(pend[t], ro, pend_off + t * 8u * N32 * es, 0, kStoreAux);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) pend[t] = v[t];
        const uint32_t tc = (uint32_t)(wn * 128 + j0 * 32);            // column of the unit within the tile
        const bool ok = (uint32_t)n0 + tc < (uint32_t)p.N;
        pend_off = ok ? ((uint32_t)(wm * 128 + i * 32 + (elane >> 3)) * N32 + (uint32_t)cbase + tc) * es + ((uint32_t)elane & 7u) * 16u
                      : 0x80000000u;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) __builtin_amdgcn_raw_buffer_store_b128(pend[t], ro, pend_off + t * 8u * N32 * es, 0, kStoreAux);
    }
    if (tst) {
      tc_epi += __builtin_amdgcn_s_memtime() - tc_t;
      ++n_items;
    }
    cur = nxt;
    dc = dn;
  }
  wait_vmcnt<0>();
  if (tst && lane == 0 && !(kRole == kRoleDgradFc1 && p.split == 2)) {   // (split parts: the main pass's)
    uint32_t* o = p.tstat + ((size_t)blockIdx.x * 4 + wave) * kTileStatWords;
    o[0] = (uint32_t)tc_main;
    o[1] = (uint32_t)tc_epi;
    o[2] = n_items;
    o[3] = kTileStatTag;
  }
}

template <int kRole, bool kMx>
hipError_t launch_role(const BwdKArgs& k, bool out_f32, hipStream_t st) {
  // MXFP8 wgrad, and MXFP8 dgrad whose scale rows are whole 16-byte groups (K % 512 == 0, so at
  // least four stages of 128 values): the deep pipeline; other K keep the loop with one scale word
  // per row per stage
  if constexpr (kMx) {
    if (kRole == kRoleWgrad || k.K % 512 == 0) {
      if (out_f32) bwd_gemm_kernel<kRole, kMx, true, true><<<kGemmGrid, 256, 0, st>>>(k);
      else bwd_gemm_kernel<kRole, kMx, false, true><<<kGemmGrid, 256, 0, st>>>(k);
      return hipGetLastError();
    }
  }
  if (out_f32) bwd_gemm_kernel<kRole, kMx, true><<<kGemmGrid, 256, 0, st>>>(k);
  else bwd_gemm_kernel<kRole, kMx, false><<<kGemmGrid, 256, 0, st>>>(k);
  return hipGetLastError();
}

BwdKArgs base_args(const BwdGemm& g) {
  BwdKArgs k{};
  k.a = reinterpret_cast<const uint8_t*>(g.a);
  k.lda = g.lda;
  k.as = g.a_scales;
  k.ldas = g.ldas;
  k.b = reinterpret_cast<const uint8_t*>(g.b);
  k.ldb = g.ldb;
  k.b_stride = g.b_stride;
  k.bs = g.b_scales;
  k.ldbs = g.ldbs;
  k.bs_stride = g.bs_stride;
  k.M = g.M;
  k.N = g.N;
  k.K = g.K;
  k.E = g.E;
  k.nM = (int)((g.M + kBM - 1) / kBM);
  k.nN = (int)((g.N + kBN - 1) / kBN);
  k.pad = g.pad;
  k.split_sizes = g.split_sizes;
  k.gu = g.gu;
  k.prob_perm = g.prob_perm;
  k.dgu = g.dgu;
  k.dgu_q = g.dgu_q;
  k.dgu_s = g.dgu_s;
  k.dgu_tq = g.dgu_tq;
  k.dgu_ts = g.dgu_ts;
  k.rows_pad = g.rows_pad;
  k.dprob_part = g.dprob_part;
  k.I = g.I;
  k.out = reinterpret_cast<uint8_t*>(g.out);
  k.tstat = g.tstat;
  if (g.tab)
    for (int e = 0; e < g.E; ++e) k.tab[e] = reinterpret_cast<const uint8_t*>(g.tab[e]);
  return k;
}

}  // namespace

hipError_t launch_bwd_dgrad_fc2(const BwdGemm& g, bool mx, hipStream_t st) {
  BwdKArgs k = base_args(g);
  return mx ? launch_role<kRoleDgradFc2, true>(k, false, st) : launch_role<kRoleDgradFc2, false>(k, false, st);
}

hipError_t launch_bwd_dgrad_fc1(const BwdGemm& g, bool mx, hipStream_t st) {
  BwdKArgs k = base_args(g);
  // a split needs at least 2 parts of kMinSplitUnits K units each
  const int kU = (int)(g.K * (mx ? 1 : 2) / kRowBytes);
  const bool split = g.part != nullptr && kU / kMinSplitUnits >= 2;
  k.part = g.part;
  k.split = split ? 1 : 0;
  hipError_t err = mx ? launch_role<kRoleDgradFc1, true>(k, g.out_f32, st) : launch_role<kRoleDgradFc1, false>(k, g.out_f32, st);
  if (err != hipSuccess || !split) return err;
  // pass 2: the split parts (whether there are any is decided on the device), then the fixup
  k.split = 2;
  err = mx ? launch_role<kRoleDgradFc1, true>(k, true, st) : launch_role<kRoleDgradFc1, false>(k, true, st);
  if (err != hipSuccess) return err;
  return launch_split_fixup(g.split_sizes, g.E, g.N, g.part, g.out, g.out_f32, kU, st);
}

hipError_t launch_bwd_wgrad(const BwdGemm& g, bool mx, hipStream_t st) {
  BwdKArgs k = base_args(g);
  return mx ? launch_role<kRoleWgrad, true>(k, g.out_f32, st) : launch_role<kRoleWgrad, false>(k, g.out_f32, st);
}

int bwd_dprob_parts(int64_t I) { return (int)((I + kBN - 1) / kBN); }

namespace {
// Row r's scale bytes from the end of the last 128-padded segment to ld: zero.  Every workgroup
// recomputes that end from split_sizes.
__global__ __launch_bounds__(256) void scale_tail_zero_kernel(uint8_t* __restrict__ scales, int64_t rows, int64_t ld,
                                                              const int32_t* __restrict__ split_sizes, int E) {
  __shared__ int s_end;
  if (threadIdx.x == 0) {
    int64_t pt = 0;
    for (int e = 0; e < E; ++e) pt += ((int64_t)max(split_sizes[e], 0) + 127) / 128 * 128;
    s_end = (int)min(pt / 32, ld);
  }
  __syncthreads();
  const int64_t b0 = s_end, n = ld - b0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t c = threadIdx.x; c < n; c += 256) scales[r * ld + b0 + c] = 0;
}
}  // namespace

hipError_t launch_scale_tail_zero(uint8_t* scales, int64_t rows, int64_t ld, const int32_t* split_sizes, int E,
                                  hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const unsigned g = (unsigned)(rows < 4096 ? rows : 4096);
  scale_tail_zero_kernel<<<g, 256, 0, st>>>(scales, rows, ld, split_sizes, E);
  return hipGetLastError();
}

}  // namespace moe
