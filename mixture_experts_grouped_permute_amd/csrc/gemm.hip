// Persistent grouped GEMMs for gfx950: BF16 (v_mfma_f32_32x32x16_bf16) and
// MXFP8 (v_mfma_scale_f32_32x32x64_f8f6f4 with E8M0 block scales).
//
// All local experts run in one launch (page "BioNeMo Uses Grouped Kernels and
// MXFP8", Grouping fragmented expert workloads: the grouped linear submits
// every expert's GEMM together, each expert keeping its own weights, with
// split_sizes giving the uneven token counts).  The FC1 epilogue applies
// ScaledSwiGLU with the routing probability and writes h straight in the FC2
// operand format, so the 2I-wide gate-up result is never stored (Fusing
// precision conversion and expert computation, Figure 4).
//
// Structure
//   * 256 threads = 4 waves in a 2x2 grid; a workgroup owns a 256 x 256 output
//     tile (FC1: 128 h columns = 128 gate + 128 up weight rows); each wave a
//     128 x 128 block = 4 x 4 MFMA 32x32 blocks accumulated in fp32.  The weight
//     block is the MFMA's first operand, so a lane ends up holding one token row
//     and runs of 4 consecutive output columns, and the epilogues store straight
//     from the accumulators (no LDS staging).
//   * K is consumed in 128-byte steps (64 bf16 or 128 E4M3 values per row),
//     double-buffered in LDS (2 x 64 KB) in the swz layout, filled by
//     direct-to-LDS buffer loads.  Inside a stage the next stage's loads and the
//     next substep's fragment reads are interleaved one by one between the MFMAs,
//     so the wave's in-order issue never stalls behind a burst of memory
//     instructions; the last stage of a tile loads the first stage of the
//     workgroup's next tile, which lands while the epilogue runs.
//   * Global reads are buffer loads whose range is the expert's valid rows,
//     so ragged tiles read zeros instead of neighbouring experts' data; the
//     epilogue's buffer stores end at the tile's last valid row the same way.
//   * Scheduler: every workgroup recomputes the per-expert tile prefix sum
//     from split_sizes in LDS (no host sync), then walks tiles in rounds of
//     gridDim.x.  Tile order is expert, N-panel, M-block (M fastest) and a
//     round hands each XCD (workgroup id mod 8) a contiguous slice, so the
//     M-blocks that share one weight panel run together on one L2.
#include "gemm_core.h"

namespace moe {
namespace {
using namespace gemm;

// Kernel arguments: scalars plus the per-expert weight pointer table inline.
struct FwdKArgs {
  const uint8_t* a;
  const uint8_t* a_scales;
  const uint8_t* wq;
  const uint8_t* ws;
  int64_t wq_stride, ws_stride;
  int64_t K, N;
  int E, nN;
  const int32_t* split_sizes;
  const float* prob_perm;
  uint8_t* out;
  uint8_t* out_scales;
  uint16_t* save_gu;
  uint16_t* save_h;
  int out_f32;
  float* part;               // split tiles' fp32 partial accumulators, kGemmGrid x 64K floats
  int split;                 // 0: every tile; 1: tiles before the split ones; 2: the split parts
  const float* pt_s_a;       // per-tensor FP8: per expert scale s of the A rows and of the weight
  const float* pt_s_b;
  uint32_t* pt_amax_out;     // per-tensor FP8, FC1: per expert max |bf16 h| (float bits, atomic max)
  float* h_f32;              // FC1: h in fp32 as the epilogue computes it, before rounding, or null
  uint32_t* tstat;           // per-wave cycle counts (diagnostic), or null
  const uint8_t* w[kMaxExperts];
};

// Reads w[e] straight from the kernel-argument segment (a uniform scalar load)
// instead of letting the compiler copy the by-value table to private memory.
__device__ __forceinline__ const uint8_t* kernarg_table(int e) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint8_t* const* tab = reinterpret_cast<const uint8_t* const*>(
      reinterpret_cast<const char*>(__builtin_amdgcn_kernarg_segment_ptr()) + offsetof(FwdKArgs, w));
  return tab[e];
#else
  (void)e;
  return nullptr;
#endif
}

// One work item: a 256 x 256 output tile, or one K part of a split tile.
struct FwdItem {
  int t, tile, part, e, mt, nt, row0, mrows, u0, u1;
};

// kDeep (K of at least two stages): the stage barrier sits inside the stage and stage loads are
// issued two stages ahead (mma_stage_mx_deep, mma_stage_bf16_deep).  MXFP8 scale rows of a whole
// number of 16-byte groups (K % 512 == 0) load a group with one 16-byte load per row; kSc4 (MXFP8
// deep with other K, e.g. the 44-byte rows of K = 1408) takes the four-lane word form instead, fixed
// at compile time because no branch may sit among the MFMAs.
// kPt (with kMx): per-tensor-scaled FP8 -- unit block scales, the per-expert dequantization in
// the epilogue, and FC1's h written as bf16 (a separate instance, so the MXFP8 epilogue keeps
// its own code)
template <bool kMx, bool kFc1, bool kOutF32, bool kDeep, bool kPt = false, bool kSc4 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_gemm_kernel(const FwdKArgs p) {
  // 2 pipeline stages, then the MXFP8 scales of groups of 4 stages (2 x 8 KB), then the routing
  // probabilities of the tile's rows (FC1, double-buffered by work item)
  constexpr int kScOff = 2 * kStageBytes;
  constexpr int kScBuf = 8192;
  constexpr int kPrOff = kScOff + (kMx ? 2 * kScBuf : 0);
  // a 2 KB slot per wave for the epilogue's full-line stores
  constexpr int kFOff = kPrOff + (kFc1 ? 2 * 1024 : 16);
  __shared__ __attribute__((aligned(16))) uint8_t smem[kFOff + 4 * 2048];
  __shared__ Sched sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = p.E;
  build_sched(sched, p.split_sizes, E, p.nN);
  const int total = __builtin_amdgcn_readfirstlane(sched.tile[E]);
  const int G = gridDim.x, per = G >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int64_t K = p.K, N = p.N;
  const int esz = kMx ? 1 : 2;
  const uint32_t rowb = (uint32_t)(K * esz);           // bytes per operand row
  const uint32_t kscale_row = (uint32_t)(K / 32);      // scale bytes per row
  const int kU = (int)(rowb / 128);                    // K units of 128 bytes

  // Load balance of the last round: with `total` tiles over G workgroups, the last round holds
  // rem = total % G tiles and would leave G - rem workgroups idle for a whole tile.  FC2 splits
  // each of those rem tiles into S parts along K (S = G / rem, at least kMinSplitUnits K units
  // per part): pass 1 runs tiles [0, full), pass 2 (the fp32-output instance) runs the rem * S
  // parts and writes their fp32 tiles to p.part, and fc2_fixup_kernel sums the S partials of
  // each tile in part order -- deterministic -- into the output.  split = 0: all tiles, one pass.
  int full = total, S = 1;
  if (p.split) split_policy(total, G, kU, full, S);
  const int lo = p.split == 2 ? full : 0;
  const int hi = p.split == 0 ? total : (p.split == 1 ? full : (S > 1 ? full + (total - full) * S : full));

  // Work item of round r of this workgroup (uniform; valid iff it.t < hi).
  auto decode = [&](int round, FwdItem& it) {
    it.t = lo + round * G + xcd * per + slot;
    it.u0 = 0;
    if (it.t >= hi) return;
    it.tile = it.t;
    it.part = -1;
    if (kOutF32 && p.split == 2) {
      it.tile = full + (it.t - full) / S;
      it.part = (it.t - full) % S;
    }
    it.e = __builtin_amdgcn_readfirstlane(find_expert(sched, E, it.tile));
    const int Me = __builtin_amdgcn_readfirstlane(sched.cnt[it.e]);
    const int nM = (Me + kBM - 1) / kBM;
    const int local = it.tile - __builtin_amdgcn_readfirstlane(sched.tile[it.e]);
    tile_coords(local, nM, p.nN, it.mt, it.nt);
    it.row0 = __builtin_amdgcn_readfirstlane(sched.off[it.e]) + it.mt * kBM;
    it.mrows = min(kBM, Me - it.mt * kBM);
    it.u0 = it.part < 0 ? 0 : it.part * kU / S;
    it.u1 = it.part < 0 ? kU : (it.part + 1) * kU / S;
  };
  // Buffer descriptors of an item's operands: the A rows of its tile (zero past the expert's
  // rows), and the weight rows from the tile's first one.  FC1 B rows [0,128) of a tile are gate
  // rows n0h + r, rows [128,256) the up rows I + n0h + r; gate rows past I only feed masked
  // columns, up rows past 2I fall outside the range and read zero.  An invalid item gets
  // zero-range descriptors: its loads touch no memory.
  struct Desc { i32x4 va, vb, vas, vbs; };
  auto descs = [&](const FwdItem& it, Desc& d) {
    if (it.t >= hi) {
      d.va = make_vsharp(p.a, 0); d.vb = d.va; d.vas = d.va; d.vbs = d.va;
      return;
    }
    const int64_t b0 = kFc1 ? (int64_t)it.nt * 128 : (int64_t)it.nt * kBN;        // first weight row
    const int64_t brows = kFc1 ? 2 * N - b0 : min((int64_t)kBN, N - b0);
    const uint8_t* wbase = kMx ? (p.wq + (int64_t)it.e * p.wq_stride) : kernarg_table(it.e);
    d.va = make_vsharp(p.a + (int64_t)it.row0 * rowb, (uint32_t)it.mrows * rowb);
    d.vb = make_vsharp(wbase + b0 * rowb, (uint32_t)(brows * rowb));
    if constexpr (kMx) {
      const uint8_t* sbase = p.ws + (int64_t)it.e * p.ws_stride;
      d.vas = make_vsharp(p.a_scales + (int64_t)it.row0 * kscale_row, (uint32_t)it.mrows * kscale_row);
      d.vbs = make_vsharp(sbase + b0 * kscale_row, (uint32_t)(brows * kscale_row));
    } else {
      d.vas = d.va;
      d.vbs = d.vb;
    }
  };

  // Direct-to-LDS loads (buffer_load_dwordx4 ... lds), one 16-byte chunk per lane, each load
  // filling a contiguous 1 KB of LDS: load q of wave w fills row pairs j = 4 (8w + q) + L / 16,
  // lane L's 16-byte LDS slot s = L % 16 holding (row parity, chunk) = s ^ hs(j), so the
  // stage lands in the swz layout.  Whole 128-byte rows per load keep every L2 request a full
  // line.  MXFP8 adds one 4-byte load per operand per stage: the E8M0 scales of the stage's four
  // 32-value blocks of row 64 w + L.  The voffsets are the same for every tile.
  uint32_t a_vo[8], b_vo[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int j = (wave * 8 + q) * 4 + (lane >> 4);
    const uint32_t hs = (uint32_t)((j & 7) | ((j & 4) << 1));
    const uint32_t sl = (uint32_t)(lane & 15) ^ hs;
    const int r = 2 * j + (int)(sl >> 3);
    const uint32_t c = sl & 7u;
    const int64_t br = kFc1 ? (r < 128 ? (int64_t)r : N + (r - 128)) : (int64_t)r;
    a_vo[q] = (uint32_t)r * rowb + c * 16;
    b_vo[q] = (uint32_t)(br * rowb) + c * 16;
  }
  // MXFP8 scales, loaded a group of 4 stages at a time: 16 bytes of E8M0 per row (stage kt's 4
  // bytes at (kt & 3) * 4), row r's 16 bytes at r * 16 of the buffer (A rows, then B rows at 4096).
  //   * 16-byte scale rows (K % 512 == 0): one 16-byte load per row, lane L of wave w fetching row
  //     64 w + L (direct-to-LDS loads of 4 bytes cost about as much issue time each as one of 16).
  //   * otherwise (the scale rows of K = 1408 are 44 bytes): four lanes per row, reading its
  //     consecutive words, which the load merges into one request; load j < 4 of wave w covers
  //     rows 64 w + 16 j + L / 4, lane L's word landing at slot L of a 256-byte block.
  const bool sc16 = kDeep ? !kSc4 : (kscale_row & 15u) == 0;
  uint32_t as_vo[4] = {0, 0, 0, 0}, bs_vo[4] = {0, 0, 0, 0};
  if constexpr (kMx) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = sc16 ? wave * 64 + lane : wave * 64 + j * 16 + (lane >> 2);
      const int64_t br = kFc1 ? (r < 128 ? (int64_t)r : N + (r - 128)) : (int64_t)r;
      const uint32_t w4 = sc16 ? 0u : (uint32_t)(lane & 3) * 4u;
      as_vo[j] = (uint32_t)r * kscale_row + w4;
      bs_vo[j] = (uint32_t)(br * kscale_row) + w4;
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (uint32_t)(wave * 8) * 1024u);
  const uint32_t lds_sc = __builtin_amdgcn_readfirstlane(lds_addr(smem + kScOff) + (uint32_t)wave * 1024u);
  // stage kt of the item described by d into buffer b
  auto dma_a = [&](const Desc& d, int b, int kt, int q) {
    dma16(d.va, lds0 + (uint32_t)b * (uint32_t)kStageBytes + q * 1024u, a_vo[q], (uint32_t)kt * kRowBytes);
  };
  auto dma_b = [&](const Desc& d, int b, int kt, int q) {
    dma16(d.vb, lds0 + (uint32_t)b * (uint32_t)kStageBytes + kTileBytes + q * 1024u, b_vo[q], (uint32_t)kt * kRowBytes);
  };
  // the scales of stage group g (stages 4 g .. 4 g + 3) of the item described by d into buffer sb
  // (called at a stage's top, outside its MFMAs, except in the deep pipeline, where the form is
  // fixed at compile time: no branch may sit among the MFMAs)
  auto dma_s = [&](const Desc& d, int sb, int g) {
    if constexpr (kMx) {
      const uint32_t ss = lds_sc + (uint32_t)sb * (uint32_t)kScBuf;
      if (sc16) {
        dma16(d.vas, ss, as_vo[0], (uint32_t)g * 16u);
        dma16(d.vbs, ss + 4096u, bs_vo[0], (uint32_t)g * 16u);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dma4(d.vas, ss + (uint32_t)j * 256u, as_vo[j], (uint32_t)g * 16u);
          dma4(d.vbs, ss + 4096u + (uint32_t)j * 256u, bs_vo[j], (uint32_t)g * 16u);
        }
      }
    }
  };

  // the scale group load of the deep pipeline, predicated by its descriptor: off, it reads no memory
  // but still writes (zeros) to its LDS buffer, so it always targets the buffer that no pending
  // stage uses
  auto dma_s_pred = [&](const Desc& d, bool on, int sb, int g) {
    if constexpr (kMx) {
      const i32x4 z = make_vsharp(p.a, 0);
      Desc e;
      e.vas = on ? d.vas : z;
      e.vbs = on ? d.vbs : z;
      dma_s(e, sb, g);
    }
  };

  FwdItem cur, nxt;
  Desc dc, dn;
  decode(0, cur);
  descs(cur, dc);
  int par = 0;    // buffer of the current item's first stage
  int spar = 0;   // scale buffer of the current item's first stage group
  int sbc = 0, sbn = 0;   // deep pipeline: scale buffers of the current and the next stage
  if (cur.t < hi) {
#pragma unroll
    for (int q = 0; q < 8; ++q) { dma_a(dc, 0, cur.u0, q); dma_b(dc, 0, cur.u0, q); }
    dma_s(dc, 0, cur.u0 >> 2);
    if constexpr (kDeep) {
      // the first stage landed before the loop; the second (every item has at least two) follows
      wait_vmcnt<0>();
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 8; ++q) { dma_a(dc, 1, cur.u0 + 1, q); dma_b(dc, 1, cur.u0 + 1, q); }
      const bool ng = ((cur.u0 + 1) & 3) == 0;
      sbn = ng ? 1 : 0;
      dma_s_pred(dc, ng, 1, (cur.u0 + 1) >> 2);
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
    const int ipar = round & 1;                          // probability buffer of this item
    if constexpr (kFc1) {
      const float pr = tid < cur.mrows ? p.prob_perm[cur.row0 + tid] : 0.f;
      reinterpret_cast<float*>(smem + kPrOff)[ipar * 256 + tid] = pr;
    }
    TileCore<kMx, kFc1> core;
    core.zero();
    const int n = cur.u1 - cur.u0;
    // scale groups: the item's are g0 .. glast, group g in buffer (spar + g - g0) & 1.  The first
    // stage of the item and the first stage of each later group load the next group -- after the
    // last group, the next item's first one -- into the buffer of the group before the current one,
    // which every wave finished reading before this stage's barrier.
    const int g0 = cur.u0 >> 2, glast = (cur.u1 - 1) >> 2;
    if constexpr (kDeep) {
      // the item's first stage landed before the barrier of the previous stage (or the prologue's)
      StepFrag<kMx> f0;
      read_first<kMx, kFc1, false, false, 16>(f0, smem + par * kStageBytes,
                                              smem + kScOff + sbc * kScBuf + (cur.u0 & 3) * 4, wm, wn, lane);
#pragma unroll 1
      for (int s = 0; s < n; ++s) {
        const int kt = cur.u0 + s, b = (par + s) & 1, bn = b ^ 1;
        const int kn = s + 1 < n ? kt + 1 : nxt.u0;           // the next stage
        const bool in2 = s + 2 < n;                           // the stage after next: this item's or the next's
        const Desc& dt = in2 ? dc : dn;
        const int k2 = in2 ? kt + 2 : nxt.u0 + (s + 2 - n);
        // a new scale group goes to the buffer the next stage does not use: it holds this stage's
        // group (read before the barrier) or an older one
        const bool ng = (!in2 && s + 2 == n) || (k2 & 3) == 0;  // it starts a scale group
        const int sbd = ng ? (sbn ^ 1) : sbn;
        auto sync = [&]() {
          wait_vmcnt<0>();
          __syncthreads();
        };
        if constexpr (kMx)
          mma_stage_mx_deep<kFc1>(
              core, f0, smem + b * kStageBytes, smem + kScOff + sbc * kScBuf + (kt & 3) * 4, smem + bn * kStageBytes,
              smem + kScOff + sbn * kScBuf + (kn & 3) * 4, wm, wn, lane, [&](int q) { dma_a(dt, b, k2, q); },
              [&](int q) { dma_b(dt, b, k2, q); }, [&]() { dma_s_pred(dt, ng, sbn ^ 1, k2 >> 2); }, sync);
        else
          mma_stage_bf16_deep<kFc1>(core, f0, smem + b * kStageBytes, smem + bn * kStageBytes, wm, wn, lane,
                                    [&](int q) { dma_a(dt, b, k2, q); }, [&](int q) { dma_b(dt, b, k2, q); }, sync);
        sbc = sbn;
        sbn = sbd;
      }
    } else {
#pragma unroll 1
    for (int s = 0; s < n; ++s) {
      const int kt = cur.u0 + s, b = (par + s) & 1;
      const int g = kt >> 2;
      // stage kt landed (own loads + barrier); every wave finished reading the other buffer, which
      // takes the next stage -- of this item, or the first of the next item -- while this one is
      // multiplied
      wait_vmcnt<0>();
      __syncthreads();
      const bool last = s + 1 == n;
      const Desc& dd = last ? dn : dc;
      const int kn = last ? nxt.u0 : kt + 1;
      const int bn = b ^ 1;
      const uint8_t* sA = smem + b * kStageBytes;
      const uint8_t* sS = smem + kScOff + ((spar + g - g0) & 1) * kScBuf + (kt & 3) * 4;
      // the scale group load is issued here, ahead of the stage's fragment reads: a branch among
      // the MFMAs would split the block and make the compiler re-extend every scale byte read
      // before it, waiting for all of them at once
      if (kMx && (s == 0 || (kt & 3) == 0)) {
        const bool snext = g == glast;                   // the next item's first group
        dma_s(snext ? dn : dc, (spar + g - g0 + 1) & 1, snext ? nxt.u0 >> 2 : g + 1);
      }
      mma_stage<kMx, kFc1, false, false, 16>(
          core, sA, sS, wm, wn, lane, [&](int q) { dma_a(dd, bn, kn, q); }, [&](int q) { dma_b(dd, bn, kn, q); },
          []() {});
    }
    }
    par = (par + n) & 1;
    spar = (spar + glast - g0 + 1) & 1;

    if (tst) {
      const uint64_t t = __builtin_amdgcn_s_memtime();
      tc_main += t - tc_t;
      tc_t = t;
    }
    // ---- epilogue straight from the accumulators.  acc[i][j][4 q + c] of lane l is token row
    // wm*128 + 32 i + l % 32 of the tile and output column (weight block j) + 8 q + 4 (l / 32) + c.
    // Stores go through buffer descriptors that end at the tile's last row, so the rows of a
    // ragged tile past the expert's tokens are dropped by the range check instead of by a branch.
    // The lane id is laundered so the address arithmetic is redone per tile instead of being
    // hoisted above the main loop, and each 32 x 32 block is finished before the next one is
    // started, so only its accumulators are copied out of the AGPRs at a time.
    int elane = lane;
    asm volatile("" : "+v"(elane));
    const int r32 = elane & 31, ch = (elane >> 5) * 4;
    if constexpr (kFc1) {
      const int64_t I = N;
      const uint32_t I32 = (uint32_t)I;
      const float* prs = reinterpret_cast<const float*>(smem + kPrOff) + ipar * 256;
      const uint32_t mr = (uint32_t)cur.mrows;
      const int64_t r0 = cur.row0;
      const rsrc_t ro = kMx ? make_rsrc(p.out + r0 * I, mr * I32) : make_rsrc(p.out + r0 * I * 2, mr * I32 * 2);
      const rsrc_t rsc = make_rsrc(kMx ? p.out_scales + r0 * (I / 32) : p.out, kMx ? mr * (I32 / 32) : 0);
      const rsrc_t rh = make_rsrc(p.save_h ? p.save_h + r0 * I : nullptr, p.save_h ? mr * I32 * 2 : 0);
      const rsrc_t rg = make_rsrc(p.save_gu ? p.save_gu + r0 * 2 * I : nullptr, p.save_gu ? mr * I32 * 4 : 0);
      const rsrc_t rf = make_rsrc(p.h_f32 ? p.h_f32 + r0 * I : nullptr, p.h_f32 ? mr * I32 * 4 : 0);
      // per-tensor FP8: the products of unit-scaled codes times 1 / (s_a s_b) of the tile's
      // expert, and h leaves as bf16 (its scale needs the amax of the expert's whole h)
      constexpr bool pt = kMx && kPt;
      const float dq = pt ? (1.0f / p.pt_s_a[cur.e]) * (1.0f / p.pt_s_b[cur.e]) : 1.0f;
      float hmax = 0.f;   // per-tensor FP8: the largest |h| of the wave's blocks (rows past the tile's
                          // end are zero: zero A rows and probability)
      // bf16 outputs (h, the saved g / u, the saved h): the wave's two 32-column blocks of a row
      // block make 128 bytes per row, which leave through the wave's LDS slot as whole rows
      // (stage_rows32) once the second block is done; kept[.] holds the first block's runs
      uint8_t* sl = smem + kFOff + wave * 2048;
      const uint32_t cw = (uint32_t)cur.nt * 128u + (uint32_t)(wn * 64);   // the wave's first h column
      auto stage_pair = [&](const u32x4 (&e)[2], const u32x4 (&o)[2], const rsrc_t& rs, uint32_t row_bytes,
                            uint32_t col_byte, int i) {
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          lo[k] = e[0][k];
          lo[4 + k] = e[1][k];
          hi[k] = o[0][k];
          hi[4 + k] = o[1][k];
        }
        u32x4 v[4];
        stage_rows32(sl, lo, hi, elane, v);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t mm = (uint32_t)(wm * 128 + i * 32 + 8 * t + (elane >> 3));
          __builtin_amdgcn_raw_buffer_store_b128(v[t], rs, mm * row_bytes + col_byte + ((uint32_t)elane & 7u) * 16u, 0, 0);
        }
      };
      u32x4 kg[2], ku[2], kh[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 128 + i * 32 + r32;
        const float pr = prs[m];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const uint32_t col = cw + (uint32_t)(jj * 32);                                     // h column of the block
          if (cw >= I32) continue;                 // wave-uniform; I % 64 == 0: both blocks or neither
          float g[16], u[16];
          agpr_read16(core.acc[i][jj], g);
          agpr_read16(core.acc[i][jj + 2], u);
          if constexpr (pt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) { g[r] *= dq; u[r] *= dq; }
          }
          // the lane-paired layout (pack_bf16_runs8 / swap_runs8): the lane's 8 consecutive columns
          // 16 pp + 8 hh + [0, 8) of the block
          const uint32_t e8 = (uint32_t)m * I32 + col + 2u * (uint32_t)ch;                  // element of h
          if (p.save_gu) {
            u32x4 og[2], ou[2];
            pack_bf16_runs8(g, og);
            pack_bf16_runs8(u, ou);
            if (jj == 0) {
              kg[0] = og[0]; kg[1] = og[1]; ku[0] = ou[0]; ku[1] = ou[1];
            } else {
              stage_pair(kg, og, rg, I32 * 4u, cw * 2u, i);
              stage_pair(ku, ou, rg, I32 * 4u, (I32 + cw) * 2u, i);
            }
          }
          float v[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) v[r] = (silu_f(g[r]) * u[r]) * pr;
          if (p.h_f32) {
            // the fp32 h ahead of its rounding: runs of 4 columns 8 q + ch of the block
            const uint32_t e4 = (uint32_t)m * I32 + col + (uint32_t)ch;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              __builtin_amdgcn_raw_buffer_store_b128(f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]}, rf,
                                                     (e4 + 8u * q) * 4u, 0, 0);
          }
          if constexpr (pt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) hmax = fmaxf(hmax, fabsf(v[r]));
          }
          if (!kMx || pt || p.save_h) {
            u32x4 oh[2];
            pack_bf16_runs8(v, oh);
            if (jj == 0) {
              kh[0] = oh[0]; kh[1] = oh[1];
            } else {
              stage_pair(kh, oh, kMx ? rh : ro, I32 * 2u, cw * 2u, i);
            }
          }
          if constexpr (kMx && !pt) {
            // the 32-column block of this row is split between lanes l and l ^ 32
            float am = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(v[r]));
            am = max_xor32(am);
            const int sx = mx_shared_exp(am);
            uint32_t cq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) cq[q] = mx_pack4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], sx);
            u32x2 oc[2];
            swap_runs8(cq, oc);
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) __builtin_amdgcn_raw_buffer_store_b64(oc[pp], ro, e8 + 16u * pp, 0, 0);
            // one scale byte per row and block, from the lane holding its first columns
            const uint32_t so = ch == 0 ? (uint32_t)m * (I32 / 32) + col / 32 : 0xFFFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(sx + 127), rsc, so, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (pt) {
        // the wave's largest |h| rounded to bf16 (rounding is monotone, so this is the largest
        // stored value) raises the expert's amax for the quantization of h
        float hm = hmax;
#pragma unroll
        for (int mk = 32; mk >= 1; mk >>= 1) hm = fmaxf(hm, __shfl_xor(hm, mk, 64));
        hm = bf16_to_f32(f32_to_bf16(hm));
        if (lane == 0) atomicMax(p.pt_amax_out + cur.e, __builtin_bit_cast(uint32_t, hm));
      }
    } else {
      const uint32_t N32 = (uint32_t)N;
      const uint32_t esz_o = kOutF32 ? 4u : 2u;
      rsrc_t ro;
      uint32_t ld;                                   // row pitch in elements
      if (kOutF32 && cur.part >= 0) {
        // a split part stores its whole fp32 tile, row-major [256][256], to its slot of p.part;
        // fc2_fixup_kernel sums the parts
        ro = make_rsrc(p.part + (size_t)(cur.t - full) * 65536, 65536u * 4u);
        ld = 256;
      } else {
        ro = make_rsrc(p.out + (int64_t)cur.row0 * N * esz_o, (uint32_t)cur.mrows * N32 * esz_o);
        ld = N32;
      }
      // first column of the tile in the destination (0 for a part slot)
      const uint32_t c0 = (kOutF32 && cur.part >= 0) ? 0u : (uint32_t)cur.nt * kBN;
      const float dq = (kMx && kPt) ? (1.0f / p.pt_s_a[cur.e]) * (1.0f / p.pt_s_b[cur.e]) : 1.0f;
      // A row of a 32 x 32 fp32 block, or of a pair of bf16 blocks j = 2 jp, 2 jp + 1, is 128 bytes,
      // which lanes l and l + 32 hold as 16-byte chunks 2 q + l / 32: it goes through the wave's
      // LDS slot (stage_rows32) and out 8 whole rows per store, each unit's stores issued after the
      // next unit's LDS round trip.  A unit past N (a ragged last N tile; N is a multiple of 64)
      // gets offsets past the descriptor's range, so its stores are dropped.
      constexpr uint32_t kEsz = kOutF32 ? 4u : 2u;
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
            lo[k] = __builtin_bit_cast(uint32_t, a[k] * dq);
            hi[k] = __builtin_bit_cast(uint32_t, a[8 + k] * dq);
          }
        } else {
          float a0[16], a1[16];
          agpr_read16(core.acc[i][j0], a0);
          agpr_read16(core.acc[i][j0 + 1], a1);
          if constexpr (kMx && kPt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) { a0[r] *= dq; a1[r] *= dq; }
          }
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
          for (int t = 0; t < 4; ++t) __builtin_amdgcn_raw_buffer_store_b128(pend[t], ro, pend_off + t * 8u * ld * kEsz, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) pend[t] = v[t];
        const uint32_t tc = (uint32_t)(wn * 128 + j0 * 32);            // column of the unit within the tile
        const bool ok = (uint32_t)cur.nt * kBN + tc < N32;
        pend_off = ok ? ((uint32_t)(wm * 128 + i * 32 + (elane >> 3)) * ld + c0 + tc) * kEsz + ((uint32_t)elane & 7u) * 16u
                      : 0x80000000u;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) __builtin_amdgcn_raw_buffer_store_b128(pend[t], ro, pend_off + t * 8u * ld * kEsz, 0, 0);
    }
    if (tst) {
      tc_epi += __builtin_amdgcn_s_memtime() - tc_t;
      ++n_items;
    }
    cur = nxt;
    dc = dn;
  }
  wait_vmcnt<0>();
  if (tst && lane == 0 && p.split != 2) {   // (a split-parts pass leaves the main pass's counts)
    uint32_t* o = p.tstat + ((size_t)blockIdx.x * 4 + wave) * kTileStatWords;
    o[0] = (uint32_t)tc_main;
    o[1] = (uint32_t)tc_epi;
    o[2] = n_items;
    o[3] = kTileStatTag;
  }
}

// Finishes the split tiles of an FC2 launch: the S row-major [256][256] fp32 partials of tile
// full + blockIdx.x are summed in part order and stored to z (bf16 or fp32).  Thread tid owns
// 8 consecutive columns of rows 32 blockIdx.y + tid / 32 + 8 q.
template <bool kOutF32>
__global__ __launch_bounds__(256) void fc2_fixup_kernel(const FwdKArgs p, int kU) {
  __shared__ Sched sched;
  const int E = p.E;
  build_sched(sched, p.split_sizes, E, p.nN);
  const int total = sched.tile[E];
  int full, S;
  split_policy(total, gridDim.x, kU, full, S);
  const int b = blockIdx.x;
  if (S < 2 || full + b >= total) return;
  const int tile = full + b;
  const int e = find_expert(sched, E, tile);
  const int Me = sched.cnt[e];
  const int nM = (Me + kBM - 1) / kBM;
  const int local = tile - sched.tile[e];
  int mt, nt;
  tile_coords(local, nM, p.nN, mt, nt);
  const int row0 = sched.off[e] + mt * kBM;
  const int mrows = min(kBM, Me - mt * kBM);
  const int64_t N = p.N, n0 = (int64_t)nt * kBN;
  const int c = (threadIdx.x & 31) * 8;
  const float* src = p.part + (size_t)b * S * 65536;
  // blockIdx.y takes rows [32 y, 32 y + 32) of the tile
  const int mend = min(mrows, (int)(blockIdx.y + 1) * 32);
  for (int m = blockIdx.y * 32 + (threadIdx.x >> 5); m < mend; m += 8) {
    if (n0 + c >= N) continue;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < S; ++q) {
      const f32x4* s4 = reinterpret_cast<const f32x4*>(src + (size_t)q * 65536 + m * 256 + c);
      const f32x4 x0 = s4[0], x1 = s4[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += x0[i];
        acc[4 + i] += x1[i];
      }
    }
    const int64_t o = (int64_t)(row0 + m) * N + n0 + c;
    if (kOutF32) {
      f32x4* d = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + o);
      d[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      d[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
    } else {
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + o) =
          u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
                pack_bf16x2(acc[6], acc[7])};
    }
  }
}

FwdKArgs make_fwd_args(const FwdGemm& g, bool mx, bool fc1) {
  FwdKArgs k{};
  k.a = reinterpret_cast<const uint8_t*>(g.a);
  k.a_scales = g.a_scales;
  k.wq = g.wq;
  k.ws = g.ws;
  k.wq_stride = g.wq_stride;
  k.ws_stride = g.ws_stride;
  k.K = g.K;
  k.N = g.N;
  k.E = g.E;
  k.nN = (int)(fc1 ? (g.N + 127) / 128 : (g.N + kBN - 1) / kBN);
  k.split_sizes = g.split_sizes;
  k.prob_perm = g.prob_perm;
  k.out = reinterpret_cast<uint8_t*>(g.out);
  k.out_scales = g.out_scales;
  k.save_gu = g.save_gu;
  k.save_h = g.save_h;
  k.out_f32 = g.out_f32 ? 1 : 0;
  k.pt_s_a = g.pt_s_a;
  k.pt_s_b = g.pt_s_b;
  k.pt_amax_out = g.pt_amax_out;
  k.h_f32 = g.h_f32;
  k.tstat = g.tstat;
  if (!mx)
    for (int e = 0; e < g.E; ++e) k.w[e] = reinterpret_cast<const uint8_t*>(g.w_tab[e]);
  return k;
}

}  // namespace

hipError_t launch_fc1(const FwdGemm& g, bool mx, hipStream_t st) {
  FwdKArgs k = make_fwd_args(g, mx, true);
  const bool pt = mx && g.pt_s_a != nullptr;
  if (pt && g.K >= 256 && g.K % 512 == 0) fwd_gemm_kernel<true, true, false, true, true><<<kGemmGrid, 256, 0, st>>>(k);
  else if (pt) fwd_gemm_kernel<true, true, false, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  else if (mx && g.K >= 256 && g.K % 512 == 0) fwd_gemm_kernel<true, true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  else if (mx && g.K >= 256) fwd_gemm_kernel<true, true, false, true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  else if (mx) fwd_gemm_kernel<true, true, false, false><<<kGemmGrid, 256, 0, st>>>(k);
  else if (g.K >= 128) fwd_gemm_kernel<false, true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  else fwd_gemm_kernel<false, true, false, false><<<kGemmGrid, 256, 0, st>>>(k);
  return hipGetLastError();
}

hipError_t launch_fc2(const FwdGemm& g, bool mx, hipStream_t st) {
  FwdKArgs k = make_fwd_args(g, mx, false);
  k.part = g.part;
  // a split needs at least 2 parts of kMinSplitUnits K units each
  const int kU = (int)(g.K * (mx ? 1 : 2) / 128);
  const bool split = g.part != nullptr && kU / kMinSplitUnits >= 2;
  // pass 1 (or the only pass): the output-dtype instance
  k.split = split ? 1 : 0;
  // K of at least two 128-byte stages takes the deep pipeline (split parts have at least
  // kMinSplitUnits stages); MXFP8 scale rows that are not whole 16-byte groups take its kSc4 form
  const bool deep = mx ? g.K >= 256 : g.K >= 128;
  const bool sc4 = mx && g.K % 512 != 0;
  const bool pt = mx && g.pt_s_a != nullptr;
  // the per-tensor FP8 instances keep the deep pipeline to 16-byte scale rows
  const bool pdeep = deep && !sc4;
  auto launch = [&](bool out_f32) {
    if (pt) {
      if (out_f32 && pdeep) fwd_gemm_kernel<true, false, true, true, true><<<kGemmGrid, 256, 0, st>>>(k);
      else if (out_f32) fwd_gemm_kernel<true, false, true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
      else if (pdeep) fwd_gemm_kernel<true, false, false, true, true><<<kGemmGrid, 256, 0, st>>>(k);
      else fwd_gemm_kernel<true, false, false, false, true><<<kGemmGrid, 256, 0, st>>>(k);
    } else if (out_f32) {
      if (mx && deep && sc4) fwd_gemm_kernel<true, false, true, true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
      else if (mx && deep) fwd_gemm_kernel<true, false, true, true><<<kGemmGrid, 256, 0, st>>>(k);
      else if (mx) fwd_gemm_kernel<true, false, true, false><<<kGemmGrid, 256, 0, st>>>(k);
      else if (deep) fwd_gemm_kernel<false, false, true, true><<<kGemmGrid, 256, 0, st>>>(k);
      else fwd_gemm_kernel<false, false, true, false><<<kGemmGrid, 256, 0, st>>>(k);
    } else {
      if (mx && deep && sc4) fwd_gemm_kernel<true, false, false, true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
      else if (mx && deep) fwd_gemm_kernel<true, false, false, true><<<kGemmGrid, 256, 0, st>>>(k);
      else if (mx) fwd_gemm_kernel<true, false, false, false><<<kGemmGrid, 256, 0, st>>>(k);
      else if (deep) fwd_gemm_kernel<false, false, false, true><<<kGemmGrid, 256, 0, st>>>(k);
      else fwd_gemm_kernel<false, false, false, false><<<kGemmGrid, 256, 0, st>>>(k);
    }
    return hipGetLastError();
  };
  hipError_t err = launch(g.out_f32);
  if (err != hipSuccess || !split) return err;
  // pass 2: the split parts (whether there are any is decided on the device), then the fixup
  k.split = 2;
  err = launch(true);
  if (err != hipSuccess) return err;
  const dim3 fgrid(kGemmGrid, kBM / 32);
  if (g.out_f32) fc2_fixup_kernel<true><<<fgrid, 256, 0, st>>>(k, kU);
  else fc2_fixup_kernel<false><<<fgrid, 256, 0, st>>>(k, kU);
  return hipGetLastError();
}

hipError_t launch_split_fixup(const int32_t* split_sizes, int E, int64_t N, float* part, void* out, bool out_f32,
                              int kU, hipStream_t st) {
  FwdKArgs k{};
  k.split_sizes = split_sizes;
  k.E = E;
  k.N = N;
  k.nN = (int)((N + kBN - 1) / kBN);
  k.part = part;
  k.out = reinterpret_cast<uint8_t*>(out);
  const dim3 fgrid(kGemmGrid, kBM / 32);
  if (out_f32) fc2_fixup_kernel<true><<<fgrid, 256, 0, st>>>(k, kU);
  else fc2_fixup_kernel<false><<<fgrid, 256, 0, st>>>(k, kU);
  return hipGetLastError();
}

}  // namespace moe
