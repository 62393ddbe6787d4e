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
//     128 x 128 block = 4 x 4 MFMA 32x32 fragments accumulated in fp32.
//   * K is consumed in 128-byte steps (64 bf16 or 128 E4M3 values per row),
//     double-buffered in LDS (2 x 64 KB) with the 16-byte chunks of each row
//     XOR-swizzled by (row & 7) so both the row-wise stores and the MFMA
//     fragment reads are bank-conflict free.
//   * Global reads are buffer loads whose range is the expert's valid rows,
//     so ragged tiles read zeros instead of neighbouring experts' data.
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

// Split of the last round: tiles [full, total) are split into S parts along K (S = 1: none).
__device__ __forceinline__ void split_policy(int total, int G, int kU, int& full, int& S) {
  const int rem = total % G;
  full = total;
  S = 1;
  if (rem > 0) {
    const int sk = min(G / rem, kU / kMinSplitUnits);
    if (sk >= 2) {
      S = sk;
      full = total - rem;
    }
  }
}

template <bool kMx, bool kFc1, bool kOutF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_gemm_kernel(const FwdKArgs p) {
  // 2 pipeline stages (the epilogue reuses them), plus the MXFP8 scale words (2 x 2 KB)
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes + (kMx ? 2 * 2048 : 16)];
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

  for (int round = 0;; ++round) {
    const int t = lo + round * G + xcd * per + slot;
    if (t >= hi) break;
    int tile = t, part = -1;
    if (kOutF32 && p.split == 2) {
      tile = full + (t - full) / S;
      part = (t - full) % S;
    }
    // the tile decode is uniform across the workgroup; readfirstlane makes it scalar so the
    // buffer descriptors built from it live in SGPRs
    const int e = __builtin_amdgcn_readfirstlane(find_expert(sched, E, tile));
    const int Me = __builtin_amdgcn_readfirstlane(sched.cnt[e]);
    const int nM = (Me + kBM - 1) / kBM;
    const int local = tile - __builtin_amdgcn_readfirstlane(sched.tile[e]);
    const int mt = local % nM, nt = local / nM;
    const int row0 = __builtin_amdgcn_readfirstlane(sched.off[e]) + mt * kBM;   // first permuted row of the tile
    const int mrows = min(kBM, Me - mt * kBM);
    const uint8_t* wbase = kMx ? (p.wq + (int64_t)e * p.wq_stride) : kernarg_table(e);
    TileCore<kMx, kFc1> core;
    core.zero();
    {
      // K units [u0, u1) of this work item (all of K unless the tile is split)
      const int u0 = part < 0 ? 0 : part * kU / S;
      const int u1 = part < 0 ? kU : (part + 1) * kU / S;
      // ---- main loop: direct-to-LDS loads (buffer_load_dwordx4 ... lds), one 16-byte chunk per
      // lane, each load filling a contiguous 1 KB of LDS.
      // FC1 B rows [0,128) are gate rows n0h + r, rows [128,256) up rows I + n0h + r: gate rows
      // past I only feed masked columns, up rows past 2I fall outside the range and read zero.
      auto b_row = [&](int r) -> int64_t {
        return kFc1 ? (r < 128 ? ((int64_t)nt * 128 + r) : (N + (int64_t)nt * 128 + (r - 128))) : (int64_t)r;
      };
      const i32x4 va = make_vsharp(p.a + (int64_t)row0 * rowb, (uint32_t)mrows * rowb);
      const i32x4 vb = kFc1 ? make_vsharp(wbase, (uint32_t)(2 * N * rowb))
                            : make_vsharp(wbase + (int64_t)nt * kBN * rowb,
                                          (uint32_t)(min((int64_t)kBN, N - (int64_t)nt * kBN) * rowb));
      {
        // Two 64 KB stages of 128 bytes of K per row (64 bf16 = 4 MFMA K steps, or 128 E4M3 = 2
        // MX MFMA K steps), in the 128-byte-row swizzle (swz) the MFMA core reads.  Whole
        // 128-byte rows per load keep every L2 request a full line.  Load q of wave w fills row
        // pairs j = 4 (8w + q) + L / 16; lane L's 16-byte LDS slot s = L % 16 holds (row parity,
        // chunk) = s ^ hs(j).  MXFP8 adds one 4-byte load per operand per stage: the E8M0 scales
        // of the stage's four 32-value blocks of row 64w + L.
        uint32_t a_vo[8], b_vo[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int j = (wave * 8 + q) * 4 + (lane >> 4);
          const uint32_t hs = (uint32_t)((j & 7) | ((j & 4) << 1));
          const uint32_t sl = (uint32_t)(lane & 15) ^ hs;
          const int r = 2 * j + (int)(sl >> 3);
          const uint32_t c = sl & 7u;
          a_vo[q] = (uint32_t)r * rowb + c * 16;
          b_vo[q] = (uint32_t)(b_row(r) * rowb) + c * 16;
        }
        const uint32_t lds0 = lds_addr(smem) + (uint32_t)(wave * 8) * 1024u;
        const uint32_t lds_sc = lds_addr(smem + 2 * kStageBytes) + (uint32_t)wave * 256u;
        i32x4 vas = va, vbs = vb;
        uint32_t as_vo = 0, bs_vo = 0;
        if constexpr (kMx) {
          const int r = wave * 64 + lane;
          vas = make_vsharp(p.a_scales + (int64_t)row0 * kscale_row, (uint32_t)mrows * kscale_row);
          as_vo = (uint32_t)r * kscale_row;
          const uint8_t* sbase = p.ws + (int64_t)e * p.ws_stride;
          vbs = kFc1 ? make_vsharp(sbase, (uint32_t)(2 * N * kscale_row))
                     : make_vsharp(sbase + (int64_t)nt * kBN * kscale_row,
                                   (uint32_t)(min((int64_t)kBN, N - (int64_t)nt * kBN) * kscale_row));
          bs_vo = (uint32_t)(b_row(r) * kscale_row);
        }
        auto issue = [&](int kt) {
          const uint32_t sa = lds0 + (uint32_t)(kt & 1) * (uint32_t)kStageBytes;
          const uint32_t so = (uint32_t)kt * kRowBytes;
#pragma unroll
          for (int q = 0; q < 8; ++q) dma16(va, sa + q * 1024u, a_vo[q], so);
#pragma unroll
          for (int q = 0; q < 8; ++q) dma16(vb, sa + kTileBytes + q * 1024u, b_vo[q], so);
          if constexpr (kMx) {
            const uint32_t ss = lds_sc + (uint32_t)(kt & 1) * 2048u;
            dma4(vas, ss, as_vo, (uint32_t)kt * 4u);
            dma4(vbs, ss + 1024u, bs_vo, (uint32_t)kt * 4u);
          }
        };
        issue(u0);
        for (int kt = u0; kt < u1; ++kt) {
          // stage kt landed (own loads + barrier); every wave finished reading stage kt-1, whose
          // buffer takes stage kt+1 while stage kt is multiplied
          wait_vmcnt<0>();
          __syncthreads();
          if (kt + 1 < u1) issue(kt + 1);
          const uint8_t* sA = smem + (kt & 1) * kStageBytes;
          const uint32_t* sS = reinterpret_cast<const uint32_t*>(smem + 2 * kStageBytes + (kt & 1) * 2048);
          core.compute(sA, sA + kTileBytes, sS, sS + 256, wm, wn, lane);
        }
      }
      __syncthreads();
    }

    // ---- epilogue, staged through LDS (the stage buffers are free after the last barrier).
    // The lane id is laundered so the address arithmetic below is redone per tile instead of
    // being hoisted above the main loop (where it would occupy ~100 VGPRs for the whole loop).
    int elane = lane, etid = tid;
    asm volatile("" : "+v"(elane), "+v"(etid));
    const int r32 = elane & 31, g4 = (elane >> 5) * 4;
    if constexpr (kFc1) {
      const int64_t I = N;
      const int64_t n0h = (int64_t)nt * 128;
      if (p.save_gu) {
        // training: the gate-up output as bf16, staged as a [256][256] tile (gate columns
        // [0,128), up columns [128,256)) and stored as 128-byte row segments
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = (j >> 1) * 128 + wn * 64 + (j & 1) * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int mb = wm * 128 + g4 + (r & 3);
              const uint32_t off = epi_off(mb, n >> 3) + (n & 7) * 2 + (uint32_t)((i * 32 + (r >> 2) * 8) * 512);
              *reinterpret_cast<uint16_t*>(smem + off) = f32_to_bf16(core.acc[i][j][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = q * 256 + etid;
          const int m = u >> 2, b = u & 3;
          const int64_t col = n0h + (b & 1) * 64;
          if (m < mrows && col < I) {
            uint16_t* dst = p.save_gu + (int64_t)(row0 + m) * 2 * I + (b >> 1) * I + col;
            u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
            for (int c = 0; c < 8; ++c) d[c] = *reinterpret_cast<const u32x4*>(smem + epi_off(m, b * 8 + c));
          }
        }
        __syncthreads();
      }
      // (A) silu(g) * u per element, fp32, into a rotated [256][128] LDS tile
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int n = wn * 64 + jj * 32 + r32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float gv = core.acc[i][jj][r], uv = core.acc[i][jj + 2][r];
            // m & 7 and the chunk rotation depend only on (lane, r & 3); i and r >> 2 add constants
            const int mb = wm * 128 + g4 + (r & 3);
            const uint32_t off = epi_off(mb, n >> 2) + (n & 3) * 4 + (uint32_t)((i * 32 + (r >> 2) * 8) * 512);
            *reinterpret_cast<float*>(smem + off) = silu_f(gv) * uv;
          }
          __builtin_amdgcn_sched_barrier(0);   // keep the accumulator reads of one fragment pair together
        }
      }
      __syncthreads();
      // (B) a thread owns whole 32-column blocks of a row: scale by prob, round or quantize
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = q * 256 + etid;
        const int m = u >> 2, b = u & 3;
        const int64_t col = n0h + b * 32;
        if (m < mrows && col < I) {
          const int64_t grow = row0 + m;
          const float pr = p.prob_perm[grow];
          float v[32];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(smem + epi_off(m, b * 8 + c));
            v[4 * c] = w[0] * pr; v[4 * c + 1] = w[1] * pr; v[4 * c + 2] = w[2] * pr; v[4 * c + 3] = w[3] * pr;
          }
          if (!kMx || p.save_h) {
            uint16_t* dst = kMx ? p.save_h : reinterpret_cast<uint16_t*>(p.out);
            u32x4* d = reinterpret_cast<u32x4*>(dst + grow * I + col);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              d[c] = u32x4{pack_bf16x2(v[8 * c], v[8 * c + 1]), pack_bf16x2(v[8 * c + 2], v[8 * c + 3]),
                           pack_bf16x2(v[8 * c + 4], v[8 * c + 5]), pack_bf16x2(v[8 * c + 6], v[8 * c + 7])};
          }
          if constexpr (kMx) {
            float am = 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) am = fmaxf(am, fabsf(v[c]));
            const int sx = mx_shared_exp(am);
            u32x4 lo, hi;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              lo[c] = mx_pack4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3], sx);
              hi[c] = mx_pack4(v[16 + 4 * c], v[16 + 4 * c + 1], v[16 + 4 * c + 2], v[16 + 4 * c + 3], sx);
            }
            u32x4* d = reinterpret_cast<u32x4*>(p.out + grow * I + col);
            d[0] = lo;
            d[1] = hi;
            p.out_scales[grow * (I / 32) + col / 32] = (uint8_t)(sx + 127);
          }
        }
      }
      __syncthreads();
    } else {
      const int64_t n0 = (int64_t)nt * kBN;
      // a split part stores its whole fp32 tile, row-major [256][256], to its slot of p.part;
      // fc2_fixup_kernel sums the parts
      if constexpr (kOutF32) {
        const bool sp = part >= 0;
        float* const fdst = sp ? p.part + (size_t)(t - full) * 65536 : reinterpret_cast<float*>(p.out);
        const int64_t fld = sp ? 256 : N;
        const int64_t frow0 = sp ? 0 : row0, fcol0 = sp ? 0 : n0;
        const int fmrows = sp ? kBM : mrows;
        const int64_t fN = sp ? 256 : N;
        // fp32 output: two passes of 128 rows (a [128][256] fp32 tile is 128 KB)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          if (wm == half) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int n = wn * 128 + j * 32 + r32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const int mb = g4 + (r & 3);
                  const uint32_t off = epi_off_wide(mb, n >> 2) + (n & 3) * 4 + (uint32_t)((i * 32 + (r >> 2) * 8) * 1024);
                  *reinterpret_cast<float*>(smem + off) = core.acc[i][j][r];
                }
                __builtin_amdgcn_sched_barrier(0);
              }
          }
          __syncthreads();
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int u = q * 256 + etid;
            const int ml = u >> 2, b = u & 3;     // 64-column block b of local row ml
            const int m = half * 128 + ml;
            const int64_t col = fcol0 + b * 64;
            if (m < fmrows && col < fN) {
              u32x4* d = reinterpret_cast<u32x4*>(fdst + (frow0 + m) * fld + col);
#pragma unroll
              for (int c = 0; c < 16; ++c) d[c] = *reinterpret_cast<const u32x4*>(smem + epi_off_wide(ml, b * 16 + c));
            }
          }
          __syncthreads();
        }
      } else {
        // (A) bf16 into a rotated [256][256] LDS tile
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = wn * 128 + j * 32 + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int m = wm * 128 + i * 32 + (r >> 2) * 8 + g4 + (r & 3);
              const int mb = wm * 128 + g4 + (r & 3);
              const uint32_t off = epi_off(mb, n >> 3) + (n & 7) * 2 + (uint32_t)((i * 32 + (r >> 2) * 8) * 512);
              *reinterpret_cast<uint16_t*>(smem + off) = f32_to_bf16(core.acc[i][j][r]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        __syncthreads();
        // (B) a thread copies 64-column (128-byte) row segments out with 16-byte stores
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int u = q * 256 + etid;
          const int m = u >> 2, b = u & 3;
          const int64_t col = n0 + b * 64;
          if (m < mrows && col < N) {
            u32x4* d = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)(row0 + m) * N + col);
#pragma unroll
            for (int c = 0; c < 8; ++c) d[c] = *reinterpret_cast<const u32x4*>(smem + epi_off(m, b * 8 + c));
          }
        }
        __syncthreads();
      }
    }
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
  const int mt = local % nM, nt = local / nM;
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
  if (!mx)
    for (int e = 0; e < g.E; ++e) k.w[e] = reinterpret_cast<const uint8_t*>(g.w_tab[e]);
  return k;
}

}  // namespace

hipError_t launch_fc1(const FwdGemm& g, bool mx, hipStream_t st) {
  FwdKArgs k = make_fwd_args(g, mx, true);
  if (mx) fwd_gemm_kernel<true, true, false><<<kGemmGrid, 256, 0, st>>>(k);
  else fwd_gemm_kernel<false, true, false><<<kGemmGrid, 256, 0, st>>>(k);
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
  if (g.out_f32) {
    if (mx) fwd_gemm_kernel<true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
    else fwd_gemm_kernel<false, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  } else {
    if (mx) fwd_gemm_kernel<true, false, false><<<kGemmGrid, 256, 0, st>>>(k);
    else fwd_gemm_kernel<false, false, false><<<kGemmGrid, 256, 0, st>>>(k);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !split) return err;
  // pass 2: the split parts (whether there are any is decided on the device), then the fixup
  k.split = 2;
  if (mx) fwd_gemm_kernel<true, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  else fwd_gemm_kernel<false, false, true><<<kGemmGrid, 256, 0, st>>>(k);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 fgrid(kGemmGrid, kBM / 32);
  if (g.out_f32) fc2_fixup_kernel<true><<<fgrid, 256, 0, st>>>(k, kU);
  else fc2_fixup_kernel<false><<<fgrid, 256, 0, st>>>(k, kU);
  return hipGetLastError();
}

}  // namespace moe
