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
// both token-major activations in wgrad) are loaded as 8 x 8 bf16 blocks and
// transposed in registers (v_perm_b32) into the same K-major, XOR-swizzled LDS
// layout the MFMA core reads.  MXFP8 operands arrive already quantized along
// each GEMM's K in K-major layout, so they use the plain row loader.
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

// Write a 256 x 256 fp32 accumulator tile to dst (row stride ld elements), rows < mrows and
// columns < ncols (a multiple of 64) only, through LDS: bf16 in one pass, fp32 in two halves.
template <bool kF32, class Core>
__device__ __forceinline__ void store_tile(const Core& core, uint8_t* smem, uint8_t* dst, int64_t ld, int mrows,
                                           int ncols, int wm, int wn, int elane, int etid) {
  const int r32 = elane & 31, g4 = (elane >> 5) * 4;
  if constexpr (!kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 128 + j * 32 + r32;
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
      if (m < mrows && b * 64 < ncols) {
        u32x4* d = reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(dst) + (int64_t)m * ld + b * 64);
#pragma unroll
        for (int c = 0; c < 8; ++c) d[c] = *reinterpret_cast<const u32x4*>(smem + epi_off(m, b * 8 + c));
      }
    }
    __syncthreads();
  } else {
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
              const uint32_t off =
                  epi_off_wide(mb, n >> 2) + (n & 3) * 4 + (uint32_t)((i * 32 + (r >> 2) * 8) * 1024);
              *reinterpret_cast<float*>(smem + off) = core.acc[i][j][r];
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int u = q * 256 + etid;
        const int ml = u >> 2, b = u & 3;
        const int m = half * 128 + ml;
        if (m < mrows && b * 64 < ncols) {
          u32x4* d = reinterpret_cast<u32x4*>(reinterpret_cast<float*>(dst) + (int64_t)m * ld + b * 64);
#pragma unroll
          for (int c = 0; c < 16; ++c) d[c] = *reinterpret_cast<const u32x4*>(smem + epi_off_wide(ml, b * 16 + c));
        }
      }
      __syncthreads();
    }
  }
}

// Store the 8 transposed columns of one 8x8 block: column c goes to LDS row nb*8 + c, chunk kb.
__device__ __forceinline__ void store_t8(uint8_t* s, const u32x4 w[8], int nb, int kb) {
#pragma unroll
  for (int c = 0; c < 8; ++c) *reinterpret_cast<u32x4*>(s + swz(nb * 8 + c, kb)) = w[c];
}

template <int kRole, bool kMx, bool kOutF32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_gemm_kernel(const BwdKArgs p) {
  constexpr bool kWg = kRole == kRoleWgrad;
  constexpr bool kAMN = kWg && !kMx;   // bf16 wgrad: A is token-major
  constexpr bool kBMN = !kMx;          // bf16: B is N-contiguous (weights in dgrad, activations in wgrad)
  // two stages of A + B (64 KB each; the epilogue reuses them) plus the MXFP8 scale words
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes + (kMx ? 2 * 2048 : 16)];
  __shared__ Sched sched;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = p.E;
  build_sched(sched, p.split_sizes, E, p.nN, kWg ? (kMx ? p.pad : 1) : 0);
  const int total = kWg ? E * p.nM * p.nN : __builtin_amdgcn_readfirstlane(sched.tile[E]);
  const int G = gridDim.x, per = G >> 3, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  constexpr int kKStep = kMx ? 128 : 64;                  // K values per LDS stage

  for (int round = 0;; ++round) {
    const int t = round * G + xcd * per + slot;
    if (t >= total) break;
    int e, mt, nt, row0, mrows, ncols, kT;
    int64_t koff = 0;
    if constexpr (kWg) {
      const int pe = p.nM * p.nN;
      e = t / pe;
      const int local = t - e * pe;
      mt = local % p.nM;
      nt = local / p.nM;
      const int Me = __builtin_amdgcn_readfirstlane(sched.cnt[e]);
      koff = kMx ? __builtin_amdgcn_readfirstlane(sched.tile[e]) : __builtin_amdgcn_readfirstlane(sched.off[e]);
      kT = (Me + kKStep - 1) / kKStep;
      row0 = mt * kBM;
      mrows = (int)min((int64_t)kBM, p.M - row0);
      ncols = (int)min((int64_t)kBN, p.N - (int64_t)nt * kBN);
    } else {
      e = __builtin_amdgcn_readfirstlane(find_expert(sched, E, t));
      const int Me = __builtin_amdgcn_readfirstlane(sched.cnt[e]);
      const int nMe = (Me + kBM - 1) / kBM;
      const int local = t - __builtin_amdgcn_readfirstlane(sched.tile[e]);
      mt = local % nMe;
      nt = local / nMe;
      row0 = __builtin_amdgcn_readfirstlane(sched.off[e]) + mt * kBM;
      mrows = min(kBM, Me - mt * kBM);
      ncols = (int)min((int64_t)kBN, p.N - (int64_t)nt * kBN);
      kT = (int)(p.K * (kMx ? 1 : 2) / kRowBytes);
    }
    const int64_t n0 = (int64_t)nt * kBN;
    const int64_t m0w = (int64_t)mt * kBM;                // wgrad output row origin

    // ---- operands: two LDS stages of A and B (32 KB each) filled by direct-to-LDS loads
    // (buffer_load_dwordx4 ... lds, lane L's 16 bytes to slot L of a contiguous 1 KB block).
    //   K-major operand: 256 rows x 128 bytes of K in the swz layout; load q of wave w fills row
    //     pairs j = 4 (8w + q) + L / 16, slot s = L % 16 holding (row parity, chunk) = s ^ hs(j).
    //   MN-major operand (bf16, K rows of 256 contiguous columns): 64 K rows x 512 bytes in the
    //     mnswz layout; load q of wave w fills rows 2 (8w + q) + L / 32, physical chunk L % 32.
    //     The K row advance is carried in the per-lane offset so that rows past the end of the
    //     operand (a ragged token segment in wgrad) fall outside the descriptor and read zero.
    //   MXFP8 operands are K-major, with one 4-byte E8M0 word per row per stage.
    int64_t a_base_off, b_base_off;
    uint32_t a_range, b_range;
    const uint8_t* abase;
    const uint8_t* bbase;
    if constexpr (kAMN) {            // bf16 wgrad: A^T = token-major rows [tok][M]
      const int Me = __builtin_amdgcn_readfirstlane(sched.cnt[e]);
      abase = p.a; a_base_off = koff * p.lda + m0w * 2; a_range = (uint32_t)max((int64_t)0, Me * p.lda - m0w * 2);
    } else if constexpr (kWg) {      // MXFP8 wgrad: A^T quantized [M][Rpad], segment at koff
      abase = p.a; a_base_off = m0w * p.lda + koff; a_range = (uint32_t)(mrows * p.lda);
    } else {
      abase = p.a; a_base_off = (int64_t)row0 * p.lda; a_range = (uint32_t)(mrows * p.lda);
    }
    if constexpr (kBMN) {
      if constexpr (kWg) {           // bf16 wgrad: token-major rows [tok][N]
        const int Me = __builtin_amdgcn_readfirstlane(sched.cnt[e]);
        bbase = p.b; b_base_off = koff * p.ldb + n0 * 2; b_range = (uint32_t)max((int64_t)0, Me * p.ldb - n0 * 2);
      } else {                       // bf16 dgrad: W_e [K][N]
        bbase = bwd_table(e); b_base_off = n0 * 2; b_range = (uint32_t)(p.K * p.ldb - n0 * 2);
      }
    } else if constexpr (kWg) {      // MXFP8 wgrad: B^T quantized [N][Rpad]
      bbase = p.b; b_base_off = n0 * p.ldb + koff; b_range = (uint32_t)(ncols * p.ldb);
    } else {                         // MXFP8 dgrad: W^T quantized [N][K] per expert
      bbase = p.b + (int64_t)e * p.b_stride; b_base_off = n0 * p.ldb; b_range = (uint32_t)(ncols * p.ldb);
    }
    const i32x4 va = make_vsharp(abase + a_base_off, a_range);
    const i32x4 vb = make_vsharp(bbase + b_base_off, b_range);
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
    const uint32_t lds0 = lds_addr(smem) + (uint32_t)(wave * 8) * 1024u;
    i32x4 vas = va, vbs = vb;
    uint32_t as_vo = 0, bs_vo = 0;
    if constexpr (kMx) {
      const int r = wave * 64 + lane;
      if constexpr (kWg) {
        vas = make_vsharp(p.as + m0w * p.ldas + koff / 32, (uint32_t)(mrows * p.ldas));
        vbs = make_vsharp(p.bs + n0 * p.ldbs + koff / 32, (uint32_t)(ncols * p.ldbs));
      } else {
        vas = make_vsharp(p.as + (int64_t)row0 * p.ldas, (uint32_t)(mrows * p.ldas));
        vbs = make_vsharp(p.bs + (int64_t)e * p.bs_stride + n0 * p.ldbs, (uint32_t)(ncols * p.ldbs));
      }
      as_vo = (uint32_t)(r * p.ldas);
      bs_vo = (uint32_t)(r * p.ldbs);
    }
    const uint32_t lds_sc = lds_addr(smem + 2 * kStageBytes) + (uint32_t)wave * 256u;

    TileCore<kMx, false> core;
    core.zero();
    auto issue = [&](int kt) {
      const uint32_t sa = lds0 + (uint32_t)(kt & 1) * (uint32_t)kStageBytes;
      const uint32_t ao = (uint32_t)kt * a_step, bo = (uint32_t)kt * b_step;
#pragma unroll
      for (int q = 0; q < 8; ++q) dma16(va, sa + q * 1024u, a_vo[q] + ao, 0);
#pragma unroll
      for (int q = 0; q < 8; ++q) dma16(vb, sa + kTileBytes + q * 1024u, b_vo[q] + bo, 0);
      if constexpr (kMx) {
        const uint32_t ss = lds_sc + (uint32_t)(kt & 1) * 2048u;
        dma4(vas, ss, as_vo + (uint32_t)kt * 4u, 0);
        dma4(vbs, ss + 1024u, bs_vo + (uint32_t)kt * 4u, 0);
      }
    };
    if (kT > 0) {
      issue(0);
      for (int kt = 0; kt < kT; ++kt) {
        // stage kt landed (own loads + barrier); every wave finished stage kt-1, whose buffer
        // takes stage kt+1 while stage kt is multiplied
        wait_vmcnt<0>();
        __syncthreads();
        if (kt + 1 < kT) issue(kt + 1);
        const uint8_t* sA = smem + (kt & 1) * kStageBytes;
        if constexpr (kMx) {
          const uint32_t* sS = reinterpret_cast<const uint32_t*>(smem + 2 * kStageBytes + (kt & 1) * 2048);
          core.compute(sA, sA + kTileBytes, sS, sS + 256, wm, wn, lane);
        } else {
          core.template compute_x<kAMN, kBMN>(sA, sA + kTileBytes, wm, wn, lane);
        }
      }
      __syncthreads();
    }

    // ---- epilogue
    int elane = lane, etid = tid;
    asm volatile("" : "+v"(elane), "+v"(etid));
    if constexpr (kRole == kRoleDgradFc2) {
      const int r32 = elane & 31, g4 = (elane >> 5) * 4;
      const int64_t I = p.I;
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
                const uint32_t off =
                    epi_off_wide(mb, n >> 2) + (n & 3) * 4 + (uint32_t)((i * 32 + (r >> 2) * 8) * 1024);
                *reinterpret_cast<float*>(smem + off) = core.acc[i][j][r];
              }
              __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int u = q * 256 + etid;
          const int ml = u >> 2, b = u & 3;
          const int m = half * 128 + ml;
          const int64_t col = n0 + b * 64;
          float part = 0.f;
          if (m < mrows && col < I) {
            const int64_t grow = row0 + m;
            const float pr = p.prob_perm[grow];
            const uint16_t* gp = p.gu + grow * 2 * I + col;
            uint16_t* dgp = p.dgu + grow * 2 * I + col;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const f32x4 d0 = *reinterpret_cast<const f32x4*>(smem + epi_off_wide(ml, b * 16 + 2 * c));
              const f32x4 d1 = *reinterpret_cast<const f32x4*>(smem + epi_off_wide(ml, b * 16 + 2 * c + 1));
              const u32x4 gw = *reinterpret_cast<const u32x4*>(gp + 8 * c);
              const u32x4 uw = *reinterpret_cast<const u32x4*>(gp + I + 8 * c);
              float dgv[8], duv[8];
#pragma unroll
              for (int x = 0; x < 8; ++x) {
                const float dh = x < 4 ? d0[x] : d1[x - 4];
                const uint32_t gwd = gw[x >> 1], uwd = uw[x >> 1];
                const float g = bf16_to_f32((uint16_t)((x & 1) ? (gwd >> 16) : (gwd & 0xFFFF)));
                const float uu = bf16_to_f32((uint16_t)((x & 1) ? (uwd >> 16) : (uwd & 0xFFFF)));
                const float s = sigmoid_f(g);
                const float sl = g * s;
                part += dh * (sl * uu);
                const float da = dh * pr;
                duv[x] = da * sl;
                dgv[x] = da * uu * (s * (1.0f + g * (1.0f - s)));
              }
              *reinterpret_cast<u32x4*>(dgp + 8 * c) =
                  u32x4{pack_bf16x2(dgv[0], dgv[1]), pack_bf16x2(dgv[2], dgv[3]), pack_bf16x2(dgv[4], dgv[5]),
                        pack_bf16x2(dgv[6], dgv[7])};
              *reinterpret_cast<u32x4*>(dgp + I + 8 * c) =
                  u32x4{pack_bf16x2(duv[0], duv[1]), pack_bf16x2(duv[2], duv[3]), pack_bf16x2(duv[4], duv[5]),
                        pack_bf16x2(duv[6], duv[7])};
            }
          }
          // the 4 column blocks of a row sit in 4 consecutive lanes: fixed-order pairwise sum
          part += __shfl_xor(part, 1, 64);
          part += __shfl_xor(part, 2, 64);
          if (b == 0 && m < mrows) p.dprob_part[(int64_t)(row0 + m) * p.nN + nt] = part;
        }
        __syncthreads();
      }
    } else if constexpr (kRole == kRoleDgradFc1) {
      uint8_t* dst = p.out + ((int64_t)row0 * p.N + n0) * (kOutF32 ? 4 : 2);
      store_tile<kOutF32>(core, smem, dst, p.N, mrows, ncols, wm, wn, elane, etid);
    } else {
      uint8_t* dst = const_cast<uint8_t*>(bwd_table(e)) + (m0w * p.N + n0) * (kOutF32 ? 4 : 2);
      store_tile<kOutF32>(core, smem, dst, p.N, mrows, ncols, wm, wn, elane, etid);
    }
  }
}

template <int kRole, bool kMx>
hipError_t launch_role(const BwdKArgs& k, bool out_f32, hipStream_t st) {
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
  k.dprob_part = g.dprob_part;
  k.I = g.I;
  k.out = reinterpret_cast<uint8_t*>(g.out);
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
  return mx ? launch_role<kRoleDgradFc1, true>(k, g.out_f32, st) : launch_role<kRoleDgradFc1, false>(k, g.out_f32, st);
}

hipError_t launch_bwd_wgrad(const BwdGemm& g, bool mx, hipStream_t st) {
  BwdKArgs k = base_args(g);
  return mx ? launch_role<kRoleWgrad, true>(k, g.out_f32, st) : launch_role<kRoleWgrad, false>(k, g.out_f32, st);
}

int bwd_dprob_parts(int64_t I) { return (int)((I + kBN - 1) / kBN); }

}  // namespace moe
