// Shared pieces of the grouped GEMMs for gfx950: buffer descriptors and
// direct-to-LDS loads, the swizzled LDS layouts, the in-kernel per-expert tile
// scheduler, the 256x256 tile's accumulators and the interleaved stage schedule
// of its MFMAs (BF16 32x32x16 and MX-scaled FP8 32x32x64).
#pragma once
#include <cstddef>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace gemm {

constexpr int kBM = 256, kBN = 256;
constexpr int kRowBytes = 128;
constexpr int kTileBytes = 256 * kRowBytes;     // 32 KB per operand tile
constexpr int kStageBytes = 2 * kTileBytes;     // A + B

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// 128-byte rows, stored in pairs: rows 2j and 2j+1 share one 256-byte bank line (16 slots
// of 16 bytes), and chunk c of row r sits in slot (((r & 1) << 3) | c) ^ hs(j),
// hs(j) = (j & 7) | ((j & 4) << 1).  LDS serves a 16-byte-per-lane access 16 lanes (256 bytes,
// 64 banks) at a time, and each of these 16-lane patterns lands in 16 distinct slots:
//   * MFMA fragment reads: 16 consecutive rows at one chunk;
//   * row-wise stores: two adjacent rows, all 8 chunks each;
//   * transposed 8x8-block stores: rows R and R + 8 (same parity), all 8 chunks each --
//     hs(j) and hs(j + 4) differ in bit 3, which moves the second row to the other half.
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  const uint32_t j = row >> 1;
  const uint32_t hs = (j & 7u) | ((j & 4u) << 1);
  return j * 256u + (((((row & 1u) << 3) | chunk) ^ hs) << 4);
}

// Per-expert counts, row offsets and tile prefix (ceil(M_e / 256) * nN) in LDS.
struct Sched {
  int cnt[kMaxExperts];
  int off[kMaxExperts + 1];
  int tile[kMaxExperts + 1];
};

// Per-expert counts and row offsets; tile[e] = prefix of ceil(cnt / 256) * nN when pad == 0,
// or of ceil(cnt / pad) * pad (padded token offsets) when pad > 0.
__device__ void build_sched(Sched& s, const int32_t* split_sizes, int E, int nN, int pad = 0) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c = tid < E ? split_sizes[tid] : 0;
  int t = pad ? (c + pad - 1) / pad * pad : (c + kBM - 1) / kBM * nN;
  // inclusive wave scans of c and t
  int ic = c, it = t;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int oc = __shfl_up(ic, d, 64), ot = __shfl_up(it, d, 64);
    if (lane >= d) { ic += oc; it += ot; }
  }
  __shared__ int wsum_t[4];
  if (lane == 63) { wsum[wave] = ic; wsum_t[wave] = it; }
  __syncthreads();
  int bc = 0, bt = 0;
  for (int w = 0; w < wave; ++w) { bc += wsum[w]; bt += wsum_t[w]; }
  if (tid < E) {
    s.cnt[tid] = c;
    s.off[tid] = bc + ic - c;
    s.tile[tid] = bt + it - t;
  }
  if (tid == E - 1) { s.off[E] = bc + ic; s.tile[E] = bt + it; }
  __syncthreads();
}

// Coordinates (mt, nt) of tile `local` of one expert's nM x nN tile grid.  The M-tiles are split
// into ng = ceil(nM / group_m) groups of balanced size (group_m: kGroupM unless the caller picks one) (the first nM % ng groups one larger), and
// each group is walked panel by panel with its M-tiles fastest.  The 32 consecutive tiles an XCD
// takes in a round then span at most kGroupM M-tiles and several panels, whose operand slices the
// XCD's L2 shares, instead of up to 32 M-tiles of one panel.  With nM <= kGroupM this is the plain
// M-fastest order.
constexpr int kGroupM = 8;
__device__ __forceinline__ void tile_coords(int local, int nM, int nN, int& mt, int& nt, int group_m = kGroupM) {
  const int ng = (nM + group_m - 1) / group_m;
  const int base = nM / ng, r = nM - base * ng;      // r groups of base + 1 M-tiles, then base
  const int big = r * (base + 1) * nN;               // tiles of the larger groups
  int gm, m0, l;
  if (local < big) {
    const int g = local / ((base + 1) * nN);
    gm = base + 1;
    m0 = g * gm;
    l = local - g * gm * nN;
  } else {
    const int g = (local - big) / (base * nN);
    gm = base;
    m0 = r * (base + 1) + g * base;
    l = local - big - g * base * nN;
  }
  mt = m0 + l % gm;
  nt = l / gm;
}

__device__ __forceinline__ int find_expert(const Sched& s, int E, int t) {
  int lo = 0, hi = E - 1;   // largest e with tile[e] <= t (tile[] is non-decreasing)
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s.tile[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// silu(g) = g * sigmoid(g) with the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32, ~1 ulp each)
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_f(float g) { return g * sigmoid_f(g); }

// ---- MN-major (N-contiguous) bf16 tiles: a stage of 64 K rows x 256 columns (512 bytes per row).
// Row k's 16-byte chunk c is stored at chunk c ^ ((k & 3) << 2) of the row.  A transposing read
// (ds_read_b64_tr_b16) by 16 lanes covers 4 K rows x 16 columns: source lane 4 j + q reads the
// 8 bytes of row k0 + j at columns c0 + 4q..4q+3, and lane i of the group receives column c0 + i at
// rows k0..k0+3.  The swizzle puts those 4 rows x 32 bytes (and the neighbouring group's) in 16
// distinct 16-byte bank groups.
__device__ __forceinline__ uint32_t mnswz(uint32_t k, uint32_t col) {
  return k * 512u + ((((col >> 3) ^ ((k & 3u) << 2))) << 4) + (col & 7u) * 2u;
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));

// The MFMA bf16 operand of rows (M or N) rb + 0..31, K step kk (16 values) of an MN-major stage:
// lane l holds row rb + l % 32 at K values 16 kk + 8 (l / 32) + 0..7.
__device__ __forceinline__ bf16x8 load_mn_frag(const uint8_t* s, int rb, int kk, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int col = rb + 16 * (G & 1) + 4 * (sl & 3);
  const int k = kk * 16 + 8 * (G >> 1) + (sl >> 2);
  typedef __attribute__((address_space(3))) bf16x4_t lds_v4;
  const auto base = (__attribute__((address_space(3))) uint8_t*)(s);
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(base + mnswz(k, col)));
  const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4*)(base + mnswz(k + 4, col)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---- direct-to-LDS loads: the LDS-DMA form of buffer_load places lane L's 16 bytes at
// slot L of a contiguous 1 KB block, so the swizzle of the LDS tile (swz) is applied on the
// global side, by choosing which row and chunk each lane fetches.
// K units of 128 bytes per part of a split tile, at least: a split costs two short extra launches
// (the parts and the fixup), so it only pays for long tiles.  (Measured on the 64-expert layer's
// FC2, K = 1408 with a last round of 8 tiles: parts of 2 units made the layer 1.5-2.5 % slower.)
constexpr int kMinSplitUnits = 16;

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
// s_waitcnt vmcnt(n) with the other counters left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer descriptor as four SGPR words, for the inline-asm LDS-DMA loads below.
__device__ __forceinline__ i32x4 make_vsharp(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 v;
  v[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  v[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  v[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  v[3] = 0x00020000;
  return v;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(lds_ptr_t)p);
}

// 16-byte buffer load straight into LDS: lane L's bytes land at lds + 16 L.  Issued as inline
// asm so the compiler does not treat it as an LDS write that every later LDS read must wait
// for; the kernel orders it explicitly with wait_vmcnt and barriers.  Offsets past `bytes`
// of the descriptor read zero.
__device__ __forceinline__ void dma16(const i32x4& vs, uint32_t lds, uint32_t voff, uint32_t soff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);   // wave-uniform by construction
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(l), "v"(voff), "s"(vs), "s"(soff)
               : "memory", "m0");
}

// 4-byte variant: lane L's word lands at lds + 4 L.
__device__ __forceinline__ void dma4(const i32x4& vs, uint32_t lds, uint32_t voff, uint32_t soff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(l), "v"(voff), "s"(vs), "s"(soff)
               : "memory", "m0");
}

// The 256 x 256 tile's accumulators: wave (wm, wn) owns A rows wm*128 + [0, 128) and B rows
// brow(wn, j) + [0, 32), j < 4, as 4 x 4 blocks of 32 x 32 fp32.  kFc1 selects the B row map of
// the gate-up projection (gate rows [0, 128), the matching up rows [128, 256)).
template <bool kMx, bool kFc1>
struct TileCore {
  f32x16 acc[4][4];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }

  // LDS row of B holding n-fragment j of wave column wn
  static __device__ __forceinline__ int brow(int wn, int j) {
    if (kFc1) return (j < 2) ? (wn * 64 + j * 32) : (128 + wn * 64 + (j - 2) * 32);
    return wn * 128 + j * 32;
  }
};

// ---------------------------------------------------------------------------
// The interleaved stage schedule shared by the forward and backward GEMMs.
// ---------------------------------------------------------------------------
// Fragments of one MFMA K substep of a wave: 4 A blocks (token rows in dgrad and the forward, M
// rows in wgrad) and 4 B blocks of 32 rows, plus the E8M0 scale bytes of the lane's rows (MXFP8).
template <bool kMx>
struct StepFrag {
  typename std::conditional<kMx, i32x8, bf16x8>::type a[4], b[4];
  int sa[4], sb[4];
};

// Element e of the fragments of substep kk, e in the order the 16 MFMAs of a substep consume them
// (A block i outer, B block j inner): a0, b0, b1, b2, b3, a1, a2, a3.  MXFP8 scales: the stage's
// four E8M0 bytes of row r (A rows 0..255, then B rows) at sS + r * kScRow.  BF16 operands are K-major
// (swz layout, one 16-byte read) or MN-major (mnswz layout, two transposing reads); MXFP8 ones are
// K-major, two 16-byte reads plus the scale byte of the lane's 32-value block, read on its own (a
// shift of the whole scale word would make the read wait for LDS on the spot).
template <bool kMx, bool kFc1, bool kAMN, bool kBMN, int kScRow>
__device__ __forceinline__ void read_elem(StepFrag<kMx>& f, const uint8_t* sA, const uint8_t* sS, int kk, int e,
                                          int wm, int wn, int lane) {
  const int r32 = lane & 31, g = lane >> 5;
  const bool isA = e == 0 || e >= 5;
  const int idx = e == 0 ? 0 : (e >= 5 ? e - 4 : e - 1);
  const int rb = isA ? wm * 128 + idx * 32 : TileCore<kMx, kFc1>::brow(wn, idx);
  const uint8_t* base = isA ? sA : sA + kTileBytes;
  if constexpr (!kMx) {
    const bool mn = isA ? kAMN : kBMN;
    const bf16x8 v = mn ? load_mn_frag(base, rb, kk, lane)
                        : *reinterpret_cast<const bf16x8*>(base + swz(rb + r32, (uint32_t)(kk * 2 + g)));
    if (isA) f.a[idx] = v; else f.b[idx] = v;
  } else {
    const int row = rb + r32;
    const u32x4 lo = *reinterpret_cast<const u32x4*>(base + swz(row, (uint32_t)(kk * 4 + g)));
    const u32x4 hi = *reinterpret_cast<const u32x4*>(base + swz(row, (uint32_t)(kk * 4 + 2 + g)));
    const i32x8 v{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    const int sc = sS[((isA ? 0 : 256) + row) * kScRow + 2 * kk + g];
    if (isA) { f.a[idx] = v; f.sa[idx] = sc; } else { f.b[idx] = v; f.sb[idx] = sc; }
  }
}

// Order of the reads of the next substep's elements while the current substep's MFMAs run:
// b0 b1 a0 b2 a1 b3 a2 a3 -- each a block is read only after the MFMAs that use the current one
// are issued, so the two fragment sets share the a registers.
__device__ __forceinline__ constexpr int next_elem(int s) {
  return s == 0 ? 1 : s == 1 ? 2 : s == 2 ? 0 : s == 3 ? 3 : s == 4 ? 5 : s == 5 ? 4 : s;
}

// MFMA of A block i and B block j with the B block as the instruction's first operand: lane l
// accumulates A row 32 i + l % 32 of the wave's block at B rows (output columns) 32 j + 8 q +
// 4 (l / 32) + c in acc[i][j][4 q + c] -- one output row and runs of 4 consecutive columns, which
// the epilogues store straight from the accumulators.
template <bool kMx, bool kFc1>
__device__ __forceinline__ void mma_ij(TileCore<kMx, kFc1>& core, const StepFrag<kMx>& f, int q) {
  const int i = q >> 2, j = q & 3;
  if constexpr (!kMx)
    core.acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], core.acc[i][j], 0, 0, 0);
  else
    core.acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], core.acc[i][j], 0, 0, 0, f.sb[j],
                                                                       0, f.sa[i]);
}

// The MFMAs of one LDS stage (sA: A tile, then B tile; sS: MXFP8 scale words), with the loads of
// the next stage and the next substep's fragment reads interleaved one by one between them, so the
// wave's in-order issue never stalls behind a burst of memory instructions.  dma_a(q) / dma_b(q)
// (q < 8) issue the next stage's A / B loads, dma_s() its MXFP8 scale loads.
//   BF16 (4 substeps): A loads and the substep-1 reads between the MFMAs of substep 0, B loads and
//     the substep-2 reads in substep 1, the substep-3 reads in substep 2.
//   MXFP8 (2 substeps of MFMAs twice as long): all loads and the substep-1 reads in substep 0, the
//     scale loads (dma_s) right after the first MFMA.
// No branch may sit among the MFMAs: the scale bytes read before it would be re-extended after it,
// each behind a wait for its LDS read.
template <bool kMx, bool kFc1, bool kAMN, bool kBMN, int kScRow, class DA, class DB, class DS>
__device__ __forceinline__ void mma_stage(TileCore<kMx, kFc1>& core, const uint8_t* sA, const uint8_t* sS, int wm,
                                          int wn, int lane, DA&& dma_a, DB&& dma_b, DS&& dma_s) {
  StepFrag<kMx> f0, f1;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    read_elem<kMx, kFc1, kAMN, kBMN, kScRow>(f0, sA, sS, 0, e, wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!kMx) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mma_ij(core, f0, q);
      if (q & 1) read_elem<kMx, kFc1, kAMN, kBMN, kScRow>(f1, sA, sS, 1, next_elem(q >> 1), wm, wn, lane);
      else dma_a(q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mma_ij(core, f1, q);
      if (q & 1) read_elem<kMx, kFc1, kAMN, kBMN, kScRow>(f0, sA, sS, 2, next_elem(q >> 1), wm, wn, lane);
      else dma_b(q >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mma_ij(core, f0, q);
      if (q & 1) read_elem<kMx, kFc1, kAMN, kBMN, kScRow>(f1, sA, sS, 3, next_elem(q >> 1), wm, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mma_ij(core, f1, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mma_ij(core, f0, q);
      if (q & 1) {
        read_elem<kMx, kFc1, kAMN, kBMN, kScRow>(f1, sA, sS, 1, next_elem(q >> 1), wm, wn, lane);
        dma_b(q >> 1);
      } else {
        dma_a(q >> 1);
      }
      if (q == 0) dma_s();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      mma_ij(core, f1, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// The substep-0 fragments of the stage in sA / sS, ahead of a deep stage loop.  The MXFP8 scale
// values leave as opaque 32-bit values: were they byte loads on both edges into the loop, the
// compiler would carry them as bytes and re-extend them at the top of every stage, waiting there
// for every LDS read in flight.
template <bool kMx, bool kFc1, bool kAMN, bool kBMN, int kScRow>
__device__ __forceinline__ void read_first(StepFrag<kMx>& f0, const uint8_t* sA, const uint8_t* sS, int wm, int wn,
                                           int lane) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    read_elem<kMx, kFc1, kAMN, kBMN, kScRow>(f0, sA, sS, 0, e, wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kMx) {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(f0.sa[i]), "+v"(f0.sb[i]));
  }
}

// MXFP8 stage with its barrier between the two substeps (the forward GEMM with K of at least two
// stages).  On entry f0 holds this stage's substep-0 fragments, read during the previous stage's
// substep 1 (or by read_first).  Substep 0 reads the substep-1 fragments of this stage (sA, sS).
// sync() then waits for the next stage's loads and for every wave, after which this stage's buffer
// is free: substep 1 reads the next stage's substep-0 fragments (sAn, sSn) into f0, and issues the
// loads of the stage after next into this stage's buffer (dma_a / dma_b, q < 8; dma_s its scale
// group, predicated by its descriptor, since no branch may sit among the MFMAs).  The fragment
// reads of both halves overlap MFMAs, instead of every wave reading its first fragments at once
// after a barrier, and the loads have a whole stage to land.
template <bool kFc1, class DA, class DB, class DS, class SY>
__device__ __forceinline__ void mma_stage_mx_deep(TileCore<true, kFc1>& core, StepFrag<true>& f0, const uint8_t* sA,
                                                  const uint8_t* sS, const uint8_t* sAn, const uint8_t* sSn, int wm,
                                                  int wn, int lane, DA&& dma_a, DB&& dma_b, DS&& dma_s, SY&& sync) {
  StepFrag<true> f1;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mma_ij(core, f0, q);
    if (q & 1) read_elem<true, kFc1, false, false, 16>(f1, sA, sS, 1, next_elem(q >> 1), wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  sync();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mma_ij(core, f1, q);
    if (q & 1) {
      read_elem<true, kFc1, false, false, 16>(f0, sAn, sSn, 0, next_elem(q >> 1), wm, wn, lane);
      dma_b(q >> 1);
    } else {
      dma_a(q >> 1);
    }
    if (q == 0) dma_s();
    __builtin_amdgcn_sched_barrier(0);
  }
}

// BF16 stage with its barrier after the second of its four substeps (the forward GEMM with K of at
// least two stages).  On entry f0 holds this stage's substep-0 fragments.  Substeps 0 and 1 read
// the fragments of substeps 1, 2 and 3 (this stage's buffer is then fully read); sync() waits for
// the next stage's loads and for every wave; substep 2 reads the next stage's substep-0 fragments
// (sAn) into f0 and, with substep 3, issues the loads of the stage after next into this stage's
// buffer.  Memory instructions per substep: 16, 8, 16, 8; three fragment sets live at most.
template <bool kFc1, class DA, class DB, class SY>
__device__ __forceinline__ void mma_stage_bf16_deep(TileCore<false, kFc1>& core, StepFrag<false>& f0,
                                                    const uint8_t* sA, const uint8_t* sAn, int wm, int wn, int lane,
                                                    DA&& dma_a, DB&& dma_b, SY&& sync) {
  StepFrag<false> f1, f2, f3;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mma_ij(core, f0, q);
    if (q & 1) read_elem<false, kFc1, false, false, 4>(f1, sA, sA, 1, next_elem(q >> 1), wm, wn, lane);
    else read_elem<false, kFc1, false, false, 4>(f2, sA, sA, 2, next_elem(q >> 1), wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mma_ij(core, f1, q);
    if (q & 1) read_elem<false, kFc1, false, false, 4>(f3, sA, sA, 3, next_elem(q >> 1), wm, wn, lane);
    __builtin_amdgcn_sched_barrier(0);
  }
  sync();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mma_ij(core, f2, q);
    if (q & 1) read_elem<false, kFc1, false, false, 4>(f0, sAn, sAn, 0, next_elem(q >> 1), wm, wn, lane);
    else dma_a(q >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    mma_ij(core, f3, q);
    if (!(q & 1)) dma_b(q >> 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Lane pairing for epilogue stores.  A lane holds its row's columns 8 q + 4 hh + c (q, c < 4,
// hh = lane / 32) of a 32 x 32 accumulator block; v_permlane32_swap of runs 2 pp and 2 pp + 1 with
// lane l ^ 32 leaves it 8 consecutive columns 16 pp + 8 hh + [0, 8) instead, so that stores move 16
// (bf16) or 8 (E4M3) bytes per lane and 32 or 16 contiguous bytes per row.
//   pack_bf16_runs8: the 16 values to bf16, o[pp] = columns 16 pp + 8 hh + [0, 8);
//   swap_runs8: 4 words of 4 E4M3 codes (run q each), o[pp] = columns 16 pp + 8 hh + [0, 8).
__device__ __forceinline__ void pack_bf16_runs8(const float (&v)[16], u32x4 (&o)[2]) {
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    uint32_t w0[2], w1[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      w0[k] = pack_bf16x2(v[8 * pp + 2 * k], v[8 * pp + 2 * k + 1]);
      w1[k] = pack_bf16x2(v[8 * pp + 4 + 2 * k], v[8 * pp + 4 + 2 * k + 1]);
      const auto r = __builtin_amdgcn_permlane32_swap(w0[k], w1[k], false, false);
      w0[k] = (uint32_t)r[0];
      w1[k] = (uint32_t)r[1];
    }
    o[pp] = u32x4{w0[0], w0[1], w1[0], w1[1]};
  }
}
__device__ __forceinline__ void swap_runs8(const uint32_t (&c)[4], u32x2 (&o)[2]) {
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const auto r = __builtin_amdgcn_permlane32_swap(c[2 * pp], c[2 * pp + 1], false, false);
    o[pp] = u32x2{(uint32_t)r[0], (uint32_t)r[1]};
  }
}

// max(v, v of lane l ^ 32) by v_permlane32_swap (a VALU exchange of the wave's halves, no LDS round
// trip): swapping a register with itself leaves each lane its own value in one result and its
// partner's in the other.
__device__ __forceinline__ float max_xor32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}

// A 32-row x 128-byte output block held one row per lane pair: lane l holds 16-byte chunks
// 2 q + l / 32 (q < 4) of row l % 32, as lo (q = 0, 1) and hi (q = 2, 3), four words per chunk.
// The block passes through a 2 KB LDS slot 16 rows at a time and comes back as out[t] = chunk
// l % 8 of row 8 t + l / 8, ready for stores of 8 whole 128-byte rows per instruction (the
// lane-pair layout itself stores 32-byte pieces of 32 rows, and partial lines cost the write path
// several times their bytes).  A permlane16 swap first trades the hi chunks of rows 0-15 for the
// lo chunks of rows 16-31, so each half is written by all 64 lanes in two instructions.  Chunk c
// of slot row r sits at chunk c ^ (r & 7): conflict-free writes and reads.  The LDS unit runs
// one wave's operations in issue order, so the reads see the writes and the next writes cannot
// overtake the reads without any counter wait; the empty asm statements only keep the compiler
// from moving LDS accesses across them.
__device__ __forceinline__ void stage_rows32(uint8_t* slot, uint32_t (&lo)[8], uint32_t (&hi)[8], int lane,
                                             u32x4 (&out)[4]) {
  const uint32_t r32 = (uint32_t)lane & 31u, cb = (uint32_t)lane >> 5, h16 = r32 >> 4, rr = r32 & 15u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto sw = __builtin_amdgcn_permlane16_swap(lo[k], hi[k], false, false);
    lo[k] = sw[0];
    hi[k] = sw[1];
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t* d = h ? hi : lo;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      *reinterpret_cast<u32x4*>(slot + rr * 128u + (((2u * ((uint32_t)t + 2u * h16) + cb) ^ (rr & 7u)) << 4)) =
          u32x4{d[4 * t], d[4 * t + 1], d[4 * t + 2], d[4 * t + 3]};
    asm volatile("" ::: "memory");
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t row = 8u * (uint32_t)t + ((uint32_t)lane >> 3);
      out[2 * h + t] = *reinterpret_cast<const u32x4*>(slot + row * 128u + ((((uint32_t)lane & 7u) ^ (row & 7u)) << 4));
    }
    asm volatile("" ::: "memory");
  }
}

// Copy of an accumulator out of its AGPR at this point of the program.  Without it the register
// allocator copies all 256 accumulators to VGPRs where the main loop ends, which does not fit
// and spills.
__device__ __forceinline__ float agpr_read(float x) {
  float y;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(y) : "a"(x));
  return y;
}
__device__ __forceinline__ void agpr_read16(const f32x16& a, float (&o)[16]) {
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = agpr_read(a[r]);
}

}  // namespace gemm
}  // namespace moe
