// Shared pieces of the grouped GEMMs for gfx950: buffer-resource loads, the
// swizzled LDS layout, the in-kernel per-expert tile scheduler, the 256x256
// MFMA tile core (BF16 32x32x16 and MX-scaled FP8 32x32x64) and the rotated
// LDS staging layout of the epilogues.
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
constexpr int kScaleBytes = 2 * 256 * 4;        // A + B scale words per stage (MXFP8)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
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

// Same rotation for a 1024-byte-per-row tile (c16 in 0..63).
__device__ __forceinline__ uint32_t epi_off_wide(int m, int c16) {
  const int b = c16 >> 3, low = c16 & 7;
  return (uint32_t)(m * 1024 + ((b << 3) + ((low + 2 * b + m) & 7)) * 16);
}

// Byte offset of 16-byte chunk c16 (0..31) of row m in a 512-byte-per-row LDS
// staging tile.  Chunks are rotated within each group of 8 by (2 * group + m),
// so both the column-wise writes from the MFMA layout and the row-wise reads
// of whole groups touch 8 different bank groups per 8 lanes.
__device__ __forceinline__ uint32_t epi_off(int m, int c16) {
  const int b = c16 >> 3, low = c16 & 7;
  return (uint32_t)(m * 512 + ((b << 3) + ((low + 2 * b + m) & 7)) * 16);
}

// ---------------------------------------------------------------------------
// One K-pass of a 256x256 tile.  kFc1 selects the B row map (gate/up halves).
// ---------------------------------------------------------------------------
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
// K units of 128 bytes per part of a split tile, at least: a split costs two short extra launches,
// so it only pays for long tiles
constexpr int kMinSplitUnits = 16;
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

// Transpose an 8x8 block of bf16: v[r] holds 8 consecutive values of row r,
// w[c] receives column c (8 values, one per row) -- v_perm_b32 picks the low or
// high halves of two words at a time.
__device__ __forceinline__ void transpose8x8_b16(const u32x4 v[8], u32x4 w[8]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[c][q] = __builtin_amdgcn_perm(v[2 * q + 1][c >> 1], v[2 * q][c >> 1], sel);
  }
}

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

  // Fragments of one MFMA K-substep: 4 A and 4 B operands (+ scales).
  struct Frag {
    typename std::conditional<kMx, i32x8, bf16x8>::type a[4], b[4];
    int sa[4], sb[4];
  };

  static constexpr int kSub = kMx ? 2 : 4;   // MFMA K-substeps per 128-byte K step

  __device__ __forceinline__ void load_frag(Frag& f, int kk, const uint8_t* sA, const uint8_t* sB,
                                            const uint32_t* sAs, const uint32_t* sBs, int wm, int wn,
                                            int lane) const {
    const int r32 = lane & 31, g = lane >> 5;
    if constexpr (!kMx) {
      const uint32_t ch = (uint32_t)(kk * 2 + g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f.a[i] = *reinterpret_cast<const bf16x8*>(sA + swz(wm * 128 + i * 32 + r32, ch));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f.b[j] = *reinterpret_cast<const bf16x8*>(sB + swz(brow(wn, j) + r32, ch));
    } else {
      const uint32_t c0 = (uint32_t)(kk * 4 + g), c1 = (uint32_t)(kk * 4 + 2 + g);
      const int sh = 8 * (2 * kk + g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + r32;
        u32x4 lo = *reinterpret_cast<const u32x4*>(sA + swz(row, c0));
        u32x4 hi = *reinterpret_cast<const u32x4*>(sA + swz(row, c1));
        f.a[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        f.sa[i] = (int)(sAs[row] >> sh);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = brow(wn, j) + r32;
        u32x4 lo = *reinterpret_cast<const u32x4*>(sB + swz(row, c0));
        u32x4 hi = *reinterpret_cast<const u32x4*>(sB + swz(row, c1));
        f.b[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        f.sb[j] = (int)(sBs[row] >> sh);
      }
    }
  }

  // MFMAs of fragment rows i in [i0, i0 + 2)
  __device__ __forceinline__ void mma_half(const Frag& f, int i0) {
#pragma unroll
    for (int i = i0; i < i0 + 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (!kMx)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0, f.sa[i], 0,
                                                                        f.sb[j]);
      }
  }

  __device__ __forceinline__ void mma(const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (!kMx)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0, 0, f.sa[i], 0,
                                                                        f.sb[j]);
      }
  }

  // BF16 fragments of K step kk with either operand stored MN-major (transposing reads) or
  // K-major (swz layout).
  template <bool kAMN, bool kBMN>
  __device__ __forceinline__ void load_frag_x(Frag& f, int kk, const uint8_t* sA, const uint8_t* sB, int wm,
                                              int wn, int lane) const {
    const int r32 = lane & 31, g = lane >> 5;
    const uint32_t ch = (uint32_t)(kk * 2 + g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (kAMN) f.a[i] = load_mn_frag(sA, wm * 128 + i * 32, kk, lane);
      else f.a[i] = *reinterpret_cast<const bf16x8*>(sA + swz(wm * 128 + i * 32 + r32, ch));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kBMN) f.b[j] = load_mn_frag(sB, brow(wn, j), kk, lane);
      else f.b[j] = *reinterpret_cast<const bf16x8*>(sB + swz(brow(wn, j) + r32, ch));
    }
  }

  template <bool kAMN, bool kBMN>
  __device__ __forceinline__ void compute_x(const uint8_t* sA, const uint8_t* sB, int wm, int wn, int lane) {
    static_assert(!kMx, "MN-major operands are bf16 only");
    Frag f0, f1;
    load_frag_x<kAMN, kBMN>(f0, 0, sA, sB, wm, wn, lane);
#pragma unroll
    for (int kk = 0; kk < kSub; kk += 2) {
      load_frag_x<kAMN, kBMN>(f1, kk + 1, sA, sB, wm, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
      mma(f0);
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 2 < kSub) load_frag_x<kAMN, kBMN>(f0, kk + 2, sA, sB, wm, wn, lane);
      __builtin_amdgcn_sched_barrier(0);
      mma(f1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // All substeps of one LDS stage.  BF16 fragments are double-buffered in
  // registers (2 x 32 VGPRs); the MXFP8 ones are twice as wide, so they are
  // single-buffered and the compiler overlaps the reads with the MFMAs.
  __device__ __forceinline__ void compute(const uint8_t* sA, const uint8_t* sB, const uint32_t* sAs,
                                          const uint32_t* sBs, int wm, int wn, int lane) {
    if constexpr (kMx) {
#pragma unroll
      for (int kk = 0; kk < kSub; ++kk) {
        Frag f;
        load_frag(f, kk, sA, sB, sAs, sBs, wm, wn, lane);
        mma(f);
      }
    } else {
      Frag f0, f1;
      load_frag(f0, 0, sA, sB, sAs, sBs, wm, wn, lane);
#pragma unroll
      for (int kk = 0; kk < kSub; kk += 2) {
        load_frag(f1, kk + 1, sA, sB, sAs, sBs, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
        mma(f0);
        __builtin_amdgcn_sched_barrier(0);
        if (kk + 2 < kSub) load_frag(f0, kk + 2, sA, sB, sAs, sBs, wm, wn, lane);
        __builtin_amdgcn_sched_barrier(0);
        mma(f1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

}  // namespace gemm
}  // namespace moe
