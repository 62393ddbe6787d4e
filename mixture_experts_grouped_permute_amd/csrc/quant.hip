// MXFP8 block quantization kernels for gfx950 (the Quantize step of Figure 4
// on page "BioNeMo Uses Grouped Kernels and MXFP8"; format from Reducing
// memory pressure with MXFP8, Figure 3: E4M3 values plus one E8M0 scale per
// 32 consecutive values).  The element and scale rule (mx_shared_exp,
// mx_e4m3_code in common.h) is integer arithmetic, so the bytes are exact.
//
// Row-wise kernels stream 16-byte loads: a lane owns 8 consecutive values, 4
// lanes share one 32-value block and reduce its amax with two xor shuffles.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ void load8(const void* x, bool f32, int64_t off, float v[8]) {
  if (f32) {
    const float4* s = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + off);
    float4 a = s[0], b = s[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFF));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
}

// 8-value group g of a [rows, cols] matrix: row = g / (cols/8), col = 8 * (g % (cols/8)).
// Every lane handles groups tid, tid + stride, ...  cols % 32 == 0, so the 4 lanes of
// one 32-value block are always consecutive lanes of one wave and step together.
template <bool kF32>
__global__ __launch_bounds__(256) void mx_rows_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ scales) {
  const int64_t groups = rows * (cols / 8);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // the loop bound is uniform per 4-lane block because groups % 4 == 0
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups; gi += stride) {
    const int64_t off = gi * 8;
    float v[8];
    load8(x, kF32, off, v);
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[i]));
    am = wave_xor_max(am, 1);
    am = wave_xor_max(am, 2);
    const int s = mx_shared_exp(am);
    u32x2 o;
    o[0] = mx_pack4(v[0], v[1], v[2], v[3], s);
    o[1] = mx_pack4(v[4], v[5], v[6], v[7], s);
    *reinterpret_cast<u32x2*>(q + off) = o;
    // scale bytes: the blocks of 16 consecutive groups are 4 consecutive bytes, 4-byte aligned in
    // an aligned array (gi of the group's first lane is a multiple of 16); a group wholly in range
    // stores them as one word from its first lane, the last partial group one byte per block
    const int64_t g0 = gi & ~(int64_t)15;
    if (g0 + 16 <= groups && (reinterpret_cast<uintptr_t>(scales) & 3u) == 0) {
      const int l16 = (int)(threadIdx.x & 63) & ~15;
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) word |= ((uint32_t)(__shfl(s, l16 + 4 * i, 64) + 127) & 0xFFu) << (8 * i);
      if ((threadIdx.x & 15) == 0) *reinterpret_cast<uint32_t*>(scales + off / 32) = word;
    } else if ((threadIdx.x & 3) == 0) {
      scales[off / 32] = (uint8_t)(s + 127);
    }
  }
}

// Weight tables: blockIdx.y = expert.  Skips experts with no tokens when asked.
struct WTab {
  const uint16_t* w[kMaxExperts];
};

__global__ __launch_bounds__(256) void mx_weights_kernel(const WTab tab, int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ scales,
                                                           const int32_t* __restrict__ skip_if_empty) {
  const int e = blockIdx.y;
  if (skip_if_empty && skip_if_empty[e] == 0) return;
  const uint16_t* x;
#if defined(__HIP_DEVICE_COMPILE__)
  {
    const uint16_t* const* t = reinterpret_cast<const uint16_t* const*>(
        reinterpret_cast<const char*>(__builtin_amdgcn_kernarg_segment_ptr()));
    x = t[e];
  }
#else
  x = tab.w[e];
#endif
  const int64_t n = rows * cols;
  uint8_t* qe = q + (int64_t)e * n;
  uint8_t* se = scales + (int64_t)e * (n / 32);
  // a lane quantizes 16 consecutive values (two 16-byte loads, one 16-byte store of codes); the
  // 2 lanes of a 32-value block are neighbours and reduce its amax with one xor shuffle
  const int64_t groups = n / 16;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups; gi += stride) {
    const int64_t off = gi * 16;
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(x + off);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(x + off + 8);
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)(w0[i] & 0xFFFF));
      v[2 * i + 1] = bf16_to_f32((uint16_t)(w0[i] >> 16));
      v[8 + 2 * i] = bf16_to_f32((uint16_t)(w1[i] & 0xFFFF));
      v[8 + 2 * i + 1] = bf16_to_f32((uint16_t)(w1[i] >> 16));
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    am = wave_xor_max(am, 1);
    const int sx = mx_shared_exp(am);
    u32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = mx_pack4(v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3], sx);
    *reinterpret_cast<u32x4*>(qe + off) = o;
    if ((threadIdx.x & 1) == 0) se[off / 32] = (uint8_t)(sx + 127);
  }
}

// Column-wise quantization with per-segment restart, transposed output.
// The padded token axis (each segment padded to a multiple of seg_align rows) is cut into
// 32-row blocks.  A workgroup of 256 lanes takes 4 consecutive blocks (128 padded rows) of 64
// columns:
//   * the source row of each padded row (or none: padding, or past the last segment) goes to LDS;
//   * the 128 x 64 tile is loaded with 16-byte row-contiguous loads (zero for rows with no
//     source) and kept in LDS as loaded (bf16 input: its raw 16 KB, which leaves room for more
//     workgroups per CU than an fp32 copy; f32 input: fp32);
//   * lane (c, b) = (t % 64, t / 64) reduces block b of column c down its 32 rows, stores its
//     scale byte, and puts its 32 codes in an LDS staging area [column][padded row];
//   * the staged codes go out as 16-byte pieces with consecutive lanes along one output row, so
//     a store instruction writes 8 whole 128-byte stretches of the transposed output.
constexpr int kColRows = 128;   // padded rows per workgroup
//
// src_index (optional): row r of the segmented matrix is row src_index[r] / src_k of x (the
// permuted rows of a token-major x, e.g. the gradient rows of the backward read straight from dY).

template <bool kF32>
__global__ __launch_bounds__(256) void mx_cols_kernel(const void* __restrict__ x, int64_t rows, int64_t cols,
                                                        const int32_t* __restrict__ goff, int num_groups,
                                                        int64_t rows_pad, uint8_t* __restrict__ q,
                                                        uint8_t* __restrict__ scales, int seg_align,
                                                        const int32_t* __restrict__ src_index, int src_k) {
  __shared__ int s_pad[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 1];
  using TT = typename std::conditional<kF32, float, uint16_t>::type;
  __shared__ int s_src[kColRows];
  __shared__ __attribute__((aligned(16))) TT tile[kColRows][64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (!goff) {  // a single segment covering every row
    if (t == 0) {
      s_off[0] = 0;
      s_off[1] = (int)rows;
      s_pad[0] = 0;
      s_pad[1] = (int)((rows + seg_align - 1) / seg_align * seg_align);
    }
    num_groups = 1;
  } else if (wave == 0) {
    // padded segment starts: one wave scans the groups 64 at a time
    int carry = 0;
    for (int g0 = 0; g0 < num_groups; g0 += 64) {
      const int g = g0 + lane;
      int pad = 0;
      if (g < num_groups) {
        // offsets are the caller's device data: clamped into [0, rows] and non-decreasing, so
        // that a bad array cannot take the kernel outside its buffers
        const int o = min(max(goff[g], 0), (int)rows);
        const int o1 = min(max(goff[g + 1], o), (int)rows);
        s_off[g] = o;
        pad = (o1 - o + seg_align - 1) / seg_align * seg_align;
      }
      int inc = pad;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(inc, d, 64);
        if (lane >= d) inc += v;
      }
      if (g < num_groups) s_pad[g] = carry + inc - pad;
      carry += __shfl(inc, 63, 64);
    }
    if (lane == 0) {
      s_off[num_groups] = min(max(goff[num_groups], 0), (int)rows);
      s_pad[num_groups] = carry;
    }
  }
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kColRows;   // first padded row of this workgroup
  const int64_t ptotal = s_pad[num_groups];
  // padded rows past the last segment, up to rows_pad, are written as padding too (codes 0, scale
  // bytes 0): a reader may then take a whole group of scale bytes past its segment's end and find
  // finite scales there
  if (p0 >= rows_pad) return;                           // uniform
  if (t < kColRows) {
    const int64_t pr = p0 + t;
    int src = -1;
    if (pr < ptotal) {
      int lo = 0, hi = num_groups - 1;                  // largest g with s_pad[g] <= pr
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_pad[mid] <= pr) lo = mid; else hi = mid - 1;
      }
      const int64_t sr = s_off[lo] + (pr - s_pad[lo]);
      const int64_t end = lo + 1 < num_groups ? min(s_off[lo + 1], (int)rows) : s_off[num_groups];
      if (sr < end && sr < rows) src = (int)sr;
      if (src >= 0 && src_index) src = src_index[src] / src_k;
    }
    s_src[t] = src;
  }
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  // the tile, in chunks of 8 values: all four loads are issued before any is used (a chunk with no
  // source reads x's first chunk unconditionally and is replaced by zeros, so that no branch
  // separates the loads); rows == 0 leaves every chunk without a source
  if (rows > 0) {
    [[maybe_unused]] float v[4][8];
    [[maybe_unused]] u32x4 wr[4];
    bool ok[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int id = t + 256 * it;                      // 1024 chunks: 128 rows x 8 chunks of 8 columns
      const int rr = id >> 3, ck = id & 7;
      const int64_t col = c0 + 8 * ck;
      const int src = s_src[rr];
      ok[it] = src >= 0 && col < cols;
      const int64_t off = ok[it] ? (int64_t)src * cols + col : 0;
      if constexpr (kF32) load8(x, true, off, v[it]);
      else wr[it] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + off);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int id = t + 256 * it;
      const int rr = id >> 3, ck = id & 7;
      if constexpr (kF32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[rr][8 * ck + e] = ok[it] ? v[it][e] : 0.f;
      } else {
        *reinterpret_cast<u32x4*>(&tile[rr][8 * ck]) = ok[it] ? wr[it] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int id = t + 256 * it;
      const int rr = id >> 3, ck = id & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) tile[rr][8 * ck + e] = 0;
    }
  }
  __syncthreads();
  // codes staged [column][padded row], padded by 16 bytes per column against bank conflicts
  __shared__ __attribute__((aligned(16))) uint8_t ostage[64][kColRows + 16];
  const int64_t c = c0 + lane;
  const int64_t pblk = p0 + 32 * wave;                  // padded row of this lane's block
  const bool valid = c < cols && pblk + 32 <= rows_pad;
  float v[32];
  float am = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if constexpr (kF32) v[r] = tile[32 * wave + r][lane];
    else v[r] = bf16_to_f32(tile[32 * wave + r][lane]);
    am = fmaxf(am, fabsf(v[r]));
  }
  const int s = mx_shared_exp(am);
  u32x4 o0, o1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o0[i] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], s);
    o1[i] = mx_pack4(v[16 + 4 * i], v[16 + 4 * i + 1], v[16 + 4 * i + 2], v[16 + 4 * i + 3], s);
  }
  *reinterpret_cast<u32x4*>(&ostage[lane][32 * wave]) = o0;
  *reinterpret_cast<u32x4*>(&ostage[lane][32 * wave + 16]) = o1;
  if (valid) scales[c * (rows_pad / 32) + pblk / 32] = (uint8_t)(s + 127);
  __syncthreads();
  // piece pc (16 padded rows) of column lc; 8 pieces per column, 2 per 32-row block
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = t + 256 * it;
    const int lc = id >> 3, pc = id & 7;
    const int64_t cc = c0 + lc;
    const int64_t pb = p0 + 32 * (pc >> 1);
    if (cc < cols && pb + 32 <= rows_pad)
      *reinterpret_cast<u32x4*>(q + cc * rows_pad + p0 + 16 * pc) =
          *reinterpret_cast<const u32x4*>(&ostage[lc][16 * pc]);
  }
}

// Weight tables quantized column-wise into the transposed layout (the backward's dgrad operands:
// blocks of 32 along the rows of each matrix), and with kRows also row-wise (the forward's: blocks
// of 32 along the columns, mx_weights_kernel's layout and rule), from one read of the bf16 weights.
// A workgroup takes a 128 x 128 tile of matrix blockIdx.z (rows % 32 == 0, cols % 32 == 0;
// matrices with skip[e] == 0 are left alone):
//   * the tile is loaded with 16-byte loads, 16 lanes per 256-byte row, and kept in LDS as bf16
//     (rows padded by 16 bytes, so that the row-wise reads below hit distinct banks);
//   * row-wise: thread t takes row t / 2, columns 64 (t % 2) + [0, 64) -- two blocks, 64 code bytes
//     and 2 scale bytes, so the two threads of a row write its whole 128-byte stretch;
//   * column-wise: thread t takes column t % 128, rows 64 (t / 128) + [0, 64) -- two blocks along
//     the rows; their codes go to an LDS staging area [column][row] (rows padded by 16 bytes),
//     from which consecutive lanes store a column's 128 bytes of the transposed output, 8 whole
//     128-byte stretches per store instruction; the two scale bytes go out as one 2-byte word.
// Matrix e's outputs: qt + e * cols * rows [cols, rows], st + e * cols * rows / 32 [cols, rows / 32],
// qr + e * rows * cols [rows, cols], sr + e * rows * cols / 32 [rows, cols / 32].
constexpr int kWT = 128;
template <bool kRows>
__global__ __launch_bounds__(256) void mx_wt_kernel(const WTab tab, int64_t rows, int64_t cols, uint8_t* __restrict__ qt,
                                                    uint8_t* __restrict__ st, uint8_t* __restrict__ qr,
                                                    uint8_t* __restrict__ sr, const int32_t* __restrict__ skip) {
  const int e = blockIdx.z;
  if (skip && skip[e] == 0) return;
#if defined(__HIP_DEVICE_COMPILE__)
  const uint16_t* x = reinterpret_cast<const uint16_t* const*>(
      reinterpret_cast<const char*>(__builtin_amdgcn_kernarg_segment_ptr()))[e];
#else
  const uint16_t* x = tab.w[e];
#endif
  qt += (int64_t)e * cols * rows;
  st += (int64_t)e * cols * (rows / 32);
  if constexpr (kRows) {
    qr += (int64_t)e * rows * cols;
    sr += (int64_t)e * rows * (cols / 32);
  }
  __shared__ __attribute__((aligned(16))) uint16_t tile[kWT][kWT + 8];
  __shared__ __attribute__((aligned(16))) uint8_t ostage[kWT][kWT + 16];
  const int t = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kWT, c0 = (int64_t)blockIdx.y * kWT;
  {
    // all eight loads before any is used: a chunk past the matrix reads its first chunk
    // unconditionally and is replaced by zeros, so that no branch separates the loads
    u32x4 w[8];
    bool ok[8];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int id = t + 256 * it;                     // 128 rows x 16 chunks of 8 values
      const int rr = id >> 4, ck = id & 15;
      const int64_t row = r0 + rr, col = c0 + 8 * ck;
      ok[it] = row < rows && col < cols;
      w[it] = *reinterpret_cast<const u32x4*>(x + (ok[it] ? row * cols + col : 0));
    }
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int id = t + 256 * it;
      const int rr = id >> 4, ck = id & 15;
      *reinterpret_cast<u32x4*>(&tile[rr][8 * ck]) = ok[it] ? w[it] : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();
  // 32 values -> their scale byte and 32 codes (two 16-byte words)
  auto quant32 = [](const float (&v)[32], u32x4& o0, u32x4& o1) -> uint8_t {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
    const int sx = mx_shared_exp(am);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o0[i] = mx_pack4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], sx);
      o1[i] = mx_pack4(v[16 + 4 * i], v[16 + 4 * i + 1], v[16 + 4 * i + 2], v[16 + 4 * i + 3], sx);
    }
    return (uint8_t)(sx + 127);
  };
  if constexpr (kRows) {
    const int rr = t >> 1, hb = t & 1;
    const int64_t row = r0 + rr;
    if (row < rows) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int64_t cb = c0 + 64 * hb + 32 * b;
        if (cb >= cols) continue;
        float v[32];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x4 u = *reinterpret_cast<const u32x4*>(&tile[rr][64 * hb + 32 * b + 8 * k]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[8 * k + 2 * i] = bf16_to_f32((uint16_t)(u[i] & 0xFFFF));
            v[8 * k + 2 * i + 1] = bf16_to_f32((uint16_t)(u[i] >> 16));
          }
        }
        u32x4 o0, o1;
        const uint8_t sb = quant32(v, o0, o1);
        uint8_t* d = qr + row * cols + cb;
        *reinterpret_cast<u32x4*>(d) = o0;
        *reinterpret_cast<u32x4*>(d + 16) = o1;
        sr[row * (cols / 32) + cb / 32] = sb;
      }
    }
  }
  {
    const int cl = t & 127, rb = 64 * (t >> 7);
    const int64_t col = c0 + cl;
    uint32_t sw = 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float v[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) v[r] = bf16_to_f32(tile[rb + 32 * b + r][cl]);
      u32x4 o0, o1;
      sw |= (uint32_t)quant32(v, o0, o1) << (8 * b);
      *reinterpret_cast<u32x4*>(&ostage[cl][rb + 32 * b]) = o0;
      *reinterpret_cast<u32x4*>(&ostage[cl][rb + 32 * b + 16]) = o1;
    }
    // rows % 32 == 0: both blocks are in or past the matrix together only when rows - row0 >= 64
    const int64_t row = r0 + rb;
    if (col < cols && row < rows) {
      uint8_t* sp = st + col * (rows / 32) + row / 32;
      if (row + 64 <= rows && ((rows / 32) & 1) == 0) {
        *reinterpret_cast<uint16_t*>(sp) = (uint16_t)sw;   // 2-byte aligned: row / 32 and rows / 32 even
      } else {
        sp[0] = (uint8_t)sw;
        if (row + 64 <= rows) sp[1] = (uint8_t)(sw >> 8);
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int id = t + 256 * it;                     // 128 columns x 8 pieces of 16 rows
      const int lc = id >> 3, pc = id & 7;
      const int64_t cc = c0 + lc, rr = r0 + 16 * pc;
      if (cc < cols && rr < rows)
        *reinterpret_cast<u32x4*>(qt + cc * rows + rr) = *reinterpret_cast<const u32x4*>(&ostage[lc][16 * pc]);
    }
  }
}

// ---------------------------------------------------------------------------
// Per-tensor-scaled FP8 (FP8 beside MXFP8 on page "BioNeMo Uses Grouped Kernels
// and MXFP8", Reducing memory pressure with MXFP8: the same E4M3 elements with a
// coarser scale -- here one fp32 scale per tensor).  A tensor is a row segment
// [offsets[g], offsets[g+1]) of a contiguous [rows, cols] matrix, or one matrix
// of a weight table.  Two passes: amax partials over each tensor (grid nb x G,
// part[g * nb + b]), then each block reduces its tensor's nb partials, forms
//   s = 448 / amax (fp32 division, correctly rounded; 1 for amax == 0; the
//       largest finite float if the quotient overflows)
// and stores E4M3FN(fp32(v * s)): the product clamped to +-448 (the saturation
// rule) and rounded by v_cvt_pk_fp8_f32 (nearest, ties to even, zero keeps its
// sign).  Max is order-free, so the result does not depend on the grid.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float pt_scale(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const float s = 448.0f / amax;
  return s > 3.402823466e38f ? 3.402823466e38f : s;
}

// the tensor of block row g: its first element and element count
template <bool kTab>
__device__ __forceinline__ void pt_range(const WTab& tab, const void* x, bool f32, const int32_t* offsets,
                                         int64_t rows, int64_t cols, int g, const void*& base, int64_t& first,
                                         int64_t& n) {
  if constexpr (kTab) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint16_t* const* t = reinterpret_cast<const uint16_t* const*>(
        reinterpret_cast<const char*>(__builtin_amdgcn_kernarg_segment_ptr()));
    base = t[g];
#else
    base = tab.w[g];
#endif
    first = 0;
    n = rows * cols;
  } else {
    (void)tab;
    (void)f32;
    // offsets are device data: clamped into [0, rows] and non-decreasing (memory-safe for any array)
    int64_t lo = offsets ? (int64_t)offsets[g] : 0, hi = offsets ? (int64_t)offsets[g + 1] : rows;
    lo = lo < 0 ? 0 : (lo > rows ? rows : lo);
    hi = hi < lo ? lo : (hi > rows ? rows : hi);
    base = x;
    first = lo * cols;
    n = (hi - lo) * cols;
  }
}

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = wave_xor_max(v, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

template <bool kF32, bool kTab>
__global__ __launch_bounds__(256) void pt_amax_kernel(const WTab tab, const void* x, const int32_t* offsets,
                                                       int64_t rows, int64_t cols, float* part) {
  __shared__ float red[4];
  const int g = blockIdx.y, nb = gridDim.x;
  const void* base;
  int64_t first, n;
  pt_range<kTab>(tab, x, kF32, offsets, rows, cols, g, base, first, n);
  float am = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n / 8; i += (int64_t)nb * 256) {
    float v[8];
    load8(base, kF32, first + i * 8, v);
#pragma unroll
    for (int c = 0; c < 8; ++c) am = fmaxf(am, fabsf(v[c]));
  }
  am = block_max(am, red);
  if (threadIdx.x == 0) part[g * nb + blockIdx.x] = am;
}

template <bool kF32, bool kTab>
__global__ __launch_bounds__(256) void pt_quant_kernel(const WTab tab, const void* x, const int32_t* offsets,
                                                        int64_t rows, int64_t cols, const float* part,
                                                        uint8_t* __restrict__ q, float* scales, float* inv,
                                                        const uint32_t* amax_in) {
  __shared__ float red[4];
  const int g = blockIdx.y, nb = gridDim.x;
  const void* base;
  int64_t first, n;
  pt_range<kTab>(tab, x, kF32, offsets, rows, cols, g, base, first, n);
  float am = 0.f;
  if (amax_in) {
    am = __builtin_bit_cast(float, amax_in[g]);
  } else {
    for (int i = threadIdx.x; i < nb; i += 256) am = fmaxf(am, part[g * nb + i]);
    am = block_max(am, red);
  }
  const float s = pt_scale(am);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    scales[g] = s;
    if (inv) inv[g] = 1.0f / s;
  }
  uint8_t* qg = q + (kTab ? (int64_t)g * n : first);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n / 8; i += (int64_t)nb * 256) {
    float v[8];
    load8(base, kF32, first + i * 8, v);
    auto c = [s](float a) { return __builtin_amdgcn_fmed3f(a * s, -448.0f, 448.0f); };
    u32x2 o;
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c(v[0]), c(v[1]), 0, false);
    o[0] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c(v[2]), c(v[3]), w, true);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c(v[4]), c(v[5]), 0, false);
    o[1] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c(v[6]), c(v[7]), w, true);
    *reinterpret_cast<u32x2*>(qg + i * 8) = o;
  }
}

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

int grid_for(int64_t groups) {
  int64_t b = (groups + 255) / 256;
  return (int)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

}  // namespace

hipError_t launch_mx_quant_rows(const void* x, bool x_f32, int64_t rows, int64_t cols, uint8_t* q,
                                uint8_t* scales, hipStream_t st) {
  const int64_t groups = rows * (cols / 8);
  if (groups == 0) return hipSuccess;
  if (x_f32) mx_rows_kernel<true><<<grid_for(groups), 256, 0, st>>>(x, rows, cols, q, scales);
  else mx_rows_kernel<false><<<grid_for(groups), 256, 0, st>>>(x, rows, cols, q, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_weights(const void* const* w, int E, int64_t rows, int64_t cols, uint8_t* q,
                                   uint8_t* scales, const int32_t* skip_if_empty, hipStream_t st) {
  WTab tab{};
  for (int e = 0; e < E; ++e) tab.w[e] = reinterpret_cast<const uint16_t*>(w[e]);
  const int64_t groups = rows * cols / 16;
  int gx = grid_for(groups);
  int per = (2048 + E - 1) / E;                 // about 2048 workgroups over all experts
  if (gx > per) gx = per < 1 ? 1 : per;
  mx_weights_kernel<<<dim3(gx, E), 256, 0, st>>>(tab, rows, cols, q, scales, skip_if_empty);
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(const void* x, bool x_f32, int64_t rows, int64_t cols, const int32_t* group_offsets,
                                int num_groups, int64_t rows_pad, uint8_t* q, uint8_t* scales, hipStream_t st,
                                int seg_align, const int32_t* src_index, int src_k) {
  dim3 grid((unsigned)((rows_pad + kColRows - 1) / kColRows), (unsigned)((cols + 63) / 64));
  if (grid.x == 0) return hipSuccess;
  if (x_f32)
    mx_cols_kernel<true><<<grid, 256, 0, st>>>(x, rows, cols, group_offsets, num_groups, rows_pad, q, scales,
                                               seg_align, src_index, src_k);
  else
    mx_cols_kernel<false><<<grid, 256, 0, st>>>(x, rows, cols, group_offsets, num_groups, rows_pad, q, scales,
                                                seg_align, src_index, src_k);
  return hipGetLastError();
}

hipError_t launch_mx_quant_weights_t(const void* const* w, int E, int64_t rows, int64_t cols, uint8_t* q,
                                     uint8_t* scales, const int32_t* skip_if_empty, hipStream_t st, uint8_t* q_rows,
                                     uint8_t* s_rows) {
  WTab tab{};
  for (int e = 0; e < E; ++e) tab.w[e] = reinterpret_cast<const uint16_t*>(w[e]);
  const dim3 grid((unsigned)((rows + kWT - 1) / kWT), (unsigned)((cols + kWT - 1) / kWT), (unsigned)E);
  if (grid.x == 0 || grid.y == 0 || E == 0) return hipSuccess;
  if (q_rows)
    mx_wt_kernel<true><<<grid, 256, 0, st>>>(tab, rows, cols, q, scales, q_rows, s_rows, skip_if_empty);
  else
    mx_wt_kernel<false><<<grid, 256, 0, st>>>(tab, rows, cols, q, scales, nullptr, nullptr, skip_if_empty);
  return hipGetLastError();
}

int pt_blocks(int G) {
  const int nb = 2048 / (G < 1 ? 1 : G);
  return nb < 1 ? 1 : (nb > 256 ? 256 : nb);
}

size_t pt_part_floats(int G) { return (size_t)G * (size_t)pt_blocks(G); }

hipError_t launch_pt_quant(const void* x, bool x_f32, int64_t rows, int64_t cols, const int32_t* offsets, int G,
                           uint8_t* q, float* scales, float* inv, float* part, hipStream_t st,
                           const uint32_t* amax_in) {
  if (G <= 0) return hipSuccess;
  const dim3 grid((unsigned)pt_blocks(G), (unsigned)G);
  WTab tab{};
  if (x_f32) {
    if (!amax_in) pt_amax_kernel<true, false><<<grid, 256, 0, st>>>(tab, x, offsets, rows, cols, part);
    pt_quant_kernel<true, false><<<grid, 256, 0, st>>>(tab, x, offsets, rows, cols, part, q, scales, inv, amax_in);
  } else {
    if (!amax_in) pt_amax_kernel<false, false><<<grid, 256, 0, st>>>(tab, x, offsets, rows, cols, part);
    pt_quant_kernel<false, false><<<grid, 256, 0, st>>>(tab, x, offsets, rows, cols, part, q, scales, inv, amax_in);
  }
  return hipGetLastError();
}

hipError_t launch_pt_quant_weights(const void* const* w, int E, int64_t rows, int64_t cols, uint8_t* q,
                                   float* scales, float* inv, float* part, hipStream_t st) {
  WTab tab{};
  for (int e = 0; e < E; ++e) tab.w[e] = reinterpret_cast<const uint16_t*>(w[e]);
  const dim3 grid((unsigned)pt_blocks(E), (unsigned)E);
  pt_amax_kernel<false, true><<<grid, 256, 0, st>>>(tab, nullptr, nullptr, rows, cols, part);
  pt_quant_kernel<false, true><<<grid, 256, 0, st>>>(tab, nullptr, nullptr, rows, cols, part, q, scales, inv, nullptr);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_u32_kernel<<<grid_for(n), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace moe
