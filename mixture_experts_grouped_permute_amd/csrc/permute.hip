// Token permutation by expert: histogram -> prefix sum -> stable scatter ->
// row copy (bf16 cast or MXFP8 row quantization), for gfx950.
//
// The grouped linear of page "BioNeMo Uses Grouped Kernels and MXFP8"
// (Grouping fragmented expert workloads) consumes each expert's tokens as one
// contiguous group described by split_sizes; this file builds that grouping.
// Rows inside a group are in ascending (token, slot) order, so every output
// index is unique and the permutation is deterministic.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// K1: per-block expert histogram over the chunk of kPermTokens tokens = kPermTokens * k
// consecutive (token, slot) ids.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t* __restrict__ idx, int64_t R, int k, int E,
                                                          int32_t* __restrict__ block_counts,
                                                          int32_t* __restrict__ block_bad) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int nbad;
  if (threadIdx.x == 0) nbad = 0;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int chunk = kPermTokens * k;
  int64_t base = (int64_t)blockIdx.x * chunk;
  int bad = 0;
  for (int i = threadIdx.x; i < chunk; i += blockDim.x) {
    int64_t p = base + i;
    if (p < R) {
      int e = idx[p];
      if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);
      else bad = 1;
    }
  }
  if (bad) atomicOr(&nbad, 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) block_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
  if (threadIdx.x == 0) block_bad[blockIdx.x] = nbad;
}

// ---------------------------------------------------------------------------
// K2: split_sizes, offsets and the per-(block, expert) base rows.  One workgroup of 1024
// threads: expert e's column of block counts is cut into S = 1024 / E slices and thread
// (e, s), e fastest so that a slice's threads read each block's row of counts contiguously,
// sums its slice.  Laid out expert-major (position e * S + s), the exclusive prefix sum of the
// slice sums is at once expert e's first row plus the rows of its earlier slices, so one
// block-wide scan gives every slice's base; the thread then writes the running base of every
// block in its slice.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ block_counts,
                                                           const int32_t* __restrict__ block_bad, int nb, int E,
                                                           int32_t* __restrict__ err_flag,
                                                           int32_t* __restrict__ split_sizes,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ block_base) {
  __shared__ int slice_sum[1024];
  __shared__ int slice_base[1024];
  __shared__ int wave_base[16];
  __shared__ int total, bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = 1024 / E;                 // >= 4 slices per expert (E <= 256)
  const int e = tid % E, sl = tid / E;
  const bool act = sl < S;                // exactly the threads tid < E * S
  const int per = (nb + S - 1) / S;
  const int b0 = min(nb, sl * per), b1 = min(nb, b0 + per);
  if (tid == 0) bad = 0;
  // a slice's counts in batches of 8 blocks, all 8 loads issued before the first add (a block past
  // the slice reads the slice's last one and adds 0)
  auto count_at = [&](int b) { return block_counts[(int64_t)b * E + e]; };
  int s = 0;
  if (act)
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = count_at(min(b + u, b1 - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u) s += b + u < b1 ? v[u] : 0;
    }
  // (e, sl) -> e * S + sl maps the active threads onto [0, E * S); the positions above hold 0
  slice_sum[act ? e * S + sl : tid] = act ? s : 0;
  int bd = 0;
  for (int b = tid; b < nb; b += 1024) bd |= block_bad[b];
  __syncthreads();
  if (bd) atomicOr(&bad, 1);
  // block-wide exclusive scan of slice_sum: within each wave, then over the 16 wave totals
  const int x = slice_sum[tid];
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  if (lane == 63) wave_base[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? wave_base[lane] : 0;
    int wi = w;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const int y = __shfl_up(wi, d, 64);
      if (lane >= d) wi += y;
    }
    if (lane < 16) wave_base[lane] = wi - w;   // each lane rewrites only the entry it read
  }
  __syncthreads();
  slice_base[tid] = wave_base[wave] + inc - x;
  if (tid == 1023) total = wave_base[wave] + inc;
  __syncthreads();
  if (act) {
    if (sl == 0) {
      const int first = slice_base[e * S];
      split_sizes[e] = (e + 1 < E ? slice_base[(e + 1) * S] : total) - first;
      offsets[e] = first;
    }
    int run = slice_base[e * S + sl];
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = count_at(min(b + u, b1 - 1));
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (b + u < b1) {
          block_base[(int64_t)(b + u) * E + e] = run;
          run += v[u];
        }
    }
  }
  if (tid == 0) {
    offsets[E] = total;
    err_flag[0] = bad;   // the flag describes this call only
  }
}

// ---------------------------------------------------------------------------
// K3: stable scatter of the indices.  Block b walks its chunk in rounds of 256
// ids; inside a round a (token, slot) id's rank among equal experts is the
// number of equal ids in lower lanes of its wave (ballot match on the 8 bits of
// the expert id) plus the counts of earlier waves, on top of the running count.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                             const float* __restrict__ prob, int64_t R, int k, int E,
                                                             const int32_t* __restrict__ block_base,
                                                             int32_t* __restrict__ row_id_map,
                                                             int32_t* __restrict__ src_index,
                                                             float* __restrict__ prob_perm) {
  __shared__ int run[kMaxExperts];
  __shared__ int wcnt[4][kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int e = tid; e < E; e += 256) run[e] = block_base[(int64_t)blockIdx.x * E + e];
  const int chunk = kPermTokens * k;
  int64_t base = (int64_t)blockIdx.x * chunk;
  for (int r = 0; r * 256 < chunk; ++r) {   // the chunk's ids in rounds of 256
    for (int i = tid; i < 4 * kMaxExperts; i += 256) (&wcnt[0][0])[i] = 0;
    __syncthreads();
    int64_t p = base + r * 256 + tid;
    int e = -1;
    const bool in_chunk = r * 256 + tid < chunk;
    if (in_chunk && p < R) {
      e = idx[p];
      if ((unsigned)e >= (unsigned)E) e = -1;
    }
    uint64_t peers = __ballot(e >= 0);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      uint64_t b = __ballot(e >= 0 && ((e >> bit) & 1));
      peers &= ((e >> bit) & 1) ? b : ~b;
    }
    int rank = __popcll(peers & lanemask_lt());
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (e >= 0) {
      int row = run[e] + rank;
      for (int w = 0; w < wave; ++w) row += wcnt[w][e];
      row_id_map[p] = row;
      src_index[row] = (int32_t)p;
      if (prob_perm) prob_perm[row] = prob[p];
    } else if (in_chunk && p < R) {
      row_id_map[p] = -1;
    }
    __syncthreads();
    for (int x = tid; x < E; x += 256) run[x] += wcnt[0][x] + wcnt[1][x] + wcnt[2][x] + wcnt[3][x];
    // the next round's clear of wcnt happens after this barrier
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// K4: copy each token row once from X and write it to its k permuted rows,
// rounding to bf16 or quantizing to MXFP8 on the way.  One wave per token;
// a lane owns 8 consecutive values per 512-column chunk (4 lanes per MXFP8
// block), and loads kBatch chunks before it converts and stores any, so each
// lane keeps several 16-byte loads in flight.
// ---------------------------------------------------------------------------
template <bool kInF32, bool kMx>
__global__ __launch_bounds__(256) void perm_rows_kernel(const void* __restrict__ x, int64_t T, int64_t H, int k,
                                                          const int32_t* __restrict__ row_id_map,
                                                          void* __restrict__ out, uint8_t* __restrict__ out_scales) {
  // 8 chunks in flight (a 4096-wide bf16 row at once) for the plain copy; the MXFP8 path's extra
  // registers make 4 the faster choice there
  constexpr int kBatch = kMx ? 4 : 8;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) rows[j] = j < k ? row_id_map[t * k + j] : -1;
  // MXFP8 scale bytes: with H % 128 == 0 (and a 4-byte aligned scale array) every 16-lane group
  // covers 4 whole blocks and their 4 bytes are 4-byte aligned, so the group's first lane stores
  // them as one word; otherwise one byte per block
  const bool pack = ((H / 32) & 3) == 0 && ((reinterpret_cast<uintptr_t>(out_scales) & 3u) == 0);
  for (int64_t c0 = 0; c0 < H; c0 += 512 * kBatch) {
    float v[kBatch][8];
    // H % 32 == 0 keeps every MXFP8 block's 4 lanes together (all in or all past the end)
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t c = c0 + 512 * b + lane * 8;
      if (c >= H) continue;
      if (kInF32) {
        const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + t * H + c);
        const float4 a = src[0], d = src[1];
        v[b][0] = a.x; v[b][1] = a.y; v[b][2] = a.z; v[b][3] = a.w;
        v[b][4] = d.x; v[b][5] = d.y; v[b][6] = d.z; v[b][7] = d.w;
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + t * H + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[b][2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFF));
          v[b][2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t c = c0 + 512 * b + lane * 8;
      if (c >= H) continue;
      if (!kMx) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(v[b][2 * i], v[b][2 * i + 1]);
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          if (j >= k || rows[j] < 0) continue;
          *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + (int64_t)rows[j] * H + c) = o;
        }
      } else {
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(v[b][i]));
        am = wave_xor_max(am, 1);
        am = wave_xor_max(am, 2);
        const int s = mx_shared_exp(am);
        u32x2 o;
        o[0] = mx_pack4(v[b][0], v[b][1], v[b][2], v[b][3], s);
        o[1] = mx_pack4(v[b][4], v[b][5], v[b][6], v[b][7], s);
        // the scale bytes of the 16-lane group's 4 blocks (lanes 16 w + 4 i hold block 4 w + i);
        // the group is wholly in range here when pack holds
        uint32_t word = 0;
        if (pack) {
          const int g16 = lane & ~15;
#pragma unroll
          for (int i = 0; i < 4; ++i) word |= ((uint32_t)(__shfl(s, g16 + 4 * i, 64) + 127) & 0xFFu) << (8 * i);
        }
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
          if (j >= k || rows[j] < 0) continue;
          *reinterpret_cast<u32x2*>(reinterpret_cast<uint8_t*>(out) + (int64_t)rows[j] * H + c) = o;
          uint8_t* sc = out_scales + (int64_t)rows[j] * (H / 32) + c / 32;
          if (pack) {
            if ((lane & 15) == 0) *reinterpret_cast<uint32_t*>(sc) = word;
          } else if ((lane & 3) == 0) {
            *sc = (uint8_t)(s + 127);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_permute_indices(const int32_t* idx, const float* prob, int64_t T, int k, int E,
                                  int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                                  int32_t* src_index, float* prob_perm, int32_t* err_flag, int32_t* block_counts,
                                  int32_t* block_base, hipStream_t st, bool counts_ready) {
  const int64_t R = T * k;
  const int nb = perm_blocks(T);
  int32_t* block_bad = block_counts + (int64_t)nb * E;
  if (!counts_ready) perm_hist_kernel<<<nb, 256, 0, st>>>(idx, R, k, E, block_counts, block_bad);
  perm_scan_kernel<<<1, 1024, 0, st>>>(block_counts, block_bad, nb, E, err_flag, split_sizes, offsets, block_base);
  perm_scatter_kernel<<<nb, 256, 0, st>>>(idx, prob, R, k, E, block_base, row_id_map, src_index, prob_perm);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const void* x, bool x_f32, int64_t T, int64_t H, int k, const int32_t* row_id_map,
                               void* out, uint8_t* out_scales, bool mx, hipStream_t st) {
  dim3 grid((unsigned)((T + 3) / 4));
  if (x_f32) {
    if (mx) perm_rows_kernel<true, true><<<grid, 256, 0, st>>>(x, T, H, k, row_id_map, out, out_scales);
    else perm_rows_kernel<true, false><<<grid, 256, 0, st>>>(x, T, H, k, row_id_map, out, out_scales);
  } else {
    if (mx) perm_rows_kernel<false, true><<<grid, 256, 0, st>>>(x, T, H, k, row_id_map, out, out_scales);
    else perm_rows_kernel<false, false><<<grid, 256, 0, st>>>(x, T, H, k, row_id_map, out, out_scales);
  }
  return hipGetLastError();
}

}  // namespace moe
