// Un-permute / combine kernels for gfx950.
//
// Forward (page "BioNeMo Uses Grouped Kernels and MXFP8", Figure 1: the k
// expert outputs of a token are combined as a weighted sum; the weights were
// already applied to h by ScaledSwiGLU, so this is a plain sum):
//   out[t] = sum_j z[row_id_map[t*k + j]]   (fp32, slot order, rounded once)
// The same kernel sums dx_perm into dx in the backward.  A wave owns one token
// and streams its k source rows with 16-byte loads.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

template <bool kInF32, bool kOutF32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ z, int64_t T, int64_t H, int k,
                                                        const int32_t* __restrict__ row_id_map,
                                                        void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) rows[j] = j < k ? row_id_map[t * k + j] : -1;
  // bf16 input: two 512-column passes at a time, so a lane has 2 k loads in flight
  constexpr int kU = kInF32 ? 1 : 2;
  for (int64_t c0 = (int64_t)lane * 8; c0 < H; c0 += 512 * kU) {
    float acc[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k || rows[j] < 0) continue;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + 512 * u;
        if (c >= H) continue;
        const int64_t o = (int64_t)rows[j] * H + c;
        if (kInF32) {
          const float4* s = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(z) + o);
          float4 a = s[0], b = s[1];
          acc[u][0] += a.x; acc[u][1] += a.y; acc[u][2] += a.z; acc[u][3] += a.w;
          acc[u][4] += b.x; acc[u][5] += b.y; acc[u][6] += b.z; acc[u][7] += b.w;
        } else {
          u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(z) + o);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[u][2 * i] += bf16_to_f32((uint16_t)(w[i] & 0xFFFF));
            acc[u][2 * i + 1] += bf16_to_f32((uint16_t)(w[i] >> 16));
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t c = c0 + 512 * u;
      if (c >= H) continue;
      const int64_t o = t * H + c;
      if (kOutF32) {
        float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o);
        d[0] = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
        d[1] = make_float4(acc[u][4], acc[u][5], acc[u][6], acc[u][7]);
      } else {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + o) = w;
      }
    }
  }
}

// dz[r] = bf16(dy[src_index[r] / k]) for the rows of valid experts (rows past offsets[E] untouched).
template <bool kF32>
__global__ __launch_bounds__(256) void gather_kernel(const void* __restrict__ x, int64_t R, int64_t H, int k,
                                                       const int32_t* __restrict__ src_index,
                                                       const int32_t* __restrict__ offsets, int E,
                                                       void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R || r >= offsets[E]) return;
  const int64_t t = src_index[r] / k;
  uint16_t* dst = reinterpret_cast<uint16_t*>(out) + r * H;
  // four 512-column chunks loaded before any is stored: several loads in flight per lane
  constexpr int kBatch = 4;
  for (int64_t c0 = (int64_t)lane * 8; c0 < H; c0 += 512 * kBatch) {
    u32x4 w[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t c = c0 + 512 * b;
      if (c >= H) continue;
      if (kF32) {
        const float4* s4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(x) + t * H + c);
        const float4 a = s4[0], d = s4[1];
        w[b] = u32x4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(d.x, d.y), pack_bf16x2(d.z, d.w)};
      } else {
        w[b] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(x) + t * H + c);
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int64_t c = c0 + 512 * b;
      if (c < H) *reinterpret_cast<u32x4*>(dst + c) = w[b];
    }
  }
}

// dprob[t, j] = sum over parts of partial[row, part], row = row_id_map[t*k + j] (fixed order).
__global__ __launch_bounds__(256) void dprob_kernel(const float* __restrict__ partial, int parts,
                                                      const int32_t* __restrict__ row_id_map, int64_t Tk,
                                                      float* __restrict__ dprob) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= Tk) return;
  const int r = row_id_map[p];
  float s = 0.f;
  if (r >= 0)
    for (int q = 0; q < parts; ++q) s += partial[(int64_t)r * parts + q];
  dprob[p] = s;
}

// The same sum with k fixed at compile time: each pass issues the loads of all k source rows before
// the first add, instead of a load-and-wait per row behind the runtime row loop's branches (which
// made k round trips per pass).  A row slot holding no row (-1), or a column past H, loads row 0,
// column 0 and is left out of the sum by a select, so every slot's result is the runtime loop's.
template <bool kInF32, bool kOutF32, int kK>
__global__ __launch_bounds__(256) void combine_k_kernel(const void* __restrict__ z, int64_t T, int64_t H,
                                                          const int32_t* __restrict__ row_id_map,
                                                          void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[kK];
#pragma unroll
  for (int j = 0; j < kK; ++j) rows[j] = row_id_map[t * kK + j];
  constexpr int kU = kInF32 ? 1 : 2;
  for (int64_t c0 = (int64_t)lane * 8; c0 < H; c0 += 512 * kU) {
    bool ok[kK][kU];
    u32x4 w[kK][kU][kInF32 ? 2 : 1];
#pragma unroll
    for (int j = 0; j < kK; ++j)
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t c = c0 + 512 * u;
        ok[j][u] = rows[j] >= 0 && c < H;
        const int64_t o = ok[j][u] ? (int64_t)rows[j] * H + c : 0;
        if constexpr (kInF32) {
          const u32x4* s = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(z) + o);
          w[j][u][0] = s[0];
          w[j][u][1] = s[1];
        } else {
          w[j][u][0] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(z) + o);
        }
      }
    float acc[kU][8];
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[u][i] = 0.f;
#pragma unroll
    for (int j = 0; j < kK; ++j)
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float v[8];
        if constexpr (kInF32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // (a vector element copied out first: bit-casting the element expression in place
            // read element 0)
            const uint32_t lo = w[j][u][0][i], hi = w[j][u][1][i];
            v[i] = __builtin_bit_cast(float, lo);
            v[4 + i] = __builtin_bit_cast(float, hi);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_to_f32((uint16_t)(w[j][u][0][i] & 0xFFFF));
            v[2 * i + 1] = bf16_to_f32((uint16_t)(w[j][u][0][i] >> 16));
          }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = ok[j][u] ? acc[u][i] + v[i] : acc[u][i];
      }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t c = c0 + 512 * u;
      if (c >= H) continue;
      const int64_t o = t * H + c;
      if (kOutF32) {
        float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + o);
        d[0] = make_float4(acc[u][0], acc[u][1], acc[u][2], acc[u][3]);
        d[1] = make_float4(acc[u][4], acc[u][5], acc[u][6], acc[u][7]);
      } else {
        u32x4 wo;
#pragma unroll
        for (int i = 0; i < 4; ++i) wo[i] = pack_bf16x2(acc[u][2 * i], acc[u][2 * i + 1]);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(out) + o) = wo;
      }
    }
  }
}

template <bool kInF32, bool kOutF32>
void launch_combine_t(dim3 grid, const void* z, int64_t T, int64_t H, int k, const int32_t* row_id_map, void* out,
                      hipStream_t st) {
  switch (k) {
    case 1: combine_k_kernel<kInF32, kOutF32, 1><<<grid, 256, 0, st>>>(z, T, H, row_id_map, out); break;
    case 2: combine_k_kernel<kInF32, kOutF32, 2><<<grid, 256, 0, st>>>(z, T, H, row_id_map, out); break;
    case 4: combine_k_kernel<kInF32, kOutF32, 4><<<grid, 256, 0, st>>>(z, T, H, row_id_map, out); break;
    case 6: combine_k_kernel<kInF32, kOutF32, 6><<<grid, 256, 0, st>>>(z, T, H, row_id_map, out); break;
    case 8: combine_k_kernel<kInF32, kOutF32, 8><<<grid, 256, 0, st>>>(z, T, H, row_id_map, out); break;
    default: combine_kernel<kInF32, kOutF32><<<grid, 256, 0, st>>>(z, T, H, k, row_id_map, out); break;
  }
}

}  // namespace

hipError_t launch_combine(const void* z, bool z_f32, int64_t T, int64_t H, int k, const int32_t* row_id_map,
                          void* out, bool out_f32, hipStream_t st) {
  dim3 grid((unsigned)((T + 3) / 4));
  if (T == 0) return hipSuccess;
  if (z_f32) {
    if (out_f32) launch_combine_t<true, true>(grid, z, T, H, k, row_id_map, out, st);
    else launch_combine_t<true, false>(grid, z, T, H, k, row_id_map, out, st);
  } else {
    if (out_f32) launch_combine_t<false, true>(grid, z, T, H, k, row_id_map, out, st);
    else launch_combine_t<false, false>(grid, z, T, H, k, row_id_map, out, st);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, bool f32, int64_t R, int64_t H, int k, const int32_t* src_index,
                              const int32_t* offsets, int E, void* out, hipStream_t st) {
  dim3 grid((unsigned)((R + 3) / 4));
  if (R == 0) return hipSuccess;
  if (f32) gather_kernel<true><<<grid, 256, 0, st>>>(x, R, H, k, src_index, offsets, E, out);
  else gather_kernel<false><<<grid, 256, 0, st>>>(x, R, H, k, src_index, offsets, E, out);
  return hipGetLastError();
}

hipError_t launch_dprob_reduce(const float* partial, int64_t R, int parts, const int32_t* row_id_map, int64_t T,
                               int k, float* dprob, hipStream_t st) {
  (void)R;
  const int64_t Tk = T * k;
  if (Tk == 0) return hipSuccess;
  dprob_kernel<<<(unsigned)((Tk + 255) / 256), 256, 0, st>>>(partial, parts, row_id_map, Tk, dprob);
  return hipGetLastError();
}

}  // namespace moe
