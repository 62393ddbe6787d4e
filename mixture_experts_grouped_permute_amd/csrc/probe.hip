// Matrix-core issue rate probe: the ceiling the grouped GEMMs' main loops are compared against.
//
// Every wave (one per SIMD, 256 workgroups of 4 waves) issues `iters` rounds of 16 MFMAs into 16
// independent 32 x 32 fp32 accumulators -- the accumulator count and instruction the GEMM tiles
// use -- with operands held in registers: no memory or LDS traffic, no dependent MFMA closer than
// 16 instructions apart.  Each wave's first lane records the shader-clock cycles (s_memtime) of
// the loop, so the caller gets cycles per MFMA (the issue cost of one instruction) and, with a
// host timer around the launch, the clock the chip ran at under this load.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8p __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef int32_t i32x4p __attribute__((ext_vector_type(4)));   // a buffer descriptor, 4 SGPRs

// Pseudo-random operand bits: Knuth's multiplicative hash of the counter (2^32 / golden ratio),
// then two of Marsaglia's xorshift32 steps (shifts 13, 17, 5).
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x *= 0x9E3779B9u;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
  }
  return x;
}

// kKind: 0 MFMA-scale 32x32x64 E4M3 with per-lane E8M0 scale registers (the MXFP8 GEMMs), 1 the
// same with constant scales, 2 MFMA 32x32x16 bf16 (the BF16 GEMMs) -- one operand pair for all
// 16 MFMAs, a few distinct values; 3 (bf16) and 4 (E4M3 with scale registers): the GEMM tiles'
// pattern, 4 A and 4 B fragments of pseudo-random values, MFMA q of a round multiplying A q / 4 by
// B q % 4, so that the operands change from one MFMA to the next as in the GEMMs
template <int kKind>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_probe_kernel(float* sink, uint64_t* cycles, int iters) {
  f32x16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  const int tid = threadIdx.x;
  i32x8p a, b;
  bf16x8p ab, bb;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    // E4M3 bytes of moderate magnitude (no NaN code): 0x38 + small offsets
    a[r] = 0x38383838 + ((tid + r) & 7);
    b[r] = 0x30303030 + ((tid * 3 + r) & 7);
    ab[r] = (__bf16)(float)((tid + r) & 15);
    bb[r] = (__bf16)(float)(r + 1);
  }
  int sa = 127, sb = 127 + (tid & 1);
  // opaque to the compiler, so the loop cannot be folded
  asm volatile("" : "+v"(a), "+v"(b), "+v"(sa), "+v"(sb), "+v"(ab), "+v"(bb));
  // kinds 3 and 4: pseudo-random fragments; bf16 values of either sign with exponents 2^-7 .. 2^7
  // and random mantissas, E4M3 bytes of either sign with exponent fields 0 .. 14 (no NaN code)
  bf16x8p fa[4], fb[4];
  i32x8p ga[4], gb[4];
  int gsa[4], gsb[4];
  if constexpr (kKind >= 3) {
    const uint32_t seed = (uint32_t)(blockIdx.x * 256 + tid) * 64u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const uint32_t ha = probe_hash(seed + (uint32_t)(i * 16 + r)), hb = probe_hash(seed + (uint32_t)(i * 16 + 8 + r));
        if constexpr (kKind == 3) {
          fa[i][r] = __builtin_bit_cast(__bf16, (uint16_t)((ha & 0x807Fu) | ((120u + (ha >> 16) % 15u) << 7)));
          fb[i][r] = __builtin_bit_cast(__bf16, (uint16_t)((hb & 0x807Fu) | ((120u + (hb >> 16) % 15u) << 7)));
        } else {
          ga[i][r] = (int)(ha & 0xF7F7F7F7u);
          gb[i][r] = (int)(hb & 0xF7F7F7F7u);
        }
      }
      gsa[i] = 120 + (int)(probe_hash(seed + 100u + (uint32_t)i) & 7u);
      gsb[i] = 120 + (int)(probe_hash(seed + 200u + (uint32_t)i) & 7u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(fa[i]), "+v"(fb[i]), "+v"(ga[i]), "+v"(gb[i]), "+v"(gsa[i]), "+v"(gsb[i]));
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (kKind == 0)
        acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[q], 0, 0, 0, sa, 0, sb);
      else if constexpr (kKind == 1)
        acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[q], 0, 0, 0, 127, 0, 127);
      else if constexpr (kKind == 2)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[q], 0, 0, 0);
      else if constexpr (kKind == 3)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[q & 3], fa[q >> 2], acc[q], 0, 0, 0);
      else
        acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(gb[q & 3], ga[q >> 2], acc[q], 0, 0, 0, gsb[q & 3], 0,
                                                                 gsa[q >> 2]);
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  sink[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) cycles[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

// LDS fill-rate probe: each of 256 workgroups (one per CU) loads 64 KB per stage straight into
// LDS with the GEMMs' direct-to-LDS loads (16 bytes per lane, 1 KB per wave and instruction, 16
// instructions per wave and stage), two stages in flight, a barrier per stage, nothing else.  XCD
// x (workgroup b: x = b % 8, slot j = b / 8) reads the region [x * region, (x + 1) * region) of the
// buffer; stage s of slot j, with sharer group g = j % 4 and sharer m = j / 4, reads
//   pattern 0, 1: the 64 KB chunk (s + 7 j) mod (region / 64 KB) -- every workgroup its own data
//     (pattern 0 on a 2 MB region that stays in L2, pattern 1 on 64 MB that streams from HBM);
//   pattern 2: chunk (4 s + g) mod ... -- 8 workgroups share each chunk in lockstep (64 MB);
//   pattern 3: the GEMM operands' access with the same sharing: 512 rows of 4 KB, row block
//     (4 (s / 32) + g) mod (region / 2 MB), 128-byte slice s mod 32 of each row (64 MB).
__device__ __forceinline__ void probe_lds_load16(const i32x4p& vs, uint32_t lds, uint32_t voff) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" : : "s"(l), "v"(voff), "s"(vs) : "memory", "m0");
}

template <int kPattern>
__global__ __launch_bounds__(256) void load_probe_kernel(const uint8_t* base, uint32_t region, int stages,
                                                         uint64_t* cycles) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 65536];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t xcd = blockIdx.x & 7u, slot = blockIdx.x >> 3;
  const uint32_t g = slot & 3u;
  const uint64_t a = reinterpret_cast<uint64_t>(base + (size_t)xcd * region);
  i32x4p vs;
  vs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  vs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  vs[2] = __builtin_amdgcn_readfirstlane((int)region);
  vs[3] = 0x00020000;
  const uint32_t nchunk = region / 65536u, nblock = region / (512u * 4096u);
  const uint32_t lbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)(__attribute__((address_space(3))) void*)lds);
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int s = 0; s < stages; ++s) {
    const uint32_t b = (uint32_t)s & 1u;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      uint32_t off;
      if constexpr (kPattern == 3) {
        const uint32_t rb = ((uint32_t)s / 32u * 4u + g) % nblock;
        const uint32_t row = (uint32_t)wave * 128u + (uint32_t)q * 8u + (uint32_t)(lane >> 3);
        off = rb * 512u * 4096u + row * 4096u + ((uint32_t)s % 32u) * 128u + (uint32_t)(lane & 7) * 16u;
      } else {
        const uint32_t chunk = kPattern == 2 ? ((uint32_t)s * 4u + g) % nchunk : ((uint32_t)s + slot * 7u) % nchunk;
        off = chunk * 65536u + (uint32_t)wave * 16384u + (uint32_t)q * 1024u + (uint32_t)lane * 16u;
      }
      probe_lds_load16(vs, lbase + b * 65536u + (uint32_t)wave * 16384u + (uint32_t)q * 1024u, off);
    }
    __builtin_amdgcn_s_waitcnt((16 & 0xF) | ((16 >> 4) << 14) | (0x7 << 4) | (0xF << 8));   // vmcnt(16)
    __syncthreads();
  }
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));                                        // vmcnt(0)
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (tid == 0) cycles[blockIdx.x] = t1 - t0;
}

}  // namespace

extern "C" {

size_t moe_load_probe_bytes(void) { return (size_t)8 * 64 * 1048576; }

moe_status moe_load_probe(int pattern, int stages, const void* buf, size_t bytes, uint64_t* cycles, void* stream) {
  if (pattern < 0 || pattern > 3 || stages <= 0 || stages > (1 << 16) || !buf || !cycles ||
      bytes < moe_load_probe_bytes())
    return MOE_ERR_INVALID_ARG;
  const uint32_t region = pattern == 0 ? 2u * 1048576u : 64u * 1048576u;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  if (pattern == 0) hipLaunchKernelGGL(load_probe_kernel<0>, dim3(256), dim3(256), 0, st, b, region, stages, cycles);
  else if (pattern == 1) hipLaunchKernelGGL(load_probe_kernel<1>, dim3(256), dim3(256), 0, st, b, region, stages, cycles);
  else if (pattern == 2) hipLaunchKernelGGL(load_probe_kernel<2>, dim3(256), dim3(256), 0, st, b, region, stages, cycles);
  else hipLaunchKernelGGL(load_probe_kernel<3>, dim3(256), dim3(256), 0, st, b, region, stages, cycles);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

int moe_probe_workgroups(void) { return 256; }

moe_status moe_mfma_probe(int kind, int iters, float* sink, uint64_t* cycles, void* stream) {
  if (kind < 0 || kind > 4 || iters <= 0 || iters > (1 << 20) || !sink || !cycles) return MOE_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(256), block(256);
  if (kind == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, st, sink, cycles, iters);
  else if (kind == 1) hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, st, sink, cycles, iters);
  else if (kind == 2) hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, st, sink, cycles, iters);
  else if (kind == 3) hipLaunchKernelGGL(mfma_probe_kernel<3>, grid, block, 0, st, sink, cycles, iters);
  else hipLaunchKernelGGL(mfma_probe_kernel<4>, grid, block, 0, st, sink, cycles, iters);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
