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

// kKind: 0 MFMA-scale 32x32x64 E4M3 with per-lane E8M0 scale registers (the MXFP8 GEMMs), 1 the
// same with constant scales, 2 MFMA 32x32x16 bf16 (the BF16 GEMMs)
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
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (kKind == 0)
        acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[q], 0, 0, 0, sa, 0, sb);
      else if constexpr (kKind == 1)
        acc[q] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[q], 0, 0, 0, 127, 0, 127);
      else
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[q], 0, 0, 0);
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

}  // namespace

extern "C" {

int moe_probe_workgroups(void) { return 256; }

moe_status moe_mfma_probe(int kind, int iters, float* sink, uint64_t* cycles, void* stream) {
  if (kind < 0 || kind > 2 || iters <= 0 || iters > (1 << 20) || !sink || !cycles) return MOE_ERR_INVALID_ARG;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(256), block(256);
  if (kind == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, grid, block, 0, st, sink, cycles, iters);
  else if (kind == 1) hipLaunchKernelGGL(mfma_probe_kernel<1>, grid, block, 0, st, sink, cycles, iters);
  else hipLaunchKernelGGL(mfma_probe_kernel<2>, grid, block, 0, st, sink, cycles, iters);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // extern "C"
