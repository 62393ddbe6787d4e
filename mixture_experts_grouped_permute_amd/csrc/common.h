// Shared device helpers for the gfx950 kernels: vector types, bf16 rounding,
// the OCP MXFP8 element/scale rule in integer arithmetic, wave reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxExperts = 256;

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// Round-to-nearest-even float32 -> bf16 bits (NaN kept quiet).  On the device this is
// gfx950's v_cvt_pk_bf16_f32 (round to nearest even under the default rounding mode);
// the host keeps the integer form.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__host__ __device__ inline uint16_t f32_to_bf16(float f) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint16_t, (__bf16)f);
#else
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
#endif
}

__host__ __device__ inline uint32_t pack_bf16x2(float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
#else
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
#endif
}

// ---------------------------------------------------------------------------
// OCP MXFP8 (E4M3FN elements, E8M0 shared exponent) in integer arithmetic so
// that the bytes do not depend on the float unit's denormal or rounding mode.
//   shared exponent s = floor(log2(amax)) - 8, clamped to [-127, 127]
//   code = E4M3FN(v / 2^s), round to nearest even, saturate to +-448,
//   zero keeps its sign.
// ---------------------------------------------------------------------------

// Shared exponent from the bit pattern of |amax| (a non-negative float).
__host__ __device__ inline int mx_shared_exp(float amax) {
  uint32_t u = __builtin_bit_cast(uint32_t, amax);
  int ef = (int)((u >> 23) & 0xFF);
  if (ef == 0) return -127;          // zero or subnormal amax: floor(log2) <= -127
  int s = ef - 127 - 8;
  return s < -127 ? -127 : s;        // ef <= 254 keeps s <= 119
}

// E4M3FN code of v / 2^s.
__host__ __device__ inline uint32_t mx_e4m3_code(float v, int s) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  uint32_t sign = (u >> 24) & 0x80u;
  int ef = (int)((u >> 23) & 0xFF);
  uint32_t mant = u & 0x7FFFFFu;
  int e;                             // unbiased exponent of bit 23 of `mant`
  if (ef == 0) {
    if (mant == 0) return sign;      // signed zero
    int lz = __builtin_clz(mant) - 8; // shift the leading one to bit 23
    mant <<= lz;
    e = -126 - lz;
  } else {
    mant |= 0x800000u;
    e = ef - 127;
  }
  int eq = e - s;                    // exponent of q = v / 2^s
  uint32_t code;
  if (eq >= -6) {
    // normal E4M3: keep 4 significant bits (1.mmm), round at bit 20
    uint32_t r = (mant + 0x7FFFFu + ((mant >> 20) & 1u)) >> 20;   // in [8, 16]
    if (r == 16) { r = 8; ++eq; }
    if (eq > 8 || (eq == 8 && r > 14)) return sign | 0x7Eu;      // saturate to 448
    code = ((uint32_t)(eq + 7) << 3) | (r - 8);
  } else {
    // subnormal E4M3: n * 2^-9 with n = RNE(mant * 2^(eq - 14))
    int sh = 14 - eq;                // >= 21
    uint32_t n;
    if (sh >= 32) {
      n = 0;
    } else {
      n = (mant + (1u << (sh - 1)) - 1u + ((mant >> sh) & 1u)) >> sh;   // n in [0, 8]
    }
    code = n;                        // n == 8 is the smallest normal, code 0x08
  }
  return sign | code;
}

// 4-byte pack of the codes of v[0..3] with exponent s.
// Device: the magnitudes are clamped to 448 * 2^s (exact: 448 = 1.75 * 2^8; with the scaling this
// is exactly the saturation rule), and gfx950's scaled conversion v_cvt_scalef32_pk_fp8_f32 divides
// by 2^s -- exact, a power of two -- and rounds to the nearest E4M3FN value, ties to even, keeping
// the sign of zero: the same code as mx_e4m3_code, two values per instruction.  The scale operand
// is 2^s as an fp32 bit pattern (s = -127 gives exponent field 0, which the conversion reads as
// 2^-127 like an E8M0 byte).  Without the clamp the conversion would give NaN past 448.
__host__ __device__ inline uint32_t mx_pack4(float a, float b, float c, float d, int s) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short short2_t __attribute__((ext_vector_type(2)));
  const float sc = __builtin_bit_cast(float, (uint32_t)(127 + s) << 23);                 // s in [-127, 119]
  const float lim = __builtin_bit_cast(float, ((uint32_t)(135 + s) << 23) | 0x600000u);   // 448 * 2^s
  auto q = [lim](float v) { return __builtin_amdgcn_fmed3f(v, -lim, lim); };
  short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32((short2_t){0, 0}, q(a), q(b), sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, q(c), q(d), sc, true);
  return __builtin_bit_cast(uint32_t, r);
#else
  return mx_e4m3_code(a, s) | (mx_e4m3_code(b, s) << 8) | (mx_e4m3_code(c, s) << 16) |
         (mx_e4m3_code(d, s) << 24);
#endif
}

// The same for four bf16 values packed two per word (w01 = values 0, 1; w23 = values 2, 3), without
// unpacking: the clamp of the magnitudes is an unsigned 16-bit min on the bit patterns (for
// non-negative bf16 values the integer order is the numeric order), and the conversion reads bf16.
__device__ inline uint32_t mx_pack4_bf16(uint32_t w01, uint32_t w23, int s) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef short short2_t __attribute__((ext_vector_type(2)));
  typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const float sc = __builtin_bit_cast(float, (uint32_t)(127 + s) << 23);
  const uint32_t l16 = ((uint32_t)(135 + s) << 7) | 0x60u;                               // 448 * 2^s in bf16
  const ushort2_t lim = __builtin_bit_cast(ushort2_t, l16 | (l16 << 16));
  auto clamp = [lim](uint32_t w) {
    const ushort2_t m = __builtin_elementwise_min(__builtin_bit_cast(ushort2_t, w & 0x7FFF7FFFu), lim);
    return __builtin_bit_cast(bf16x2_t, __builtin_bit_cast(uint32_t, m) | (w & 0x80008000u));
  };
  short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16((short2_t){0, 0}, clamp(w01), sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, clamp(w23), sc, true);
  return __builtin_bit_cast(uint32_t, r);
#else
  (void)w01;
  (void)w23;
  (void)s;
  return 0;
#endif
}

// The largest magnitude of the 2 n bf16 values packed in w[0..n-1], as an fp32 (bit patterns of
// non-negative bf16 values order as the values do).
template <int n>
__device__ inline float bf16_amax(const uint32_t* w) {
  typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
  ushort2_t m = __builtin_bit_cast(ushort2_t, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int i = 1; i < n; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(ushort2_t, w[i] & 0x7FFF7FFFu));
  const uint32_t h = m[0] > m[1] ? m[0] : m[1];
  return __builtin_bit_cast(float, h << 16);
}

// ---------------------------------------------------------------------------
// wave64 helpers
// ---------------------------------------------------------------------------
__device__ inline float wave_xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

__device__ inline uint64_t lanemask_lt() {
  int lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <typename T>
__device__ inline T* ptr_add_bytes(T* p, size_t bytes) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + bytes);
}

}  // namespace moe
