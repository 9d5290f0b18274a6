// Device-side helpers shared by the gfx950 kernels of the DSA decode path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kPage = 64;
constexpr int kIdxHeads = 32;
constexpr int kIdxDim = 128;
constexpr int kIdxPageKeyBytes = kPage * kIdxDim;  // 8192, then 64 fp32 scales
constexpr int kMlaHeads = 96;
constexpr int kLatDim = 576;
constexpr int kVDim = 512;
constexpr float kE4M3Max = 448.0f;

#define DSA_LDS __attribute__((address_space(3)))

// D[32x32] += A[32x64] * B[64x32], E4M3 x E4M3 -> fp32.
// Lane l holds A row (l % 32), B column (l % 32), 32 consecutive k starting at 32*(l/32).
// Output register i of lane l is D[8*(i/4) + 4*(l/32) + i%4][l % 32].
__device__ __forceinline__ v16f mfma_32x32x64_fp8(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Two fp32 -> two E4M3 codes in the low 16 bits (round to nearest even; inputs within +-448).
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
// Four fp32 -> one dword of four E4M3 codes (byte j = code of x_j).
__device__ __forceinline__ uint32_t cvt4_e4m3(float x0, float x1, float x2, float x3) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, lo, true);
}

// Smallest power-of-two exponent e with absmax <= 448 * 2^e (0 when absmax == 0).
// All comparisons are exact: ldexpf by an integer is exact in this range.
__device__ __forceinline__ int pow2_scale_exp(float absmax) {
  if (!(absmax > 0.0f)) return 0;
  int E;
  (void)frexpf(absmax, &E);
  int e = E - 12;
#pragma unroll 1
  while (absmax > ldexpf(kE4M3Max, e)) ++e;
  return e;
}

// Order-preserving map of an fp32 score to uint32 (larger key = larger score);
// -0.0 maps like +0.0 and NaN to 0, the lowest key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

}  // namespace dsa
