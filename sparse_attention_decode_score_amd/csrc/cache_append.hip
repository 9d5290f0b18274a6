// Cache append: quantises the step's new tokens into the paged caches by physical slot.
//
// The vLLM Kimi K3.1 Pro page stores one FP8 index key per token, 132 bytes with its scale
// ("What changed in Kimi K3.1 Pro"), and a 576-byte FP8 latent ("Packed KV cache for three
// kinds of state"); its fused indexer front writes the new token's index key in the same
// kernel as the query prep ("Fused low-latency decode for DSA layers").  Here the append is
// its own small launch (the projections that produce the key and latent are outside this
// library).  Per token: the key's fp32 scale s = absmax / 448 (1 for an all-zero key) and
// codes E4M3(k / s), round to nearest even, saturating; the latent's codes E4M3(x / c) with
// the cache's per-tensor scale c.  Divisions are IEEE fp32 (correctly rounded), so the
// codes are exactly those of the same arithmetic on the host.
//
// An MXFP4 index-key cache (the page's opt-in 68-byte key, "Native MXFP4 indexer") takes the
// OCP microscaling recipe instead: per block of 32 dims the E8M0 scale 2^e with
// e = floor(log2 absmax) - 2 (2 = E2M1's largest exponent), at least -127 (2^0 for an
// all-zero block), and each element the E2M1 value nearest |x| / 2^e, ties to the even code,
// saturating at 6, with x's sign bit.  Scaling by a power of two is exact wherever the
// rounding can matter, so the codes are exact too.
//
// One wave per token: lane l converts key dims 2l, 2l+1 (two bytes of one 16-byte column
// block of an E4M3 page; one byte of 32-dim block l / 16 of an MXFP4 page) and latent dims
// 8l .. 8l+7 plus 512 + l.
#include "dsa_device.hpp"
#include "dsa_index_core.hpp"  // the MXFP4 page layout (kMxPageKeyBytes)
#include "dsa_internal.hpp"

namespace dsa {

namespace {

__device__ __forceinline__ float sat448(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }

// floor(log2 a) of a finite a > 0, from its bits (fp32 subnormals included)
__device__ __forceinline__ int floor_log2_bits(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ex = (int)(u >> 23);
  return ex != 0 ? ex - 127 : (31 - __clz(u & 0x7FFFFFu)) - 149;
}

// E2M1 nibble of x / 2^e (|x / 2^e| < 8): nearest of 0, .5, 1, 1.5, 2, 3, 4, 6, ties to the
// even code, saturating at 6; the sign bit is x's
__device__ __forceinline__ uint32_t e2m1_code(float x, float inv_scale) {
  const float a = fabsf(x) * inv_scale;
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(x) >> 28) & 8u);
}

template <bool MX>
__global__ __launch_bounds__(256) void cache_append_kernel(
    int n_tok, const int32_t* __restrict__ slots, const uint16_t* __restrict__ key,
    const uint16_t* __restrict__ lat, float lat_scale, uint8_t* __restrict__ key_pages,
    int64_t key_page_stride, uint8_t* __restrict__ lat_pages, int64_t lat_page_stride) {
  const int i = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (i >= n_tok) return;  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int slot = slots[i];
  if (slot < 0) return;
  const int64_t page = slot >> 6;
  const int o = slot & (kPage - 1);
  if (MX && key) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(key + (int64_t)i * kIdxDim)[lane];
    const float x0 = bf16_lo(w), x1 = bf16_hi(w);
    float a = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) a = fmaxf(a, __shfl_xor(a, m, 64));  // the 32-dim block
    const int e = a > 0.f ? max(floor_log2_bits(a) - 2, -127) : 0;
    const float inv = ldexpf(1.0f, -e);  // 2^-127 .. 2^127: a normal fp32
    uint8_t* pg = key_pages + page * key_page_stride;
    pg[(lane >> 4) * 1024 + o * 16 + (lane & 15)] = (uint8_t)(e2m1_code(x0, inv) | (e2m1_code(x1, inv) << 4));
    if ((lane & 15) == 0) pg[kMxPageKeyBytes + 4 * o + (lane >> 4)] = (uint8_t)(e + 127);
  } else if (key) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(key + (int64_t)i * kIdxDim)[lane];
    const float x0 = bf16_lo(w), x1 = bf16_hi(w);
    const float a = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
    const float s = a > 0.f ? a / kE4M3Max : 1.0f;
    const uint32_t c = cvt2_e4m3(sat448(x0 / s), sat448(x1 / s));
    uint8_t* pg = key_pages + page * key_page_stride;
    const int d = 2 * lane;
    *reinterpret_cast<uint16_t*>(pg + (d >> 4) * 1024 + o * 16 + (d & 15)) = (uint16_t)c;
    if (lane == 0) *reinterpret_cast<float*>(pg + kIdxPageKeyBytes + 4 * o) = s;
  }
  if (lat) {
    const uint16_t* src = lat + (int64_t)i * kLatDim;
    const v4i raw = *reinterpret_cast<const v4i*>(src + 8 * lane);
    uint32_t c[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w0 = (uint32_t)raw[2 * h], w1 = (uint32_t)raw[2 * h + 1];
      c[h] = cvt4_e4m3(sat448(bf16_lo(w0) / lat_scale), sat448(bf16_hi(w0) / lat_scale),
                       sat448(bf16_lo(w1) / lat_scale), sat448(bf16_hi(w1) / lat_scale));
    }
    uint8_t* row = lat_pages + page * lat_page_stride + (int64_t)o * kLatDim;
    *reinterpret_cast<v2i*>(row + 8 * lane) = v2i{(int)c[0], (int)c[1]};
    const float xt = __uint_as_float((uint32_t)src[kVDim + lane] << 16);
    row[kVDim + lane] = (uint8_t)(cvt2_e4m3(sat448(xt / lat_scale), 0.f) & 0xFFu);
  }
}

}  // namespace

hipError_t launch_cache_append(int n_tok, const int32_t* slots, const uint16_t* key,
                               const uint16_t* lat, float lat_scale, uint8_t* key_pages,
                               int64_t key_page_stride, uint8_t* lat_pages,
                               int64_t lat_page_stride, bool mx_keys, hipStream_t st) {
  if (n_tok == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_tok + 3) / 4));
  if (mx_keys)
    hipLaunchKernelGGL(cache_append_kernel<true>, grid, dim3(256), 0, st, n_tok, slots, key, lat,
                       lat_scale, key_pages, key_page_stride, lat_pages, lat_page_stride);
  else
    hipLaunchKernelGGL(cache_append_kernel<false>, grid, dim3(256), 0, st, n_tok, slots, key, lat,
                       lat_scale, key_pages, key_page_stride, lat_pages, lat_page_stride);
  return hipGetLastError();
}

}  // namespace dsa
