// The lightning indexer's per-page arithmetic, shared by the scoring kernel and by the final
// top-k pass when it recomputes the scores of a group (the scores are then not stored), so
// that both produce bitwise the same fp32 score: the same query quantisation, the same
// MFMA sequence and the same head-reduction order.
//
// score[t] = sum_h w_h * sq_h * ReLU(q8_h . k8_t) * s_t, the head-weighted ReLU form of
// DeepSeek-V3.2's lightning indexer that the vLLM Kimi K3.1 Pro page defers to ("What changed
// in Kimi K3.1 Pro"), with fp32 accumulation ("Native MXFP4 indexer").
#pragma once

#include "dsa_device.hpp"

namespace dsa {

constexpr int kQRowStride = 144;  // LDS row stride of the FP8 query (128 + 16 pad: no bank conflicts)

struct KeyPage {
  v8i k[2][2];  // [half][k-block]
  float s;
};

// Keys are streamed once per step and never reused, so they are read with non-temporal
// loads: on gfx950 this lets a shuffled page stream run near the HBM rate instead of
// thrashing the L2 and the last-level cache (measured 6.5 vs 3.5 TB/s for this pattern).
__device__ __forceinline__ void load_key_page(KeyPage& kp, const uint8_t* base, int lane) {
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const uint8_t* tok = base + (32 * hf + n) * 16;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const v4i a = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tok + (4 * g + 2 * kb) * 1024));
      const v4i b = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tok + (4 * g + 2 * kb + 1) * 1024));
      kp.k[hf][kb] = v8i{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
  }
  kp.s = __builtin_nontemporal_load(reinterpret_cast<const float*>(base + kIdxPageKeyBytes + 4 * lane));
}

// ReLU as a signed-integer max on the float's bits: positive values keep their bits,
// negative values and -0.0 become +0.0.  One v_max_i32; a float max would first have to
// quiet possible signalling NaNs of the MFMA result (two instructions per value).
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

// Query prep of one (row, head, 16-dim part): 8 consecutive lanes hold the 8 parts of a
// head (raw: 16 bf16 values, hw: the head weight).  E4M3 codes of q / sq go to q8 (16 bytes),
// sq = one power of two per (row, head) from the head's absmax, and the lane of part 0
// writes w_h * sq to *w.
__device__ __forceinline__ void quantize_index_query_part(const v4i (&raw)[2], float hw,
                                                          int qpart, uint8_t* q8, float* w) {
  float x[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = bf16_lo((uint32_t)raw[0][j]);
    x[2 * j + 1] = bf16_hi((uint32_t)raw[0][j]);
    x[8 + 2 * j] = bf16_lo((uint32_t)raw[1][j]);
    x[8 + 2 * j + 1] = bf16_hi((uint32_t)raw[1][j]);
  }
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) am = fmaxf(am, fabsf(x[j]));
  am = fmaxf(am, __shfl_xor(am, 1, 64));
  am = fmaxf(am, __shfl_xor(am, 2, 64));
  am = fmaxf(am, __shfl_xor(am, 4, 64));
  const int e = pow2_scale_exp(am);
  const float inv = ldexpf(1.0f, -e);
  v4i c;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    c[j] = (int)cvt4_e4m3(x[4 * j] * inv, x[4 * j + 1] * inv, x[4 * j + 2] * inv,
                          x[4 * j + 3] * inv);
  *reinterpret_cast<v4i*>(q8) = c;
  if (qpart == 0) *w = hw * ldexpf(1.0f, e);
}

// Score of token `lane` of a key page for one query row: q8 is the row's [32][kQRowStride]
// FP8 query in LDS, w its 32 folded head weights in LDS.
//   D[head][token] = Q8[32 heads x 128] * K8^T[128 x 32 tokens]  (2 x v_mfma 32x32x64 per half)
// Output register i of lane l is head 8*(i/4) + 4*(l/32) + i%4 for token l%32 of the half;
// the head reduction is 16 in-register FMAs per half, then one permlane32 swap that gives
// lane l the two partial sums of token l of the page.
__device__ __forceinline__ float score_key_page(const uint8_t* q8, const float* w,
                                                const KeyPage& cur, int lane) {
  const int n = lane & 31, g = lane >> 5;
  const uint8_t* qa = q8 + n * kQRowStride + 64 * g;
  const v4i a0 = *reinterpret_cast<const v4i*>(qa);
  const v4i a1 = *reinterpret_cast<const v4i*>(qa + 16);
  const v4i a2 = *reinterpret_cast<const v4i*>(qa + 32);
  const v4i a3 = *reinterpret_cast<const v4i*>(qa + 48);
  const v8i A0 = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const v8i A1 = v8i{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
  const v16f z = {};
  v16f d0 = mfma_32x32x64_fp8(A0, cur.k[0][0], z);
  d0 = mfma_32x32x64_fp8(A1, cur.k[0][1], d0);
  v16f d1 = mfma_32x32x64_fp8(A0, cur.k[1][0], z);
  d1 = mfma_32x32x64_fp8(A1, cur.k[1][1], d1);
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const v4f wv = *reinterpret_cast<const v4f*>(w + 8 * a + 4 * g);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc0 = fmaf(wv[c], relu(d0[4 * a + c]), acc0);
      acc1 = fmaf(wv[c], relu(d1[4 * a + c]), acc1);
    }
  }
  // lanes 0..31: (half-0 partial, partner's half-0 partial); lanes 32..63: half 1
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0), __float_as_uint(acc1),
                                                   false, false);
  return (__uint_as_float(sw[0]) + __uint_as_float(sw[1])) * cur.s;
}

// ---------------------------------------------------------------------------------------
// MXFP4 index keys (68 B per token: the "Native MXFP4 indexer" of the K3.1 page, with its
// FP4 matrix instructions and FP32 accumulation).  Page of 4,352 B: block b (dims 32b ..
// 32b+31) of token o is 16 bytes of E2M1 codes at b * 1024 + o * 16 (byte j: dims 32b + 2j,
// low nibble, and 32b + 2j + 1); the E8M0 scale of block b is the byte at 4096 + 4 o + b.
constexpr int kMxPageKeyBytes = kPage * kIdxDim / 2;  // 4096
constexpr int kMxPageBytes = kMxPageKeyBytes + kPage * 4;  // 4352

// The scaled FP8 x FP4 MFMA of gfx950 takes, in lane (n, g) of a 32x32x64 product, 32 E2M1
// values of column n at k positions 16g .. 16g+15 (nibbles 0..15, low nibble first) and
// 32+16g .. 32+16g+15 (nibbles 16..31), scaled by that lane's E8M0 byte.  So chunk c of a key
// (dims 64c .. 64c+63) is laid out with lane g holding MX block 2c+g as it is stored, and the
// FP8 query lane g holds dims 64c+16g .. +15 and 64c+32+16g .. +15 in k order, which pairs
// every query dim with the same key dim.
struct KeyPageMx {
  v4i k[2][2];     // [half][chunk]: 16 bytes = MX block 2 * chunk + g of token l%32 of the half
  uint32_t sw[2];  // [half]: the four E8M0 block scales of that token
};

__device__ __forceinline__ void load_key_page(KeyPageMx& kp, const uint8_t* base, int lane) {
  const int n = lane & 31, g = lane >> 5;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const uint8_t* tok = base + (32 * hf + n) * 16;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      kp.k[hf][c] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(tok + (2 * c + g) * 1024));
    kp.sw[hf] = __builtin_nontemporal_load(
        reinterpret_cast<const uint32_t*>(base + kMxPageKeyBytes + 4 * (32 * hf + n)));
  }
}

__device__ __forceinline__ v16f mfma_32x32x64_fp8_mxfp4(const v8i& a, const v4i& b, int scale_b,
                                                        const v16f& c) {
  const v8i bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  // A: FP8 E4M3 with unit scale (E8M0 127); B: FP4 E2M1 (format 4) with its block scale
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, c, 0, 4, 0, 127, 0, scale_b);
}

// Score of token `lane` of an MXFP4 key page (same head reduction as the FP8 page; the block
// scales are inside the product, so there is no per-token scale).
__device__ __forceinline__ float score_key_page(const uint8_t* q8, const float* w,
                                                const KeyPageMx& cur, int lane) {
  const int n = lane & 31, g = lane >> 5;
  const uint8_t* qa = q8 + n * kQRowStride + 16 * g;
  const v4i a0 = *reinterpret_cast<const v4i*>(qa);
  const v4i a1 = *reinterpret_cast<const v4i*>(qa + 32);
  const v4i a2 = *reinterpret_cast<const v4i*>(qa + 64);
  const v4i a3 = *reinterpret_cast<const v4i*>(qa + 96);
  const v8i A0 = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
  const v8i A1 = v8i{a2[0], a2[1], a2[2], a2[3], a3[0], a3[1], a3[2], a3[3]};
  const v16f z = {};
  v16f d[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int s0 = (int)((cur.sw[hf] >> (8 * g)) & 0xFFu);
    const int s1 = (int)((cur.sw[hf] >> (8 * (2 + g))) & 0xFFu);
    d[hf] = mfma_32x32x64_fp8_mxfp4(A0, cur.k[hf][0], s0, z);
    d[hf] = mfma_32x32x64_fp8_mxfp4(A1, cur.k[hf][1], s1, d[hf]);
  }
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const v4f wv = *reinterpret_cast<const v4f*>(w + 8 * a + 4 * g);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      acc0 = fmaf(wv[c], relu(d[0][4 * a + c]), acc0);
      acc1 = fmaf(wv[c], relu(d[1][4 * a + c]), acc1);
    }
  }
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc0), __float_as_uint(acc1),
                                                   false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

}  // namespace dsa
