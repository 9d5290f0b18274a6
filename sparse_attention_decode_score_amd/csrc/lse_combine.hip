// Stage 4 of the DSA decode path: log-sum-exp merge of split partial outputs.
//
// Partial attention outputs, each normalised by its own softmax sum and carrying its LSE,
// are merged as LSE = m + ln sum_s exp(LSE_s - m), O = sum_s exp(LSE_s - LSE) O_s (the
// vLLM Kimi K3.1 Pro page combines DCP partial outputs by log-sum-exp, "Decode context
// parallelism with the sparse indexer"; the same merge joins the split-context partials of
// one GPU).  One 128-thread workgroup per (row, head): thread t owns dims 4t .. 4t+3.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

namespace dsa {

namespace {

__global__ __launch_bounds__(128) void lse_combine_kernel(const float* __restrict__ o_part,
                                                          const float* __restrict__ lse_part,
                                                          int num_splits, int64_t rows_heads,
                                                          uint16_t* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  const int64_t rh = blockIdx.x;  // row * 96 + head
  const int t = threadIdx.x;
  float m = -INFINITY;
  for (int s = 0; s < num_splits; ++s) m = fmaxf(m, lse_part[s * rows_heads + rh]);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < num_splits; ++s) {
      const float l = lse_part[s * rows_heads + rh];
      const float w = l == -INFINITY ? 0.f : expf(l - m);
      tot += w;
      const v4f o = *reinterpret_cast<const v4f*>(o_part + (s * rows_heads + rh) * kVDim + 4 * t);
      acc += w * o;
    }
  }
  const float inv = tot > 0.f ? 1.0f / tot : 0.f;
  uint32_t u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b = __float_as_uint(acc[j] * inv);  // round to nearest even bf16
    b += 0x7FFFu + ((b >> 16) & 1u);
    u[j] = b >> 16;
  }
  v2i packed = {(int)(u[0] | (u[1] << 16)), (int)(u[2] | (u[3] << 16))};
  *reinterpret_cast<v2i*>(out + rh * kVDim + 4 * t) = packed;
  if (t == 0) lse_out[rh] = (m == -INFINITY) ? -INFINITY : m + logf(tot);
}

// The same merge over fp16 partials that hold O_s / latent_scale; the result is scaled back.
__global__ __launch_bounds__(128) void lse_combine_f16_kernel(const uint16_t* __restrict__ o_part,
                                                              const float* __restrict__ lse_part,
                                                              int num_splits, int64_t rows_heads,
                                                              float scale,
                                                              uint16_t* __restrict__ out,
                                                              float* __restrict__ lse_out) {
  const int64_t rh = blockIdx.x;
  const int t = threadIdx.x;
  float m = -INFINITY;
  for (int s = 0; s < num_splits; ++s) m = fmaxf(m, lse_part[s * rows_heads + rh]);
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < num_splits; ++s) {
      const float l = lse_part[s * rows_heads + rh];
      const float w = l == -INFINITY ? 0.f : expf(l - m);
      tot += w;
      const v2i raw = *reinterpret_cast<const v2i*>(o_part + (s * rows_heads + rh) * kVDim + 4 * t);
      const _Float16* h = reinterpret_cast<const _Float16*>(&raw);
      acc += w * v4f{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
    }
  }
  const float inv = tot > 0.f ? scale / tot : 0.f;
  uint32_t u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t b = __float_as_uint(acc[j] * inv);  // round to nearest even bf16
    b += 0x7FFFu + ((b >> 16) & 1u);
    u[j] = b >> 16;
  }
  v2i packed = {(int)(u[0] | (u[1] << 16)), (int)(u[2] | (u[3] << 16))};
  *reinterpret_cast<v2i*>(out + rh * kVDim + 4 * t) = packed;
  if (t == 0) lse_out[rh] = (m == -INFINITY) ? -INFINITY : m + logf(tot);
}

}  // namespace

hipError_t launch_lse_combine(int num_splits, int n_q, const float* o_part, const float* lse_part,
                              uint16_t* out_bf16, float* lse, hipStream_t st) {
  const int64_t rh = (int64_t)n_q * kMlaHeads;
  if (rh == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_combine_kernel, dim3((unsigned)rh), dim3(128), 0, st, o_part, lse_part,
                     num_splits, rh, out_bf16, lse);
  return hipGetLastError();
}

hipError_t launch_lse_combine_f16(int num_splits, int n_q, const uint16_t* o_part,
                                  const float* lse_part, float scale, uint16_t* out_bf16,
                                  float* lse, hipStream_t st) {
  const int64_t rh = (int64_t)n_q * kMlaHeads;
  if (rh == 0) return hipSuccess;
  hipLaunchKernelGGL(lse_combine_f16_kernel, dim3((unsigned)rh), dim3(128), 0, st, o_part,
                     lse_part, num_splits, rh, scale, out_bf16, lse);
  return hipGetLastError();
}

}  // namespace dsa
