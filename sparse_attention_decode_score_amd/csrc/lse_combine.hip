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

// Partial s of (row, head) rh as four fp32 values of dims 4t .. 4t+3.
struct PartF32 {
  const float* p;
  __device__ v4f load(int64_t off) const { return *reinterpret_cast<const v4f*>(p + off); }
};
// fp16 partials (O_s / latent_scale), widened to fp32.
struct PartF16 {
  const uint16_t* p;
  __device__ v4f load(int64_t off) const {
    const v2i raw = *reinterpret_cast<const v2i*>(p + off);
    const _Float16* h = reinterpret_cast<const _Float16*>(&raw);
    return v4f{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  }
};

// SMAX > 0: every split's LSE and partial are requested before any is used (one memory
// round trip; splits past num_splits re-read the last one and are ignored).  SMAX == 0: any
// number of splits, read split by split.  The sums run over s in increasing order either
// way, so both give the same bits.
template <int SMAX, class Part>
__global__ __launch_bounds__(128) void lse_combine_kernel(Part o_part, const float* __restrict__ lse_part,
                                                          int num_splits, int64_t rows_heads,
                                                          float scale, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse_out) {
  // (row, head) = row * 96 + head.  Workgroups are dealt to the 8 XCDs round-robin by
  // linear id; when the grid divides evenly, XCD x takes the contiguous eighth x of the rows,
  // as the attention kernel's split partials of those rows were written from that XCD.
  int64_t rh = blockIdx.x;
  if ((gridDim.x & 7) == 0) rh = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int t = threadIdx.x;
  float m = -INFINITY;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if constexpr (SMAX > 0) {
    float l[SMAX];
    v4f o[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int64_t sp = min(s, num_splits - 1) * rows_heads + rh;
      l[s] = lse_part[sp];
      o[s] = o_part.load(sp * kVDim + 4 * t);
    }
#pragma unroll
    for (int s = 0; s < SMAX; ++s)
      if (s < num_splits) m = fmaxf(m, l[s]);
    if (m != -INFINITY) {
#pragma unroll
      for (int s = 0; s < SMAX; ++s) {
        if (s < num_splits) {
          const float w = l[s] == -INFINITY ? 0.f : expf(l[s] - m);
          tot += w;
          acc += w * o[s];
        }
      }
    }
  } else {
    for (int s = 0; s < num_splits; ++s) m = fmaxf(m, lse_part[s * rows_heads + rh]);
    if (m != -INFINITY) {
      for (int s = 0; s < num_splits; ++s) {
        const float l = lse_part[s * rows_heads + rh];
        const float w = l == -INFINITY ? 0.f : expf(l - m);
        tot += w;
        acc += w * o_part.load((s * rows_heads + rh) * kVDim + 4 * t);
      }
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

template <class Part>
hipError_t launch_combine(int num_splits, int64_t rh, Part part, const float* lse_part, float scale,
                          uint16_t* out_bf16, float* lse, hipStream_t st) {
  const dim3 grid((unsigned)rh), block(128);
  if (num_splits <= 8)
    hipLaunchKernelGGL((lse_combine_kernel<8, Part>), grid, block, 0, st, part, lse_part, num_splits,
                       rh, scale, out_bf16, lse);
  else if (num_splits <= 16)
    hipLaunchKernelGGL((lse_combine_kernel<16, Part>), grid, block, 0, st, part, lse_part,
                       num_splits, rh, scale, out_bf16, lse);
  else
    hipLaunchKernelGGL((lse_combine_kernel<0, Part>), grid, block, 0, st, part, lse_part,
                       num_splits, rh, scale, out_bf16, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_combine(int num_splits, int n_q, const float* o_part, const float* lse_part,
                              uint16_t* out_bf16, float* lse, hipStream_t st) {
  const int64_t rh = (int64_t)n_q * kMlaHeads;
  if (rh == 0) return hipSuccess;
  return launch_combine(num_splits, rh, PartF32{o_part}, lse_part, 1.0f, out_bf16, lse, st);
}

hipError_t launch_lse_combine_f16(int num_splits, int n_q, const uint16_t* o_part,
                                  const float* lse_part, float scale, uint16_t* out_bf16,
                                  float* lse, hipStream_t st) {
  const int64_t rh = (int64_t)n_q * kMlaHeads;
  if (rh == 0) return hipSuccess;
  return launch_combine(num_splits, rh, PartF16{o_part}, lse_part, scale, out_bf16, lse, st);
}

}  // namespace dsa
