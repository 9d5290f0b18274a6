// Measurement kernels for the benchmark (not part of the DSA path): the achievable
// streaming-read rate of this GPU, and the rate of reading whole index-key pages through a
// block table with the indexer's exact per-lane load pattern (non-temporal loads, as the
// indexer issues them) but no arithmetic: the ceiling the indexer's key stream can reach.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const v4i* __restrict__ p, int64_t n16,
                                                          int* __restrict__ out) {
  v4i acc = {0, 0, 0, 0};
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride)
    acc ^= p[i] ^ p[i + stride] ^ p[i + 2 * stride] ^ p[i + 3 * stride];
  for (; i < n16; i += stride) acc ^= p[i];
  if (acc[0] == 0x7A5C3E1F && acc[1] == 0x1 && acc[2] == 0x2 && acc[3] == 0x3) out[0] = 1;
}

// one wave per page: lane l reads 16-byte pieces 4*(l/32) + j of tokens l%32 and 32 + l%32,
// then its token's fp32 scale, as the indexer does (non-temporal loads)
__global__ __launch_bounds__(256) void page_read_kernel(const uint8_t* __restrict__ pool,
                                                        int64_t page_stride,
                                                        const int32_t* __restrict__ pages,
                                                        int n_pages, int* __restrict__ out) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= n_pages) return;
  const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
  const uint8_t* base = pool + (int64_t)pages[w] * page_stride;
  v4i acc = {0, 0, 0, 0};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc ^= __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(base + (4 * g + j) * 1024 + (32 * hf + n) * 16));
  acc[0] ^= __builtin_nontemporal_load(reinterpret_cast<const int*>(base + 8192 + 4 * lane));
  if (acc[0] == 0x7A5C3E1F && acc[1] == 0x1 && acc[2] == 0x2 && acc[3] == 0x3) out[0] = 1;
}

// the same for an MXFP4 index-key page (4,352 bytes): lane l reads the 16-byte code blocks
// 2c + l/32 (c = 0, 1) of tokens l%32 and 32 + l%32, and those tokens' scale words
__global__ __launch_bounds__(256) void page_read_mx_kernel(const uint8_t* __restrict__ pool,
                                                           int64_t page_stride,
                                                           const int32_t* __restrict__ pages,
                                                           int n_pages, int* __restrict__ out) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= n_pages) return;
  const int lane = threadIdx.x & 63, n = lane & 31, g = lane >> 5;
  const uint8_t* base = pool + (int64_t)pages[w] * page_stride;
  v4i acc = {0, 0, 0, 0};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      acc ^= __builtin_nontemporal_load(
          reinterpret_cast<const v4i*>(base + (2 * c + g) * 1024 + (32 * hf + n) * 16));
    acc[1] ^= __builtin_nontemporal_load(
        reinterpret_cast<const int*>(base + 4096 + 4 * (32 * hf + n)));
  }
  if (acc[0] == 0x7A5C3E1F && acc[1] == 0x1 && acc[2] == 0x2 && acc[3] == 0x3) out[0] = 1;
}

}  // namespace

extern "C" {

// Reads `bytes` (multiple of 16) of device memory once.  Returns a hipError_t code.
int dsa_probe_stream_read(const void* buf, int64_t bytes, int* sink, int grid, void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const v4i*)buf, bytes / 16, sink);
  return (int)hipGetLastError();
}

// Reads the 8,448 data bytes of each listed page.  Returns a hipError_t code.
int dsa_probe_page_read(const void* pool, int64_t page_stride, const int32_t* pages, int n_pages,
                        int* sink, void* stream) {
  hipLaunchKernelGGL(page_read_kernel, dim3((n_pages + 3) / 4), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)pool, page_stride, pages, n_pages, sink);
  return (int)hipGetLastError();
}

// Reads the 4,352 data bytes of each listed MXFP4 page.  Returns a hipError_t code.
int dsa_probe_page_read_mx(const void* pool, int64_t page_stride, const int32_t* pages,
                           int n_pages, int* sink, void* stream) {
  hipLaunchKernelGGL(page_read_mx_kernel, dim3((n_pages + 3) / 4), dim3(256), 0,
                     (hipStream_t)stream, (const uint8_t*)pool, page_stride, pages, n_pages, sink);
  return (int)hipGetLastError();
}

}  // extern "C"
