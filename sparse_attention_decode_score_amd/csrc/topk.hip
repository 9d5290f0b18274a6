// Stage 2 of the DSA decode path: exact top-k (k <= 4096) of each query row's visible scores.
//
// Total order: score descending, then token index ascending; -0.0 ties +0.0 and NaN ranks
// lowest (the vLLM Kimi K3.1 Pro page keeps the top 2,048 tokens, "What changed in Kimi K3.1
// Pro", with exact selection and a consistent tie rule, "Exact top-k merge with ~10x less
// traffic" and "Inter-GPU communication").
//
// Two passes, the on-chip form of the page's exact one-round merge:
//  pass 1  one workgroup per (row, 8,192-token chunk) selects the chunk's best m candidates
//          (radix select on order-preserving uint32 keys in LDS, 11+11+10-bit digits) and
//          writes them in token order, padded with sentinels, plus the chunk's m-th element.
//  pass 2  one workgroup per row radix-selects the top k of the candidates.  A chunk that
//          had more than m visible tokens could hold more winners than it sent exactly when
//          its m-th element beats the selection's k-th; then the row is re-selected from all
//          of its scores ("detect and resend"), so the output is always exact.
// Selections are written in increasing token order; no float atomics, so the result does
// not depend on how rows are batched.
#include "dsa_device.hpp"
#include "dsa_internal.hpp"

namespace dsa {

namespace {

constexpr int kNT = 256;       // threads per workgroup
constexpr int kE = 8;          // consecutive elements per thread per compaction round
constexpr int kChunk = 8192;   // tokens per first-pass chunk
constexpr uint32_t kSentinel = 0u;  // below every real key (NaN maps to 1)
constexpr int kFinalLds = 12288;    // candidates the final pass keeps in LDS

__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t k = order_key(f);
  return k == 0u ? 1u : k;
}

// Block-wide exclusive prefix sum over thread order; *total gets the block sum.
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* sh /*>= 5 ints*/) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kNT / 64; ++i) {
    const int s = sh[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Block-wide sum of v over threads with a larger index than this one.
__device__ __forceinline__ int block_suffix_excl(int v, int* sh) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(x, o, 64);
    if (lane + o < 64) x += y;
  }
  if (lane == 0) sh[w] = x;
  __syncthreads();
  int after = 0;
#pragma unroll
  for (int i = 0; i < kNT / 64; ++i) after += (i > w) ? sh[i] : 0;
  __syncthreads();
  return after + x - v;
}

// Finds the key K of the want-th largest element (1 <= want <= n) among get(0..n-1) and
// the number r >= 1 of elements equal to K that belong to the top `want` (the first r
// equal ones in index order).  hist: 2048 LDS counters.  sh: >= 8 LDS ints.
template <class Get>
__device__ void radix_threshold(const Get& get, int n, int want, uint32_t* hist, int* sh,
                                uint32_t& K, int& r) {
  uint32_t prefix = 0, mask = 0;
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int bits = pass == 2 ? 10 : 11;
    const uint32_t dmask = (1u << bits) - 1u;
    for (int i = tid; i < 2048; i += kNT) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kNT) {
      const uint32_t k = get(i);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    int local = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) local += (int)hist[tid * 8 + j];
    const int above = block_suffix_excl(local, sh);
    if (above < want && above + local >= want) {
      int c = above;
      for (int j = 7; j >= 0; --j) {
        const int hcount = (int)hist[tid * 8 + j];
        if (c + hcount >= want) {
          sh[4] = tid * 8 + j;
          sh[5] = want - c;
          break;
        }
        c += hcount;
      }
    }
    __syncthreads();
    const uint32_t bin = (uint32_t)sh[4];
    want = sh[5];
    __syncthreads();
    prefix |= bin << shift;
    mask |= dmask << shift;
  }
  K = prefix;
  r = want;
}

// Visits, in index order, every element with key > K plus the first r with key == K,
// calling emit(position, index, key); positions are 0, 1, ... in index order.  `limit` is
// the number that will be emitted (elements above K plus r).  Returns the number emitted;
// *last_eq gets the index of the r-th equal element (-1 if r == 0).
template <class Get, class Emit>
__device__ int ordered_compact(const Get& get, int n, uint32_t K, int r, int limit,
                               const Emit& emit, int* sh, int* last_eq) {
  const int tid = threadIdx.x;
  int out_base = 0, eq_base = 0;
  if (tid == 0) sh[6] = -1;
#pragma unroll 1
  for (int base = 0; base < n; base += kNT * kE) {
    uint32_t keys[kE];
    int n_eq = 0, n_gt = 0;
    const int i0 = base + tid * kE;
#pragma unroll
    for (int j = 0; j < kE; ++j) {
      keys[j] = (i0 + j < n) ? get(i0 + j) : 0u;
      const bool valid = i0 + j < n;
      n_eq += (valid && keys[j] == K) ? 1 : 0;
      n_gt += (valid && keys[j] > K) ? 1 : 0;
    }
    int eq_tot;
    const int eq_before = eq_base + block_excl_scan(n_eq, &eq_tot, sh);
    int n_take = n_gt;
    {
      int e = eq_before;
#pragma unroll
      for (int j = 0; j < kE; ++j)
        if (i0 + j < n && keys[j] == K) { n_take += (e < r) ? 1 : 0; ++e; }
    }
    int take_tot;
    int pos = out_base + block_excl_scan(n_take, &take_tot, sh);
    {
      int e = eq_before;
#pragma unroll
      for (int j = 0; j < kE; ++j) {
        if (i0 + j >= n) break;
        const bool gt = keys[j] > K;
        const bool eq = keys[j] == K;
        bool take = gt;
        if (eq) {
          take = e < r;
          if (e == r - 1) sh[6] = i0 + j;
          ++e;
        }
        if (take) emit(pos++, i0 + j, keys[j]);
      }
    }
    out_base += take_tot;
    eq_base += eq_tot;
    if (out_base >= limit) break;  // block-uniform: everything selected has been emitted
  }
  __syncthreads();
  *last_eq = sh[6];
  __syncthreads();
  return out_base;
}

// Request and absolute position of query row `row`: one wave-wide ballot over cu_q per 64
// requests (rows are grouped by request and are its last tokens).
__device__ __forceinline__ void row_of(const int32_t* cu_q, const int32_t* seq_lens, int num_seqs,
                                       int row, int& b, int& pos) {
  const int lane = lane_id();
  int count = 0;
  for (int base = 0; base < num_seqs; base += 64) {  // uniform loop
    const int i = base + lane;
    const bool le = i < num_seqs && cu_q[i] <= row;
    count += __popcll(__ballot(le));
  }
  b = count - 1;
  const int c0 = cu_q[b], c1 = cu_q[b + 1];
  pos = seq_lens[b] - (c1 - c0) + (row - c0);
}

// Candidates kept per chunk for a row with n_vis visible tokens: 1.5x the winners a full
// chunk holds on average (the page's exact merge sends 1.5 x 2048 / W per shard), rounded
// up to 64, at least 64 and at most a whole chunk.
__host__ __device__ __forceinline__ int cand_per_chunk(int n_vis, int k) {
  const int64_t num = (int64_t)3 * k * kChunk;
  const int64_t den = (int64_t)2 * n_vis;
  int64_t m = (num + den - 1) / den;
  m = (m + 63) / 64 * 64;
  if (m < 64) m = 64;
  if (m > kChunk) m = kChunk;
  return (int)m;
}

struct ChunkInfo {
  int count;      // candidates written (<= m), rest are sentinels
  int saturated;  // the chunk had more than m visible tokens
  uint32_t key;   // its m-th element (when saturated)
  int idx;
};

// ---------------------------------------------------------------- pass 1
__global__ __launch_bounds__(kNT) void topk_chunk_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int num_seqs,
    const float* __restrict__ scores, int64_t score_stride, int k, int num_chunks,
    int64_t row_cap, uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx,
    ChunkInfo* __restrict__ info) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[kChunk];
  __shared__ uint32_t hist[2048];
  __shared__ int sh[8];
  const int row = blockIdx.y, c = blockIdx.x;
  int b, pos;
  row_of(cu_q, seq_lens, num_seqs, row, b, pos);
  const int n_vis = pos + 1;
  if (n_vis <= k) return;  // pass 2 takes every visible token
  const int start = c * kChunk;
  if (start >= n_vis) return;
  const int n = min(kChunk, n_vis - start);
  const int m = cand_per_chunk(n_vis, k);
  const float* src = scores + (int64_t)row * score_stride + start;
  const int tid = threadIdx.x;
  for (int i = tid; i < n; i += kNT) keys[i] = score_key(src[i]);
  __syncthreads();

  const int64_t cbase = (int64_t)row * row_cap + (int64_t)c * m;
  uint32_t* ck = cand_key + cbase;
  int32_t* ci = cand_idx + cbase;
  ChunkInfo* inf = info + (int64_t)row * num_chunks + c;
  if (n <= m) {
    for (int i = tid; i < m; i += kNT) {
      ck[i] = i < n ? keys[i] : kSentinel;
      ci[i] = i < n ? start + i : 0x7FFFFFFF;
    }
    if (tid == 0) *inf = ChunkInfo{n, 0, 0u, -1};
    return;
  }
  auto get = [&](int i) { return keys[i]; };
  uint32_t K;
  int r;
  radix_threshold(get, n, m, hist, sh, K, r);
  int last_eq;
  auto emit = [&](int p, int i, uint32_t key) {
    ck[p] = key;
    ci[p] = start + i;
  };
  ordered_compact(get, n, K, r, m, emit, sh, &last_eq);
  if (tid == 0) *inf = ChunkInfo{m, 1, K, start + last_eq};
}

// ---------------------------------------------------------------- pass 2
__global__ __launch_bounds__(kNT) void topk_final_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int num_seqs,
    const float* __restrict__ scores, int64_t score_stride, int k, int num_chunks,
    int64_t row_cap, const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_idx,
    const ChunkInfo* __restrict__ info, const int32_t* __restrict__ block_table, int bt_stride,
    int32_t* __restrict__ topk_idx, int32_t* __restrict__ topk_slot) {
  __shared__ int out[4096];
  __shared__ uint32_t hist[2048];
  __shared__ int sh[8];
  __shared__ int redo;
  __shared__ __attribute__((aligned(16))) uint32_t lkey[kFinalLds];
  __shared__ __attribute__((aligned(16))) int32_t lidx[kFinalLds];
  const int row = blockIdx.x, tid = threadIdx.x;
  int b, pos;
  row_of(cu_q, seq_lens, num_seqs, row, b, pos);
  const int n_vis = pos + 1;
  int32_t* oi = topk_idx + (int64_t)row * k;
  int32_t* os = topk_slot ? topk_slot + (int64_t)row * k : nullptr;
  const int32_t* bt = block_table ? block_table + (int64_t)b * bt_stride : nullptr;

  int n_out;
  if (n_vis <= k) {
    for (int i = tid; i < n_vis; i += kNT) out[i] = i;
    n_out = n_vis;
    __syncthreads();
  } else {
    const int n_chunks = (n_vis + kChunk - 1) / kChunk;
    const int m = cand_per_chunk(n_vis, k);
    const int n_cand = n_chunks * m;  // >= 1.5 k by construction of m
    const uint32_t* ck = cand_key + (int64_t)row * row_cap;
    const int32_t* ci = cand_idx + (int64_t)row * row_cap;
    uint32_t K;
    int r;
    int last_eq;
    int I;
    if (n_cand <= kFinalLds) {
      // candidates fit in LDS: one coalesced read, then every pass runs on-chip
      for (int i = tid; i < n_cand; i += kNT) {
        lkey[i] = ck[i];
        lidx[i] = ci[i];
      }
      __syncthreads();
      auto getc = [&](int i) { return lkey[i]; };
      radix_threshold(getc, n_cand, k, hist, sh, K, r);
      auto emitc = [&](int p, int i, uint32_t) { out[p] = lidx[i]; };
      ordered_compact(getc, n_cand, K, r, k, emitc, sh, &last_eq);
      I = last_eq >= 0 ? lidx[last_eq] : 0x7FFFFFFF;
    } else {
      auto getc = [&](int i) { return ck[i]; };
      radix_threshold(getc, n_cand, k, hist, sh, K, r);
      auto emitc = [&](int p, int i, uint32_t) { out[p] = ci[i]; };
      ordered_compact(getc, n_cand, K, r, k, emitc, sh, &last_eq);
      I = last_eq >= 0 ? ci[last_eq] : 0x7FFFFFFF;
    }
    if (tid == 0) redo = 0;
    __syncthreads();
    const ChunkInfo* inf = info + (int64_t)row * num_chunks;
    for (int c = tid; c < n_chunks; c += kNT) {
      const ChunkInfo ic = inf[c];
      // a saturated chunk whose m-th element beats the k-th selected may hide winners
      if (ic.saturated && (ic.key > K || (ic.key == K && ic.idx < I))) redo = 1;
    }
    __syncthreads();
    if (redo) {
      const float* src = scores + (int64_t)row * score_stride;
      auto gets = [&](int i) { return score_key(src[i]); };
      radix_threshold(gets, n_vis, k, hist, sh, K, r);
      auto emits = [&](int p, int i, uint32_t) { out[p] = i; };
      ordered_compact(gets, n_vis, K, r, k, emits, sh, &last_eq);
    }
    n_out = k;
    __syncthreads();
  }
  for (int i = tid; i < k; i += kNT) {
    const int t = i < n_out ? out[i] : -1;
    oi[i] = t;
    if (os) os[i] = t < 0 ? -1 : bt[t >> 6] * kPage + (t & (kPage - 1));
  }
}

}  // namespace

TopkPlan topk_plan(int max_seq_len, int k) {
  TopkPlan p;
  p.chunk = kChunk;
  p.num_chunks = (max_seq_len + kChunk - 1) / kChunk;
  if (p.num_chunks < 1) p.num_chunks = 1;
  // worst case over rows: for c chunks the smallest visible length is (c-1)*chunk + 1
  int64_t cap = 0;
  for (int c = 1; c <= p.num_chunks; ++c) {
    const int n_vis = c == 1 ? k + 1 : (c - 1) * kChunk + 1;
    const int64_t need = (int64_t)c * cand_per_chunk(n_vis, k);
    if (need > cap) cap = need;
  }
  p.row_cap = (cap + 63) / 64 * 64;
  return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t topk_workspace_bytes(int n_q, int max_seq_len, int k) {
  const TopkPlan p = topk_plan(max_seq_len, k);
  const size_t nc = (size_t)n_q * p.row_cap;
  return align256(nc * 4) * 2 + align256((size_t)n_q * p.num_chunks * sizeof(ChunkInfo));
}

hipError_t launch_topk(int num_seqs, int n_q, int max_seq_len, const int32_t* cu_q,
                       const int32_t* seq_lens, const float* scores, int64_t score_stride, int k,
                       const int32_t* block_table, int bt_stride, int32_t* topk_idx,
                       int32_t* topk_slot, void* workspace, hipStream_t st) {
  const TopkPlan p = topk_plan(max_seq_len, k);
  const size_t nc = (size_t)n_q * p.row_cap;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint32_t* cand_key = reinterpret_cast<uint32_t*>(ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(ws + align256(nc * 4));
  ChunkInfo* info = reinterpret_cast<ChunkInfo*>(ws + 2 * align256(nc * 4));
  hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)p.num_chunks, (unsigned)n_q), dim3(kNT), 0,
                     st, cu_q, seq_lens, num_seqs, scores, score_stride, k, p.num_chunks,
                     (int64_t)p.row_cap, cand_key, cand_idx, info);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)n_q), dim3(kNT), 0, st, cu_q, seq_lens,
                     num_seqs, scores, score_stride, k, p.num_chunks, (int64_t)p.row_cap,
                     cand_key, cand_idx, info, block_table, bt_stride, topk_idx, topk_slot);
  return hipGetLastError();
}

}  // namespace dsa
