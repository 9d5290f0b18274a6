// Stage 2 of the DSA decode path: exact top-k (k <= 4096) of each query row's visible scores.
//
// Total order: score descending, then token index ascending; -0.0 ties +0.0 and NaN ranks
// lowest (the vLLM Kimi K3.1 Pro page keeps the top 2,048 tokens, "What changed in Kimi K3.1
// Pro", with exact selection and a consistent tie rule, "Exact top-k merge with ~10x less
// traffic" and "Inter-GPU communication").
//
// Two passes, the on-chip form of the page's exact one-round merge, with 256-token groups in
// the role of the page's per-GPU shards:
//  pass 1  one wave per (row, group) keeps the group's best m candidates (m from
//          group_cand_count) in token order, plus the group's m-th element.  The fused
//          indexer runs this pass while the scores are still in registers; the kernel below
//          runs it from stored scores.
//  pass 2  one 512-thread workgroup per row selects the top k of the candidates.  A group
//          that had more than m visible tokens can hide winners exactly when its m-th
//          element beats the selection's k-th; those groups (only) are re-read in full from
//          the scores and the row is selected again, which is exact (every unsent token of
//          an unflagged group ranks below the candidates' k-th, hence below the true k-th).
// Selections are written in increasing token order; no float atomics, so the result does
// not depend on how rows are batched.
#include <algorithm>
#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_internal.hpp"
#include "dsa_select.hpp"
#include "dsa_topk_final.hpp"

namespace dsa {

namespace {

// ---------------------------------------------------------------- pass 1 from stored scores
// grid (ceil(groups / 4), n_q), 4 waves: wave w takes group 4 * blockIdx.x + w of the row.
__global__ __launch_bounds__(256) void topk_group_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int num_seqs,
    const float* __restrict__ scores, int64_t score_stride, int k, int num_groups,
    int64_t row_cap, uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx,
    ChunkInfo* __restrict__ info, WsLayout layout) {
  __shared__ __attribute__((aligned(16))) uint32_t ghist[4][256];  // per wave
  write_ws_layout(layout);
  const int row = blockIdx.y;
  int b, pos;
  row_of(cu_q, seq_lens, num_seqs, row, b, pos);
  const int n_vis = pos + 1;
  const int g = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = g * kGroupTok;
  if (n_vis <= k || t0 >= n_vis) return;  // wave-uniform; no barriers in this kernel
  const int lane = lane_id();
  const float* src = scores + (int64_t)row * score_stride + t0;
  const int n = min(kGroupTok, n_vis - t0);
  uint32_t keys[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) keys[j] = 64 * j + lane < n ? score_key(src[64 * j + lane]) : kSentinel;
  const int m = group_cand_count(n_vis, k);
  const int64_t base = (int64_t)row * row_cap + (int64_t)g * m;
  group_select(keys, n, m, t0, cand_key + base, cand_idx + base,
               info + (int64_t)row * num_groups + g, &ghist[threadIdx.x >> 6][0]);
}

// ---------------------------------------------------------------- pass 2
__global__ __launch_bounds__(kFinalThreads) void topk_final_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens, int num_seqs,
    float* scores, int64_t score_stride, int k, int num_groups, int64_t row_cap,
    const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_idx,
    const ChunkInfo* __restrict__ info, IndexRescore rs, const int32_t* __restrict__ block_table,
    int bt_stride, int32_t* __restrict__ topk_idx, int32_t* __restrict__ topk_slot,
    WsLayout layout) {
  __shared__ __attribute__((aligned(16))) uint32_t lkey[kFinalTile];
  __shared__ __attribute__((aligned(16))) int32_t lidx[kFinalTile];
  __shared__ int out[kMaxTopk];
  __shared__ __attribute__((aligned(16))) int red[4 * kFinalWaves];
  __shared__ int note;
  __shared__ __attribute__((aligned(16))) uint32_t hist[kHistWords];
  const int row = blockIdx.x, tid = threadIdx.x;
  int b, pos;
  row_of(cu_q, seq_lens, num_seqs, row, b, pos);
  const int n_vis = pos + 1;
  int32_t* oi = topk_idx + (int64_t)row * k;
  int32_t* os = topk_slot ? topk_slot + (int64_t)row * k : nullptr;
  const int32_t* bt = block_table ? block_table + (int64_t)b * bt_stride : nullptr;
  FinalScratch sc{lkey, lidx, red, &note, hist};
  // candidates written for another layout: nothing is selected (see WsLayout)
  const bool layout_ok = ws_layout_ok(layout);
  if (!layout_ok) flag_ws_layout(layout);
  const int n_out = layout_ok ? final_select_row(row, n_vis, scores, score_stride, k, num_groups,
                                                 row_cap, cand_key, cand_idx, info, rs, bt, out, sc)
                              : 0;
#pragma unroll 8
  for (int i = tid; i < k; i += kFinalThreads) {
    const int t = i < n_out ? out[i] : -1;
    oi[i] = t;
    if (os) os[i] = t < 0 ? -1 : bt[t >> 6] * kPage + (t & (kPage - 1));
  }
}

}  // namespace

// Candidate slots reserved per row: the worst case over rows of groups x candidates; for c
// groups the smallest visible length with candidates is max(k + 1, (c - 1) * 256 + 1).
TopkPlan topk_plan(int max_seq_len, int k) {
  TopkPlan p;
  p.num_groups = (max_seq_len + kGroupTok - 1) / kGroupTok;
  if (p.num_groups < 1) p.num_groups = 1;
  int64_t cap = 0;
  for (int c = 1; c <= p.num_groups; ++c) {
    const int lo = std::max(k + 1, (c - 1) * kGroupTok + 1);
    if (lo > c * kGroupTok) continue;
    const int64_t need = (int64_t)c * group_cand_count(lo, k);
    if (need > cap) cap = need;
  }
  p.row_cap = (cap + 63) / 64 * 64;
  if (p.row_cap < 64) p.row_cap = 64;
  return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t topk_workspace_bytes(int n_q, int max_seq_len, int k) {
  const TopkPlan p = topk_plan(max_seq_len, k);
  const size_t nc = (size_t)n_q * p.row_cap;
  return kWsHeaderBytes + align256(nc * 4) * 2 +
         align256((size_t)n_q * p.num_groups * sizeof(ChunkInfo));
}

TopkBuffers topk_buffers(void* workspace, int n_q, int max_seq_len, int k) {
  const TopkPlan p = topk_plan(max_seq_len, k);
  const size_t nc = (size_t)n_q * p.row_cap;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  TopkBuffers t;
  t.layout = WsLayout{reinterpret_cast<int32_t*>(ws), k, max_seq_len, n_q};
  ws += kWsHeaderBytes;
  t.plan = p;
  t.cand_key = reinterpret_cast<uint32_t*>(ws);
  t.cand_idx = reinterpret_cast<int32_t*>(ws + align256(nc * 4));
  t.info = reinterpret_cast<ChunkInfo*>(ws + 2 * align256(nc * 4));
  return t;
}

hipError_t launch_topk_final(int num_seqs, int n_q, const int32_t* cu_q, const int32_t* seq_lens,
                             const float* scores, int64_t score_stride, int k,
                             const TopkBuffers& t, const IndexRescore& rs,
                             const int32_t* block_table, int bt_stride, int32_t* topk_idx,
                             int32_t* topk_slot, hipStream_t st) {
  // (scores is written only when rs.q is set: it is then the caller's scratch)
  hipLaunchKernelGGL(topk_final_kernel, dim3((unsigned)n_q), dim3(kFinalThreads), 0, st, cu_q,
                     seq_lens, num_seqs, const_cast<float*>(scores), score_stride, k,
                     t.plan.num_groups, (int64_t)t.plan.row_cap, t.cand_key, t.cand_idx, t.info,
                     rs, block_table, bt_stride, topk_idx, topk_slot, t.layout);
  return hipGetLastError();
}

hipError_t launch_topk(int num_seqs, int n_q, int max_seq_len, const int32_t* cu_q,
                       const int32_t* seq_lens, const float* scores, int64_t score_stride, int k,
                       const int32_t* block_table, int bt_stride, int32_t* topk_idx,
                       int32_t* topk_slot, void* workspace, hipStream_t st) {
  const TopkBuffers t = topk_buffers(workspace, n_q, max_seq_len, k);
  hipLaunchKernelGGL(topk_group_kernel, dim3((unsigned)((t.plan.num_groups + 3) / 4), (unsigned)n_q),
                     dim3(256), 0, st, cu_q, seq_lens, num_seqs, scores, score_stride, k,
                     t.plan.num_groups, (int64_t)t.plan.row_cap, t.cand_key, t.cand_idx, t.info,
                     t.layout);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_final(num_seqs, n_q, cu_q, seq_lens, scores, score_stride, k, t,
                           IndexRescore{nullptr, nullptr, nullptr, 0, 0}, block_table, bt_stride,
                           topk_idx, topk_slot, st);
}

}  // namespace dsa
