// Stage 1 of the DSA decode path: lightning-indexer scores over a paged FP8 key cache.
//
// score[i][t] = sum_h w_h * sq_h * ReLU(q8_h . k8_t) * s_t  (the head-weighted ReLU form of
// DeepSeek-V3.2's lightning indexer that the vLLM Kimi K3.1 Pro page defers to in "What
// changed in Kimi K3.1 Pro"; fp32 accumulation and head-weighted reduction as in its
// "Native MXFP4 indexer" section).  The per-(row, head) power-of-two query scale sq is
// folded into the head weight, so the FP8 product needs no rescaling inside the loop.
//
// Work split: one workgroup per (request, segment of 16 G pages, group of up to R query
// rows); each of its 4 waves owns G groups of 4 consecutive pages (256 tokens).  Every
// workgroup streams its keys exactly once from HBM and reuses them for all R rows of the
// request (keys are shared by the verification rows of a speculative step, as the page's
// MI355X indexer does), so the grid is balanced by keys, not by requests.  A wave keeps a
// ring of pages in flight across its groups, so the fused first top-k pass of a group (see
// dsa_select.hpp) runs while the next group's keys stream in.
//
// One wave handles one 64-token page at a time as two 32-token halves:
//   D[head][token] = Q8[32 heads x 128] * K8^T[128 x 32 tokens]  (2 x v_mfma 32x32x64 fp8)
// Lane l reads 64 contiguous key bytes of token l%32 (bytes 64*(l/32) ..); the page stores
// keys in 16-byte column blocks so each of the 8 loads per lane is a fully coalesced 1 KB
// wave access.  The head reduction is 16 in-register FMAs, then one permlane32 swap that
// also places token l of the page in lane l for a coalesced 256-byte score store.
#include <algorithm>
#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_internal.hpp"
#include "dsa_index_core.hpp"
#include "dsa_select.hpp"

namespace dsa {

namespace {

constexpr int kWaves = 4;
constexpr int kGroupPages = kGroupTok / kPage;  // 4

// Pages each wave keeps in flight: four for two rows, two for larger row groups (register
// budget); one row runs three waves per SIMD (see the kernel) with two E4M3 pages or four
// (half-size) MXFP4 pages in flight per wave.  A group's four pages cycle through the ring
// in order, so the ring size divides four.  Groups per wave at most: the staged scores of a workgroup are
// 16 KB of LDS for up to four rows; eight rows store directly and take up to four groups,
// which the grid rule below gives them only when there are many row groups (a prefill),
// where long segments amortise the eight rows' query set-up.
template <int R>
struct IdxCfg {
  template <bool MX>
  static constexpr int kInFlight = R == 1 ? (MX ? 4 : 2) : R == 2 ? 4 : 2;
  static constexpr bool kStage = R <= 4;
  static constexpr int kMaxGroups = (R == 1 || R == 8) ? 4 : (R == 2 ? 2 : 1);
  static constexpr int kSegTok = kWaves * kGroupTok * kMaxGroups;  // tokens per workgroup
  static constexpr int kCandSlots = kWaves * kMaxGroups * kGroupTok;  // worst case (m = 256)
  static constexpr int kIdxSlots = kWaves * kMaxGroups * kMaxPartialCand;  // rows not full
};

// Candidate output of the fused first top-k pass.
struct CandOut {
  uint32_t* key;
  int32_t* idx;
  ChunkInfo* info;
  int64_t row_cap;
  int num_groups;
  int k;
  WsLayout layout;  // the workspace's layout record, written by one thread of the launch
};

// E4M3 codes and power-of-two scale of one (row, head) of dim = 64 * PPL values: 8
// consecutive lanes hold the head, lane i of the 8 converting dims PPL*8*i .. +PPL*8-1 from
// raw (16-byte bf16 loads); the head's absmax is reduced across its 8 lanes.  live = false:
// the lanes take part in the reduction only.
template <int PPL>
__device__ __forceinline__ void quantize_head(const v4i (&raw)[PPL], uint8_t* codes, float* scales,
                                              int64_t rh, bool live) {
  constexpr int dim = PPL * 64;
  const int lane8 = threadIdx.x & 7;
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < PPL; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      am = fmaxf(am, fmaxf(fabsf(bf16_lo((uint32_t)raw[i][j])), fabsf(bf16_hi((uint32_t)raw[i][j]))));
  am = fmaxf(am, __shfl_xor(am, 1, 64));
  am = fmaxf(am, __shfl_xor(am, 2, 64));
  am = fmaxf(am, __shfl_xor(am, 4, 64));
  const int e = pow2_scale_exp(am);
  const float inv = ldexpf(1.0f, -e);
  if (!live) return;
  const int64_t base = rh * dim + lane8 * (PPL * 8);
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    v2i c;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t w0 = (uint32_t)raw[i][2 * j], w1 = (uint32_t)raw[i][2 * j + 1];
      c[j] = (int)cvt4_e4m3(bf16_lo(w0) * inv, bf16_hi(w0) * inv, bf16_lo(w1) * inv,
                            bf16_hi(w1) * inv);
    }
    *reinterpret_cast<v2i*>(codes + base + 8 * i) = c;
  }
  if (lane8 == 0) scales[rh] = ldexpf(1.0f, e);
}

// The MLA query rows r0 .. r0+nr-1 (96 heads x 576 dims each) quantised by one 256-thread
// workgroup, one row (three passes of 32 heads, all loads first) at a time.
__device__ __forceinline__ void quantize_mla_rows(const MlaQueryPrep& pp, int r0, int nr) {
  constexpr int PPL = kLatDim / 64;  // 9
  const int hs = threadIdx.x >> 3, lane8 = threadIdx.x & 7;
#pragma unroll 1
  for (int r = r0; r < r0 + nr; ++r) {
    v4i raw[3][PPL];
#pragma unroll
    for (int ps = 0; ps < 3; ++ps) {
      const int64_t rh = (int64_t)r * kMlaHeads + 32 * ps + hs;
      const uint16_t* src = pp.q + rh * kLatDim + lane8 * (PPL * 8);
#pragma unroll
      for (int i = 0; i < PPL; ++i) raw[ps][i] = *reinterpret_cast<const v4i*>(src + 8 * i);
    }
#pragma unroll
    for (int ps = 0; ps < 3; ++ps)
      quantize_head<PPL>(raw[ps], pp.codes, pp.scales, (int64_t)r * kMlaHeads + 32 * ps + hs, true);
  }
}

// Why the structure below: the key loads of a wave's ring are issued unconditionally
// (page indices past the segment are clamped to a visible page, and the last group issues
// no loads past itself), and nothing is stored to global memory until every load has
// returned (scores and candidates are staged in LDS for up to four rows).  gfx950 counts
// loads and stores in one counter that may complete out of order, so a store in flight,
// or loads under data-dependent branches, would force a full drain of the ring at every
// wait instead of a wait for the oldest page only.
// Eight-row groups are held to three workgroups per CU (168 VGPRs, three waves per SIMD: the
// LDS of three fits): their rows' products and selections are latency-bound, and the third
// wave hides more of it than the registers it costs (a few spills; speculative decode
// indexer 44 -> 35 us).  So are one-row groups: three waves at <= 168 VGPRs without spills
// (two E4M3 pages in flight per wave instead of four; MXFP4 pages are half the size) and
// 50 KB of LDS each (at 128K x 32: E4M3 indexer ~94 -> ~92 us, MXFP4 58.1 -> 55.3 us).
template <int R, bool CAND, bool MX>
__global__ __launch_bounds__(256, (R == 8 || R == 1 ? 3 : 1)) void index_score_kernel(
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ seq_lens,
    const uint16_t* __restrict__ q, const float* __restrict__ head_w,
    const uint8_t* __restrict__ key_pages, int64_t page_stride,
    const int32_t* __restrict__ block_table, int bt_stride, float* __restrict__ scores,
    int64_t score_stride, int groups_per_wave, CandOut cand, MlaQueryPrep prep) {
  using Cfg = IdxCfg<R>;
  constexpr int NF = Cfg::template kInFlight<MX>;
  static_assert(kGroupPages % NF == 0, "ring slot of page s is s % NF = jj % NF");
  constexpr bool STAGE = Cfg::kStage;
  constexpr bool CSTAGE = CAND && STAGE;
  __shared__ __attribute__((aligned(16))) uint8_t q8s[R][kIdxHeads][kQRowStride];
  __shared__ __attribute__((aligned(16))) float wps[R][kIdxHeads];
  __shared__ __attribute__((aligned(16))) float sbuf[STAGE ? R : 1][STAGE ? Cfg::kSegTok : 1];
  __shared__ __attribute__((aligned(16))) uint32_t cbuf_key[CSTAGE ? R : 1][CSTAGE ? Cfg::kCandSlots : 1];
  // token indices only for rows that are not full (at most kMaxPartialCand per group)
  __shared__ __attribute__((aligned(16))) int32_t cbuf_idx[CSTAGE ? R : 1][CSTAGE ? Cfg::kIdxSlots : 1];
  __shared__ __attribute__((aligned(16))) ChunkInfo cbuf_info[CSTAGE ? R : 1][CSTAGE ? kWaves * Cfg::kMaxGroups : 1];
  __shared__ __attribute__((aligned(16))) uint32_t ghist[CAND ? kWaves : 1][256];  // per wave

  const int G = groups_per_wave;  // <= Cfg::kMaxGroups (host-checked)
  if constexpr (CAND) write_ws_layout(cand.layout);
  const int b = blockIdx.y;
  const int q0 = cu_q[b], q1 = cu_q[b + 1];
  const int r0 = q0 + (int)blockIdx.z * R;
  if (r0 >= q1) return;
  const int nr = min(R, q1 - r0);
  if (prep.q != nullptr && blockIdx.x == gridDim.x - 1) {  // the extra x slice
    quantize_mla_rows(prep, r0, nr);
    return;
  }
  const int L = seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const int p0 = (int)blockIdx.x * kWaves * kGroupPages * G;
  // the last position any row of this group may see
  const int max_pos = L - (q1 - q0) + (r0 + nr - 1 - q0);
  if (p0 >= n_pages || p0 * kPage > max_pos) return;
  const int p_end = min(min(n_pages, p0 + kWaves * kGroupPages * G), max_pos / kPage + 1);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31, g = lane >> 5;
  const int32_t* bt = block_table + (int64_t)b * bt_stride;
  // the wave's s-th page (s = 0 .. 4G-1): page s % 4 of its group s / 4
  auto page_of = [&](int s) { return p0 + kGroupPages * (kWaves * (s >> 2) + wave) + (s & 3); };
  // groups of this wave that hold a visible page
  const int seg_groups = (p_end - p0 + kGroupPages - 1) / kGroupPages;
  const int ng = max(0, (seg_groups - wave + kWaves - 1) / kWaves);

  // 1. one vector load fetches the wave's block-table entries (lane s: its s-th page,
  //    clamped to a visible page); it is the only load the key stream depends on, so it
  //    goes first.  2. the query and head weights (32 heads x 8 parts of 16 dims per row;
  //    rows past the group repeat its last row).  3. the first NF pages of the ring, as
  //    soon as the block-table entries are back (waiting for them does not wait for the
  //    query, issued after them).  The scheduling barriers keep this order: the query's
  //    arithmetic must not be hoisted above the key loads.
  const int bt_lane = bt[min(page_of(lane % (kGroupPages * G)), p_end - 1)];
  const int qh = tid >> 3, qpart = tid & 7;
  v4i qraw[R][2];
  float hw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = r0 + min(r, nr - 1);
    const uint16_t* src = q + ((int64_t)row * kIdxHeads + qh) * kIdxDim + qpart * 16;
    qraw[r][0] = *reinterpret_cast<const v4i*>(src);
    qraw[r][1] = *reinterpret_cast<const v4i*>(src + 8);
    hw[r] = head_w[(int64_t)row * kIdxHeads + qh];
  }
  __builtin_amdgcn_sched_barrier(0);
  auto page_ptr = [&](int s) {
    return key_pages + (int64_t)__builtin_amdgcn_readlane(bt_lane, s) * page_stride;
  };
  // (unconditional, also for a wave without groups in a request's last segment: a branch
  // here would leave the block-table load in doubt at every later wait)
  using Page = std::conditional_t<MX, KeyPageMx, KeyPage>;  // MXFP4 or E4M3 + scale keys
  Page kp[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j) load_key_page(kp[j], page_ptr(j), lane);
  __builtin_amdgcn_sched_barrier(0);
  // 3. fused query prep while the keys stream in: E4M3 codes, one power-of-two scale per
  //    (row, head), the scale folded into the head weight
#pragma unroll
  for (int r = 0; r < R; ++r)
    quantize_index_query_part(qraw[r], hw[r], qpart, &q8s[r][qh][qpart * 16], &wps[r][qh]);
  __syncthreads();

  // 4. the wave's groups: score each ring slot, refill it at once, and after four pages
  //    select the group's candidates while the next group's keys stream in
  uint32_t keys[R][4];
  auto score_page = [&](int s, int jj, const Page& cur) {
    const int p = page_of(s);
    const bool valid = p < p_end;
    const int t = p * kPage + lane;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // a group of eight rows holding fewer (five verification rows, say) skips the rest
      if (R > 4 && r >= nr) {  // uniform
        keys[r][jj] = kSentinel;
        continue;
      }
      const float score = score_key_page(&q8s[r][0][0], &wps[r][0], cur, lane);
      if constexpr (STAGE) {
        if (valid && scores) sbuf[r][(p - p0) * kPage + lane] = score;
      } else {
        if (valid && scores && r < nr && t < L) scores[(int64_t)(r0 + r) * score_stride + t] = score;
      }
      keys[r][jj] = valid ? score_key(score) : kSentinel;
    }
  };
  auto select_group = [&](int gi) {
    if constexpr (CAND) {
      const int grp = p0 / kGroupPages + kWaves * gi + wave;  // group index in the request
      const int t0 = grp * kGroupTok;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = r0 + r;
        const int n_vis = L - (q1 - q0) + (row - q0) + 1;
        if (r < nr && n_vis > cand.k && t0 < n_vis) {
          const int m = group_cand_count(n_vis, cand.k);
          const int gl = kWaves * gi + wave;  // group index in the workgroup
          if constexpr (CSTAGE) {
            group_select(keys[r], min(kGroupTok, n_vis - t0), m, t0, &cbuf_key[r][gl * m],
                         &cbuf_idx[r][m == kGroupTok ? 0 : gl * m],  // (full: unused)
                         &cbuf_info[r][gl], &ghist[wave][0]);
          } else {
            const int64_t base = (int64_t)row * cand.row_cap + (int64_t)grp * m;
            group_select(keys[r], min(kGroupTok, n_vis - t0), m, t0, cand.key + base,
                         cand.idx + base, cand.info + (int64_t)row * cand.num_groups + grp,
                         &ghist[wave][0]);
          }
        }
      }
    }
  };
#pragma unroll 1
  for (int gi = 0; gi + 1 < ng; ++gi) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int s = 4 * gi + jj;
      score_page(s, jj, kp[jj % NF]);
      load_key_page(kp[jj % NF], page_ptr(s + NF), lane);
    }
    select_group(gi);
  }
  if (ng > 0) {  // the last group loads nothing past itself
    const int gi = ng - 1;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int s = 4 * gi + jj;
      score_page(s, jj, kp[jj % NF]);
      if (jj + NF < 4) load_key_page(kp[jj % NF], page_ptr(s + NF), lane);
    }
    select_group(gi);
  }

  // 5. write what was staged: scores (and candidates) of the workgroup, coalesced
  if constexpr (STAGE) {
    __syncthreads();
    // non-temporal stores: the scores are read again only by the rare resend of a group,
    // and plain stores interleaved with the key stream cost the stream about 8% of its rate
    const int seg_tok = min(p_end * kPage, L) - p0 * kPage;
    for (int r = 0; r < (scores ? nr : 0); ++r) {
      float* dst = scores + (int64_t)(r0 + r) * score_stride + p0 * kPage;
      const bool vec = (((uintptr_t)dst) & 15) == 0;
      for (int i = 4 * tid; i < seg_tok; i += 1024) {
        if (vec && i + 3 < seg_tok) {
          __builtin_nontemporal_store(*reinterpret_cast<const v4f*>(&sbuf[r][i]),
                                      reinterpret_cast<v4f*>(dst + i));
        } else {
          for (int j = i; j < min(i + 4, seg_tok); ++j) __builtin_nontemporal_store(sbuf[r][j], dst + j);
        }
      }
    }
    if constexpr (CAND) {
      const int g_lo = p0 / kGroupPages;
      for (int r = 0; r < nr; ++r) {
        const int row = r0 + r;
        const int n_vis = L - (q1 - q0) + (row - q0) + 1;
        if (n_vis <= cand.k) continue;
        const int n_grp = min(g_lo + seg_groups, (n_vis + kGroupTok - 1) / kGroupTok) - g_lo;
        if (n_grp <= 0) continue;
        const int m = group_cand_count(n_vis, cand.k);
        const bool full = m == kGroupTok;  // keys only (group_select wrote nothing else)
        const int64_t base = (int64_t)row * cand.row_cap + (int64_t)g_lo * m;
        for (int i = tid; i < n_grp * m; i += 256) {
          cand.key[base + i] = cbuf_key[r][i];
          if (!full) cand.idx[base + i] = cbuf_idx[r][i];
        }
        for (int i = tid; !full && i < n_grp; i += 256)
          cand.info[(int64_t)row * cand.num_groups + g_lo + i] = cbuf_info[r][i];
      }
    }
  }
}

// Per-(row, head) query quantisation: 8 lanes per head, each converting dim/8 consecutive
// values (16-byte loads), the head's absmax reduced across its 8 lanes.  One 64-lane
// workgroup covers 8 heads.
template <int PPL>  // 16-byte pieces per lane = dim / 64
__global__ __launch_bounds__(64) void quantize_q_kernel(const uint16_t* __restrict__ q,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales,
                                                        int64_t rows_heads) {
  constexpr int dim = PPL * 64;
  const int lane = threadIdx.x;
  const int64_t rh = (int64_t)blockIdx.x * 8 + (lane >> 3);
  const bool live = rh < rows_heads;
  const int64_t base = (live ? rh : 0) * dim + (lane & 7) * (PPL * 8);
  v4i raw[PPL];
#pragma unroll
  for (int i = 0; i < PPL; ++i) raw[i] = *reinterpret_cast<const v4i*>(q + base + 8 * i);
  quantize_head<PPL>(raw, codes, scales, rh, live);
}

}  // namespace

hipError_t launch_quantize_q(int rows, int heads, int dim, const uint16_t* q, uint8_t* codes,
                             float* scales, hipStream_t st) {
  const int64_t n = (int64_t)rows * heads;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 7) / 8));
  if (dim == kIdxDim)
    hipLaunchKernelGGL(quantize_q_kernel<kIdxDim / 64>, grid, dim3(64), 0, st, q, codes, scales, n);
  else if (dim == kLatDim)
    hipLaunchKernelGGL(quantize_q_kernel<kLatDim / 64>, grid, dim3(64), 0, st, q, codes, scales, n);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_index_score(int num_seqs, int n_q, int max_seq_len, int max_q_per_seq,
                              const int32_t* cu_q, const int32_t* seq_lens, const uint16_t* q,
                              const float* head_w, const uint8_t* key_pages, int64_t key_page_stride,
                              const int32_t* block_table, int bt_stride, float* scores,
                              int64_t score_stride, int k, void* topk_ws, bool mxfp4,
                              hipStream_t st, MlaQueryPrep prep) {
  const int max_pages = (max_seq_len + kPage - 1) / kPage;
  int R = 8;
  if (max_q_per_seq <= 1) R = 1;
  else if (max_q_per_seq <= 2) R = 2;
  else if (max_q_per_seq <= 4) R = 4;
#ifdef DSA_INDEX_MAX_ROWS  // build-time override for tuning sweeps: rows per workgroup at most
  R = std::min(R, DSA_INDEX_MAX_ROWS);
#endif
  const unsigned gz = (unsigned)((max_q_per_seq + R - 1) / R);
  // groups per wave: the longest segments (up to the staging limit of R) that still give
  // >= 1,024 workgroups (4 per CU); one-row MXFP4 groups at most two (measured: at 128K x 32
  // the MXFP4 indexer takes 54.1 us with two groups per wave, 55.8 us with four; E4M3 keys
  // are indifferent)
  int G = (R == 1 || R == 8) ? (R == 1 && mxfp4 ? 2 : 4) : (R == 2 ? 2 : 1);
  while (G > 1 && (int64_t)num_seqs * gz *
                          ((max_pages + kWaves * kGroupPages * G - 1) / (kWaves * kGroupPages * G)) <
                      1024)
    G >>= 1;
#ifdef DSA_INDEX_GROUPS_PER_WAVE  // build-time override for tuning sweeps (at most the limit)
  G = std::min(DSA_INDEX_GROUPS_PER_WAVE, (R == 1 || R == 8) ? 4 : (R == 2 ? 2 : 1));
#endif
  const unsigned gx = (unsigned)((max_pages + kWaves * kGroupPages * G - 1) / (kWaves * kGroupPages * G));
  // with a query preparation, one more x slice of workgroups: the MLA query rows of each
  // (request, row group)
  const dim3 grid(gx + (prep.q ? 1u : 0u), (unsigned)num_seqs, gz), block(256);
  CandOut cand{nullptr, nullptr, nullptr, 0, 0, k, WsLayout{nullptr, 0, 0, 0}};
  if (topk_ws) {
    const TopkBuffers t = topk_buffers(topk_ws, n_q, max_seq_len, k);
    cand = CandOut{t.cand_key, t.cand_idx, t.info, (int64_t)t.plan.row_cap, t.plan.num_groups, k,
                   t.layout};
  }
#define DSA_LAUNCH_IDX(RR, CC)                                                                    \
  do {                                                                                           \
    if (mxfp4)                                                                                   \
      hipLaunchKernelGGL((index_score_kernel<RR, CC, true>), grid, block, 0, st, cu_q, seq_lens, \
                         q, head_w, key_pages, key_page_stride, block_table, bt_stride, scores,  \
                         score_stride, G, cand, prep);                                            \
    else                                                                                         \
      hipLaunchKernelGGL((index_score_kernel<RR, CC, false>), grid, block, 0, st, cu_q,          \
                         seq_lens, q, head_w, key_pages, key_page_stride, block_table, bt_stride, \
                         scores, score_stride, G, cand, prep);                                    \
  } while (0)
#define DSA_LAUNCH_R(CC)                 \
  switch (R) {                           \
    case 1: DSA_LAUNCH_IDX(1, CC); break; \
    case 2: DSA_LAUNCH_IDX(2, CC); break; \
    case 4: DSA_LAUNCH_IDX(4, CC); break; \
    default: DSA_LAUNCH_IDX(8, CC); break; \
  }
  if (topk_ws) {
    DSA_LAUNCH_R(true)
  } else {
    DSA_LAUNCH_R(false)
  }
#undef DSA_LAUNCH_R
#undef DSA_LAUNCH_IDX
  return hipGetLastError();
}

}  // namespace dsa
