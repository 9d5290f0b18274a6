// Pass 2 of the exact top-k (see topk.hip) as a function of one workgroup of kFinalThreads
// threads and one query row, so that the standalone final kernel and the fused
// select-and-attend kernel run the same code.
#pragma once

#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_index_core.hpp"
#include "dsa_internal.hpp"
#include "dsa_select.hpp"

namespace dsa {


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

// Copies, in element order, every element e < n with keep(key, token) into lkey / lidx, where
// get(e, key, token) gives element e, while they fit in kFinalTile slots.  Returns the number
// of such elements (more than kFinalTile: the copy is incomplete).
template <class Get, class Keep>
__device__ int gather_kept(const Get& get, int n, const Keep& keep, uint32_t* lkey, int32_t* lidx,
                           int* red, int& parity) {
  const int tid = threadIdx.x;
  constexpr int E = 16;
  constexpr int kTile = kFinalThreads * E;
  int kept = 0;
#pragma unroll 1
  for (int base = 0; base < n; base += kTile) {
    uint32_t tk[E];
    int ti[E];
    int c = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = base + tid * E + j;
      tk[j] = kSentinel;
      ti[j] = 0;
      if (e < n) get(e, tk[j], ti[j]);
      const bool in = e < n && keep(tk[j], ti[j]);
      tk[j] = in ? tk[j] : kSentinel;
      c += in ? 1 : 0;
    }
    int tot;
    int pos = kept + block_excl_scan(c, &tot, red, parity);
    if (kept + tot <= kFinalTile) {
#pragma unroll
      for (int j = 0; j < E; ++j) {
        if (tk[j] != kSentinel) {
          lkey[pos] = tk[j];
          lidx[pos] = ti[j];
          ++pos;
        }
      }
    }
    kept += tot;
    if (kept > kFinalTile) break;  // uniform
  }
  __syncthreads();
  return kept;
}

// Recomputes into row_scores (the row's score buffer, [0, n_vis)) the scores of every
// group g of row `row` with need(g), with the indexer's own arithmetic, so the values are
// bitwise those the indexer would have stored.  need() is called by every wave for every
// group (keep it cheap: an LDS read).  q8 / w: LDS for the row's quantised query
// (32 * kQRowStride bytes, 16-byte aligned) and folded head weights (32 floats, 16-byte
// aligned).  Starts and ends with a barrier; every thread of the workgroup calls it.
template <class Need>
__device__ void rescore_groups(const IndexRescore rs, int row, int n_vis, int n_groups,
                               const int32_t* bt_row, float* row_scores, Need need, uint8_t* q8,
                               float* w) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __syncthreads();
  if (tid < kIdxHeads * 8) {  // whole waves: 8 lanes per head
    const int qh = tid >> 3, qpart = tid & 7;
    const uint16_t* src = rs.q + ((int64_t)row * kIdxHeads + qh) * kIdxDim + qpart * 16;
    const v4i raw[2] = {*reinterpret_cast<const v4i*>(src), *reinterpret_cast<const v4i*>(src + 8)};
    quantize_index_query_part(raw, rs.head_w[(int64_t)row * kIdxHeads + qh], qpart,
                              q8 + qh * kQRowStride + qpart * 16, w + qh);
  }
  __syncthreads();
  constexpr int kPagesPerGroup = kGroupTok / kPage;
  const int n_pages = (n_vis + kPage - 1) / kPage;
  // the pages of the needed groups are dealt to the waves in turn: every wave walks the
  // groups 64 at a time (one per lane) and counts the pages dealt so far
  int dealt = 0;  // wave-uniform
#pragma unroll 1
  for (int base = 0; base < n_groups; base += 64) {
    uint64_t todo = __ballot(base + lane < n_groups && need(base + lane));
    while (todo) {
      const int g = base + (int)__builtin_ctzll(todo);
      todo &= todo - 1;
      const int pg0 = g * kPagesPerGroup, pg1 = min(n_pages, pg0 + kPagesPerGroup);
      const int first = pg0 + ((wave - dealt) % kFinalWaves + kFinalWaves) % kFinalWaves;
      dealt += pg1 - pg0;
      for (int p = first; p < pg1; p += kFinalWaves) {
        const uint8_t* page = rs.key_pages + (int64_t)bt_row[p] * rs.page_stride;
        float sc;
        if (rs.mxfp4) {
          KeyPageMx kp;
          load_key_page(kp, page, lane);
          sc = score_key_page(q8, w, kp, lane);
        } else {
          KeyPage kp;
          load_key_page(kp, page, lane);
          sc = score_key_page(q8, w, kp, lane);
        }
        const int t = p * kPage + lane;
        if (t < n_vis) row_scores[t] = sc;
      }
    }
  }
  __syncthreads();
}

// LDS the final pass needs besides its output: the on-chip candidate tile (keys, token
// indices), the reduction scratch and the radix histograms of the selection.
struct FinalScratch {
  uint32_t* lkey;   // kFinalTile
  int32_t* lidx;    // kFinalTile
  int* red;         // 4 * kFinalWaves, 16-byte aligned
  int* note;        // 1
  uint32_t* hist;   // kHistWords
};

// The resend of the final pass (see final_select_row).  Everything is passed by value: a
// pointer into the kernel's argument block would make the compiler copy that block to
// scratch memory at the kernel's start.
struct ResendArgs {
  int row, n_vis, k, n_groups, m, parity;
  uint32_t K;
  int I;
  const uint32_t* ck;
  const int32_t* ci;
  const ChunkInfo* inf;
  IndexRescore rs;
  const int32_t* bt_row;
  float* row_scores;
  int* out;
  uint32_t* lkey;
  int32_t* lidx;
  int* red;
  int* note_p;
  uint32_t* hist;
  uint8_t* rq8;
  float* rw;
};

__device__ __forceinline__ void final_resend(const ResendArgs a) {
  const int tid = threadIdx.x;
  const int row = a.row, n_vis = a.n_vis, k = a.k, n_groups = a.n_groups, m = a.m;
  int parity = a.parity;
  const uint32_t K = a.K;
  const int I = a.I;
  const uint32_t* __restrict__ ck = a.ck;
  const int32_t* __restrict__ ci = a.ci;
  const ChunkInfo* __restrict__ inf = a.inf;
  const IndexRescore rs = a.rs;
  const int32_t* bt_row = a.bt_row;
  float* const row_scores = a.row_scores;
  const float* src = row_scores;
  int* out = a.out;
  uint32_t* lkey = a.lkey;
  int32_t* lidx = a.lidx;
  int* red = a.red;
  int* note_p = a.note_p;
  uint32_t* hist = a.hist;
  uint8_t* const rq8 = a.rq8;
  float* const rw = a.rw;
  auto score_get = [src](int i) { return score_key(src[i]); };
  auto ident = [](int i) { return i; };
  auto flag_of = [&](const ChunkInfo& ic) {
    return ic.saturated && (ic.key > K || (ic.key == K && ic.idx < I));
  };
  auto flagged = [&](int g) { return flag_of(inf[g]); };
    // Rebuild the candidate list in token order, flagged groups in full and the others as
    // sent: thread t owns groups GPT t .. GPT t + GPT-1, and one scan of their lengths gives
    // every thread the list position of its elements.  out[g] (free until the next
    // selection) = start of group g | kFlagBit if g is flagged, for the recomputation.
    constexpr uint32_t kFlagBit = 0x80000000u, kStartMask = 0x7FFFFFFFu;
    uint32_t* const starts = reinterpret_cast<uint32_t*>(out);
    int total = 0;
    constexpr int GPT = kMaxTopk / kFinalThreads;  // groups per thread: GPT tid .. +GPT-1
    int len[GPT];   // elements of each of them in the resend list
    uint32_t fl = 0;  // which of them are flagged
    int at0 = 0;      // the resend-list position of this thread's first element
    if (n_groups <= kMaxTopk) {
      int sum = 0;
#pragma unroll
      for (int q = 0; q < GPT; ++q) {
        const int g = GPT * tid + q;
        const bool f = g < n_groups && flagged(g);
        fl |= f ? 1u << q : 0u;
        len[q] = g >= n_groups ? 0 : (f ? min(kGroupTok, n_vis - g * kGroupTok) : inf[g].count);
        sum += len[q];
      }
      int at = block_excl_scan(sum, &total, red, parity);
      at0 = at;
#pragma unroll
      for (int q = 0; q < GPT; ++q) {
        const int g = GPT * tid + q;  // every group has >= 1 element: starts increase
        starts[g] = g < n_groups ? ((uint32_t)at | (((fl >> q) & 1u) ? kFlagBit : 0u)) : kStartMask;
        at += len[q];
      }
    } else {
#pragma unroll
      for (int q = 0; q < GPT; ++q) len[q] = 0;
      total = kFinalTile + 1;
    }
    __syncthreads();
    auto flagged_lds = [starts](int g) { return (starts[g] & kFlagBit) != 0u; };
    // no stored scores: the flagged groups, which the resend reads in full, are recomputed
    if (rs.q && n_groups <= kMaxTopk)
      rescore_groups(rs, row, n_vis, n_groups, bt_row, row_scores, flagged_lds, rq8, rw);
    // The list is written group by group in token order.  A thread copies the candidates of
    // its own unflagged groups; the flagged groups (256 recomputed scores each) are copied by
    // the wave of the thread that owns them, 4 elements per lane.  keep(key, token) filters
    // the elements; off[q] is the position of group q's kept elements after this thread's
    // first.
    const int lane = tid & 63;
    // fn(q, key, token) for every candidate of this thread's unflagged groups, in token
    // order within each group: 4 candidates of every group per step, all of a step's loads
    // issued together (a group's m slots are a multiple of 4 and 16-byte aligned)
    int max_len = 0;
#pragma unroll
    for (int q = 0; q < GPT; ++q) max_len = ((fl >> q) & 1u) ? max_len : max(max_len, len[q]);
    auto each_candidate = [&](auto fn) {
#pragma unroll 1
      for (int i4 = 0; i4 < max_len; i4 += 4) {
        v4i kk[GPT], ii[GPT];
#pragma unroll
        for (int q = 0; q < GPT; ++q) {
          const bool on = !((fl >> q) & 1u) && i4 < len[q];
          const int64_t o = on ? (int64_t)(GPT * tid + q) * m + i4 : 0;
          kk[q] = *reinterpret_cast<const v4i*>(ck + o);
          ii[q] = *reinterpret_cast<const v4i*>(ci + o);
        }
#pragma unroll
        for (int q = 0; q < GPT; ++q)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (!((fl >> q) & 1u) && i4 + c < len[q]) fn(q, (uint32_t)kk[q][c], ii[q][c]);
      }
    };
    // kept elements of every group of this thread (flagged ones counted by the wave)
    auto count_kept = [&](auto keep, int (&cnt)[GPT]) {
#pragma unroll
      for (int q = 0; q < GPT; ++q) cnt[q] = 0;
      each_candidate([&](int q, uint32_t key, int t) {
#pragma unroll
        for (int qq = 0; qq < GPT; ++qq) cnt[qq] += (qq == q && keep(key, t)) ? 1 : 0;
      });
      for (uint64_t owners = __ballot(fl != 0u); owners; owners &= owners - 1) {  // uniform
        const int ol = (int)__builtin_ctzll(owners);
        const uint32_t ofl = (uint32_t)__builtin_amdgcn_readlane((int)fl, ol);
        for (uint32_t qs = ofl; qs; qs &= qs - 1) {
          const int q = (int)__builtin_ctz(qs);
          const int g = GPT * (tid - lane + ol) + q;
          int c = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 64 * j + lane;
            const int t = g * kGroupTok + i;
            const bool in = i < kGroupTok && t < n_vis && keep(score_key(src[t]), t);
            c += __popcll(__ballot(in));
          }
#pragma unroll
          for (int qq = 0; qq < GPT; ++qq)
            if (qq == q && lane == ol) cnt[qq] = c;
        }
      }
    };
    // writes the kept elements, this thread's first at position base
    auto write_kept = [&](auto keep, int base, const int (&cnt)[GPT]) {
      int off[GPT];
      int run = base;
#pragma unroll
      for (int q = 0; q < GPT; ++q) {
        off[q] = run;
        run += cnt[q];
      }
      {
        int wpos[GPT];
#pragma unroll
        for (int q = 0; q < GPT; ++q) wpos[q] = off[q];
        each_candidate([&](int q, uint32_t key, int t) {
          if (keep(key, t)) {
            int pos = 0;
#pragma unroll
            for (int qq = 0; qq < GPT; ++qq) pos = qq == q ? wpos[qq] : pos;
            lkey[pos] = key;
            lidx[pos] = t;
#pragma unroll
            for (int qq = 0; qq < GPT; ++qq) wpos[qq] += qq == q ? 1 : 0;
          }
        });
      }
      for (uint64_t owners = __ballot(fl != 0u); owners; owners &= owners - 1) {  // uniform
        const int ol = (int)__builtin_ctzll(owners);
        const uint32_t ofl = (uint32_t)__builtin_amdgcn_readlane((int)fl, ol);
        for (uint32_t qs = ofl; qs; qs &= qs - 1) {
          const int q = (int)__builtin_ctz(qs);
          const int g = GPT * (tid - lane + ol) + q;
          int o = 0;
#pragma unroll
          for (int qq = 0; qq < GPT; ++qq) o = qq == q ? off[qq] : o;
          int pos = __builtin_amdgcn_readlane(o, ol);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 64 * j + lane;
            const int t = g * kGroupTok + i;
            const uint32_t key = (i < kGroupTok && t < n_vis) ? score_key(src[t]) : kSentinel;
            const bool in = i < kGroupTok && t < n_vis && keep(key, t);
            const uint64_t b = __ballot(in);
            if (in) {
              lkey[pos + lanes_below(b)] = key;
              lidx[pos + lanes_below(b)] = t;
            }
            pos += __popcll(b);
          }
        }
      }
    };
    if (total <= kFinalTile) {
      auto all = [](uint32_t, int) { return true; };
      int cnt[GPT];
#pragma unroll
      for (int q = 0; q < GPT; ++q) cnt[q] = len[q];
      write_kept(all, at0, cnt);
      __syncthreads();
      block_topk([lkey](int i) { return lkey[i]; }, [lidx](int i) { return lidx[i]; }, total, k,
                 out, red, note_p, hist);
    } else {
      // Too many to hold.  Every winner ranks at or above the candidates' k-th (K, I) (the
      // k-th of a subset is a lower bound of the true k-th), so only those elements of the
      // resend list are kept (counted, then written in list order); if even they do not
      // fit, the whole row is filtered by K.
      auto ranked = [K, I](uint32_t key, int t) { return key > K || (key == K && t <= I); };
      int kept = kFinalTile + 1;
      if (n_groups <= kMaxTopk) {
        int cnt[GPT];
        count_kept(ranked, cnt);
        int mine = 0;
#pragma unroll
        for (int q = 0; q < GPT; ++q) mine += cnt[q];
        const int pos = block_excl_scan(mine, &kept, red, parity);
        if (kept <= kFinalTile) write_kept(ranked, pos, cnt);
        __syncthreads();
      }
      if (kept <= kFinalTile) {
        block_topk([lkey](int i) { return lkey[i]; }, [lidx](int i) { return lidx[i]; }, kept,
                   k, out, red, note_p, hist);
      } else {
        // no stored scores: the rest of the row is recomputed first
        if (rs.q) {
          if (n_groups <= kMaxTopk)
            rescore_groups(rs, row, n_vis, n_groups, bt_row, row_scores,
                           [&](int g) { return !flagged_lds(g); }, rq8, rw);
          else
            rescore_groups(rs, row, n_vis, n_groups, bt_row, row_scores,
                           [](int) { return true; }, rq8, rw);
        }
        auto score_at = [src](int e, uint32_t& key, int& t) {
          key = score_key(src[e]);
          t = e;
        };
        auto at_least = [K](uint32_t key, int) { return key >= K; };
        kept = gather_kept(score_at, n_vis, at_least, lkey, lidx, red, parity);
        if (kept <= kFinalTile) {
          block_topk([lkey](int i) { return lkey[i]; }, [lidx](int i) { return lidx[i]; }, kept,
                     k, out, red, note_p, hist);
        } else {
          block_topk(score_get, ident, n_vis, k, out, red, note_p, hist);
        }
      }
    }
  }

// The exact top k (token order) of row `row` (request position pos, n_vis = pos + 1 visible
// tokens) from its group candidates, resending flagged groups from the scores.  Writes the
// selected token indices to out[0 .. n_out) (LDS, kMaxTopk entries) and returns n_out =
// min(k, n_vis).  Ends with a barrier, so out[] is visible to the whole workgroup.
// rs.q set: the indexer stored no scores; the groups that must be re-read are first
// recomputed into the row's score buffer (bt_row: the request's block-table row).
// Only the resend uses sc.lkey / sc.lidx (and `out` before the selection): every thread
// calls before_scratch() once before it does, so a caller can keep other data in that LDS
// until then.
struct NoHook {
  __device__ void operator()() const {}
};
template <class Hook = NoHook>
__device__ inline int final_select_row(int row, int n_vis, float* scores, int64_t score_stride,
                                       int k, int num_groups, int64_t row_cap,
                                       const uint32_t* __restrict__ cand_key,
                                       const int32_t* __restrict__ cand_idx,
                                       const ChunkInfo* __restrict__ info,
                                       const IndexRescore& rs, const int32_t* bt_row, int* out,
                                       const FinalScratch& sc, Hook before_scratch = Hook{}) {
  const int tid = threadIdx.x;
  uint32_t* lkey = sc.lkey;
  int32_t* lidx = sc.lidx;
  int* red = sc.red;
  int* note_p = sc.note;
  uint32_t* hist = sc.hist;
  float* const row_scores = scores + (int64_t)row * score_stride;
  const float* src = row_scores;
  // LDS of a recomputation (the candidate tile is free until the resend rebuilds it)
  uint8_t* const rq8 = reinterpret_cast<uint8_t*>(sc.lkey);
  float* const rw = reinterpret_cast<float*>(sc.lkey) + kIdxHeads * kQRowStride / 4;
  auto score_get = [src](int i) { return score_key(src[i]); };
  auto ident = [](int i) { return i; };
  int n_out;
  if (n_vis <= k) {
    for (int i = tid; i < n_vis; i += kFinalThreads) out[i] = i;
    n_out = n_vis;
  } else {
    const int n_groups = (n_vis + kGroupTok - 1) / kGroupTok;
    const int m = group_cand_count(n_vis, k);
    const int n_cand = n_groups * m;
    const uint32_t* ck = cand_key + (int64_t)row * row_cap;
    const int32_t* ci = cand_idx + (int64_t)row * row_cap;
    const ChunkInfo* inf = info + (int64_t)row * num_groups;
    // a full row (m = 256): its candidate slots are the row's tokens in order, no group
    // record was written and none can hide a winner
    const bool full = m == kGroupTok;
    // this thread's first group record, loaded now so that the flag check after the
    // selection does not wait for it
    const ChunkInfo info0 = full ? ChunkInfo{0, 0, 0u, 0} : inf[min(tid, n_groups - 1)];
    KthKey kth;
    if (n_cand <= kFinalRegTile) {
      // this thread's E consecutive candidates straight into registers (n_cand and the
      // row's slots are multiples of 4 and 16-byte aligned)
      auto run = [&](auto e_tag) {
        constexpr int E = decltype(e_tag)::value;
        uint32_t kv[E];
        // the keys, then (up to 32 per thread) the token indices: the search waits for the
        // keys only, and the chosen elements' tokens are in registers when they are written
        // out.  A full row's token is its position.  With 64 per thread the index of a chosen
        // element is read when it is written out.  (A quad past the end reads element 0 and
        // is masked below.)
        constexpr bool kIdxRegs = E <= 32;
        v4i a[E / 4], c[kIdxRegs ? E / 4 : 1];
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const int e = tid * E + 4 * q;
          a[q] = *reinterpret_cast<const v4i*>(ck + (e < n_cand ? e : 0));
        }
        if constexpr (kIdxRegs) {
#pragma unroll
          for (int q = 0; q < E / 4; ++q) {
            const int e = tid * E + 4 * q;
            c[q] = full ? v4i{0, 0, 0, 0} : *reinterpret_cast<const v4i*>(ci + (e < n_cand ? e : 0));
          }
        }
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
          const bool in = tid * E + 4 * q < n_cand;
#pragma unroll
          for (int j = 0; j < 4; ++j) kv[4 * q + j] = in ? (uint32_t)a[q][j] : kSentinel;
        }
        const auto val = [ci, full](int e) { return full ? e : ci[e]; };
        if constexpr (kIdxRegs) {
          kth = block_topk_regs<E>(
              kv, val, [&](int j) { return full ? tid * E + j : (int)c[j / 4][j % 4]; }, true, k,
              out, red, note_p, hist);
        } else {
          kth = block_topk_regs<E>(kv, val, [tid](int j) { return tid * E + j; }, full, k, out,
                                   red, note_p, hist);
        }
      };
      switch (final_per_thread(n_cand)) {
        case 8: run(std::integral_constant<int, 8>()); break;
        case 16: run(std::integral_constant<int, 16>()); break;
        case 32: run(std::integral_constant<int, 32>()); break;
        default: run(std::integral_constant<int, 64>()); break;
      }
    } else {
      kth = block_topk([ck](int i) { return ck[i]; }, [ci](int i) { return ci[i]; }, n_cand, k,
                       out, red, note_p, hist);
    }
    const uint32_t K = kth.key;
    const int I = kth.idx;
    // groups whose m-th element beats the k-th selected may hide winners
    auto flag_of = [&](const ChunkInfo& ic) {
      return ic.saturated && (ic.key > K || (ic.key == K && ic.idx < I));
    };
    auto flagged = [&](int g) { return flag_of(inf[g]); };
    int any = !full && tid < n_groups && flag_of(info0) ? 1 : 0;
#pragma unroll 4
    for (int g = tid + kFinalThreads; !full && g < n_groups; g += kFinalThreads)
      any |= flagged(g) ? 1 : 0;
    int parity = 0;
    if (!full && block_sum(any, red, parity) > 0) {
      before_scratch();
      final_resend(ResendArgs{row, n_vis, k, n_groups, m, parity, K, I, ck, ci, inf, rs, bt_row,
                              row_scores, out, lkey, lidx, red, note_p, hist, rq8, rw});
    }
    n_out = k;
  }
  __syncthreads();
  return n_out;
}

}  // namespace dsa
