// Exact selection primitives of the top-k stage: order-preserving keys, the per-group
// candidate rule, one wave's top-m of a 256-token group (a radix select on the wave's own LDS
// counters, keys in registers) and one 512-thread workgroup's top-k of up to 32,768 keys held
// in registers (a radix select with 8-bit digits), with slower paths for more.
//
// Total order everywhere: larger key first, equal keys by lower element index (token order).
#pragma once

#include "dsa_device.hpp"
#include "dsa_internal.hpp"

namespace dsa {

constexpr uint32_t kSentinel = 0u;  // below every real key (NaN maps to 1)
constexpr int kGroupTok = 256;      // tokens per first-pass group (one wave, 4 pages)
#ifndef DSA_FINAL_THREADS
#define DSA_FINAL_THREADS 512
#endif
constexpr int kFinalThreads = DSA_FINAL_THREADS;  // threads of the final pass
constexpr int kFinalWaves = kFinalThreads / 64;
constexpr int kFinalPerThread = 32;     // keys per thread of the on-chip candidate list (LDS)
constexpr int kFinalRegPerThread = 64;  // keys per thread the selection holds in registers
constexpr int kRadixBits = 8;                  // key bits one pass of the final selection settles
constexpr int kRadixBins = 1 << kRadixBits;
// The final selection's histogram of a pass is kept in four copies (lane % 4 picks one), so
// that lanes of one instruction adding to a crowded digit hit four addresses instead of one
// (LDS serialises atomics on one address); a copy is 260 words, so one digit's four copies
// sit on four different banks and each lane's four digits stay 16-byte aligned.
constexpr int kHistCopies = 4;
constexpr int kHistStride = kRadixBins + 4;
constexpr int kHistSet = kHistCopies * kHistStride;  // one pass's counters
constexpr int kHistWords = 3 * kHistSet;             // three in rotation
constexpr int kFinalTile = kFinalThreads * kFinalPerThread;  // keys the final pass holds in LDS
constexpr int kFinalRegTile = kFinalThreads * kFinalRegPerThread;  // ... and in registers

// Per-group record of the first selection pass.
struct ChunkInfo {
  int count;      // real candidates written (<= m); the rest of the m slots are sentinels
  int saturated;  // the group had more than m visible tokens
  uint32_t key;   // its m-th element (when saturated): key and token index
  int idx;
};

// The top-k workspace's layout record (see WsLayout): written once per launch by the pass
// that fills the candidates, checked by the final pass.
__device__ __forceinline__ void write_ws_layout(const WsLayout& l) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) {
    *reinterpret_cast<v4i*>(l.header) = v4i{kWsMagic, l.k, l.max_seq_len, l.n_q};
    l.header[4] = 0;
  }
}
__device__ __forceinline__ bool ws_layout_ok(const WsLayout& l) {
  const v4i h = *reinterpret_cast<const v4i*>(l.header);
  return h[0] == kWsMagic && h[1] == l.k && h[2] == l.max_seq_len && h[3] == l.n_q;
}
__device__ __forceinline__ void flag_ws_layout(const WsLayout& l) {
  if (threadIdx.x == 0) l.header[4] = 1;
}

// Score -> key: larger score = larger key, -0.0 == +0.0, NaN just above the sentinel.
__device__ __forceinline__ uint32_t score_key(float f) {
  const uint32_t k = order_key(f);
  return k == 0u ? 1u : k;
}

// Candidates a first-pass group keeps, m.  A full group holds lambda = k * 256 / n_vis of the
// winners on average (the on-chip form of the per-shard rule of the exact top-k merge, with
// slack because a group is small): m = 4 lambda where lambda >= 4, else 4 lambda + 4 and at
// least 8, rounded up to 4 and at most the group.  A group holding m or more winners is
// resent (read again in full) by the final pass; for independent scores that is about one
// group in 10^5 rows at lambda = 4 (131,072 visible tokens, k = 2,048: m = 16) and rarer at
// smaller lambda (1,048,576 tokens: lambda = 1/2, m = 8, 32,768 candidates).
#ifndef DSA_FULL_ROW_MAX
#define DSA_FULL_ROW_MAX (kFinalThreads * kFinalRegPerThread)
#endif
// Rows of at most this many visible tokens keep every token (m = 256, "full" rows): the final
// pass then selects from the whole row in registers, which costs less than a first-pass
// selection that would keep a large share of each group anyway (m >= 64 below 32,768 tokens).
constexpr int kFullRowMax = DSA_FULL_ROW_MAX;
static_assert(kFullRowMax <= kFinalThreads * kFinalRegPerThread, "full rows fit the registers");
__host__ __device__ __forceinline__ constexpr int group_cand_count(int n_vis, int k) {
  if (n_vis <= kFullRowMax) return kGroupTok;
  const int64_t num = 4 * (int64_t)k * kGroupTok;  // 4 lambda n_vis
  int64_t m = (num + n_vis - 1) / n_vis;           // ceil(4 lambda)
  if (num < 16 * (int64_t)n_vis) {                 // lambda < 4
    m += 4;
    if (m < 8) m = 8;
  }
  m = (m + 3) / 4 * 4;
  if (m > kGroupTok) m = kGroupTok;
  return (int)m;
}

constexpr int kMaxTopk = 4096;  // the largest k the library accepts
// The most candidates a group of a row that is not full keeps (k = 4096 just past 32,768
// tokens): what a buffer of candidate token indices must hold per group.
constexpr int kMaxPartialCand = group_cand_count(kFullRowMax + 1, kMaxTopk);  // 128
static_assert(kMaxPartialCand % 4 == 0 && kMaxPartialCand <= kGroupTok, "partial-row bound");

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Sum of v over the wave, returned wave-uniform: DPP butterflies inside each row of 16 lanes
// (quad swaps, half-row and row mirrors), then the four row sums.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// Maximum / minimum of an unsigned value over the wave (same butterflies), wave-uniform.
#define DSA_DPP_U32(v, ctrl) \
  ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(v), (ctrl), 0xF, 0xF, false))
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, DSA_DPP_U32(v, 0xB1));
  v = max(v, DSA_DPP_U32(v, 0x4E));
  v = max(v, DSA_DPP_U32(v, 0x141));
  v = max(v, DSA_DPP_U32(v, 0x140));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, DSA_DPP_U32(v, 0xB1));
  v = min(v, DSA_DPP_U32(v, 0x4E));
  v = min(v, DSA_DPP_U32(v, 0x141));
  v = min(v, DSA_DPP_U32(v, 0x140));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
#undef DSA_DPP_U32

// Inclusive prefix sum over the lanes of the wave: shifted DPP adds inside each row of 16
// lanes (a lane whose source is outside its row adds 0), then the totals of the rows below.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = lane_id() >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// One wave's top-m of a group: lane l holds element 64*j + l in keys[j] (element i is token
// t0 + i; elements i >= n are not visible).  Writes the min(n, m) chosen keys and token
// indices in token order to ck / ci, sentinels (key 0, index INT_MAX) after them, and the
// group's record.  Wave-uniform control flow only.  wave_hist: 256 counters of LDS (16-byte
// aligned) that only this wave uses.
__device__ __forceinline__ void group_select(const uint32_t (&keys)[4], int n, int m, int t0,
                                             uint32_t* ck, int32_t* ci, ChunkInfo* inf,
                                             uint32_t* wave_hist) {
  const int lane = lane_id();
  uint32_t kv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kv[j] = (64 * j + lane < n) ? keys[j] : kSentinel;
  if (n <= m) {
    // with m = 256 (a full row) the slots hold the row's tokens in order: the final pass
    // takes a slot's token from its position and reads no group record, so neither is written
    const bool full = m == kGroupTok;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 64 * j + lane;
      if (i < m) {
        ck[i] = kv[j];
        if (!full) ci[i] = i < n ? t0 + i : 0x7FFFFFFF;
      }
    }
    if (!full && lane == 0) *inf = ChunkInfo{n, 0, 0u, -1};
    return;
  }
  // K = the m-th largest key, found 8 bits at a time (a radix select within the wave).  The
  // visible keys (>= 1) share the bits of their maximum and minimum above the highest bit
  // where those differ; below it, each step histograms the next 8 bits of the keys that still
  // match the digits found so far (LDS atomics on this wave's counters, which LDS applies in
  // the wave's order, so no wait is needed before reading them back) and takes the largest
  // digit whose suffix count reaches the number of keys still wanted.  The search stops when
  // the bracket holds exactly the keys still wanted; K is then its smallest key.
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    mx = max(mx, kv[j]);
    mn = min(mn, kv[j] == kSentinel ? 0xFFFFFFFFu : kv[j]);
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  uint32_t K = mx;
  DSA_LDS uint32_t* const hist = (DSA_LDS uint32_t*)wave_hist;
  if (mx != mn) {
    int need = m;
    int lo_bit = 32 - __builtin_clz(mx ^ mn);  // bits lo_bit .. 31 are those of mx
    uint32_t prefix = lo_bit >= 32 ? 0u : (mx >> lo_bit) << lo_bit;
    bool exact = true;
#pragma unroll 1
    while (lo_bit > 0) {  // uniform
      const int width = lo_bit < 8 ? lo_bit : 8;
      const int sh = lo_bit - width;
      *reinterpret_cast<DSA_LDS v4i*>(hist + 4 * lane) = v4i{0, 0, 0, 0};
      const uint64_t want = (uint64_t)prefix >> lo_bit;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (kv[j] != kSentinel && ((uint64_t)kv[j] >> lo_bit) == want)
          __hip_atomic_fetch_add(hist + __builtin_amdgcn_ubfe(kv[j], sh, width), 1u,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      const v4i c4 = *reinterpret_cast<const DSA_LDS v4i*>(hist + 4 * lane);
      const int s3 = c4[3], s2 = s3 + c4[2], s1 = s2 + c4[1], s0 = s1 + c4[0];
      const int incl = wave_incl_scan(s0);
      const int above_lane = __builtin_amdgcn_readlane(incl, 63) - incl;
      const int S0 = above_lane + s0, S1 = above_lane + s1, S2 = above_lane + s2,
                S3 = above_lane + s3;
      const uint64_t ok = __ballot(S0 >= need);  // lane 0 always
      const int L = 63 - __builtin_clzll(ok);
      const int i_l = S3 >= need ? 3 : S2 >= need ? 2 : S1 >= need ? 1 : 0;
      const int s_next = i_l == 3 ? above_lane : i_l == 2 ? S3 : i_l == 1 ? S2 : S1;
      const int s_at = i_l == 3 ? S3 : i_l == 2 ? S2 : i_l == 1 ? S1 : S0;
      const int D = 4 * L + __builtin_amdgcn_readlane(i_l, L);
      const int taken = __builtin_amdgcn_readlane(s_next, L);
      const int in_d = __builtin_amdgcn_readlane(s_at, L) - taken;
      need -= taken;
      prefix |= (uint32_t)D << sh;
      lo_bit = sh;
      if (in_d == need) {  // every key left in the bracket is taken
        exact = lo_bit == 0;
        break;
      }
    }
    K = prefix;
    if (!exact) {
      const uint64_t want = (uint64_t)prefix >> lo_bit;
      uint32_t bmin = 0xFFFFFFFFu;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (kv[j] != kSentinel && ((uint64_t)kv[j] >> lo_bit) == want) bmin = min(bmin, kv[j]);
      K = wave_min_u32(bmin);
    }
  }
  int gt = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) gt += __popcll(__ballot(kv[j] > K));
  const int r = m - gt;  // equal keys taken, the first r in token order
  int base = 0, eq_seen = 0, last = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool eq = kv[j] == K;
    const uint64_t eqm = __ballot(eq);
    const int rank = eq_seen + lanes_below(eqm);
    const bool take = kv[j] > K || (eq && rank < r);
    if (eq && rank == r - 1) last = 64 * j + lane;
    const uint64_t tm = __ballot(take);
    if (take) {
      const int pos = base + lanes_below(tm);
      ck[pos] = kv[j];
      ci[pos] = t0 + 64 * j + lane;
    }
    base += __popcll(tm);
    eq_seen += __popcll(eqm);
  }
  const uint64_t who = __ballot(last >= 0);
  const int last_i = __shfl(last, (int)__builtin_ctzll(who), 64);
  if (lane == 0) *inf = ChunkInfo{m, 1, K, t0 + last_i};
}

// ----------------------------------------------------------------------------------------
// Workgroup (kFinalThreads threads) primitives.  Exchanges go through `red`: 4 * kFinalWaves
// ints of LDS, 16-byte aligned, used as two buffers of 2 * kFinalWaves ints in turn (parity
// flips), so one barrier per exchange suffices: a wave writes a buffer again only after the
// barrier of the exchange in between, which every wave reaches after reading it.
__device__ __forceinline__ int* red_buf(int* red, int& parity) {
  int* buf = red + 2 * kFinalWaves * parity;
  parity ^= 1;
  return buf;
}

// Sum over the workgroup of a per-wave value (wave-uniform v).
__device__ __forceinline__ int block_sum_waves(int v, int* red, int& parity) {
  int* buf = red_buf(red, parity);
  if (lane_id() == 0) buf[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int i = 0; i < kFinalWaves; i += 4) {
    const v4i a = *reinterpret_cast<const v4i*>(buf + i);
    t += (a[0] + a[1]) + (a[2] + a[3]);
  }
  return t;
}

// Sum over the workgroup of a per-thread value.
__device__ __forceinline__ int block_sum(int v, int* red, int& parity) {
  return block_sum_waves(wave_sum(v), red, parity);
}

// Workgroup maximum and minimum of per-thread values (both in one exchange).
__device__ __forceinline__ void block_max_min(uint32_t& mx, uint32_t& mn, int* red, int& parity) {
  const uint32_t a = wave_max_u32(mx), b = wave_min_u32(mn);
  int* buf = red_buf(red, parity);
  if (lane_id() == 0) {
    buf[threadIdx.x >> 6] = (int)a;
    buf[kFinalWaves + (threadIdx.x >> 6)] = (int)b;
  }
  __syncthreads();
  mx = 0u;
  mn = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < kFinalWaves; ++i) {
    mx = max(mx, (uint32_t)buf[i]);
    mn = min(mn, (uint32_t)buf[kFinalWaves + i]);
  }
}

// Exclusive prefix sum over thread order; *total gets the workgroup sum.
__device__ __forceinline__ int block_excl_scan(int v, int* total, int* red, int& parity) {
  const int w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  int* buf = red_buf(red, parity);
  if (lane_id() == 63) buf[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kFinalWaves; ++i) {
    const int s = buf[i];
    before += i < w ? s : 0;
    tot += s;
  }
  *total = tot;
  return before + x - v;
}

// Exact top-k (1 <= k <= number of real keys) of up to kFinalThreads * E keys held in
// registers: thread t holds elements t*E .. t*E+E-1 (keys kv; elements past the end hold the
// sentinel key).  Writes the values of the chosen elements, in element order, to out[0..k)
// (LDS) and returns the k-th element's key and value.  elem(j) names this thread's element j:
// its value itself when elem_is_value (a value held in registers, no further reads), else
// its element index, which val() turns into the value after the selection.
//
// K, the k-th largest key, is found digit by digit (a radix select).  All real keys share
// the bits of their maximum and minimum above the highest bit where those differ; below it,
// each pass histograms the next 8 bits (fewer in the last pass) of the keys that still
// match the digits found so far (LDS atomics), and after one barrier every wave reads the
// 256 counts and takes the largest digit whose suffix count still reaches the number of
// keys wanted from the bracket.  The keys of larger digits are all selected; the wanted
// count drops by them.  The search ends after the last bit, or as soon as the bracket holds
// exactly the keys still wanted (K is then its smallest key, one more exchange).  The keys
// equal to K that are taken are the first k - #{> K} in element order.  Sentinels never
// count.
// Three histograms rotate, so one barrier per pass suffices: the one a pass clears was last
// read two passes before, which every wave finished before the previous barrier.
// red: 4 * kFinalWaves ints of LDS (16-byte aligned); note: 1 int; hist: kHistWords.
struct KthKey {
  uint32_t key;
  int idx;
};

template <int E, class Val, class Elem>
__device__ KthKey block_topk_regs(const uint32_t (&kv)[E], Val val, Elem elem, bool elem_is_value,
                                  int k, int* out, int* red, int* note, uint32_t* hist) {
  const int tid = threadIdx.x, lane = tid & 63;
  int parity = 0;
  for (int i = tid; i < 2 * kHistSet; i += kFinalThreads) hist[i] = 0u;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    mx = max(mx, kv[j]);
    mn = min(mn, kv[j] == kSentinel ? 0xFFFFFFFFu : kv[j]);
  }
  block_max_min(mx, mn, red, parity);  // its barrier also publishes the cleared histograms
  uint32_t K = mx;
  if (mx != mn) {
    int need = k;                              // keys wanted from the current bracket
    int lo_bit = 32 - __builtin_clz(mx ^ mn);  // bits lo_bit .. 31 are those of mx
    uint32_t prefix = lo_bit >= 32 ? 0u : (mx >> lo_bit) << lo_bit;
    bool open = true;  // the bracket still holds more keys than are wanted from it
#pragma unroll 1
    for (int pass = 0; lo_bit > 0; ++pass) {  // uniform
      const int width = lo_bit < kRadixBits ? lo_bit : kRadixBits;
      const int sh = lo_bit - width;
      uint32_t* h = hist + kHistSet * (pass % 3);
      if (pass > 0) {
        uint32_t* h2 = hist + kHistSet * ((pass + 1) % 3);
        for (int i = tid; i < kHistSet; i += kFinalThreads) h2[i] = 0u;
      }
      const uint64_t want = (uint64_t)prefix >> lo_bit;  // the bits found so far
      uint32_t* const hc = h + kHistStride * (lane & (kHistCopies - 1));
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (kv[j] != kSentinel && ((uint64_t)kv[j] >> lo_bit) == want)
          atomicAdd(&hc[__builtin_amdgcn_ubfe(kv[j], sh, width)], 1u);
      __syncthreads();
      // lane l holds the counts of digits 4l .. 4l+3 (summed over the copies); suffix sums
      // over the digits, from the lane's own four and the totals of the lanes above it
      v4i c4 = *reinterpret_cast<const v4i*>(&h[4 * lane]);
#pragma unroll
      for (int c = 1; c < kHistCopies; ++c) c4 += *reinterpret_cast<const v4i*>(&h[kHistStride * c + 4 * lane]);
      const int s3 = c4[3], s2 = s3 + c4[2], s1 = s2 + c4[1], s0 = s1 + c4[0];
      const int incl = wave_incl_scan(s0);
      const int above_lane = __builtin_amdgcn_readlane(incl, 63) - incl;
      const int S0 = above_lane + s0, S1 = above_lane + s1, S2 = above_lane + s2,
                S3 = above_lane + s3;
      // the digit D: largest with S(D) >= need (S falls as the digit grows)
      const uint64_t ok = __ballot(S0 >= need);  // lane 0 always (S(0) = all in bracket)
      const int L = 63 - __builtin_clzll(ok);
      const int i_l = S3 >= need ? 3 : S2 >= need ? 2 : S1 >= need ? 1 : 0;
      const int s_next = i_l == 3 ? above_lane : i_l == 2 ? S3 : i_l == 1 ? S2 : S1;
      const int s_at = i_l == 3 ? S3 : i_l == 2 ? S2 : i_l == 1 ? S1 : S0;
      const int D = 4 * L + __builtin_amdgcn_readlane(i_l, L);
      const int taken = __builtin_amdgcn_readlane(s_next, L);   // keys of larger digits
      const int in_d = __builtin_amdgcn_readlane(s_at, L) - taken;  // keys of digit D
      need -= taken;
      prefix |= (uint32_t)D << sh;
      lo_bit = sh;
      if (in_d == need) {  // uniform: every key left in the bracket is taken
        open = false;
        break;
      }
    }
    K = prefix;
    if (!open && lo_bit > 0) {
      // the k-th key is the smallest of the bracket
      const uint64_t want = (uint64_t)prefix >> lo_bit;
      uint32_t bmin = 0xFFFFFFFFu, dummy = 0u;
#pragma unroll
      for (int j = 0; j < E; ++j)
        if (kv[j] != kSentinel && ((uint64_t)kv[j] >> lo_bit) == want) bmin = min(bmin, kv[j]);
      block_max_min(dummy, bmin, red, parity);
      K = bmin;
    }
  }
  // one scan of (#{> K}, #{== K}) per thread (each field stays below 2^16): equal keys are
  // taken in element order until r = k - #{> K} of them are, so the output position is the
  // keys above K before this thread plus min(equal keys before it, r)
  int n_eq = 0, n_gt = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    n_eq += kv[j] == K ? 1 : 0;
    n_gt += kv[j] > K ? 1 : 0;
  }
  int tot;
  const int before = block_excl_scan(n_gt | (n_eq << 16), &tot, red, parity);
  const int r = k - (tot & 0xFFFF);  // equal keys taken (>= 1)
  const int eq_before = before >> 16;
  int pos = (before & 0xFFFF) + min(eq_before, r);
  int e_rank = eq_before;
  // values, or element indices (no loads in this loop) that every thread then turns, k / 512
  // of them, into values with independent loads
#pragma unroll
  for (int j = 0; j < E; ++j) {
    bool take = kv[j] > K;
    if (kv[j] == K) {
      take = e_rank < r;
      if (e_rank == r - 1) *note = elem(j);
      ++e_rank;
    }
    if (take) out[pos++] = elem(j);
  }
  __syncthreads();
  if (elem_is_value) return KthKey{K, *note};
  const int I = val(*note);
#pragma unroll 4
  for (int i = tid; i < k; i += kFinalThreads) out[i] = val(out[i]);
  __syncthreads();
  return KthKey{K, I};
}

// Smallest per-thread count E in {8, 16, 32, 64} with kFinalThreads * E >= n.
__host__ __device__ __forceinline__ int final_per_thread(int n) {
  return n <= 8 * kFinalThreads ? 8 : n <= 16 * kFinalThreads ? 16 : n <= 32 * kFinalThreads ? 32 : 64;
}

// The same selection over get(0 .. n-1) / val(0 .. n-1) (1 <= k <= real keys, any n): up to
// kFinalTile elements go through registers, more are re-read tile by tile (slow; only the
// exact fallbacks of the final pass come here).
template <int E, class Get, class Val>
__device__ KthKey block_topk_e(Get get, Val val, int n, int k, int* out, int* red, int* note,
                               uint32_t* hist) {
  const int tid = threadIdx.x;
  uint32_t kv[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = tid * E + j;
    kv[j] = e < n ? get(e) : kSentinel;
  }
  return block_topk_regs<E>(kv, val, [tid](int j) { return tid * E + j; }, false, k, out, red,
                            note, hist);
}

// (get / val are taken by value: they hold a pointer or two, and the slow path is a call.)
template <class Get, class Val>
__device__ KthKey block_topk(Get get, Val val, int n, int k, int* out, int* red, int* note,
                             uint32_t* hist) {
  const int tid = threadIdx.x;
  if (n <= kFinalTile) {
    switch (final_per_thread(n)) {
      case 8: return block_topk_e<8>(get, val, n, k, out, red, note, hist);
      case 16: return block_topk_e<16>(get, val, n, k, out, red, note, hist);
      default: return block_topk_e<32>(get, val, n, k, out, red, note, hist);
    }
  }
  constexpr int E = 16;  // tile of the re-read path
  constexpr int kTile = kFinalThreads * E;
  int parity = 0;
  const int n_tiles = (n + kTile - 1) / kTile;
  auto count = [&](uint32_t T, bool strict) {
    int c = 0;
    for (int tile = 0; tile < n_tiles; ++tile)
#pragma unroll 4
      for (int j = 0; j < E; ++j) {
        const int e = tile * kTile + tid * E + j;
        const uint32_t x = e < n ? get(e) : kSentinel;
        c += __popcll(__ballot(strict ? x > T : x >= T));
      }
    return c;
  };
  uint32_t K = 0;
#pragma unroll 1
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t T = K | (1u << bit);
    if (block_sum_waves(count(T, false), red, parity) >= k) K = T;
  }
  const int r = k - block_sum_waves(count(K, true), red, parity);
  if (tid == 0) *note = -1;
  int eq_base = 0, out_base = 0;
#pragma unroll 1
  for (int tile = 0; tile < n_tiles; ++tile) {
    uint32_t tk[E];
    int n_eq = 0, n_gt = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = tile * kTile + tid * E + j;
      tk[j] = e < n ? get(e) : kSentinel;
      n_eq += tk[j] == K ? 1 : 0;
      n_gt += tk[j] > K ? 1 : 0;
    }
    int eq_tot, take_tot;
    const int eq_before = eq_base + block_excl_scan(n_eq, &eq_tot, red, parity);
    const int eq_take = min(max(r - eq_before, 0), n_eq);
    int pos = out_base + block_excl_scan(n_gt + eq_take, &take_tot, red, parity);
    int e_rank = eq_before;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int e = tile * kTile + tid * E + j;
      bool take = tk[j] > K;
      if (tk[j] == K) {
        take = e_rank < r;
        if (e_rank == r - 1) *note = val(e);
        ++e_rank;
      }
      if (take) out[pos++] = val(e);
    }
    eq_base += eq_tot;
    out_base += take_tot;
    if (out_base >= k) break;  // uniform
  }
  __syncthreads();
  const int I = *note;
  __syncthreads();
  return KthKey{K, I};
}

}  // namespace dsa
