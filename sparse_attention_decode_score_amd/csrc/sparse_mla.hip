// Stage 3 of the DSA decode path: exact MLA over the selected latent slots (NoPE).
//
// The vLLM Kimi K3.1 Pro page runs MLA exactly over only the 2,048 tokens the indexer
// keeps ("What changed in Kimi K3.1 Pro"), reading the full 576-byte FP8 latent of each
// ("Sparse attention cuts long-context decode bandwidth"); keys are all 576 dims, values
// the first 512, 96 heads share one latent.  Its MI355X kernel reads the selected tokens
// straight from the FP8 cache with one workgroup per query row across the heads, and small
// batches add parallelism inside each row ("Context-parallel sparse-attention prefill"):
// here that is the split index s of a (split, row) workgroup.
//
// Workgroup = 8 waves, one per CU (two per SIMD).  The split's slots sit in LDS; 64-token
// latent tiles are gathered straight into a 3-tile LDS ring with 16-byte global-to-LDS loads
// (every wave moves 4 or 5 of a tile's 36 16-byte columns; lane l moves token l; the first
// two tiles come from the two value waves alone while the others prepare the query), so
// tile t+2 is in flight while tile t is used and no register holds gathered bytes.  A tile is
// stored column-blocked, [36 columns][64 tokens][16 B], which serves both products without
// bank conflicts:
//   logits  S[token][head] = L8[32 tokens x 576] * Q8^T   (9 x v_mfma 32x32x64 per 32 tokens)
//           by waves 0..5, wave w for head tile w/2 (32 heads) and 32-token block w%2, with
//           its head tile's E4M3 query held in registers (72 VGPRs);
//   values  O^T[dim][head] += V8^T[32 dims x 64 tokens] * P8^T[64 tokens x 32 heads]
//           by all 8 waves over 48 (head tile, 32-dim tile) accumulators (see the roles
//           below), V read through ds_read_b64_tr_b8 (8 tokens of one dim per lane) so the
//           latent is never transposed in memory; each lane's accumulators belong to one head,
//           so per-head rescaling and normalisation are lane-local.
// Softmax per (head, 32-token block): the block's maximum is rounded up to an integer m_b in
// log2 units, p = 2^(x - m_b) in (0, 1], and p * 2^8 enters the value product as a two-term
// E4M3 pair (hi, and the residual scaled by 2^4) whose scale 2^(m_b - m_ref - 8) (and 2^-4
// less for the residual) is the E8M0 operand scale of the MFMA: one scale per lane, and a
// lane holds exactly one head's 32-token block.  So every block keeps ~8 significant bits
// however far its maximum lies below the row's, and the accumulator's reference m_ref (an
// integer, raised only when a block exceeds it by more than 2^16) changes by exact powers of
// two.  Block sums of the fp32 p give the softmax denominator and the LSE.
//
// One barrier per tile.  In the step of tile t every wave: waits for its own gathers of tile
// t; barrier; requests tile t+2 into the buffer tile t-1 used; multiplies tile t-1's
// probabilities (published before the barrier) with its value registers; then (waves 0..5)
// forms tile t's logits and probabilities into a double-buffered LDS exchange, and (all)
// reads tile t's values into registers, so the tile's LDS buffer is free at the next barrier.
#include <mutex>
#include <type_traits>

#include "dsa_device.hpp"
#include "dsa_internal.hpp"
#include "dsa_select.hpp"
#include "dsa_topk_final.hpp"

namespace dsa {

namespace {

constexpr int kTile = 64;
constexpr int kThreads = 512;     // 8 waves
constexpr int kWaves = kThreads / 64;
constexpr int kRing = 3;          // latent tiles in LDS: the one in use and two in flight
constexpr int kCols = kLatDim / 16;          // 36 16-byte columns per latent row
constexpr int kTileBytes = kTile * kLatDim;  // 36,864
constexpr int kSlotsLds = 4096;   // slots of a split held in LDS (k <= 4096)
constexpr int kDutyWaves = 6;     // waves forming logits: 3 head tiles x 2 token blocks
constexpr int kQStride = 592;     // staging row of the query codes (576 + 16: conflict-free reads)
constexpr int kTau = 16;          // accumulator reference slack, log2 units
constexpr int kNoMax = -(1 << 29);  // block maximum of a block without a visible token
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The latent row gathered for padding: a slot of -1 or a position past the split.
__device__ __attribute__((aligned(64))) uint8_t g_zero_row[kLatDim];

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier for LDS data, after this wave's global-to-LDS gathers have completed down
// to the newest `pending` instructions (the loads' completion is not tracked by the compiler).
// The memory clobber keeps every LDS access on its side.
template <int pending>
__device__ __forceinline__ void ring_barrier() {
  static_assert(pending >= 0 && pending < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(pending) : "memory");
}

// The value operand of ND dim tiles, read with ds_read_b64_tr_b8 from LDS byte address
// `addr` (+ 2048 per dim tile; + 0, 128, 512, 640 for tokens +0, +8, +32, +40: the operand's
// K positions 16 g .. +15 and 32 + 16 g .. +15, see the probabilities).  The reads and their wait are one asm
// block: written as builtins, the compiler orders these transposed reads after every
// global-to-LDS gather in flight (it cannot tell they touch another buffer), which would
// drain the ring at every tile.
template <int ND>
__device__ __forceinline__ void read_values(uint32_t addr, v8i (&vb)[ND]);

#define DSA_TR(i, off) "ds_read_b64_tr_b8 %" #i ", %[a] offset:" #off "\n\t"
template <>
__device__ __forceinline__ void read_values<3>(uint32_t addr, v8i (&vb)[3]) {
  v2i r[12];
  asm volatile(DSA_TR(0, 0) DSA_TR(1, 128) DSA_TR(2, 512) DSA_TR(3, 640)
               DSA_TR(4, 2048) DSA_TR(5, 2176) DSA_TR(6, 2560) DSA_TR(7, 2688)
               DSA_TR(8, 4096) DSA_TR(9, 4224) DSA_TR(10, 4608) DSA_TR(11, 4736)
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                 "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11])
               : [a] "v"(addr)
               : "memory");
#pragma unroll
  for (int d = 0; d < 3; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vb[d][2 * j] = r[4 * d + j][0];
      vb[d][2 * j + 1] = r[4 * d + j][1];
    }
}
template <>
__device__ __forceinline__ void read_values<5>(uint32_t addr, v8i (&vb)[5]) {
  v2i r[20];
  asm volatile(DSA_TR(0, 0) DSA_TR(1, 128) DSA_TR(2, 512) DSA_TR(3, 640)
               DSA_TR(4, 2048) DSA_TR(5, 2176) DSA_TR(6, 2560) DSA_TR(7, 2688)
               DSA_TR(8, 4096) DSA_TR(9, 4224) DSA_TR(10, 4608) DSA_TR(11, 4736)
               DSA_TR(12, 6144) DSA_TR(13, 6272) DSA_TR(14, 6656) DSA_TR(15, 6784)
               DSA_TR(16, 8192) DSA_TR(17, 8320) DSA_TR(18, 8704) DSA_TR(19, 8832)
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
                 "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
                 "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]),
                 "=&v"(r[17]), "=&v"(r[18]), "=&v"(r[19])
               : [a] "v"(addr)
               : "memory");
#pragma unroll
  for (int d = 0; d < 5; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vb[d][2 * j] = r[4 * d + j][0];
      vb[d][2 * j + 1] = r[4 * d + j][1];
    }
}
#undef DSA_TR

// Two floats -> two bf16 (round to nearest even) / two fp16 in one dword, low half first.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {  // one v_cvt_pk_bf16_f32
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{x0, x1}, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16(float x0, float x1) {  // one v_cvt_pk_f16_f32
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{x0, x1}, f16x2_t));
}

// Workgroup barrier for LDS data only (global loads and gathers stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Output of a workgroup: the row's bf16 O and LSE (one split), or its split's partial O
// (fp32, or fp16 divided by the latent scale, which bounds it by 448) and LSE.
enum PartMode { kDirect = 0, kPartF32 = 1, kPartF16 = 2 };

struct MlaSmem {
  uint8_t lat[kRing][kTileBytes];            // [column][token][16 B] per tile
  uint8_t pbuf[2][3][2][2][2][32][16];       // [tile parity][head tile][block][hi/lo][half][head][16 tokens]
  int bmax[2][3][2][32];                     // integer block maxima (log2 units), kNoMax if empty
  float bsum[2][3][2][32];                   // block sums of 2^(x - m_b)
  uint8_t qtail[4][kMlaHeads][16];           // E4M3 query dims 512..575: [16-byte part][head][16 B]
  int32_t slot_l[kSlotsLds];
};
// The final top-k pass of the fused kernel runs before any of the above is used: its
// scratch overlays the latent ring and the exchange buffers, and its output (the row's
// selected token indices) is written straight into slot_l.
struct SelectSmem {
  uint32_t lkey[kFinalTile];
  int32_t lidx[kFinalTile];
  alignas(16) int red[4 * kFinalWaves];
  int note;
  alignas(16) uint32_t hist[kHistWords];
};
static_assert(sizeof(SelectSmem) <= offsetof(MlaSmem, slot_l), "selection scratch overlaps slot_l");
static_assert(kFinalThreads == kThreads, "the fused kernel runs the final pass on its own threads");
static_assert(sizeof(MlaSmem) <= 160 * 1024, "LDS budget of one workgroup");
static_assert(kMlaHeads * kQStride <= kTileBytes + sizeof(MlaSmem::pbuf),
              "query staging fits ring buffer 2 and the probability exchange");
static_assert(offsetof(MlaSmem, pbuf) == 3 * kTileBytes, "staging spans buffer 2 and pbuf");

// Inputs of the fused final top-k pass (stage 2) of the select-and-attend kernel.
struct SelectArgs {
  const int32_t* cu_q;
  const int32_t* seq_lens;
  int num_seqs;
  float* scores;  // written only by a recomputation (rs.q set)
  int64_t score_stride;
  int num_groups;
  int64_t row_cap;
  const uint32_t* cand_key;
  const int32_t* cand_idx;
  const ChunkInfo* info;
  IndexRescore rs;
  const int32_t* block_table;
  int bt_stride;
  int32_t* topk_idx;   // optional outputs, written by split 0 of each row
  int32_t* topk_slot;
  WsLayout layout;     // the candidate workspace's layout record
};

template <bool SELECT>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(
    SelectArgs sel, const uint16_t* __restrict__ q, const uint8_t* __restrict__ q8_in,
    const float* __restrict__ qs_in, const uint8_t* __restrict__ lat_pages, int64_t page_stride,
    float lat_scale, const int32_t* __restrict__ topk_slot, int k, float sm_scale,
    int num_splits, int n_q, int mode, void* __restrict__ o_part, float* __restrict__ lse_part,
    uint16_t* __restrict__ out_bf16, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) MlaSmem sm;
  auto& slot_l = sm.slot_l;

  // Workgroups are dealt to the 8 XCDs round-robin by linear id; when the grid divides
  // evenly, all splits of a row go to one XCD, so the row's query and candidates (read by
  // every split) come from that XCD's L2 after the first read.
  int s = blockIdx.x, row = blockIdx.y;
  {
    const int total = num_splits * n_q;
    if ((total & 7) == 0) {
      const int lin = blockIdx.x + num_splits * blockIdx.y;
      const int i = (lin & 7) * (total >> 3) + (lin >> 3);
      row = i / num_splits;
      s = i - row * num_splits;
    }
  }
  const int beg = (int)((int64_t)s * k / num_splits);
  const int end = (int)((int64_t)(s + 1) * k / num_splits);
  const int n_tok = end - beg;
  const int n_tiles = (n_tok + kTile - 1) / kTile;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31, g = lane >> 5;

  // The row's query goes to LDS first, by direct gathers, so that its latency hides behind
  // the selection or the slot-list load: bf16 values (110,592 bytes: the three latent
  // buffers exactly) or prepared E4M3 codes (55,296 bytes) and their 96 scales just after
  // them.  The selection leaves that LDS alone unless it resends groups; it then waits for
  // the gathers first, and the query is staged again after it.
  constexpr int kQ8Bytes = kMlaHeads * kLatDim;  // 55,296
  auto stage_query = [&]() {
    DSA_LDS uint8_t* dst = (DSA_LDS uint8_t*)(&sm.lat[0][0]);
    if (q8_in) {
      const uint8_t* qrow = q8_in + (int64_t)row * kQ8Bytes;
      for (int c = wave; c < kQ8Bytes / 1024; c += kWaves)  // wave-uniform
        __builtin_amdgcn_global_load_lds(qrow + 1024 * c + 16 * lane, dst + 1024 * c, 16, 0, 0);
      if (wave == 0 && lane < kMlaHeads / 4)  // the scales: 384 bytes
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(qs_in + (int64_t)row * kMlaHeads) + 16 * lane,
                                         dst + kQ8Bytes, 16, 0, 0);
    } else {
      constexpr int kQChunks = kMlaHeads * kLatDim * 2 / 1024;  // 108 chunks of 1 KB
      static_assert(kQChunks * 1024 == kRing * kTileBytes, "the bf16 query fills the ring");
      const uint8_t* qrow = reinterpret_cast<const uint8_t*>(q + (int64_t)row * kMlaHeads * kLatDim);
      for (int c = wave; c < kQChunks; c += kWaves)  // wave-uniform
        __builtin_amdgcn_global_load_lds(qrow + 1024 * c + 16 * lane, dst + 1024 * c, 16, 0, 0);
    }
  };
  static_assert(kQ8Bytes + 4 * kMlaHeads <= kRing * kTileBytes, "the prepared query fits the ring");
  stage_query();
  bool q_in_lds = true;

  if constexpr (SELECT) {
    // stage 2 for this row (every split of the row runs it: it is latency-bound), then the
    // split's slice of the selected tokens -> physical slots in slot_l
    SelectSmem& ss = *reinterpret_cast<SelectSmem*>(&sm);
    int b, pos;
    row_of(sel.cu_q, sel.seq_lens, sel.num_seqs, row, b, pos);
    const FinalScratch sc{ss.lkey, ss.lidx, ss.red, &ss.note, ss.hist};
    const int32_t* bt = sel.block_table + (int64_t)b * sel.bt_stride;
    // a resend overwrites the staged query: its gathers must have landed first
    auto before_resend = [&]() {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      q_in_lds = false;
    };
    // candidates written for another layout: nothing is selected (see WsLayout)
    const bool layout_ok = ws_layout_ok(sel.layout);
    if (!layout_ok && s == 0) flag_ws_layout(sel.layout);
    const int n_out = layout_ok ? final_select_row(row, pos + 1, sel.scores, sel.score_stride, k,
                                                   sel.num_groups, sel.row_cap, sel.cand_key,
                                                   sel.cand_idx, sel.info, sel.rs, bt, slot_l, sc,
                                                   before_resend)
                                : 0;
    auto to_slot = [&](int t) { return t < 0 ? -1 : bt[t >> 6] * kPage + (t & (kPage - 1)); };
    if (s == 0 && (sel.topk_idx || sel.topk_slot)) {
      for (int i = threadIdx.x; i < k; i += kThreads) {
        const int t = i < n_out ? slot_l[i] : -1;
        if (sel.topk_idx) sel.topk_idx[(int64_t)row * k + i] = t;
        if (sel.topk_slot) sel.topk_slot[(int64_t)row * k + i] = to_slot(t);
      }
    }
    constexpr int kPer = kSlotsLds / kThreads;
    int mine[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = threadIdx.x + u * kThreads;
      mine[u] = (j < n_tok && beg + j < n_out) ? to_slot(slot_l[beg + j]) : -1;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int j = threadIdx.x + u * kThreads;
      if (j < n_tok) slot_l[j] = mine[u];
    }
  } else {
    // the split's slot list -> LDS
    const int32_t* slots = topk_slot + (int64_t)row * k + beg;
    for (int i = threadIdx.x; i < n_tok; i += kThreads) slot_l[i] = slots[i];
  }
  // slot_l holds the split's slots, the selection scratch is dead, and every query gather
  // has landed (a resend overwrote the staged query: it is staged again)
  if (!q_in_lds) stage_query();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- gathers: wave w moves columns w, w+8, .. (< 36) of every row of a tile; lane l
  // moves token l.  Tiles past the split gather zero rows into a buffer nobody reads, so
  // every wave issues a fixed number of loads per tile (tiles 0 and 1: the value waves
  // only, see issue_value_half) and its wait counts are fixed.
  // Steps jj0 .. jj1-1 (of 5) of tile t's gathers; a wave may issue them in pieces.
  auto issue = [&](int t, int jj0, int jj1) {
    const int j = t * kTile + lane;
    const int slot = j < n_tok ? slot_l[j] : -1;
    const uint8_t* src = slot >= 0 ? lat_pages + (int64_t)(slot >> 6) * page_stride +
                                         (int64_t)(slot & (kPage - 1)) * kLatDim
                                   : g_zero_row;
    DSA_LDS uint8_t* dst = (DSA_LDS uint8_t*)(&sm.lat[t % kRing][0]);
#pragma unroll
    for (int jj = 0; jj < 5; ++jj) {
      const int c = wave + kWaves * jj;
      if (jj >= jj0 && jj < jj1 && (jj < 4 || c < kCols))  // wave-uniform
        __builtin_amdgcn_global_load_lds(src + 16 * c, dst + 1024 * c, 16, 0, 0);
    }
  };
  // All of tile t's gathers from the two value waves: wave 6 the even columns, wave 7 the
  // odd ones (18 each).  Tiles 0 and 1 go out this way, so that the duty waves prepare the
  // query meanwhile instead of queueing behind 80 gathers.
  auto issue_value_half = [&](int t) {
    const int j = t * kTile + lane;
    const int slot = j < n_tok ? slot_l[j] : -1;
    const uint8_t* src = slot >= 0 ? lat_pages + (int64_t)(slot >> 6) * page_stride +
                                         (int64_t)(slot & (kPage - 1)) * kLatDim
                                   : g_zero_row;
    DSA_LDS uint8_t* dst = (DSA_LDS uint8_t*)(&sm.lat[t % kRing][0]);
    const int c0 = wave - kDutyWaves;  // 0 or 1
#pragma unroll
    for (int i = 0; i < kCols / 2; ++i)
      __builtin_amdgcn_global_load_lds(src + 16 * (c0 + 2 * i), dst + 1024 * (c0 + 2 * i), 16, 0, 0);
  };

  // Two roles, so that no wave needs more than 256 registers and every SIMD (waves w and
  // w + 4) carries the same matrix work per tile (37-38 MFMAs):
  //  duty waves 0..5   logits of head tile w/2 for token block w%2 (its E4M3 query in
  //                    registers), and the values of that head tile for dim tiles
  //                    6 + 5 (w%2) .. +4 (5 accumulators);
  //  value waves 6, 7  the values of all three head tiles for dim tiles 3 (w-6) .. +2
  //                    (9 accumulators).
  auto run = [&](auto role) {
    constexpr int ROLE = decltype(role)::value;  // 0: duty, PV first; 1: duty, PV last; 2: value
    constexpr bool DUTY = ROLE < 2;
    constexpr bool PV_FIRST = ROLE != 1;
    constexpr int NH = DUTY ? 1 : 3;  // head tiles whose values this wave accumulates
    constexpr int ND = DUTY ? 5 : 3;  // dim tiles (32 dims each)
    const int ht_d = wave >> 1, blk = wave & 1;
    const int ht0 = DUTY ? ht_d : 0;
    const int dt0 = DUTY ? 6 + 5 * blk : 3 * (wave - kDutyWaves);

    // ---- the query: the row's 96 x 576 E4M3 query goes to a staging area (ring buffer 2 and
    // the probability exchange, unused until the first barrier of the loop), 4 threads per
    // head; then every duty wave loads its head tile's codes as the B operand of the logits:
    // lane (n, g) holds head 32 ht + n, bytes 64 kb + 32 g .. +31 of each 64-byte chunk kb.
    // A bf16 query is read from LDS before the first two tiles' gathers and quantised after
    // them.
    uint8_t* const qstage = &sm.lat[2][0];   // [96][kQStride] codes; scales in bsum
    float* const qsc = &sm.bsum[0][0][0][0];
    // every wave reads its part of the staged query (4 threads per head, 144 dims each)
    // before any gather may overwrite it
    const bool qthread = threadIdx.x < 4 * kMlaHeads;
    const int qh = threadIdx.x >> 2, qpart = threadIdx.x & 3;
    v4i raw[18];
    float qs_given = 0.f;
    if (qthread) {
      if (q8_in) {
        const uint8_t* src = &sm.lat[0][0] + qh * kLatDim + qpart * 144;
#pragma unroll
        for (int i = 0; i < 9; ++i) raw[i] = *reinterpret_cast<const v4i*>(src + 16 * i);
        qs_given = reinterpret_cast<const float*>(&sm.lat[0][0] + kQ8Bytes)[qh];
      } else {
        const uint8_t* src = &sm.lat[0][0] + (qh * kLatDim + qpart * 144) * 2;
#pragma unroll
        for (int i = 0; i < 18; ++i) raw[i] = *reinterpret_cast<const v4i*>(src + 16 * i);
      }
    }
    lds_barrier();
    if constexpr (!DUTY) {
      issue_value_half(0);
      issue_value_half(1);
    }
    if (q8_in && qthread) {
      uint8_t* dst = qstage + qh * kQStride + qpart * 144;
#pragma unroll
      for (int i = 0; i < 9; ++i) *reinterpret_cast<v4i*>(dst + 16 * i) = raw[i];
      if (qpart == 0) qsc[qh] = qs_given;
    }
    if (!q8_in && qthread) {
      uint8_t* dst = qstage + qh * kQStride + qpart * 144;
      // one power-of-two scale per head: the smallest 2^e with absmax <= 448 * 2^e
      float am = 0.f;
#pragma unroll
      for (int i = 0; i < 18; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          am = fmaxf(am, fmaxf(fabsf(bf16_lo((uint32_t)raw[i][j])), fabsf(bf16_hi((uint32_t)raw[i][j]))));
      am = fmaxf(am, __shfl_xor(am, 1, 64));
      am = fmaxf(am, __shfl_xor(am, 2, 64));
      const int e = pow2_scale_exp(am);
      const float inv = ldexpf(1.0f, -e);
#pragma unroll
      for (int i = 0; i < 9; ++i) {
        v4i c;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w0 = (uint32_t)raw[2 * i + j / 2][2 * (j % 2)];
          const uint32_t w1 = (uint32_t)raw[2 * i + j / 2][2 * (j % 2) + 1];
          c[j] = (int)cvt4_e4m3(bf16_lo(w0) * inv, bf16_hi(w0) * inv, bf16_lo(w1) * inv,
                                bf16_hi(w1) * inv);
        }
        *reinterpret_cast<v4i*>(dst + 16 * i) = c;
      }
      if (qpart == 0) qsc[qh] = ldexpf(1.0f, e);
    }
    lds_barrier();  // the staged query is visible (the gathers stay in flight)
    v8i qb[DUTY ? 8 : 1];  // chunks 0..7; chunk 8 (dims 512..575) stays in LDS (qtail)
    float mult = 0.f;
    if constexpr (DUTY) {
      const int h = 32 * ht_d + n;
      const uint8_t* qr = qstage + h * kQStride + 32 * g;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const v4i a0 = *reinterpret_cast<const v4i*>(qr + 64 * kb);
        const v4i a1 = *reinterpret_cast<const v4i*>(qr + 64 * kb + 16);
        qb[kb] = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
      mult = qsc[h] * lat_scale * sm_scale * kLog2e;
      // the last chunk goes to its own LDS array (read back at every tile), which keeps the
      // duty waves within their registers; published by the first barrier of the loop
      if (blk == 0) {
        *reinterpret_cast<v4i*>(&sm.qtail[2 * g][h][0]) = *reinterpret_cast<const v4i*>(qr + 512);
        *reinterpret_cast<v4i*>(&sm.qtail[2 * g + 1][h][0]) =
            *reinterpret_cast<const v4i*>(qr + 512 + 16);
      }
    }

    v16f acc[NH][ND];  // O^T: lane (n, g) holds head 32 (ht0 + hh) + n, dims 32 (dt0 + dd) +
                       // 8 a + 4 g + c in register 4 a + c
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int dd = 0; dd < ND; ++dd) acc[hh][dd] = v16f{};
    int m_ref[NH];    // accumulator reference of head 32 ht + n (log2 units), same in every wave
    float z_run[NH];  // this lane's block-g share of head 32 ht + n's softmax sum
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      m_ref[hh] = kNoMax;
      z_run[hh] = 0.f;
    }
    // V operand of the last tile read: dims 32 dt + n, tokens 16 g .. +15 and 32 + 16 g .. +15
    // (the K positions of lane (n, g)).  16-lane group vgrp reads the 16 dims of column
    // 2 dt + vgrp % 2 for 8 tokens at a time; lanes 2r, 2r+1 address the two halves of token
    // row r
    v8i vb[ND];

    // ---- values of tile t-1 (PV): O^T += V8^T * P8^T with the blocks' E8M0 scales
    auto values_of = [&](int tp, int n, int g) {
      const int pb = tp & 1;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int ht = ht0 + hh;
        const int mi = sm.bmax[pb][ht][g][n];
        const float zb = sm.bsum[pb][ht][g][n];
        const int mnew = max(mi, __shfl_xor(mi, 32, 64));
        if (__ballot(mnew > m_ref[hh] + kTau) != 0ull) {
          // rare: raise the reference and rescale by an exact power of two (every
          // accumulator register of lane (n, g) belongs to head n)
          const int mr = max(m_ref[hh], mnew);
          const float f = exp2f((float)(m_ref[hh] - mr));
          m_ref[hh] = mr;
          z_run[hh] *= f;
#pragma unroll
          for (int dd = 0; dd < ND; ++dd) acc[hh][dd] *= f;
        }
        const int e = max(mi - m_ref[hh], -200);  // <= kTau
        z_run[hh] += ldexpf(zb, e);
        const int sc_hi = min(max(127 - 8 + e, 0), 254);
        const int sc_lo = min(max(127 - 12 + e, 0), 254);
        // the FP8 operands of v_mfma_scale 32x32x64 hold, in lane (n, g), K positions
        // 16 g .. +15 in bytes 0..15 and 32 + 16 g .. +15 in bytes 16..31, and the E8M0 scale
        // of lane (n, j) scales K positions 32 j .. 32 j + 31: so lane (n, g) takes tokens
        // 16 g .. +15 of block 0 and of block 1, and supplies block g's scale
        v8i ph, pl;
        ph.lo = *reinterpret_cast<const v4i*>(&sm.pbuf[pb][ht][0][0][g][n][0]);
        ph.hi = *reinterpret_cast<const v4i*>(&sm.pbuf[pb][ht][1][0][g][n][0]);
        pl.lo = *reinterpret_cast<const v4i*>(&sm.pbuf[pb][ht][0][1][g][n][0]);
        pl.hi = *reinterpret_cast<const v4i*>(&sm.pbuf[pb][ht][1][1][g][n][0]);
#pragma unroll
        for (int dd = 0; dd < ND; ++dd) {
          // O^T[dim][head]: the values are the A operand (unscaled), the probabilities the
          // B operand with the block's E8M0 scale
          acc[hh][dd] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb[dd], ph, acc[hh][dd], 0,
                                                                        0, 0, 127, 0, sc_hi);
          acc[hh][dd] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb[dd], pl, acc[hh][dd], 0,
                                                                        0, 0, 127, 0, sc_lo);
        }
      }
    };

#pragma unroll 1
    for (int t = 0; t <= n_tiles; ++t) {
      // tile t is in LDS once every wave's own gathers of it are done (tile t+1 may still
      // be in flight); the barrier also publishes tile t-1's probabilities and frees the
      // buffer tile t-1 used
      // (tiles 0 and 1: 18 gathers each from every value wave and none from the duty waves)
      if (!DUTY && t == 0) ring_barrier<kCols / 2>();
      else if (wave < kCols - 4 * kWaves) ring_barrier<5>();
      else ring_barrier<4>();
      // the lane index as an opaque value of this step: the LDS addresses derived from it are
      // recomputed here (a few ALU ops) instead of being hoisted out of the loop and spilled
      int lane_t = lane;
      asm volatile("" : "+v"(lane_t));
      const int n = lane_t & 31, g = lane_t >> 5;
      const int tile_off = __builtin_amdgcn_readfirstlane((t % kRing) * kTileBytes);
      const uint8_t* tile = &sm.lat[0][0] + tile_off;

      if constexpr (DUTY) {
        if (PV_FIRST && t > 0) values_of(t - 1, n, g);
        if (t < n_tiles) {
          issue(t + 2, 0, 2);
          // ---- logits of head tile ht_d, tokens 32 blk .. +31 of tile t: lane (n, g) gets
          // head 32 ht + n for tokens 8 (i / 4) + 4 g + i % 4 of the block in register i.  The
          // accumulator starts at 0 for a visible token and at -inf for a hidden one, so the
          // softmax below needs no masking.
          const int pb = t & 1;
          const int j0 = t * kTile + 32 * blk;
          const bool vis = j0 + n < n_tok && slot_l[j0 + n] >= 0;
          const uint32_t vmask = (uint32_t)__ballot(vis);  // lanes 0..31: token n of the block
          v16f d;
          if (vmask == 0xFFFFFFFFu) {  // uniform: the whole block is visible
            d = v16f{};
          } else {
            const uint32_t vm_g = vmask >> (4 * g);  // bit 8 a + c: token 8 a + 4 g + c
#pragma unroll
            for (int i = 0; i < 16; ++i) d[i] = ((vm_g >> (8 * (i >> 2) + (i & 3))) & 1u) ? 0.f : -INFINITY;
          }
          if (vmask != 0u) {  // uniform
            const uint8_t* arow = tile + (32 * blk + n) * 16 + 2 * g * 1024;
#pragma unroll
            for (int kb = 0; kb < 9; ++kb) {
              v8i A, B;
              A.lo = *reinterpret_cast<const v4i*>(arow + 4 * kb * 1024);
              A.hi = *reinterpret_cast<const v4i*>(arow + (4 * kb + 1) * 1024);
              if (kb < 8) {
                B = qb[kb < 8 ? kb : 0];
              } else {
                B.lo = *reinterpret_cast<const v4i*>(&sm.qtail[2 * g][32 * ht_d + n][0]);
                B.hi = *reinterpret_cast<const v4i*>(&sm.qtail[2 * g + 1][32 * ht_d + n][0]);
              }
              d = mfma_32x32x64_fp8(A, B, d);
            }
          }
          float mx = d[0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, d[i]);
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          // integer block maximum in log2 units (mult > 0; clamped: far-out logits only
          // saturate it); p * 2^8 = 2^(d * mult + 8 - m_b) in (0, 2^8]
          const int mi = vmask != 0u ? (int)ceilf(fminf(fmaxf(mx * mult, -1e8f), 1e8f)) : kNoMax;
          const float off = 8.0f - (float)mi;
          float zs = 0.f;
          uint8_t* pw = &sm.pbuf[pb][ht_d][blk][0][0][n][0];
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            float ph[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              ph[c] = __builtin_amdgcn_exp2f(fmaf(d[4 * a + c], mult, off));  // -inf -> 0
              zs += ph[c];
            }
            // two-term E4M3: hi = E4M3(p 2^8), lo = E4M3((p 2^8 - hi) 2^4)
            const uint32_t hi = cvt4_e4m3(ph[0], ph[1], ph[2], ph[3]);
            const v2f d01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
            const v2f d23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
            const v2s lo01 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, ph[0] - d01[0],
                                                                      ph[1] - d01[1], 0.0625f, false);
            const v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo01, ph[2] - d23[0],
                                                                    ph[3] - d23[1], 0.0625f, true);
            // tokens 8 a + 4 g .. +3: half a / 2, byte 8 (a % 2) + 4 g
            const int off_b = (a >> 1) * 32 * 16 + 8 * (a & 1) + 4 * g;
            *reinterpret_cast<uint32_t*>(pw + off_b) = hi;
            *reinterpret_cast<v2s*>(pw + 2 * 32 * 16 + off_b) = lo;
          }
          issue(t + 2, 2, 5);
          zs += __shfl_xor(zs, 32, 64);
          if (g == 0) {
            sm.bmax[pb][ht_d][blk][n] = mi;
            sm.bsum[pb][ht_d][blk][n] = zs * (1.0f / 256.0f);
          }
        }
        // the second duty wave of a SIMD takes the values product last: its softmax then
        // runs while the other duty wave's matrix products do
        if (!PV_FIRST && t > 0) values_of(t - 1, n, g);
      } else {
        if (t < n_tiles) issue(t + 2, 0, 5);
        if (t > 0) values_of(t - 1, n, g);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (t < n_tiles) {
        // ---- values of tile t into registers (A operand of the next step's PV)
        const int vgrp = lane_t >> 4, vli = lane_t & 15;
        const uint8_t* vbase = tile + (2 * dt0 + (vgrp & 1)) * 1024 +
                               (16 * (vgrp >> 1) + (vli >> 1)) * 16 + 8 * (vli & 1);
        read_values<ND>((uint32_t)(uintptr_t)(DSA_LDS const uint8_t*)vbase, vb);
      }
    }
    // the zero-row gathers past the split may still be in flight: every wave waits for its
    // own, and the barrier below for everyone's, before the ring holds the output
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // ---------------------------------------------------------------- finalize
    // softmax sum of head 32 ht + n: both block shares; values are latent_scale * L8.  Lane
    // (n, g) owns head n of each accumulator tile, dims 8 a + 4 g .. +3 in registers 4 a ..
    // 4 a + 3.  The 16-bit outputs (bf16 O, or fp16 O / latent_scale partials) are staged in
    // the ring as [96 heads][512 dims] (16-byte chunks swizzled within a head's row) and leave
    // with 16-byte stores; fp32 partials are stored directly.
    lds_barrier();  // the ring is free: no wave reads it any more and every gather has landed
    uint8_t* const ostage = &sm.lat[0][0];
    // one branch on the output mode, outside the unrolled stores
    auto emit = [&](auto mode_tag) {
      constexpr int M = decltype(mode_tag)::value;
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) {
        const int h = 32 * (ht0 + hh) + n;
        const float z = z_run[hh] + __shfl_xor(z_run[hh], 32, 64);
        const bool empty = !(z > 0.f);
        const float f = empty ? 0.f : (M == kPartF16 ? 1.0f : lat_scale) / z;
#pragma unroll
        for (int dd = 0; dd < ND; ++dd) {
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int d = 32 * (dt0 + dd) + 8 * a + 4 * g;
            const v16f& o = acc[hh][dd];
            const float v0 = o[4 * a] * f, v1 = o[4 * a + 1] * f, v2 = o[4 * a + 2] * f,
                        v3 = o[4 * a + 3] * f;
            if constexpr (M == kPartF32) {
              float* op = static_cast<float*>(o_part) + ((int64_t)s * n_q + row) * kMlaHeads * kVDim;
              *reinterpret_cast<v4f*>(op + (int64_t)h * kVDim + d) = v4f{v0, v1, v2, v3};
            } else {
              v2i w;
              w[0] = (int)(M == kDirect ? pack_bf16(v0, v1) : pack_f16(v0, v1));
              w[1] = (int)(M == kDirect ? pack_bf16(v2, v3) : pack_f16(v2, v3));
              // 16-byte chunk (d / 8) of head h's 1 KB row sits at chunk (d / 8) ^ (h % 32):
              // the 32 heads of one store then fall on distinct banks
              *reinterpret_cast<v2i*>(ostage + h * (2 * kVDim) + 16 * ((d >> 3) ^ n) + 8 * g) = w;
            }
          }
        }
        if (DUTY && blk == 0 && g == 0) {  // one wave per head tile writes the LSE
          const float lse_h = empty ? -INFINITY : ((float)m_ref[hh] + log2f(z)) * kLn2;
          if constexpr (M == kDirect) lse_out[(int64_t)row * kMlaHeads + h] = lse_h;
          else lse_part[((int64_t)s * n_q + row) * kMlaHeads + h] = lse_h;
        }
      }
      if constexpr (M != kPartF32) {
        lds_barrier();
        uint8_t* dst = reinterpret_cast<uint8_t*>(
            M == kDirect ? out_bf16 + (int64_t)row * kMlaHeads * kVDim
                         : static_cast<uint16_t*>(o_part) + ((int64_t)s * n_q + row) * kMlaHeads * kVDim);
        constexpr int kPieces = kMlaHeads * kVDim * 2 / 16;  // 6,144 16-byte pieces
#pragma unroll
        for (int i = 0; i < kPieces / kThreads; ++i) {
          const int c = i * kThreads + (int)threadIdx.x;
          const int hc = c >> 6, ch = c & 63;  // head, 16-byte chunk of its row
          *reinterpret_cast<v4i*>(dst + 16 * c) =
              *reinterpret_cast<const v4i*>(ostage + hc * (2 * kVDim) + 16 * (ch ^ (hc & 31)));
        }
      }
    };
    if (mode == kDirect)
      emit(std::integral_constant<int, kDirect>{});
    else if (mode == kPartF16)
      emit(std::integral_constant<int, kPartF16>{});
    else
      emit(std::integral_constant<int, kPartF32>{});
  };
  // waves w and w + 4 share a SIMD: waves 0..3 and 6, 7 run their products first, the
  // duty waves 4, 5 (on the SIMDs of duty waves 0, 1) last
  if (wave < 4)
    run(std::integral_constant<int, 0>{});
  else if (wave < kDutyWaves)
    run(std::integral_constant<int, 1>{});
  else
    run(std::integral_constant<int, 2>{});
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t sparse_mla_workspace_bytes(int n_q, int num_splits) {
  if (num_splits <= 1) return 256;
  const size_t parts = (size_t)num_splits * n_q * kMlaHeads;
  return align256(parts * kVDim * sizeof(uint16_t)) + align256(parts * sizeof(float));
}

static hipError_t launch_mla_common(const SelectArgs* sel, int n_q, const uint16_t* q,
                                    const uint8_t* q8, const float* q_scale,
                                    const uint8_t* latent_pages, int64_t latent_page_stride,
                                    float latent_scale, const int32_t* topk_slot, int k,
                                    float softmax_scale, int num_splits, float* o_part,
                                    float* lse_part, uint16_t* out_bf16, float* lse,
                                    void* workspace, hipStream_t st) {
  int mode = kDirect;
  void* op = o_part;
  float* lp = lse_part;
  if (o_part) {
    mode = kPartF32;
  } else if (num_splits > 1) {
    mode = kPartF16;
    const size_t parts = (size_t)num_splits * n_q * kMlaHeads;
    op = workspace;
    lp = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                  align256(parts * kVDim * sizeof(uint16_t)));
  }
  const dim3 grid((unsigned)num_splits, (unsigned)n_q), block(kThreads);
  if (sel) {
    hipLaunchKernelGGL(sparse_mla_kernel<true>, grid, block, 0, st, *sel, q, q8, q_scale,
                       latent_pages, latent_page_stride, latent_scale, topk_slot, k,
                       softmax_scale, num_splits, n_q, mode, op, lp, out_bf16, lse);
  } else {
    hipLaunchKernelGGL(sparse_mla_kernel<false>, grid, block, 0, st, SelectArgs{}, q, q8,
                       q_scale, latent_pages, latent_page_stride, latent_scale, topk_slot, k,
                       softmax_scale, num_splits, n_q, mode, op, lp, out_bf16, lse);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || mode != kPartF16) return e;
  return launch_lse_combine_f16(num_splits, n_q, static_cast<const uint16_t*>(op), lp,
                                latent_scale, out_bf16, lse, st);
}

hipError_t launch_sparse_mla(int n_q, const uint16_t* q, const uint8_t* q8, const float* q_scale,
                             const uint8_t* latent_pages, int64_t latent_page_stride,
                             float latent_scale, const int32_t* topk_slot, int k,
                             float softmax_scale, int num_splits, float* o_part, float* lse_part,
                             uint16_t* out_bf16, float* lse, void* workspace, hipStream_t st) {
  return launch_mla_common(nullptr, n_q, q, q8, q_scale, latent_pages, latent_page_stride,
                           latent_scale, topk_slot, k, softmax_scale, num_splits, o_part,
                           lse_part, out_bf16, lse, workspace, st);
}

// ------------------------------------------------------------------------------------------
// Scratch of the allocation-free entry point: the fp16 split partials and their LSEs live in
// a file-scope device array instead of a caller workspace.  Each GPU the library runs on holds
// its own copy until the process ends.  In host code `scratch` names a host-side stand-in, so
// its device address is looked up once per device (with that device current) and only that
// address is ever handed to kernels.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

size_t sparse_mla_noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

static hipError_t noalloc_scratch_ptr(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_sparse_mla_noalloc(int n_q, const uint16_t* q, const uint8_t* q8,
                                     const float* q_scale, const uint8_t* latent_pages,
                                     int64_t latent_page_stride, float latent_scale,
                                     const int32_t* topk_slot, int k, float softmax_scale,
                                     int num_splits, float* o_part, float* lse_part,
                                     uint16_t* out_bf16, float* lse, hipStream_t st) {
  void* ws = nullptr;
  if (!o_part && num_splits > 1) {  // the only case whose kernels use scratch
    if (sparse_mla_workspace_bytes(n_q, num_splits) > kNoAllocScratchBytes)
      return hipErrorInvalidValue;  // (the C ABI rejects this case before calling)
    const hipError_t e = noalloc_scratch_ptr(&ws);
    if (e != hipSuccess) return e;
  }
  return launch_sparse_mla(n_q, q, q8, q_scale, latent_pages, latent_page_stride, latent_scale,
                           topk_slot, k, softmax_scale, num_splits, o_part, lse_part, out_bf16,
                           lse, ws, st);
}

hipError_t launch_topk_sparse_mla(int num_seqs, int n_q, const int32_t* cu_q,
                                  const int32_t* seq_lens, float* scores,
                                  int64_t score_stride, const TopkBuffers& t,
                                  const IndexRescore& rs, const int32_t* block_table,
                                  int bt_stride, int32_t* topk_idx, int32_t* topk_slot,
                                  const uint16_t* q, const uint8_t* q8,
                                  const float* q_scale, const uint8_t* latent_pages,
                                  int64_t latent_page_stride, float latent_scale, int k,
                                  float softmax_scale, int num_splits, uint16_t* out_bf16,
                                  float* lse, void* workspace, hipStream_t st) {
  const SelectArgs sel{cu_q, seq_lens, num_seqs, scores, score_stride, t.plan.num_groups,
                       (int64_t)t.plan.row_cap, t.cand_key, t.cand_idx, t.info, rs, block_table,
                       bt_stride, topk_idx, topk_slot, t.layout};
  return launch_mla_common(&sel, n_q, q, q8, q_scale, latent_pages, latent_page_stride,
                           latent_scale, nullptr, k, softmax_scale, num_splits, nullptr, nullptr,
                           out_bf16, lse, workspace, st);
}

}  // namespace dsa
