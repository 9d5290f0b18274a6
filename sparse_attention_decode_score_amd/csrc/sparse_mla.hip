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
// Workgroup = 8 waves on one CU.  Waves 6, 7 gather 64-token latent tiles (slot -> page ->
// 576 bytes, non-temporal loads): they keep three tiles in flight in registers and write
// each into a double-buffered LDS ring one tile ahead of the compute waves.  Every gather is
// issued unconditionally (a slot of -1 or a token past the split reads a zero row), so the
// compiler's wait counts stay exact and only the oldest tile is ever waited for.  Waves
// 0..5 each own 32 heads x 256 value dims of the row.  They quantise the row's query to
// E4M3 with one power-of-two scale per head (as dsa_quantize_q does) straight into LDS,
// where it is the B operand of
//   S[token][head] = L8[32 tokens x 576] * Q8^T          (9 x v_mfma 32x32x64 per 32 tokens)
// The two waves of a head tile each form the logits of one 32-token half of a tile; the A
// rows are permuted so that lane l holds head l%32's logits for tokens 32*(l/32) + 16*half
// + i.  They exchange per-head maxima and the probabilities through LDS, so each wave gets
// the E4M3 A operand of
//   O[head][dim] += P8[32 heads x 64 tokens] * V8[64 tokens x 256 dims]   (8 x v_mfma 32x32x64)
// whose B operand comes from the same LDS tile through ds_read_b64_tr_b8 (8 tokens of one
// dim per lane), so the value matrix is never transposed in memory.  Each compute wave keeps
// its 32x256 fp32 accumulator in registers.  The running max is only raised when a tile's
// max exceeds it by more than 2^4, so the accumulator rescale is rare; probabilities stay
// below 2^4 and are scaled by 2^4 before conversion to a two-term E4M3 pair (hi + residual),
// which keeps about 8 significant bits through the value product.
#include <mutex>

#include "dsa_device.hpp"
#include "dsa_internal.hpp"
#include "dsa_select.hpp"
#include "dsa_topk_final.hpp"

namespace dsa {

namespace {

constexpr int kTile = 64;
constexpr int kRowStride = 592;  // LDS bytes per latent / query row (576 + 16: conflict-free b128 reads)
constexpr int kThreads = 512;    // 6 compute waves + 2 loader waves
constexpr int kRing = 3;         // tiles the loader waves keep in flight in registers
constexpr int kSlotsLds = 4096;  // slots of a split held in LDS (k <= 4096)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 4.0f;      // running-max slack in log2 units
constexpr float kPScale = 16.0f;  // probabilities are converted to E4M3 as P * 2^4 <= 2^8

// The latent row gathered for padding: a slot of -1 or a position past the split.
__device__ __attribute__((aligned(64))) uint8_t g_zero_row[kLatDim];

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Output of a workgroup: the row's bf16 O and LSE (one split), or its split's partial O
// (fp32, or fp16 divided by the latent scale, which bounds it by 448) and LSE.
enum PartMode { kDirect = 0, kPartF32 = 1, kPartF16 = 2 };

struct MlaSmem {
  uint8_t lat[2][kTile * kRowStride];
  uint8_t q8s[kMlaHeads * kRowStride];
  uint8_t pbuf[3][2][32][64];  // [head tile][hi/lo][head][token]
  float xmax[3][2][32];
  float xfer[6][32];
  float qsc[kMlaHeads];
  int32_t slot_l[kSlotsLds];
  uint64_t valid_mask[2];
};
// The final top-k pass of the fused kernel runs before any of the above is used: its
// scratch overlays the latent ring, the query and the probability buffers, and its output
// (the row's selected token indices) is written straight into slot_l.
struct SelectSmem {
  uint32_t lkey[kFinalTile];
  int32_t lidx[kFinalTile];
  alignas(16) int red[4 * kFinalWaves];
  int note;
  uint32_t bucket[kBucketMax];
};
static_assert(sizeof(SelectSmem) <= offsetof(MlaSmem, slot_l), "selection scratch overlaps slot_l");
static_assert(kFinalThreads == kThreads, "the fused kernel runs the final pass on its own threads");

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
};

template <bool SELECT>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(
    SelectArgs sel, const uint16_t* __restrict__ q, const uint8_t* __restrict__ q8_in,
    const float* __restrict__ qs_in, const uint8_t* __restrict__ lat_pages, int64_t page_stride,
    float lat_scale, const int32_t* __restrict__ topk_slot, int k, float sm_scale,
    int num_splits, int n_q, int mode, void* __restrict__ o_part, float* __restrict__ lse_part,
    uint16_t* __restrict__ out_bf16, float* __restrict__ lse_out) {
  __shared__ __attribute__((aligned(16))) MlaSmem sm;
  auto& lat = sm.lat;
  auto& q8s = sm.q8s;
  auto& pbuf = sm.pbuf;
  auto& xmax = sm.xmax;
  auto& xfer = sm.xfer;
  auto& qsc = sm.qsc;
  auto& slot_l = sm.slot_l;
  auto& valid_mask = sm.valid_mask;

  // Workgroups are dealt to the 8 XCDs round-robin by linear id; when the grid divides
  // evenly, all splits of a row go to one XCD, so the row's query (read by every split)
  // comes from that XCD's L2 after the first read.
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

  if constexpr (SELECT) {
    // stage 2 for this row (every split of the row runs it: it is latency-bound), then the
    // split's slice of the selected tokens -> physical slots in slot_l
    SelectSmem& ss = *reinterpret_cast<SelectSmem*>(&sm);
    int b, pos;
    row_of(sel.cu_q, sel.seq_lens, sel.num_seqs, row, b, pos);
    const FinalScratch sc{ss.lkey, ss.lidx, ss.red, &ss.note, ss.bucket};
    const int32_t* bt = sel.block_table + (int64_t)b * sel.bt_stride;
    const int n_out = final_select_row(row, pos + 1, sel.scores, sel.score_stride, k,
                                       sel.num_groups, sel.row_cap, sel.cand_key, sel.cand_idx,
                                       sel.info, sel.rs, bt, slot_l, sc);
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
    __syncthreads();  // barrier 0: the selection scratch is dead, slot_l holds the split's slots
  } else {
    // the split's slot list -> LDS (barrier 0)
    const int32_t* slots = topk_slot + (int64_t)row * k + beg;
    for (int i = threadIdx.x; i < n_tok; i += kThreads) slot_l[i] = slots[i];
    __syncthreads();
  }
  auto slot_of = [&](int j) { return j < n_tok ? slot_l[j] : -1; };

  if (wave >= 6) {
    // ---------------------------------------------------------------- loader waves
    // wave 6 moves tile rows 0..31, wave 7 rows 32..63; lane l moves 16-byte pieces
    // (l%4) + 4c (c = 0..8) of rows 16*qq + l/4 of its half.
    const int half = wave - 6;
    typedef v4i TileRegs[2][9];
    auto issue = [&](int t, TileRegs& d) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int j = t * kTile + 32 * half + 16 * qq + (lane >> 2);
        const int slot = slot_of(j);
        const uint8_t* src = slot >= 0 ? lat_pages + (int64_t)(slot >> 6) * page_stride +
                                             (int64_t)(slot & (kPage - 1)) * kLatDim
                                       : g_zero_row;
#pragma unroll
        for (int c = 0; c < 9; ++c)
          d[qq][c] = __builtin_nontemporal_load(
              reinterpret_cast<const v4i*>(src + ((lane & 3) + 4 * c) * 16));
      }
    };
    auto store = [&](int t, const TileRegs& d, int buf) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const int r = 32 * half + 16 * qq + (lane >> 2);
#pragma unroll
        for (int c = 0; c < 9; ++c)
          *reinterpret_cast<v4i*>(&lat[buf][r * kRowStride + ((lane & 3) + 4 * c) * 16]) = d[qq][c];
      }
      if (half == 0) {
        const uint64_t m = __ballot(slot_of(t * kTile + lane) >= 0);
        if (lane == 0) valid_mask[buf] = m;
      }
    };
    // Every wave executes the same barriers: barrier 1, two per tile (A, B), one after the
    // last tile and the two of the compute waves' finalize step.  Tile i lives in
    // ring[i % kRing].  Under load a gather request can wait a long time to issue (every
    // workgroup of the chip gathers at once), and a loader wave late for a barrier holds
    // all six compute waves, so the loader requests one tile per step and at most two are
    // in flight: tile 0 alone first, tile 1 after barrier 1; in the step of tile t it writes
    // tile t+1 into the other LDS buffer between A and B (every wave has finished tile t-1,
    // which read that buffer, before A), and requests tile t+kRing after B.  It stops at the
    // last tile: requests past it (zero rows) are left unread.
    static_assert(kRing == 3, "the schedule below is written for a ring of three tiles");
    TileRegs ring[kRing];
    issue(0, ring[0]);
    store(0, ring[0], 0);
    __syncthreads();  // barrier 1: tile 0 and the query are in LDS
    issue(1, ring[1]);
    __syncthreads();  // tile 0: A
    issue(2, ring[2]);
    store(1, ring[1], 1);
    __syncthreads();  // B
    issue(3, ring[0]);
#pragma unroll 1
    for (int t0 = 1; t0 < n_tiles; t0 += kRing) {
#pragma unroll
      for (int u = 0; u < kRing; ++u) {
        const int t = t0 + u;  // t % kRing == (1 + u) % kRing
        if (t >= n_tiles) break;  // uniform
        __syncthreads();  // A
        store(t + 1, ring[(u + 2) % kRing], (t + 1) & 1);
        __syncthreads();  // B
        issue(t + kRing, ring[(u + 1) % kRing]);
      }
    }
    __syncthreads();  // after the last tile
    __syncthreads();
    __syncthreads();
    return;
  }

  // ------------------------------------------------------------------ compute waves
  if (q8_in) {
    // codes and scales prepared by the query quantisation: coalesced copy to LDS
    const uint8_t* src = q8_in + (int64_t)row * kMlaHeads * kLatDim;
    for (int i = threadIdx.x; i < kMlaHeads * (kLatDim / 16); i += 384) {
      const int h = i / (kLatDim / 16), pc = i % (kLatDim / 16);
      *reinterpret_cast<v4i*>(&q8s[h * kRowStride + pc * 16]) =
          *reinterpret_cast<const v4i*>(src + (int64_t)i * 16);
    }
    if (threadIdx.x < kMlaHeads) qsc[threadIdx.x] = qs_in[(int64_t)row * kMlaHeads + threadIdx.x];
  } else {
    // query prep: 4 threads per head, 144 dims each -> E4M3 codes in LDS and the head's
    // power-of-two scale (smallest 2^e with absmax <= 448 * 2^e)
    const int h = threadIdx.x >> 2, part = threadIdx.x & 3;
    const uint16_t* src = q + ((int64_t)row * kMlaHeads + h) * kLatDim + part * 144;
    v4i raw[18];
#pragma unroll
    for (int i = 0; i < 18; ++i) raw[i] = *reinterpret_cast<const v4i*>(src + 8 * i);
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
    uint8_t* dst = q8s + h * kRowStride + part * 144;
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
    if (part == 0) qsc[h] = ldexpf(1.0f, e);
  }
  const int ht = wave >> 1;  // head tile: heads 32*ht .. +31
  const int hf = wave & 1;   // token half of each tile for the logits, value-dim half for O
  const uint8_t* qrow = q8s + (32 * ht + n) * kRowStride + 32 * g;
  v16f acc[8];  // O[32 heads][256 dims] of this wave; acc[dt] covers dims 256*hf + 32*dt .. +31
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc[dt] = v16f{};
  float m_run = -INFINITY;  // running max (log2 units) of head n, identical in both waves
  float z_run = 0.f;        // this lane's share of the running sum of head n
  bool started = false;
  __syncthreads();  // barrier 1
  const float mult = qsc[32 * ht + n] * lat_scale * sm_scale * kLog2e;

  const int grp = lane >> 4, li = lane & 15;
  // MFMA row n -> tile token 32*((n>>2)&1) + 16*hf + 4*(n>>3) + (n&3)
  const int tok = 32 * ((n >> 2) & 1) + 16 * hf + 4 * (n >> 3) + (n & 3);
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const uint8_t* tile = lat[buf];
    const uint64_t vm = valid_mask[buf];
    // ---- logits of this wave's token half: lane holds head n, tokens 32*g + 16*hf + i
    float x[16];
    float mx = -INFINITY;
    if (vm != 0ull) {
      const uint8_t* arow = tile + tok * kRowStride + 32 * g;
      v16f d = {};
      v4i a0 = *reinterpret_cast<const v4i*>(arow);
      v4i a1 = *reinterpret_cast<const v4i*>(arow + 16);
      v4i b0 = *reinterpret_cast<const v4i*>(qrow);
      v4i b1 = *reinterpret_cast<const v4i*>(qrow + 16);
#pragma unroll
      for (int kb = 0; kb < 9; ++kb) {
        const v8i A = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        const v8i B = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        const int nx = kb < 8 ? 64 * (kb + 1) : 64 * kb;
        a0 = *reinterpret_cast<const v4i*>(arow + nx);
        a1 = *reinterpret_cast<const v4i*>(arow + nx + 16);
        b0 = *reinterpret_cast<const v4i*>(qrow + nx);
        b1 = *reinterpret_cast<const v4i*>(qrow + nx + 16);
        d = mfma_32x32x64_fp8(A, B, d);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tk = 32 * g + 16 * hf + i;
        x[i] = ((vm >> tk) & 1ull) ? d[i] * mult : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (g == 0) xmax[ht][hf][n] = mx;
    }
    __syncthreads();
    if (vm != 0ull) {
      mx = fmaxf(mx, xmax[ht][hf ^ 1][n]);  // the tile max of head n, same in both waves
      if (!started) {
        m_run = mx;
        started = true;
      } else if (__ballot(mx > m_run + kTau) != 0ull) {
        const float m_new = fmaxf(m_run, mx);
        const float f = exp2f(m_run - m_new);
        m_run = m_new;
        z_run *= f;
        if (g == 0) xfer[wave][n] = f;
        wave_lds_sync();
        // accumulator register i holds head 8*(i/4) + 4*g + i%4
        float fr[16];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const v4f v = *reinterpret_cast<const v4f*>(&xfer[wave][8 * a + 4 * g]);
#pragma unroll
          for (int c = 0; c < 4; ++c) fr[4 * a + c] = v[c];
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= fr[i];
        wave_lds_sync();
      }
      // ---- probabilities of this half -> two E4M3 terms (hi = E4M3(p), lo = E4M3(p - hi)),
      // stored as bytes 32*g + 16*hf + i of head n's row
      v4i phi, plo;
      float zsum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float p4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float p = exp2f(x[4 * j + c] - m_run);  // x = -inf -> 0
          zsum += p;
          p4[c] = p * kPScale;
        }
        const uint32_t hi = cvt4_e4m3(p4[0], p4[1], p4[2], p4[3]);
        const v2f d01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
        const v2f d23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
        phi[j] = (int)hi;
        plo[j] = (int)cvt4_e4m3(p4[0] - d01[0], p4[1] - d01[1], p4[2] - d23[0], p4[3] - d23[1]);
      }
      z_run += zsum;
      *reinterpret_cast<v4i*>(&pbuf[ht][0][n][32 * g + 16 * hf]) = phi;
      *reinterpret_cast<v4i*>(&pbuf[ht][1][n][32 * g + 16 * hf]) = plo;
    }
    __syncthreads();
    if (vm != 0ull) {
      // ---- A operands: head n, tokens 32*g .. +31 of the tile (both halves)
      const v4i h0 = *reinterpret_cast<const v4i*>(&pbuf[ht][0][n][32 * g]);
      const v4i h1 = *reinterpret_cast<const v4i*>(&pbuf[ht][0][n][32 * g + 16]);
      const v4i l0 = *reinterpret_cast<const v4i*>(&pbuf[ht][1][n][32 * g]);
      const v4i l1 = *reinterpret_cast<const v4i*>(&pbuf[ht][1][n][32 * g + 16]);
      const v8i pa = v8i{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      const v8i pl = v8i{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
      // ---- O += P8 * V8: B operand via LDS transpose reads.  In each 16-lane group,
      // lanes 2r, 2r+1 address the two 8-byte halves of token row r (8 rows), and lane i
      // then receives dim (group base + i) of those 8 tokens.
      const uint8_t* vb = tile + (32 * (grp >> 1) + (li >> 1)) * kRowStride + 256 * hf +
                          16 * (grp & 1) + 8 * (li & 1);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        v8i B;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const v2i r2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (DSA_LDS v2i*)(vb + 8 * jj * kRowStride + 32 * dt));
          B[2 * jj] = r2[0];
          B[2 * jj + 1] = r2[1];
        }
        acc[dt] = mfma_32x32x64_fp8(pa, B, acc[dt]);
        acc[dt] = mfma_32x32x64_fp8(pl, B, acc[dt]);
      }
    }
    // (no barrier here: the next tile's maxima and probabilities are written only after
    // its barrier A, which every wave reaches after this tile's values product)
  }
  __syncthreads();  // after the last tile

  // ------------------------------------------------------------------ finalize
  // each wave summed the probabilities of its own token halves: add the partner's
  const float zl = z_run + __shfl_xor(z_run, 32, 64);
  if (g == 0) xfer[wave][n] = zl;
  __syncthreads();
  const float z = zl + xfer[wave ^ 1][n];
  const bool empty = !(z > 0.f);
  const float lse = empty ? -INFINITY : (m_run + log2f(z)) * kLn2;
  // values are latent_scale * L8; probabilities entered the product scaled by 2^4
  const float invz = empty ? 0.f : lat_scale / (z * kPScale);
  __syncthreads();
  if (g == 0) xfer[wave][n] = invz;
  wave_lds_sync();
  float fr[16];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const v4f v = *reinterpret_cast<const v4f*>(&xfer[wave][8 * a + 4 * g]);
#pragma unroll
    for (int c = 0; c < 4; ++c) fr[4 * a + c] = v[c];
  }
  const int head0 = 32 * ht;
  const int dim0 = 256 * hf + n;
  if (mode == kDirect) {
    uint16_t* ob = out_bf16 + (int64_t)row * kMlaHeads * kVDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = head0 + 8 * (i / 4) + 4 * g + (i % 4);
        uint32_t u = __float_as_uint(acc[dt][i] * fr[i]);  // round to nearest even bf16
        u += 0x7FFFu + ((u >> 16) & 1u);
        ob[(int64_t)h * kVDim + dim0 + 32 * dt] = (uint16_t)(u >> 16);
      }
    if (g == 0 && hf == 0) lse_out[(int64_t)row * kMlaHeads + head0 + n] = lse;
  } else if (mode == kPartF32) {
    float* op = static_cast<float*>(o_part) + ((int64_t)s * n_q + row) * kMlaHeads * kVDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = head0 + 8 * (i / 4) + 4 * g + (i % 4);
        op[(int64_t)h * kVDim + dim0 + 32 * dt] = acc[dt][i] * fr[i];
      }
    if (g == 0 && hf == 0) lse_part[((int64_t)s * n_q + row) * kMlaHeads + head0 + n] = lse;
  } else {
    _Float16* op = static_cast<_Float16*>(o_part) + ((int64_t)s * n_q + row) * kMlaHeads * kVDim;
    const float unscale = 1.0f / lat_scale;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int h = head0 + 8 * (i / 4) + 4 * g + (i % 4);
        op[(int64_t)h * kVDim + dim0 + 32 * dt] = (_Float16)(acc[dt][i] * (fr[i] * unscale));
      }
    if (g == 0 && hf == 0) lse_part[((int64_t)s * n_q + row) * kMlaHeads + head0 + n] = lse;
  }
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
                       bt_stride, topk_idx, topk_slot};
  return launch_mla_common(&sel, n_q, q, q8, q_scale, latent_pages, latent_page_stride,
                           latent_scale, nullptr, k, softmax_scale, num_splits, nullptr, nullptr,
                           out_bf16, lse, workspace, st);
}

}  // namespace dsa
