/*
 * dsa.h — C ABI of the MI355X (gfx950) DSA decode hot path.
 *
 * DeepSeek Sparse Attention as served for Kimi K3.1 Pro's full-attention layers
 * (the vLLM day-0 page on Kimi K3.1 Pro: sparse attention, DCP and zero-mismatch RL):
 * a lightning indexer scores every prior token, the best 2,048 are kept, MLA runs
 * exactly over those only, and split partial outputs are merged by log-sum-exp.
 *
 *   dsa_index_score       stage 1  indexer scores           ("What changed in Kimi K3.1 Pro")
 *   dsa_index_score_mxfp4 stage 1 on MXFP4 index keys        ("Native MXFP4 indexer")
 *   dsa_index_score_quantize_q  stage 1 plus stage 3's query quantisation in one launch
 *   dsa_topk              stage 2  exact top-k select       ("Exact top-k merge with ~10x less traffic")
 *                         Stage 1 can also emit each 256-token group's top-k candidates while
 *                         its scores are on chip; stage 2 then only runs its final pass (the
 *                         scorer + exact top-k pair of "Fused low-latency decode for DSA layers").
 *   dsa_sparse_mla_decode stage 3  MLA over selected tokens ("Sparse attention cuts long-context
 *                                                             decode bandwidth")
 *   dsa_topk_sparse_mla   stages 2-4 in one launch: each attention workgroup first runs its
 *                         row's final top-k pass over the stage-1 candidates
 *   dsa_lse_combine       stage 4  LSE merge of splits      ("Decode context parallelism with the
 *                                                             sparse indexer")
 *   dsa_cache_append      quantises the step's new tokens into the two paged caches
 *   dsa_cache_append_mxfp4  the same for MXFP4 index keys  ("Native MXFP4 indexer")
 *   dsa_quantize_q        the query quantisation the stages 1 and 3 apply internally
 *                         (fused indexer front of "Fused low-latency decode for DSA layers"),
 *                         exposed so callers and tests can see the exact FP8 codes.
 *
 * Conventions shared by every call
 *  - Every pointer is a DEVICE pointer on the current HIP device unless marked (host).
 *    The caller owns and allocates all memory, including the workspaces.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work
 *    on it: no allocation, no host synchronisation, no device-to-host reads.
 *  - Host scalars and pointer nullness/alignment are validated before anything is
 *    launched; on failure nothing is launched and the call returns a non-OK status with
 *    a message available from dsa_last_error() (thread-local).
 *  - Device array CONTENTS are trusted preconditions (block-table entries in range,
 *    seq_lens >= rows of the request, slots in range or -1).  They are not checked.
 *  - Fixed shapes: page 64 tokens, indexer 32 heads x 128 dims, MLA 96 heads on a
 *    576-dim latent whose first 512 dims are the values.  FP8 is OCP E4M3FN.
 *
 * Batch description (used by stages 1 and 2).  Query rows are grouped by request: the
 * rows of request b are cu_q[b] .. cu_q[b+1]-1 and they are the LAST
 * n_b = cu_q[b+1]-cu_q[b] tokens of that request, so row j of request b sits at
 * position seq_lens[b] - n_b + j and sees tokens 0..position (inclusive causal).
 * This covers plain decode (n_b = 1), speculative verification (n_b <= 8, causal among
 * the new tokens) and prefill append (n_b new tokens on a cached prefix).
 *
 * Cache layouts ("Packed KV cache for three kinds of state": 132 B per index key,
 * 576 B per latent, small fixed-size pages addressed through a block table).
 *  - block_table: int32 [num_seqs][bt_stride]; entry j is the physical page holding
 *    logical tokens 64j .. 64j+63 of the request.  A physical slot is page*64 + offset.
 *  - index-key page (at key_pages + page * key_page_stride, 16-byte aligned):
 *      bytes [0, 8192): E4M3 codes; byte d of token o at (d/16)*1024 + o*16 + d%16
 *      bytes [8192, 8448): fp32 scale of token o at 8192 + 4*o (key = codes * scale)
 *  - latent page (at latent_pages + page * latent_page_stride, 16-byte aligned):
 *      token o's 576 E4M3 codes at o*576; latent = codes * latent_scale (per tensor).
 *  Page strides are in bytes, multiples of 16, at least 8448 / 36864, so several
 *  per-layer pages can share one packed block row.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or inconsistent host scalars */
  DSA_ERR_UNSUPPORTED = 2,   /* shape the library does not implement */
  DSA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than its *_workspace_size() */
  DSA_ERR_LAUNCH = 4         /* the HIP runtime rejected a launch */
} dsa_status;

#define DSA_PAGE_SIZE 64
#define DSA_IDX_HEADS 32
#define DSA_IDX_DIM 128
#define DSA_IDX_PAGE_BYTES 8448
#define DSA_IDX_MXFP4_PAGE_BYTES 4352
#define DSA_MLA_HEADS 96
#define DSA_LATENT_DIM 576
#define DSA_V_DIM 512
#define DSA_LATENT_PAGE_BYTES 36864
#define DSA_MAX_TOPK 4096
#define DSA_MAX_SPLITS 64

/*
 * Stage 1 — lightning-indexer scores.
 *   score[i][t] = sum_h w'[i][h] * ReLU(sum_d q8[i][h][d] * k8[t][d]) * s[t]
 * where q8 / sq are the E4M3 codes and power-of-two scale of dsa_quantize_q applied to
 * q_bf16 row i, head h, and w' = head_w * sq.  Because sq, s > 0 this equals
 * sum_h w_h ReLU(q_h . k_t s_t) with q_h the dequantised query, the head-weighted ReLU
 * form of DeepSeek-V3.2's lightning indexer that the K3.1 page defers to.
 * FP8 MFMA products, fp32 accumulation.
 *
 *   num_seqs, n_q       (host) requests and total query rows (>= 1 each)
 *   max_seq_len         (host) >= every seq_lens[b]; sizes the grid
 *   max_q_per_seq       (host) >= every request's row count
 *   cu_q [num_seqs+1], seq_lens [num_seqs]   batch description above
 *   q_bf16   [n_q][32][128] bf16            head_w [n_q][32] fp32
 *   key_pages, key_page_stride, block_table, bt_stride   index-key cache
 *   scores   fp32 [n_q][score_stride], score_stride >= max_seq_len.  Row i's columns
 *            0 .. seq_lens[b]-1 are written; columns past its position hold scores of
 *            keys it may not see (ignored by dsa_topk); other columns are not touched.
 *            NULL with cand_workspace given: candidates only, no score is stored (the
 *            scorer + per-chunk candidates with no materialised scores of the page's exact
 *            one-round merge, "Exact top-k merge with ~10x less traffic"); dsa_topk and
 *            dsa_topk_sparse_mla then recompute the few groups they must re-read from the
 *            same q_bf16 / head_w / key cache (pass them there).
 *   cand_k, cand_workspace, cand_workspace_bytes: if cand_workspace is not NULL the
 *            scoring waves also write, for a top-k of cand_k (1..4096), every 256-token
 *            group's best candidates (4x the winners a full group holds on average, at
 *            least 8 below 4 winners, in token order) and the group's boundary element
 *            into it, and the workspace's layout record (see dsa_topk_workspace_status);
 *            rows of at most 32,768 visible tokens send every key instead (the final pass
 *            then selects from the whole row).  It must hold
 *            dsa_topk_workspace_size(n_q, max_seq_len, cand_k) bytes, 256-byte aligned.
 *            Pass it to dsa_topk with from_candidates = 1.  NULL: scores only.
 */
dsa_status dsa_index_score(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                           int32_t max_q_per_seq, const int32_t* cu_q, const int32_t* seq_lens,
                           const void* q_bf16, const float* head_w, const void* key_pages,
                           int64_t key_page_stride, const int32_t* block_table, int32_t bt_stride,
                           float* scores, int64_t score_stride, int32_t cand_k,
                           void* cand_workspace, size_t cand_workspace_bytes, void* stream);

/*
 * Stage 1 on MXFP4 index keys (68 bytes per token: the opt-in MXFP4 index key of "Packed KV
 * cache for three kinds of state", scored with FP4 matrix instructions and FP32
 * accumulation as in "Native MXFP4 indexer").
 *   score[i][t] = sum_h w'[i][h] * ReLU(sum_d q8[i][h][d] * k[t][d]),  k = E2M1 * 2^(E8M0-127)
 * (the block scales are inside the product; there is no per-token scale).  The query is
 * E4M3 as for dsa_index_score.
 *   MXFP4 index-key page (at key_pages + page * key_page_stride, 16-byte aligned,
 *   key_page_stride >= 4352): block b (dims 32b .. 32b+31) of token o is 16 bytes at
 *   b * 1024 + o * 16, byte j holding dims 32b + 2j (low nibble) and 32b + 2j + 1 (high
 *   nibble) as E2M1 (OCP MX); the E8M0 scale of block b of token o is the byte at
 *   4096 + 4 * o + b.
 *   Every other argument as for dsa_index_score (with scores = NULL, pass key_format = 1
 *   to the final top-k pass).
 */
dsa_status dsa_index_score_mxfp4(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                                 int32_t max_q_per_seq, const int32_t* cu_q,
                                 const int32_t* seq_lens, const void* q_bf16, const float* head_w,
                                 const void* key_pages, int64_t key_page_stride,
                                 const int32_t* block_table, int32_t bt_stride, float* scores,
                                 int64_t score_stride, int32_t cand_k, void* cand_workspace,
                                 size_t cand_workspace_bytes, void* stream);

/*
 * Stage 1 with the MLA query's quantisation in the same launch: exactly
 * dsa_index_score (key_format 0) or dsa_index_score_mxfp4 (key_format 1) with the same
 * arguments, plus dsa_quantize_q(n_q, 96, 576, q_mla_bf16, q8_mla, q_mla_scale) -- the
 * E4M3 codes and per-(row, head) power-of-two scales that stage 3 applies to the query
 * ("Sparse attention cuts long-context decode bandwidth": the 576-dim FP8 product over the
 * selected latents), bitwise identical to that call.  One more workgroup per request and
 * row group does it while the keys stream, so a decode step needs no launch of its own
 * for it; stage 3 then takes q8_mla / q_mla_scale as a prepared query.
 *   q_mla_bf16: bf16 [n_q][96][576], 16-byte aligned (read only).
 *   q8_mla: uint8 [n_q][96][576], 16-byte aligned; q_mla_scale: fp32 [n_q][96] (written).
 * Errors: those of dsa_index_score; DSA_ERR_UNSUPPORTED for another key_format;
 * DSA_ERR_INVALID_ARG for a null or misaligned query buffer.
 */
dsa_status dsa_index_score_quantize_q(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                                      int32_t max_q_per_seq, const int32_t* cu_q,
                                      const int32_t* seq_lens, const void* q_bf16,
                                      const float* head_w, const void* key_pages,
                                      int64_t key_page_stride, int32_t key_format,
                                      const int32_t* block_table, int32_t bt_stride, float* scores,
                                      int64_t score_stride, int32_t cand_k, void* cand_workspace,
                                      size_t cand_workspace_bytes, const void* q_mla_bf16,
                                      uint8_t* q8_mla, float* q_mla_scale, void* stream);

/*
 * Stage 2 — exact top-k over each row's visible scores (tokens 0..position).
 * Order: score descending, then token index ascending (-0.0 == +0.0; NaN ranks lowest).
 * scores is only read, unless the scores were not stored (see q_idx_bf16 below).
 * Two passes: every 256-token group keeps its best m candidates (4x the winners a full
 * group holds on average), then one workgroup per row selects from the candidates; the
 * groups that could have held more of the winners than they sent (the detection rule of
 * the K3.1 page's exact one-round merge) are re-read in full from the scores and the row is
 * selected again, so the result is always exact.  from_candidates = 0: this call runs both
 * passes.  from_candidates = 1: the workspace already holds the candidates dsa_index_score
 * wrote for the same batch, scores and k, and only the final pass runs.
 *
 *   k in 1..4096.  topk_idx int32 [n_q][k]: the min(k, position+1) selected logical
 *   token indices in increasing index order, then -1.  topk_slot int32 [n_q][k]: the
 *   physical slots of the same tokens (page*64 + offset via block_table), -1 padded;
 *   pass block_table = NULL and topk_slot = NULL to skip slots.
 *   workspace: device memory of at least dsa_topk_workspace_size(n_q, max_seq_len, k)
 *   bytes, 256-byte aligned; with from_candidates = 0 its contents need no
 *   initialisation.  It is scratch after the call.
 *   q_idx_bf16, head_w, key_pages, key_page_stride, key_format: all NULL / 0 when the
 *   scores were stored.  When dsa_index_score or dsa_index_score_mxfp4 stored none
 *   (scores = NULL there), pass its query, head weights and index-key cache here, with
 *   key_format 0 (E4M3 keys) or 1 (MXFP4 keys) (from_candidates = 1 and block_table
 *   required): the groups that must be re-read are recomputed with the indexer's own
 *   arithmetic (bitwise its scores) into `scores`, which is then scratch of
 *   [n_q][score_stride] fp32 whose contents need no initialisation.
 */
size_t dsa_topk_workspace_size(int32_t n_q, int32_t max_seq_len, int32_t k);

/*
 * The top-k workspace's layout record.  Its first 256 bytes hold (magic, k, max_seq_len, n_q,
 * status), written by the call that writes the candidates (dsa_index_score* with a workspace,
 * or dsa_topk's own first pass).  A final pass (dsa_topk with from_candidates = 1, or
 * dsa_topk_sparse_mla) whose (k, max_seq_len, n_q) differ from the record's reads the
 * candidates of another layout: it selects nothing (every row's topk_idx / topk_slot -1, and
 * in dsa_topk_sparse_mla O = 0, LSE = -inf) and sets status to 1.  This call reads the
 * record (it waits for `stream`: a diagnostic, not for the hot path) and returns DSA_OK, or
 * DSA_ERR_WORKSPACE when no record was written or a final pass found a mismatch (the message
 * names the record's values).  workspace_bytes >= 256.
 */
dsa_status dsa_topk_workspace_status(const void* workspace, size_t workspace_bytes, void* stream);

dsa_status dsa_topk(int32_t num_seqs, int32_t n_q, int32_t max_seq_len, const int32_t* cu_q,
                    const int32_t* seq_lens, float* scores, int64_t score_stride, int32_t k,
                    const int32_t* block_table, int32_t bt_stride, int32_t* topk_idx,
                    int32_t* topk_slot, void* workspace, size_t workspace_bytes,
                    int32_t from_candidates, const void* q_idx_bf16, const float* head_w,
                    const void* key_pages, int64_t key_page_stride, int32_t key_format,
                    void* stream);

/*
 * Stage 3 — exact MLA (NoPE) over the selected slots, one query row at a time.
 *   logit[h][t] = softmax_scale * (q8[h] * sq[h]) . (latent_scale * L8[t])   (576 dims)
 *   O[h] = sum_t softmax(logit[h])[t] * latent_scale * L8[t][0:512],
 *   LSE[h] = log(sum_t exp(logit[h][t]))   (natural log)
 * The query is E4M3-quantised per (row, head) as dsa_quantize_q does.  Both
 * contractions run on FP8 MFMA; the probabilities enter the value product as E4M3.
 *
 *   Query: q8 (uint8 E4M3 codes [n_q][96][576]) and q_scale (fp32 [n_q][96]) as
 *   dsa_quantize_q(n_q, 96, 576, ...) writes them, when both are given (the caller can
 *   prepare them on another stream while stages 1 and 2 run; both 16-byte aligned);
 *   otherwise q_bf16 [n_q][96][576] bf16 (16-byte aligned), quantised inside the call.
 *   topk_slot int32 [n_q][k]; -1 entries are skipped.
 *   num_splits S in 1..64, S <= k: split s of a row covers entries [s*k/S, (s+1)*k/S)
 *   of its slot list (splits add workgroups for small batches).
 *   Outputs, one of:
 *   - o_part and lse_part given: o_part fp32 [S][n_q][96][512] (each split normalised by
 *     its own sum) and lse_part fp32 [S][n_q][96] are written; an empty split has O = 0
 *     and LSE = -inf.  Merge them with dsa_lse_combine.  out_bf16 / lse are unused.
 *   - otherwise out_bf16 [n_q][96][512] bf16 and lse [n_q][96] fp32 are written.  With
 *     S > 1 the splits pass through the workspace as fp16 partials (O_s / latent_scale,
 *     bounded by 448) and are merged by log-sum-exp inside the call (stage 4).
 *   workspace: with S > 1 and no o_part, device memory of at least
 *   dsa_sparse_mla_workspace_size(n_q, S) bytes, 256-byte aligned, scratch for the call;
 *   unused (may be NULL) otherwise.
 */
size_t dsa_sparse_mla_workspace_size(int32_t n_q, int32_t num_splits);
dsa_status dsa_sparse_mla_decode(int32_t n_q, const void* q_bf16, const void* q8,
                                 const float* q_scale, const void* latent_pages,
                                 int64_t latent_page_stride, float latent_scale,
                                 const int32_t* topk_slot, int32_t k, float softmax_scale,
                                 int32_t num_splits, void* out_bf16, float* lse, float* o_part,
                                 float* lse_part, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * dsa_sparse_mla_decode without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Every
 * argument means what it means for dsa_sparse_mla_decode and the kernels are the same, so the
 * results are bitwise those of that call.  When the splits are merged inside the call
 * (num_splits > 1, o_part NULL) their fp16 partials go to a scratch array the library holds
 * in device memory, 64 MiB per GPU, kept until the process ends: calls needing more than that,
 * dsa_sparse_mla_workspace_size(n_q, num_splits) > 64 MiB (about n_q * num_splits > 680), return
 * DSA_ERR_WORKSPACE.  Nothing is allocated and nothing is cleared: every split writes its whole
 * partial.  All calls on one GPU share that GPU's scratch, so calls that overlap in time on one
 * GPU (on different streams, or from different threads) race; issue them on one stream.
 */
dsa_status dsa_sparse_mla_decode_noalloc(int32_t n_q, const void* q_bf16, const void* q8,
                                         const float* q_scale, const void* latent_pages,
                                         int64_t latent_page_stride, float latent_scale,
                                         const int32_t* topk_slot, int32_t k, float softmax_scale,
                                         int32_t num_splits, void* out_bf16, float* lse,
                                         float* o_part, float* lse_part, void* stream);

/*
 * Stages 2 + 3 (+ 4) in one launch: the final top-k pass and the sparse MLA.  Every
 * (split, row) workgroup of the attention first selects its row's top k from the
 * candidates dsa_index_score wrote (cand_workspace, written with cand_k = k for this batch
 * and these scores), exactly as dsa_topk(..., from_candidates = 1) does, then attends over
 * its split's slice of the selection.  The pairing of a scorer with an exact top-k ahead of
 * the attention in one low-latency decode path is that of "Fused low-latency decode for DSA
 * layers"; putting the row's final pass inside the attention's workgroups (each split of a
 * row repeats it) removes one launch and the wait on a single workgroup per row.
 *   Batch, scores, k, block_table (required here): as for dsa_topk.
 *   cand_workspace: dsa_topk_workspace_size(n_q, max_seq_len, k) bytes, 256-byte aligned,
 *   read only.  q_idx_bf16, head_w, key_pages, key_page_stride, key_format: as for
 *   dsa_topk (scores not stored: `scores` is scratch).
 *   topk_idx, topk_slot: optional outputs (each may be NULL), as dsa_topk writes them.
 *   Query, latent cache, softmax_scale, num_splits (S <= k), out_bf16 [n_q][96][512] bf16,
 *   lse [n_q][96] fp32, workspace (S > 1: dsa_sparse_mla_workspace_size(n_q, S) bytes,
 *   256-byte aligned): as for dsa_sparse_mla_decode without o_part.  The results are
 *   bitwise those of dsa_topk(from_candidates = 1) followed by dsa_sparse_mla_decode.
 */
dsa_status dsa_topk_sparse_mla(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                               const int32_t* cu_q, const int32_t* seq_lens, float* scores,
                               int64_t score_stride, int32_t k, const int32_t* block_table,
                               int32_t bt_stride, const void* cand_workspace,
                               size_t cand_workspace_bytes, const void* q_idx_bf16,
                               const float* head_w, const void* key_pages,
                               int64_t key_page_stride, int32_t key_format, int32_t* topk_idx,
                               int32_t* topk_slot, const void* q_bf16, const void* q8,
                               const float* q_scale, const void* latent_pages,
                               int64_t latent_page_stride, float latent_scale,
                               float softmax_scale, int32_t num_splits, void* out_bf16,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 4 — log-sum-exp merge of split partials:
 *   LSE = m + log(sum_s exp(LSE_s - m)),  O = sum_s exp(LSE_s - LSE) * O_s.
 * Splits with LSE_s = -inf contribute nothing; if all are empty, O = 0, LSE = -inf.
 *   o_part fp32 [S][n_q][96][512], lse_part fp32 [S][n_q][96]  ->
 *   out_bf16 [n_q][96][512] bf16, lse [n_q][96] fp32.   S in 1..64.
 */
dsa_status dsa_lse_combine(int32_t num_splits, int32_t n_q, const float* o_part,
                           const float* lse_part, void* out_bf16, float* lse, void* stream);

/*
 * Cache append (the step just before the path in a decode): quantises the step's new tokens
 * into the two paged caches at their physical slots, in the layouts above.  One FP8 index
 * key of 132 bytes with its scale per token ("What changed in Kimi K3.1 Pro") and a 576-byte
 * FP8 latent ("Packed KV cache for three kinds of state"); the page's fused indexer front
 * writes the new token's index key ("Fused low-latency decode for DSA layers").
 *   index key: s = absmax / 448 in fp32 (1 if the key is all zero), stored as the token's
 *              fp32 scale; codes = E4M3 round-to-nearest-even of k / s, saturating at 448.
 *   latent:    codes = E4M3 round-to-nearest-even of x / latent_scale (the cache's
 *              per-tensor scale), saturating at 448.
 * Divisions are IEEE fp32.
 *   n_tok (host) >= 0; slots int32 [n_tok]: page * 64 + offset, -1 = skip (no two valid
 *   entries may be equal); key_bf16 bf16 [n_tok][128] and/or latent_bf16 bf16
 *   [n_tok][576] (either may be NULL: that cache is not touched), 16-byte aligned;
 *   key_pages / latent_pages and their strides as for stages 1 and 3.  Only the bytes of
 *   the given slots are written.
 */
dsa_status dsa_cache_append(int32_t n_tok, const int32_t* slots, const void* key_bf16,
                            const void* latent_bf16, float latent_scale, void* key_pages,
                            int64_t key_page_stride, void* latent_pages,
                            int64_t latent_page_stride, void* stream);

/*
 * dsa_cache_append for a cache whose index keys are the page's opt-in 68-byte MXFP4 keys
 * ("Native MXFP4 indexer"; the page layout of dsa_index_score_mxfp4).  Per block of 32
 * dims (OCP microscaling): the E8M0 scale 2^e, e = floor(log2 absmax) - 2 (2 = E2M1's
 * largest exponent), e >= -127, and e = 0 for an all-zero block; each element the E2M1 value
 * nearest |x| / 2^e, ties to the even code, saturating at 6, with x's sign bit (a negative
 * value that rounds to zero is -0).  Keys must be finite.  key_page_stride >= 4352; the
 * latent and every other argument as for dsa_cache_append.
 */
dsa_status dsa_cache_append_mxfp4(int32_t n_tok, const int32_t* slots, const void* key_bf16,
                                  const void* latent_bf16, float latent_scale, void* key_pages,
                                  int64_t key_page_stride, void* latent_pages,
                                  int64_t latent_page_stride, void* stream);

/*
 * Per-(row, head) E4M3 query quantisation used inside stages 1 and 3.
 *   sq = smallest power of two 2^e with max_d |q[d]| <= 448 * 2^e (1 if all zero);
 *   codes[d] = E4M3 round-to-nearest-even of q[d] / sq.
 *   q_bf16 [rows][heads][dim] bf16 -> codes uint8 [rows][heads][dim], scales fp32
 *   [rows][heads].  dim must be 128 or 576.
 */
dsa_status dsa_quantize_q(int32_t rows, int32_t heads, int32_t dim, const void* q_bf16,
                          uint8_t* codes, float* scales, void* stream);

/*
 * Host-side checks of the device-array CONTENTS the calls above trust without checking (the
 * block tables and slots that the serving stack translates to page addresses before each step,
 * "Packed KV cache for three kinds of state").  They run on the CPU over HOST copies of those
 * arrays (every pointer here is a host pointer), touch no GPU and launch nothing; a caller
 * runs them when debugging a batch, before the device calls.  DSA_OK, or DSA_ERR_INVALID_ARG
 * with the first violation in dsa_last_error().
 *
 * dsa_validate_batch: the batch description of stages 1-2 and the block table:
 *   cu_q[0] == 0, every request has 1..max_q_per_seq rows, cu_q[num_seqs] == n_q;
 *   1 <= seq_lens[b] <= max_seq_len and at least the request's row count;
 *   bt_stride >= ceil(max_seq_len / 64), and block_table[b][j] in 0..num_pages-1 for every
 *   page j holding a token of request b.
 *   topk_slot [n_q][k] (may be NULL: not checked): every entry is -1 or the slot of a token
 *   the row sees (page block_table[b][j], offset o, 64 j + o <= the row's position), and the
 *   valid entries of a row are distinct.
 * dsa_validate_slots: the slots of dsa_cache_append: each -1 or page * 64 + offset with
 *   page < num_pages, and no valid slot twice.
 */
dsa_status dsa_validate_batch(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                              int32_t max_q_per_seq, const int32_t* cu_q, const int32_t* seq_lens,
                              const int32_t* block_table, int32_t bt_stride, int64_t num_pages,
                              const int32_t* topk_slot, int32_t k);
dsa_status dsa_validate_slots(int32_t n_tok, const int32_t* slots, int64_t num_pages);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* dsa_last_error(void);

/* Library version string. */
const char* dsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
