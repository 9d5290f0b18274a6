// C ABI of the DSA decode library: argument validation, then launches on the caller's stream.
// Every check here runs on the host before anything is enqueued; a failed check launches
// nothing and records a message for dsa_last_error().
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <string>
#include <unordered_map>
#include <unordered_set>

#include "../../include/dsa.h"
#include "dsa_internal.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status ok() {
  g_last_error.clear();
  return DSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dsa_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DSA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

#define DSA_REQUIRE(cond, ...)                                  \
  do {                                                          \
    if (!(cond)) return fail(DSA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

dsa_status check_batch(int32_t num_seqs, int32_t n_q, int32_t max_seq_len, const int32_t* cu_q,
                       const int32_t* seq_lens) {
  DSA_REQUIRE(num_seqs >= 1, "num_seqs must be >= 1 (got %d)", num_seqs);
  DSA_REQUIRE(n_q >= 1, "n_q must be >= 1 (got %d)", n_q);
  DSA_REQUIRE(n_q >= num_seqs, "n_q (%d) must be >= num_seqs (%d): every request has a row", n_q,
              num_seqs);
  DSA_REQUIRE(max_seq_len >= 1, "max_seq_len must be >= 1 (got %d)", max_seq_len);
  DSA_REQUIRE(cu_q != nullptr && seq_lens != nullptr, "cu_q and seq_lens must be non-null");
  return DSA_OK;
}

// Shared checks of the query, the latent cache and the scalars of stage 3.
dsa_status check_mla_inputs(int32_t n_q, const void* q_bf16, const void* q8,
                                   const float* q_scale, const void* latent_pages,
                                   int64_t latent_page_stride, float latent_scale, int32_t k,
                                   float softmax_scale, int32_t num_splits) {
  DSA_REQUIRE(n_q >= 1, "n_q must be >= 1 (got %d)", n_q);
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k must be in 1..4096 (got %d)", k);
  if (num_splits < 1 || num_splits > DSA_MAX_SPLITS)
    return fail(DSA_ERR_UNSUPPORTED, "num_splits must be in 1..64 (got %d)", num_splits);
  DSA_REQUIRE(num_splits <= k, "num_splits (%d) must be <= k (%d)", num_splits, k);
  const bool prepared = q8 != nullptr && q_scale != nullptr;
  DSA_REQUIRE((q8 == nullptr) == (q_scale == nullptr), "q8 and q_scale must both be given or both be NULL");
  DSA_REQUIRE(prepared || q_bf16, "the query is missing: give q_bf16 or q8 and q_scale");
  DSA_REQUIRE(latent_pages, "latent_pages must be non-null");
  DSA_REQUIRE(prepared ? aligned(q8, 16) && aligned(q_scale, 16) : aligned(q_bf16, 16),
              "the query (codes and scales) must be 16-byte aligned");
  DSA_REQUIRE(aligned(latent_pages, 16), "latent_pages must be 16-byte aligned");
  DSA_REQUIRE(latent_page_stride >= DSA_LATENT_PAGE_BYTES && latent_page_stride % 16 == 0,
              "latent_page_stride must be >= 36864 and a multiple of 16 (got %lld)",
              (long long)latent_page_stride);
  DSA_REQUIRE(latent_scale > 0.f, "latent_scale must be > 0");
  DSA_REQUIRE(softmax_scale > 0.f, "softmax_scale must be > 0");
  return DSA_OK;
}

// The indexer inputs the final top-k pass recomputes scores from (all NULL: scores stored).
dsa_status check_rescore(const void* q_idx_bf16, const float* head_w, const void* key_pages,
                         int64_t key_page_stride, int32_t key_format,
                         const int32_t* block_table, int32_t from_candidates) {
  if (!q_idx_bf16 && !head_w && !key_pages) return DSA_OK;
  if (key_format != 0 && key_format != 1)
    return fail(DSA_ERR_UNSUPPORTED, "key_format must be 0 (E4M3) or 1 (MXFP4) (got %d)", key_format);
  DSA_REQUIRE(q_idx_bf16 && head_w && key_pages,
              "q_idx_bf16, head_w and key_pages must all be given (scores not stored) or all be NULL");
  DSA_REQUIRE(from_candidates, "recomputing scores needs the indexer's candidates (from_candidates)");
  DSA_REQUIRE(block_table, "recomputing scores needs block_table");
  DSA_REQUIRE(aligned(q_idx_bf16, 16) && aligned(head_w, 16) && aligned(key_pages, 16),
              "q_idx_bf16, head_w and key_pages must be 16-byte aligned");
  const int64_t page_bytes = key_format ? DSA_IDX_MXFP4_PAGE_BYTES : DSA_IDX_PAGE_BYTES;
  DSA_REQUIRE(key_page_stride >= page_bytes && key_page_stride % 16 == 0,
              "key_page_stride must be >= %lld and a multiple of 16 (got %lld)",
              (long long)page_bytes, (long long)key_page_stride);
  return DSA_OK;
}

dsa_status check_merged_outputs(int32_t n_q, int32_t num_splits, const void* out_bf16,
                                       const float* lse, const void* workspace,
                                       size_t workspace_bytes) {
  DSA_REQUIRE(out_bf16 && lse, "out_bf16 and lse are needed when o_part is NULL");
  DSA_REQUIRE(aligned(out_bf16, 16), "out_bf16 must be 16-byte aligned");
  if (num_splits > 1) {
    const size_t need = dsa::sparse_mla_workspace_bytes(n_q, num_splits);
    if (workspace == nullptr || workspace_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  workspace ? workspace_bytes : (size_t)0, need);
    DSA_REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
  }
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_last_error(void) { return g_last_error.c_str(); }

const char* dsa_version(void) { return "dsa-mi355x 0.1.0 (gfx950)"; }

dsa_status dsa_quantize_q(int32_t rows, int32_t heads, int32_t dim, const void* q_bf16,
                          uint8_t* codes, float* scales, void* stream) {
  DSA_REQUIRE(rows >= 0 && heads >= 1, "rows must be >= 0 and heads >= 1");
  if (dim != DSA_IDX_DIM && dim != DSA_LATENT_DIM)
    return fail(DSA_ERR_UNSUPPORTED, "dim must be 128 or 576 (got %d)", dim);
  DSA_REQUIRE(q_bf16 && codes && scales, "q_bf16, codes and scales must be non-null");
  DSA_REQUIRE(aligned(q_bf16, 16) && aligned(codes, 16), "q_bf16 and codes must be 16-byte aligned");
  return launched(dsa::launch_quantize_q(rows, heads, dim, static_cast<const uint16_t*>(q_bf16),
                                         codes, scales, static_cast<hipStream_t>(stream)),
                  "dsa_quantize_q");
}

namespace {

dsa_status index_score_checked(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                               int32_t max_q_per_seq, const int32_t* cu_q,
                               const int32_t* seq_lens, const void* q_bf16, const float* head_w,
                               const void* key_pages, int64_t key_page_stride,
                               const int32_t* block_table, int32_t bt_stride, float* scores,
                               int64_t score_stride, int32_t cand_k, void* cand_workspace,
                               size_t cand_workspace_bytes, bool mxfp4, void* stream,
                               const char* name,
                               dsa::MlaQueryPrep prep = dsa::MlaQueryPrep{nullptr, nullptr, nullptr}) {
  dsa_status st = check_batch(num_seqs, n_q, max_seq_len, cu_q, seq_lens);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(max_q_per_seq >= 1 && max_q_per_seq <= n_q,
              "max_q_per_seq must be in 1..n_q (got %d)", max_q_per_seq);
  DSA_REQUIRE(q_bf16 && head_w && key_pages && block_table,
              "q_bf16, head_w, key_pages and block_table must be non-null");
  DSA_REQUIRE(scores || cand_workspace,
              "scores may be NULL only when cand_workspace is given (candidates only)");
  DSA_REQUIRE(aligned(q_bf16, 16), "q_bf16 must be 16-byte aligned");
  DSA_REQUIRE(aligned(head_w, 16), "head_w must be 16-byte aligned");
  DSA_REQUIRE(aligned(key_pages, 16), "key_pages must be 16-byte aligned");
  if (mxfp4) {
    DSA_REQUIRE(key_page_stride >= DSA_IDX_MXFP4_PAGE_BYTES && key_page_stride % 16 == 0,
                "key_page_stride must be >= 4352 and a multiple of 16 (got %lld)",
                (long long)key_page_stride);
  } else {
    DSA_REQUIRE(key_page_stride >= DSA_IDX_PAGE_BYTES && key_page_stride % 16 == 0,
                "key_page_stride must be >= 8448 and a multiple of 16 (got %lld)",
                (long long)key_page_stride);
  }
  DSA_REQUIRE(bt_stride >= (max_seq_len + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE,
              "bt_stride (%d) must cover max_seq_len (%d) in pages of 64", bt_stride, max_seq_len);
  if (scores)
    DSA_REQUIRE(score_stride >= max_seq_len, "score_stride (%lld) must be >= max_seq_len (%d)",
                (long long)score_stride, max_seq_len);
  if (cand_workspace) {
    if (cand_k < 1 || cand_k > DSA_MAX_TOPK)
      return fail(DSA_ERR_UNSUPPORTED, "cand_k must be in 1..4096 (got %d)", cand_k);
    const size_t need = dsa::topk_workspace_bytes(n_q, max_seq_len, cand_k);
    if (cand_workspace_bytes < need)
      return fail(DSA_ERR_WORKSPACE, "candidate workspace of %zu bytes is smaller than the %zu needed",
                  cand_workspace_bytes, need);
    DSA_REQUIRE(aligned(cand_workspace, 256), "cand_workspace must be 256-byte aligned");
  }
  return launched(dsa::launch_index_score(num_seqs, n_q, max_seq_len, max_q_per_seq, cu_q, seq_lens,
                                          static_cast<const uint16_t*>(q_bf16), head_w,
                                          static_cast<const uint8_t*>(key_pages), key_page_stride,
                                          block_table, bt_stride, scores, score_stride, cand_k,
                                          cand_workspace, mxfp4, static_cast<hipStream_t>(stream),
                                          prep),
                  name);
}

}  // namespace

dsa_status dsa_index_score(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                           int32_t max_q_per_seq, const int32_t* cu_q, const int32_t* seq_lens,
                           const void* q_bf16, const float* head_w, const void* key_pages,
                           int64_t key_page_stride, const int32_t* block_table, int32_t bt_stride,
                           float* scores, int64_t score_stride, int32_t cand_k,
                           void* cand_workspace, size_t cand_workspace_bytes, void* stream) {
  return index_score_checked(num_seqs, n_q, max_seq_len, max_q_per_seq, cu_q, seq_lens, q_bf16,
                             head_w, key_pages, key_page_stride, block_table, bt_stride, scores,
                             score_stride, cand_k, cand_workspace, cand_workspace_bytes, false,
                             stream, "dsa_index_score");
}

dsa_status dsa_index_score_mxfp4(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                                 int32_t max_q_per_seq, const int32_t* cu_q,
                                 const int32_t* seq_lens, const void* q_bf16, const float* head_w,
                                 const void* key_pages, int64_t key_page_stride,
                                 const int32_t* block_table, int32_t bt_stride, float* scores,
                                 int64_t score_stride, int32_t cand_k, void* cand_workspace,
                                 size_t cand_workspace_bytes, void* stream) {
  return index_score_checked(num_seqs, n_q, max_seq_len, max_q_per_seq, cu_q, seq_lens, q_bf16,
                             head_w, key_pages, key_page_stride, block_table, bt_stride, scores,
                             score_stride, cand_k, cand_workspace, cand_workspace_bytes, true,
                             stream, "dsa_index_score_mxfp4");
}

dsa_status dsa_index_score_quantize_q(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                                      int32_t max_q_per_seq, const int32_t* cu_q,
                                      const int32_t* seq_lens, const void* q_bf16,
                                      const float* head_w, const void* key_pages,
                                      int64_t key_page_stride, int32_t key_format,
                                      const int32_t* block_table, int32_t bt_stride, float* scores,
                                      int64_t score_stride, int32_t cand_k, void* cand_workspace,
                                      size_t cand_workspace_bytes, const void* q_mla_bf16,
                                      uint8_t* q8_mla, float* q_mla_scale, void* stream) {
  if (key_format != 0 && key_format != 1)
    return fail(DSA_ERR_UNSUPPORTED, "key_format must be 0 (E4M3) or 1 (MXFP4) (got %d)", key_format);
  DSA_REQUIRE(q_mla_bf16 && q8_mla && q_mla_scale,
              "q_mla_bf16, q8_mla and q_mla_scale must be non-null");
  DSA_REQUIRE(aligned(q_mla_bf16, 16) && aligned(q8_mla, 16),
              "q_mla_bf16 and q8_mla must be 16-byte aligned");
  return index_score_checked(num_seqs, n_q, max_seq_len, max_q_per_seq, cu_q, seq_lens, q_bf16,
                             head_w, key_pages, key_page_stride, block_table, bt_stride, scores,
                             score_stride, cand_k, cand_workspace, cand_workspace_bytes,
                             key_format == 1, stream, "dsa_index_score_quantize_q",
                             dsa::MlaQueryPrep{static_cast<const uint16_t*>(q_mla_bf16), q8_mla,
                                               q_mla_scale});
}

size_t dsa_topk_workspace_size(int32_t n_q, int32_t max_seq_len, int32_t k) {
  if (n_q < 1 || max_seq_len < 1 || k < 1 || k > DSA_MAX_TOPK) return 0;
  return dsa::topk_workspace_bytes(n_q, max_seq_len, k);
}

dsa_status dsa_topk_workspace_status(const void* workspace, size_t workspace_bytes, void* stream) {
  DSA_REQUIRE(workspace != nullptr, "workspace must be non-null");
  DSA_REQUIRE(workspace_bytes >= dsa::kWsHeaderBytes, "workspace_bytes (%zu) must be >= %zu",
              workspace_bytes, dsa::kWsHeaderBytes);
  int32_t h[5] = {0, 0, 0, 0, 0};
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(h, workspace, sizeof h, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess)
    return fail(DSA_ERR_LAUNCH, "reading the workspace's layout record: %s", hipGetErrorString(e));
  if (h[0] != dsa::kWsMagic)
    return fail(DSA_ERR_WORKSPACE, "the workspace holds no layout record: no call wrote "
                                   "candidates into it");
  if (h[4] != 0)
    return fail(DSA_ERR_WORKSPACE,
                "a final top-k pass found candidates written for k = %d, max_seq_len = %d, "
                "n_q = %d, which differ from its own arguments, and selected nothing",
                h[1], h[2], h[3]);
  return ok();
}

dsa_status dsa_topk(int32_t num_seqs, int32_t n_q, int32_t max_seq_len, const int32_t* cu_q,
                    const int32_t* seq_lens, float* scores, int64_t score_stride, int32_t k,
                    const int32_t* block_table, int32_t bt_stride, int32_t* topk_idx,
                    int32_t* topk_slot, void* workspace, size_t workspace_bytes,
                    int32_t from_candidates, const void* q_idx_bf16, const float* head_w,
                    const void* key_pages, int64_t key_page_stride, int32_t key_format,
                    void* stream) {
  dsa_status st = check_batch(num_seqs, n_q, max_seq_len, cu_q, seq_lens);
  if (st != DSA_OK) return st;
  st = check_rescore(q_idx_bf16, head_w, key_pages, key_page_stride, key_format, block_table,
                     from_candidates);
  if (st != DSA_OK) return st;
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_UNSUPPORTED, "k must be in 1..4096 (got %d)", k);
  DSA_REQUIRE(scores && topk_idx, "scores and topk_idx must be non-null");
  DSA_REQUIRE((block_table == nullptr) == (topk_slot == nullptr),
              "block_table and topk_slot must both be given or both be NULL");
  DSA_REQUIRE(score_stride >= max_seq_len, "score_stride (%lld) must be >= max_seq_len (%d)",
              (long long)score_stride, max_seq_len);
  if (block_table)
    DSA_REQUIRE(bt_stride >= (max_seq_len + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE,
                "bt_stride (%d) must cover max_seq_len (%d) in pages of 64", bt_stride, max_seq_len);
  const size_t need = dsa::topk_workspace_bytes(n_q, max_seq_len, k);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                workspace ? workspace_bytes : (size_t)0, need);
  DSA_REQUIRE(aligned(workspace, 256), "workspace must be 256-byte aligned");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (from_candidates) {
    const dsa::TopkBuffers t = dsa::topk_buffers(workspace, n_q, max_seq_len, k);
    const dsa::IndexRescore rs{static_cast<const uint16_t*>(q_idx_bf16), head_w,
                               static_cast<const uint8_t*>(key_pages), key_page_stride,
                               key_format};
    return launched(dsa::launch_topk_final(num_seqs, n_q, cu_q, seq_lens, scores, score_stride, k,
                                           t, rs, block_table, bt_stride, topk_idx, topk_slot, hs),
                    "dsa_topk");
  }
  return launched(dsa::launch_topk(num_seqs, n_q, max_seq_len, cu_q, seq_lens, scores, score_stride,
                                   k, block_table, bt_stride, topk_idx, topk_slot, workspace, hs),
                  "dsa_topk");
}

size_t dsa_sparse_mla_workspace_size(int32_t n_q, int32_t num_splits) {
  if (n_q < 1 || num_splits < 1 || num_splits > DSA_MAX_SPLITS) return 0;
  return dsa::sparse_mla_workspace_bytes(n_q, num_splits);
}

dsa_status dsa_sparse_mla_decode(int32_t n_q, const void* q_bf16, const void* q8,
                                 const float* q_scale, const void* latent_pages,
                                 int64_t latent_page_stride, float latent_scale,
                                 const int32_t* topk_slot, int32_t k, float softmax_scale,
                                 int32_t num_splits, void* out_bf16, float* lse, float* o_part,
                                 float* lse_part, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  dsa_status st = check_mla_inputs(n_q, q_bf16, q8, q_scale, latent_pages, latent_page_stride,
                                   latent_scale, k, softmax_scale, num_splits);
  if (st != DSA_OK) return st;
  const bool prepared = q8 != nullptr;
  DSA_REQUIRE(topk_slot, "topk_slot must be non-null");
  DSA_REQUIRE((o_part == nullptr) == (lse_part == nullptr),
              "o_part and lse_part must both be given or both be NULL");
  if (o_part) {
    DSA_REQUIRE(aligned(o_part, 16), "o_part must be 16-byte aligned");
  } else {
    st = check_merged_outputs(n_q, num_splits, out_bf16, lse, workspace, workspace_bytes);
    if (st != DSA_OK) return st;
  }
  return launched(dsa::launch_sparse_mla(n_q, static_cast<const uint16_t*>(q_bf16),
                                         prepared ? static_cast<const uint8_t*>(q8) : nullptr,
                                         prepared ? q_scale : nullptr,
                                         static_cast<const uint8_t*>(latent_pages),
                                         latent_page_stride, latent_scale, topk_slot, k,
                                         softmax_scale, num_splits, o_part, lse_part,
                                         static_cast<uint16_t*>(out_bf16), lse, workspace,
                                         static_cast<hipStream_t>(stream)),
                  "dsa_sparse_mla_decode");
}

dsa_status dsa_sparse_mla_decode_noalloc(int32_t n_q, const void* q_bf16, const void* q8,
                                         const float* q_scale, const void* latent_pages,
                                         int64_t latent_page_stride, float latent_scale,
                                         const int32_t* topk_slot, int32_t k, float softmax_scale,
                                         int32_t num_splits, void* out_bf16, float* lse,
                                         float* o_part, float* lse_part, void* stream) {
  dsa_status st = check_mla_inputs(n_q, q_bf16, q8, q_scale, latent_pages, latent_page_stride,
                                   latent_scale, k, softmax_scale, num_splits);
  if (st != DSA_OK) return st;
  const bool prepared = q8 != nullptr;
  DSA_REQUIRE(topk_slot, "topk_slot must be non-null");
  DSA_REQUIRE((o_part == nullptr) == (lse_part == nullptr),
              "o_part and lse_part must both be given or both be NULL");
  if (o_part) {
    DSA_REQUIRE(aligned(o_part, 16), "o_part must be 16-byte aligned");
  } else {
    DSA_REQUIRE(out_bf16 && lse, "out_bf16 and lse are needed when o_part is NULL");
    DSA_REQUIRE(aligned(out_bf16, 16), "out_bf16 must be 16-byte aligned");
    const size_t need = num_splits > 1 ? dsa::sparse_mla_workspace_bytes(n_q, num_splits) : 0;
    if (need > dsa::sparse_mla_noalloc_scratch_bytes())
      return fail(DSA_ERR_WORKSPACE,
                  "n_q = %d rows x %d splits need %zu bytes of split partials; the library's "
                  "static scratch holds %zu (use dsa_sparse_mla_decode with a workspace)",
                  n_q, num_splits, need, dsa::sparse_mla_noalloc_scratch_bytes());
  }
  return launched(dsa::launch_sparse_mla_noalloc(
                      n_q, static_cast<const uint16_t*>(q_bf16),
                      prepared ? static_cast<const uint8_t*>(q8) : nullptr,
                      prepared ? q_scale : nullptr, static_cast<const uint8_t*>(latent_pages),
                      latent_page_stride, latent_scale, topk_slot, k, softmax_scale, num_splits,
                      o_part, lse_part, static_cast<uint16_t*>(out_bf16), lse,
                      static_cast<hipStream_t>(stream)),
                  "dsa_sparse_mla_decode_noalloc");
}

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
                               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  dsa_status st = check_batch(num_seqs, n_q, max_seq_len, cu_q, seq_lens);
  if (st != DSA_OK) return st;
  st = check_mla_inputs(n_q, q_bf16, q8, q_scale, latent_pages, latent_page_stride, latent_scale,
                        k, softmax_scale, num_splits);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(scores && block_table, "scores and block_table must be non-null");
  st = check_rescore(q_idx_bf16, head_w, key_pages, key_page_stride, key_format, block_table, 1);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(score_stride >= max_seq_len, "score_stride (%lld) must be >= max_seq_len (%d)",
              (long long)score_stride, max_seq_len);
  DSA_REQUIRE(bt_stride >= (max_seq_len + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE,
              "bt_stride (%d) must cover max_seq_len (%d) in pages of 64", bt_stride, max_seq_len);
  const size_t need = dsa::topk_workspace_bytes(n_q, max_seq_len, k);
  if (cand_workspace == nullptr || cand_workspace_bytes < need)
    return fail(DSA_ERR_WORKSPACE, "candidate workspace of %zu bytes is smaller than the %zu needed",
                cand_workspace ? cand_workspace_bytes : (size_t)0, need);
  DSA_REQUIRE(aligned(cand_workspace, 256), "cand_workspace must be 256-byte aligned");
  st = check_merged_outputs(n_q, num_splits, out_bf16, lse, workspace, workspace_bytes);
  if (st != DSA_OK) return st;
  const bool prepared = q8 != nullptr;
  const dsa::TopkBuffers t =
      dsa::topk_buffers(const_cast<void*>(cand_workspace), n_q, max_seq_len, k);
  const dsa::IndexRescore rs{static_cast<const uint16_t*>(q_idx_bf16), head_w,
                             static_cast<const uint8_t*>(key_pages), key_page_stride, key_format};
  return launched(dsa::launch_topk_sparse_mla(
                      num_seqs, n_q, cu_q, seq_lens, scores, score_stride, t,
                      rs, block_table,
                      bt_stride, topk_idx, topk_slot, static_cast<const uint16_t*>(q_bf16),
                      prepared ? static_cast<const uint8_t*>(q8) : nullptr,
                      prepared ? q_scale : nullptr, static_cast<const uint8_t*>(latent_pages),
                      latent_page_stride, latent_scale, k, softmax_scale, num_splits,
                      static_cast<uint16_t*>(out_bf16), lse, workspace,
                      static_cast<hipStream_t>(stream)),
                  "dsa_topk_sparse_mla");
}

namespace {
dsa_status cache_append(int32_t n_tok, const int32_t* slots, const void* key_bf16,
                        const void* latent_bf16, float latent_scale, void* key_pages,
                        int64_t key_page_stride, void* latent_pages, int64_t latent_page_stride,
                        void* stream, bool mx_keys, const char* name) {
  DSA_REQUIRE(n_tok >= 0, "n_tok must be >= 0 (got %d)", n_tok);
  DSA_REQUIRE(slots, "slots must be non-null");
  DSA_REQUIRE(key_bf16 || latent_bf16, "give key_bf16, latent_bf16 or both");
  if (key_bf16) {
    const int64_t min_stride = mx_keys ? DSA_IDX_MXFP4_PAGE_BYTES : DSA_IDX_PAGE_BYTES;
    DSA_REQUIRE(key_pages, "key_pages must be non-null when key_bf16 is given");
    DSA_REQUIRE(aligned(key_bf16, 16) && aligned(key_pages, 16),
                "key_bf16 and key_pages must be 16-byte aligned");
    DSA_REQUIRE(key_page_stride >= min_stride && key_page_stride % 16 == 0,
                "key_page_stride must be >= %lld and a multiple of 16 (got %lld)",
                (long long)min_stride, (long long)key_page_stride);
  }
  if (latent_bf16) {
    DSA_REQUIRE(latent_pages, "latent_pages must be non-null when latent_bf16 is given");
    DSA_REQUIRE(aligned(latent_bf16, 16) && aligned(latent_pages, 16),
                "latent_bf16 and latent_pages must be 16-byte aligned");
    DSA_REQUIRE(latent_page_stride >= DSA_LATENT_PAGE_BYTES && latent_page_stride % 16 == 0,
                "latent_page_stride must be >= 36864 and a multiple of 16 (got %lld)",
                (long long)latent_page_stride);
    DSA_REQUIRE(latent_scale > 0.f, "latent_scale must be > 0");
  }
  return launched(dsa::launch_cache_append(n_tok, slots, static_cast<const uint16_t*>(key_bf16),
                                           static_cast<const uint16_t*>(latent_bf16),
                                           latent_scale, static_cast<uint8_t*>(key_pages),
                                           key_page_stride, static_cast<uint8_t*>(latent_pages),
                                           latent_page_stride, mx_keys,
                                           static_cast<hipStream_t>(stream)),
                  name);
}
}  // namespace

dsa_status dsa_cache_append(int32_t n_tok, const int32_t* slots, const void* key_bf16,
                            const void* latent_bf16, float latent_scale, void* key_pages,
                            int64_t key_page_stride, void* latent_pages,
                            int64_t latent_page_stride, void* stream) {
  return cache_append(n_tok, slots, key_bf16, latent_bf16, latent_scale, key_pages,
                      key_page_stride, latent_pages, latent_page_stride, stream, false,
                      "dsa_cache_append");
}

dsa_status dsa_cache_append_mxfp4(int32_t n_tok, const int32_t* slots, const void* key_bf16,
                                  const void* latent_bf16, float latent_scale, void* key_pages,
                                  int64_t key_page_stride, void* latent_pages,
                                  int64_t latent_page_stride, void* stream) {
  return cache_append(n_tok, slots, key_bf16, latent_bf16, latent_scale, key_pages,
                      key_page_stride, latent_pages, latent_page_stride, stream, true,
                      "dsa_cache_append_mxfp4");
}

dsa_status dsa_validate_batch(int32_t num_seqs, int32_t n_q, int32_t max_seq_len,
                              int32_t max_q_per_seq, const int32_t* cu_q, const int32_t* seq_lens,
                              const int32_t* block_table, int32_t bt_stride, int64_t num_pages,
                              const int32_t* topk_slot, int32_t k) {
  dsa_status st = check_batch(num_seqs, n_q, max_seq_len, cu_q, seq_lens);
  if (st != DSA_OK) return st;
  DSA_REQUIRE(max_q_per_seq >= 1, "max_q_per_seq must be >= 1 (got %d)", max_q_per_seq);
  DSA_REQUIRE(block_table, "block_table must be non-null");
  DSA_REQUIRE(num_pages >= 1, "num_pages must be >= 1 (got %lld)", (long long)num_pages);
  const int64_t max_pages = ((int64_t)max_seq_len + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE;
  DSA_REQUIRE(bt_stride >= max_pages, "bt_stride (%d) must be >= ceil(max_seq_len / 64) = %lld",
              bt_stride, (long long)max_pages);
  DSA_REQUIRE(cu_q[0] == 0, "cu_q[0] must be 0 (got %d)", cu_q[0]);
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t nb = cu_q[b + 1] - cu_q[b];
    DSA_REQUIRE(nb >= 1 && nb <= max_q_per_seq,
                "request %d has %d query rows (cu_q must increase, by 1..max_q_per_seq = %d)", b,
                nb, max_q_per_seq);
    const int32_t L = seq_lens[b];
    DSA_REQUIRE(L >= 1 && L <= max_seq_len, "seq_lens[%d] = %d is outside 1..max_seq_len (%d)", b,
                L, max_seq_len);
    DSA_REQUIRE(nb <= L, "request %d has %d rows but only %d tokens (its rows are its last tokens)",
                b, nb, L);
    const int32_t* bt = block_table + (int64_t)b * bt_stride;
    for (int32_t j = 0; j < (L + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE; ++j)
      DSA_REQUIRE(bt[j] >= 0 && bt[j] < num_pages,
                  "block_table[%d][%d] = %d is not a page of the pool (0..%lld)", b, j, bt[j],
                  (long long)num_pages - 1);
  }
  DSA_REQUIRE(cu_q[num_seqs] == n_q, "cu_q[num_seqs] = %d must equal n_q = %d", cu_q[num_seqs], n_q);
  if (!topk_slot) return ok();
  DSA_REQUIRE(k >= 1 && k <= DSA_MAX_TOPK, "k must be in 1..4096 (got %d)", k);
  // every slot of row i must hold a token the row sees: page BT[b][j] and offset o with
  // 64 j + o <= position; valid slots of a row are distinct
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t* bt = block_table + (int64_t)b * bt_stride;
    const int32_t nb = cu_q[b + 1] - cu_q[b];
    std::unordered_map<int32_t, int32_t> first_page;  // physical page -> lowest logical page
    for (int32_t j = (seq_lens[b] + DSA_PAGE_SIZE - 1) / DSA_PAGE_SIZE - 1; j >= 0; --j)
      first_page[bt[j]] = j;
    for (int32_t r = 0; r < nb; ++r) {
      const int32_t row = cu_q[b] + r;
      const int64_t pos = (int64_t)seq_lens[b] - nb + r;
      const int32_t* sl = topk_slot + (int64_t)row * k;
      std::unordered_set<int32_t> seen;
      for (int32_t i = 0; i < k; ++i) {
        const int32_t s = sl[i];
        if (s == -1) continue;
        DSA_REQUIRE(s >= 0, "topk_slot[%d][%d] = %d is neither -1 nor a slot", row, i, s);
        const auto it = first_page.find(s / DSA_PAGE_SIZE);
        DSA_REQUIRE(it != first_page.end() &&
                        (int64_t)it->second * DSA_PAGE_SIZE + s % DSA_PAGE_SIZE <= pos,
                    "topk_slot[%d][%d] = %d is not a token row %d sees (position %lld)", row, i, s,
                    row, (long long)pos);
        DSA_REQUIRE(seen.insert(s).second, "topk_slot[%d] holds slot %d twice", row, s);
      }
    }
  }
  return ok();
}

dsa_status dsa_validate_slots(int32_t n_tok, const int32_t* slots, int64_t num_pages) {
  DSA_REQUIRE(n_tok >= 0, "n_tok must be >= 0 (got %d)", n_tok);
  DSA_REQUIRE(n_tok == 0 || slots, "slots must be non-null");
  DSA_REQUIRE(num_pages >= 1, "num_pages must be >= 1 (got %lld)", (long long)num_pages);
  std::unordered_set<int32_t> seen;
  for (int32_t i = 0; i < n_tok; ++i) {
    const int32_t s = slots[i];
    if (s == -1) continue;
    DSA_REQUIRE(s >= 0 && s / DSA_PAGE_SIZE < num_pages,
                "slots[%d] = %d is neither -1 nor a slot of the pool (%lld pages)", i, s,
                (long long)num_pages);
    DSA_REQUIRE(seen.insert(s).second, "slot %d appears twice (entry %d)", s, i);
  }
  return ok();
}

dsa_status dsa_lse_combine(int32_t num_splits, int32_t n_q, const float* o_part,
                           const float* lse_part, void* out_bf16, float* lse, void* stream) {
  if (num_splits < 1 || num_splits > DSA_MAX_SPLITS)
    return fail(DSA_ERR_UNSUPPORTED, "num_splits must be in 1..64 (got %d)", num_splits);
  DSA_REQUIRE(n_q >= 1, "n_q must be >= 1 (got %d)", n_q);
  DSA_REQUIRE(o_part && lse_part && out_bf16 && lse, "o_part, lse_part, out_bf16, lse must be non-null");
  DSA_REQUIRE(aligned(o_part, 16) && aligned(out_bf16, 8), "o_part must be 16-byte and out_bf16 8-byte aligned");
  return launched(dsa::launch_lse_combine(num_splits, n_q, o_part, lse_part,
                                          static_cast<uint16_t*>(out_bf16), lse,
                                          static_cast<hipStream_t>(stream)),
                  "dsa_lse_combine");
}

}  // extern "C"
