// Host-side launchers of the gfx950 kernels (called by the C ABI after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct TopkPlan {
  int num_groups;   // 256-token first-pass groups covering max_seq_len
  int row_cap;      // candidate slots reserved per row
};

struct ChunkInfo;

// Inputs the final top-k pass recomputes scores from when the indexer did not store them
// (q == nullptr: the scores are stored).
struct IndexRescore {
  const uint16_t* q;       // indexer query bf16 [n_q][32][128]
  const float* head_w;     // [n_q][32]
  const uint8_t* key_pages;
  int64_t page_stride;
  int mxfp4;               // key cache format: 0 E4M3 + fp32 scale, 1 MXFP4
};

// The first 256 bytes of a top-k workspace hold a layout record: the pass that writes the
// candidates (the indexer, or the first pass of dsa_topk) stores (magic, k, max_seq_len, n_q,
// status = 0); the final pass compares it with its own arguments, and on a mismatch (the two
// calls disagree about where the candidates lie) selects nothing (-1) and sets status to 1.
constexpr int32_t kWsMagic = 0x44534131;  // "DSA1"
constexpr size_t kWsHeaderBytes = 256;
struct WsLayout {
  int32_t* header;  // the workspace's first bytes
  int k, max_seq_len, n_q;
};

struct TopkBuffers {
  TopkPlan plan;
  uint32_t* cand_key;
  int32_t* cand_idx;
  ChunkInfo* info;
  WsLayout layout;
};

TopkPlan topk_plan(int max_seq_len, int k);
size_t topk_workspace_bytes(int n_q, int max_seq_len, int k);
TopkBuffers topk_buffers(void* workspace, int n_q, int max_seq_len, int k);
// Final pass only: the workspace already holds every group's candidates.
// With rs.q set, scores is scratch: the pass recomputes there the groups it must re-read.
hipError_t launch_topk_final(int num_seqs, int n_q, const int32_t* cu_q, const int32_t* seq_lens,
                             const float* scores, int64_t score_stride, int k,
                             const TopkBuffers& t, const IndexRescore& rs,
                             const int32_t* block_table, int bt_stride, int32_t* topk_idx,
                             int32_t* topk_slot, hipStream_t st);

hipError_t launch_quantize_q(int rows, int heads, int dim, const uint16_t* q, uint8_t* codes,
                             float* scales, hipStream_t st);

// The MLA query's E4M3 quantisation carried by an indexer launch: codes [n_q][96][576] and
// scales [n_q][96], bitwise what launch_quantize_q(n_q, 96, 576, q, ...) writes.
struct MlaQueryPrep {
  const uint16_t* q;  // bf16 [n_q][96][576]; nullptr: no preparation
  uint8_t* codes;
  float* scales;
};

// topk_ws == nullptr: scores only.  Otherwise the kernel also writes every 256-token group's
// top-k candidates for a top-k of k into topk_ws (see topk_buffers).  mxfp4: the key cache
// holds MXFP4 keys (4,352-byte pages) instead of E4M3 keys with an fp32 scale.  prep.q set:
// one more workgroup per request and row group quantises those rows' MLA query.
hipError_t launch_index_score(int num_seqs, int n_q, int max_seq_len, int max_q_per_seq,
                              const int32_t* cu_q, const int32_t* seq_lens, const uint16_t* q,
                              const float* head_w, const uint8_t* key_pages, int64_t key_page_stride,
                              const int32_t* block_table, int bt_stride, float* scores,
                              int64_t score_stride, int k, void* topk_ws, bool mxfp4,
                              hipStream_t st, MlaQueryPrep prep = MlaQueryPrep{nullptr, nullptr, nullptr});

hipError_t launch_topk(int num_seqs, int n_q, int max_seq_len, const int32_t* cu_q,
                       const int32_t* seq_lens, const float* scores, int64_t score_stride, int k,
                       const int32_t* block_table, int bt_stride, int32_t* topk_idx,
                       int32_t* topk_slot, void* workspace, hipStream_t st);

// workspace: fp16 split partials (num_splits > 1 and no o_part)
size_t sparse_mla_workspace_bytes(int n_q, int num_splits);
// q8 / q_scale: the prepared query (both non-null) or nullptr to quantise q in the kernel.
// o_part != nullptr: fp32 partials of every split; else out/lse, merged through the
// workspace when num_splits > 1.
hipError_t launch_sparse_mla(int n_q, const uint16_t* q, const uint8_t* q8, const float* q_scale,
                             const uint8_t* latent_pages, int64_t latent_page_stride,
                             float latent_scale, const int32_t* topk_slot, int k,
                             float softmax_scale, int num_splits, float* o_part, float* lse_part,
                             uint16_t* out_bf16, float* lse, void* workspace, hipStream_t st);

// The same without a workspace: the fp16 split partials go to the library's static device
// scratch (sparse_mla_noalloc_scratch_bytes() bytes per device; calls on one GPU share it).
size_t sparse_mla_noalloc_scratch_bytes();
hipError_t launch_sparse_mla_noalloc(int n_q, const uint16_t* q, const uint8_t* q8,
                                     const float* q_scale, const uint8_t* latent_pages,
                                     int64_t latent_page_stride, float latent_scale,
                                     const int32_t* topk_slot, int k, float softmax_scale,
                                     int num_splits, float* o_part, float* lse_part,
                                     uint16_t* out_bf16, float* lse, hipStream_t st);

// Stage 2's final pass fused into the sparse MLA: every (split, row) workgroup selects its
// row's top k from the candidates in t, then attends (out/lse, fp16-merged when S > 1).
hipError_t launch_topk_sparse_mla(int num_seqs, int n_q, const int32_t* cu_q,
                                  const int32_t* seq_lens, float* scores,
                                  int64_t score_stride, const TopkBuffers& t,
                                  const IndexRescore& rs, const int32_t* block_table,
                                  int bt_stride, int32_t* topk_idx, int32_t* topk_slot,
                                  const uint16_t* q, const uint8_t* q8,
                                  const float* q_scale, const uint8_t* latent_pages,
                                  int64_t latent_page_stride, float latent_scale, int k,
                                  float softmax_scale, int num_splits, uint16_t* out_bf16,
                                  float* lse, void* workspace, hipStream_t st);

// New tokens' index keys (bf16 [n][128]) and latents (bf16 [n][576]) quantised into the
// paged caches at their physical slots (-1: skipped); key or lat may be null.  mx_keys: the
// index-key cache holds MXFP4 pages (else E4M3 pages).
hipError_t launch_cache_append(int n_tok, const int32_t* slots, const uint16_t* key,
                               const uint16_t* lat, float lat_scale, uint8_t* key_pages,
                               int64_t key_page_stride, uint8_t* lat_pages,
                               int64_t lat_page_stride, bool mx_keys, hipStream_t st);

hipError_t launch_lse_combine(int num_splits, int n_q, const float* o_part, const float* lse_part,
                              uint16_t* out_bf16, float* lse, hipStream_t st);
hipError_t launch_lse_combine_f16(int num_splits, int n_q, const uint16_t* o_part,
                                  const float* lse_part, float scale, uint16_t* out_bf16,
                                  float* lse, hipStream_t st);

}  // namespace dsa
