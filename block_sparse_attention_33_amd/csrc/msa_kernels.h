// Host-side launchers of the MSA kernels.  Every launcher enqueues on the
// given stream and returns the launch status; shapes are validated by the
// C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Tokens of one main-branch work item hold at most this many query rows
// (tokens x heads of the group).
constexpr int kItemRows = 256;

struct PrefillShape {
  int B, S, Hq, G, r, bs, bs_log2, nb, top_k;
  float scale_log2;  // softmax scale * log2(e)
};

// Block summary keys: k_idx [U, S, 64] -> block_keys [U, nb, 64].
hipError_t launch_pool(const int8_t* k_idx, int8_t* block_keys, int units, int S, int bs,
                       hipStream_t st);

// Scores + per-(query, group) top-k.  counts (nullable) [U, nb] receives,
// for every query, +1 on each selected block before the query's own block.
hipError_t launch_index_topk(const int8_t* q_idx, const int8_t* block_keys, int32_t* sel,
                             int32_t* counts, int units, int S, int bs, int top_k, hipStream_t st);

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t st);

// Query -> block inversion.
//   scan:    counts [n] -> row_ptr [n + 1], item_ptr [n + 1] (exclusive, int32),
//            items of a block = ceil(count / tokens_per_item)
//   items:   item list {block id, first entry} for every block
//   scatter: entries[row_ptr[blk] + pos] = (t << 5) | slot for every
//            selected off-diagonal block of every query
hipError_t launch_scan(const int32_t* counts, int32_t* row_ptr, int32_t* item_ptr, int n,
                       int tokens_per_item, hipStream_t st);
hipError_t launch_build_items(const int32_t* row_ptr, const int32_t* item_ptr, int2* items, int n,
                              int tokens_per_item, hipStream_t st);
hipError_t launch_scatter(const int32_t* sel, const int32_t* row_ptr, int32_t* fill,
                          uint32_t* entries, int units, int S, int bs, int top_k, int nb,
                          hipStream_t st);

// Main branch, off-diagonal blocks: one work item = one KV block and up to
// kItemRows query rows that selected it; writes normalised bf16 partials and
// their base-2 log-sum-exp.  Items [item_ptr[u0 * nb], item_ptr[u1 * nb]).
hipError_t launch_main_offdiag(const PrefillShape& sh, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr,
                               const int2* items, const uint32_t* entries, uint16_t* part_o,
                               float* part_lse, int u0, int u1, int max_items, hipStream_t st);

// Main branch, own (diagonal) block of every query + merge of the partials
// -> out, for units [u0, u1).
hipError_t launch_diag_merge(const PrefillShape& sh, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const uint16_t* part_o, const float* part_lse,
                             uint16_t* out, int u0, int u1, hipStream_t st);

// Decode.
struct DecodeShape {
  int B, L, Hq, G, r, bs, nb, top_k, n_chunks, chunk;
  float scale_log2;
};
hipError_t launch_decode_index(const DecodeShape& sh, const int8_t* q_idx, const int8_t* block_keys,
                               int64_t* chunk_best, int32_t* counters, hipStream_t st);
hipError_t launch_decode_attend(const DecodeShape& sh, const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int64_t* chunk_best, int32_t* sel,
                                float* part_o, float* part_ml, int32_t* counters, uint16_t* out,
                                hipStream_t st);

}  // namespace msa
