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

// Scores + per-(query, group) top-k -> sel [U, S, top_k].
hipError_t launch_index_topk(const int8_t* q_idx, const int8_t* block_keys, int32_t* sel, int units,
                             int S, int bs, int top_k, hipStream_t st);

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t st);

// Query -> block inversion (no global atomics).  Queries are cut into
// n_chunks chunks of tpc tokens; H [U, n_chunks, nb] int32 holds per-chunk
// block counts, then (in place) each chunk's first position in a block list.
//   chunk_hist:    sel -> H (counts of kept blocks before the own block)
//   chunk_total:   H -> counts [U * nb]
//   scan:          counts -> row_ptr [n + 1], item_ptr [n + 1] (exclusive),
//                  items of a block = ceil(count / tokens_per_item)
//   offsets_items: H -> chunk offsets (in place); item list {block id, first entry}
//   scatter:       entries[...] = (t << 5) | slot for every kept block before
//                  the query's own block
constexpr int kMaxInvertBlocks = 36864;  // nb limit: LDS histogram of nb int32
hipError_t launch_chunk_hist(const int32_t* sel, int32_t* H, int units, int S, int nb, int bs, int top_k,
                             int tpc, int n_chunks, hipStream_t st);
hipError_t launch_chunk_total(const int32_t* H, int32_t* counts, int units, int nb, int n_chunks,
                              hipStream_t st);
hipError_t launch_scan(const int32_t* counts, int32_t* row_ptr, int32_t* item_ptr, int n,
                       int tokens_per_item, hipStream_t st);
hipError_t launch_offsets_items(int32_t* H, const int32_t* row_ptr, const int32_t* item_ptr, int2* items,
                                int units, int nb, int n_chunks, int tokens_per_item, hipStream_t st);
hipError_t launch_scatter(const int32_t* sel, const int32_t* H, uint32_t* entries, int units, int S, int nb,
                          int bs, int top_k, int tpc, int n_chunks, hipStream_t st);

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
  int B, L, Hq, G, r, bs, nb, top_k;
  float scale_log2;
};
constexpr int kDecodeCandPerThread = 32;  // candidates per thread of the index workgroup
constexpr int kDecodeMaxCandidates = 256 * kDecodeCandPerThread;
hipError_t launch_decode_index(const DecodeShape& sh, const int8_t* q_idx, const int8_t* block_keys,
                               int32_t* sel_out, hipStream_t st);
hipError_t launch_decode_attend(const DecodeShape& sh, const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int32_t* sel, float* part_o, float* part_ml,
                                hipStream_t st);
hipError_t launch_decode_merge(const DecodeShape& sh, const float* part_o, const float* part_ml, uint16_t* out,
                               hipStream_t st);

}  // namespace msa
