// Host-side launchers of the MSA kernels.  Every launcher enqueues on the
// given stream and returns the launch status; shapes are validated by the
// C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Compute units of the current device (queried once per device).
hipError_t current_cu_count(int* n_cu);
// Raises the dynamic-LDS limit of kernel `fn` on the current device to at
// least `bytes` (once per device and kernel; thread-safe).
hipError_t ensure_dynamic_lds(const void* fn, int bytes);

// Tokens of one main-branch work item hold at most this many query rows
// (tokens x heads of the group).
constexpr int kItemRows = 256;

struct PrefillShape {
  int B, S, Hq, G, r, bs, bs_log2, nb, top_k;  // S: query rows per unit, nb: CSR blocks per unit
  int q0;            // position of query row 0 (queries are tokens q0 .. q0 + S - 1)
  int q_stride;      // rows per unit (batch) of q and out: S, or more for a slice of longer tensors
  int kv_rows;       // K/V rows per unit (stride); keys present: q0 + S
  int n_ranges;      // query ranges per unit: CSR rows are (unit, range, block)
  int range_tokens;  // tokens per query range
  float scale_log2;  // softmax scale * log2(e)
  float* lse;        // [B, q_stride, Hq] natural log-sum-exp of each row's scores, or null
};

// One pass of the main branch: units [u0, u1) x query range `rng` (always
// range 0 when a unit has a single range).  Partials of the pass are indexed
// ((u - u0) * pass_tokens + (t - t0)) * top_k + slot.
struct PassInfo {
  int u0, u1, rng, t0, t1, pass_tokens;
  int row_begin, row_end;  // CSR rows of the pass
};

// Block summary keys: k_idx [U, S, 64] -> block_keys [U, nb, 64].
hipError_t launch_pool(const int8_t* k_idx, int8_t* block_keys, int units, int S, int bs,
                       hipStream_t st);
// The same over the first S tokens of rows s_stride apart, summaries
// nb_stride apart, blocks j0 .. ceil(S / bs) - 1 only; open_sums [U, 64]
// (optional) receives the int32 sums of the block the next token goes to
// (zero when S is a multiple of bs).
hipError_t launch_pool_strided(const int8_t* k_idx, int8_t* block_keys, int32_t* open_sums, int units, int S,
                               long s_stride, int nb_stride, int bs, int j0, hipStream_t st);

// Scores + per-(query, group) top-k -> sel [U, S, top_k].  Launches whose
// queries rank at least kIndexMfmaMinBlocks blocks score on the matrix
// cores, the others with dot4 instructions; the selections are the same.
// (Measured on MI355X with the matrix-core kernel at four workgroups per
// CU: 16K queries over 256 blocks 0.075 -> 0.069 ms, 2048 tokens over 32
// blocks 0.015 -> 0.010 ms.)
constexpr int kIndexMfmaMinBlocks = 16;
hipError_t launch_index_topk(const int8_t* q_idx, const int8_t* block_keys, int32_t* sel, int units,
                             int S, int bs, int top_k, hipStream_t st);
// The same for queries at positions q0 .. q0 + S - 1 (rows 0 .. S - 1 of
// q_idx and sel, q_stride and sel_stride rows apart per unit), summaries
// nb_stride rows apart per unit.
hipError_t launch_index_topk_at(const int8_t* q_idx, const int8_t* block_keys, int32_t* sel, int units, int S,
                                int q0, int q_stride, int sel_stride, int nb_stride, int bs, int top_k,
                                hipStream_t st);

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t st);

// Measurement aid: n_workgroups workgroups of 4 waves, each wave iters
// rounds of 4 independent bf16 MFMAs on register operands; one float per
// thread to out.  mfma_probe_flop: the FLOP one such launch performs.
hipError_t launch_mfma_probe(float* out, int n_workgroups, int iters, hipStream_t st);
double mfma_probe_flop(int n_workgroups, int iters);

// Query -> block inversion (no global atomics).  Each query range of T
// tokens is cut into m chunks of tpc tokens (n_chunks = n_ranges * m per
// unit); H [U, n_chunks, nb] int32 holds per-chunk block counts, then (in
// place) each chunk's first position in its (unit, range, block) list.
//   chunk_hist:    sel -> H (counts of kept blocks, the own block only if
//                  with_own)
//   chunk_total:   H -> counts [U * n_ranges * nb]
//   scan:          counts -> row_ptr [n + 1], item_ptr [n + 1] (exclusive),
//                  items of a row = ceil(count / tokens_per_item)
//   offsets_items: H -> chunk offsets (in place); item list {row id, first entry}
//   scatter:       entries[...] = (t << 5) | slot for every kept block (the
//                  own block sits at slot min(top_k - 1, t / block_size) and
//                  is listed only if with_own)
constexpr int kMaxInvertBlocks = 36864;  // nb limit: LDS histogram of nb int32
struct ChunkPlan {
  int T, m, tpc, n_chunks, n_ranges;
  int q_stride;  // rows per unit of sel
};
// (query rows are tokens q0 .. q0 + S - 1)
hipError_t launch_chunk_hist(const int32_t* sel, int32_t* H, int units, int S, int nb, int bs, int top_k,
                             const ChunkPlan& cp, int q0, bool with_own, hipStream_t st);
hipError_t launch_chunk_total(const int32_t* H, int32_t* counts, int units, int nb, const ChunkPlan& cp,
                              hipStream_t st);
hipError_t launch_scan(const int32_t* counts, int32_t* row_ptr, int32_t* item_ptr, int n,
                       int tokens_per_item, hipStream_t st);
hipError_t launch_offsets_items(int32_t* H, const int32_t* row_ptr, const int32_t* item_ptr, int2* items,
                                int units, int nb, const ChunkPlan& cp, int tokens_per_item, hipStream_t st);
hipError_t launch_scatter(const int32_t* sel, const int32_t* H, uint32_t* entries, int units, int S, int nb,
                          int bs, int top_k, const ChunkPlan& cp, int q0, bool with_own, hipStream_t st);

// Main branch: one work item = one KV block of a (unit, range) row and up to
// kItemChunks chunks of kItemRows gathered query rows (the lists hold the
// blocks before each query's own); writes unnormalised bf16 partials +
// (running max, sum) in base-2 units per (token, selection slot, head), the
// 16-byte pieces of a (token, slot)'s heads interleaved.  Items
// [item_ptr[row_begin], item_ptr[row_end]).
// Chunks per work item: more chunks load a block's K/V for fewer items
// (measured on MI355X against 4: the 32K prefill 2.3 %, the structured 128K
// 3.4 %, the 1M 0.8 % faster; 8 was slower at 32K and 128K), and the LDS
// entry rings (three items' entries per wave) still fit beside the two K/V
// buffers at one query head per group.
constexpr int kItemChunks = 6;
// sched: one int of scratch (the run counter), zeroed by the launch.
hipError_t launch_attend(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr, const int2* items,
                         const uint32_t* entries, uint16_t* part_o, float2* part_ml, int* sched, int max_items,
                         hipStream_t st);

// Dense causal attention of every query row (for top_k >= nb, when the
// selection keeps every block up to the own one, and for the short-sequence
// switch) -> out, and that selection -> sel [U, sel_rows, top_k] when
// non-null.
hipError_t launch_dense(const PrefillShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* out, int32_t* sel, int sel_rows, hipStream_t st);

// Attention of the pass's query rows over their own blocks, merged with
// every other partial of the rows -> out (and lse when sh.lse is set).
hipError_t launch_merge(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* part_o, const float2* part_ml, uint16_t* out,
                        hipStream_t st);

// Backward of the main branch (selection fixed).
struct BwdShape {
  int B, S, Hq, G, r, r_log2, bs, bs_log2, nb, top_k, U;
  float scale, scale_log2;
  int q0, n_q;           // this pass: query rows q0 .. q0 + n_q - 1 (CSR entries and dq partials relative to q0)
  float *acc_k, *acc_v;  // [U, S, 128] fp32 sums of dK^T (unscaled) and dV^T over passes, or null: one pass, bf16 out
};
// delta[row] = sum_d dout[row][d] * out[row][d] (fp32) for rows of 128 dims.
hipError_t launch_bwd_delta(const uint16_t* out, const uint16_t* dout, float* delta, long rows, hipStream_t st);
// One workgroup per CSR row (unit, block), rows (u, j) with j-major order:
// dk, dv [U, S, 128] of the block's keys (or their fp32 sums added to
// acc_k, acc_v) and the bf16 dq partials part_dq [U, n_q, top_k, r, 128] of
// every (query row, slot) of the row.
// lse [B, S, Hq] natural log-sum-exp of the forward, delta as above.
hipError_t launch_bwd_kv(const BwdShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, const float* lse, const float* delta, const int32_t* row_ptr,
                         const uint32_t* entries, uint16_t* dk, uint16_t* dv, uint16_t* part_dq, hipStream_t st);
// dq [B, S, Hq, 128] of the pass's rows = scale * sum of each row's partials.
hipError_t launch_bwd_dq(const BwdShape& sh, const uint16_t* part_dq, uint16_t* dq, hipStream_t st);
// dk = bf16(scale * acc_k), dv = bf16(acc_v) after the last pass.
hipError_t launch_bwd_acc(const BwdShape& sh, uint16_t* dk, uint16_t* dv, hipStream_t st);

// Decode.
struct DecodeShape {
  int B, L, Hq, G, r, bs, nb, top_k;  // L tokens in the caches, nb = ceil(L / bs)
  int Lc, nbc;                        // cache rows and summary rows per unit (capacity)
  float scale_log2;
  // device int32 [B]: sequence b holds lens[b] tokens (1 .. Lc) and L, nb
  // are the largest; null: every sequence holds L
  const int32_t* lens;
};
// Up to kLengthBatch host lengths carried by value in one launch's arguments.
constexpr int kLengthBatch = 512;
struct LengthBatch {
  int32_t v[kLengthBatch];
};
// dst[0 .. n) = lengths[0 .. n) (host), in launches of kLengthBatch values.
hipError_t launch_set_lengths(int32_t* dst, const int32_t* lengths, int n, hipStream_t st);
constexpr int kDecodeMaxCandidates = 16 * 512;  // 512 threads x 16 candidates
// Selection (-> sel [U, top_k]: ascending, own block last, -1 padding) and
// attention over the kept blocks.  n_split workgroups share a unit's slots;
// with n_split = 1 the kernel writes out [B, Hq, 128], otherwise each
// workgroup writes its state [U, n_split, r, 128 + 2] (o, max, sum) and
// launch_decode_merge combines them into out.
hipError_t launch_decode(const DecodeShape& sh, const uint16_t* q, const int8_t* q_idx, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int8_t* block_keys, int32_t* sel_out, uint16_t* out,
                         float* state, int n_split, hipStream_t st);
// Device address, on the current device, of the library's fixed decode
// scratch (kDecodeScratchBytes, 256-byte aligned), looked up once per device.
constexpr size_t kDecodeScratchBytes = 16u << 20;
hipError_t decode_scratch(void** ptr);
// Append of token pos of every unit: k_new/v_new [U, 128] -> cache row pos,
// k_idx_new [U, 64] -> open_sums [U, 64] and block_keys[u][pos / bs].
hipError_t launch_append(const DecodeShape& sh, const uint16_t* k_new, const uint16_t* v_new,
                         const int8_t* k_idx_new, uint16_t* k_cache, uint16_t* v_cache, int32_t* open_sums,
                         int8_t* block_keys, int pos, hipStream_t st);
hipError_t launch_decode_merge(const DecodeShape& sh, const float* state, int n_split, uint16_t* out,
                               hipStream_t st);

}  // namespace msa
