/*
 * msa.h -- C ABI of the MiniMax Sparse Attention (MSA) hot path for AMD
 * Instinct MI355X (gfx950).
 *
 * MSA is grouped-query attention (GQA) split into two branches.  An index
 * branch ranks the key/value blocks that precede a query and lets every GQA
 * group keep its own top-k set; a main branch runs exact softmax attention
 * over the kept blocks only ("深度解析 MiniMax-M3：稀疏注意力机制、基准测试与
 * API 集成指南", section "架构核心：MoE 与 MSA 的深度融合", items 1 and 2; the
 * wiki.500nian.com digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI
 * Agents", flowchart nodes "Index Branch" and "Main Branch").  The ranking is
 * exponent-free: integer scores are compared directly (same flowchart, node
 * "exp-free Top-k").  The pages give no formula for the index branch; this
 * library fixes it as follows:
 *
 *   summary key of block j  s_j = floor( sum_{t in block j} k_idx[t] / n_j )
 *                                  (int8, floor toward -inf, n_j = tokens in j)
 *   score of block j        q_idx[t] . s_j   (exact int32 dot product)
 *   candidates of query t   blocks 0 .. b_t - 1, b_t = floor(t / block_size)
 *   selection               the best top_k - 1 candidates by score, ties to the
 *                           lower block index (all of them if fewer exist),
 *                           plus the own block b_t, listed ascending and padded
 *                           with -1 to top_k entries
 *   attention               one softmax over every key of the selected blocks
 *                           at a position <= t, scale softmax_scale
 *
 * Query head h belongs to group g = h / (n_q_heads / n_kv_heads).
 *
 * Layouts (row-major, contiguous, element types as named):
 *   q, out       [B, S, Hq, D]    bf16 bits (uint16_t)
 *   k, v         [B, G, S, D]     bf16 bits, G = n_kv_heads
 *   q_idx, k_idx [B, G, S, di]    int8
 *   block_keys   [B, G, nb, di]   int8, nb = ceil(S / block_size)
 *   sel          [B, G, S, top_k] int32
 *   decode: q/out [B, Hq, D], q_idx [B, G, di], k_cache/v_cache [B, G, L, D],
 *           block_keys [B, G, nb, di], sel [B, G, top_k]; the query sits at
 *           position L - 1 and its own key/value are already in the cache.
 *
 * Ownership: every tensor pointer is a device pointer owned by the caller.
 * The library allocates no device memory: scratch space comes from the
 * caller's workspace (size from msa_workspace_bytes), which must be 256-byte
 * aligned.  The library keeps no state between calls, apart from the
 * optional kernel-timing record (msa_profile_enable / msa_profile_read).
 *
 * Streams: each call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t; NULL = the default stream) and returns
 * without synchronising.  Results are valid once the stream has reached
 * them.  Calls that share a workspace must be ordered on one stream.
 *
 * Errors: every entry point returns MSA_OK (0) or a negative status; invalid
 * arguments are rejected before anything is enqueued.  No exception or abort
 * crosses the ABI.
 *
 * Limits: head_dim 128, idx_dim 64, block_size 32, 64 or 128, 1 <= top_k <=
 * 32 (msa_prefill and msa_prefill_lse also take any top_k >= nb; the
 * backward keeps top_k <= 32), n_q_heads = r * n_kv_heads
 * with r in {1, 2, 4, 8, 16}, S < 2^26 and B * G * S * top_k < 2^31; prefill
 * needs nb <= 36864 and decode nb <= 8193.  Anything else returns
 * MSA_ERR_UNSUPPORTED.
 *
 * When top_k >= nb every query keeps all earlier blocks and its own, so
 * msa_prefill computes plain causal GQA attention with a dense kernel (no
 * index branch, no partials, no workspace); one page names short sequences
 * as the case where the selection does not pay and standard attention is
 * used instead (devpress.csdn.net article on MiniMax M3, section "M3的技术局限
 * 与改进方向", first limitation).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1)  /* null pointer, non-positive size, bad ratio */
#define MSA_ERR_UNSUPPORTED (-2)  /* valid but outside the supported limits */
#define MSA_ERR_WORKSPACE (-3)    /* workspace missing, too small or misaligned */
#define MSA_ERR_HIP (-4)          /* a HIP runtime call or launch failed */
#define MSA_ERR_SCRATCH (-5)      /* msa_decode_noalloc: shape needs more than the fixed scratch */

/* Operations, for msa_workspace_bytes. */
#define MSA_OP_POOL 0
#define MSA_OP_INDEX 1
#define MSA_OP_PREFILL 2
#define MSA_OP_DECODE 3
#define MSA_OP_BACKWARD 4
#define MSA_OP_PREFILL_VARLEN 5  /* msa_prefill_varlen: dims.seq_len = the longest sequence */

typedef struct msa_dims {
  int32_t batch;        /* B */
  int32_t seq_len;      /* S for prefill/index/pool, cache length L for decode */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* G, the number of GQA groups (one KV head each) */
  int32_t head_dim;     /* D, must be 128 */
  int32_t idx_dim;      /* di, width of the int8 index vectors, must be 64 */
  int32_t block_size;   /* tokens per KV block: 32, 64 or 128 */
  int32_t top_k;        /* blocks kept per (query, group), own block included */
  float softmax_scale;  /* <= 0 selects 1 / sqrt(head_dim) */
} msa_dims;

/* Human-readable name of a status code (static storage, never NULL). */
const char* msa_status_string(int status);

/* ABI version: major * 10000 + minor * 100 + patch. */
int msa_version(void);

/* Workspace sizes in bytes for `op` at `dims`.
 * *min_bytes: the least workspace the call accepts.  *full_bytes: the size at
 * which the call runs in one pass (MSA_OP_PREFILL processes the (batch,
 * group) units in as few passes as the workspace allows, MSA_OP_BACKWARD
 * the query rows in passes of the largest multiple of 256 rows it holds;
 * every size between the two works).  Either output pointer may be NULL. */
int msa_workspace_bytes(int op, const msa_dims* dims, size_t* min_bytes, size_t* full_bytes);

/* Query rows per pass of msa_prefill_backward with a workspace of ws_bytes
 * (host only, nothing enqueued): *rows = seq_len when the full workspace
 * fits (one pass), else the largest multiple of 256 rows that fits, or 0
 * when ws_bytes is below the minimum (the backward then returns
 * MSA_ERR_WORKSPACE).  The backward runs ceil(seq_len / *rows) passes. */
int msa_backward_pass_rows(const msa_dims* dims, size_t ws_bytes, int32_t* rows);

/* Host-only check of the launch plan of msa_prefill (op MSA_OP_PREFILL) or
 * msa_prefill_backward (op MSA_OP_BACKWARD) at dims with a workspace of
 * ws_bytes; nothing is enqueued and no HIP call is made.  Returns MSA_OK
 * when every query chunk / pass the call would run lays out inside the
 * workspace and its inversion fits the regions reserved for it, with
 * *launches (optional) = the attention launches (prefill: query chunks x
 * unit passes; backward: query passes); MSA_ERR_WORKSPACE when ws_bytes is
 * below the minimum.  The two entry points run this same check before their
 * first launch. */
int msa_plan_check(int op, const msa_dims* dims, size_t ws_bytes, int32_t* launches);

/* Index branch, pooling step: block summary keys.
 * k_idx [B, G, S, di] int8 -> block_keys [B, G, nb, di] int8.
 * Needs no workspace. */
int msa_pool_block_keys(const msa_dims* dims, const int8_t* k_idx, int8_t* block_keys,
                        void* stream);

/* Index branch: pooling, scores and per-(query, group) top-k.
 * q_idx, k_idx [B, G, S, di] int8 -> block_keys [B, G, nb, di] int8 and
 * sel [B, G, S, top_k] int32 (both outputs required).
 * ws/ws_bytes: reserved.  The call uses no workspace
 * (msa_workspace_bytes(MSA_OP_INDEX) reports 0); pass NULL/0.  The
 * arguments stay so that a future version may take scratch without an ABI
 * change; they are not read now. */
int msa_index_select(const msa_dims* dims, const int8_t* q_idx, const int8_t* k_idx,
                     int8_t* block_keys, int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* Whole MSA prefill: index branch, then the main branch over the selected
 * blocks.  q [B, S, Hq, D], k, v [B, G, S, D] bf16; q_idx, k_idx [B, G, S, di]
 * int8 -> out [B, S, Hq, D] bf16 (round to nearest even).  sel [B, G, S,
 * top_k] int32 receives the selection when non-NULL.  The main branch reads
 * each selected key/value block once per batch of the queries that picked
 * it and merges the per-block partial results of a query in log-sum-exp
 * form.  ws/ws_bytes: at least the minimum of msa_workspace_bytes(
 * MSA_OP_PREFILL). */
int msa_prefill(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel, void* ws,
                size_t ws_bytes, void* stream);

/* Ragged batch (varlen) prefill: dims->batch sequences of different lengths
 * packed along the token axis, each an independent MSA prefill (its blocks
 * start at its own first token; it sees only its own keys).  The pages use
 * MSA for prompts of up to 1M tokens served side by side ("深度解析
 * MiniMax-M3：稀疏注意力机制、基准测试与 API 集成指南", section "技术细节"), which
 * real batches of uneven lengths need.
 *
 * cu_seqlens: HOST int32 [batch + 1], cu_seqlens[0] = 0, non-decreasing;
 * sequence s holds tokens cu_seqlens[s] .. cu_seqlens[s + 1] - 1 of the packed
 * tensors (a length of 0 is allowed and skipped), T = cu_seqlens[batch] >= 1.
 * dims->seq_len: the longest sequence (no length may exceed it).
 *   q, out       [T, Hq, D]     bf16
 *   k, v         [G, T, D]      bf16
 *   q_idx, k_idx [G, T, di]     int8
 *   sel          [G, T, top_k]  int32, when non-NULL
 * Row t of sequence s gets exactly what msa_prefill gives row t -
 * cu_seqlens[s] of that sequence on its own.  The sequences run one after
 * another on `stream`, sharing the workspace: ws/ws_bytes at least the
 * minimum of msa_workspace_bytes(MSA_OP_PREFILL_VARLEN, dims) (the sizes of
 * the longest sequence alone).  Every sequence's plan is checked before the
 * first launch; G * T * top_k < 2^31. */
int msa_prefill_varlen(const msa_dims* dims, const int32_t* cu_seqlens, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel,
                       void* ws, size_t ws_bytes, void* stream);

/* Prefill with the short-sequence switch one page describes: below a length
 * the index branch's screening does not pay and standard attention is used
 * instead (devpress.csdn.net article on MiniMax M3, section "M3的技术局限与改进
 * 方向", first limitation).  With seq_len >= dense_below (<= 0 selects 8192,
 * the page's figure) this is msa_prefill, same arguments and results.
 * Below it the call computes STANDARD causal GQA attention -- every key at a
 * position <= t, whatever top_k is -- which differs from MSA's result
 * whenever top_k < nb: the index tensors are not read, sel (when non-NULL,
 * [B, G, S, top_k]) is filled with -1 (no selection was made) and no
 * workspace is used (ws may be NULL).  *took_dense (optional, host) is set
 * to 1 when the standard route ran, else 0. */
int msa_prefill_switched(const msa_dims* dims, int32_t dense_below, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int8_t* q_idx, const int8_t* k_idx, uint16_t* out,
                         int32_t* sel, void* ws, size_t ws_bytes, void* stream, int32_t* took_dense);

/* Whole prefill for training: msa_prefill, plus lse [B, S, Hq] fp32 (required),
 * the natural log-sum-exp of each query row's scaled scores over the keys it
 * attends to, log sum_key exp(softmax_scale * q . k) -- what the backward
 * pass rebuilds the attention weights from.  Same workspace as msa_prefill. */
int msa_prefill_lse(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel, float* lse,
                    void* ws, size_t ws_bytes, void* stream);

/* Backward of the main branch with the selection held fixed (the index
 * branch is integer arithmetic and has no gradient).  The pages report
 * trained MSA models and their training cost (wiki.500nian.com digest of
 * "MiniMax M3 Review", the ablation paragraph; devpress.csdn.net article,
 * section "M3的技术局限与改进方向", third limitation) without a backward
 * formula; this is the chain rule of the forward's single softmax:
 *   P = exp(scale q.k - lse) over the attended keys, dP = dout . v,
 *   dS = P (dP - sum_d dout * out),
 *   dq = scale dS k, dk = scale dS^T q, dv = P^T dout.
 * Inputs: q, out, dout [B, S, Hq, D] bf16; k, v [B, G, S, D] bf16; lse
 * [B, S, Hq] fp32 and sel [B, G, S, top_k] int32 exactly as msa_prefill_lse
 * wrote them (sel must be a valid selection: ascending kept blocks, the own
 * block included, -1 padding).  Outputs dq [B, S, Hq, D], dk, dv [B, G, S, D]
 * bf16, every element written.  top_k <= 32.  ws/ws_bytes: between the
 * minimum and full sizes of msa_workspace_bytes(MSA_OP_BACKWARD).  At the
 * full size the call runs in one pass; the workspace then holds one bf16
 * partial of dq per (query row, kept block), B * Hq * S * top_k * D * 2
 * bytes (8.6 GB at 32K tokens with 64 query heads and top_k 16), and the
 * inversion of sel.  A smaller workspace runs the query rows in passes of
 * the largest multiple of 256 rows it holds, plus fp32 sums of dk and dv
 * over the passes (2 * B * G * S * D * 4 bytes); dq is the same, dk and dv
 * are rounded once from the fp32 sums. */
int msa_prefill_backward(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* out, const uint16_t* dout, const float* lse, const int32_t* sel,
                         uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, size_t ws_bytes, void* stream);

/* Chunked prefill against a cache.  Here dims->seq_len is the capacity C
 * of the caches: k_cache/v_cache [B, G, C, D] bf16 and k_idx [B, G, C, di]
 * int8 already hold the tokens 0 .. start + count - 1 (the caller writes
 * the chunk's rows before the call); block_keys [B, G, ceil(C/block_size),
 * di] int8 holds the summaries of the blocks before start / block_size
 * (from earlier chunks or msa_decode_init) and receives those of the
 * blocks the chunk's tokens fall in.  The count queries at positions
 * start .. start + count - 1, q [B, count, Hq, D] bf16 and q_idx [B, G,
 * count, di] int8, give out [B, count, Hq, D] bf16 and sel [B, G, count,
 * top_k] int32 when non-NULL: the rows msa_prefill gives for those
 * positions of the whole sequence (the pages use MSA for 1M-token prompts,
 * which a chunked prefill bounds in memory: "深度解析 MiniMax-M3：
 * 稀疏注意力机制、基准测试与 API 集成指南", section "技术细节").
 * 0 <= start, 1 <= count, start + count <= C.  ws/ws_bytes: at least the
 * minimum of msa_prefill_chunk_workspace_bytes(dims, count). */
int msa_prefill_chunk_workspace_bytes(const msa_dims* dims, int32_t count, size_t* min_bytes,
                                      size_t* full_bytes);
int msa_prefill_chunk(const msa_dims* dims, int32_t start, int32_t count, const uint16_t* q,
                      const int8_t* q_idx, const uint16_t* k_cache, const uint16_t* v_cache,
                      const int8_t* k_idx, int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws,
                      size_t ws_bytes, void* stream);

/* Ragged chunked prefill: each of the dims->batch sequences adds its own
 * chunk of queries against its own cache, so prompts of uneven lengths that
 * arrive piece by piece share one call (the pages serve prompts of up to 1M
 * tokens side by side: "深度解析 MiniMax-M3：稀疏注意力机制、基准测试与 API 集成指南",
 * section "技术细节").
 *
 * starts, counts: HOST int32 [batch].  Sequence b adds the counts[b] queries
 * at positions starts[b] .. starts[b] + counts[b] - 1 (counts[b] = 0: the
 * sequence is skipped); 0 <= starts[b], starts[b] + counts[b] <= C =
 * dims->seq_len (the caches' capacity), T = sum of counts >= 1.  The caches
 * are laid out as for msa_prefill_chunk, one per sequence: k_cache, v_cache
 * [B, G, C, D] bf16 and k_idx [B, G, C, di] int8 already hold each
 * sequence's tokens 0 .. starts[b] + counts[b] - 1; block_keys [B, G,
 * ceil(C / block_size), di] int8 holds the summaries of its blocks before
 * starts[b] / block_size and receives those of the blocks its new tokens
 * fall in.  The queries are packed along the token axis in sequence order
 * (sequence b's rows start at the sum of the counts before it):
 *   q, out       [T, Hq, D]     bf16
 *   q_idx        [G, T, di]     int8
 *   sel          [G, T, top_k]  int32, when non-NULL
 * Sequence b's rows are exactly what msa_prefill_chunk gives that sequence
 * alone (a batch of one) for the same start and count.  The sequences run
 * one after another on `stream`, sharing the workspace: ws/ws_bytes at least
 * the minimum of msa_prefill_chunk_workspace_bytes for a batch of one and
 * the largest count.  Every sequence's plan is checked before the first
 * launch; G * T * top_k < 2^31. */
int msa_prefill_chunk_varlen(const msa_dims* dims, const int32_t* starts, const int32_t* counts,
                             const uint16_t* q, const int8_t* q_idx, const uint16_t* k_cache,
                             const uint16_t* v_cache, const int8_t* k_idx, int8_t* block_keys, uint16_t* out,
                             int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* One decode step per sequence: the query at position L - 1 of each of the B
 * caches.  q [B, Hq, D] bf16, q_idx [B, G, di] int8, k_cache, v_cache
 * [B, G, L, D] bf16, block_keys [B, G, nb, di] int8 (summaries of the cache's
 * index keys, e.g. from msa_pool_block_keys) -> out [B, Hq, D] bf16; sel
 * [B, G, top_k] int32 when non-NULL.  ws/ws_bytes: at least
 * msa_workspace_bytes(MSA_OP_DECODE). */
int msa_decode(const msa_dims* dims, const uint16_t* q, const int8_t* q_idx,
               const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* block_keys,
               uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* msa_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and kernels as msa_decode; the
 * scratch msa_decode takes from the caller's workspace (the selection when
 * sel is NULL and the per-workgroup softmax states) lives instead in one
 * fixed array of MSA_DECODE_SCRATCH_BYTES per device, compiled into the
 * library and held until the process ends.  The call allocates nothing: no
 * hipMalloc, hipFree or allocating library routine.  Returns
 * MSA_ERR_SCRATCH, before anything is enqueued, when the shape needs more
 * than that (msa_workspace_bytes(MSA_OP_DECODE) tells the need; about 1.1 MB
 * for 16 sequences x 8 groups x 8 heads).  Every call on one device shares
 * its array: calls that overlap in time on one device (other streams or
 * host threads) race and must be ordered by the caller; calls in one stream
 * are ordered.  Each call writes all the scratch it later reads, so nothing
 * carries over from an earlier call. */
#define MSA_DECODE_SCRATCH_BYTES (16u << 20)
int msa_decode_noalloc(const msa_dims* dims, const uint16_t* q, const int8_t* q_idx,
                       const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* block_keys,
                       uint16_t* out, int32_t* sel, void* stream);

/* Generation with caches that grow by one token per step.  The decode
 * pages describe the KV cache holding past keys and values so that each new
 * token attends to them (wiki.500nian.com digest of "MiniMax M3 Review: 1M
 * Tokens, 15X Faster AI Agents", paragraph on the quadratic wall and the KV
 * cache); these two calls keep that cache and its block summaries current.
 *
 * Here dims->seq_len is the capacity C of the caches: k_cache/v_cache
 * [B, G, C, D] bf16, block_keys [B, G, ceil(C / block_size), di] int8 and
 * open_sums [B, G, di] int32, all caller-owned device memory.  open_sums
 * holds the exact integer sum of the index keys already in the block the
 * next token goes to, so that block's summary can be refreshed at every
 * step without re-reading its tokens; the summaries always equal
 * msa_pool_block_keys over the tokens present (a partial last block divides
 * by its own token count).
 *
 * msa_decode_init: for caches that already hold `length` tokens (0 <= length
 * <= C), k_idx [B, G, C, di] int8 their index keys (rows >= length are not
 * read) -> block_keys of blocks 0 .. ceil(length / block_size) - 1 and
 * open_sums (zero when length is a multiple of block_size).  Needs no
 * workspace; length 0 enqueues nothing.
 *
 * msa_decode_step: one token per sequence at position pos = length - 1
 * (1 <= length <= C): k_new, v_new [B, G, D] bf16 go to cache row pos,
 * k_idx_new [B, G, di] int8 updates open_sums (restarted when pos opens a
 * block) and block_keys[pos / block_size]; then the query q [B, Hq, D] /
 * q_idx [B, G, di] at pos is decoded over the `length` cached tokens exactly
 * as msa_decode does for L = length -> out [B, Hq, D], sel [B, G, top_k]
 * when non-NULL.  ws/ws_bytes: at least msa_workspace_bytes(MSA_OP_DECODE)
 * at dims.  A step with length L must follow the state left by init or by
 * the step with length L - 1; the call itself cannot check this. */
int msa_decode_init(const msa_dims* dims, int32_t length, const int8_t* k_idx, int8_t* block_keys,
                    int32_t* open_sums, void* stream);
int msa_decode_step(const msa_dims* dims, int32_t length, const uint16_t* q, const int8_t* q_idx,
                    const uint16_t* k_new, const uint16_t* v_new, const int8_t* k_idx_new,
                    uint16_t* k_cache, uint16_t* v_cache, int32_t* open_sums, int8_t* block_keys,
                    uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes, void* stream);

/* Decode and generation for a ragged batch: sequence b's caches hold its
 * own number of tokens, lengths[b], out of the common capacity C =
 * dims->seq_len (a served batch mixes prompts of any length; the pages
 * decode over resident KV caches up to 1M tokens: wiki.500nian.com digest of
 * "MiniMax M3 Review: 1M Tokens, 15X Faster AI Agents", paragraph on the
 * quadratic wall and the KV cache).  lengths: HOST int32 [batch]; the
 * values are checked on the host and carried to the device in the
 * arguments of a small kernel (no host memory is read after the call
 * returns).  Layouts as for msa_decode_step: k_cache, v_cache [B, G, C, D]
 * bf16, block_keys [B, G, ceil(C / block_size), di] int8, open_sums
 * [B, G, di] int32.
 *
 * msa_decode_varlen: the query of sequence b at position lengths[b] - 1
 * over its first lengths[b] tokens (1 <= lengths[b] <= C); q [B, Hq, D],
 * q_idx [B, G, di] -> out [B, Hq, D], sel [B, G, top_k] when non-NULL.
 * Sequence b's row equals msa_decode on that sequence alone with L =
 * lengths[b].
 * msa_decode_init_varlen: msa_decode_init with each sequence's own length
 * (0 <= lengths[b] <= C; a length of 0 enqueues nothing for it).
 * msa_decode_step_varlen: msa_decode_step with each sequence's own length
 * (1 <= lengths[b] <= C): its new token goes to row lengths[b] - 1, then
 * its query there is decoded.
 * ws/ws_bytes (decode, step): at least msa_workspace_bytes(MSA_OP_DECODE). */
int msa_decode_varlen(const msa_dims* dims, const int32_t* lengths, const uint16_t* q, const int8_t* q_idx,
                      const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* block_keys,
                      uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes, void* stream);
int msa_decode_init_varlen(const msa_dims* dims, const int32_t* lengths, const int8_t* k_idx,
                           int8_t* block_keys, int32_t* open_sums, void* stream);
int msa_decode_step_varlen(const msa_dims* dims, const int32_t* lengths, const uint16_t* q,
                           const int8_t* q_idx, const uint16_t* k_new, const uint16_t* v_new,
                           const int8_t* k_idx_new, uint16_t* k_cache, uint16_t* v_cache,
                           int32_t* open_sums, int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws,
                           size_t ws_bytes, void* stream);

/* The same two calls with the lengths in DEVICE memory (int32 [batch]), read
 * by the kernels when they run: a generation loop captured once in a HIP
 * graph then replays every step, the caller advancing the lengths on the
 * device between replays (host lengths travel in the captured kernel
 * arguments and stay those of the capture).  The values cannot be checked
 * on the host; a sequence whose length lies outside 1 .. C gets a zero
 * output row and sel row -1, and its caches, summaries and open sums are
 * left as they are -- no memory outside the given arrays is touched.  For
 * lengths in range the results are those of msa_decode_varlen and
 * msa_decode_step_varlen.  ws/ws_bytes: at least
 * msa_workspace_bytes(MSA_OP_DECODE). */
int msa_decode_varlen_device(const msa_dims* dims, const int32_t* lengths, const uint16_t* q,
                             const int8_t* q_idx, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes,
                             void* stream);
int msa_decode_step_varlen_device(const msa_dims* dims, const int32_t* lengths, const uint16_t* q,
                                  const int8_t* q_idx, const uint16_t* k_new, const uint16_t* v_new,
                                  const int8_t* k_idx_new, uint16_t* k_cache, uint16_t* v_cache,
                                  int32_t* open_sums, int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws,
                                  size_t ws_bytes, void* stream);

/* Measurement aid, not a step of the attention path: enqueues on `stream`
 * one kernel made only of bf16 matrix-core products
 * (v_mfma_f32_32x32x16_bf16 on register operands, four independent
 * accumulators per wave, no memory traffic in its loop), so that the rate the
 * chip sustains under load can be read beside its published dense peak.
 * n_workgroups (1 .. 2^20) workgroups of 4 waves each run iters (1 .. 2^24)
 * rounds of 4 products; out (device, n_workgroups * 256 floats, caller
 * owned) receives one float per thread (the products' sum, finite).
 * *flop (host; may be NULL) = the FLOP the launch performs.  Returns
 * MSA_ERR_INVALID_ARG for arguments outside those ranges or out == NULL,
 * MSA_ERR_HIP if the launch fails; time it with events on `stream`. */
int msa_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out, double* flop, void* stream);

/* Optional per-kernel timing.  While enabled (on != 0), every kernel the
 * entry points enqueue is bracketed by two HIP events on the same stream and
 * recorded under its kernel name; disabled by default.  Returns MSA_OK, or
 * MSA_ERR_HIP if events cannot be created. */
int msa_profile_enable(int on);

typedef struct msa_kernel_time {
  char name[32];      /* kernel name, e.g. "attend" */
  int32_t launches;   /* launches recorded since the last read */
  float total_ms;     /* summed event-to-event duration of those launches */
} msa_kernel_time;

/* Waits for every recorded launch to finish, writes one aggregate per kernel
 * name into out[0 .. max_entries) (*n_out = number of names), and clears
 * the record.  out may be NULL when max_entries is 0. */
int msa_profile_read(msa_kernel_time* out, int max_entries, int* n_out);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
