// C ABI of the MSA hot path: argument checks, workspace planning and the
// launch sequence of each entry point.  Everything here runs on the host;
// argument checks and workspace sizes touch no HIP API, so they work (and
// are tested) on machines without a GPU.

#include "../../include/msa.h"

#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <string.h>
#include <vector>

#include "msa_kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool pow2_in(int x, int lo, int hi) { return x >= lo && x <= hi && (x & (x - 1)) == 0; }

static_assert(MSA_DECODE_SCRATCH_BYTES == msa::kDecodeScratchBytes, "msa.h and the decode scratch disagree");

constexpr long kMaxSparseTopK = 32;
// msa_prefill_switched runs standard attention below this many tokens when
// the caller passes no threshold (the figure one page gives for where the
// selection stops paying).
constexpr long kDefaultDenseBelow = 8192;  // selection slots of the sparse paths (5 bits in a CSR entry)

struct Dims {
  long B, S, Hq, G, r, D, di, bs, nb, k, kp, U;
  float scale;
};

// Shape checks shared by every entry point.
int check_dims(const msa_dims* d, Dims* o) {
  if (d == nullptr) return MSA_ERR_INVALID_ARG;
  if (d->batch <= 0 || d->seq_len <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 ||
      d->head_dim <= 0 || d->idx_dim <= 0 || d->block_size <= 0 || d->top_k <= 0)
    return MSA_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return MSA_ERR_INVALID_ARG;
  if (!(d->softmax_scale == d->softmax_scale) || isinf(d->softmax_scale)) return MSA_ERR_INVALID_ARG;
  const int r = d->n_q_heads / d->n_kv_heads;
  if (d->head_dim != 128 || d->idx_dim != 64) return MSA_ERR_UNSUPPORTED;
  if (d->block_size != 32 && d->block_size != 64 && d->block_size != 128) return MSA_ERR_UNSUPPORTED;
  // more than 32 kept blocks only where they are all the blocks (a dense
  // prefill); the sparse paths keep at most 32 (checked by each of them)
  if (d->top_k > kMaxSparseTopK && d->top_k < ((long)d->seq_len + d->block_size - 1) / d->block_size)
    return MSA_ERR_UNSUPPORTED;
  if (!pow2_in(r, 1, 16)) return MSA_ERR_UNSUPPORTED;
  if (d->seq_len >= (1 << 26)) return MSA_ERR_UNSUPPORTED;
  const long units = (long)d->batch * d->n_kv_heads;
  if (units * (long)d->seq_len * d->top_k >= (1L << 31)) return MSA_ERR_UNSUPPORTED;
  if (units * (long)d->seq_len * d->n_q_heads / d->n_kv_heads >= (1L << 40)) return MSA_ERR_UNSUPPORTED;
  o->B = d->batch;
  o->S = d->seq_len;
  o->Hq = d->n_q_heads;
  o->G = d->n_kv_heads;
  o->r = r;
  o->D = d->head_dim;
  o->di = d->idx_dim;
  o->bs = d->block_size;
  o->nb = (o->S + o->bs - 1) / o->bs;
  o->k = d->top_k;
  o->kp = d->top_k - 1;
  o->U = units;
  o->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  return MSA_OK;
}

// ---- prefill planning
//
// A long prefill runs in query chunks (prefill_query_chunk); within a chunk
// the main branch runs in passes of as many (batch, group) units as the
// workspace holds partials for (all of them at the full workspace size).
// The CSR rows are (unit, block): one query range per unit.  (The kernels
// also take (unit, range, block) rows, several ranges per unit; that split,
// one unit's range per pass, measured slower on MI355X than query chunks
// over all units, so it is not planned here.)
constexpr long kMaxChunkCounters = 1L << 22;

struct PrefillPlan {
  long T, n_ranges, m, tpc, n_chunks, rows, tokens_per_item, max_items_per_range;
  // histogram chunks of a plan for at most this many queries: the rounding
  // of tpc can give a shorter query range more chunks than a longer one
  // (at 1M tokens, 62 for 253952 queries but 64 for 32768), so regions
  // that serve several ranges are sized by this bound, not by n_chunks
  long max_chunks;
};

PrefillPlan plan_prefill(const Dims& d) {
  PrefillPlan p{};
  p.tokens_per_item = msa::kItemChunks * msa::kItemRows / d.r;
  p.T = (d.S + 255) / 256 * 256;
  p.n_ranges = 1;
  p.rows = d.U * d.nb;
  // token chunks of the inversion's histograms: multiples of 256 tokens, a
  // bounded number of counters
  const long by_tokens = p.T / 256;
  const long by_size = std::max(1L, kMaxChunkCounters / (d.U * d.nb));
  p.m = std::max(1L, std::min(by_tokens, by_size));
  p.max_chunks = p.m;  // n_chunks <= min(by_tokens, by_size), both monotone in S
  p.tpc = (p.T / 256 + p.m - 1) / p.m * 256;
  p.m = (p.T + p.tpc - 1) / p.tpc;
  p.n_chunks = p.m;
  p.max_items_per_range = (d.S * d.k + p.tokens_per_item - 1) / p.tokens_per_item + d.nb;
  return p;
}

struct PrefillLayout {
  size_t block_keys, sel, counts, hist, row_ptr, item_ptr, entries, items, sched, part_o, part_ml, total;
};

// Workspace: fixed part + partials of `units_per_pass` units of pass_tokens.
PrefillLayout prefill_layout(const Dims& d, const PrefillPlan& p, long units_per_pass) {
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  const long pass_tokens = d.S;
  L.block_keys = take((size_t)d.U * d.nb * d.di);
  L.sel = take((size_t)d.U * d.S * d.k * 4);
  L.counts = take((size_t)p.rows * 4);
  L.hist = take((size_t)d.U * p.max_chunks * d.nb * 4);
  L.row_ptr = take((size_t)(p.rows + 1) * 4);
  L.item_ptr = take((size_t)(p.rows + 1) * 4);
  L.entries = take((size_t)d.U * d.S * d.k * 4);
  L.items = take((size_t)(d.U * p.n_ranges * p.max_items_per_range + 1) * 8);
  L.sched = take(4);  // the attention kernel's run counter
  L.part_o = take((size_t)units_per_pass * pass_tokens * d.k * d.r * d.D * 2);
  L.part_ml = take((size_t)units_per_pass * pass_tokens * d.k * d.r * 8);
  L.total = off;
  return L;
}

// A unit's kept blocks are shared by two workgroups (so that the whole chip
// streams the blocks) unless there are fewer than four of them.
int decode_split(const Dims& d) { return d.k >= 4 ? 2 : 1; }

struct DecodeLayout {
  size_t sel, state, lens, total;
};

// Decode workspace: the selection (when the caller passes no sel), the
// workgroups' states (max, sum, unnormalised o per head) and the sequences'
// lengths of a ragged batch.
int decode_layout(const Dims& d, DecodeLayout* L) {
  if (d.nb - 1 > msa::kDecodeMaxCandidates) return MSA_ERR_UNSUPPORTED;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L->sel = take((size_t)d.U * d.k * 4);
  L->state = take((size_t)d.U * decode_split(d) * d.r * (d.D + 2) * 4);
  L->lens = take((size_t)d.B * 4);
  L->total = off;
  return MSA_OK;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MSA_OK;
  if (ws == nullptr || ws_bytes < need) return MSA_ERR_WORKSPACE;
  if (((uintptr_t)ws) % kAlign != 0) return MSA_ERR_WORKSPACE;
  return MSA_OK;
}

// ---- optional kernel timing (msa_profile_enable / msa_profile_read)
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Brackets one launch with events when timing is enabled.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s) : name_(name), s_(s) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!g_prof_on) return;
    a_ = prof_event();
    if (a_ && hipEventRecord(a_, s_) != hipSuccess) a_ = nullptr;
  }
  ~ProfScope() {
    if (!a_) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    hipEvent_t b = prof_event();
    if (b && hipEventRecord(b, s_) == hipSuccess) g_prof_recs.push_back({name_, a_, b});
  }

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};

#define MSA_LAUNCH_NAMED(name, stream, call)       \
  do {                                             \
    ProfScope prof_scope_(name, stream);           \
    if ((call) != hipSuccess) return MSA_ERR_HIP;  \
  } while (0)

int bs_log2_of(long bs) {
  int l = 0;
  while ((1L << l) < bs) ++l;
  return l;
}


msa::DecodeShape decode_shape(const Dims& d, long length) {
  msa::DecodeShape sh;
  sh.B = (int)d.B;
  sh.L = (int)length;
  sh.Hq = (int)d.Hq;
  sh.G = (int)d.G;
  sh.r = (int)d.r;
  sh.bs = (int)d.bs;
  sh.nb = (int)((length + d.bs - 1) / d.bs);
  sh.top_k = (int)d.k;
  sh.Lc = (int)d.S;
  sh.nbc = (int)d.nb;
  sh.scale_log2 = d.scale * 1.4426950408889634f;
  sh.lens = nullptr;
  return sh;
}

// Decode of the query at position length - 1 over caches with room for d.S
// tokens per unit (arguments already checked); with lens (device int32 [B],
// already written) sequence b's query is at lens[b] - 1 and length is the
// largest of them.
int run_decode(const Dims& d, long length, const int32_t* lens, const uint16_t* q, const int8_t* q_idx,
               const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* block_keys, uint16_t* out,
               int32_t* sel, void* ws, size_t ws_bytes, hipStream_t s) {
  DecodeLayout L;
  int st = decode_layout(d, &L);
  if (st != MSA_OK) return st;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MSA_OK) return st;
  char* base = static_cast<char*>(ws);
  msa::DecodeShape sh = decode_shape(d, length);
  sh.lens = lens;
  int32_t* sel_use = sel ? sel : reinterpret_cast<int32_t*>(base + L.sel);
  float* state = reinterpret_cast<float*>(base + L.state);
  const int n_split = decode_split(d);
  MSA_LAUNCH_NAMED("decode", s,
                   msa::launch_decode(sh, q, q_idx, k_cache, v_cache, block_keys, sel_use, out, state, n_split, s));
  if (n_split > 1) MSA_LAUNCH_NAMED("decode_merge", s, msa::launch_decode_merge(sh, state, n_split, out, s));
  return MSA_OK;
}

// Dims of the query side of a prefill: n_q query rows per unit; nb stays
// the block count of dc (all CSR rows a query of the sequence can reach).
Dims chunk_dims(const Dims& dc, long n_q) {
  Dims d = dc;
  d.S = n_q;
  return d;
}

// Dims of one sequence of length L of a ragged batch (dims.batch sequences,
// dims.seq_len the longest): a batch of one.
Dims seq_dims(const Dims& d, long L) {
  Dims o = d;
  o.B = 1;
  o.S = L;
  o.nb = (L + d.bs - 1) / d.bs;
  o.U = d.G;
  return o;
}

// The sequence lengths of a ragged batch from host cu_seqlens [n + 1]:
// cu_seqlens[0] = 0, non-decreasing, no length above dims.seq_len, at least
// one token in all; *total = cu_seqlens[n].
int check_cu_seqlens(const Dims& d, const int32_t* cu, long* total) {
  if (cu == nullptr || cu[0] != 0) return MSA_ERR_INVALID_ARG;
  for (long s = 0; s < d.B; ++s) {
    const long L = (long)cu[s + 1] - cu[s];
    if (L < 0 || L > d.S) return MSA_ERR_INVALID_ARG;
  }
  *total = cu[d.B];
  if (*total < 1) return MSA_ERR_INVALID_ARG;
  // row offsets of the packed tensors stay within int32 arithmetic of the
  // kernels' per-unit strides
  if ((long)d.G * *total * d.k >= (1L << 31) || *total >= (1L << 30)) return MSA_ERR_UNSUPPORTED;
  return MSA_OK;
}

// A long prefill runs in query chunks.  Up to 128K tokens a chunk holds
// 16384 queries: its partials (about 280 MB for 64 query heads and top_k 16)
// then mostly stay in the 256 MB memory-side cache until the merge reads
// them (measured on MI355X: 3 % faster at 32K and 6 % at 128K than one
// pass, and at 128K faster than 32K or 64K chunks).  Every chunk reads the
// K/V blocks its queries kept once, so when the blocks far outnumber a
// chunk's queries (a 16K chunk of a 1M-token prefill keeps each block for
// about 32 tokens) that re-reading dominates; beyond 128K tokens a chunk is
// a quarter of the sequence (1M tokens: 251 ms against 328 ms with 16K
// chunks, 260 ms with 128K and 257 ms with 512K).
constexpr long kPrefillQueryChunk = 16384;
constexpr long kShortPrefill = 131072;

long prefill_query_chunk(const Dims& d) {
  if (d.S <= kPrefillQueryChunk) return d.S;
  if (d.S <= kShortPrefill) return kPrefillQueryChunk;
  const long quarter = (d.S + 3) / 4;
  return (quarter + kPrefillQueryChunk - 1) / kPrefillQueryChunk * kPrefillQueryChunk;
}

// Row strides of the tensors a prefill reads and writes, in rows of D (or
// di, or top_k) elements: q, out and lse per batch entry; k, v and k_idx per
// (batch, group) unit; q_idx and sel per unit.  A whole prefill of [B, S]
// tensors has S everywhere; a chunk against a cache of capacity C has C for
// the caches; a packed ragged batch has the total token count for k, v and
// the index tensors.
struct Strides {
  long q_rows, kv_rows, qi_rows, sel_rows;
};

Strides dense_strides(const Dims& d) { return Strides{d.S, d.S, d.S, d.S}; }

// The plan of one query chunk (n_q rows of a prefill of dc) in a workspace
// of ws_bytes: the inversion's plan, the workspace layout and the (batch,
// group) units per pass -- as many as the workspace holds partials for.
// Checks what the kernels rely on: every region inside the workspace, the
// histogram chunks within their region, the persistent summaries at offset
// 0 (query chunks of one prefill share them).
struct ChunkRun {
  PrefillPlan P;
  PrefillLayout L;
  long upp;
};

int plan_chunk(const Dims& dc, long n_q, size_t ws_bytes, ChunkRun* run) {
  const Dims d = chunk_dims(dc, n_q);
  run->P = plan_prefill(d);
  const PrefillPlan& P = run->P;
  const PrefillLayout one = prefill_layout(d, P, 1);
  if (ws_bytes < one.total) return MSA_ERR_WORKSPACE;
  const size_t per_unit = prefill_layout(d, P, 2).total - one.total;
  long upp = per_unit > 0 ? std::min<long>(d.U, 1 + (long)((ws_bytes - one.total) / per_unit)) : d.U;
  PrefillLayout L = prefill_layout(d, P, upp);
  while (L.total > ws_bytes && upp > 1) L = prefill_layout(d, P, --upp);
  if (L.total > ws_bytes || upp < 1) return MSA_ERR_WORKSPACE;
  if (L.block_keys != 0 || P.n_chunks > P.max_chunks || P.m * P.tpc < P.T || P.T < n_q) return MSA_ERR_WORKSPACE;
  run->L = L;
  run->upp = upp;
  return MSA_OK;
}

// Prefill of the queries at positions q0 .. q0 + n_q - 1 of sequences whose
// keys, values and index keys are rows 0 .. q0 + n_q - 1 of k, v and k_idx
// (q0 = 0 and n_q = dc.S for a whole prefill); q, q_idx, out, sel (when
// given) and lse (when given) hold the n_q query rows.  ext_keys: block
// summaries that persist across calls (dc.nb rows per unit; blocks before
// q0 / bs already pooled), or null to pool every block into the workspace.
int run_prefill(const Dims& dc, long q0, long n_q, const Strides& str, const uint16_t* q, const uint16_t* k,
                const uint16_t* v, const int8_t* q_idx, const int8_t* k_idx, int8_t* ext_keys, uint16_t* out,
                int32_t* sel, float* lse, void* ws, size_t ws_bytes, hipStream_t s) {
  const Dims d = chunk_dims(dc, n_q);
  int st = check_ws(ws, ws_bytes, 1);
  if (st != MSA_OK) return st;
  ChunkRun run;
  st = plan_chunk(dc, n_q, ws_bytes, &run);
  if (st != MSA_OK) return st;
  const PrefillPlan& P = run.P;
  const PrefillLayout& L = run.L;
  const long upp = run.upp;

  char* base = static_cast<char*>(ws);
  int8_t* bkeys = reinterpret_cast<int8_t*>(base + L.block_keys);
  int32_t* sel_use = sel ? sel : reinterpret_cast<int32_t*>(base + L.sel);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  int32_t* row_ptr = reinterpret_cast<int32_t*>(base + L.row_ptr);
  int32_t* item_ptr = reinterpret_cast<int32_t*>(base + L.item_ptr);
  uint32_t* entries = reinterpret_cast<uint32_t*>(base + L.entries);
  int2* items = reinterpret_cast<int2*>(base + L.items);
  int* sched = reinterpret_cast<int*>(base + L.sched);
  uint16_t* part_o = reinterpret_cast<uint16_t*>(base + L.part_o);
  float2* part_ml = reinterpret_cast<float2*>(base + L.part_ml);

  const int U = (int)d.U, S = (int)d.S, bs = (int)d.bs, nb = (int)d.nb, K = (int)d.k;
  msa::ChunkPlan cp;
  cp.T = (int)P.T;
  cp.m = (int)P.m;
  cp.tpc = (int)P.tpc;
  cp.n_chunks = (int)P.n_chunks;
  cp.n_ranges = (int)P.n_ranges;
  const int sel_stride = sel ? (int)str.sel_rows : S;  // the workspace's sel holds the n_q rows only
  cp.q_stride = sel_stride;
  const int tpi = (int)P.tokens_per_item;
  const int iq0 = (int)q0;
  if (ext_keys != nullptr) {
    // the blocks the new tokens fall in; earlier ones are the caller's
    bkeys = ext_keys;
    MSA_LAUNCH_NAMED("pool", s, msa::launch_pool_strided(k_idx, bkeys, nullptr, U, (int)(q0 + n_q), str.kv_rows,
                                                         nb, bs, (int)(q0 / bs), s));
  } else {
    MSA_LAUNCH_NAMED("pool", s, msa::launch_pool_strided(k_idx, bkeys, nullptr, U, S, str.kv_rows, nb, bs, 0, s));
  }
  MSA_LAUNCH_NAMED("index_topk", s, msa::launch_index_topk_at(q_idx, bkeys, sel_use, U, S, iq0, (int)str.qi_rows,
                                                               sel_stride, nb, bs, K, s));
  MSA_LAUNCH_NAMED("chunk_hist", s, msa::launch_chunk_hist(sel_use, hist, U, S, nb, bs, K, cp, iq0, false, s));
  MSA_LAUNCH_NAMED("chunk_total", s, msa::launch_chunk_total(hist, counts, U, nb, cp, s));
  MSA_LAUNCH_NAMED("scan", s, msa::launch_scan(counts, row_ptr, item_ptr, (int)P.rows, tpi, s));
  MSA_LAUNCH_NAMED("offsets_items", s, msa::launch_offsets_items(hist, row_ptr, item_ptr, items, U, nb, cp, tpi, s));
  MSA_LAUNCH_NAMED("scatter", s, msa::launch_scatter(sel_use, hist, entries, U, S, nb, bs, K, cp, iq0, false, s));
  msa::PrefillShape sh;
  sh.B = (int)d.B;
  sh.S = S;
  sh.Hq = (int)d.Hq;
  sh.G = (int)d.G;
  sh.r = (int)d.r;
  sh.bs = bs;
  sh.bs_log2 = bs_log2_of(bs);
  sh.nb = nb;
  sh.top_k = K;
  sh.n_ranges = (int)P.n_ranges;
  sh.range_tokens = (int)P.T;
  sh.scale_log2 = d.scale * 1.4426950408889634f;
  sh.q0 = iq0;
  sh.q_stride = (int)str.q_rows;
  sh.kv_rows = (int)str.kv_rows;
  sh.lse = lse;
  auto run_pass = [&](long u0, long u1) -> int {
    msa::PassInfo ps;
    ps.u0 = (int)u0;
    ps.u1 = (int)u1;
    ps.rng = 0;
    ps.t0 = 0;
    ps.t1 = S;
    ps.pass_tokens = S;
    ps.row_begin = (int)(u0 * nb);
    ps.row_end = (int)(u1 * nb);
    const long max_items = (u1 - u0) * P.max_items_per_range;
    MSA_LAUNCH_NAMED("attend", s, msa::launch_attend(sh, ps, q, k, v, row_ptr, item_ptr, items, entries, part_o,
                                                     part_ml, sched, (int)max_items, s));
    MSA_LAUNCH_NAMED("merge", s, msa::launch_merge(sh, ps, q, k, v, part_o, part_ml, out, s));
    return MSA_OK;
  };
  for (long u0 = 0; u0 < d.U; u0 += upp) {
    st = run_pass(u0, std::min<long>(d.U, u0 + upp));
    if (st != MSA_OK) return st;
  }
  return MSA_OK;
}


// Backward workspace: delta of every row, the inversion of sel for the
// query rows of one pass (as in a prefill), one bf16 dq partial per (query
// row of the pass, selection slot), and -- when the pass holds fewer rows
// than the sequence -- fp32 sums of dK and dV over the passes.
struct BackwardLayout {
  size_t delta, counts, hist, row_ptr, item_ptr, entries, items, part_dq, acc_k, acc_v, total;
  long max_chunks, max_items;  // the inversion regions' capacity, per unit
};

constexpr long kBackwardPassGranule = 256;  // query rows of a pass: the whole sequence or a multiple of this

BackwardLayout backward_layout(const Dims& d, long pass_rows) {
  const Dims dc = chunk_dims(d, pass_rows);
  const PrefillPlan p = plan_prefill(dc);
  const bool passes = pass_rows < d.S;
  BackwardLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  };
  L.delta = take((size_t)d.B * d.S * d.Hq * 4);
  L.counts = take((size_t)p.rows * 4);
  L.hist = take((size_t)d.U * p.max_chunks * d.nb * 4);  // every pass, the last and shortest too
  L.row_ptr = take((size_t)(p.rows + 1) * 4);
  L.item_ptr = take((size_t)(p.rows + 1) * 4);
  L.entries = take((size_t)d.U * pass_rows * d.k * 4);
  L.items = take((size_t)(d.U * p.n_ranges * p.max_items_per_range + 1) * 8);
  L.part_dq = take((size_t)d.U * pass_rows * d.k * d.r * d.D * 2);
  L.acc_k = take(passes ? (size_t)d.U * d.S * d.D * 4 : 0);
  L.acc_v = take(passes ? (size_t)d.U * d.S * d.D * 4 : 0);
  L.total = off;
  L.max_chunks = p.max_chunks;
  L.max_items = p.max_items_per_range;
  return L;
}

// Query rows per backward pass for a workspace of ws_bytes: the whole
// sequence when the workspace holds it, else the largest multiple of the
// granule that fits (0: not even one granule fits).
long backward_pass_rows(const Dims& d, size_t ws_bytes) {
  if (backward_layout(d, d.S).total <= ws_bytes) return d.S;
  long lo = 0, hi = (d.S - 1) / kBackwardPassGranule;  // granules: hi * granule < S
  while (lo < hi) {
    const long mid = (lo + hi + 1) / 2;
    if (backward_layout(d, mid * kBackwardPassGranule).total <= ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  return lo * kBackwardPassGranule;
}

// Plans of every query chunk of a whole sparse prefill in ws_bytes;
// *launches (optional) = the attention launches (chunks x unit passes).
int check_prefill_plans(const Dims& d, size_t ws_bytes, long* launches) {
  const long T = prefill_query_chunk(d);
  long n = 0;
  for (long q0 = 0; q0 < d.S; q0 += T) {
    ChunkRun run;
    const int st = plan_chunk(d, std::min(T, d.S - q0), ws_bytes, &run);
    if (st != MSA_OK) return st;
    n += (d.U + run.upp - 1) / run.upp;
  }
  if (launches) *launches = n;
  return MSA_OK;
}

// Plans of every query pass of a backward with passes of T rows against the
// layout sized for T rows: the histogram chunks and work items of each pass
// within their regions (a shorter last pass can plan more histogram chunks
// than a full one: its chunk length rounds to whole 256-token granules).
int check_backward_plans(const Dims& d, long T, const BackwardLayout& L) {
  if (T < 1 || T > d.S) return MSA_ERR_WORKSPACE;
  for (long q0 = 0; q0 < d.S; q0 += T) {
    const long n_q = std::min(T, d.S - q0);
    const PrefillPlan P = plan_prefill(chunk_dims(d, n_q));
    if (P.n_chunks > L.max_chunks || P.max_items_per_range > L.max_items || P.m * P.tpc < P.T || P.T < n_q)
      return MSA_ERR_WORKSPACE;
  }
  return MSA_OK;
}

// Plain causal GQA attention of every query of d (the dense kernel), and,
// when sel is given, the selection that keeps every block up to the own one.
int dense_impl(const Dims& d, const Strides& str, const uint16_t* q, const uint16_t* k, const uint16_t* v,
               uint16_t* out, int32_t* sel, float* lse, hipStream_t s) {
  msa::PrefillShape sh{};
  sh.B = (int)d.B;
  sh.S = (int)d.S;
  sh.Hq = (int)d.Hq;
  sh.G = (int)d.G;
  sh.r = (int)d.r;
  sh.bs = (int)d.bs;
  sh.bs_log2 = bs_log2_of(d.bs);
  sh.nb = (int)d.nb;
  sh.top_k = (int)d.k;
  sh.q0 = 0;
  sh.q_stride = (int)str.q_rows;
  sh.kv_rows = (int)str.kv_rows;
  sh.scale_log2 = d.scale * 1.4426950408889634f;
  sh.lse = lse;
  MSA_LAUNCH_NAMED("dense", s, msa::launch_dense(sh, q, k, v, out, sel, (int)str.sel_rows, s));
  return MSA_OK;
}

// Whole prefill (msa_prefill, msa_prefill_lse, each sequence of
// msa_prefill_varlen), arguments checked and every plan checked.
int prefill_impl(const Dims& d, const Strides& str, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                 const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel, float* lse, void* ws,
                 size_t ws_bytes, hipStream_t s) {
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  if (d.k >= d.nb) {
    // top_k covers every block: each query keeps all earlier blocks and its
    // own, which is plain causal attention (no index branch, no partials)
    return dense_impl(d, str, q, k, v, out, sel, lse, s);
  }
  const long T = prefill_query_chunk(d);
  // every chunk is planned and checked before anything is enqueued
  int st = check_prefill_plans(d, ws_bytes, nullptr);
  if (st != MSA_OK) return st;
  if (T >= d.S) return run_prefill(d, 0, d.S, str, q, k, v, q_idx, k_idx, nullptr, out, sel, lse, ws, ws_bytes, s);
  // query chunks of T tokens; the summaries persist in the workspace's first
  // region (block_keys, which every layout places at offset 0)
  int8_t* keys = static_cast<int8_t*>(ws);
  for (long q0 = 0; q0 < d.S; q0 += T) {
    const long n = std::min(T, d.S - q0);
    const int st2 = run_prefill(d, q0, n, str, q + q0 * d.Hq * d.D, k, v, q_idx + q0 * d.di, k_idx, keys,
                                out + q0 * d.Hq * d.D, sel ? sel + q0 * d.k : nullptr,
                                lse ? lse + q0 * d.Hq : nullptr, ws, ws_bytes, s);
    if (st2 != MSA_OK) return st2;
  }
  return MSA_OK;
}

// Host lengths of a ragged decode batch: every one in lo .. d.S (the
// capacity); *longest = the largest (0 when all are 0).
int check_lengths(const Dims& d, const int32_t* lengths, long lo, long* longest) {
  if (lengths == nullptr) return MSA_ERR_INVALID_ARG;
  long m = 0;
  for (long b = 0; b < d.B; ++b) {
    if (lengths[b] < lo || lengths[b] > d.S) return MSA_ERR_INVALID_ARG;
    m = std::max<long>(m, lengths[b]);
  }
  *longest = m;
  return MSA_OK;
}

}  // namespace

extern "C" {

const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK:
      return "MSA_OK";
    case MSA_ERR_INVALID_ARG:
      return "MSA_ERR_INVALID_ARG: null pointer, non-positive size or inconsistent shape";
    case MSA_ERR_UNSUPPORTED:
      return "MSA_ERR_UNSUPPORTED: shape outside the supported limits";
    case MSA_ERR_WORKSPACE:
      return "MSA_ERR_WORKSPACE: workspace missing, too small or not 256-byte aligned";
    case MSA_ERR_HIP:
      return "MSA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case MSA_ERR_SCRATCH:
      return "MSA_ERR_SCRATCH: the shape needs more than the library's fixed decode scratch (msa_decode_noalloc)";
    default:
      return "unknown MSA status";
  }
}

int msa_version(void) { return 10900; }

int msa_backward_pass_rows(const msa_dims* dims, size_t ws_bytes, int32_t* rows) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK || d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  if (!rows) return MSA_ERR_INVALID_ARG;
  *rows = (int32_t)backward_pass_rows(d, ws_bytes);
  return MSA_OK;
}

int msa_plan_check(int op, const msa_dims* dims, size_t ws_bytes, int32_t* launches) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  long n = 0;
  if (op == MSA_OP_PREFILL) {
    if (d.k >= d.nb) {
      n = 1;  // the dense kernel: no workspace, nothing to plan
    } else {
      st = check_prefill_plans(d, ws_bytes, &n);
      if (st != MSA_OK) return st;
    }
  } else if (op == MSA_OP_BACKWARD) {
    if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
    const long T = backward_pass_rows(d, ws_bytes);
    if (T == 0) return MSA_ERR_WORKSPACE;
    const BackwardLayout L = backward_layout(d, T);
    if (L.total > ws_bytes) return MSA_ERR_WORKSPACE;
    st = check_backward_plans(d, T, L);
    if (st != MSA_OK) return st;
    n = (d.S + T - 1) / T;
  } else {
    return MSA_ERR_INVALID_ARG;
  }
  if (launches) *launches = (int32_t)n;
  return MSA_OK;
}

int msa_workspace_bytes(int op, const msa_dims* dims, size_t* min_bytes, size_t* full_bytes) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  size_t lo = 0, hi = 0;
  switch (op) {
    case MSA_OP_POOL:
      break;
    case MSA_OP_INDEX:
      if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
      break;
    case MSA_OP_PREFILL: {
      if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
      if (d.k >= d.nb) break;  // dense causal attention needs no workspace
      const Dims dq = chunk_dims(d, std::min(d.S, prefill_query_chunk(d)));
      const PrefillPlan p = plan_prefill(dq);
      lo = prefill_layout(dq, p, 1).total;
      hi = prefill_layout(dq, p, dq.U).total;
      break;
    }
    case MSA_OP_PREFILL_VARLEN: {
      // one sequence at a time, the longest (dims.seq_len) sizing the
      // workspace; a shorter one plans within it
      if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
      const Dims d1 = seq_dims(d, d.S);
      if (d1.k >= d1.nb) break;
      const Dims dq = chunk_dims(d1, std::min(d1.S, prefill_query_chunk(d1)));
      const PrefillPlan p = plan_prefill(dq);
      lo = prefill_layout(dq, p, 1).total;
      hi = prefill_layout(dq, p, dq.U).total;
      break;
    }
    case MSA_OP_BACKWARD: {
      if (d.k > kMaxSparseTopK || d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
      hi = backward_layout(d, d.S).total;
      lo = d.S > kBackwardPassGranule ? std::min(hi, backward_layout(d, kBackwardPassGranule).total) : hi;
      break;
    }
    case MSA_OP_DECODE: {
      if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
      DecodeLayout L;
      st = decode_layout(d, &L);
      if (st != MSA_OK) return st;
      lo = hi = L.total;
      break;
    }
    default:
      return MSA_ERR_INVALID_ARG;
  }
  if (min_bytes) *min_bytes = lo;
  if (full_bytes) *full_bytes = hi;
  return MSA_OK;
}

int msa_pool_block_keys(const msa_dims* dims, const int8_t* k_idx, int8_t* block_keys, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (k_idx == nullptr || block_keys == nullptr) return MSA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  MSA_LAUNCH_NAMED("pool", s, msa::launch_pool(k_idx, block_keys, (int)d.U, (int)d.S, (int)d.bs, s));
  return MSA_OK;
}

int msa_index_select(const msa_dims* dims, const int8_t* q_idx, const int8_t* k_idx, int8_t* block_keys,
                     int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;  // reserved (msa.h): the index branch needs no workspace
  (void)ws_bytes;
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (q_idx == nullptr || k_idx == nullptr || block_keys == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  MSA_LAUNCH_NAMED("pool", s, msa::launch_pool(k_idx, block_keys, (int)d.U, (int)d.S, (int)d.bs, s));
  MSA_LAUNCH_NAMED("index_topk", s, msa::launch_index_topk(q_idx, block_keys, sel, (int)d.U, (int)d.S, (int)d.bs, (int)d.k, s));
  return MSA_OK;
}

int msa_prefill(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel, void* ws,
                size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !out) return MSA_ERR_INVALID_ARG;
  return prefill_impl(d, dense_strides(d), q, k, v, q_idx, k_idx, out, sel, nullptr, ws, ws_bytes,
                      (hipStream_t)stream);
}

int msa_prefill_varlen(const msa_dims* dims, const int32_t* cu_seqlens, const uint16_t* q, const uint16_t* k,
                       const uint16_t* v, const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel,
                       void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !out) return MSA_ERR_INVALID_ARG;
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  long T = 0;
  st = check_cu_seqlens(d, cu_seqlens, &T);
  if (st != MSA_OK) return st;
  // every sequence's plan is checked before the first launch
  bool sparse = false;
  for (long b = 0; b < d.B; ++b) {
    const long L = (long)cu_seqlens[b + 1] - cu_seqlens[b];
    if (L == 0) continue;
    const Dims ds = seq_dims(d, L);
    if (ds.k >= ds.nb) continue;
    sparse = true;
    st = check_prefill_plans(ds, ws_bytes, nullptr);
    if (st != MSA_OK) return st;
  }
  if (sparse && (ws == nullptr || ((uintptr_t)ws) % kAlign != 0)) return MSA_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  for (long b = 0; b < d.B; ++b) {
    const long o = cu_seqlens[b], L = (long)cu_seqlens[b + 1] - o;
    if (L == 0) continue;
    const Dims ds = seq_dims(d, L);
    st = prefill_impl(ds, Strides{L, T, T, T}, q + o * d.Hq * d.D, k + o * d.D, v + o * d.D, q_idx + o * d.di,
                      k_idx + o * d.di, out + o * d.Hq * d.D, sel ? sel + o * d.k : nullptr, nullptr, ws, ws_bytes,
                      s);
    if (st != MSA_OK) return st;
  }
  return MSA_OK;
}

int msa_prefill_switched(const msa_dims* dims, int32_t dense_below, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel,
                         void* ws, size_t ws_bytes, void* stream, int32_t* took_dense) {
  if (dims == nullptr) return MSA_ERR_INVALID_ARG;
  const long below = dense_below > 0 ? dense_below : kDefaultDenseBelow;
  if (dims->seq_len >= below) {
    Dims d;
    int st = check_dims(dims, &d);
    if (st != MSA_OK) return st;
    if (!q || !k || !v || !q_idx || !k_idx || !out) return MSA_ERR_INVALID_ARG;
    if (took_dense) *took_dense = 0;
    return prefill_impl(d, dense_strides(d), q, k, v, q_idx, k_idx, out, sel, nullptr, ws, ws_bytes,
                        (hipStream_t)stream);
  }
  // standard causal GQA attention: the index branch is skipped, so top_k
  // plays no part beyond the layout of sel (checked as if it kept every
  // block)
  msa_dims dd = *dims;
  if (dd.block_size > 0 && dd.seq_len > 0)
    dd.top_k = std::max<int32_t>(dd.top_k, (int32_t)((dd.seq_len + (long)dd.block_size - 1) / dd.block_size));
  Dims d;
  int st = check_dims(&dd, &d);
  if (st != MSA_OK) return st;
  if (dims->top_k <= 0) return MSA_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return MSA_ERR_INVALID_ARG;
  if (took_dense) *took_dense = 1;
  hipStream_t s = (hipStream_t)stream;
  st = dense_impl(d, dense_strides(d), q, k, v, out, nullptr, nullptr, s);
  if (st != MSA_OK) return st;
  if (sel != nullptr)
    MSA_LAUNCH_NAMED("fill", s, msa::launch_fill_i32(sel, -1, (size_t)d.B * d.G * d.S * dims->top_k, s));
  return MSA_OK;
}

int msa_prefill_lse(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                    const int8_t* q_idx, const int8_t* k_idx, uint16_t* out, int32_t* sel, float* lse, void* ws,
                    size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !q_idx || !k_idx || !out || !lse) return MSA_ERR_INVALID_ARG;
  return prefill_impl(d, dense_strides(d), q, k, v, q_idx, k_idx, out, sel, lse, ws, ws_bytes,
                      (hipStream_t)stream);
}

int msa_prefill_backward(const msa_dims* dims, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* out, const uint16_t* dout, const float* lse, const int32_t* sel,
                         uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !out || !dout || !lse || !sel || !dq || !dk || !dv) return MSA_ERR_INVALID_ARG;
  if (ws == nullptr || ((uintptr_t)ws) % kAlign != 0) return MSA_ERR_WORKSPACE;
  const long T = backward_pass_rows(d, ws_bytes);
  if (T == 0) return MSA_ERR_WORKSPACE;
  const BackwardLayout L = backward_layout(d, T);
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MSA_OK) return st;
  // every pass's inversion must fit the regions sized for T rows (it does,
  // by the bounds in backward_layout); checked for all passes before the
  // first launch, so that a planning mistake is an error, not a write past
  // a region
  st = check_backward_plans(d, T, L);
  if (st != MSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* base = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(base + L.delta);
  int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  int32_t* row_ptr = reinterpret_cast<int32_t*>(base + L.row_ptr);
  int32_t* item_ptr = reinterpret_cast<int32_t*>(base + L.item_ptr);
  uint32_t* entries = reinterpret_cast<uint32_t*>(base + L.entries);
  int2* items = reinterpret_cast<int2*>(base + L.items);
  uint16_t* part_dq = reinterpret_cast<uint16_t*>(base + L.part_dq);
  const bool passes = T < d.S;
  const int U = (int)d.U, S = (int)d.S, bs = (int)d.bs, nb = (int)d.nb, K = (int)d.k;
  msa::BwdShape sh;
  sh.B = (int)d.B;
  sh.S = S;
  sh.Hq = (int)d.Hq;
  sh.G = (int)d.G;
  sh.r = (int)d.r;
  sh.r_log2 = bs_log2_of(d.r);
  sh.bs = bs;
  sh.bs_log2 = bs_log2_of(bs);
  sh.nb = nb;
  sh.top_k = K;
  sh.U = U;
  sh.scale = d.scale;
  sh.scale_log2 = d.scale * 1.4426950408889634f;
  sh.acc_k = passes ? reinterpret_cast<float*>(base + L.acc_k) : nullptr;
  sh.acc_v = passes ? reinterpret_cast<float*>(base + L.acc_v) : nullptr;
  MSA_LAUNCH_NAMED("bwd_delta", s, msa::launch_bwd_delta(out, dout, delta, d.B * d.S * d.Hq, s));
  if (passes) {
    // fp32 zeros: a fill kernel (no memset node, so the call can be captured)
    const size_t n = (size_t)U * S * d.D;
    MSA_LAUNCH_NAMED("fill", s, msa::launch_fill_i32(reinterpret_cast<int32_t*>(sh.acc_k), 0, n, s));
    MSA_LAUNCH_NAMED("fill", s, msa::launch_fill_i32(reinterpret_cast<int32_t*>(sh.acc_v), 0, n, s));
  }
  // passes of T query rows: the rows' selections inverted into CSR rows
  // (unit, block), then dK / dV of every kept block and the rows' dq
  for (long q0 = 0; q0 < S; q0 += T) {
    const long n_q = std::min(T, (long)S - q0);
    const Dims dc = chunk_dims(d, n_q);
    const PrefillPlan P = plan_prefill(dc);
    msa::ChunkPlan cp;
    cp.T = (int)P.T;
    cp.m = (int)P.m;
    cp.tpc = (int)P.tpc;
    cp.n_chunks = (int)P.n_chunks;
    cp.n_ranges = (int)P.n_ranges;
    cp.q_stride = S;  // sel rows per unit
    const int tpi = (int)P.tokens_per_item;
    const int32_t* psel = sel + q0 * K;
    const int iq0 = (int)q0, in_q = (int)n_q;
    MSA_LAUNCH_NAMED("chunk_hist", s, msa::launch_chunk_hist(psel, hist, U, in_q, nb, bs, K, cp, iq0, true, s));
    MSA_LAUNCH_NAMED("chunk_total", s, msa::launch_chunk_total(hist, counts, U, nb, cp, s));
    MSA_LAUNCH_NAMED("scan", s, msa::launch_scan(counts, row_ptr, item_ptr, (int)P.rows, tpi, s));
    MSA_LAUNCH_NAMED("offsets_items", s,
                     msa::launch_offsets_items(hist, row_ptr, item_ptr, items, U, nb, cp, tpi, s));
    MSA_LAUNCH_NAMED("scatter", s, msa::launch_scatter(psel, hist, entries, U, in_q, nb, bs, K, cp, iq0, true, s));
    sh.q0 = iq0;
    sh.n_q = in_q;
    MSA_LAUNCH_NAMED("bwd_kv", s,
                     msa::launch_bwd_kv(sh, q, k, v, dout, lse, delta, row_ptr, entries, dk, dv, part_dq, s));
    MSA_LAUNCH_NAMED("bwd_dq", s, msa::launch_bwd_dq(sh, part_dq, dq, s));
  }
  if (passes) MSA_LAUNCH_NAMED("bwd_acc", s, msa::launch_bwd_acc(sh, dk, dv, s));
  return MSA_OK;
}


int msa_prefill_chunk_workspace_bytes(const msa_dims* dims, int32_t count, size_t* min_bytes, size_t* full_bytes) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (count < 1 || count > d.S) return MSA_ERR_INVALID_ARG;
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  const Dims dq = chunk_dims(d, count);
  const PrefillPlan p = plan_prefill(dq);
  const size_t lo = prefill_layout(dq, p, 1).total;
  const size_t hi = prefill_layout(dq, p, dq.U).total;
  if (min_bytes) *min_bytes = lo;
  if (full_bytes) *full_bytes = hi;
  return MSA_OK;
}

int msa_prefill_chunk(const msa_dims* dims, int32_t start, int32_t count, const uint16_t* q, const int8_t* q_idx,
                      const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* k_idx, int8_t* block_keys,
                      uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!q || !q_idx || !k_cache || !v_cache || !k_idx || !block_keys || !out) return MSA_ERR_INVALID_ARG;
  if (start < 0 || count < 1 || (long)start + count > d.S) return MSA_ERR_INVALID_ARG;
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  return run_prefill(d, start, count, Strides{count, d.S, count, count}, q, k_cache, v_cache, q_idx, k_idx,
                     block_keys, out, sel, nullptr, ws, ws_bytes, (hipStream_t)stream);
}

int msa_prefill_chunk_varlen(const msa_dims* dims, const int32_t* starts, const int32_t* counts, const uint16_t* q,
                             const int8_t* q_idx, const uint16_t* k_cache, const uint16_t* v_cache,
                             const int8_t* k_idx, int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws,
                             size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!starts || !counts || !q || !q_idx || !k_cache || !v_cache || !k_idx || !block_keys || !out)
    return MSA_ERR_INVALID_ARG;
  if (d.nb > msa::kMaxInvertBlocks) return MSA_ERR_UNSUPPORTED;
  long T = 0;
  for (long b = 0; b < d.B; ++b) {
    if (starts[b] < 0 || counts[b] < 0 || (long)starts[b] + counts[b] > d.S) return MSA_ERR_INVALID_ARG;
    T += counts[b];
  }
  if (T < 1) return MSA_ERR_INVALID_ARG;
  if ((long)d.G * T * d.k >= (1L << 31) || T >= (1L << 30)) return MSA_ERR_UNSUPPORTED;
  // one sequence at a time: a batch of one against its cache of capacity C
  Dims d1 = d;
  d1.B = 1;
  d1.U = d.G;
  // every sequence's plan is checked before the first launch
  for (long b = 0; b < d.B; ++b) {
    if (counts[b] == 0) continue;
    st = check_ws(ws, ws_bytes, 1);
    if (st != MSA_OK) return st;
    ChunkRun run;
    st = plan_chunk(d1, counts[b], ws_bytes, &run);
    if (st != MSA_OK) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  const size_t cache_rows = (size_t)d.G * d.S;  // rows of one sequence's cache
  long o = 0;                                   // packed row of the sequence's first query
  for (long b = 0; b < d.B; ++b) {
    const long n = counts[b];
    if (n == 0) continue;
    st = run_prefill(d1, starts[b], n, Strides{n, d.S, T, T}, q + o * d.Hq * d.D, k_cache + b * cache_rows * d.D,
                     v_cache + b * cache_rows * d.D, q_idx + o * d.di, k_idx + b * cache_rows * d.di,
                     block_keys + (size_t)b * d.G * d.nb * d.di, out + o * d.Hq * d.D, sel ? sel + o * d.k : nullptr,
                     nullptr, ws, ws_bytes, s);
    if (st != MSA_OK) return st;
    o += n;
  }
  return MSA_OK;
}

int msa_decode(const msa_dims* dims, const uint16_t* q, const int8_t* q_idx, const uint16_t* k_cache,
               const uint16_t* v_cache, const int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws,
               size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!q || !q_idx || !k_cache || !v_cache || !block_keys || !out) return MSA_ERR_INVALID_ARG;
  return run_decode(d, d.S, nullptr, q, q_idx, k_cache, v_cache, block_keys, out, sel, ws, ws_bytes,
                    (hipStream_t)stream);
}

int msa_decode_noalloc(const msa_dims* dims, const uint16_t* q, const int8_t* q_idx, const uint16_t* k_cache,
                       const uint16_t* v_cache, const int8_t* block_keys, uint16_t* out, int32_t* sel,
                       void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!q || !q_idx || !k_cache || !v_cache || !block_keys || !out) return MSA_ERR_INVALID_ARG;
  DecodeLayout L;
  st = decode_layout(d, &L);
  if (st != MSA_OK) return st;
  if (L.total > msa::kDecodeScratchBytes) return MSA_ERR_SCRATCH;
  // the current device's copy of the fixed scratch (looked up once per
  // device); no allocation, no memset: the decode kernels write every byte
  // of the scratch they later read
  void* scratch = nullptr;
  if (msa::decode_scratch(&scratch) != hipSuccess) return MSA_ERR_HIP;
  return run_decode(d, d.S, nullptr, q, q_idx, k_cache, v_cache, block_keys, out, sel, scratch,
                    msa::kDecodeScratchBytes, (hipStream_t)stream);
}

int msa_decode_init(const msa_dims* dims, int32_t length, const int8_t* k_idx, int8_t* block_keys,
                    int32_t* open_sums, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!k_idx || !block_keys || !open_sums || length < 0 || length > d.S) return MSA_ERR_INVALID_ARG;
  if (length == 0) return MSA_OK;  // the first append opens block 0 and ignores open_sums
  hipStream_t s = (hipStream_t)stream;
  MSA_LAUNCH_NAMED("pool", s, msa::launch_pool_strided(k_idx, block_keys, open_sums, (int)d.U, (int)length, d.S,
                                                       (int)d.nb, (int)d.bs, 0, s));
  return MSA_OK;
}

int msa_decode_step(const msa_dims* dims, int32_t length, const uint16_t* q, const int8_t* q_idx,
                    const uint16_t* k_new, const uint16_t* v_new, const int8_t* k_idx_new, uint16_t* k_cache,
                    uint16_t* v_cache, int32_t* open_sums, int8_t* block_keys, uint16_t* out, int32_t* sel,
                    void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!q || !q_idx || !k_new || !v_new || !k_idx_new || !k_cache || !v_cache || !open_sums || !block_keys || !out)
    return MSA_ERR_INVALID_ARG;
  if (length < 1 || length > d.S) return MSA_ERR_INVALID_ARG;
  DecodeLayout L;
  st = decode_layout(d, &L);
  if (st != MSA_OK) return st;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const msa::DecodeShape sh = decode_shape(d, length);
  MSA_LAUNCH_NAMED("append", s, msa::launch_append(sh, k_new, v_new, k_idx_new, k_cache, v_cache, open_sums,
                                                   block_keys, (int)length - 1, s));
  return run_decode(d, length, nullptr, q, q_idx, k_cache, v_cache, block_keys, out, sel, ws, ws_bytes, s);
}

int msa_decode_varlen(const msa_dims* dims, const int32_t* lengths, const uint16_t* q, const int8_t* q_idx,
                      const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* block_keys, uint16_t* out,
                      int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!q || !q_idx || !k_cache || !v_cache || !block_keys || !out) return MSA_ERR_INVALID_ARG;
  long longest = 0;
  st = check_lengths(d, lengths, 1, &longest);
  if (st != MSA_OK) return st;
  DecodeLayout L;
  st = decode_layout(d, &L);
  if (st != MSA_OK) return st;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  int32_t* lens = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.lens);
  MSA_LAUNCH_NAMED("lengths", s, msa::launch_set_lengths(lens, lengths, (int)d.B, s));
  return run_decode(d, longest, lens, q, q_idx, k_cache, v_cache, block_keys, out, sel, ws, ws_bytes, s);
}

int msa_decode_init_varlen(const msa_dims* dims, const int32_t* lengths, const int8_t* k_idx, int8_t* block_keys,
                           int32_t* open_sums, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!k_idx || !block_keys || !open_sums) return MSA_ERR_INVALID_ARG;
  long longest = 0;
  st = check_lengths(d, lengths, 0, &longest);
  if (st != MSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  // each sequence's caches as a batch of one (a length of 0 enqueues nothing)
  for (long b = 0; b < d.B; ++b) {
    if (lengths[b] == 0) continue;
    MSA_LAUNCH_NAMED("pool", s, msa::launch_pool_strided(k_idx + (size_t)b * d.G * d.S * d.di,
                                                         block_keys + (size_t)b * d.G * d.nb * d.di,
                                                         open_sums + (size_t)b * d.G * d.di, (int)d.G,
                                                         (int)lengths[b], d.S, (int)d.nb, (int)d.bs, 0, s));
  }
  return MSA_OK;
}

int msa_decode_step_varlen(const msa_dims* dims, const int32_t* lengths, const uint16_t* q, const int8_t* q_idx,
                           const uint16_t* k_new, const uint16_t* v_new, const int8_t* k_idx_new,
                           uint16_t* k_cache, uint16_t* v_cache, int32_t* open_sums, int8_t* block_keys,
                           uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!q || !q_idx || !k_new || !v_new || !k_idx_new || !k_cache || !v_cache || !open_sums || !block_keys || !out)
    return MSA_ERR_INVALID_ARG;
  long longest = 0;
  st = check_lengths(d, lengths, 1, &longest);
  if (st != MSA_OK) return st;
  DecodeLayout L;
  st = decode_layout(d, &L);
  if (st != MSA_OK) return st;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  int32_t* lens = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + L.lens);
  MSA_LAUNCH_NAMED("lengths", s, msa::launch_set_lengths(lens, lengths, (int)d.B, s));
  msa::DecodeShape sh = decode_shape(d, longest);
  sh.lens = lens;
  MSA_LAUNCH_NAMED("append", s, msa::launch_append(sh, k_new, v_new, k_idx_new, k_cache, v_cache, open_sums,
                                                   block_keys, (int)longest - 1, s));
  return run_decode(d, longest, lens, q, q_idx, k_cache, v_cache, block_keys, out, sel, ws, ws_bytes, s);
}

int msa_decode_varlen_device(const msa_dims* dims, const int32_t* lengths, const uint16_t* q, const int8_t* q_idx,
                             const uint16_t* k_cache, const uint16_t* v_cache, const int8_t* block_keys,
                             uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!lengths || !q || !q_idx || !k_cache || !v_cache || !block_keys || !out) return MSA_ERR_INVALID_ARG;
  // the kernels read each sequence's length and treat one outside 1 .. C
  // as an empty row; the launch is sized for the capacity
  return run_decode(d, d.S, lengths, q, q_idx, k_cache, v_cache, block_keys, out, sel, ws, ws_bytes,
                    (hipStream_t)stream);
}

int msa_decode_step_varlen_device(const msa_dims* dims, const int32_t* lengths, const uint16_t* q,
                                  const int8_t* q_idx, const uint16_t* k_new, const uint16_t* v_new,
                                  const int8_t* k_idx_new, uint16_t* k_cache, uint16_t* v_cache, int32_t* open_sums,
                                  int8_t* block_keys, uint16_t* out, int32_t* sel, void* ws, size_t ws_bytes,
                                  void* stream) {
  Dims d;
  int st = check_dims(dims, &d);
  if (st != MSA_OK) return st;
  if (d.k > kMaxSparseTopK) return MSA_ERR_UNSUPPORTED;
  if (!lengths || !q || !q_idx || !k_new || !v_new || !k_idx_new || !k_cache || !v_cache || !open_sums ||
      !block_keys || !out)
    return MSA_ERR_INVALID_ARG;
  DecodeLayout L;
  st = decode_layout(d, &L);
  if (st != MSA_OK) return st;
  st = check_ws(ws, ws_bytes, L.total);
  if (st != MSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  msa::DecodeShape sh = decode_shape(d, d.S);
  sh.lens = lengths;
  MSA_LAUNCH_NAMED("append", s, msa::launch_append(sh, k_new, v_new, k_idx_new, k_cache, v_cache, open_sums,
                                                   block_keys, 0, s));
  return run_decode(d, d.S, lengths, q, q_idx, k_cache, v_cache, block_keys, out, sel, ws, ws_bytes, s);
}

int msa_probe_mfma_bf16(int32_t n_workgroups, int32_t iters, float* out, double* flop, void* stream) {
  if (n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 1 || iters > (1 << 24) || out == nullptr)
    return MSA_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (flop != nullptr) *flop = msa::mfma_probe_flop(n_workgroups, iters);
  MSA_LAUNCH_NAMED("mfma_probe", s, msa::launch_mfma_probe(out, n_workgroups, iters, s));
  return MSA_OK;
}

int msa_profile_enable(int on) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_on = on != 0;
  return MSA_OK;
}

int msa_profile_read(msa_kernel_time* out, int max_entries, int* n_out) {
  if (max_entries < 0 || (max_entries > 0 && out == nullptr)) return MSA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(g_prof_mu);
  struct Agg {
    const char* name;
    int n;
    double ms;
  };
  std::vector<Agg> agg;
  int status = MSA_OK;
  for (const ProfRec& r : g_prof_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      status = MSA_ERR_HIP;
    auto it = std::find_if(agg.begin(), agg.end(), [&](const Agg& a) { return strcmp(a.name, r.name) == 0; });
    if (it == agg.end()) agg.push_back({r.name, 1, ms});
    else {
      it->n += 1;
      it->ms += ms;
    }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  const int n = (int)agg.size();
  for (int i = 0; i < n && i < max_entries; ++i) {
    memset(out[i].name, 0, sizeof(out[i].name));
    strncpy(out[i].name, agg[i].name, sizeof(out[i].name) - 1);
    out[i].launches = agg[i].n;
    out[i].total_ms = (float)agg[i].ms;
  }
  if (n_out) *n_out = n;
  return status;
}

}  // extern "C"
