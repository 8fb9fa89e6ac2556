// MSA main branch: exact softmax attention over the selected KV blocks.
//
// The main branch computes exact block-sparse attention on the blocks the
// index branch kept ("深度解析 MiniMax-M3：稀疏注意力机制、基准测试与 API 集成指南",
// section "架构核心：MoE 与 MSA 的深度融合", item 2), with the KV block in the outer
// loop: each block is read once and the query rows that selected it are
// gathered inward (yunpan.plus article on MiniMax M3, paragraph on the
// operator level; wiki.500nian.com digest of "MiniMax M3 Review", flowchart
// node "KV-outer gather Q").
//
//   attend_kernel  one work item = one KV block j of one (batch, group) unit
//                  and up to 6 chunks of 256 query rows (tokens x heads) whose
//                  selection holds j as one of the blocks before the query's
//                  own.  The kernel is persistent: one workgroup of four
//                  waves per CU walks its items, K_j and V_j^T go through one
//                  of two LDS buffers while the next item's block is staged
//                  into the other, and each wave loads the 64 gathered query
//                  rows of its next chunk during the current one.  Every row
//                  leaves an unnormalised bf16 partial and its (max, sum) in
//                  base-2 units at its selection slot.  No key of such a
//                  block is after a query that selected it: no mask.
//   merge_kernel   the own block (the one kept block holding keys after some
//                  of its queries): causal attention of 128-row tiles with P
//                  split into two bf16 terms, so P.V keeps ~16 mantissa bits
//                  for the first tokens of a block, which see only a few
//                  keys; the result, in fp32 registers, is merged with the
//                  row's partials by log-sum-exp -> out.

// Tile shapes (wave64, v_mfma_f32_32x32x16_bf16):
//   S^T = K Q^T : 32 keys x 32 query rows per tile, K from LDS (A operand),
//                 Q rows straight from HBM into registers (B operand).
//   O^T = V^T P^T : 32 head dims x 32 query rows per tile, V^T from LDS (A),
//                 P^T from the S^T accumulators (B).  A lane holds the keys
//                 8 * (i / 4) + 4 * (lane / 32) + i % 4 of its column, so the
//                 V^T reads pick those keys in the same order.
//
// Partial rows hold their 128 values lane-half-major: position
// 64 * hf + 16 * dt + i is head dim 32 * dt + 8 * (i / 4) + 4 * hf + i % 4.

#include <algorithm>

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

constexpr int kKStride = 2 * kHeadDim + 16;  // bytes per key row of K in LDS

template <int BS>
struct Tile {
  static constexpr int KT = BS / 32;             // 32-key tiles per block
  static constexpr int kVtStride = 2 * BS + 8;   // bytes per head-dim row of V^T in LDS
  static constexpr int kKBytes = BS * kKStride;
  static constexpr int kVtBytes = kHeadDim * kVtStride;
  static constexpr int kLdsBytes = kKBytes + kVtBytes;
};

// A K/V block staged in registers on its way to LDS: NT threads, K as
// 16-byte pieces of key rows, V as pairs of key rows (2p, 2p + 1) x 8 head
// dims so that V^T can be written as dwords holding two keys.
template <int BS, int NT>
struct KvStage {
  static constexpr int kK = BS * 16 / NT;
  static constexpr int kV = BS * 8 / NT;
  u32x4_t k[kK];
  u32x4_t va[kV], vb[kV];
};

// Issue the loads of a block (rows beyond n_keys are clamped to a valid row
// and zeroed when written, so every load is unconditional and in flight at
// once).
template <int BS, int NT>
__device__ __forceinline__ void load_kv_regs(const uint16_t* __restrict__ kblk, const uint16_t* __restrict__ vblk,
                                             int n_keys, KvStage<BS, NT>& st) {
  // the thread index is made opaque here so that the addresses below are
  // recomputed at each use instead of being kept live (and spilled) across
  // the whole item loop
  int tid = threadIdx.x;
  __asm__ volatile("" : "+v"(tid));
#pragma unroll
  for (int m = 0; m < KvStage<BS, NT>::kK; ++m) {
    const int qid = tid + NT * m;
    st.k[m] = *reinterpret_cast<const u32x4_t*>(kblk + min(qid >> 4, n_keys - 1) * kHeadDim + (qid & 15) * 8);
  }
#pragma unroll
  for (int m = 0; m < KvStage<BS, NT>::kV; ++m) {
    const int qid = tid + NT * m;
    const int p = qid >> 4;  // 16 lanes read the two whole rows of key pair p
    const int c = qid & 15;
    st.va[m] = *reinterpret_cast<const u32x4_t*>(vblk + min(2 * p, n_keys - 1) * kHeadDim + c * 8);
    st.vb[m] = *reinterpret_cast<const u32x4_t*>(vblk + min(2 * p + 1, n_keys - 1) * kHeadDim + c * 8);
  }
}

// Write a staged block to LDS: K key-major (rows of kKStride bytes), V
// transposed (head dim major, rows of kVtStride bytes).
template <int BS, int NT>
__device__ __forceinline__ void store_kv_lds(const KvStage<BS, NT>& st, int n_keys, char* __restrict__ lds) {
  using T = Tile<BS>;
  int tid = threadIdx.x;  // opaque, as in load_kv_regs
  __asm__ volatile("" : "+v"(tid));
#pragma unroll
  for (int m = 0; m < KvStage<BS, NT>::kK; ++m) {
    const int qid = tid + NT * m;
    const int key = qid >> 4;
    const u32x4_t val = key < n_keys ? st.k[m] : u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(lds + key * kKStride + (qid & 15) * 16) = val;
  }
  char* vt = lds + T::kKBytes;
#pragma unroll
  for (int m = 0; m < KvStage<BS, NT>::kV; ++m) {
    const int qid = tid + NT * m;
    const int p = qid >> 4;
    const int c = qid & 15;
    const u32x4_t a = 2 * p < n_keys ? st.va[m] : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t b = 2 * p + 1 < n_keys ? st.vb[m] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = (e == 0) ? a.x : (e == 1) ? a.y : (e == 2) ? a.z : a.w;
      const uint32_t hi = (e == 0) ? b.x : (e == 1) ? b.y : (e == 2) ? b.z : b.w;
      // dims 8c + 2e (low halves) and 8c + 2e + 1 (high halves)
      *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e) * T::kVtStride + 4 * p) = (lo & 0xffffu) | (hi << 16);
      *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e + 1) * T::kVtStride + 4 * p) = (lo >> 16) | (hi & 0xffff0000u);
    }
  }
}

// Eight 16-byte pieces of one query row: head dims 16 * ks + 8 * hf + 0..7.
__device__ __forceinline__ void load_q_frag(const uint16_t* __restrict__ qrow, int hf, u32x4_t (&qf)[8]) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
}

// A operand of K for key tile kt, k-step ks.
__device__ __forceinline__ u32x4_t k_frag(const char* lds, int kt, int ks, int lane) {
  const int key = 32 * kt + (lane & 31);
  return *reinterpret_cast<const u32x4_t*>(lds + key * kKStride + 32 * ks + 16 * (lane >> 5));
}

// A operand of V^T for head-dim tile dt, key tile kt, half h2 (16 keys).
template <int BS>
__device__ __forceinline__ u32x4_t vt_frag(const char* lds, int dt, int kt, int h2, int lane) {
  const char* vt = lds + Tile<BS>::kKBytes;
  const int d = 32 * dt + (lane & 31);
  const int key = 32 * kt + 16 * h2 + 4 * (lane >> 5);
  const char* p = vt + d * Tile<BS>::kVtStride + 2 * key;
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(p);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(p + 16);
  u32x4_t r = {lo.x, lo.y, hi.x, hi.y};
  return r;
}

// A column tile's results packed for storing: the row's 128 values as bf16,
// lane-half-major (position 64 * hf + 16 * dt + i), 8 u32x4 per lane.
__device__ __forceinline__ void pack_tile(const f32x16_t (&o)[4], u32x4_t (&pv)[8]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    pv[2 * dt] = u32x4_t{pack_bf16x2(o[dt][0], o[dt][1]), pack_bf16x2(o[dt][2], o[dt][3]),
                         pack_bf16x2(o[dt][4], o[dt][5]), pack_bf16x2(o[dt][6], o[dt][7])};
    pv[2 * dt + 1] = u32x4_t{pack_bf16x2(o[dt][8], o[dt][9]), pack_bf16x2(o[dt][10], o[dt][11]),
                             pack_bf16x2(o[dt][12], o[dt][13]), pack_bf16x2(o[dt][14], o[dt][15])};
  }
}

// Store a packed row of the partials: (token, slot) row prow, head `head`
// of r, lane half hf, with its (max, sum).  The 16-byte pieces of the r
// heads' rows are interleaved, piece-major (piece 2 m + hf of head h at
// piece (16 prow + 2 m + hf) r + h), so that the lanes holding one token's
// heads write, and the merge reads, r consecutive pieces.  Both lane halves
// store the (max, sum) pair (the same value), so that every path issues the
// same memory operations.  The stores are non-temporal: a partial is read
// once, by the merge, long after (measured on MI355X: the 1M prefill 173.5
// -> 168.4 ms, the 32K 5.32 -> 4.99 ms, the merge faster too).
__device__ __forceinline__ void store_row(const u32x4_t (&pv)[8], float2 ml, size_t prow, int head, int r, int hf,
                                          uint16_t* __restrict__ part_o, float2* __restrict__ part_ml) {
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(part_o) + (prow * 16 + hf) * r + head;
#pragma unroll
  for (int m = 0; m < 8; ++m) __builtin_nontemporal_store(pv[m], dst + (size_t)(2 * m) * r);
  __builtin_nontemporal_store(f32x2_t{ml.x, ml.y}, reinterpret_cast<f32x2_t*>(part_ml + prow * r + head));
}

// ---------------------------------------------------------------------------
// Attention over the KV blocks of work items.  Persistent: one workgroup per
// CU walks its items, dealt round-robin, or (DYN) taken from a counter in
// runs of `run` consecutive items: items are ordered by (unit, block), so
// the items of a run mostly share their KV block, and taking runs as
// workgroups free up keeps items of unequal cost balanced.  While it
// computes item i, the K/V block of item i + 1 is staged into the
// second LDS buffer (unless both items hold the same block, which then
// stays where it is) and the entries of item i + 2 into a wave-private LDS
// ring.
//
// Per chunk c the order is: S^T = K Q^T (waits for the chunk's query rows,
// loaded during chunk c - 1), the loads of the next position's query rows,
// softmax and P.V, the stores of the chunk's partials.  Entries come from
// the LDS ring, not from global memory, so no wait in the loop is on a load
// issued after the previous chunk's stores (vector-memory operations
// complete in order).  Loads and stores are issued the same way on every
// path (rows past an item's end repeat its last entry and rewrite identical
// values).
// ---------------------------------------------------------------------------
struct ItemDesc {
  int e0, n_ent, j, u;  // first entry, entries, block, unit
};

__device__ __forceinline__ ItemDesc decode_item(const int2* __restrict__ items, const int32_t* __restrict__ row_ptr,
                                                int idx, int n_ranges, int nb, int tpi) {
  const int2 item = items[idx];
  ItemDesc d;
  d.u = item.x / (n_ranges * nb);
  d.j = item.x % nb;
  d.e0 = row_ptr[item.x] + item.y;
  d.n_ent = min(tpi, row_ptr[item.x + 1] - d.e0);
  return d;
}

template <int BS, bool DYN>
__global__ __launch_bounds__(256, 1) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ item_ptr,
    const int2* __restrict__ items, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float2* __restrict__ part_ml, PrefillShape sh, PassInfo pass, int r_log2,
    int* __restrict__ sched, int run) {
  constexpr int KT = Tile<BS>::KT;
  extern __shared__ __align__(16) char lds[];  // two K/V buffers, then the entry rings
  __shared__ int s_first[3];  // the first three runs taken
  __shared__ int s_next[2];   // the run taken at each run boundary, by its parity

  // items of this pass: round-robin, workgroup b's p'th being b + p grid;
  // DYN: in runs taken from *sched (zeroed before the launch), of which the
  // workgroup holds three -- items a, a + 1, a + 2 of the current run reach
  // at most into the third
  const int i_begin = item_ptr[pass.row_begin];
  const int it_end = item_ptr[pass.row_end] - i_begin;
  int pos = 0;                 // round-robin: items done
  int run0 = 0, run1 = 0, run2 = 0;  // DYN: the runs in hand (uniform, in scalar registers)
  int a = 0;                   // DYN: position in the current run
  int nb_runs = 0;             // DYN: run boundaries passed
  if constexpr (DYN) {
    if (threadIdx.x == 0) {
      s_first[0] = atomicAdd(sched, 1);
      s_first[1] = atomicAdd(sched, 1);
      s_first[2] = atomicAdd(sched, 1);
    }
    __syncthreads();
    run0 = __builtin_amdgcn_readfirstlane(s_first[0]);
    run1 = __builtin_amdgcn_readfirstlane(s_first[1]);
    run2 = __builtin_amdgcn_readfirstlane(s_first[2]);
  }
  auto item_at = [&](int d) -> int {  // the item d places after the current one, d <= 2
    if constexpr (DYN) {
      const int p = a + d;
      const int k = p / run;
      return (k == 0 ? run0 : k == 1 ? run1 : run2) * run + (p - k * run);
    } else {
      return (int)blockIdx.x + (pos + d) * (int)gridDim.x;
    }
  };
  if (item_at(0) >= it_end) return;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;  // rows 64 w .. 64 w + 63 of every chunk
  const int hf = lane >> 5;
  const int K = sh.top_k;
  const float c2 = sh.scale_log2;
  const int tpc = kItemRows >> r_log2;  // tokens per chunk
  const int tpi = kItemChunks * tpc;    // tokens per item
  const int epw = 64 >> r_log2;         // tokens of one wave in one chunk
  const int ring = kItemChunks * epw;   // a wave's entries of one item
  uint32_t* ering = reinterpret_cast<uint32_t*>(lds + 2 * Tile<BS>::kLdsBytes) + w * 3 * ring;
  const size_t pass_row0 = (size_t)0 - pass.t0;

  auto decode_at = [&](int idx) -> ItemDesc {
    return decode_item(items, row_ptr, i_begin + min(idx, it_end - 1), sh.n_ranges, sh.nb, tpi);
  };
  auto n_chunks_of = [&](const ItemDesc& d) -> int { return (d.n_ent + tpc - 1) / tpc; };
  auto q_base = [&](int u) -> const uint16_t* {
    const int b = u / sh.G;
    return q + ((size_t)b * sh.q_stride * sh.Hq + (u - b * sh.G) * sh.r) * kHeadDim;
  };
  // this wave's entries of item d: ring position jj = c * epw + i holds
  // the entry of token c * tpc + (64 w >> r_log2) + i (clamped to the item)
  auto load_ents = [&](const ItemDesc& d, uint32_t (&e)[kItemChunks]) {
#pragma unroll
    for (int m = 0; m < kItemChunks; ++m) {
      const int jj = min(lane + 64 * m, ring - 1);
      const int tk = (jj / epw) * tpc + ((64 * w) >> r_log2) + jj % epw;
      e[m] = entries[d.e0 + min(tk, d.n_ent - 1)];
    }
  };
  auto store_ents = [&](int slot, const uint32_t (&e)[kItemChunks]) {
#pragma unroll
    for (int m = 0; m < kItemChunks; ++m)
      if (lane + 64 * m < ring) ering[slot * ring + lane + 64 * m] = e[m];
  };
  auto ent_at = [&](int slot, int c, int ct) -> uint32_t {
    return ering[slot * ring + c * epw + ((32 * ct + (lane & 31)) >> r_log2)];
  };
  auto load_q = [&](const uint16_t* qb, const uint32_t (&e)[2], u32x4_t (&qf)[2][8]) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int qr = 64 * w + 32 * ct + (lane & 31);
      load_q_frag(qb + ((size_t)(e[ct] >> 5) * sh.Hq + (qr & (sh.r - 1))) * kHeadDim, hf, qf[ct]);
    }
  };
  auto kv_src = [&](const ItemDesc& d, size_t* off) -> int {
    *off = ((size_t)d.u * sh.kv_rows + (size_t)d.j * BS) * kHeadDim;
    return min(BS, sh.q0 + sh.S - d.j * BS);
  };

  // ---- prologue: entries of the first two items, the first block, the
  // first chunk's query rows
  ItemDesc cur = decode_at(item_at(0));
  ItemDesc nxt = decode_at(item_at(1));
  ItemDesc nxt2 = decode_at(item_at(2));
  int qn = 0;  // sequence number of the current item (entry ring slot qn % 3)
  {
    uint32_t e0r[kItemChunks], e1r[kItemChunks];
    load_ents(cur, e0r);
    load_ents(nxt, e1r);
    store_ents(0, e0r);
    store_ents(1, e1r);
  }
  u32x4_t qf[2][8];
  const uint16_t* qb = q_base(cur.u);
  {
    uint32_t e[2] = {ent_at(0, 0, 0), ent_at(0, 0, 1)};
    load_q(qb, e, qf);
  }
  KvStage<BS, 256> kv;
  {
    size_t off;
    const int nk = kv_src(cur, &off);
    load_kv_regs<BS, 256>(k + off, v + off, nk, kv);
    store_kv_lds<BS, 256>(kv, nk, lds);
  }
  __syncthreads();

  int buf = 0;
  while (true) {
    const bool has_next = item_at(1) < it_end;
    // DYN: at the last item of a run, the run after the two in hand is taken
    // (its index is needed only at the end of the item)
    const bool boundary = DYN && a == run - 1;
    int taken = 0;
    if constexpr (DYN) {
      if (threadIdx.x == 0 && boundary && has_next) taken = atomicAdd(sched, 1);
    }
    // the next item's block (DYN: unless it is this one's, which then stays
    // in its buffer) and the entries of the item after it
    const bool same_next = DYN && has_next && nxt.u == cur.u && nxt.j == cur.j;
    size_t nxt_off;
    const int nxt_keys = kv_src(nxt, &nxt_off);
    if (!same_next) load_kv_regs<BS, 256>(k + nxt_off, v + nxt_off, nxt_keys, kv);
    uint32_t e2r[kItemChunks];
    load_ents(nxt2, e2r);
    const uint16_t* nxt_qb = q_base(nxt.u);
    const size_t row0 = (size_t)(cur.u - pass.u0) * pass.pass_tokens + pass_row0;
    const int n_chunks = n_chunks_of(cur);
    const int slot_cur = qn % 3;
    const int slot_nxt = (qn + 1) % 3;

    for (int c = 0; c < n_chunks; ++c) {
      const bool first = c == 0;
      // the block's LDS offset is made opaque per chunk, so that the
      // fragment reads stay inside the loop (hoisted they would need far
      // more registers than a wave has)
      int kvo = buf * Tile<BS>::kLdsBytes;
      __asm__ volatile("" : "+v"(kvo));
      const char* kvl = lds + kvo;
      int tok[2], slot[2], head[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const uint32_t e = ent_at(slot_cur, c, ct);
        tok[ct] = (int)(e >> 5);
        slot[ct] = (int)(e & 31u);
        head[ct] = (64 * w + 32 * ct + (lane & 31)) & (sh.r - 1);
      }
      // the position after this chunk: the item's next chunk, else the
      // next item's first (or, at the very end, a repeat of this one)
      const bool in_cur = c + 1 < n_chunks;
      uint32_t ent_nx[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        ent_nx[ct] = in_cur ? ent_at(slot_cur, c + 1, ct) : ent_at(has_next ? slot_nxt : slot_cur, has_next ? 0 : c, ct);
      const uint16_t* qb_nx = (in_cur || !has_next) ? qb : nxt_qb;

      // S^T = K Q^T
      f32x16_t s[KT][2];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt][0] = f32x16_t{};
        s[kt][1] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const u32x4_t a = k_frag(kvl, kt, ks, lane);
          s[kt][0] = mfma32x32x16(a, qf[0][ks], s[kt][0]);
          s[kt][1] = mfma32x32x16(a, qf[1][ks], s[kt][1]);
        }
      }
      // the next item's block goes to the other LDS buffer after the first
      // chunk's S^T (its loads were issued at the start of the item, after
      // everything this wait also covers); the entries of the item after it
      // go to the ring
      if (first) {
        if (has_next && !same_next) store_kv_lds<BS, 256>(kv, nxt_keys, lds + (buf ^ 1) * Tile<BS>::kLdsBytes);
        store_ents((qn + 2) % 3, e2r);
      }
      load_q(qb_nx, ent_nx, qf);

      size_t prow[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) prow[ct] = (row0 + tok[ct]) * K + slot[ct];
      // softmax: the block lies wholly before every query of the chunk (the
      // own block is attended by the merge), so no key is masked
      float m2[2], sum[2];
      u32x4_t ph[KT][2][2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][ct][i]);
        m2[ct] = wave_max_pair(mx) * c2;
        sum[ct] = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            uint32_t d[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e], c2, -m2[ct]));
              const float p1 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e + 1], c2, -m2[ct]));
              sum[ct] += p0 + p1;
              d[e] = pack_bf16x2(p0, p1);
            }
            ph[kt][ct][h2] = u32x4_t{d[0], d[1], d[2], d[3]};
          }
      }
      // O^T = V^T P^T, one column tile at a time; V^T is read again for
      // the second tile (kept from the first it would take 128 registers)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        int vo = kvo;
        __asm__ volatile("" : "+v"(vo));
        const char* kvt = lds + vo;
        f32x16_t o[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
              o[dt] = mfma32x32x16(vt_frag<BS>(kvt, dt, kt, h2, lane), ph[kt][ct][h2], o[dt]);
        u32x4_t pv1[8];
        pack_tile(o, pv1);
        store_row(pv1, make_float2(m2[ct], wave_sum_pair(sum[ct])), prow[ct], head[ct], sh.r, hf, part_o, part_ml);
      }
      qb = qb_nx;
    }
    if (!has_next) break;
    // (two slots by parity: a slot is rewritten only after every wave has
    // passed the barrier that follows its read)
    if constexpr (DYN) {
      if (threadIdx.x == 0 && boundary) s_next[nb_runs & 1] = taken;
    }
    // the other buffer is complete and every wave is done with this one
    __syncthreads();
    if (!same_next) buf ^= 1;
    if constexpr (DYN) {
      if (boundary) {
        run0 = run1;
        run1 = run2;
        run2 = __builtin_amdgcn_readfirstlane(s_next[nb_runs & 1]);
        ++nb_runs;
        a = 0;
      } else {
        ++a;
      }
    } else {
      ++pos;
    }
    ++qn;
    cur = nxt;
    nxt = nxt2;
    nxt2 = decode_at(item_at(2));
  }
}

// ---------------------------------------------------------------------------
// Own block and merge.  A query's own block is the one kept block that
// holds keys after some of its queries; it is attended here, not in the
// attention kernel, and its result stays in registers in fp32 while the
// row's other partials are merged into it:
//   out = (2^(m_o - M) o_o + sum_s 2^(m_s - M) o_s) / (2^(m_o - M) l_o + sum_s 2^(m_s - M) l_s)
// with M the largest of the maxima, over the own block (o) and the
// min(top_k - 1, own) partials s of the row.  One workgroup per tile of 128
// query rows (128 / r tokens x the r heads of a group), one 32-row column
// tile per wave.  The own block's keys up to the tile's last token go to
// LDS (K key-major, V transposed), then S^T = K Q^T with the causal mask, a
// base-2 softmax and O^T += V^T P^T with P split into two bf16 terms
// (hi + lo, ~16 mantissa bits, for the first tokens of a block, which see
// few keys).  A tile whose tokens fall in two blocks takes them in turn,
// each row attending only its own.  The partials are read once, with a
// non-temporal hint, each lane reading its row's half (the lanes of one
// token's heads read consecutive pieces).  Workgroups go to the eight XCDs
// in turn; tiles are numbered so that each XCD takes runs of eight
// consecutive tiles, which mostly share their block, whose K and V then
// come from that XCD's L2 after the first read.  Measured on MI355X against
// attending the own block in the attention kernel and merging its partial
// like the others: the 1M prefill 200 -> 172 ms with the interleaved
// partial layout (the attention kernel 142 -> 113 ms, the merge 48 ms both).
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 128;  // query rows per workgroup
constexpr int kMaxOther = 31;    // partials per row besides the own block
constexpr int kMergeRowBytes = 2 * kHeadDim + 16;  // a row of O in LDS (padded)
template <int BS>
constexpr int merge_lds_bytes() {
  return Tile<BS>::kLdsBytes > kMergeRows * kMergeRowBytes ? Tile<BS>::kLdsBytes : kMergeRows * kMergeRowBytes;
}

// Value e (0..7) of a packed u32x4 of bf16 pairs.
__device__ __forceinline__ float bf16_at(const u32x4_t& v, int e) {
  const uint32_t x = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? bf16_hi(x) : bf16_lo(x);
}

template <int BS>
__global__ __launch_bounds__(256, 2) void merge_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       const uint16_t* __restrict__ part_o,
                                                       const float2* __restrict__ part_ml,
                                                       uint16_t* __restrict__ out, PrefillShape sh, PassInfo pass,
                                                       int r_log2, int n_tiles) {
  constexpr int KT = Tile<BS>::KT;
  extern __shared__ __align__(16) char lds[];  // one K/V buffer
  // workgroup i runs on XCD i % 8; its 64-tile group gives XCD x the tiles
  // 8 x .. 8 x + 7
  const int gi = (int)blockIdx.x;
  const int tile = (gi & ~63) + 8 * (gi & 7) + ((gi >> 3) & 7);
  if (tile >= n_tiles) return;
  const int u = pass.u0 + (int)blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const int K = sh.top_k;
  const float c2 = sh.scale_log2;
  const int tpt = kMergeRows >> r_log2;         // tokens per tile
  const int t_a = pass.t0 + tile * tpt;          // the tile's first token
  const int t_z = min(pass.t1, t_a + tpt) - 1;   // and its last
  // this wave's tokens tw0 .. tw1 (none if tw1 < tw0)
  const int tw0 = t_a + ((32 * w) >> r_log2);
  const int tw1 = min(t_z, t_a + ((32 * w + 31) >> r_log2));
  const bool wave_live = tw0 <= tw1;
  const int qr = 32 * w + (lane & 31);
  const int tok = t_a + (qr >> r_log2);
  const int head = qr & (sh.r - 1);
  const bool live = tok <= t_z;
  const int tc = min(tok, t_z);
  const int pos = sh.q0 + tc;
  const int jo = pos >> sh.bs_log2;  // the row's own block
  const size_t orow = ((size_t)b * sh.q_stride + tc) * sh.Hq + g * sh.r + head;

  u32x4_t qf[8];
  load_q_frag(q + orow * kHeadDim, hf, qf);
  float m = -__builtin_inff(), l = 0.f;
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};

  const int jf = (sh.q0 + t_a) >> sh.bs_log2;
  const int jl = (sh.q0 + t_z) >> sh.bs_log2;
  const int jw0 = (sh.q0 + tw0) >> sh.bs_log2;  // own blocks of this wave's rows
  const int jw1 = (sh.q0 + tw1) >> sh.bs_log2;
  for (int j = jf; j <= jl; ++j) {
    // keys of block j up to the tile's last token (rows beyond are zeroed)
    const int n_keys = min(BS, sh.q0 + t_z + 1 - j * BS);
    if (j > jf) __syncthreads();  // every wave is done with block j - 1
    {
      KvStage<BS, 256> kv;
      const size_t off = ((size_t)u * sh.kv_rows + (size_t)j * BS) * kHeadDim;
      load_kv_regs<BS, 256>(k + off, v + off, n_keys, kv);
      store_kv_lds<BS, 256>(kv, n_keys, lds);
    }
    __syncthreads();
    if (!wave_live || j < jw0 || j > jw1) continue;  // no row of this wave owns block j
    // key tiles that hold a key not after this wave's last token
    const int kt_n = j < jw1 ? KT : ((sh.q0 + tw1 - j * BS) >> 5) + 1;
    int ko = 0;
    __asm__ volatile("" : "+v"(ko));
    const char* kvl = lds + ko;
    f32x16_t sc[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      sc[kt] = f32x16_t{};
      if (kt < kt_n) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) sc[kt] = mfma32x32x16(k_frag(kvl, kt, ks, lane), qf[ks], sc[kt]);
      }
    }
    // visible: the row's own block, keys not after the query (the lane-half
    // term of the key index moved to the right-hand side)
    const int lim = jo == j ? pos - j * BS - 4 * hf : -64;
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (kt >= kt_n || 32 * kt + c_row(i, 0) > lim) sc[kt][i] = -__builtin_inff();
        mx = fmaxf(mx, sc[kt][i]);
      }
    const float m_new = fmaxf(m, wave_max_pair(mx) * c2);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;  // a row with no key yet
    const float alpha = fast_exp2(m - m_use);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
    int vo = 0;
    __asm__ volatile("" : "+v"(vo));
    const char* kvt = lds + vo;
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      if (kt < kt_n) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t dh[4], dl[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(sc[kt][8 * h2 + 2 * e], c2, -m_use));
            const float p1 = fast_exp2(fmaf(sc[kt][8 * h2 + 2 * e + 1], c2, -m_use));
            sum += p0 + p1;
            dh[e] = pack_bf16x2(p0, p1);
            dl[e] = pack_bf16x2(p0 - bf16_lo(dh[e]), p1 - bf16_hi(dh[e]));
          }
          const u32x4_t ph = u32x4_t{dh[0], dh[1], dh[2], dh[3]};
          const u32x4_t pl = u32x4_t{dl[0], dl[1], dl[2], dl[3]};
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const u32x4_t a = vt_frag<BS>(kvt, dt, kt, h2, lane);
            o[dt] = mfma32x32x16(a, ph, o[dt]);
            o[dt] = mfma32x32x16(a, pl, o[dt]);
          }
        }
      }
    }
    l = fmaf(l, alpha, wave_sum_pair(sum));
    m = m_new;
  }

  // ---- merge: the row's other partials (slots 0 .. nv - 1; the own block
  // is slot nv), four at a time, each lane reading its row's half (the
  // values o[dt][i], positions 64 hf + 16 dt + i); the running max M moves
  // up per batch
  const int nv = live ? min(K - 1, jo) : 0;
  const int nvw = wave_live ? min(K - 1, jw1) : 0;  // the most any row of the wave has
  const size_t pbase = ((size_t)(u - pass.u0) * pass.pass_tokens + (tc - pass.t0)) * K;
  const u32x4_t* pob = reinterpret_cast<const u32x4_t*>(part_o) + (pbase * 16 + hf) * sh.r + head;
  const float2* pml = part_ml + pbase * sh.r + head;
  const size_t slot_pieces = (size_t)16 * sh.r;
  float M = m;  // finite: key 0 of the own block is visible to every row
  float W = l;
  constexpr int kB = 4;
#pragma unroll
  for (int s0 = 0; s0 < kMaxOther; s0 += kB) {
    if (s0 >= nvw) break;
    u32x4_t val[kB][8];
    f32x2_t ml[kB];
#pragma unroll
    for (int s = 0; s < kB; ++s) {
      ml[s] = f32x2_t{-__builtin_inff(), 0.f};
      if (s0 + s < nv) {
        ml[s] = __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(pml + (size_t)(s0 + s) * sh.r));
        const u32x4_t* src = pob + (size_t)(s0 + s) * slot_pieces;
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) val[s][mm] = __builtin_nontemporal_load(src + (size_t)(2 * mm) * sh.r);
      }
    }
    float Mn = M;
#pragma unroll
    for (int s = 0; s < kB; ++s) Mn = fmaxf(Mn, ml[s].x);
    const float a = fast_exp2(M - Mn);
    W *= a;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= a;
#pragma unroll
    for (int s = 0; s < kB; ++s)
      if (s0 + s < nv) {
        const float wgt = fast_exp2(ml[s].x - Mn);
        W = fmaf(wgt, ml[s].y, W);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[dt][i] = fmaf(wgt, bf16_at(val[s][2 * dt + (i >> 3)], i & 7), o[dt][i]);
      }
    M = Mn;
  }
  const float inv = 1.0f / W;
  if (live && sh.lse != nullptr && hf == 0) sh.lse[orow] = (M + fast_log2(W)) * 0.6931471805599453f;
  // O goes out through LDS (every wave is past its last K/V read at the
  // barrier): each lane writes its 64 values, head dims 32 dt + 8 q4 + 4 hf
  // + 0..3, into the tile's row-major copy, and the stores then cover whole
  // rows, a token's r heads being consecutive rows of out.  (Stored straight
  // from the lanes, every store instruction touched a sliver of 64 rows:
  // measured on MI355X, the 1M prefill's merge took twice as long.)
  __syncthreads();
  char* ob = lds + qr * kMergeRowBytes;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2_t wv;
      wv.x = pack_bf16x2(o[dt][4 * q4 + 0] * inv, o[dt][4 * q4 + 1] * inv);
      wv.y = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<u32x2_t*>(ob + 2 * (32 * dt + 8 * q4 + 4 * hf)) = wv;
    }
  __syncthreads();
  // O is not read again by the prefill: non-temporal stores keep it from
  // lingering dirty in the caches (a decode right after a 32K prefill:
  // 48.5 -> 46.5 us on MI355X)
#pragma unroll
  for (int it = 0; it < kMergeRows * 16 / 256; ++it) {
    const int piece = (int)threadIdx.x + 256 * it;
    const int row = piece >> 4;
    const int tk = t_a + (row >> r_log2);
    if (tk <= t_z) {
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(lds + row * kMergeRowBytes + 16 * (piece & 15));
      uint16_t* dst = out + (((size_t)b * sh.q_stride + tk) * sh.Hq + g * sh.r + (row & (sh.r - 1))) * kHeadDim +
                      8 * (piece & 15);
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(dst));
    }
  }
}

template <int BS>
hipError_t launch_attend_bs(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr,
                            const int2* items, const uint32_t* entries, uint16_t* part_o, float2* part_ml,
                            int* sched, int max_items, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  // one workgroup per CU, never more workgroups than items
  int n_cu = 0;
  const hipError_t ce = current_cu_count(&n_cu);
  if (ce != hipSuccess) return ce;
  if (max_items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::max<long>(1, std::min<long>((long)n_cu, (long)max_items));
  // runs of 4 items taken from the counter where every workgroup has many
  // items (measured on MI355X: the 1M prefill 2.3 % faster; with fewer items
  // per workgroup, at 32K and 128K, round-robin was 1 % faster)
  const bool dyn = (long)max_items >= 512L * grid;
  const int run = dyn ? 4 : 1;
  if (dyn) {
    const hipError_t fe = launch_fill_i32(sched, 0, 1, st);
    if (fe != hipSuccess) return fe;
  }
  // two K/V buffers and, per wave, a ring of three items' entries
  const int lds_bytes = 2 * Tile<BS>::kLdsBytes + 4 * 3 * kItemChunks * (64 >> r_log2) * 4;
  const void* fn = dyn ? reinterpret_cast<const void*>(&attend_kernel<BS, true>)
                       : reinterpret_cast<const void*>(&attend_kernel<BS, false>);
  const hipError_t attr = ensure_dynamic_lds(fn, 2 * Tile<BS>::kLdsBytes + 4 * 3 * kItemChunks * 64 * 4);
  if (attr != hipSuccess) return attr;
  if (dyn)
    hipLaunchKernelGGL((attend_kernel<BS, true>), dim3(grid), dim3(256), lds_bytes, st, q, k, v, row_ptr, item_ptr,
                       items, entries, part_o, part_ml, sh, pass, r_log2, sched, run);
  else
    hipLaunchKernelGGL((attend_kernel<BS, false>), dim3(grid), dim3(256), lds_bytes, st, q, k, v, row_ptr, item_ptr,
                       items, entries, part_o, part_ml, sh, pass, r_log2, sched, run);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Dense causal attention, for a prefill whose top_k covers every block (the
// selection then keeps all earlier blocks and the own block, and MSA is
// plain causal GQA attention): one workgroup per tile of 256 query rows
// (256 / r tokens x the r heads of a group) of one unit, the longest tiles
// first.  The KV blocks 0 .. (last token of the tile) / BS stream through two
// LDS buffers (the next block's loads in flight while one is computed); per
// block S^T = K Q^T, an online softmax in base 2 and O^T += V^T P^T, with
// the causal mask and the two-term P (hi + lo in bf16) on the blocks that
// hold a tile token, as in the sparse kernel.  O is written once, no
// partials.
// ---------------------------------------------------------------------------
template <int BS, int NCT>
__global__ __launch_bounds__(512 / NCT, 1) void dense_kernel(const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             uint16_t* __restrict__ out, PrefillShape sh, int r_log2) {
  // NCT column tiles of 32 rows per wave, 8 / NCT waves per tile of 256 rows
  constexpr int KT = Tile<BS>::KT;
  constexpr int NT = 512 / NCT;
  static_assert(2 * Tile<BS>::kLdsBytes >= 128 * kMergeRowBytes, "half a tile of O must fit the K/V buffers");
  extern __shared__ __align__(16) char lds[];  // two K/V buffers
  const int tpt = kItemRows >> r_log2;          // tokens per tile
  const int n_tiles = (sh.S + tpt - 1) / tpt;
  const int tile = n_tiles - 1 - (int)blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const float c2 = sh.scale_log2;
  const int t0 = tile * tpt;
  const int last_tok = min(sh.S, t0 + tpt) - 1;
  const int j_last = last_tok >> sh.bs_log2;
  const int j_mask = t0 >> sh.bs_log2;  // blocks from here on hold keys after some tile token

  int tok[NCT], head[NCT];
  u32x4_t qf[NCT][8];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int qr = 32 * (NCT * w + ct) + (lane & 31);
    tok[ct] = t0 + (qr >> r_log2);
    head[ct] = qr & (sh.r - 1);
    const int tc = min(tok[ct], sh.S - 1);
    load_q_frag(q + (((size_t)b * sh.q_stride + tc) * sh.Hq + g * sh.r + head[ct]) * kHeadDim, hf, qf[ct]);
  }
  float m[NCT], l[NCT];
  f32x16_t o[NCT][4];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m[ct] = -__builtin_inff();
    l[ct] = 0.f;
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[ct][dt] = f32x16_t{};

  auto kv_off = [&](int j) -> size_t { return ((size_t)u * sh.kv_rows + (size_t)j * BS) * kHeadDim; };
  auto kv_keys = [&](int j) -> int { return min(BS, sh.S - j * BS); };
  KvStage<BS, NT> kv;
  load_kv_regs<BS, NT>(k + kv_off(0), v + kv_off(0), kv_keys(0), kv);
  store_kv_lds<BS, NT>(kv, kv_keys(0), lds);
  __syncthreads();

  for (int j = 0; j <= j_last; ++j) {
    const bool more = j < j_last;
    if (more) load_kv_regs<BS, NT>(k + kv_off(j + 1), v + kv_off(j + 1), kv_keys(j + 1), kv);
    int kvo = (j & 1) * Tile<BS>::kLdsBytes;
    __asm__ volatile("" : "+v"(kvo));
    const bool masked = j >= j_mask;
    const float lo_on = masked ? 1.0f : 0.0f;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // S^T = K Q^T of this column tile (K is read again for the second
      // tile: both at once would need 64 more registers)
      int ko = kvo;
      __asm__ volatile("" : "+v"(ko));
      const char* kvl = lds + ko;
      f32x16_t s[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        s[kt] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) s[kt] = mfma32x32x16(k_frag(kvl, kt, ks, lane), qf[ct][ks], s[kt]);
      }
      if (masked) {
        const int lim = tok[ct] - j * BS - 4 * hf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + c_row(i, 0) > lim) s[kt][i] = -__builtin_inff();
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
      // finite from block 0 on: key 0 is visible to every token
      const float m_new = fmaxf(m[ct], wave_max_pair(mx) * c2);
      const float alpha = fast_exp2(m[ct] - m_new);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[ct][dt][i] *= alpha;
      int vo = kvo;
      __asm__ volatile("" : "+v"(vo));
      const char* kvt = lds + vo;
      float sum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          uint32_t dh[4], dl[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(fmaf(s[kt][8 * h2 + 2 * e], c2, -m_new));
            const float p1 = fast_exp2(fmaf(s[kt][8 * h2 + 2 * e + 1], c2, -m_new));
            sum += p0 + p1;
            dh[e] = pack_bf16x2(p0, p1);
            dl[e] = pack_bf16x2((p0 - bf16_lo(dh[e])) * lo_on, (p1 - bf16_hi(dh[e])) * lo_on);
          }
          const u32x4_t ph = u32x4_t{dh[0], dh[1], dh[2], dh[3]};
          const u32x4_t pl = u32x4_t{dl[0], dl[1], dl[2], dl[3]};
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const u32x4_t a = vt_frag<BS>(kvt, dt, kt, h2, lane);
            o[ct][dt] = mfma32x32x16(a, ph, o[ct][dt]);
            if (masked) o[ct][dt] = mfma32x32x16(a, pl, o[ct][dt]);
          }
        }
      l[ct] = fmaf(l[ct], alpha, wave_sum_pair(sum));
      m[ct] = m_new;
    }
    // the next block into the other buffer (released by the barrier that
    // ended block j - 1), its loads having had this block's work to arrive
    if (more) store_kv_lds<BS, NT>(kv, kv_keys(j + 1), lds + ((j + 1) & 1) * Tile<BS>::kLdsBytes);
    __syncthreads();
  }

  // O = o / l, out through LDS in two halves of 128 rows (the loop's last
  // barrier freed it): each lane writes its values, head dims 32 dt + 8 q4 +
  // 4 hf + 0..3, into a row-major copy, and the stores then cover whole rows
  // (a token's r heads are consecutive rows of out)
  float inv[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    inv[ct] = 1.0f / l[ct];
    if (sh.lse != nullptr && hf == 0 && tok[ct] < sh.S)
      sh.lse[((size_t)b * sh.q_stride + tok[ct]) * sh.Hq + g * sh.r + head[ct]] =
          (m[ct] + fast_log2(l[ct])) * 0.6931471805599453f;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int qr = 32 * (NCT * w + ct) + (lane & 31);
      if ((qr >> 7) == half) {
        char* ob = lds + (qr & 127) * kMergeRowBytes;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            u32x2_t wv;
            wv.x = pack_bf16x2(o[ct][dt][4 * q4 + 0] * inv[ct], o[ct][dt][4 * q4 + 1] * inv[ct]);
            wv.y = pack_bf16x2(o[ct][dt][4 * q4 + 2] * inv[ct], o[ct][dt][4 * q4 + 3] * inv[ct]);
            *reinterpret_cast<u32x2_t*>(ob + 2 * (32 * dt + 8 * q4 + 4 * hf)) = wv;
          }
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 128 * 16 / NT; ++it) {
      const int piece = (int)threadIdx.x + NT * it;
      const int qr = 128 * half + (piece >> 4);
      const int tk = t0 + (qr >> r_log2);
      if (tk < sh.S) {
        const u32x4_t val = *reinterpret_cast<const u32x4_t*>(lds + (piece >> 4) * kMergeRowBytes + 16 * (piece & 15));
        *reinterpret_cast<u32x4_t*>(out + (((size_t)b * sh.q_stride + tk) * sh.Hq + g * sh.r + (qr & (sh.r - 1))) *
                                              kHeadDim + 8 * (piece & 15)) = val;
      }
    }
    __syncthreads();
  }
}

// sel of a dense prefill: every block up to the own one, ascending, then -1
// (rows of unit u at sel + u * sel_rows * top_k).
__global__ __launch_bounds__(256) void dense_sel_kernel(int32_t* __restrict__ sel, int units, int S, int bs_log2,
                                                        int top_k, int sel_rows) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)units * S * top_k) return;
  const int s = (int)(i % top_k);
  const int t = (int)((i / top_k) % S);
  const long u = i / ((long)S * top_k);
  sel[(u * sel_rows + t) * top_k + s] = s <= (t >> bs_log2) ? s : -1;
}

}  // namespace

hipError_t launch_attend(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr, const int2* items,
                         const uint32_t* entries, uint16_t* part_o, float2* part_ml, int* sched, int max_items,
                         hipStream_t st) {
  switch (sh.bs) {
    case 32:
      return launch_attend_bs<32>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_ml, sched,
                                  max_items, st);
    case 64:
      return launch_attend_bs<64>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_ml, sched,
                                  max_items, st);
    default:
      return launch_attend_bs<128>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_ml, sched,
                                   max_items, st);
  }
}

hipError_t launch_merge(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                        const uint16_t* v, const uint16_t* part_o, const float2* part_ml, uint16_t* out,
                        hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  if (pass.t0 >= pass.t1 || pass.u0 >= pass.u1) return hipSuccess;
  const int tpt = kMergeRows >> r_log2;
  const int n_tiles = (pass.t1 - pass.t0 + tpt - 1) / tpt;
  const dim3 grid((unsigned)((n_tiles + 63) / 64 * 64), (unsigned)(pass.u1 - pass.u0));
  switch (sh.bs) {
#define MSA_MERGE_LAUNCH(BS_)                                                                                     \
  {                                                                                                               \
    const hipError_t attr =                                                                                       \
        ensure_dynamic_lds(reinterpret_cast<const void*>(&merge_kernel<BS_>), merge_lds_bytes<BS_>());           \
    if (attr != hipSuccess) return attr;                                                                          \
    hipLaunchKernelGGL((merge_kernel<BS_>), grid, dim3(256), merge_lds_bytes<BS_>(), st, q, k, v, part_o, part_ml, \
                       out, sh, pass, r_log2, n_tiles);                                                           \
    break;                                                                                                        \
  }
    case 32:
      MSA_MERGE_LAUNCH(32)
    case 64:
      MSA_MERGE_LAUNCH(64)
    default:
      MSA_MERGE_LAUNCH(128)
#undef MSA_MERGE_LAUNCH
  }
  return hipGetLastError();
}


hipError_t launch_dense(const PrefillShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* out, int32_t* sel, int sel_rows, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  const int tpt = kItemRows >> r_log2;
  const dim3 grid((unsigned)((sh.S + tpt - 1) / tpt), (unsigned)(sh.B * sh.G));
  switch (sh.bs) {
#define MSA_DENSE_LAUNCH(BS_, NCT_)                                                                          \
  {                                                                                                           \
    const hipError_t attr = ensure_dynamic_lds(reinterpret_cast<const void*>(&dense_kernel<BS_, NCT_>),        \
                                               2 * Tile<BS_>::kLdsBytes);                                     \
    if (attr != hipSuccess) return attr;                                                                      \
    hipLaunchKernelGGL((dense_kernel<BS_, NCT_>), grid, dim3(512 / NCT_), 2 * Tile<BS_>::kLdsBytes, st, q, k, v, \
                       out, sh, r_log2);                                                                      \
    break;                                                                                                    \
  }
    // one column tile per wave (8 waves) where a block gives every thread
    // a piece of V to stage, two (4 waves) for 32-key blocks
    case 32:
      MSA_DENSE_LAUNCH(32, 2)
    case 64:
      MSA_DENSE_LAUNCH(64, 1)
    default:
      MSA_DENSE_LAUNCH(128, 1)
#undef MSA_DENSE_LAUNCH
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sel == nullptr) return e;
  const long n = (long)sh.B * sh.G * sh.S * sh.top_k;
  hipLaunchKernelGGL(dense_sel_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sel, sh.B * sh.G, sh.S,
                     sh.bs_log2, sh.top_k, sel_rows);
  return hipGetLastError();
}

}  // namespace msa
