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
//                  and up to 4 chunks of 256 query rows (tokens x heads) whose
//                  selection holds j, the query's own block included.  The
//                  kernel is persistent: one workgroup of four waves per CU
//                  walks its items, K_j and V_j^T go through one of two LDS
//                  buffers while the next item's block is staged into the
//                  other, and each wave loads the 64 gathered query rows of
//                  its next chunk during the current one.  Every row leaves an
//                  unnormalised bf16 partial and its (max, sum) in base-2
//                  units at its selection slot (a row with no other partial,
//                  own block 0 or top_k = 1, leaves o / l with a sum of 1).
//                  Chunks holding a query's own block apply the
//                  causal mask and split P into two bf16 terms, so P.V keeps
//                  ~16 mantissa bits for the first tokens of a sequence,
//                  which see only a few keys.
//   merge_kernel   log-sum-exp merge of a query row's partials -> out.
//
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
__device__ __forceinline__ void pack_tile(const f32x16_t (&o)[4], float scale, u32x4_t (&pv)[8]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    pv[2 * dt] = u32x4_t{pack_bf16x2(o[dt][0] * scale, o[dt][1] * scale), pack_bf16x2(o[dt][2] * scale, o[dt][3] * scale),
                         pack_bf16x2(o[dt][4] * scale, o[dt][5] * scale), pack_bf16x2(o[dt][6] * scale, o[dt][7] * scale)};
    pv[2 * dt + 1] =
        u32x4_t{pack_bf16x2(o[dt][8] * scale, o[dt][9] * scale), pack_bf16x2(o[dt][10] * scale, o[dt][11] * scale),
                pack_bf16x2(o[dt][12] * scale, o[dt][13] * scale), pack_bf16x2(o[dt][14] * scale, o[dt][15] * scale)};
  }
}

// Without a scale: plain conversion.
__device__ __forceinline__ void pack_tile(const f32x16_t (&o)[4], u32x4_t (&pv)[8]) {
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    pv[2 * dt] = u32x4_t{pack_bf16x2(o[dt][0], o[dt][1]), pack_bf16x2(o[dt][2], o[dt][3]),
                         pack_bf16x2(o[dt][4], o[dt][5]), pack_bf16x2(o[dt][6], o[dt][7])};
    pv[2 * dt + 1] = u32x4_t{pack_bf16x2(o[dt][8], o[dt][9]), pack_bf16x2(o[dt][10], o[dt][11]),
                             pack_bf16x2(o[dt][12], o[dt][13]), pack_bf16x2(o[dt][14], o[dt][15])};
  }
}

// Store a packed row of the partials at row pidx, lane half hf, with its
// (max, sum).  Both lane halves store the (max, sum) pair (the same value),
// so that every path issues the same memory operations.
__device__ __forceinline__ void store_row(const u32x4_t (&pv)[8], float2 ml, size_t pidx, int hf,
                                          uint16_t* __restrict__ part_o, float2* __restrict__ part_ml) {
  uint16_t* dst = part_o + pidx * kHeadDim + 64 * hf;
#pragma unroll
  for (int m = 0; m < 8; ++m) *reinterpret_cast<u32x4_t*>(dst + 8 * m) = pv[m];
  part_ml[pidx] = ml;
}

// ---------------------------------------------------------------------------
// Attention over the KV blocks of work items.  Persistent: one workgroup per
// CU walks a static list of items; while it computes item i, the K/V block
// of item i + 1 is staged into the second LDS buffer and the entries of item
// i + 2 into a wave-private LDS ring.
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

template <int BS>
__global__ __launch_bounds__(256, 1) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ item_ptr,
    const int2* __restrict__ items, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float2* __restrict__ part_ml, PrefillShape sh, PassInfo pass, int r_log2) {
  constexpr int KT = Tile<BS>::KT;
  extern __shared__ __align__(16) char lds[];  // two K/V buffers, then the entry rings

  // items of this pass, dealt round-robin: items are ordered by (unit,
  // block), so the whole chip works on one unit's queries at a time and
  // their gathered rows stay in the memory-side cache
  const int i_begin = item_ptr[pass.row_begin];
  const int it_end = item_ptr[pass.row_end] - i_begin;
  const int stride = gridDim.x;
  int it = blockIdx.x;
  if (it >= it_end) return;

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
  auto load_ents = [&](const ItemDesc& d, uint32_t (&e)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int jj = min(lane + 64 * m, ring - 1);
      const int tk = (jj / epw) * tpc + ((64 * w) >> r_log2) + jj % epw;
      e[m] = entries[d.e0 + min(tk, d.n_ent - 1)];
    }
  };
  auto store_ents = [&](int slot, const uint32_t (&e)[4]) {
#pragma unroll
    for (int m = 0; m < 4; ++m)
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
  ItemDesc cur = decode_at(it);
  ItemDesc nxt = decode_at(it + stride);
  ItemDesc nxt2 = decode_at(it + 2 * stride);
  int qn = 0;  // sequence number of the current item (entry ring slot qn % 3)
  {
    uint32_t e0r[4], e1r[4];
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
    const bool has_next = it + stride < it_end;
    // the next item's block and the entries of the item after it
    size_t nxt_off;
    const int nxt_keys = kv_src(nxt, &nxt_off);
    load_kv_regs<BS, 256>(k + nxt_off, v + nxt_off, nxt_keys, kv);
    uint32_t e2r[4];
    load_ents(nxt2, e2r);
    const uint16_t* nxt_qb = q_base(nxt.u);
    const int key0 = cur.j * BS;
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
        if (has_next) store_kv_lds<BS, 256>(kv, nxt_keys, lds + (buf ^ 1) * Tile<BS>::kLdsBytes);
        store_ents((qn + 2) % 3, e2r);
      }
      load_q(qb_nx, ent_nx, qf);

      size_t pidx[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) pidx[ct] = ((row0 + tok[ct]) * K + slot[ct]) * sh.r + head[ct];
      const bool own[2] = {((sh.q0 + tok[0]) >> sh.bs_log2) == cur.j, ((sh.q0 + tok[1]) >> sh.bs_log2) == cur.j};
      if (!__any(own[0] || own[1])) {
        // ---- no query of this chunk owns the block: plain softmax
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
          store_row(pv1, make_float2(m2[ct], wave_sum_pair(sum[ct])), pidx[ct], hf, part_o, part_ml);
        }
      } else {
        // ---- some query owns the block: causal mask on the own columns,
        // and P = hi + lo in bf16 there (~16 mantissa bits).  The other
        // columns take a zero low term and come out bit-identical to the
        // plain path.
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          // keys 0 .. tok - key0 are not after the query; the lane-half
          // term of the key index moves to the right-hand side so that
          // every compare is against a constant
          const int lim = sh.q0 + tok[ct] - key0 - 4 * hf;
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * kt + c_row(i, 0) > lim) s[kt][ct][i] = -__builtin_inff();
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          int vo = kvo;
          __asm__ volatile("" : "+v"(vo));
          const char* kvt = lds + vo;
          float mx = -__builtin_inff();
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][ct][i]);
          const float m2 = wave_max_pair(mx) * c2;
          const float lo_on = own[ct] ? 1.0f : 0.0f;  // arithmetic select: no divergent branch
          float sum = 0.f;
          f32x16_t o[4];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};
#pragma unroll
          for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              uint32_t dh[4], dl[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float p0 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e], c2, -m2));
                const float p1 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e + 1], c2, -m2));
                sum += p0 + p1;
                dh[e] = pack_bf16x2(p0, p1);
                dl[e] = pack_bf16x2((p0 - bf16_lo(dh[e])) * lo_on, (p1 - bf16_hi(dh[e])) * lo_on);
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
          const float l = wave_sum_pair(sum);
          // a row with no other partial (own block 0, or top_k = 1) stores
          // o / l with a sum of 1: the merge then reproduces it exactly, so
          // the row is rounded to bf16 once, as every other row
          const bool single = ((sh.q0 + tok[ct]) >> sh.bs_log2) == 0 || K == 1;
          // (its max then carries log2 l, so that the merge's log-sum-exp
          // is the row's)
          u32x4_t pv1[8];
          pack_tile(o, single ? 1.0f / l : 1.0f, pv1);
          store_row(pv1, make_float2(single ? m2 + fast_log2(l) : m2, single ? 1.0f : l), pidx[ct], hf, part_o,
                    part_ml);
        }
      }
      qb = qb_nx;
    }
    if (!has_next) break;
    // the other buffer is complete and every wave is done with this one
    __syncthreads();
    buf ^= 1;
    it += stride;
    ++qn;
    cur = nxt;
    nxt = nxt2;
    nxt2 = decode_at(it + 2 * stride);
  }
}

// ---------------------------------------------------------------------------
// Merge: 16 threads per query row, 8 stored values (16 bytes) each.  Every
// partial is read once, with a non-temporal hint (measured on MI355X: the
// merge 0.97 -> 0.86 ms per 16K-query chunk).
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s
// over the row's min(top_k - 1, own) + 1 partials (a row with a single
// partial holds o / l with a sum of 1, which the merge reproduces exactly).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(const uint16_t* __restrict__ part_o,
                                                    const float2* __restrict__ part_ml,
                                                    uint16_t* __restrict__ out, PrefillShape sh, PassInfo pass,
                                                    int t_first, int r_log2) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const int c16 = (int)(gid & 15);
  const long qr = gid >> 4;
  const int h = (int)(qr & (sh.r - 1));
  const int t = t_first + (int)(qr >> r_log2);
  if (t >= pass.t1) return;
  const int u = pass.u0 + (int)blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int K = sh.top_k;
  const int n = min(K - 1, (sh.q0 + t) >> sh.bs_log2) + 1;
  const size_t base = ((size_t)(u - pass.u0) * pass.pass_tokens + (t - pass.t0)) * K;

  float m[32], l[32];
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const f32x2_t ml = (s < n) ? __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(part_ml + (base + s) * sh.r + h))
                               : f32x2_t{-__builtin_inff(), 0.f};
    m[s] = ml.x;
    l[s] = ml.y;
    M = fmaxf(M, m[s]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
#pragma unroll
  for (int s0 = 0; s0 < 32; s0 += 8) {
    if (s0 >= n) break;
    u32x4_t val[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s0 + s < n)
        val[s] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(part_o + ((base + s0 + s) * sh.r + h) * kHeadDim + 8 * c16));
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s0 + s < n) {
        const float wgt = fast_exp2(m[s0 + s] - M);
        W = fmaf(wgt, l[s0 + s], W);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(wgt, bf16_lo(val[s][e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wgt, bf16_hi(val[s][e]), acc[2 * e + 1]);
        }
      }
    }
  }
  const float inv = 1.0f / W;
  if (sh.lse != nullptr && c16 == 0)
    sh.lse[((size_t)b * sh.q_stride + t) * sh.Hq + g * sh.r + h] = (M + fast_log2(W)) * 0.6931471805599453f;
  // stored positions 8 * c16 .. + 7 = lane half hf, tile dt, i0 .. i0 + 7
  const int p0 = 8 * c16;
  const int hfp = p0 >> 6, dt = (p0 >> 4) & 3, i0 = p0 & 15;
  const int d0 = 32 * dt + 8 * (i0 >> 2) + 4 * hfp;
  uint16_t* orow = out + (((size_t)b * sh.q_stride + t) * sh.Hq + g * sh.r + h) * kHeadDim;
  u32x2_t w0, w1;
  w0.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w0.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  w1.x = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  w1.y = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  // O is not read again by the prefill: non-temporal stores keep it from
  // lingering dirty in the caches (a decode right after a 32K prefill:
  // 48.5 -> 46.5 us on MI355X; the same hint on the partials, which the
  // merge reads back, made the prefill 3x slower)
  __builtin_nontemporal_store(w0, reinterpret_cast<u32x2_t*>(orow + d0));
  __builtin_nontemporal_store(w1, reinterpret_cast<u32x2_t*>(orow + d0 + 8));
}

template <int BS>
hipError_t launch_attend_bs(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr,
                            const int2* items, const uint32_t* entries, uint16_t* part_o, float2* part_ml,
                            int max_items, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  // one workgroup per CU, never more workgroups than items
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
  }
  if (max_items <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::max<long>(1, std::min<long>((long)n_cu, (long)max_items));
  // two K/V buffers and, per wave, a ring of three items' entries
  const int lds_bytes = 2 * Tile<BS>::kLdsBytes + 4 * 3 * kItemChunks * (64 >> r_log2) * 4;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_kernel<BS>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     2 * Tile<BS>::kLdsBytes + 4 * 3 * kItemChunks * 64 * 4);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(attend_kernel<BS>, dim3(grid), dim3(256), lds_bytes, st, q, k, v, row_ptr, item_ptr, items,
                     entries, part_o, part_ml, sh, pass, r_log2);
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

  // O = o / l, head dims 32 dt + 8 q4 + 4 hf + 0..3 of this lane's row
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    if (tok[ct] >= sh.S) continue;
    const float inv = 1.0f / l[ct];
    if (sh.lse != nullptr && hf == 0)
      sh.lse[((size_t)b * sh.q_stride + tok[ct]) * sh.Hq + g * sh.r + head[ct]] =
          (m[ct] + fast_log2(l[ct])) * 0.6931471805599453f;
    uint16_t* orow = out + (((size_t)b * sh.q_stride + tok[ct]) * sh.Hq + g * sh.r + head[ct]) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2_t wv;
        wv.x = pack_bf16x2(o[ct][dt][4 * q4 + 0] * inv, o[ct][dt][4 * q4 + 1] * inv);
        wv.y = pack_bf16x2(o[ct][dt][4 * q4 + 2] * inv, o[ct][dt][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * q4 + 4 * hf) = wv;
      }
  }
}

// sel of a dense prefill: every block up to the own one, ascending, then -1.
__global__ __launch_bounds__(256) void dense_sel_kernel(int32_t* __restrict__ sel, int units, int S, int bs_log2,
                                                        int top_k) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)units * S * top_k) return;
  const int s = (int)(i % top_k);
  const int t = (int)((i / top_k) % S);
  sel[i] = s <= (t >> bs_log2) ? s : -1;
}

}  // namespace

hipError_t launch_attend(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr, const int2* items,
                         const uint32_t* entries, uint16_t* part_o, float2* part_ml, int max_items, hipStream_t st) {
  switch (sh.bs) {
    case 32:
      return launch_attend_bs<32>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_ml, max_items,
                                  st);
    case 64:
      return launch_attend_bs<64>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_ml, max_items,
                                  st);
    default:
      return launch_attend_bs<128>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_ml, max_items,
                                   st);
  }
}

hipError_t launch_merge(const PrefillShape& sh, const PassInfo& pass, const uint16_t* part_o,
                        const float2* part_ml, uint16_t* out, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  const int t_first = pass.t0;
  if (t_first >= pass.t1) return hipSuccess;
  const long threads = (long)(pass.t1 - t_first) * sh.r * 16;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((threads + 255) / 256), pass.u1 - pass.u0), dim3(256), 0, st,
                     part_o, part_ml, out, sh, pass, t_first, r_log2);
  return hipGetLastError();
}


hipError_t launch_dense(const PrefillShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        uint16_t* out, int32_t* sel, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  const int tpt = kItemRows >> r_log2;
  const dim3 grid((unsigned)((sh.S + tpt - 1) / tpt), (unsigned)(sh.B * sh.G));
  switch (sh.bs) {
#define MSA_DENSE_LAUNCH(BS_, NCT_)                                                                          \
  {                                                                                                           \
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&dense_kernel<BS_, NCT_>), \
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,           \
                                                       2 * Tile<BS_>::kLdsBytes);                             \
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
                     sh.bs_log2, sh.top_k);
  return hipGetLastError();
}

}  // namespace msa
