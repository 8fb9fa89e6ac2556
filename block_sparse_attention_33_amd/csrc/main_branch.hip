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
//                  and up to 4 chunks of the query rows (tokens x heads) whose
//                  selection holds j, the query's own block included.  K_j
//                  and V_j^T go through LDS once per item; four waves take 64
//                  gathered query rows of every chunk, two workgroups share a
//                  CU so one's gathers overlap the other's MFMAs.  Every row
//                  leaves a normalised bf16 partial and its base-2
//                  log-sum-exp at its selection slot; rows whose own block is
//                  block 0 (they attend nothing else) are written to the
//                  output directly.  Chunks holding a query's own block apply
//                  the causal mask and split P into two bf16 terms, so P.V
//                  keeps ~16 mantissa bits for the first tokens of a sequence,
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

// Copy K rows [0, n_keys) of a block into LDS (zero beyond n_keys) and V
// transposed (head dim major), with NT threads.
template <int BS, int NT>
__device__ __forceinline__ void load_kv_lds(const uint16_t* __restrict__ kblk,
                                            const uint16_t* __restrict__ vblk, int n_keys,
                                            char* __restrict__ lds) {
  using T = Tile<BS>;
  const int tid = threadIdx.x;
  // K: 16-byte chunks, 16 per key row
#pragma unroll
  for (int m = 0; m < BS * 16 / NT; ++m) {
    const int qid = tid + NT * m;
    const int key = qid >> 4;
    const int c = qid & 15;
    // unconditional (clamped) loads, so that all of them are in flight at once
    u32x4_t val = *reinterpret_cast<const u32x4_t*>(kblk + min(key, n_keys - 1) * kHeadDim + c * 8);
    if (key >= n_keys) val = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(lds + key * kKStride + c * 16) = val;
  }
  // V^T: a thread takes keys (2p, 2p + 1) x 8 head dims and writes 8 dwords
  char* vt = lds + T::kKBytes;
#pragma unroll
  for (int m = 0; m < BS * 8 / NT; ++m) {
    const int qid = tid + NT * m;
    const int p = qid % (BS / 2);
    const int c = qid / (BS / 2);
    u32x4_t a = *reinterpret_cast<const u32x4_t*>(vblk + min(2 * p, n_keys - 1) * kHeadDim + c * 8);
    u32x4_t b = *reinterpret_cast<const u32x4_t*>(vblk + min(2 * p + 1, n_keys - 1) * kHeadDim + c * 8);
    if (2 * p >= n_keys) a = u32x4_t{0u, 0u, 0u, 0u};
    if (2 * p + 1 >= n_keys) b = u32x4_t{0u, 0u, 0u, 0u};
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

// One column tile's rows: rows whose own block is block 0 attend nothing else
// and are written to the output; every other row leaves its partial (lane-
// half-major bf16) and base-2 log-sum-exp at (token, slot, head).
__device__ __forceinline__ void store_rows(const f32x16_t (&o)[4], float m2, float l, bool live, int tok,
                                           int slot, int head, int hf, int b, int g, int K, size_t pass_row0,
                                           const PrefillShape& sh, uint16_t* __restrict__ part_o,
                                           float* __restrict__ part_lse, uint16_t* __restrict__ out) {
  if (!live) return;
  const float inv = 1.0f / l;
  if ((tok >> sh.bs_log2) == 0) {
    uint16_t* orow = out + (((size_t)b * sh.S + tok) * sh.Hq + g * sh.r + head) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2_t wv;
        wv.x = pack_bf16x2(o[dt][4 * q4 + 0] * inv, o[dt][4 * q4 + 1] * inv);
        wv.y = pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * q4 + 4 * hf) = wv;
      }
    return;
  }
  const size_t pidx = ((pass_row0 + tok) * K + slot) * sh.r + head;
  uint16_t* dst = part_o + pidx * kHeadDim + 64 * hf;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    u32x4_t w0, w1;
    w0.x = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
    w0.y = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
    w0.z = pack_bf16x2(o[dt][4] * inv, o[dt][5] * inv);
    w0.w = pack_bf16x2(o[dt][6] * inv, o[dt][7] * inv);
    w1.x = pack_bf16x2(o[dt][8] * inv, o[dt][9] * inv);
    w1.y = pack_bf16x2(o[dt][10] * inv, o[dt][11] * inv);
    w1.z = pack_bf16x2(o[dt][12] * inv, o[dt][13] * inv);
    w1.w = pack_bf16x2(o[dt][14] * inv, o[dt][15] * inv);
    *reinterpret_cast<u32x4_t*>(dst + 16 * dt) = w0;
    *reinterpret_cast<u32x4_t*>(dst + 16 * dt + 8) = w1;
  }
  if (hf == 0) part_lse[pidx] = m2 + fast_log2(l);
}

// ---------------------------------------------------------------------------
// Attention over one KV block for the gathered query rows of a work item.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256, 2) void attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ item_ptr,
    const int2* __restrict__ items, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, uint16_t* __restrict__ out,
    PrefillShape sh, PassInfo pass, int r_log2) {
  constexpr int KT = Tile<BS>::KT;
  extern __shared__ __align__(16) char lds[];

  // items of this pass, spread so that each XCD takes a contiguous range
  const int i_begin = item_ptr[pass.row_begin];
  const int n_items = item_ptr[pass.row_end] - i_begin;
  const int per_xcd = (n_items + 7) >> 3;
  const int bid = blockIdx.x;
  const int slot_in_xcd = bid >> 3;
  const int it = (bid & 7) * per_xcd + slot_in_xcd;
  if (slot_in_xcd >= per_xcd || it >= n_items) return;

  const int2 item = items[i_begin + it];
  const int bi = item.x;  // CSR row (unit, range, block)
  const int u = bi / (sh.n_ranges * sh.nb);
  const int j = bi % sh.nb;
  const int e0 = row_ptr[bi] + item.y;
  const int tpc = kItemRows >> r_log2;  // tokens per chunk
  const int n_ent = min(kItemChunks * tpc, row_ptr[bi + 1] - e0);
  const int n_chunks = (n_ent + tpc - 1) / tpc;
  const int b = u / sh.G;
  const int g = u - b * sh.G;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;  // rows 64 w .. 64 w + 63 of every chunk
  const int hf = lane >> 5;
  const int K = sh.top_k;
  const float c2 = sh.scale_log2;
  const int key0 = j * BS;
  const size_t pass_row0 = (size_t)(u - pass.u0) * pass.pass_tokens - pass.t0;
  const uint16_t* qbase = q + ((size_t)b * sh.S * sh.Hq + g * sh.r) * kHeadDim;

  // entries of chunk c (clamped: always a valid entry, no branch)
  auto entry_of = [&](int c, int ct) -> uint32_t {
    const int tk = c * tpc + ((64 * w + 32 * ct + (lane & 31)) >> r_log2);
    return entries[e0 + min(tk, n_ent - 1)];
  };
  uint32_t ent[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) ent[ct] = entry_of(0, ct);

  const size_t kv_off = ((size_t)u * sh.S + (size_t)j * BS) * kHeadDim;
  load_kv_lds<BS, 256>(k + kv_off, v + kv_off, min(BS, sh.S - j * BS), lds);
  __syncthreads();

  for (int c = 0; c < n_chunks; ++c) {
    // keep the LDS fragment reads inside the loop (hoisted they would need
    // far more registers than a wave has)
    __asm__ volatile("" ::: "memory");
    int tok[2], slot[2], head[2];
    bool live[2];
    u32x4_t qf[2][8];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int qr = 64 * w + 32 * ct + (lane & 31);
      live[ct] = c * tpc + (qr >> r_log2) < n_ent;
      tok[ct] = (int)(ent[ct] >> 5);
      slot[ct] = (int)(ent[ct] & 31u);
      head[ct] = qr & (sh.r - 1);
      load_q_frag(qbase + ((size_t)tok[ct] * sh.Hq + head[ct]) * kHeadDim, hf, qf[ct]);
    }
    // the next chunk's entries are in flight during this chunk
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) ent[ct] = entry_of(c + 1, ct);
    // waves whose rows are all past the item's end skip the math
    const bool wave_live = c * tpc + ((64 * w) >> r_log2) < n_ent;

    if (wave_live) {
    // S^T = K Q^T
    f32x16_t s[KT][2];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt][0] = f32x16_t{};
      s[kt][1] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4_t a = k_frag(lds, kt, ks, lane);
        s[kt][0] = mfma32x32x16(a, qf[0][ks], s[kt][0]);
        s[kt][1] = mfma32x32x16(a, qf[1][ks], s[kt][1]);
      }
    }

    // a chunk holding some query's own block: causal mask + two-term P
    const bool own[2] = {(tok[0] >> sh.bs_log2) == j, (tok[1] >> sh.bs_log2) == j};
    const bool diag = __any(own[0] || own[1]);
    if (diag) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        // keys 0 .. tok - key0 are not after the query; the lane-half term of
        // the key index moves to the right-hand side so that every compare
        // is against a constant
        const int lim = tok[ct] - key0 - 4 * hf;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * kt + c_row(i, 0) > lim) s[kt][ct][i] = -__builtin_inff();
      }
    }
    float m2[2], sum[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][ct][i]);
      m2[ct] = wave_max_pair(mx) * c2;
      sum[ct] = 0.f;
    }

    // O^T = V^T P^T one column tile at a time (32 accumulator registers
    // less than both at once), then the tile's partials (or final values).
    // A column whose own block this is gets P = hi + lo in bf16; the other
    // columns add a zero low term and round exactly as outside such chunks.
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
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
            const float p0 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e], c2, -m2[ct]));
            const float p1 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e + 1], c2, -m2[ct]));
            dh[e] = pack_bf16x2(p0, p1);
            if (diag) {
              dl[e] = own[ct] ? pack_bf16x2(p0 - bf16_lo(dh[e]), p1 - bf16_hi(dh[e])) : 0u;
              sum[ct] += (bf16_lo(dh[e]) + bf16_lo(dl[e])) + (bf16_hi(dh[e]) + bf16_hi(dl[e]));
            } else {
              sum[ct] += bf16_lo(dh[e]) + bf16_hi(dh[e]);  // normalise with the rounded weights
            }
          }
          const u32x4_t ph = u32x4_t{dh[0], dh[1], dh[2], dh[3]};
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const u32x4_t a = vt_frag<BS>(lds, dt, kt, h2, lane);
            o[dt] = mfma32x32x16(a, ph, o[dt]);
            if (diag) o[dt] = mfma32x32x16(a, u32x4_t{dl[0], dl[1], dl[2], dl[3]}, o[dt]);
          }
        }
      store_rows(o, m2[ct], wave_sum_pair(sum[ct]), live[ct], tok[ct], slot[ct], head[ct], hf, b, g, K,
                 pass_row0, sh, part_o, part_lse, out);
    }
    }  // wave_live
  }
}

// ---------------------------------------------------------------------------
// Merge: 16 threads per query row, 8 stored values (16 bytes) each.
//   out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M)
// over the row's min(top_k - 1, own) + 1 partials.  Rows of block 0 were
// finished by the attention kernel.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void merge_kernel(const uint16_t* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
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
  const int n = min(K - 1, t >> sh.bs_log2) + 1;
  const size_t base = ((size_t)(u - pass.u0) * pass.pass_tokens + (t - pass.t0)) * K;

  float lse[32];
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    lse[s] = (s < n) ? part_lse[(base + s) * sh.r + h] : -__builtin_inff();
    M = fmaxf(M, lse[s]);
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
        val[s] = *reinterpret_cast<const u32x4_t*>(part_o + ((base + s0 + s) * sh.r + h) * kHeadDim + 8 * c16);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s0 + s < n) {
        const float wgt = fast_exp2(lse[s0 + s] - M);
        W += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(wgt, bf16_lo(val[s][e]), acc[2 * e]);
          acc[2 * e + 1] = fmaf(wgt, bf16_hi(val[s][e]), acc[2 * e + 1]);
        }
      }
    }
  }
  const float inv = 1.0f / W;
  // stored positions 8 * c16 .. + 7 = lane half hf, tile dt, i0 .. i0 + 7
  const int p0 = 8 * c16;
  const int hfp = p0 >> 6, dt = (p0 >> 4) & 3, i0 = p0 & 15;
  const int d0 = 32 * dt + 8 * (i0 >> 2) + 4 * hfp;
  uint16_t* orow = out + (((size_t)b * sh.S + t) * sh.Hq + g * sh.r + h) * kHeadDim;
  u32x2_t w0, w1;
  w0.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  w0.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  w1.x = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  w1.y = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<u32x2_t*>(orow + d0) = w0;
  *reinterpret_cast<u32x2_t*>(orow + d0 + 8) = w1;
}

template <int BS>
hipError_t launch_attend_bs(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                            const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr,
                            const int2* items, const uint32_t* entries, uint16_t* part_o, float* part_lse,
                            uint16_t* out, int max_items, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  const unsigned grid = (unsigned)(((long)max_items + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&attend_kernel<BS>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Tile<BS>::kLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(attend_kernel<BS>, dim3(grid), dim3(256), Tile<BS>::kLdsBytes, st, q, k, v, row_ptr,
                     item_ptr, items, entries, part_o, part_lse, out, sh, pass, r_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const PrefillShape& sh, const PassInfo& pass, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr, const int2* items,
                         const uint32_t* entries, uint16_t* part_o, float* part_lse, uint16_t* out,
                         int max_items, hipStream_t st) {
  switch (sh.bs) {
    case 32:
      return launch_attend_bs<32>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_lse, out,
                                  max_items, st);
    case 64:
      return launch_attend_bs<64>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_lse, out,
                                  max_items, st);
    default:
      return launch_attend_bs<128>(sh, pass, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_lse, out,
                                   max_items, st);
  }
}

hipError_t launch_merge(const PrefillShape& sh, const PassInfo& pass, const uint16_t* part_o,
                        const float* part_lse, uint16_t* out, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  const int t_first = max(pass.t0, sh.bs);  // rows of block 0 are already final
  if (t_first >= pass.t1) return hipSuccess;
  const long threads = (long)(pass.t1 - t_first) * sh.r * 16;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((threads + 255) / 256), pass.u1 - pass.u0), dim3(256), 0, st,
                     part_o, part_lse, out, sh, pass, t_first, r_log2);
  return hipGetLastError();
}

}  // namespace msa
