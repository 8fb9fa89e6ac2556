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
// Two kernels share the MFMA tile code:
//   offdiag_kernel   one work item = one KV block j of one (batch, group) unit
//                    and up to 256 query rows (tokens x heads) whose selection
//                    holds j before their own block; K_j and V_j^T go through
//                    LDS once, the rows are gathered from HBM, and every row
//                    leaves a normalised bf16 partial plus its base-2
//                    log-sum-exp.
//   diag_merge_kernel one workgroup = one query block of one unit: causal
//                    attention of the block's tokens on their own block (P
//                    split into two bf16 terms so P.V keeps ~16 mantissa bits:
//                    the first tokens of a sequence see only a few keys), then
//                    the log-sum-exp merge of the off-diagonal partials -> out.
//
// Tile shapes (wave64, v_mfma_f32_32x32x16_bf16):
//   S^T = K Q^T : 32 keys x 32 query rows per tile, K from LDS (A operand),
//                 Q rows straight from HBM into registers (B operand).
//   O^T = V^T P^T : 32 head dims x 32 query rows per tile, V^T from LDS (A),
//                 P^T from the S^T accumulators (B).  A lane holds the keys
//                 8 * (i / 4) + 4 * (lane / 32) + i % 4 of its column, so the
//                 V^T reads pick those keys in the same order.

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
// transposed (head dim major).  256 threads.
template <int BS>
__device__ __forceinline__ void load_kv_lds(const uint16_t* __restrict__ kblk,
                                            const uint16_t* __restrict__ vblk, int n_keys,
                                            char* __restrict__ lds) {
  using T = Tile<BS>;
  const int tid = threadIdx.x;
  // K: 16-byte chunks, 16 per key row
#pragma unroll
  for (int m = 0; m < BS / 16; ++m) {
    const int qid = tid + 256 * m;
    const int key = qid >> 4;
    const int c = qid & 15;
    u32x4_t val = {0u, 0u, 0u, 0u};
    if (key < n_keys) val = *reinterpret_cast<const u32x4_t*>(kblk + key * kHeadDim + c * 8);
    *reinterpret_cast<u32x4_t*>(lds + key * kKStride + c * 16) = val;
  }
  // V^T: a thread takes keys (2p, 2p + 1) x 8 head dims and writes 8 dwords
  char* vt = lds + T::kKBytes;
#pragma unroll
  for (int m = 0; m < BS / 32; ++m) {
    const int qid = tid + 256 * m;
    const int p = qid % (BS / 2);
    const int c = qid / (BS / 2);
    u32x4_t a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (2 * p < n_keys) a = *reinterpret_cast<const u32x4_t*>(vblk + (2 * p) * kHeadDim + c * 8);
    if (2 * p + 1 < n_keys) b = *reinterpret_cast<const u32x4_t*>(vblk + (2 * p + 1) * kHeadDim + c * 8);
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

// ---------------------------------------------------------------------------
// Off-diagonal work items.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256, 2) void offdiag_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ item_ptr,
    const int2* __restrict__ items, const uint32_t* __restrict__ entries,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, PrefillShape sh, int u0, int u1,
    int r_log2) {
  using T = Tile<BS>;
  constexpr int KT = T::KT;
  extern __shared__ __align__(16) char lds[];

  // items of this pass, spread so that each XCD takes a contiguous range
  const int i_begin = item_ptr[u0 * sh.nb];
  const int n_items = item_ptr[u1 * sh.nb] - i_begin;
  const int per_xcd = (n_items + 7) >> 3;
  const int bid = blockIdx.x;
  const int slot_in_xcd = bid >> 3;
  const int it = (bid & 7) * per_xcd + slot_in_xcd;
  if (slot_in_xcd >= per_xcd || it >= n_items) return;

  const int2 item = items[i_begin + it];
  const int bi = item.x;
  const int u = bi / sh.nb;
  const int j = bi - u * sh.nb;
  const int e0 = row_ptr[bi] + item.y;
  const int n_tok = min(kItemRows >> r_log2, row_ptr[bi + 1] - e0);
  const int b = u / sh.G;
  const int g = u - b * sh.G;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const int kp = sh.top_k - 1;

  // gather this lane's two query rows (column tiles ct = 0, 1)
  u32x4_t qf[2][8];
  int tok[2], slot[2], head[2];
  bool live[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int qr = 64 * w + 32 * ct + (lane & 31);
    const int tk = qr >> r_log2;
    live[ct] = tk < n_tok;
    const uint32_t ent = entries[e0 + (live[ct] ? tk : 0)];
    tok[ct] = (int)(ent >> 5);
    slot[ct] = (int)(ent & 31u);
    head[ct] = qr & (sh.r - 1);
    const uint16_t* qrow = q + (((size_t)b * sh.S + tok[ct]) * sh.Hq + g * sh.r + head[ct]) * kHeadDim;
    load_q_frag(qrow, hf, qf[ct]);
  }

  const size_t kv_off = ((size_t)u * sh.S + (size_t)j * BS) * kHeadDim;
  load_kv_lds<BS>(k + kv_off, v + kv_off, BS, lds);
  __syncthreads();

  // waves whose rows are all past the item's end have nothing to do
  if (64 * w >= (n_tok << r_log2)) return;

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

  // softmax statistics per column (query row); every key of the block is
  // before the query, so nothing is masked
  const float c2 = sh.scale_log2;
  float m2[2], l[2];
  u32x4_t pk[2][KT][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    float mx = s[0][ct][0];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][ct][i]);
    mx = wave_max_pair(mx);
    m2[ct] = mx * c2;
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint32_t d[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e], c2, -m2[ct]));
          const float p1 = fast_exp2(fmaf(s[kt][ct][8 * h2 + 2 * e + 1], c2, -m2[ct]));
          d[e] = pack_bf16x2(p0, p1);
          sum += bf16_lo(d[e]) + bf16_hi(d[e]);  // normalise with the rounded weights
        }
        pk[ct][kt][h2] = u32x4_t{d[0], d[1], d[2], d[3]};
      }
    }
    l[ct] = wave_sum_pair(sum);
  }

  // O^T = V^T P^T
  f32x16_t o[4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    o[dt][0] = f32x16_t{};
    o[dt][1] = f32x16_t{};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const u32x4_t a = vt_frag<BS>(lds, dt, kt, h2, lane);
        o[dt][0] = mfma32x32x16(a, pk[0][kt][h2], o[dt][0]);
        o[dt][1] = mfma32x32x16(a, pk[1][kt][h2], o[dt][1]);
      }
  }

  // partial rows: 128 bf16 stored lane-half-major (this lane's 64 values
  // contiguous), and the base-2 log-sum-exp
  const int units_off = u - u0;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    if (!live[ct]) continue;
    const size_t pidx = (((size_t)units_off * sh.S + tok[ct]) * kp + slot[ct]) * sh.r + head[ct];
    const float inv = 1.0f / l[ct];
    uint16_t* dst = part_o + pidx * kHeadDim + 64 * hf;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      u32x4_t w0, w1;
      w0.x = pack_bf16x2(o[dt][ct][0] * inv, o[dt][ct][1] * inv);
      w0.y = pack_bf16x2(o[dt][ct][2] * inv, o[dt][ct][3] * inv);
      w0.z = pack_bf16x2(o[dt][ct][4] * inv, o[dt][ct][5] * inv);
      w0.w = pack_bf16x2(o[dt][ct][6] * inv, o[dt][ct][7] * inv);
      w1.x = pack_bf16x2(o[dt][ct][8] * inv, o[dt][ct][9] * inv);
      w1.y = pack_bf16x2(o[dt][ct][10] * inv, o[dt][ct][11] * inv);
      w1.z = pack_bf16x2(o[dt][ct][12] * inv, o[dt][ct][13] * inv);
      w1.w = pack_bf16x2(o[dt][ct][14] * inv, o[dt][ct][15] * inv);
      *reinterpret_cast<u32x4_t*>(dst + 16 * dt) = w0;
      *reinterpret_cast<u32x4_t*>(dst + 16 * dt + 8) = w1;
    }
    if (hf == 0) part_lse[pidx] = m2[ct] + fast_log2(l[ct]);
  }
}

// ---------------------------------------------------------------------------
// Own block + merge.
// ---------------------------------------------------------------------------
template <int BS>
__global__ __launch_bounds__(256, 2) void diag_merge_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
    uint16_t* __restrict__ out, PrefillShape sh, int u0, int r_log2) {
  constexpr int KT = Tile<BS>::KT;
  extern __shared__ __align__(16) char lds[];

  const int qb = blockIdx.x;
  const int u = u0 + (int)blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int t0 = qb * BS;
  const int n_tokb = min(BS, sh.S - t0);
  const int kp = sh.top_k - 1;
  const int n_off = min(kp, qb);  // off-diagonal partials of every token here

  const size_t kv_off = ((size_t)u * sh.S + t0) * kHeadDim;
  load_kv_lds<BS>(k + kv_off, v + kv_off, n_tokb, lds);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hf = lane >> 5;
  const float c2 = sh.scale_log2;
  const int n_rows = n_tokb << r_log2;

  for (int ti = w; 32 * ti < n_rows; ti += 4) {
    // keep the LDS fragment reads inside the loop (hoisting them all out
    // would need ~256 registers)
    __asm__ volatile("" ::: "memory");
    const int qr = 32 * ti + (lane & 31);
    const bool live = qr < n_rows;
    const int tk = live ? (qr >> r_log2) : n_tokb - 1;
    const int h = qr & (sh.r - 1);
    const int t = t0 + tk;
    const uint16_t* qrow = q + (((size_t)b * sh.S + t) * sh.Hq + g * sh.r + h) * kHeadDim;
    u32x4_t qf[8];
    load_q_frag(qrow, hf, qf);

    f32x16_t s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s[kt] = mfma32x32x16(k_frag(lds, kt, ks, lane), qf[ks], s[kt]);
    }

    // causal mask: key position (within the block) <= token position
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kt + c_row(i, hf);
        if (key <= tk) mx = fmaxf(mx, s[kt][i]);
      }
    mx = wave_max_pair(mx);
    const float m2 = mx * c2;
    // P in two bf16 terms (hi + lo) per key tile, consumed at once by P.V
    float sum = 0.f;
    f32x16_t o[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        uint32_t dh[4], dl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i0 = 8 * h2 + 2 * e;
          const int key0 = 32 * kt + c_row(i0, hf);
          const int key1 = 32 * kt + c_row(i0 + 1, hf);
          const float p0 = key0 <= tk ? fast_exp2(fmaf(s[kt][i0], c2, -m2)) : 0.f;
          const float p1 = key1 <= tk ? fast_exp2(fmaf(s[kt][i0 + 1], c2, -m2)) : 0.f;
          dh[e] = pack_bf16x2(p0, p1);
          const float r0 = p0 - bf16_lo(dh[e]);
          const float r1 = p1 - bf16_hi(dh[e]);
          dl[e] = pack_bf16x2(r0, r1);
          sum += (bf16_lo(dh[e]) + bf16_lo(dl[e])) + (bf16_hi(dh[e]) + bf16_hi(dl[e]));
        }
        const u32x4_t phi = u32x4_t{dh[0], dh[1], dh[2], dh[3]};
        const u32x4_t plo = u32x4_t{dl[0], dl[1], dl[2], dl[3]};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const u32x4_t a = vt_frag<BS>(lds, dt, kt, h2, lane);
          o[dt] = mfma32x32x16(a, phi, o[dt]);
          o[dt] = mfma32x32x16(a, plo, o[dt]);
        }
      }
    }
    const float l = wave_sum_pair(sum);

    // merge: out = sum_s 2^(lse_s - M) o_s / sum_s 2^(lse_s - M), own block
    // included with lse = m2 + log2(l) and o = acc / l
    const float lse_own = m2 + fast_log2(l);
    const size_t prow = ((size_t)(u - u0) * sh.S + t) * kp;
    float M = lse_own;
    for (int sl = 0; sl < n_off; ++sl) M = fmaxf(M, part_lse[(prow + sl) * sh.r + h]);
    const float w_own = fast_exp2(lse_own - M);
    float W = w_own;
    const float f_own = w_own / l;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[dt][i] *= f_own;
#pragma unroll 2
    for (int sl = 0; sl < n_off; ++sl) {
      const size_t pidx = (prow + sl) * sh.r + h;
      const float ws = fast_exp2(part_lse[pidx] - M);
      W += ws;
      const uint16_t* src = part_o + pidx * kHeadDim + 64 * hf;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x4_t w0 = *reinterpret_cast<const u32x4_t*>(src + 16 * dt);
        const u32x4_t w1 = *reinterpret_cast<const u32x4_t*>(src + 16 * dt + 8);
        o[dt][0] = fmaf(ws, bf16_lo(w0.x), o[dt][0]);
        o[dt][1] = fmaf(ws, bf16_hi(w0.x), o[dt][1]);
        o[dt][2] = fmaf(ws, bf16_lo(w0.y), o[dt][2]);
        o[dt][3] = fmaf(ws, bf16_hi(w0.y), o[dt][3]);
        o[dt][4] = fmaf(ws, bf16_lo(w0.z), o[dt][4]);
        o[dt][5] = fmaf(ws, bf16_hi(w0.z), o[dt][5]);
        o[dt][6] = fmaf(ws, bf16_lo(w0.w), o[dt][6]);
        o[dt][7] = fmaf(ws, bf16_hi(w0.w), o[dt][7]);
        o[dt][8] = fmaf(ws, bf16_lo(w1.x), o[dt][8]);
        o[dt][9] = fmaf(ws, bf16_hi(w1.x), o[dt][9]);
        o[dt][10] = fmaf(ws, bf16_lo(w1.y), o[dt][10]);
        o[dt][11] = fmaf(ws, bf16_hi(w1.y), o[dt][11]);
        o[dt][12] = fmaf(ws, bf16_lo(w1.z), o[dt][12]);
        o[dt][13] = fmaf(ws, bf16_hi(w1.z), o[dt][13]);
        o[dt][14] = fmaf(ws, bf16_lo(w1.w), o[dt][14]);
        o[dt][15] = fmaf(ws, bf16_hi(w1.w), o[dt][15]);
      }
    }
    if (!live) continue;
    const float invW = 1.0f / W;
    uint16_t* orow = out + (((size_t)b * sh.S + t) * sh.Hq + g * sh.r + h) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        u32x2_t wv;
        wv.x = pack_bf16x2(o[dt][4 * q4 + 0] * invW, o[dt][4 * q4 + 1] * invW);
        wv.y = pack_bf16x2(o[dt][4 * q4 + 2] * invW, o[dt][4 * q4 + 3] * invW);
        *reinterpret_cast<u32x2_t*>(orow + 32 * dt + 8 * q4 + 4 * hf) = wv;
      }
  }
}

template <int BS>
hipError_t launch_offdiag_bs(const PrefillShape& sh, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr,
                             const int2* items, const uint32_t* entries, uint16_t* part_o,
                             float* part_lse, int u0, int u1, int max_items, hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  const unsigned grid = (unsigned)(((long)max_items + 7) / 8 * 8);
  if (grid == 0) return hipSuccess;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&offdiag_kernel<BS>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Tile<BS>::kLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(offdiag_kernel<BS>, dim3(grid), dim3(256), Tile<BS>::kLdsBytes, st, q, k, v, row_ptr,
                     item_ptr, items, entries, part_o, part_lse, sh, u0, u1, r_log2);
  return hipGetLastError();
}

template <int BS>
hipError_t launch_diag_bs(const PrefillShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const uint16_t* part_o, const float* part_lse, uint16_t* out, int u0, int u1,
                          hipStream_t st) {
  int r_log2 = 0;
  while ((1 << r_log2) < sh.r) ++r_log2;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&diag_merge_kernel<BS>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     Tile<BS>::kLdsBytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(diag_merge_kernel<BS>, dim3(sh.nb, u1 - u0), dim3(256), Tile<BS>::kLdsBytes, st, q, k, v,
                     part_o, part_lse, out, sh, u0, r_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_main_offdiag(const PrefillShape& sh, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* row_ptr, const int32_t* item_ptr,
                               const int2* items, const uint32_t* entries, uint16_t* part_o,
                               float* part_lse, int u0, int u1, int max_items, hipStream_t st) {
  switch (sh.bs) {
    case 32:
      return launch_offdiag_bs<32>(sh, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_lse, u0, u1,
                                   max_items, st);
    case 64:
      return launch_offdiag_bs<64>(sh, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_lse, u0, u1,
                                   max_items, st);
    default:
      return launch_offdiag_bs<128>(sh, q, k, v, row_ptr, item_ptr, items, entries, part_o, part_lse, u0, u1,
                                    max_items, st);
  }
}

hipError_t launch_diag_merge(const PrefillShape& sh, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const uint16_t* part_o, const float* part_lse,
                             uint16_t* out, int u0, int u1, hipStream_t st) {
  switch (sh.bs) {
    case 32:
      return launch_diag_bs<32>(sh, q, k, v, part_o, part_lse, out, u0, u1, st);
    case 64:
      return launch_diag_bs<64>(sh, q, k, v, part_o, part_lse, out, u0, u1, st);
    default:
      return launch_diag_bs<128>(sh, q, k, v, part_o, part_lse, out, u0, u1, st);
  }
}

}  // namespace msa
