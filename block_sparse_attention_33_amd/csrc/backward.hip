// MSA main branch, backward: gradients of the attention output with respect
// to q, k and v, the block selection held fixed.
//
// The index branch is integer arithmetic and carries no gradient; the pages
// report trained MSA models (wiki.500nian.com digest of "MiniMax M3 Review",
// the ablation paragraph; devpress.csdn.net article, section
// "M3的技术局限与改进方向", third limitation, on the training cost) but print no
// backward, so this is the chain rule of the forward -- one softmax over the
// attended keys of the kept blocks -- with P rebuilt from the forward's
// log-sum-exp.  The loop order is the forward's: the KV block outside, the
// query rows that selected it gathered inward (yunpan.plus article on
// MiniMax M3, the paragraph on the operator level), which is also the order
// that lets dK and dV of a block stay in registers until the block is done.
//
//   bwd_delta_kernel  delta[row] = sum_d dO[row][d] O[row][d] in fp32.
//   bwd_kv_kernel     one workgroup per CSR row (unit, KV block j), the
//                     block's keys split over BS / 32 waves of 32 keys (K and
//                     V rows of a wave's keys held in registers; dK^T and
//                     dV^T accumulated there over every gathered row).  Per
//                     chunk of 64 (128-key blocks) or 32 gathered query rows
//                     (tokens x heads of the group), staged in LDS as rows
//                     and as transposes:
//                       S = Q K^T, P = exp2(S c2 - lse2) (0 past the query),
//                       dP = dO V^T, dS = P (dP - delta),
//                       dV^T += dO^T P, dK^T += Q^T dS;
//                     dS then goes through LDS and every wave forms
//                     dQ^T = K^T dS^T for its share of the head dims, stored
//                     as one bf16 partial per (query row, selection slot).
//   bwd_dq_kernel     dq = scale * sum of a query row's partials.
//
// MFMA shapes (v_mfma_f32_32x32x16_bf16, wave64): in the contraction over
// query rows, operand element e of a lane in half hf stands for row
// 32 rt + 16 h2 + 8 (e / 4) + 4 hf + e % 4 at k-step h2 of row tile rt -- the
// rows that the S / dP accumulators of tile rt hold in their elements
// 8 h2 .. 8 h2 + 7 -- so P and dS feed the next products straight from
// registers, and the Q^T / dO^T reads pick the same rows.

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

constexpr int kNatStride = 2 * kHeadDim + 16;  // bytes per row of Q / dO / the dq tile in LDS

// Gathered query rows per chunk: 64 for 128-key blocks (half the barriers
// and row bookkeeping per row; measured 6 % faster than 32 on MI355X), 32
// for smaller blocks, whose waves hold more staged rows each.
template <int BS>
struct Chunk {
  static constexpr int kRows = BS == 128 ? 64 : 32;
  static constexpr int kRT = kRows / 32;           // 32-row tiles per chunk
  static constexpr int kTrStride = 2 * kRows + 8;  // bytes per head-dim row of Q^T / dO^T
};

template <int BS>
struct BwdLds {
  static constexpr int kChunkRows = Chunk<BS>::kRows;
  static constexpr int kTrStride = Chunk<BS>::kTrStride;
  static constexpr int kKtStride = 2 * BS + 16;  // bytes per head-dim row of K^T
  static constexpr int kDsStride = 2 * BS + 16;  // bytes per query row of dS
  // the row info first: its 24 reads per chunk then take immediate offsets
  // (a ds instruction's offset field reaches 64 KiB)
  static constexpr int kInfo = 0;  // lse2, delta, lim, entry: kChunkRows each
  static constexpr int kQn = kInfo + 4 * kChunkRows * 4;
  static constexpr int kDn = kQn + kChunkRows * kNatStride;
  static constexpr int kQt = kDn + kChunkRows * kNatStride;
  static constexpr int kDt = kQt + kHeadDim * kTrStride;
  static constexpr int kDs = kDt + kHeadDim * kTrStride;
  static constexpr int kKt = kDs + kChunkRows * kDsStride;
  static constexpr int kDq = kKt + kHeadDim * kKtStride;  // dq tile: rows x head dims (bf16)
  static constexpr int kBytes = kDq + kChunkRows * kNatStride;
};

// One chunk's gathered rows on their way to LDS: NT threads, each holding
// jobs (row pair p, head dims 8 c .. 8 c + 7) of Q and dO, plus (threads
// 0 .. rows - 1) one row's lse2, delta, visible-key limit and CSR entry.
// Job q is row pair (q % 16) + 16 (q / 256), dims 8 ((q / 16) % 16): the 32
// lanes of an LDS write cycle then cover 16 row pairs of two head-dim rows
// 8 apart, so the transposed writes hit 32 distinct banks.
template <int NT, int CR>
struct RowStage {
  static constexpr int kJobs = CR / 2 * 16 / NT;
  u32x4_t qa[kJobs], qb[kJobs], da[kJobs], db[kJobs];
  float lse2, delta;
  int lim;
  uint32_t ent;
};

// CSR entries of the rows a thread stages for chunk cc (clamped to the row's
// last entry past its end).
template <int NT, int CR>
struct RowEnts {
  uint32_t e[RowStage<NT, CR>::kJobs][2];
  uint32_t info;
};

// The low halves of a and b as one word (a's in the low half), and the high
// halves: one byte permute each (v_perm_b32 numbers b's bytes 4..7 and a's
// 0..3).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <int TRS>
__device__ __forceinline__ u32x4_t tr_frag(const char* base, int d, int rt, int h2, int hf) {
  const char* p = base + d * TRS + 2 * (32 * rt + 16 * h2 + 4 * hf);
  const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(p);
  const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(p + 16);
  return u32x4_t{lo.x, lo.y, hi.x, hi.y};
}

template <int BS>
__global__ __launch_bounds__(2 * BS, 1) void bwd_kv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ row_ptr, const uint32_t* __restrict__ entries, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, uint16_t* __restrict__ part_dq, BwdShape sh) {
  constexpr int NW = BS / 32;
  constexpr int NT = 64 * NW;
  constexpr int DT = 4 / NW;  // head-dim tiles of dQ per wave
  using L = BwdLds<BS>;
  constexpr int kChunkRows = Chunk<BS>::kRows;
  constexpr int kRT = Chunk<BS>::kRT;
  constexpr int kTrStride = Chunk<BS>::kTrStride;
  using Stage = RowStage<NT, kChunkRows>;
  using Ents = RowEnts<NT, kChunkRows>;
  extern __shared__ __align__(16) char lds[];

  // blocks in ascending order, the units of one block side by side: early
  // blocks are kept by more queries, so the longest rows start first
  const int u = blockIdx.x % sh.U;
  const int j = blockIdx.x / sh.U;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hf = lane >> 5;
  const int crow = u * sh.nb + j;
  const int e0 = row_ptr[crow];
  const int n = row_ptr[crow + 1] - e0;
  // a pass whose queries did not keep the block adds nothing to its sums
  if (n == 0 && sh.acc_k != nullptr) return;
  const int n_keys = min(BS, sh.S - j * BS);
  const int tpc = kChunkRows >> sh.r_log2;  // tokens per chunk
  const int n_chunks = (n + tpc - 1) / tpc;
  const float c2 = sh.scale_log2;
  const size_t kv_base = ((size_t)u * sh.S + (size_t)j * BS) * kHeadDim;

  // ---- the wave's K and V rows (B operands: key = lane % 32, head dims
  // 16 ks + 8 hf .. + 7), K^T of the whole block into LDS
  u32x4_t kb[8], vb[8];
  {
    const int key = min(32 * w + (lane & 31), n_keys - 1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kb[ks] = *reinterpret_cast<const u32x4_t*>(k + kv_base + (size_t)key * kHeadDim + 16 * ks + 8 * hf);
      vb[ks] = *reinterpret_cast<const u32x4_t*>(v + kv_base + (size_t)key * kHeadDim + 16 * ks + 8 * hf);
    }
    constexpr int kKJobs = 8 * BS / NT;  // (key pair, 8 head dims) jobs per thread
#pragma unroll
    for (int m = 0; m < kKJobs; ++m) {
      const int qid = tid + NT * m;
      const int p = qid >> 4;
      const int c = qid & 15;
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(k + kv_base + (size_t)min(2 * p, n_keys - 1) * kHeadDim + 8 * c);
      const u32x4_t bb =
          *reinterpret_cast<const u32x4_t*>(k + kv_base + (size_t)min(2 * p + 1, n_keys - 1) * kHeadDim + 8 * c);
      char* kt = lds + L::kKt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint32_t*>(kt + (8 * c + 2 * e) * L::kKtStride + 4 * p) = lo_halves(a[e], bb[e]);
        *reinterpret_cast<uint32_t*>(kt + (8 * c + 2 * e + 1) * L::kKtStride + 4 * p) =
            hi_halves(a[e], bb[e]);
      }
    }
  }

  f32x16_t dkt[4], dvt[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    dkt[dt] = f32x16_t{};
    dvt[dt] = f32x16_t{};
  }

  // entries of chunk cc for this thread's rows
  // Index arithmetic in 32 bits where it fits: a CSR row holds at most one
  // entry per query token (< 2^26), b S + t < units S < 2^31, and
  // (unit, token, slot) numbers stay below units S top_k < 2^31 (both
  // checked on the host); row numbers of (token, head) take one 32 x 32 ->
  // 64-bit multiply-add.
  const uint32_t* ents = entries + e0;
  auto ent_at = [&](int i) -> uint32_t {
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(ents) + ((uint32_t)i << 2));
  };
  auto load_ents = [&](int cc, Ents& re) {
#pragma unroll
    for (int m = 0; m < Stage::kJobs; ++m) {
      const int p = ((tid + NT * m) & 15) + 16 * ((tid + NT * m) >> 8);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int tk = cc * tpc + ((2 * p + x) >> sh.r_log2);
        re.e[m][x] = ent_at(min(tk, n - 1));
      }
    }
    re.info = ent_at(min(cc * tpc + ((tid & (kChunkRows - 1)) >> sh.r_log2), n - 1));
  };
  const uint32_t tok0 = (uint32_t)(b * sh.S + sh.q0);  // row b S + t of token t = q0 + (ent >> 5)
  const uint32_t head0 = (uint32_t)(g * sh.r);
  auto qrow = [&](uint32_t ent, int rho) -> uint64_t {
    return (uint64_t)(tok0 + (ent >> 5)) * (uint32_t)sh.Hq + (head0 + (uint32_t)(rho & (sh.r - 1)));
  };
  auto row_ptr_q = [&](const uint16_t* base, uint32_t ent, int rho) -> const uint16_t* {
    return base + qrow(ent, rho) * kHeadDim;
  };
  auto load_rows = [&](int cc, const Ents& re, Stage& st) {
#pragma unroll
    for (int m = 0; m < Stage::kJobs; ++m) {
      const int qid = tid + NT * m;
      const int p = (qid & 15) + 16 * (qid >> 8);
      const int c = (qid >> 4) & 15;
      st.qa[m] = *reinterpret_cast<const u32x4_t*>(row_ptr_q(q, re.e[m][0], 2 * p) + 8 * c);
      st.qb[m] = *reinterpret_cast<const u32x4_t*>(row_ptr_q(q, re.e[m][1], 2 * p + 1) + 8 * c);
      st.da[m] = *reinterpret_cast<const u32x4_t*>(row_ptr_q(dout, re.e[m][0], 2 * p) + 8 * c);
      st.db[m] = *reinterpret_cast<const u32x4_t*>(row_ptr_q(dout, re.e[m][1], 2 * p + 1) + 8 * c);
    }
    // row info: threads 0 .. kChunkRows - 1, row = tid (other threads load a copy)
    const int rho = tid & (kChunkRows - 1);
    const int tk = cc * tpc + (rho >> sh.r_log2);
    const bool valid = tk < n;
    const int t = sh.q0 + (int)(re.info >> 5);
    const uint64_t ri = qrow(re.info, rho);
    const float l2 = lse[ri] * kLog2e;
    st.lse2 = valid ? l2 : __builtin_inff();
    st.delta = delta[ri];
    st.lim = t - j * BS;
    st.ent = valid ? re.info : 0xffffffffu;
  };
  auto store_rows = [&](const Stage& st) {
#pragma unroll
    for (int m = 0; m < Stage::kJobs; ++m) {
      const int qid = tid + NT * m;
      const int p = (qid & 15) + 16 * (qid >> 8);
      const int c = (qid >> 4) & 15;
      *reinterpret_cast<u32x4_t*>(lds + L::kQn + (2 * p) * kNatStride + 16 * c) = st.qa[m];
      *reinterpret_cast<u32x4_t*>(lds + L::kQn + (2 * p + 1) * kNatStride + 16 * c) = st.qb[m];
      *reinterpret_cast<u32x4_t*>(lds + L::kDn + (2 * p) * kNatStride + 16 * c) = st.da[m];
      *reinterpret_cast<u32x4_t*>(lds + L::kDn + (2 * p + 1) * kNatStride + 16 * c) = st.db[m];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        char* qt = lds + L::kQt;
        char* dt = lds + L::kDt;
        *reinterpret_cast<uint32_t*>(qt + (8 * c + 2 * e) * kTrStride + 4 * p) =
            lo_halves(st.qa[m][e], st.qb[m][e]);
        *reinterpret_cast<uint32_t*>(qt + (8 * c + 2 * e + 1) * kTrStride + 4 * p) =
            hi_halves(st.qa[m][e], st.qb[m][e]);
        *reinterpret_cast<uint32_t*>(dt + (8 * c + 2 * e) * kTrStride + 4 * p) =
            lo_halves(st.da[m][e], st.db[m][e]);
        *reinterpret_cast<uint32_t*>(dt + (8 * c + 2 * e + 1) * kTrStride + 4 * p) =
            hi_halves(st.da[m][e], st.db[m][e]);
      }
    }
    if (tid < kChunkRows) {
      reinterpret_cast<float*>(lds + L::kInfo)[tid] = st.lse2;
      reinterpret_cast<float*>(lds + L::kInfo + 4 * kChunkRows)[tid] = st.delta;
      reinterpret_cast<int*>(lds + L::kInfo + 8 * kChunkRows)[tid] = st.lim;
      reinterpret_cast<uint32_t*>(lds + L::kInfo + 12 * kChunkRows)[tid] = st.ent;
    }
  };

  // Pipeline per chunk c (one register stage, loads a full chunk ahead; a
  // second stage, loads two chunks ahead, measured no faster):
  //   phase 1 on the LDS rows of chunk c; dS -> LDS        | barrier A
  //   rows of chunk c + 1 (registers) -> LDS; loads of chunk c + 2
  //   phase 2: dQ^T -> the LDS dq tile                     | barrier B
  //   the dq tile -> part_dq, 16 bytes per thread
  // Every wait on a load is on one issued before the previous chunk's
  // stores (vector-memory operations complete in order), and loads and
  // stores are issued the same way on every path: past the row's end they
  // repeat its last entry, and their rows are masked (lse2 = +inf, no dq
  // store).
  constexpr int kCopyRows = kChunkRows * 16 / NT;  // dq tile rows each thread stores
  Ents ent_next;
  Stage stage;
  const bool any = n_chunks > 0;
  if (any) {
    load_ents(0, ent_next);
    load_rows(0, ent_next, stage);
    store_rows(stage);
    load_ents(1, ent_next);
    load_rows(1, ent_next, stage);
    load_ents(2, ent_next);
  }
  // every load issued so far (the wave's K and V rows above all) is complete
  // before the loop, so that no wait inside it is on them
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int key = 32 * w + (lane & 31);  // this lane's key within the block (S / dP columns)
  for (int c = 0; c < n_chunks; ++c) {
    // ---- S = Q K^T and dP = dO V^T for the wave's 32 keys, per row tile
    f32x16_t s[kRT], dp[kRT];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      s[rt] = f32x16_t{};
      dp[rt] = f32x16_t{};
      const char* qrow = lds + L::kQn + (32 * rt + (lane & 31)) * kNatStride + 16 * hf;
      const char* drow = lds + L::kDn + (32 * rt + (lane & 31)) * kNatStride + 16 * hf;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[rt] = mfma32x32x16(*reinterpret_cast<const u32x4_t*>(qrow + 32 * ks), kb[ks], s[rt]);
        dp[rt] = mfma32x32x16(*reinterpret_cast<const u32x4_t*>(drow + 32 * ks), vb[ks], dp[rt]);
      }
    }
    // ---- P and dS; element i of tile rt is query row 32 rt + c_row(i, hf), column = key
    u32x4_t ph[kRT][2], dsh[kRT][2];
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt) {
      float pv[16], dsv[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = 32 * rt + 8 * q4 + 4 * hf;
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lds + L::kInfo + 4 * r0);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(lds + L::kInfo + 4 * kChunkRows + 4 * r0);
        const i32x4_t m4 = *reinterpret_cast<const i32x4_t*>(lds + L::kInfo + 8 * kChunkRows + 4 * r0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = 4 * q4 + x;
          const float p = key <= m4[x] ? fast_exp2(fmaf(s[rt][i], c2, -l4[x])) : 0.f;
          pv[i] = p;
          dsv[i] = p * (dp[rt][i] - d4[x]);
        }
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        ph[rt][h2] = u32x4_t{pack_bf16x2(pv[8 * h2], pv[8 * h2 + 1]), pack_bf16x2(pv[8 * h2 + 2], pv[8 * h2 + 3]),
                             pack_bf16x2(pv[8 * h2 + 4], pv[8 * h2 + 5]), pack_bf16x2(pv[8 * h2 + 6], pv[8 * h2 + 7])};
        dsh[rt][h2] =
            u32x4_t{pack_bf16x2(dsv[8 * h2], dsv[8 * h2 + 1]), pack_bf16x2(dsv[8 * h2 + 2], dsv[8 * h2 + 3]),
                    pack_bf16x2(dsv[8 * h2 + 4], dsv[8 * h2 + 5]), pack_bf16x2(dsv[8 * h2 + 6], dsv[8 * h2 + 7])};
      }
    }
    // entries of the dq tile rows this thread stores after phase 2
    uint32_t copy_ent[kCopyRows];
#pragma unroll
    for (int m = 0; m < kCopyRows; ++m)
      copy_ent[m] = reinterpret_cast<const uint32_t*>(lds + L::kInfo + 12 * kChunkRows)[(tid >> 4) + (NT >> 4) * m];
    // ---- dV^T += dO^T P, dK^T += Q^T dS (head dims x the wave's keys)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int d = 32 * dt + (lane & 31);
          dvt[dt] = mfma32x32x16(tr_frag<kTrStride>(lds + L::kDt, d, rt, h2, hf), ph[rt][h2], dvt[dt]);
          dkt[dt] = mfma32x32x16(tr_frag<kTrStride>(lds + L::kQt, d, rt, h2, hf), dsh[rt][h2], dkt[dt]);
        }
    // ---- dS (bf16, as used above) -> LDS, rows x keys
#pragma unroll
    for (int rt = 0; rt < kRT; ++rt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t pair = dsh[rt][h2][e];
          const int i = 8 * h2 + 2 * e;
          char* col = lds + L::kDs + 2 * key + 32 * rt * L::kDsStride;
          *reinterpret_cast<uint16_t*>(col + c_row(i, hf) * L::kDsStride) = (uint16_t)(pair & 0xffffu);
          *reinterpret_cast<uint16_t*>(col + c_row(i + 1, hf) * L::kDsStride) = (uint16_t)(pair >> 16);
        }
    __syncthreads();
    // the rows of chunk c + 1 replace this chunk's (every read of them is
    // above the barrier), then the loads of chunk c + 2
    store_rows(stage);
    load_rows(c + 2, ent_next, stage);
    load_ents(c + 3, ent_next);
    // ---- dQ^T = K^T dS^T for head-dim tiles DT w .. DT w + DT - 1, into
    // the LDS dq tile (rows x head dims)
#pragma unroll
    for (int dd = 0; dd < DT; ++dd) {
      const int dt = DT * w + dd;
#pragma unroll
      for (int rt = 0; rt < kRT; ++rt) {
        f32x16_t acc = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < BS / 16; ++ks) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(lds + L::kKt + (32 * dt + (lane & 31)) * L::kKtStride +
                                                              32 * ks + 16 * hf);
          const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(lds + L::kDs + (32 * rt + (lane & 31)) * L::kDsStride +
                                                               32 * ks + 16 * hf);
          acc = mfma32x32x16(a, bq, acc);
        }
        char* dst = lds + L::kDq + (32 * rt + (lane & 31)) * kNatStride + 2 * (32 * dt + 4 * hf);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2_t wv;
          wv.x = pack_bf16x2(acc[4 * q4], acc[4 * q4 + 1]);
          wv.y = pack_bf16x2(acc[4 * q4 + 2], acc[4 * q4 + 3]);
          *reinterpret_cast<u32x2_t*>(dst + 16 * q4) = wv;
        }
      }
    }
    __syncthreads();
    // ---- the dq tile -> one bf16 partial per (row, slot): 16 threads per
    // row, 16 bytes each, non-temporal (read once, by bwd_dq; measured on
    // MI355X: the 32K backward 11.72 -> 11.55 ms)
#pragma unroll
    for (int m = 0; m < kCopyRows; ++m) {
      const int rho = (tid >> 4) + (NT >> 4) * m;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(lds + L::kDq + rho * kNatStride + 16 * (tid & 15));
      const uint32_t e = copy_ent[m];
      if (e != 0xffffffffu) {
        const uint32_t slot = ((uint32_t)u * (uint32_t)sh.n_q + (e >> 5)) * (uint32_t)sh.top_k + (e & 31u);
        const uint64_t pidx = (uint64_t)slot * (uint32_t)sh.r + (uint32_t)(rho & (sh.r - 1));
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(part_dq + pidx * kHeadDim + 8 * (tid & 15)));
      }
    }
  }

  // ---- dK = scale * dK^T^T, dV: this lane's key, head dims 32 dt + 8 q4 + 4 hf + 0..3
  // (over several passes the unscaled fp32 sums are added to acc_k, acc_v)
  if (key < n_keys) {
    if (sh.acc_k != nullptr) {
      float* akr = sh.acc_k + kv_base + (size_t)key * kHeadDim;
      float* avr = sh.acc_v + kv_base + (size_t)key * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * dt + 8 * q4 + 4 * hf;
          f32x4_t ka = *reinterpret_cast<const f32x4_t*>(akr + d0);
          f32x4_t va = *reinterpret_cast<const f32x4_t*>(avr + d0);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            ka[x] += dkt[dt][4 * q4 + x];
            va[x] += dvt[dt][4 * q4 + x];
          }
          *reinterpret_cast<f32x4_t*>(akr + d0) = ka;
          *reinterpret_cast<f32x4_t*>(avr + d0) = va;
        }
    } else {
      uint16_t* dkr = dk + kv_base + (size_t)key * kHeadDim;
      uint16_t* dvr = dv + kv_base + (size_t)key * kHeadDim;
      const float sc = sh.scale;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * dt + 8 * q4 + 4 * hf;
          u32x2_t a, bq;
          a.x = pack_bf16x2(dkt[dt][4 * q4] * sc, dkt[dt][4 * q4 + 1] * sc);
          a.y = pack_bf16x2(dkt[dt][4 * q4 + 2] * sc, dkt[dt][4 * q4 + 3] * sc);
          bq.x = pack_bf16x2(dvt[dt][4 * q4], dvt[dt][4 * q4 + 1]);
          bq.y = pack_bf16x2(dvt[dt][4 * q4 + 2], dvt[dt][4 * q4 + 3]);
          *reinterpret_cast<u32x2_t*>(dkr + d0) = a;
          *reinterpret_cast<u32x2_t*>(dvr + d0) = bq;
        }
    }
  }
}

// delta of every row: 16 threads per row, 8 head dims each.
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, long rows) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = gid >> 4;
  const int c16 = (int)(gid & 15);
  // a row's 16 threads are all in range or all out of it
  if (row >= rows) return;
  const u32x4_t o = *reinterpret_cast<const u32x4_t*>(out + row * kHeadDim + 8 * c16);
  const u32x4_t d = *reinterpret_cast<const u32x4_t*>(dout + row * kHeadDim + 8 * c16);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc = fmaf(bf16_lo(o[e]), bf16_lo(d[e]), acc);
    acc = fmaf(bf16_hi(o[e]), bf16_hi(d[e]), acc);
  }
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) acc += __shfl_xor(acc, x);
  if (c16 == 0) delta[row] = acc;
}

// dq of every row: 16 threads per (token, head), 8 head dims each, summing
// the row's min(top_k - 1, own block) + 1 partials (each read once, with a
// non-temporal hint, as in the forward's merge).
__global__ __launch_bounds__(256) void bwd_dq_kernel(const uint16_t* __restrict__ part_dq, uint16_t* __restrict__ dq,
                                                     BwdShape sh) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const int c16 = (int)(gid & 15);
  const long qr = gid >> 4;
  const int h = (int)(qr & (sh.r - 1));
  const long t = qr >> sh.r_log2;  // row of the pass (token q0 + t)
  if (t >= sh.n_q) return;
  const int u = blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int n = min(sh.top_k - 1, (int)((sh.q0 + t) >> sh.bs_log2)) + 1;
  const uint16_t* src = part_dq + (((size_t)u * sh.n_q + t) * sh.top_k * sh.r + h) * kHeadDim + 8 * c16;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // the loads of up to 16 partials are issued together: one memory round
  // trip for top_k <= 16
  constexpr int kB = 16;
  for (int s0 = 0; s0 < n; s0 += kB) {
    u32x4_t val[kB];
#pragma unroll
    for (int s = 0; s < kB; ++s)
      if (s0 + s < n)
        val[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + (size_t)(s0 + s) * sh.r * kHeadDim));
#pragma unroll
    for (int s = 0; s < kB; ++s)
      if (s0 + s < n)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(val[s][e]);
          acc[2 * e + 1] += bf16_hi(val[s][e]);
        }
  }
  const float sc = sh.scale;
  u32x4_t wv = {pack_bf16x2(acc[0] * sc, acc[1] * sc), pack_bf16x2(acc[2] * sc, acc[3] * sc),
                pack_bf16x2(acc[4] * sc, acc[5] * sc), pack_bf16x2(acc[6] * sc, acc[7] * sc)};
  *reinterpret_cast<u32x4_t*>(dq + (((size_t)b * sh.S + sh.q0 + t) * sh.Hq + g * sh.r + h) * kHeadDim + 8 * c16) = wv;
}

// dk, dv from the fp32 sums of several passes: 4 head dims per thread.
__global__ __launch_bounds__(256) void bwd_acc_kernel(const float* __restrict__ acc_k,
                                                      const float* __restrict__ acc_v, uint16_t* __restrict__ dk,
                                                      uint16_t* __restrict__ dv, long quads, float scale) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= quads) return;
  const f32x4_t a = reinterpret_cast<const f32x4_t*>(acc_k)[i];
  const f32x4_t c = reinterpret_cast<const f32x4_t*>(acc_v)[i];
  u32x2_t wk, wv;
  wk.x = pack_bf16x2(a[0] * scale, a[1] * scale);
  wk.y = pack_bf16x2(a[2] * scale, a[3] * scale);
  wv.x = pack_bf16x2(c[0], c[1]);
  wv.y = pack_bf16x2(c[2], c[3]);
  reinterpret_cast<u32x2_t*>(dk)[i] = wk;
  reinterpret_cast<u32x2_t*>(dv)[i] = wv;
}

template <int BS>
hipError_t launch_bwd_kv_bs(const BwdShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const uint16_t* dout, const float* lse, const float* delta, const int32_t* row_ptr,
                            const uint32_t* entries, uint16_t* dk, uint16_t* dv, uint16_t* part_dq,
                            hipStream_t st) {
  constexpr int bytes = BwdLds<BS>::kBytes;
  const hipError_t attr = ensure_dynamic_lds(reinterpret_cast<const void*>(&bwd_kv_kernel<BS>), bytes);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(bwd_kv_kernel<BS>, dim3((unsigned)(sh.U * sh.nb)), dim3(2 * BS), bytes, st, q, k, v, dout, lse,
                     delta, row_ptr, entries, dk, dv, part_dq, sh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_delta(const uint16_t* out, const uint16_t* dout, float* delta, long rows, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long threads = rows * 16;
  hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, out, dout, delta,
                     rows);
  return hipGetLastError();
}

hipError_t launch_bwd_kv(const BwdShape& sh, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, const float* lse, const float* delta, const int32_t* row_ptr,
                         const uint32_t* entries, uint16_t* dk, uint16_t* dv, uint16_t* part_dq, hipStream_t st) {
  switch (sh.bs) {
    case 32:
      return launch_bwd_kv_bs<32>(sh, q, k, v, dout, lse, delta, row_ptr, entries, dk, dv, part_dq, st);
    case 64:
      return launch_bwd_kv_bs<64>(sh, q, k, v, dout, lse, delta, row_ptr, entries, dk, dv, part_dq, st);
    default:
      return launch_bwd_kv_bs<128>(sh, q, k, v, dout, lse, delta, row_ptr, entries, dk, dv, part_dq, st);
  }
}

hipError_t launch_bwd_acc(const BwdShape& sh, uint16_t* dk, uint16_t* dv, hipStream_t st) {
  const long quads = (long)sh.U * sh.S * kHeadDim / 4;
  hipLaunchKernelGGL(bwd_acc_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, sh.acc_k, sh.acc_v, dk,
                     dv, quads, sh.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const BwdShape& sh, const uint16_t* part_dq, uint16_t* dq, hipStream_t st) {
  const long threads = (long)sh.n_q * sh.r * 16;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)((threads + 255) / 256), (unsigned)sh.U), dim3(256), 0, st, part_dq,
                     dq, sh);
  return hipGetLastError();
}

}  // namespace msa
