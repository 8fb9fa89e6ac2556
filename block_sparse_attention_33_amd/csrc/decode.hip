// MSA decode: one query per sequence at the last cache position.
//
// Decode applies the same two branches to a single query over a KV cache
// whose past keys and values stay resident in device memory (wiki.500nian.com
// digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI Agents", the
// paragraph on the quadratic wall and the KV cache; its co-design paragraph
// reports the decode speed-up).  The work is bound by HBM reads: the block
// summaries (nb x 64 B per group) and the selected K/V blocks.
//
//   decode_kernel  one workgroup per (batch, group): scores every candidate
//                  block, keeps the best top_k - 1 plus the own block, and
//                  runs the r query heads of the group over the kept blocks
//                  with an online softmax (split over two groups of waves,
//                  merged at the end).  Nothing but the selection and the
//                  output leaves the workgroup.
//
// Ranking keys are 64-bit: (score << 32) | (0xffffffff - block), so a larger
// key is a higher score or, at equal score, a lower block index.

#include <limits.h>

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

constexpr int64_t kNoKey = INT64_MIN;

__device__ __forceinline__ int64_t rank_key(int score, int block) {
  return (int64_t)(((uint64_t)(int64_t)score << 32) | (uint64_t)(0xffffffffu - (uint32_t)block));
}
__device__ __forceinline__ int key_block(int64_t key) { return (int)(0xffffffffu - (uint32_t)(uint64_t)key); }

__device__ __forceinline__ int64_t max_i64(int64_t a, int64_t b) { return a > b ? a : b; }

// x combined with its DPP-moved copy (lanes the pattern does not reach keep x).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int64_t dpp_max_i64(int64_t x) {
  const int lo = (int)(uint32_t)(uint64_t)x;
  const int hi = (int)(uint32_t)((uint64_t)x >> 32);
  const int mlo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
  const int mhi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
  const int64_t y = (int64_t)(((uint64_t)(uint32_t)mhi << 32) | (uint64_t)(uint32_t)mlo);
  return max_i64(x, y);
}

// Maximum over the wave, returned in every lane: DPP steps within rows of 16
// lanes, row broadcasts towards lane 63, then a read of lane 63.
__device__ __forceinline__ int64_t wave_max_i64(int64_t x) {
  x = dpp_max_i64<0xb1, 0xf>(x);   // quad_perm [1,0,3,2]
  x = dpp_max_i64<0x4e, 0xf>(x);   // quad_perm [2,3,0,1]
  x = dpp_max_i64<0x141, 0xf>(x);  // row_half_mirror
  x = dpp_max_i64<0x140, 0xf>(x);  // row_mirror
  x = dpp_max_i64<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_max_i64<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)x, 63);
  const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), 63);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// The best `kp` keys held by one wave (NK per lane), extracted one at a time
// (keys are unique).  Winner `it` is returned in lane `it` (kNoKey if there
// are fewer keys); the other lanes return kNoKey.
template <int NK>
__device__ __forceinline__ int64_t wave_topk(int64_t (&k)[NK], int kp) {
  const int lane = threadIdx.x & 63;
  int64_t mine = kNoKey;
  for (int it = 0; it < kp; ++it) {
    int64_t best = k[0];
#pragma unroll
    for (int i = 1; i < NK; ++i) best = max_i64(best, k[i]);
    const int64_t w = wave_max_i64(best);
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (k[i] == w) k[i] = kNoKey;
    if (lane == it) mine = w;
  }
  return mine;
}

// The best kp keys (keys unique; kNoKey = none) held by one wave, NK per
// lane, by rank counting: each lane's maximum is ranked among the 64 lane
// maxima, the kp-th largest of them (T0) bounds the kp-th largest key from
// below, the keys >= T0 (at most kp * NK, from the kp lanes whose maximum
// is >= T0) are gathered in LDS and ranked exactly.  Writes the best kp,
// descending, to out[0 .. kp) (kNoKey where fewer exist).
// ws: this wave's LDS scratch of 64 + 64 * NK keys.
template <int NK>
__device__ __forceinline__ void wave_topk_rank(const int64_t (&k)[NK], int kp, int64_t* ws, int64_t* out) {
  const int lane = threadIdx.x & 63;
  int64_t* lmx = ws;
  int64_t* cand = ws + 64;
  int64_t lm = k[0];
#pragma unroll
  for (int i = 1; i < NK; ++i) lm = max_i64(lm, k[i]);
  lmx[lane] = lm;
  wave_lds_sync();
  int rank = 0;
#pragma unroll 16
  for (int i = 0; i < 64; ++i) rank += lmx[i] > lm ? 1 : 0;
  const uint64_t at = __ballot(lm != kNoKey && rank == kp - 1);
  int64_t t0 = kNoKey;
  if (at != 0) {
    const int src = __builtin_ctzll(at);
    const int lo = __builtin_amdgcn_readlane((int)(uint32_t)(uint64_t)lm, src);
    const int hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)lm >> 32), src);
    t0 = (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
  }
  int nc = 0;
#pragma unroll
  for (int m = 0; m < NK; ++m) {
    const bool c = k[m] != kNoKey && k[m] >= t0;
    const uint64_t bal = __ballot(c);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (c) cand[nc + below] = k[m];
    nc += __popcll(bal);
  }
  wave_lds_sync();
  for (int base = 0; base < nc; base += 64) {
    const int i = base + lane;
    const int64_t x = i < nc ? cand[i] : kNoKey;
    int rk = 0;
#pragma unroll 8
    for (int jj = 0; jj < nc; ++jj) rk += cand[jj] > x ? 1 : 0;
    if (i < nc && rk < kp) out[rk] = x;
  }
  if (lane >= nc && lane < kp) out[lane] = kNoKey;
  wave_lds_sync();
}

// ---------------------------------------------------------------------------
// Fused decode: one workgroup (8 waves) per (sequence, group) unit.
//
//   selection  thread i scores candidates i, i + 512, ... (NK of them), each
//              wave keeps its best kp, wave 0 picks the best kp of the 8
//              lists and ranks them by block index: slot s of the selection
//              is the s-th smallest, the own block follows them, later slots
//              are empty (-1).
//   attention  two groups of 4 waves take the even and the odd slots; per
//              slot a group runs S^T = K Q^T on 32x32x16 MFMA (wave w: keys
//              32 w .. 32 w + 31, the r query heads as columns, K straight
//              from HBM), P = 2^(S - m) goes to LDS as bf16 [head][key], V
//              to LDS transposed, and O^T = V^T P^T (wave w: head dims
//              32 w .. 32 w + 31) is added to the group's running
//              online-softmax state.  A group's next slot loads while the
//              current one is computed.
//   merge      the two groups' states are combined in LDS and written as
//              bf16, or, when a unit's slots are shared by n_split
//              workgroups (slot s goes to workgroup s % n_split), written as
//              the workgroup's (max, sum, unnormalised o) for
//              decode_merge_kernel.
// ---------------------------------------------------------------------------
constexpr int kRowStride = 2 * 128 + 16;  // bytes per 128-key row of V^T and P^T in LDS

// One slot's block in registers: K fragments of this lane's key row and V
// key pairs (2p, 2p + 1) x 8 head dims.
struct DecBlock {
  u32x4_t kf[8];
  u32x4_t va[4], vb[4];
};

// Loads of block j (a valid block index) for group thread gt, wave-in-group wg.
__device__ __forceinline__ void dec_load_block(const DecodeShape& sh, const uint16_t* __restrict__ k_cache,
                                               const uint16_t* __restrict__ v_cache, int u, int j, int gt, int wg,
                                               int lane, DecBlock& blk) {
  const int key0 = j * sh.bs;
  const int nk = min(sh.bs, sh.L - key0);
  const int col = lane & 31, hf = lane >> 5;
  const uint16_t* krow = k_cache + ((size_t)u * sh.L + key0 + min(32 * wg + col, nk - 1)) * kHeadDim;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) blk.kf[ks] = *reinterpret_cast<const u32x4_t*>(krow + 16 * ks + 8 * hf);
  const uint16_t* vblk = v_cache + ((size_t)u * sh.L + key0) * kHeadDim;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int qid = gt + 256 * m;
    const int pp = qid & 63, c = qid >> 6;
    blk.va[m] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)min(2 * pp, nk - 1) * kHeadDim + 8 * c);
    blk.vb[m] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)min(2 * pp + 1, nk - 1) * kHeadDim + 8 * c);
  }
}

// Running online-softmax state of a group: this lane's column (head) and its
// wave's 32 head dims.
struct DecState {
  f32x16_t o;
  float m, l;  // base-2 running max and sum of the column
};

// One slot (block j, or an empty slot when j < 0) added to the group's state.
// Starts and ends with a workgroup barrier-free region: the caller places
// the barriers that order the LDS buffers between slots.
__device__ __forceinline__ void dec_slot(const DecodeShape& sh, const DecBlock& blk, int j, const u32x4_t (&qf)[8],
                                         char* __restrict__ vt, char* __restrict__ pt, float (*red_m)[32],
                                         float (*red_l)[32], int gt, int wg, int lane, DecState& st) {
  const int col = lane & 31, hf = lane >> 5;
  const bool qcol = col < sh.r;
  const int nk = j < 0 ? 0 : min(sh.bs, sh.L - j * sh.bs);  // valid keys (0: empty slot)
  const int kbase = 32 * wg;
  // V^T in LDS, natural key order (zero beyond the block's keys)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int qid = gt + 256 * m;
    const int pp = qid & 63, c = qid >> 6;
    const u32x4_t a = 2 * pp < nk ? blk.va[m] : u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t bb = 2 * pp + 1 < nk ? blk.vb[m] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = a[e], hi = bb[e];
      *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e) * kRowStride + 4 * pp) = (lo & 0xffffu) | (hi << 16);
      *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e + 1) * kRowStride + 4 * pp) = (lo >> 16) | (hi & 0xffff0000u);
    }
  }
  // scores S^T (32 keys x 32 heads) of this wave, base 2
  f32x16_t s = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) s = mfma32x32x16(blk.kf[ks], qf[ks], s);
  const float c2 = sh.scale_log2;
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i] = kbase + c_row(i, hf) < nk ? s[i] * c2 : -__builtin_inff();
    mx = fmaxf(mx, s[i]);
  }
  mx = wave_max_pair(mx);
  if (hf == 0) red_m[wg][col] = mx;
  __syncthreads();
  const float m_blk = fmaxf(fmaxf(red_m[0][col], red_m[1][col]), fmaxf(red_m[2][col], red_m[3][col]));
  const float m_new = fmaxf(st.m, m_blk);
  const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;  // nothing seen yet: every p is 0
  const float alpha = fast_exp2(st.m - m_use);                   // 0 while the state is empty
  float sum = 0.f;
  // this lane's P^T row (its head): keys kbase + 8 q4 + 4 hf + 0..3
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const float p0 = fast_exp2(s[4 * q4 + 0] - m_use);
    const float p1 = fast_exp2(s[4 * q4 + 1] - m_use);
    const float p2 = fast_exp2(s[4 * q4 + 2] - m_use);
    const float p3 = fast_exp2(s[4 * q4 + 3] - m_use);
    sum += (p0 + p1) + (p2 + p3);
    u32x2_t pv;
    pv.x = pack_bf16x2(p0, p1);
    pv.y = pack_bf16x2(p2, p3);
    if (qcol) *reinterpret_cast<u32x2_t*>(pt + col * kRowStride + 2 * (kbase + 8 * q4 + 4 * hf)) = pv;
  }
  sum = wave_sum_pair(sum);
  if (hf == 0) red_l[wg][col] = sum;
  __syncthreads();
  // O^T: head dims 32 wg .. 32 wg + 31 x 32 heads over the block's keys
  f32x16_t o = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vt + (32 * wg + col) * kRowStride + 2 * (16 * kk + 8 * hf));
    // columns >= r read some head's row: their results are not used
    const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(pt + (col & 15) * kRowStride + 2 * (16 * kk + 8 * hf));
    o = mfma32x32x16(a, bq, o);
  }
  const float l_blk = red_l[0][col] + red_l[1][col] + red_l[2][col] + red_l[3][col];
#pragma unroll
  for (int i = 0; i < 16; ++i) st.o[i] = fmaf(st.o[i], alpha, o[i]);
  st.l = fmaf(st.l, alpha, l_blk);
  st.m = m_new;
}

template <int NK>
__global__ __launch_bounds__(512, 1) void decode_kernel(const uint16_t* __restrict__ q,
                                                        const int8_t* __restrict__ q_idx,
                                                        const uint16_t* __restrict__ k_cache,
                                                        const uint16_t* __restrict__ v_cache,
                                                        const int8_t* __restrict__ block_keys,
                                                        int32_t* __restrict__ sel_out, uint16_t* __restrict__ out,
                                                     float* __restrict__ state,
                                                        DecodeShape sh) {
  __shared__ __align__(16) char vt[2][kHeadDim * kRowStride];
  __shared__ __align__(16) char pt[2][16 * kRowStride];  // P^T rows of the r <= 16 heads
  __shared__ int64_t wbest[8 * 32];                // the waves' best kp, list w at w * kp
  __shared__ int64_t wscr[8][64 + 64 * NK];         // per-wave top-k scratch
  __shared__ int sorted[33];
  __shared__ float red_m[2][4][32];
  __shared__ float red_l[2][4][32];
  __shared__ float xo[16][kHeadDim];  // the odd-slot group's state for the final merge
  __shared__ float xml[16][2];

  const int u = blockIdx.x;
  const int part = blockIdx.y;  // this workgroup's share of the slots
  const int n_split = gridDim.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int col = lane & 31;
  const int gp = w >> 2;     // group: even (0) or odd (1) slots
  const int wg = w & 3;      // wave within the group
  const int gt = tid & 255;  // thread within the group
  const int r = sh.r;
  const int K = sh.top_k;
  const int kp = K - 1;
  const int own = sh.nb - 1;  // candidates are blocks 0 .. own - 1

  // ---- selection
  if (kp > 0) {
    const i32x4_t* qp = reinterpret_cast<const i32x4_t*>(q_idx + (size_t)u * kIdxDim);
    const i32x4_t q0 = qp[0], q1 = qp[1], q2 = qp[2], q3 = qp[3];
    const int8_t* kb = block_keys + (size_t)u * sh.nb * kIdxDim;
    int64_t keys[NK];
#pragma unroll
    for (int m = 0; m < NK; ++m) {
      const int j = tid + 512 * m;
      int64_t key = kNoKey;
      if (512 * m < own) {  // uniform: the loads below are unconditional within it
        const i32x4_t* sp = reinterpret_cast<const i32x4_t*>(kb + (size_t)min(j, own - 1) * kIdxDim);
        const i32x4_t a0 = sp[0], a1 = sp[1], a2 = sp[2], a3 = sp[3];
        int sc = 0;
        sc = sdot4(q0.x, a0.x, sc); sc = sdot4(q0.y, a0.y, sc); sc = sdot4(q0.z, a0.z, sc); sc = sdot4(q0.w, a0.w, sc);
        sc = sdot4(q1.x, a1.x, sc); sc = sdot4(q1.y, a1.y, sc); sc = sdot4(q1.z, a1.z, sc); sc = sdot4(q1.w, a1.w, sc);
        sc = sdot4(q2.x, a2.x, sc); sc = sdot4(q2.y, a2.y, sc); sc = sdot4(q2.z, a2.z, sc); sc = sdot4(q2.w, a2.w, sc);
        sc = sdot4(q3.x, a3.x, sc); sc = sdot4(q3.y, a3.y, sc); sc = sdot4(q3.z, a3.z, sc); sc = sdot4(q3.w, a3.w, sc);
        key = j < own ? rank_key(sc, j) : kNoKey;
      }
      keys[m] = key;
    }
    wave_topk_rank(keys, kp, wscr[w], wbest + w * kp);
  }
  __syncthreads();
  if (w == 0) {
    // the best kp of the 8 waves' lists (8 kp <= 248 keys, up to 4 a lane),
    // by rank, then ranked by block index among themselves
    const int n2 = 8 * kp;
    int64_t x[4];
    int rk[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[m] = lane + 64 * m < n2 ? wbest[lane + 64 * m] : kNoKey;
      rk[m] = 0;
    }
#pragma unroll 8
    for (int jj = 0; jj < n2; ++jj) {
      const int64_t y = wbest[jj];
#pragma unroll
      for (int m = 0; m < 4; ++m) rk[m] += y > x[m] ? 1 : 0;
    }
    int* kept = reinterpret_cast<int*>(wscr[0]);  // the kept blocks, by rank
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (x[m] != kNoKey && rk[m] < kp) kept[rk[m]] = key_block(x[m]);
    const int n_valid = min(kp, own);  // valid keys that exist
    wave_lds_sync();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (x[m] != kNoKey && rk[m] < kp) {
        const int blk = key_block(x[m]);
        int pos = 0;
#pragma unroll 8
        for (int i = 0; i < n_valid; ++i) pos += kept[i] < blk ? 1 : 0;
        sorted[pos] = blk;
      }
    }
    if (lane == n_valid) sorted[n_valid] = own;
    if (lane > n_valid && lane <= 32) sorted[lane] = -1;
  }
  __syncthreads();
  if (part == 0 && tid < K) sel_out[(size_t)u * K + tid] = sorted[tid];

  // ---- attention: group gp takes slots gp, gp + 2, ...; a group's next
  // slot loads while the current one is computed (two register sets, so
  // that no load result is moved between registers)
  u32x4_t qf[8];
  {
    const uint16_t* qrow = q + ((size_t)b * sh.Hq + g * r + min(col, r - 1)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
      if (col >= r) qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  DecState st;
  st.o = f32x16_t{};
  st.m = -__builtin_inff();
  st.l = 0.f;
  // the group's round rd is slot gp + 2 rd; the loads of an empty slot go to
  // the own block (valid memory, then ignored)
  auto slot_block = [&](int rd) -> int {
    const int s2 = (2 * rd + gp) * n_split + part;
    return s2 < K ? sorted[s2] : -1;
  };
  auto load_round = [&](int rd, DecBlock& blk) {
    const int j = slot_block(rd);
    dec_load_block(sh, k_cache, v_cache, u, j >= 0 ? j : own, gt, wg, lane, blk);
  };
  const int per_wg = 2 * n_split;
  const int n_rounds = (K + per_wg - 1) / per_wg;  // the same for both groups (barriers)
  DecBlock A, B;
  load_round(0, A);
  for (int rd = 0; rd < n_rounds; rd += 2) {
    load_round(rd + 1, B);
    if (rd > 0) __syncthreads();  // the previous slot's LDS reads are done
    dec_slot(sh, A, slot_block(rd), qf, vt[gp], pt[gp], red_m[gp], red_l[gp], gt, wg, lane, st);
    if (rd + 1 >= n_rounds) break;
    load_round(rd + 2, A);
    __syncthreads();
    dec_slot(sh, B, slot_block(rd + 1), qf, vt[gp], pt[gp], red_m[gp], red_l[gp], gt, wg, lane, st);
  }

  // ---- merge of the two groups' states -> out = o / l
  if (gp == 1 && col < r) {
#pragma unroll
    for (int i = 0; i < 16; ++i) xo[col][32 * wg + c_row(i, hf)] = st.o[i];
    if (wg == 0 && hf == 0) {
      xml[col][0] = st.m;
      xml[col][1] = st.l;
    }
  }
  __syncthreads();
  if (gp == 0 && col < r && n_split > 1) {
    // this workgroup's state (max, sum, unnormalised o) for the merge kernel
    const float m1 = xml[col][0], l1 = xml[col][1];
    const float M = fmaxf(st.m, m1);
    const float Mu = M == -__builtin_inff() ? 0.f : M;  // no key seen yet: all weights 0
    const float w0 = fast_exp2(st.m - Mu), w1 = fast_exp2(m1 - Mu);
    float* srow = state + (((size_t)u * n_split + part) * r + col) * (kHeadDim + 2);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4_t v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q4 + e;
        v4[e] = fmaf(st.o[i], w0, xo[col][32 * wg + c_row(i, hf)] * w1);
      }
      *reinterpret_cast<f32x4_t*>(srow + 32 * wg + 8 * q4 + 4 * hf) = v4;
    }
    if (wg == 0 && hf == 0) {
      srow[kHeadDim] = M;
      srow[kHeadDim + 1] = fmaf(st.l, w0, l1 * w1);
    }
  } else if (gp == 0 && col < r) {
    const float m1 = xml[col][0], l1 = xml[col][1];
    const float M = fmaxf(st.m, m1);  // finite: the own block is always kept
    const float w0 = fast_exp2(st.m - M), w1 = fast_exp2(m1 - M);
    const float inv = 1.0f / fmaf(st.l, w0, l1 * w1);
    uint16_t* orow = out + ((size_t)b * sh.Hq + g * r + col) * kHeadDim;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float v4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q4 + e;
        v4[e] = fmaf(st.o[i], w0, xo[col][32 * wg + c_row(i, hf)] * w1) * inv;
      }
      u32x2_t wv;
      wv.x = pack_bf16x2(v4[0], v4[1]);
      wv.y = pack_bf16x2(v4[2], v4[3]);
      *reinterpret_cast<u32x2_t*>(orow + 32 * wg + 8 * q4 + 4 * hf) = wv;
    }
  }
}

// Merge of a unit's n_split workgroup states: one workgroup per unit, a
// thread per (head, 4 head dims): out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ state,
                                                           uint16_t* __restrict__ out, DecodeShape sh,
                                                           int n_split) {
  const int u = blockIdx.x;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int r = sh.r;
  for (int it = threadIdx.x; it < r * 32; it += 256) {
    const int h = it >> 5;
    const int d0 = (it & 31) * 4;
    float M = -__builtin_inff();
    for (int p = 0; p < n_split; ++p)
      M = fmaxf(M, state[(((size_t)u * n_split + p) * r + h) * (kHeadDim + 2) + kHeadDim]);
    float W = 0.f;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < n_split; ++p) {
      const float* srow = state + (((size_t)u * n_split + p) * r + h) * (kHeadDim + 2);
      const float m = srow[kHeadDim];
      if (m == -__builtin_inff()) continue;  // a share with no kept block
      const float wgt = fast_exp2(m - M);
      W = fmaf(wgt, srow[kHeadDim + 1], W);
      const f32x4_t o4 = *reinterpret_cast<const f32x4_t*>(srow + d0);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, o4[e], acc[e]);
    }
    const float inv = 1.0f / W;
    u32x2_t wv;
    wv.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    wv.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2_t*>(out + ((size_t)b * sh.Hq + g * r + h) * kHeadDim + d0) = wv;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeShape& sh, const uint16_t* q, const int8_t* q_idx, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int8_t* block_keys, int32_t* sel_out, uint16_t* out,
                         float* state, int n_split, hipStream_t st) {
  const int own = sh.nb - 1;
  const dim3 grid(sh.B * sh.G, n_split), block(512);
  if (own <= 4 * 512)
    hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, st, q, q_idx, k_cache, v_cache, block_keys, sel_out, out,
                       state, sh);
  else if (own <= 8 * 512)
    hipLaunchKernelGGL(decode_kernel<8>, grid, block, 0, st, q, q_idx, k_cache, v_cache, block_keys, sel_out, out,
                       state, sh);
  else
    hipLaunchKernelGGL(decode_kernel<16>, grid, block, 0, st, q, q_idx, k_cache, v_cache, block_keys, sel_out, out,
                       state, sh);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeShape& sh, const float* state, int n_split, uint16_t* out,
                               hipStream_t st) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(sh.B * sh.G), dim3(256), 0, st, state, out, sh, n_split);
  return hipGetLastError();
}

}  // namespace msa
