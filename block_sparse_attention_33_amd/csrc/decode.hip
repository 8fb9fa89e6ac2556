// MSA decode: one query per sequence at the last cache position.
//
// Decode applies the same two branches to a single query over a KV cache
// whose past keys and values stay resident in device memory (wiki.500nian.com
// digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI Agents", the
// paragraph on the quadratic wall and the KV cache; its co-design paragraph
// reports the decode speed-up).  The work is bound by HBM reads: the block
// summaries (nb x 64 B per group) and the selected K/V blocks.
//
//   decode_kernel  two workgroups per (batch, group): each scores every
//                  candidate block, keeps the best top_k - 1 plus the own
//                  block, and runs the r query heads of the group over its
//                  share of the kept blocks with an online softmax (split
//                  over two groups of waves, merged at the end); with one
//                  workgroup per unit it writes the output directly.
//   decode_merge_kernel  combines the two workgroups' states of a unit.
//   append_kernel  one new token per unit into the caches, its index key
//                  into the running sums and the summary of its block.
//
// Ranking keys are 64-bit: (score << 32) | (0xffffffff - block), so a larger
// key is a higher score or, at equal score, a lower block index.

#include <limits.h>

#include <mutex>
#include <vector>

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

// x plus the value of lane (lane ^ 1), then of lane (lane ^ 2): the sum over
// the lane's quad, in every lane of the quad
__device__ __forceinline__ int quad_sum(int x) {
  x += __builtin_amdgcn_mov_dpp(x, 0xb1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
  x += __builtin_amdgcn_mov_dpp(x, 0x4e, 0xf, 0xf, false);  // quad_perm [2,3,0,1]
  return x;
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
//   selection  the four lanes of a quad read the four 16-byte quarters of
//              one candidate's summary (a wave load covers 16 whole
//              summaries) and sum their partial dot products; each thread
//              keeps NK candidates, each wave ranks its keys down to its
//              best kp, all eight waves rank the 8 kp survivors (four
//              threads per key) and the kept blocks are sorted by block
//              index: slot s of the selection is the s-th smallest, the own
//              block follows them, later slots are empty (-1).
//   attention  two groups of 4 waves take the even and the odd slots of
//              the workgroup's share; per slot a group runs S^T = K Q^T on
//              32x32x16 MFMA (wave w: keys 32 w .. 32 w + 31, the r query
//              heads as columns, K loaded as whole rows and passed through
//              the wave's own LDS tile, Q from LDS; measured on MI355X:
//              decode back to back 35.0 -> 34.2 us against per-lane
//              fragment loads, results identical),
//              P = 2^(S - m) goes to LDS as bf16 [head][key], V (loaded as
//              whole rows) is transposed in registers into LDS, and
//              O^T = V^T P^T (wave w: head dims 32 w .. 32 w + 31) is added
//              to the group's running online-softmax state.  A group's next
//              slot loads while the current one is computed.
//   merge      the two groups' states are combined in LDS and written as
//              bf16, or, when a unit's slots are shared by n_split
//              workgroups (slot s goes to workgroup s % n_split), written as
//              the workgroup's (max, sum, unnormalised o) for
//              decode_merge_kernel.
// ---------------------------------------------------------------------------
constexpr int kRowStride = 2 * 128 + 16;  // bytes per 128-key row of V^T and P^T in LDS

// One slot's block in registers: K rows of the wave's 32 keys as whole rows
// and an 8 x 8 tile of V.
struct DecBlock {
  u32x4_t kf[8];  // K row 32 wg + 4 m + lane / 16 (m = 0..7), head dims 8 (lane % 16) .. + 7
  u32x4_t vv[8];  // V rows 8 o + i (i = 0..7), head dims 8 c .. 8 c + 7 (o, c of the thread)
};

// Loads of block j (a valid block index) for group thread gt, wave-in-group wg.
__device__ __forceinline__ void dec_load_block(const DecodeShape& sh, const uint16_t* __restrict__ k_cache,
                                               const uint16_t* __restrict__ v_cache, int u, int L, int j, int gt,
                                               int wg, int lane, DecBlock& blk) {
  const int key0 = j * sh.bs;
  const int nk = min(sh.bs, L - key0);
  // K: every load instruction of a wave reads four whole 256-byte rows of
  // its 32 keys
  const uint16_t* kblk = k_cache + ((size_t)u * sh.Lc + key0) * kHeadDim + 8 * (lane & 15);
#pragma unroll
  for (int m = 0; m < 8; ++m)
    blk.kf[m] = *reinterpret_cast<const u32x4_t*>(kblk + (size_t)min(32 * wg + 4 * m + (lane >> 4), nk - 1) *
                                                             kHeadDim);
  // V: thread gt takes keys 8 o .. 8 o + 7 (o = gt / 16) and head dims
  // 8 c .. 8 c + 7 (c = gt % 16): every load instruction of a wave reads
  // four whole 256-byte rows
  const uint16_t* vblk = v_cache + ((size_t)u * sh.Lc + key0) * kHeadDim + 8 * (gt & 15);
  const int o8 = 8 * (gt >> 4);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    blk.vv[i] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)min(o8 + i, nk - 1) * kHeadDim);
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
__device__ __forceinline__ void dec_slot(const DecodeShape& sh, const DecBlock& blk, int L, int j,
                                         const char* __restrict__ qs, char* __restrict__ vt, char* __restrict__ pt,
                                         char* __restrict__ kt, float (*red_m)[32], float (*red_l)[32], int gt,
                                         int wg, int lane, DecState& st) {
  const int col = lane & 31, hf = lane >> 5;
  const bool qcol = col < sh.r;
  const int nk = j < 0 ? 0 : min(sh.bs, L - j * sh.bs);  // valid keys (0: empty slot)
  const int kbase = 32 * wg;
  // V^T in LDS: the thread's 8 x 8 tile is transposed in registers and row
  // d = 8 c + e gets keys 8 o .. 8 o + 7 as one 16-byte write, in 16-byte
  // column (o ^ (d >> 4)) so that the writes and the P.V reads are free of
  // bank conflicts.  Keys past the block's end hold a copy of its last
  // (finite) row; their P is 0.
  {
    const int o = gt >> 4, c = gt & 15;
    const u32x4_t (&x)[8] = blk.vv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x4_t t;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const uint32_t lo = x[2 * kk][e >> 1], hi = x[2 * kk + 1][e >> 1];
        t[kk] = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<u32x4_t*>(vt + (8 * c + e) * kRowStride + 16 * (o ^ (c >> 1))) = t;
    }
  }
  // the wave's K rows into its own LDS tile (only this wave reads it, so a
  // wave-level ordering suffices), read back as the A fragments of key col
#pragma unroll
  for (int m = 0; m < 8; ++m)
    *reinterpret_cast<u32x4_t*>(kt + (4 * m + (lane >> 4)) * kRowStride + 16 * (lane & 15)) = blk.kf[m];
  wave_lds_sync();
  // scores S^T (32 keys x 32 heads) of this wave, base 2
  f32x16_t s = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    s = mfma32x32x16(*reinterpret_cast<const u32x4_t*>(kt + col * kRowStride + 2 * (16 * ks + 8 * hf)),
                     *reinterpret_cast<const u32x4_t*>(qs + col * kRowStride + 2 * (16 * ks + 8 * hf)), s);
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
    const int d = 32 * wg + col;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vt + d * kRowStride + 16 * ((2 * kk + hf) ^ (d >> 4)));
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
  // the groups' V^T and P^T (r <= 16 heads) buffers; during the selection
  // they hold its scratch: the waves' best kp (list w at w * kp) and the
  // per-wave top-k scratch
  constexpr int kVt = kHeadDim * kRowStride, kPt = 16 * kRowStride;
  constexpr int kScr = 64 + 64 * NK;
  __shared__ __align__(16) char abuf[2 * kVt + 2 * kPt];
  static_assert(8 * (8 * 32 + 8 * kScr) <= 2 * kVt + 2 * kPt, "selection scratch exceeds the attention buffers");
  char (*vt)[kVt] = reinterpret_cast<char (*)[kVt]>(abuf);
  char (*pt)[kPt] = reinterpret_cast<char (*)[kPt]>(abuf + 2 * kVt);
  int64_t* wbest = reinterpret_cast<int64_t*>(abuf);
  int64_t (*wscr)[kScr] = reinterpret_cast<int64_t (*)[kScr]>(abuf + 8 * 8 * 32);
  __shared__ int sorted[33];
  __shared__ float red_m[2][4][32];
  __shared__ float red_l[2][4][32];
  __shared__ __align__(16) char qs[32 * kRowStride];  // query rows (bf16), rows >= r zero
  __shared__ __align__(16) char ktile[8][32 * kRowStride];  // each wave's K rows of the current slot
  // after the slots, the odd-slot group's state for the final merge, in the
  // attention buffers (every wave is past its last read of them)
  static_assert(16 * kHeadDim * 4 + 16 * 2 * 4 <= 2 * kVt, "merge state exceeds the attention buffers");
  float (*xo)[kHeadDim] = reinterpret_cast<float (*)[kHeadDim]>(abuf);
  float (*xml)[2] = reinterpret_cast<float (*)[2]>(abuf + 16 * kHeadDim * 4);

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
  const int L = sh.lens != nullptr ? sh.lens[b] : sh.L;  // the unit's cached tokens
  if (L < 1 || L > sh.Lc) {
    // a length outside 1 .. capacity (lengths read from device memory are
    // not checked on the host): no selection (-1), a zero output row, or a
    // workgroup state with no key (max -inf, sum 0), which the merge turns
    // into zeros; nothing else is read.  The test is the same for the whole
    // workgroup.
    if (part == 0 && tid < K) sel_out[(size_t)u * K + tid] = -1;
    if (tid < r * 32) {
      const int h = tid >> 5, d0 = 4 * (tid & 31);
      if (n_split > 1) {
        float* srow = state + (((size_t)u * n_split + part) * r + h) * (kHeadDim + 2);
        *reinterpret_cast<f32x4_t*>(srow + d0) = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (d0 == 0) {
          srow[kHeadDim] = -__builtin_inff();
          srow[kHeadDim + 1] = 0.f;
        }
      } else {
        *reinterpret_cast<u32x2_t*>(out + ((size_t)b * sh.Hq + g * r + h) * kHeadDim + d0) = u32x2_t{0u, 0u};
      }
    }
    return;
  }
  const int own = (L - 1) / sh.bs;  // candidates are blocks 0 .. own - 1
  // the unit's query rows in LDS (rows r .. 31 zero), read per slot
  if (tid < 32 * 16) {
    const int row = tid >> 4, ch = tid & 15;
    u32x4_t v4 = u32x4_t{0u, 0u, 0u, 0u};
    if (row < r) v4 = *reinterpret_cast<const u32x4_t*>(q + ((size_t)b * sh.Hq + g * r + row) * kHeadDim + 8 * ch);
    *reinterpret_cast<u32x4_t*>(qs + row * kRowStride + 16 * ch) = v4;
  }

  // ---- selection
  if (kp > 0) {
    // the 64-byte summary of candidate c is read as four 16-byte quarters by
    // the four lanes of a quad (each wave load covers 16 whole summaries);
    // thread tid takes quarter tid % 4 of candidates 128 i + tid / 4 and
    // keeps the keys of i = 4 m + tid % 4 (candidates 512 m + 128 (tid % 4)
    // + tid / 4), m < NK
    const int qq = tid & 3;
    const i32x4_t qv = reinterpret_cast<const i32x4_t*>(q_idx + (size_t)u * kIdxDim)[qq];
    const int8_t* kb = block_keys + (size_t)u * sh.nbc * kIdxDim + 16 * qq;
    int64_t keys[NK];
#pragma unroll
    for (int m = 0; m < NK; ++m) keys[m] = kNoKey;
    // the loads of 16 steps are issued before the first use (rows clamped to
    // a valid candidate, results past the own block dropped), so the
    // summaries take one memory round trip per 16 steps instead of one per
    // step (behind a per-step branch the compiler waited for each load;
    // measured on MI355X: decode kernel 35.7 -> 33.5 us on the decode
    // workload)
#pragma unroll
    for (int i0 = 0; i0 < 4 * NK; i0 += 16) {
      i32x4_t a[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = max(0, min(128 * (i0 + i) + (tid >> 2), own - 1));
        a[i] = *reinterpret_cast<const i32x4_t*>(kb + (size_t)c * kIdxDim);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int c = 128 * (i0 + i) + (tid >> 2);
        int sc = 0;
        sc = sdot4(qv.x, a[i].x, sc);
        sc = sdot4(qv.y, a[i].y, sc);
        sc = sdot4(qv.z, a[i].z, sc);
        sc = sdot4(qv.w, a[i].w, sc);
        sc = quad_sum(sc);  // every lane takes part: no branch around it
        if (((i0 + i) & 3) == qq && c < own) keys[(i0 + i) >> 2] = rank_key(sc, c);
      }
    }
    wave_topk_rank(keys, kp, wscr[w], wbest + w * kp);
  }
  __syncthreads();
  // the best kp of the 8 waves' lists (n2 = 8 kp keys): key ci is ranked
  // against the whole list by the four threads 4 ci .. 4 ci + 3, each over
  // a quarter of it
  int* kept = reinterpret_cast<int*>(wscr[0]);  // the kept blocks, by rank
  const int n_valid = min(kp, own);             // valid keys that exist
  {
    const int n2 = 8 * kp;
    const int qq = tid & 3;
    const int per = (n2 + 3) >> 2;
    const int j0 = qq * per, j1 = min(n2, j0 + per);
    const int passes = (n2 + 127) >> 7;  // the same for every thread (quad sums)
    for (int pz = 0; pz < passes; ++pz) {
      const int ci = 128 * pz + (tid >> 2);
      const int64_t x = ci < n2 ? wbest[ci] : kNoKey;
      int rk = 0;
#pragma unroll 4
      for (int jj = j0; jj < j1; ++jj) rk += wbest[jj] > x ? 1 : 0;
      rk = quad_sum(rk);
      if (qq == 0 && x != kNoKey && rk < kp) kept[rk] = key_block(x);
    }
  }
  __syncthreads();
  // slot order: the kept blocks ascending, the own block, then empty (-1)
  if (tid < n_valid) {
    const int blk = kept[tid];
    int pos = 0;
    for (int i = 0; i < n_valid; ++i) pos += kept[i] < blk ? 1 : 0;
    sorted[pos] = blk;
  }
  if (tid == n_valid) sorted[n_valid] = own;
  if (tid > n_valid && tid <= 32) sorted[tid] = -1;
  __syncthreads();
  if (part == 0 && tid < K) sel_out[(size_t)u * K + tid] = sorted[tid];

  // ---- attention: group gp takes slots gp, gp + 2, ...; a group's next
  // slot loads while the current one is computed (two register sets, so
  // that no load result is moved between registers)
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
    dec_load_block(sh, k_cache, v_cache, u, L, j >= 0 ? j : own, gt, wg, lane, blk);
  };
  const int per_wg = 2 * n_split;
  const int n_rounds = (K + per_wg - 1) / per_wg;  // the same for both groups (barriers)
  DecBlock A, B;
  load_round(0, A);
  for (int rd = 0; rd < n_rounds; rd += 2) {
    load_round(rd + 1, B);
    if (rd > 0) __syncthreads();  // the previous slot's LDS reads are done
    dec_slot(sh, A, L, slot_block(rd), qs, vt[gp], pt[gp], ktile[w], red_m[gp], red_l[gp], gt, wg, lane, st);
    if (rd + 1 >= n_rounds) break;
    load_round(rd + 2, A);
    __syncthreads();
    dec_slot(sh, B, L, slot_block(rd + 1), qs, vt[gp], pt[gp], ktile[w], red_m[gp], red_l[gp], gt, wg, lane, st);
  }

  // ---- merge of the two groups' states -> out = o / l
  __syncthreads();  // xo / xml overlay the attention buffers
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

// Merge of a unit's two workgroup states: one workgroup per unit, a thread
// per (head, 4 head dims): out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// Every load is issued before the first use.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ state,
                                                           uint16_t* __restrict__ out, DecodeShape sh) {
  const int u = blockIdx.x;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int r = sh.r;
  for (int it = threadIdx.x; it < r * 32; it += 256) {
    const int h = it >> 5;
    const int d0 = (it & 31) * 4;
    const float* s0 = state + (((size_t)u * 2 + 0) * r + h) * (kHeadDim + 2);
    const float* s1 = state + (((size_t)u * 2 + 1) * r + h) * (kHeadDim + 2);
    const float m0 = s0[kHeadDim], l0 = s0[kHeadDim + 1];
    const float m1 = s1[kHeadDim], l1 = s1[kHeadDim + 1];
    const f32x4_t o0 = *reinterpret_cast<const f32x4_t*>(s0 + d0);
    const f32x4_t o1 = *reinterpret_cast<const f32x4_t*>(s1 + d0);
    // a share with no kept block has m = -inf, weight 0 (M is finite: the
    // own block is always kept, unless the unit's length was out of range
    // and both states hold no key: then the row is zero)
    const float M = fmaxf(m0, m1);
    const bool none = M == -__builtin_inff();
    const float Mu = none ? 0.f : M;
    const float w0 = fast_exp2(m0 - Mu), w1 = fast_exp2(m1 - Mu);
    const float inv = none ? 0.f : 1.0f / fmaf(w0, l0, w1 * l1);
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = none ? 0.f : fmaf(w0, o0[e], w1 * o1[e]) * inv;
    u32x2_t wv;
    wv.x = pack_bf16x2(v[0], v[1]);
    wv.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2_t*>(out + ((size_t)b * sh.Hq + g * r + h) * kHeadDim + d0) = wv;
  }
}

// Append of one token per (batch, group) unit at position pos: its K and V
// rows go to the caches, its index key is added to the running int32 sums
// of its block (which restart when pos opens a block) and the block's
// summary becomes the floor-mean of the sums over the block's pos % bs + 1
// tokens, so the summaries always equal the pooling of the cache prefix.
__global__ __launch_bounds__(64) void append_kernel(const uint16_t* __restrict__ k_new,
                                                    const uint16_t* __restrict__ v_new,
                                                    const int8_t* __restrict__ k_idx_new,
                                                    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
                                                    int32_t* __restrict__ open_sums,
                                                    int8_t* __restrict__ block_keys, DecodeShape sh, int pos) {
  const int u = blockIdx.x;
  const int l = threadIdx.x;
  if (sh.lens != nullptr) {
    pos = sh.lens[u / sh.G] - 1;  // the unit's own position
    if (pos < 0 || pos >= sh.Lc) return;  // a length outside 1 .. capacity: nothing appended
  }
  const size_t row = ((size_t)u * sh.Lc + pos) * kHeadDim;
  if (l < 16)
    reinterpret_cast<u32x4_t*>(k_cache + row)[l] = reinterpret_cast<const u32x4_t*>(k_new + (size_t)u * kHeadDim)[l];
  else if (l < 32)
    reinterpret_cast<u32x4_t*>(v_cache + row)[l - 16] =
        reinterpret_cast<const u32x4_t*>(v_new + (size_t)u * kHeadDim)[l - 16];
  const int j = pos / sh.bs;
  const int n = pos - j * sh.bs + 1;  // tokens of block j after the append
  const int s = (n == 1 ? 0 : open_sums[(size_t)u * kIdxDim + l]) + (int)k_idx_new[(size_t)u * kIdxDim + l];
  open_sums[(size_t)u * kIdxDim + l] = s;
  block_keys[((size_t)u * sh.nbc + j) * kIdxDim + l] = (int8_t)floor_div(s, n);
}

// Per-sequence lengths into device memory: the values travel in the kernel
// arguments (a launch copies them), so no host memory is read after the
// launch and no copy waits for the stream.
__global__ __launch_bounds__(256) void set_lengths_kernel(int32_t* __restrict__ dst, LengthBatch v, int n) {
  for (int i = threadIdx.x; i < n; i += 256) dst[i] = v.v[i];
}

// Scratch of the allocation-free decode entry point: one array per device,
// held until the process ends.  Host code never passes `scratch` itself to
// a kernel (on the host that name is a stand-in, not a device address); it
// passes the address decode_scratch() looked up for the current device.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // by device ordinal; null = not looked up yet

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeShape& sh, const uint16_t* q, const int8_t* q_idx, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int8_t* block_keys, int32_t* sel_out, uint16_t* out,
                         float* state, int n_split, hipStream_t st) {
  if (n_split < 1 || n_split > 2) return hipErrorInvalidValue;  // the merge combines two states
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

hipError_t launch_set_lengths(int32_t* dst, const int32_t* lengths, int n, hipStream_t st) {
  for (int i0 = 0; i0 < n; i0 += kLengthBatch) {
    LengthBatch v;
    const int m = n - i0 < kLengthBatch ? n - i0 : kLengthBatch;
    for (int i = 0; i < m; ++i) v.v[i] = lengths[i0 + i];
    hipLaunchKernelGGL(set_lengths_kernel, dim3(1), dim3(256), 0, st, dst + i0, v, m);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_append(const DecodeShape& sh, const uint16_t* k_new, const uint16_t* v_new,
                         const int8_t* k_idx_new, uint16_t* k_cache, uint16_t* v_cache, int32_t* open_sums,
                         int8_t* block_keys, int pos, hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3(sh.B * sh.G), dim3(64), 0, st, k_new, v_new, k_idx_new, k_cache, v_cache,
                     open_sums, block_keys, sh, pos);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeShape& sh, const float* state, int n_split, uint16_t* out,
                               hipStream_t st) {
  if (n_split != 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(sh.B * sh.G), dim3(256), 0, st, state, out, sh);
  return hipGetLastError();
}

}  // namespace msa
