// MSA index branch: block-summary pooling and the per-(query, group) top-k.
//
// The index branch is a cheap scorer over KV blocks whose best k blocks are
// kept independently for every GQA group ("深度解析 MiniMax-M3：稀疏注意力机制、
// 基准测试与 API 集成指南", section "架构核心：MoE 与 MSA 的深度融合", item 1), and
// its top-k needs no exponentials (wiki.500nian.com digest of "MiniMax M3
// Review: 1M Tokens, 15X Faster AI Agents", flowchart node "exp-free Top-k").
// The scorer used here: int8 summaries = floor-mean of each block's int8
// index keys, score = exact int32 dot product, candidates = blocks strictly
// before the query's block, ties to the lower block index, own block added.

#include "msa_device.h"
#include "msa_kernels.h"

#include <limits.h>

namespace msa {
namespace {

// ---------------------------------------------------------------------------
// Pooling: one wave per (unit, block j0 .. nb - 1) of the first S tokens.  Lane (row, col)
// = (lane / 16, lane % 16) sums dword `col` (4 index dims) of tokens row,
// row + 4, ...; the four rows are folded with lane shuffles.  HBM-bound
// streaming read.  k_idx rows of a unit are s_stride apart, summaries
// nb_stride apart.  open_sums (optional): the int32 sums of the block the
// next token goes to, tokens nb' * bs .. S - 1 with nb' = floor(S / bs)
// (zero when S is a multiple of bs).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pool_kernel(const int8_t* __restrict__ k_idx,
                                                   int8_t* __restrict__ block_keys, int units,
                                                   int S, int bs, int nb, long s_stride, int nb_stride,
                                                   int32_t* __restrict__ open_sums, int j0) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nbp = nb - j0;  // blocks pooled per unit
  if (wid >= units * nbp) return;
  const int lane = threadIdx.x & 63;
  const int u = wid / nbp;
  const int j = j0 + (wid - u * nbp);
  const int t0 = j * bs;
  const int n = min(bs, S - t0);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(k_idx + ((size_t)u * s_stride + t0) * kIdxDim);
  const int col = lane & 15;
  const int row = lane >> 4;
  int s0 = 0, s1 = 0, s2 = 0, s3 = 0;
#pragma unroll 8
  for (int tt = row; tt < n; tt += 4) {
    const uint32_t w = __builtin_nontemporal_load(base + tt * 16 + col);
    s0 += sx8(w, 0);
    s1 += sx8(w, 1);
    s2 += sx8(w, 2);
    s3 += sx8(w, 3);
  }
  s0 += __shfl_xor(s0, 16);
  s1 += __shfl_xor(s1, 16);
  s2 += __shfl_xor(s2, 16);
  s3 += __shfl_xor(s3, 16);
  s0 += __shfl_xor(s0, 32);
  s1 += __shfl_xor(s1, 32);
  s2 += __shfl_xor(s2, 32);
  s3 += __shfl_xor(s3, 32);
  if (row == 0) {
    const uint32_t packed = (uint32_t)(floor_div(s0, n) & 0xff) |
                            ((uint32_t)(floor_div(s1, n) & 0xff) << 8) |
                            ((uint32_t)(floor_div(s2, n) & 0xff) << 16) |
                            ((uint32_t)(floor_div(s3, n) & 0xff) << 24);
    reinterpret_cast<uint32_t*>(block_keys + ((size_t)u * nb_stride + j) * kIdxDim)[col] = packed;
    if (open_sums != nullptr && j == nb - 1) {
      const bool partial = n < bs;
      i32x4_t v4;
      v4.x = partial ? s0 : 0;
      v4.y = partial ? s1 : 0;
      v4.z = partial ? s2 : 0;
      v4.w = partial ? s3 : 0;
      reinterpret_cast<i32x4_t*>(open_sums + (size_t)u * kIdxDim)[col] = v4;
    }
  }
}

// Ascending bitonic sort of N (a power of two) register values.
template <int N>
__device__ __forceinline__ void bitonic_sort(int (&x)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const int a = x[i], b = x[l];
          const bool up = (i & k) == 0;
          x[i] = up ? min(a, b) : max(a, b);
          x[l] = up ? max(a, b) : min(a, b);
        }
      }
    }
  }
}

template <int N>
struct NextPow2 {
  static constexpr int v = N <= 1 ? 1 : N <= 2 ? 2 : N <= 4 ? 4 : N <= 8 ? 8 : N <= 16 ? 16 : 32;
};

// ---------------------------------------------------------------------------
// Scores + top-k: one lane per query token, 256 consecutive tokens of one
// (batch, group) unit per workgroup.  Summaries of the candidate blocks are
// staged through LDS in chunks and read as wave-wide broadcasts; each lane
// scores every candidate with 16 v_dot4 and keeps a sorted register list of
// its best KCAP (score desc, index asc).  Candidates arrive in ascending
// block order, so a candidate can enter the list only when its score beats
// the list's last score strictly: an equal score belongs to a lower index
// already in the list.  KCAP >= top_k - 1; the best top_k - 1 are taken
// from it.  Query row t (of S per unit) is the token at position pos0 + t.
//
// The lanes of a wave hold different queries, so a sorted insertion run by
// one lane costs the whole wave.  A candidate that beats the lane's
// threshold (the list's last score when the list was last updated) is only
// appended to a short per-lane LDS buffer; the buffers are merged into the
// lists, in arrival order, when one of them fills and at the end.  A stale
// (lower) threshold lets more candidates through, never fewer, and the
// arrival order keeps the tie rule, so the lists are the same.
// ---------------------------------------------------------------------------
constexpr int kTopkBuf = 16;  // buffered candidates per lane

// Insertion of candidate (s, j) that arrives after every entry's candidate
// (a higher block index than all of them).
template <int KCAP>
__device__ __forceinline__ void topk_insert(int (&Ls)[KCAP], int (&Li)[KCAP], int s, int j) {
  if (s > Ls[KCAP - 1]) {
    // insert after every entry whose score is >= s (they all have a lower
    // block index), shifting the rest down by one
#pragma unroll
    for (int i = KCAP - 1; i >= 0; --i) {
      const bool keep = Ls[i] >= s;
      const bool prev_keep = (i == 0) ? true : (Ls[i - 1] >= s);
      const int ns = keep ? Ls[i] : (prev_keep ? s : Ls[i > 0 ? i - 1 : 0]);
      const int ni = keep ? Li[i] : (prev_keep ? j : Li[i > 0 ? i - 1 : 0]);
      Ls[i] = ns;
      Li[i] = ni;
    }
  }
}

template <int KCAP>
__global__ __launch_bounds__(256) void index_topk_kernel(const int8_t* __restrict__ q_idx,
                                                         const int8_t* __restrict__ block_keys,
                                                         int32_t* __restrict__ sel, int S,
                                                         int nb_stride, int bs_log2, int top_k, int pos0,
                                                         int q_stride, int sel_stride) {
  constexpr int CH = 256;  // summaries per LDS chunk (16 KiB)
  __shared__ i32x4_t sk[CH * 4];
  __shared__ int2 buf[kTopkBuf][256];  // per lane: (score, block) waiting for the list

  const int u = blockIdx.y;
  const int t0 = blockIdx.x * 256;
  const int t = t0 + (int)threadIdx.x;
  const bool live = t < S;
  const int tc = live ? t : S - 1;
  const int c = (pos0 + tc) >> bs_log2;  // own block = number of candidates
  const int c_last = (pos0 + min(S - 1, t0 + 255)) >> bs_log2;
  const int kp = top_k - 1;

  const i32x4_t* qp = reinterpret_cast<const i32x4_t*>(q_idx + ((size_t)u * q_stride + tc) * kIdxDim);
  const i32x4_t q0 = qp[0], q1 = qp[1], q2 = qp[2], q3 = qp[3];

  int Ls[KCAP], Li[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    Ls[i] = INT_MIN;
    Li[i] = -1;
  }
  int thr = INT_MIN;  // Ls[KCAP - 1] as of the last merge
  int nbuf = 0;
  auto merge_buf = [&]() {
    for (int i = 0; __any(i < nbuf); ++i) {
      if (i < nbuf) {
        const int2 e = buf[i][threadIdx.x];
        topk_insert<KCAP>(Ls, Li, e.x, e.y);
      }
    }
    nbuf = 0;
    thr = Ls[KCAP - 1];
  };

  const i32x4_t* kb = reinterpret_cast<const i32x4_t*>(block_keys + (size_t)u * nb_stride * kIdxDim);
  const int n_cand = kp > 0 ? c_last : 0;
  for (int base = 0; base < n_cand; base += CH) {
    const int n = min(CH, n_cand - base);
    __syncthreads();
    for (int i = threadIdx.x; i < n * 4; i += 256) sk[i] = kb[base * 4 + i];
    __syncthreads();
    for (int jj = 0; jj < n; ++jj) {
      const i32x4_t a0 = sk[4 * jj + 0], a1 = sk[4 * jj + 1];
      const i32x4_t a2 = sk[4 * jj + 2], a3 = sk[4 * jj + 3];
      int sa = 0, sb = 0;
      sa = sdot4(q0.x, a0.x, sa);
      sb = sdot4(q0.y, a0.y, sb);
      sa = sdot4(q0.z, a0.z, sa);
      sb = sdot4(q0.w, a0.w, sb);
      sa = sdot4(q1.x, a1.x, sa);
      sb = sdot4(q1.y, a1.y, sb);
      sa = sdot4(q1.z, a1.z, sa);
      sb = sdot4(q1.w, a1.w, sb);
      sa = sdot4(q2.x, a2.x, sa);
      sb = sdot4(q2.y, a2.y, sb);
      sa = sdot4(q2.z, a2.z, sa);
      sb = sdot4(q2.w, a2.w, sb);
      sa = sdot4(q3.x, a3.x, sa);
      sb = sdot4(q3.y, a3.y, sb);
      sa = sdot4(q3.z, a3.z, sa);
      sb = sdot4(q3.w, a3.w, sb);
      const int s = sa + sb;
      const int j = base + jj;
      if (j < c && s > thr) {
        buf[nbuf][threadIdx.x] = make_int2(s, j);
        ++nbuf;
      }
      if (__any(nbuf == kTopkBuf)) merge_buf();
    }
  }
  merge_buf();

  // best min(top_k - 1, c) candidates, ascending, then the own block
  const int n_valid = min(kp, c);
  constexpr int NP = NextPow2<KCAP>::v;
  int x[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) x[i] = (i < KCAP && i < n_valid) ? Li[i < KCAP ? i : 0] : INT_MAX;
  bitonic_sort<NP>(x);
  if (!live) return;
  int32_t* out = sel + ((size_t)u * sel_stride + t) * top_k;
#pragma unroll
  for (int i = 0; i <= KCAP; ++i) {
    if (i < top_k) {
      const int xv = (i < NP) ? x[i < NP ? i : 0] : INT_MAX;
      out[i] = (i < n_valid) ? xv : (i == n_valid ? c : -1);
    }
  }
}

// ---------------------------------------------------------------------------
// Scores + top-k.  A workgroup takes 128 consecutive query tokens of one
// (batch, group) unit, a wave 32 of them.  The int8 scores of 32 queries x
// 32 candidate blocks come from one exact integer contraction over the 64
// index dims on the matrix cores (v_mfma_i32_32x32x16_i8: block summaries
// staged in LDS as the A operand, the wave's query vectors as B), which
// leaves each lane the scores of one query (lane % 32) against 16 of the 32
// candidates (rows 8 (i / 4) + 4 (lane / 32) + i % 4).  Each lane keeps a
// sorted register list of its best KCAP (score desc, index asc) over its
// half of the candidates, which arrive in ascending block order: a
// candidate can enter only when its score beats the list's last score
// strictly (an equal score belongs to a lower index already in the list).
// The two half lists of a query are merged at the end with the full (score,
// index) order.  KCAP >= top_k - 1; the best top_k - 1 are taken.  Query row
// t (of S per unit) is the token at position pos0 + t.
//
// The lanes of a wave hold different lists, so a sorted insertion run by
// one lane costs the whole wave.  A candidate that beats the lane's
// threshold (the list's last score when the list was last updated) is only
// appended to a per-lane LDS buffer; the buffers are merged into the lists,
// in arrival order, before a tile could overflow one and at the end.  A
// stale (lower) threshold lets more candidates through, never fewer, and
// the arrival order keeps the tie rule, so the lists are the same.
//
// This single-sweep kernel serves what the two-sweep kernel below cannot:
// queries ranking more than 65408 blocks, and (flagged_only) the waves it
// flags for a score spread its keys cannot hold.
// ---------------------------------------------------------------------------
constexpr int kTopkBufMfma = 24;    // buffered candidates per lane (a tile adds at most 16)
constexpr int kSumStride = 64 + 8;  // bytes per staged summary (18 dwords: the 8-byte A reads of 16 rows hit 32 banks)

// Insertion in the full order: a higher score first, at equal scores the
// lower block index first.
__device__ __forceinline__ bool topk_before(int s1, int j1, int s2, int j2) {
  return s1 > s2 || (s1 == s2 && j1 < j2);
}
template <int KCAP>
__device__ __forceinline__ void topk_insert_any(int (&Ls)[KCAP], int (&Li)[KCAP], int s, int j) {
  if (topk_before(s, j, Ls[KCAP - 1], Li[KCAP - 1])) {
#pragma unroll
    for (int i = KCAP - 1; i >= 0; --i) {
      const bool keep = topk_before(Ls[i], Li[i], s, j);
      const bool prev_keep = (i == 0) ? true : topk_before(Ls[i - 1], Li[i - 1], s, j);
      const int ns = keep ? Ls[i] : (prev_keep ? s : Ls[i > 0 ? i - 1 : 0]);
      const int ni = keep ? Li[i] : (prev_keep ? j : Li[i > 0 ? i - 1 : 0]);
      Ls[i] = ns;
      Li[i] = ni;
    }
  }
}

template <int KCAP>
__global__ __launch_bounds__(256) void index_topk_mfma_kernel(const int8_t* __restrict__ q_idx,
                                                         const int8_t* __restrict__ block_keys,
                                                         int32_t* __restrict__ sel, int S,
                                                         int nb_stride, int bs_log2, int top_k, int pos0,
                                                         int q_stride, int sel_stride, int flagged_only) {
  // flagged_only: run only where the two-sweep kernel left a wave's rows
  // flagged (first entry -2), i.e. for workgroups holding such a wave
  if (flagged_only) {
    bool any = false;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const int tw = blockIdx.x * 128 + 32 * w4;
      if (tw < S) any |= sel[((size_t)blockIdx.y * sel_stride + tw) * top_k] == -2;
    }
    __syncthreads();   // every flag is read before any row is rewritten
    if (!any) return;  // the same for every thread of the workgroup
  }
  // 128 summaries per LDS chunk and 4-byte buffer entries: 33 KiB of LDS,
  // so four workgroups share a CU (the kernel waits on its MFMA results,
  // LDS reads and wave-wide tests far more than it issues; measured on
  // MI355X, 1M tokens: 23.4 ms with 66 KiB and two workgroups per CU,
  // 16.5 ms with four)
  constexpr int CH = 128;
  __shared__ __align__(16) char sk[CH * kSumStride];
  // per lane: score * 256 + (block - base), waiting for the list; |score| <=
  // 64 * 128 * 128 = 2^20, so the packed entry fits 29 bits and a sign
  __shared__ int buf[kTopkBufMfma][256];

  const int u = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hf = lane >> 5;
  const int col = lane & 31;
  const int t0 = blockIdx.x * 128;
  const int t = t0 + 32 * w + col;  // this lane's query (in both lane halves)
  const bool live = t < S;
  const int tc = live ? t : S - 1;
  const int c = (pos0 + tc) >> bs_log2;  // own block = number of candidates
  const int c_last = (pos0 + min(S - 1, t0 + 127)) >> bs_log2;
  const int kp = top_k - 1;

  // B operand: the query's index vector, bytes 16 ks + 8 hf .. + 7 at k-step ks
  const int8_t* qrow = q_idx + ((size_t)u * q_stride + tc) * kIdxDim;
  long qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qb[ks] = *reinterpret_cast<const long*>(qrow + 16 * ks + 8 * hf);

  int Ls[KCAP], Li[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    Ls[i] = INT_MIN;
    Li[i] = -1;
  }
  int thr = INT_MIN;  // Ls[KCAP - 1] as of the last merge
  int nbuf = 0;
  int base = 0;  // first candidate of the current chunk (entries hold block - base)
  auto merge_buf = [&]() {
    for (int i = 0; __any(i < nbuf); ++i) {
      if (i < nbuf) {
        const int e = buf[i][tid];
        topk_insert<KCAP>(Ls, Li, e >> 8, base + (e & 255));
      }
    }
    nbuf = 0;
    thr = Ls[KCAP - 1];
  };

  const long* kb8 = reinterpret_cast<const long*>(block_keys + (size_t)u * nb_stride * kIdxDim);
  const int n_cand = kp > 0 ? c_last : 0;
  // the next chunk's summaries (8 bytes x 8 per thread) load while the
  // current chunk is scored
  long pre[CH * 8 / 256];
  auto fetch = [&](int from) {
    const int n = min(CH, n_cand - from);
#pragma unroll
    for (int m = 0; m < CH * 8 / 256; ++m) {
      const int i = tid + 256 * m;
      pre[m] = i < n * 8 ? kb8[(size_t)from * 8 + i] : 0;
    }
  };
  if (n_cand > 0) fetch(0);
  for (base = 0; base < n_cand; base += CH) {
    const int n = min(CH, n_cand - base);
    __syncthreads();
#pragma unroll
    for (int m = 0; m < CH * 8 / 256; ++m) {
      const int i = tid + 256 * m;
      *reinterpret_cast<long*>(sk + (i >> 3) * kSumStride + 8 * (i & 7)) = pre[m];
    }
    __syncthreads();
    if (base + CH < n_cand) fetch(base + CH);
    for (int tile = 0; tile < n; tile += 32) {
      // rows past the chunk's n hold stale summaries: their candidates are
      // >= c for every query of the workgroup and are skipped below
      const char* arow = sk + (tile + col) * kSumStride + 8 * hf;
      i32x16_t acc = i32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = __builtin_amdgcn_mfma_i32_32x32x16_i8(*reinterpret_cast<const long*>(arow + 16 * ks), qb[ks], acc, 0,
                                                    0, 0);
      // most tiles, once the lists have filled, hold no candidate above any
      // lane's threshold: one test for the wave skips the 16 per-candidate ones
      int best = INT_MIN;
#pragma unroll
      for (int i = 0; i < 16; ++i) best = max(best, acc[i]);
      if (!__any(best > thr)) continue;
      if (__any(nbuf > kTopkBufMfma - 16)) merge_buf();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = base + tile + c_row(i, hf);
        if (j < c && acc[i] > thr) {
          buf[nbuf][tid] = acc[i] * 256 | (j - base);
          ++nbuf;
        }
      }
    }
    merge_buf();  // entries hold block - base: the buffer empties with its chunk
  }
  merge_buf();

  // the other half's list (lane + 32) joins this lane's in the full order
#pragma unroll
  for (int i = 0; i < KCAP; ++i) {
    const int os = __shfl(Ls[i], lane ^ 32);
    const int oi = __shfl(Li[i], lane ^ 32);
    if (hf == 0 && oi >= 0) topk_insert_any<KCAP>(Ls, Li, os, oi);
  }
  if (hf != 0) return;

  // best min(top_k - 1, c) candidates, ascending, then the own block
  const int n_valid = min(kp, c);
  constexpr int NP = NextPow2<KCAP>::v;
  int x[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) x[i] = (i < KCAP && i < n_valid) ? Li[i < KCAP ? i : 0] : INT_MAX;
  bitonic_sort<NP>(x);
  if (!live) return;
  int32_t* out = sel + ((size_t)u * sel_stride + t) * top_k;
#pragma unroll
  for (int i = 0; i <= KCAP; ++i) {
    if (i < top_k) {
      const int xv = (i < NP) ? x[i < NP ? i : 0] : INT_MAX;
      out[i] = (i < n_valid) ? xv : (i == n_valid ? c : -1);
    }
  }
}

// ---------------------------------------------------------------------------
// Scores + top-k in two sweeps over the candidates.  Layout as above: a
// workgroup takes 128 consecutive query tokens of one (batch, group) unit, a
// wave 32 of them, and one tile of 32 candidates x 32 queries comes from two
// exact integer contractions (v_mfma_i32_32x32x32_i8, 32 index dims each),
// lane (hf, col) holding query col's scores of candidates
// 8 (i / 4) + 4 hf + i % 4 of the tile.
//
// Sweep 1 keeps, per lane, the maximum of each of its 16 register slots over
// all tiles: 32 maxima per query over disjoint candidate sets.  Their top_k -
// 1'th largest, L, is a lower bound on the query's (top_k - 1)'th best score
// (that many distinct candidates reach it), so no candidate scoring below L
// can be selected.  Sweep 2 scores the candidates again and appends to a
// per-lane ring in LDS the scores of each group of four consecutive
// candidates (slots 4 g .. 4 g + 3) whose maximum reaches the filter bound;
// few do, so the per-candidate work happens for few.  When a tile would
// overflow some lane's ring, every lane moves its oldest entry into a
// per-lane list of the best KCAP (and the rings are emptied at the end),
// ranked by the unsigned key ((s - L + 1) << 16) + 65535 - j, which orders
// by score, then by lower block, and makes an insertion one median per list
// slot; a key below 65536 stands for no candidate.  The two half lists of a
// query are joined at the end.  Whenever the list is full, the bound rises
// to one above its last score: later candidates have higher block indices
// and cannot displace an entry they only tie.
//
// A query with fewer than top_k - 1 candidates keeps them all (key score
// part 1).  A wave where some query's best score is 65535 or more above its
// L cannot use the keys: it writes -2 into the first entry of its rows and
// index_topk_mfma_kernel, launched after this one with flagged_only set,
// recomputes the workgroups that hold such a wave.  The host sends queries
// that rank more than 65408 blocks (so that even the masked rows past the
// last candidate keep block indices below 65536) to index_topk_mfma_kernel
// directly.
// ---------------------------------------------------------------------------
constexpr int kSumStride32 = 80;  // bytes per staged summary (20 dwords: the 16-byte A reads of 16 rows hit distinct banks)
constexpr int kEntCap = 4;        // buffered candidate groups per lane (with 256-summary chunks: 40 KiB of
                                  // LDS per workgroup, four per CU; measured on MI355X at 1M tokens against
                                  // 128-summary chunks and 6 entries: 7.23 -> 6.92 ms, half the barriers)
constexpr int kMasked = -(1 << 30);  // score of a non-candidate (every real score is within +-2^20)

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

// Insertion of a key into a list of distinct keys sorted descending
// (unsigned): slot i becomes the median of itself, the slot before and the
// key, i.e. max(slot, min(slot before, key)).
template <int KCAP>
__device__ __forceinline__ void key_insert(int (&K)[KCAP], uint32_t x) {
#pragma unroll
  for (int i = KCAP - 1; i > 0; --i) K[i] = (int)umed3((uint32_t)K[i], (uint32_t)K[i - 1], x);
  K[0] = (int)max((uint32_t)K[0], x);
}

// Ascending sort of a bitonic sequence of N (a power of two) values.
template <int N>
__device__ __forceinline__ void bitonic_merge(int (&x)[N]) {
#pragma unroll
  for (int j = N >> 1; j > 0; j >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int l = i ^ j;
      if (l > i) {
        const int a = x[i], b = x[l];
        x[i] = min(a, b);
        x[l] = max(a, b);
      }
    }
  }
}

template <int KCAP>
__global__ __launch_bounds__(256) void index_topk_bound_kernel(const int8_t* __restrict__ q_idx,
                                                               const int8_t* __restrict__ block_keys,
                                                               int32_t* __restrict__ sel, int S, int nb_stride,
                                                               int bs_log2, int top_k, int pos0, int q_stride,
                                                               int sel_stride) {
  constexpr int CH = 256;  // summaries per LDS chunk
  __shared__ __align__(16) char sk[CH * kSumStride32];
  __shared__ i32x4_t ent[kEntCap][256];  // the four scores of a buffered group
  __shared__ int entj[kEntCap][256];     // its first block

  const int u = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hf = lane >> 5;
  const int col = lane & 31;
  const int t0 = blockIdx.x * 128;
  const int t = t0 + 32 * w + col;  // this lane's query (in both lane halves)
  const bool live = t < S;
  const int tc = live ? t : S - 1;
  const int c = (pos0 + tc) >> bs_log2;                           // own block = number of candidates
  const int c_lo = (pos0 + min(S - 1, t0 + 32 * w)) >> bs_log2;   // the wave's smallest own block
  const int c_last = (pos0 + min(S - 1, t0 + 127)) >> bs_log2;    // the workgroup's largest
  const int kp = top_k - 1;

  // B operand: the query's index bytes 32 ks + 16 hf .. + 15 at k-step ks
  const int8_t* qrow = q_idx + ((size_t)u * q_stride + tc) * kIdxDim;
  const i32x4_t qb0 = *reinterpret_cast<const i32x4_t*>(qrow + 16 * hf);
  const i32x4_t qb1 = *reinterpret_cast<const i32x4_t*>(qrow + 32 + 16 * hf);

  const i32x4_t* kb = reinterpret_cast<const i32x4_t*>(block_keys + (size_t)u * nb_stride * kIdxDim);
  const int n_cand = kp > 0 ? c_last : 0;
  // the next chunk's summaries (16 bytes x 4 per thread) load while the
  // current chunk is scored
  i32x4_t pre[CH * 4 / 256];
  auto fetch = [&](int from) {
    const int n = min(CH, n_cand - from);
#pragma unroll
    for (int m = 0; m < CH * 4 / 256; ++m) {
      const int i = tid + 256 * m;
      pre[m] = i < n * 4 ? kb[(size_t)from * 4 + i] : i32x4_t{};
    }
  };
  // one sweep: body(j0, acc) for every tile, acc[i] = the score of candidate
  // j0 + c_row(i, hf), kMasked where that is not before the query's block
  // (rows past a chunk's end hold stale summaries; they are all masked)
  auto sweep = [&](auto&& body) {
    if (n_cand > 0) fetch(0);
    for (int base = 0; base < n_cand; base += CH) {
      const int n = min(CH, n_cand - base);
      __syncthreads();
#pragma unroll
      for (int m = 0; m < CH * 4 / 256; ++m) {
        const int i = tid + 256 * m;
        *reinterpret_cast<i32x4_t*>(sk + (i >> 2) * kSumStride32 + 16 * (i & 3)) = pre[m];
      }
      __syncthreads();
      if (base + CH < n_cand) fetch(base + CH);
      // tiles in pairs, so that one tile's contractions run while the other
      // tile's scores are used (a pair past n holds only masked rows)
      for (int tile = 0; tile < n; tile += 64) {
        i32x16_t acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const char* arow = sk + (tile + 32 * h + col) * kSumStride32 + 16 * hf;
          acc[h] = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const i32x4_t*>(arow), qb0, i32x16_t{},
                                                         0, 0, 0);
          acc[h] = __builtin_amdgcn_mfma_i32_32x32x32_i8(*reinterpret_cast<const i32x4_t*>(arow + 32), qb1, acc[h],
                                                         0, 0, 0);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j0 = base + tile + 32 * h;
          if (j0 + 32 > c_lo) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (j0 + c_row(i, hf) >= c) acc[h][i] = kMasked;
          }
          body(j0, acc[h]);
        }
      }
    }
  };

  // sweep 1: slot maxima, then L = the kp'th largest of the query's 32
  int bm[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) bm[i] = kMasked;
  sweep([&](int, const i32x16_t& acc) {
#pragma unroll
    for (int i = 0; i < 16; ++i) bm[i] = max(bm[i], acc[i]);
  });
  bitonic_sort<16>(bm);
  int m32[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m32[i] = bm[i];
    m32[16 + i] = __shfl_xor(bm[15 - i], 32);  // the other half's, descending: a bitonic sequence
  }
  bitonic_merge<32>(m32);
  int L = INT_MIN;
#pragma unroll
  for (int i = 1; i < 32; ++i)
    if (i == 32 - kp) L = m32[i];
  const int U = m32[31];
  // fewer than kp candidates (L undefined): all are kept, key score part 1
  const bool all_in = L <= kMasked;
  const bool narrow = __all(all_in || U - L < 65535);

  // sweep 2: groups reaching the bound are buffered in a per-lane ring; when
  // a tile would overflow some lane's ring, every lane moves its oldest
  // entry into its list, as often as needed, and at the end the rings are
  // emptied.  A wave whose scores do not fit the keys still sweeps (the
  // workgroup's barriers need it) but buffers nothing, and flags its rows
  // for the single-sweep kernel.
  int K[KCAP];  // keys, descending (unsigned); below 65536: no candidate
#pragma unroll
  for (int i = 0; i < KCAP; ++i) K[i] = 0;
  int lf = !narrow ? INT_MAX : all_in ? kMasked + 1 : L;  // filter bound
  // key of score sc: ((clamp(sc - bias, 0, cap)) << 16) + 65535 - j; the
  // clamp's 0 marks no candidate (below L, or not before the query's block)
  const int bias = all_in ? kMasked + 1 : L - 1;
  const int cap = all_in ? 1 : 65535;
  int head = 0, cnt = 0;  // the ring: entries head .. head + cnt - 1 (mod kEntCap)
  auto drain_one = [&]() {
    // a lane with an empty ring reads a stale (or never written) slot: its
    // clamp bound 0 and block 0 make every key of it below 65536
    const bool has = cnt > 0;
    const i32x4_t s4 = ent[head][tid];
    const int jb = has ? entj[head][tid] : 0;
    const int cap_e = has ? cap : 0;
    const uint32_t lo = (uint32_t)(65535 - jb);
    uint32_t kq[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int d = min(max((int)((uint32_t)s4[r] - (uint32_t)bias), 0), cap_e);
      kq[r] = ((uint32_t)d << 16) + (lo - (uint32_t)r);
    }
    // the entry's keys, descending; a group rarely holds more than one
    // candidate of note, so the later insertions are skipped unless some
    // lane has one
    auto cx = [&](int x, int y) {
      const uint32_t p = kq[x], q = kq[y];
      kq[x] = max(p, q);
      kq[y] = min(p, q);
    };
    cx(0, 1);
    cx(2, 3);
    cx(0, 2);
    cx(1, 3);
    cx(1, 2);
    key_insert<KCAP>(K, kq[0]);
    if (__any(kq[1] >= 65536u)) {
      key_insert<KCAP>(K, kq[1]);
      if (__any(kq[2] >= 65536u)) {
        key_insert<KCAP>(K, kq[2]);
        if (__any(kq[3] >= 65536u)) key_insert<KCAP>(K, kq[3]);
      }
    }
    if (has) {
      head = head == kEntCap - 1 ? 0 : head + 1;
      --cnt;
    }
    // a full list: later candidates (higher blocks) must beat its last score
    const uint32_t kl = (uint32_t)K[KCAP - 1];
    if (kl >= 65536u && !all_in) lf = max(lf, (int)(kl >> 16) + L);
  };
  sweep([&](int j0, const i32x16_t& acc) {
    int gm[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) gm[g] = max(max(acc[4 * g], acc[4 * g + 1]), max(acc[4 * g + 2], acc[4 * g + 3]));
    const int npass = (gm[0] >= lf) + (gm[1] >= lf) + (gm[2] >= lf) + (gm[3] >= lf);
    // (a loop entered only when needed: the list's registers then move
    // through the loop's join only on tiles that drain)
    if (__any(cnt + npass > kEntCap)) {
      do {
        drain_one();
      } while (__any(cnt + npass > kEntCap));
    }
    int tail = head + cnt;
    tail = tail >= kEntCap ? tail - kEntCap : tail;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (gm[g] >= lf) {
        ent[tail][tid] = i32x4_t{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        entj[tail][tid] = j0 + 8 * g + 4 * hf;
        tail = tail == kEntCap - 1 ? 0 : tail + 1;
        ++cnt;
      }
    }
  });
  while (__any(cnt > 0)) drain_one();
  if (!narrow) {
    if (live && hf == 0) sel[((size_t)u * sel_stride + t) * top_k] = -2;
    return;
  }

  // the other half's list (lane + 32) joins this lane's: both, extended by
  // one empty key (KCAP + 1 is a power of two), are descending, so the
  // slot-wise maxima of one against the other reversed are the best KCAP + 1
  // of the union as a V-shaped sequence, which a bitonic merge sorts
  constexpr int N = KCAP + 1;
  static_assert((N & (N - 1)) == 0, "list length + 1 must be a power of two");
  uint32_t T[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int oi = N - 1 - i;
    const uint32_t mine = i < KCAP ? (uint32_t)K[i < KCAP ? i : 0] : 0u;
    const uint32_t other = (uint32_t)__shfl_xor(oi < KCAP ? K[oi < KCAP ? oi : 0] : 0, 32);
    T[i] = max(mine, other);
  }
#pragma unroll
  for (int j = N >> 1; j > 0; j >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int l = i ^ j;
      if (l > i) {
        const uint32_t a = T[i], b = T[l];
        T[i] = max(a, b);
        T[l] = min(a, b);
      }
    }
  }
  int Li[KCAP];  // the selected blocks, best first (-1: none)
#pragma unroll
  for (int i = 0; i < KCAP; ++i) Li[i] = T[i] >= 65536u ? 65535 - (int)(T[i] & 65535u) : -1;
  if (hf != 0) return;

  // best min(top_k - 1, c) candidates, ascending, then the own block
  const int n_valid = min(kp, c);
  constexpr int NP = NextPow2<KCAP>::v;
  int x[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) x[i] = (i < KCAP && i < n_valid) ? Li[i < KCAP ? i : 0] : INT_MAX;
  bitonic_sort<NP>(x);
  if (!live) return;
  int32_t* out = sel + ((size_t)u * sel_stride + t) * top_k;
#pragma unroll
  for (int i = 0; i <= KCAP; ++i) {
    if (i < top_k) {
      const int xv = (i < NP) ? x[i < NP ? i : 0] : INT_MAX;
      out[i] = (i < n_valid) ? xv : (i == n_valid ? c : -1);
    }
  }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int32_t value, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = value;
}

}  // namespace

hipError_t launch_pool(const int8_t* k_idx, int8_t* block_keys, int units, int S, int bs,
                       hipStream_t st) {
  const int nb = (S + bs - 1) / bs;
  return launch_pool_strided(k_idx, block_keys, nullptr, units, S, S, nb, bs, 0, st);
}

hipError_t launch_pool_strided(const int8_t* k_idx, int8_t* block_keys, int32_t* open_sums, int units, int S,
                               long s_stride, int nb_stride, int bs, int j0, hipStream_t st) {
  const int nb = (S + bs - 1) / bs;
  const long waves = (long)units * (nb - j0);
  if (waves <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  hipLaunchKernelGGL(pool_kernel, dim3(grid), dim3(256), 0, st, k_idx, block_keys, units, S, bs, nb, s_stride,
                     nb_stride, open_sums, j0);
  return hipGetLastError();
}

hipError_t launch_index_topk(const int8_t* q_idx, const int8_t* block_keys, int32_t* sel, int units,
                             int S, int bs, int top_k, hipStream_t st) {
  return launch_index_topk_at(q_idx, block_keys, sel, units, S, 0, S, S, (S + bs - 1) / bs, bs, top_k, st);
}

hipError_t launch_index_topk_at(const int8_t* q_idx, const int8_t* block_keys, int32_t* sel, int units, int S,
                                int q0, int q_stride, int sel_stride, int nb_stride, int bs, int top_k,
                                hipStream_t st) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const int kp = top_k - 1;
  // the matrix-core scores pay from 16 ranked blocks (measured on MI355X,
  // 2048 tokens over 32 blocks: 0.015 ms with the dot4 kernel, 0.010 ms on
  // the matrix cores); the two-sweep kernel's keys hold block indices below
  // 65536, including those of the masked rows of its last chunk (up to 127
  // past the last candidate)
  const int n_blocks = (q0 + S - 1) >> bs_log2;
  const bool mfma = n_blocks >= kIndexMfmaMinBlocks;
  const bool two_sweep = mfma && n_blocks <= 65536 - 128;
  const dim3 grid(mfma ? (S + 127) / 128 : (S + 255) / 256, units);
#define MSA_TOPK_LAUNCH(KC)                                                                                        \
  if (two_sweep) {                                                                                                 \
    hipLaunchKernelGGL(index_topk_bound_kernel<KC>, grid, dim3(256), 0, st, q_idx, block_keys, sel, S, nb_stride,  \
                       bs_log2, top_k, q0, q_stride, sel_stride);                                                  \
    hipLaunchKernelGGL(index_topk_mfma_kernel<KC>, grid, dim3(256), 0, st, q_idx, block_keys, sel, S, nb_stride,   \
                       bs_log2, top_k, q0, q_stride, sel_stride, 1);                                               \
  } else if (mfma) {                                                                                               \
    hipLaunchKernelGGL(index_topk_mfma_kernel<KC>, grid, dim3(256), 0, st, q_idx, block_keys, sel, S, nb_stride,   \
                       bs_log2, top_k, q0, q_stride, sel_stride, 0);                                               \
  } else {                                                                                                         \
    hipLaunchKernelGGL(index_topk_kernel<KC>, grid, dim3(256), 0, st, q_idx, block_keys, sel, S, nb_stride,        \
                       bs_log2, top_k, q0, q_stride, sel_stride);                                                  \
  }
  if (kp <= 1)
    MSA_TOPK_LAUNCH(1)
  else if (kp <= 3)
    MSA_TOPK_LAUNCH(3)
  else if (kp <= 7)
    MSA_TOPK_LAUNCH(7)
  else if (kp <= 15)
    MSA_TOPK_LAUNCH(15)
  else
    MSA_TOPK_LAUNCH(31)
#undef MSA_TOPK_LAUNCH
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, value, n);
  return hipGetLastError();
}

}  // namespace msa
