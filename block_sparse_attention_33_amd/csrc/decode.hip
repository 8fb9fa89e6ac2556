// MSA decode: one query per sequence at the last cache position.
//
// Decode applies the same two branches to a single query over a KV cache
// whose past keys and values stay resident in device memory (wiki.500nian.com
// digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI Agents", the
// paragraph on the quadratic wall and the KV cache; its co-design paragraph
// reports the decode speed-up).  The work is bound by HBM reads: the block
// summaries (nb x 64 B per group) and the selected K/V blocks.
//
//   decode_index_kernel   one workgroup per (batch, group): scores every
//                         candidate block, keeps the best top_k - 1 and writes
//                         the sorted selection (own block last).
//   decode_attend_kernel  one workgroup per (selected slot, unit): the r query
//                         heads of the group against the slot's block on bf16
//                         MFMA (split-KV), leaving an unnormalised partial and
//                         its base-2 max / sum per head.
//   decode_merge_kernel   one workgroup per unit: log-sum-exp merge -> out.
//
// Ranking keys are 64-bit: (score << 32) | (0xffffffff - block), so a larger
// key is a higher score or, at equal score, a lower block index.

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

constexpr int64_t kNoKey = INT64_MIN;

__device__ __forceinline__ int64_t rank_key(int score, int block) {
  return (int64_t)(((uint64_t)(int64_t)score << 32) | (uint64_t)(0xffffffffu - (uint32_t)block));
}
__device__ __forceinline__ int key_block(int64_t key) { return (int)(0xffffffffu - (uint32_t)(uint64_t)key); }

__device__ __forceinline__ int64_t wave_max_i64(int64_t x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t y = __shfl_xor(x, off);
    x = y > x ? y : x;
  }
  return x;
}

// Best `kp` of the keys held by one wave (NK per lane, kept in registers),
// descending, into out[0, kp) (LDS); missing ones are kNoKey.
template <int NK>
__device__ __forceinline__ void wave_topk_regs(int64_t (&k)[NK], int kp, int64_t* out) {
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < kp; ++it) {
    int64_t best = k[0];
#pragma unroll
    for (int i = 1; i < NK; ++i) best = k[i] > best ? k[i] : best;
    const int64_t wbest = wave_max_i64(best);
    if (wbest != kNoKey) {
#pragma unroll
      for (int i = 0; i < NK; ++i)
        if (k[i] == wbest) k[i] = kNoKey;  // keys are unique
    }
    if (lane == 0) out[it] = wbest;
  }
}

// ---------------------------------------------------------------------------
// Index: one workgroup (1024 threads) per unit.  Thread i scores candidates
// i, i + 1024, ... (up to kDecodeCandPerThread of them), each of the 16
// waves keeps its best kp, and wave 0 picks the best kp of the survivors.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void decode_index_kernel(const int8_t* __restrict__ q_idx,
                                                            const int8_t* __restrict__ block_keys,
                                                            int32_t* __restrict__ sel_out, DecodeShape sh) {
  __shared__ int64_t wbest[16][32];
  __shared__ int64_t best[32];
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int kp = sh.top_k - 1;
  const int own = sh.nb - 1;  // candidates are blocks 0 .. own - 1
  const i32x4_t* qp = reinterpret_cast<const i32x4_t*>(q_idx + (size_t)u * kIdxDim);
  const i32x4_t q0 = qp[0], q1 = qp[1], q2 = qp[2], q3 = qp[3];
  const int8_t* kb = block_keys + (size_t)u * sh.nb * kIdxDim;

  int64_t keys[kDecodeCandPerThread];
#pragma unroll
  for (int m = 0; m < kDecodeCandPerThread; ++m) {
    const int j = tid + 1024 * m;
    int64_t key = kNoKey;
    if (1024 * m < own) {  // uniform: the loads below are unconditional within it
      const i32x4_t* sp = reinterpret_cast<const i32x4_t*>(kb + (size_t)min(j, own - 1) * kIdxDim);
      const i32x4_t a0 = sp[0], a1 = sp[1], a2 = sp[2], a3 = sp[3];
      int s = 0;
      s = sdot4(q0.x, a0.x, s); s = sdot4(q0.y, a0.y, s); s = sdot4(q0.z, a0.z, s); s = sdot4(q0.w, a0.w, s);
      s = sdot4(q1.x, a1.x, s); s = sdot4(q1.y, a1.y, s); s = sdot4(q1.z, a1.z, s); s = sdot4(q1.w, a1.w, s);
      s = sdot4(q2.x, a2.x, s); s = sdot4(q2.y, a2.y, s); s = sdot4(q2.z, a2.z, s); s = sdot4(q2.w, a2.w, s);
      s = sdot4(q3.x, a3.x, s); s = sdot4(q3.y, a3.y, s); s = sdot4(q3.z, a3.z, s); s = sdot4(q3.w, a3.w, s);
      key = j < own ? rank_key(s, j) : kNoKey;
    }
    keys[m] = key;
  }
  wave_topk_regs(keys, kp, wbest[w]);
  __syncthreads();
  if (w == 0 && kp > 0) {
    int64_t k8[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int i = tid + 64 * m;
      k8[m] = (i < 16 * kp) ? wbest[i / kp][i % kp] : kNoKey;
    }
    wave_topk_regs(k8, kp, best);
  }
  __syncthreads();
  if (tid == 0) {
    // ascending block order of the kept candidates, then the own block
    const int n_valid = min(kp, own);
    int32_t* out = sel_out + (size_t)u * sh.top_k;
    int x[32];
    for (int i = 0; i < n_valid; ++i) {
      const int y = key_block(best[i]);
      int m = i - 1;
      while (m >= 0 && x[m] > y) {
        x[m + 1] = x[m];
        --m;
      }
      x[m + 1] = y;
    }
    for (int i = 0; i < sh.top_k; ++i) out[i] = i < n_valid ? x[i] : (i == n_valid ? own : -1);
  }
}

// ---------------------------------------------------------------------------
// Attend: one workgroup (4 waves) per (slot, unit); wave w takes keys
// 32 w .. 32 w + 31 of the slot's block (blocks of 32 or 64 keys leave waves
// idle).  S^T = K Q^T on 32x32x16 MFMA with the query heads as columns
// (r <= 16 of the 32 used), K fragments straight from HBM; O^T = V^T P^T
// likewise, V staged through LDS transposed (head dim major).  Partial =
// (o unnormalised, max m, sum l) per head, base 2.
// ---------------------------------------------------------------------------
constexpr int kDecVtStride = 2 * 128 + 8;  // bytes per head-dim row of V^T

__global__ __launch_bounds__(256) void decode_attend_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ k_cache,
                                                            const uint16_t* __restrict__ v_cache,
                                                            const int32_t* __restrict__ sel,
                                                            float* __restrict__ part_o,
                                                            float* __restrict__ part_ml, DecodeShape sh) {
  __shared__ __align__(16) char vt[kHeadDim * kDecVtStride];
  __shared__ float red_m[4][32];
  __shared__ float red_l[4][32];
  __shared__ float red_o[4][16][kHeadDim];

  const int slot = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int col = lane & 31;  // query head of this lane's column
  const int r = sh.r;
  float* po = part_o + ((size_t)u * sh.top_k + slot) * r * kHeadDim;
  float* pml = part_ml + ((size_t)u * sh.top_k + slot) * r * 2;

  const int j = sel[(size_t)u * sh.top_k + slot];
  if (j < 0) {
    if (tid < r) {
      pml[2 * tid] = -__builtin_inff();
      pml[2 * tid + 1] = 0.f;
    }
    return;
  }
  const int key0 = j * sh.bs;
  const int nk = min(sh.bs, sh.L - key0);  // valid keys of the block
  const int kbase = 32 * w;                // this wave's first key
  const bool wave_live = kbase < nk;

  // V: thread takes key pairs (2p, 2p + 1) x 8 head dims, 16-byte loads
  const uint16_t* vblk = v_cache + ((size_t)u * sh.L + key0) * kHeadDim;
  u32x4_t va[4], vb[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int qid = tid + 256 * m;
    const int p = qid & 63, c = qid >> 6;
    const int k0 = min(2 * p, nk - 1), k1 = min(2 * p + 1, nk - 1);
    va[m] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)k0 * kHeadDim + 8 * c);
    vb[m] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)k1 * kHeadDim + 8 * c);
  }
  // K fragments (A) straight from HBM; Q^T (B) for columns < r
  u32x4_t kf[8], qf[8];
  const int key = kbase + col;
  const uint16_t* krow = k_cache + ((size_t)u * sh.L + key0 + min(key, nk - 1)) * kHeadDim;
  const uint16_t* qrow = q + ((size_t)b * sh.Hq + g * r + min(col, r - 1)) * kHeadDim;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    kf[ks] = *reinterpret_cast<const u32x4_t*>(krow + 16 * ks + 8 * hf);
    qf[ks] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
    if (col >= r) qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int qid = tid + 256 * m;
    const int p = qid & 63, c = qid >> 6;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = va[m][e], hi = vb[m][e];
      *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e) * kDecVtStride + 4 * p) = (lo & 0xffffu) | (hi << 16);
      *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e + 1) * kDecVtStride + 4 * p) = (lo >> 16) | (hi & 0xffff0000u);
    }
  }

  // scores S^T (32 keys x 32 heads) of this wave, base 2
  f32x16_t s = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) s = mfma32x32x16(kf[ks], qf[ks], s);
  const float c2 = sh.scale_log2;
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int kk = kbase + c_row(i, hf);
    s[i] = kk < nk ? s[i] * c2 : -__builtin_inff();
    mx = fmaxf(mx, s[i]);
  }
  mx = wave_max_pair(mx);
  if (hf == 0) red_m[w][col] = mx;
  __syncthreads();  // also publishes V^T
  const float m = fmaxf(fmaxf(red_m[0][col], red_m[1][col]), fmaxf(red_m[2][col], red_m[3][col]));
  float sum = 0.f;
  u32x4_t pk[2];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    uint32_t d4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(s[8 * h2 + 2 * e] - m);
      const float p1 = fast_exp2(s[8 * h2 + 2 * e + 1] - m);
      d4[e] = pack_bf16x2(p0, p1);
      sum += bf16_lo(d4[e]) + bf16_hi(d4[e]);  // normalise with the rounded weights
    }
    pk[h2] = u32x4_t{d4[0], d4[1], d4[2], d4[3]};
  }
  sum = wave_sum_pair(sum);
  if (hf == 0) red_l[w][col] = wave_live ? sum : 0.f;

  // O^T (128 dims x 32 heads) over this wave's keys
  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) {
    o[dt] = f32x16_t{};
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const char* pv = vt + (32 * dt + col) * kDecVtStride + 2 * (kbase + 16 * h2 + 4 * hf);
      const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(pv);
      const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(pv + 16);
      o[dt] = mfma32x32x16(u32x4_t{lo.x, lo.y, hi.x, hi.y}, pk[h2], o[dt]);
    }
  }
  // sum the four waves' O^T in LDS (columns < r only)
  if (col < r) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) red_o[w][col][32 * dt + c_row(i, hf)] = wave_live ? o[dt][i] : 0.f;
  }
  __syncthreads();
  for (int i = tid; i < r * kHeadDim; i += 256) {
    const int h = i / kHeadDim, d = i - h * kHeadDim;
    po[i] = red_o[0][h][d] + red_o[1][h][d] + red_o[2][h][d] + red_o[3][h][d];
  }
  if (tid < r) {
    pml[2 * tid] = m;
    pml[2 * tid + 1] = red_l[0][tid] + red_l[1][tid] + red_l[2][tid] + red_l[3][tid];
  }
}

// One workgroup per (unit, head), thread = head dim:
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
__global__ __launch_bounds__(128) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, DecodeShape sh) {
  const int u = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int r = sh.r;
  const float* pml = part_ml + (size_t)u * sh.top_k * r * 2;
  const float* po = part_o + (size_t)u * sh.top_k * r * kHeadDim;
  float ms[32], ls[32], os[32];
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    if (s < sh.top_k) {
      ms[s] = pml[(s * r + h) * 2];
      ls[s] = pml[(s * r + h) * 2 + 1];
      os[s] = po[(size_t)(s * r + h) * kHeadDim + d];
    }
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < 32; ++s)
    if (s < sh.top_k) M = fmaxf(M, ms[s]);
  float W = 0.f, acc = 0.f;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    if (s < sh.top_k && ms[s] != -__builtin_inff()) {
      const float wgt = fast_exp2(ms[s] - M);
      W = fmaf(wgt, ls[s], W);
      acc = fmaf(wgt, os[s], acc);
    }
  }
  out[((size_t)b * sh.Hq + g * r + h) * kHeadDim + d] = to_bf16(acc / W);
}

}  // namespace

hipError_t launch_decode_index(const DecodeShape& sh, const int8_t* q_idx, const int8_t* block_keys,
                               int32_t* sel_out, hipStream_t st) {
  hipLaunchKernelGGL(decode_index_kernel, dim3(sh.B * sh.G), dim3(1024), 0, st, q_idx, block_keys, sel_out, sh);
  return hipGetLastError();
}

hipError_t launch_decode_attend(const DecodeShape& sh, const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int32_t* sel, float* part_o, float* part_ml,
                                hipStream_t st) {
  hipLaunchKernelGGL(decode_attend_kernel, dim3(sh.top_k, sh.B * sh.G), dim3(256), 0, st, q, k_cache, v_cache,
                     sel, part_o, part_ml, sh);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeShape& sh, const float* part_o, const float* part_ml, uint16_t* out,
                               hipStream_t st) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(sh.B * sh.G, sh.r), dim3(128), 0, st, part_o, part_ml, out, sh);
  return hipGetLastError();
}

}  // namespace msa
