// MSA decode: one query per sequence at the last cache position.
//
// Decode applies the same two branches to a single query over a KV cache
// whose past keys and values stay resident in device memory (wiki.500nian.com
// digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI Agents", the
// paragraph on the quadratic wall and the KV cache; its co-design paragraph
// reports the decode speed-up).  The work is bound by HBM reads: the block
// summaries (nb x 64 B per group) and the selected K/V blocks.
//
//   decode_index_kernel   one workgroup per unit: scores every candidate
//                         block, keeps the best top_k - 1 and writes the
//                         sorted selection (own block last).
//   decode_attend_kernel  one workgroup per (selected slot, unit): runs the
//                         r query heads of the group against the slot's
//                         block on bf16 MFMA (split-KV), leaving an
//                         unnormalised fp32 partial and its base-2 (max, sum)
//                         per head.
//   decode_merge_kernel   one workgroup per unit: log-sum-exp merge -> out.
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

// ---------------------------------------------------------------------------
// Index: one workgroup (16 waves) per unit.  Thread i scores candidates
// i, i + 1024, ... (NK of them); each wave keeps its best kp, wave 0 picks
// the best kp of the 16 lists, ranks them by block index and writes the
// selection: the kept blocks ascending, the own block, then -1.
// ---------------------------------------------------------------------------
template <int NK>
__global__ __launch_bounds__(1024) void decode_index_kernel(const int8_t* __restrict__ q_idx,
                                                            const int8_t* __restrict__ block_keys,
                                                            int32_t* __restrict__ sel_out, DecodeShape sh) {
  __shared__ int64_t wbest[16][32];
  const int u = blockIdx.x;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int K = sh.top_k;
  const int kp = K - 1;
  const int own = sh.nb - 1;  // candidates are blocks 0 .. own - 1
  const i32x4_t* qp = reinterpret_cast<const i32x4_t*>(q_idx + (size_t)u * kIdxDim);
  const i32x4_t q0 = qp[0], q1 = qp[1], q2 = qp[2], q3 = qp[3];
  const int8_t* kb = block_keys + (size_t)u * sh.nb * kIdxDim;

  if (kp > 0) {
    int64_t keys[NK];
#pragma unroll
    for (int m = 0; m < NK; ++m) {
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
    const int64_t mine = wave_topk(keys, kp);
    if (lane < kp) wbest[w][lane] = mine;
  }
  __syncthreads();
  if (w == 0) {
    // the best kp of the 16 waves' lists (16 kp <= 496 keys, up to 8 a lane)
    int64_t k8[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int i = lane + 64 * m;
      k8[m] = (i < 16 * kp) ? wbest[i / kp][i % kp] : kNoKey;
    }
    const int64_t mine = wave_topk(k8, kp);
    const int n_valid = min(kp, own);
    const int blk = lane < n_valid ? key_block(mine) : INT_MAX;
    int rank = 0;
    for (int m = 0; m < n_valid; ++m) rank += __builtin_amdgcn_readlane(blk, m) < blk ? 1 : 0;
    int32_t* out = sel_out + (size_t)u * K;
    if (lane < n_valid) out[rank] = blk;
    if (lane == n_valid) out[n_valid] = own;
    if (lane > n_valid && lane < K) out[lane] = -1;
  }
}

// ---------------------------------------------------------------------------
// Attend: one workgroup (4 waves) per (slot, unit) of the selection.
//   S^T = K Q^T: wave w takes keys 32 w .. 32 w + 31 on 32x32x16 MFMA with
//   the query heads as columns (r <= 16 of the 32 used), K straight from HBM.
//   P = 2^(S - m) goes to LDS as bf16 [head][key]; V goes to LDS transposed.
//   O^T = V^T P^T: wave w takes head dims 32 w .. 32 w + 31 over all keys.
// ---------------------------------------------------------------------------
constexpr int kRowStride = 2 * 128 + 16;  // bytes per 128-key row of V^T and P^T in LDS

__global__ __launch_bounds__(256) void decode_attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache, const uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ sel, float* __restrict__ part_o, float2* __restrict__ part_ml, DecodeShape sh) {
  __shared__ __align__(16) char vt[kHeadDim * kRowStride];
  __shared__ __align__(16) char pt[32 * kRowStride];
  __shared__ float red_m[4][32];
  __shared__ float red_l[4][32];

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
  const int K = sh.top_k;

  const int j = sel[(size_t)u * K + slot];
  float* po = part_o + ((size_t)u * K + slot) * r * kHeadDim;
  float2* pml = part_ml + ((size_t)u * K + slot) * r;

  if (j < 0) {
    if (tid < r) pml[tid] = make_float2(-__builtin_inff(), 0.f);
  } else {
    const int key0 = j * sh.bs;
    const int nk = min(sh.bs, sh.L - key0);  // valid keys of the block
    const int kbase = 32 * w;                // this wave's first key

    // V: thread takes key pairs (2p, 2p + 1) x 8 head dims (16-byte loads)
    const uint16_t* vblk = v_cache + ((size_t)u * sh.L + key0) * kHeadDim;
    u32x4_t va[4], vb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int qid = tid + 256 * m;
      const int pp = qid & 63, c = qid >> 6;
      va[m] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)min(2 * pp, nk - 1) * kHeadDim + 8 * c);
      vb[m] = *reinterpret_cast<const u32x4_t*>(vblk + (size_t)min(2 * pp + 1, nk - 1) * kHeadDim + 8 * c);
    }
    // K fragments (A) straight from HBM; Q^T (B) for columns < r
    u32x4_t kf[8], qf[8];
    const uint16_t* krow = k_cache + ((size_t)u * sh.L + key0 + min(kbase + col, nk - 1)) * kHeadDim;
    const uint16_t* qrow = q + ((size_t)b * sh.Hq + g * r + min(col, r - 1)) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kf[ks] = *reinterpret_cast<const u32x4_t*>(krow + 16 * ks + 8 * hf);
      qf[ks] = *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks + 8 * hf);
    }
    const bool qcol = col < r;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      if (!qcol) qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
    // V^T in LDS, natural key order (zero beyond the block's keys)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int qid = tid + 256 * m;
      const int pp = qid & 63, c = qid >> 6;
      const u32x4_t a = 2 * pp < nk ? va[m] : u32x4_t{0u, 0u, 0u, 0u};
      const u32x4_t bb = 2 * pp + 1 < nk ? vb[m] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = a[e], hi = bb[e];
        *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e) * kRowStride + 4 * pp) = (lo & 0xffffu) | (hi << 16);
        *reinterpret_cast<uint32_t*>(vt + (8 * c + 2 * e + 1) * kRowStride + 4 * pp) =
            (lo >> 16) | (hi & 0xffff0000u);
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
      s[i] = kbase + c_row(i, hf) < nk ? s[i] * c2 : -__builtin_inff();
      mx = fmaxf(mx, s[i]);
    }
    mx = wave_max_pair(mx);
    if (hf == 0) red_m[w][col] = mx;
    __syncthreads();
    const float m = fmaxf(fmaxf(red_m[0][col], red_m[1][col]), fmaxf(red_m[2][col], red_m[3][col]));
    float sum = 0.f;
    // this lane's P^T row (its head): keys kbase + 8 q4 + 4 hf + 0..3
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float p0 = fast_exp2(s[4 * q4 + 0] - m);
      const float p1 = fast_exp2(s[4 * q4 + 1] - m);
      const float p2 = fast_exp2(s[4 * q4 + 2] - m);
      const float p3 = fast_exp2(s[4 * q4 + 3] - m);
      sum += (p0 + p1) + (p2 + p3);
      u32x2_t pv;
      pv.x = pack_bf16x2(p0, p1);
      pv.y = pack_bf16x2(p2, p3);
      *reinterpret_cast<u32x2_t*>(pt + col * kRowStride + 2 * (kbase + 8 * q4 + 4 * hf)) = pv;
    }
    sum = wave_sum_pair(sum);
    if (hf == 0) red_l[w][col] = sum;
    __syncthreads();

    // O^T: head dims 32 w .. 32 w + 31 x 32 heads over the block's keys
    f32x16_t o = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(vt + (32 * w + col) * kRowStride + 2 * (16 * kk + 8 * hf));
      const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(pt + col * kRowStride + 2 * (16 * kk + 8 * hf));
      o = mfma32x32x16(a, bq, o);
    }
    if (qcol) {
      float* orow = po + (size_t)col * kHeadDim + 32 * w + 4 * hf;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4_t*>(orow + 8 * q4) = f32x4_t{o[4 * q4], o[4 * q4 + 1], o[4 * q4 + 2], o[4 * q4 + 3]};
      if (w == 0 && hf == 0)
        pml[col] = make_float2(m, red_l[0][col] + red_l[1][col] + red_l[2][col] + red_l[3][col]);
    }
  }

}

// ---------------------------------------------------------------------------
// Merge: one workgroup per unit, a thread per (head, 4 head dims):
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s  over the unit's slots.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float2* __restrict__ part_ml,
                                                           uint16_t* __restrict__ out, DecodeShape sh) {
  const int u = blockIdx.x;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int r = sh.r;
  const int K = sh.top_k;
  const float2* ml = part_ml + (size_t)u * K * r;
  const float* pou = part_o + (size_t)u * K * r * kHeadDim;
  for (int it = threadIdx.x; it < r * 32; it += 256) {
    const int h = it >> 5;
    const int d0 = (it & 31) * 4;
    // every load of the row is issued before any is used
    float2 v[32];
    f32x4_t ov[32];
#pragma unroll
    for (int s2 = 0; s2 < 32; ++s2) {
      if (s2 < K) {  // uniform
        v[s2] = ml[s2 * r + h];
        ov[s2] = *reinterpret_cast<const f32x4_t*>(pou + ((size_t)s2 * r + h) * kHeadDim + d0);
      }
    }
    float M = -__builtin_inff();
#pragma unroll
    for (int s2 = 0; s2 < 32; ++s2)
      if (s2 < K) M = fmaxf(M, v[s2].x);
    float W = 0.f;
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < 32; ++s2) {
      if (s2 < K) {
        // an empty slot (max = -inf) wrote no partial: its values are skipped
        const bool used = v[s2].x != -__builtin_inff();
        const float wgt = used ? fast_exp2(v[s2].x - M) : 0.f;
        W = fmaf(wgt, used ? v[s2].y : 0.f, W);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, used ? ov[s2][e] : 0.f, acc[e]);
      }
    }
    const float inv = 1.0f / W;
    u32x2_t wv;
    wv.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    wv.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *reinterpret_cast<u32x2_t*>(out + ((size_t)b * sh.Hq + g * r + h) * kHeadDim + d0) = wv;
  }
}

}  // namespace

hipError_t launch_decode_index(const DecodeShape& sh, const int8_t* q_idx, const int8_t* block_keys,
                               int32_t* sel_out, hipStream_t st) {
  const int own = sh.nb - 1;
  const dim3 grid(sh.B * sh.G), block(1024);
  if (own <= 2 * 1024)
    hipLaunchKernelGGL(decode_index_kernel<2>, grid, block, 0, st, q_idx, block_keys, sel_out, sh);
  else if (own <= 4 * 1024)
    hipLaunchKernelGGL(decode_index_kernel<4>, grid, block, 0, st, q_idx, block_keys, sel_out, sh);
  else
    hipLaunchKernelGGL(decode_index_kernel<8>, grid, block, 0, st, q_idx, block_keys, sel_out, sh);
  return hipGetLastError();
}

hipError_t launch_decode_attend(const DecodeShape& sh, const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int32_t* sel, float* part_o, float2* part_ml,
                                hipStream_t st) {
  hipLaunchKernelGGL(decode_attend_kernel, dim3(sh.top_k, sh.B * sh.G), dim3(256), 0, st, q, k_cache, v_cache, sel,
                     part_o, part_ml, sh);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeShape& sh, const float* part_o, const float2* part_ml, uint16_t* out,
                               hipStream_t st) {
  hipLaunchKernelGGL(decode_merge_kernel, dim3(sh.B * sh.G), dim3(256), 0, st, part_o, part_ml, out, sh);
  return hipGetLastError();
}

}  // namespace msa
