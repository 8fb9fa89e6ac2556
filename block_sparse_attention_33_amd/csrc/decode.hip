// MSA decode: one query per sequence at the last cache position.
//
// Decode applies the same two branches to a single query over a KV cache
// whose past keys and values stay resident in device memory (wiki.500nian.com
// digest of "MiniMax M3 Review: 1M Tokens, 15X Faster AI Agents", the
// paragraph on the quadratic wall and the KV cache; its co-design paragraph
// reports the decode speed-up).  Work is bound by HBM reads: the block
// summaries (nb x 64 B per group) and the selected K/V blocks (64 KiB each).
//
//   decode_index_kernel   (chunk, unit): scores a chunk of candidate blocks
//                         and keeps its best top_k - 1 keys; zeroes the
//                         unit's arrival counter.
//   decode_attend_kernel  (slot, unit): merges the chunk lists into the final
//                         selection, attends the r query heads of the group to
//                         the slot's block (split-KV), writes an unnormalised
//                         partial; the last workgroup of the unit to arrive
//                         merges all partials into the output.
//
// Ranking keys are 64-bit: (score << 32) | (0xffffffff - block), so a larger
// key is a higher score or, at equal score, a lower block index.

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

constexpr int64_t kNoKey = INT64_MIN;
constexpr int kMaxMergeKeys = 4096;  // chunk lists merged by one workgroup
constexpr int kMaxChunk = 512;       // candidates scored by one index wave

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

// The best `kp` keys of keys[0, n) (LDS), in descending order, by repeated
// wave-wide argmax; one wave; destroys keys.  Missing keys are kNoKey.
__device__ void wave_topk(int64_t* keys, int n, int kp, int64_t* out) {
  const int lane = threadIdx.x & 63;
  for (int it = 0; it < kp; ++it) {
    int64_t best = kNoKey;
    int pos = -1;
    for (int i = lane; i < n; i += 64) {
      const int64_t x = keys[i];
      if (x > best) {
        best = x;
        pos = i;
      }
    }
    const int64_t wbest = wave_max_i64(best);
    if (wbest != kNoKey && best == wbest) keys[pos] = kNoKey;  // keys are unique
    if (lane == 0) out[it] = wbest;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  }
}

// One wave per (chunk, unit).
__global__ __launch_bounds__(64) void decode_index_kernel(const int8_t* __restrict__ q_idx,
                                                          const int8_t* __restrict__ block_keys,
                                                          int64_t* __restrict__ chunk_best,
                                                          int32_t* __restrict__ counters, DecodeShape sh) {
  __shared__ int64_t keys[kMaxChunk];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int lane = threadIdx.x;
  const int kp = sh.top_k - 1;
  if (c == 0 && lane == 0) counters[u] = 0;
  const int n_cand = sh.nb - 1;  // blocks before the own (last) block
  const int j0 = c * sh.chunk;
  const int j1 = min(n_cand, j0 + sh.chunk);
  const i32x4_t* qp = reinterpret_cast<const i32x4_t*>(q_idx + (size_t)u * kIdxDim);
  const i32x4_t q0 = qp[0], q1 = qp[1], q2 = qp[2], q3 = qp[3];
  const int8_t* kb = block_keys + (size_t)u * sh.nb * kIdxDim;
  for (int jj = lane; jj < sh.chunk; jj += 64) {
    const int j = j0 + jj;
    int64_t key = kNoKey;
    if (j < j1) {
      const i32x4_t* sp = reinterpret_cast<const i32x4_t*>(kb + (size_t)j * kIdxDim);
      const i32x4_t a0 = sp[0], a1 = sp[1], a2 = sp[2], a3 = sp[3];
      int s = 0;
      s = sdot4(q0.x, a0.x, s); s = sdot4(q0.y, a0.y, s); s = sdot4(q0.z, a0.z, s); s = sdot4(q0.w, a0.w, s);
      s = sdot4(q1.x, a1.x, s); s = sdot4(q1.y, a1.y, s); s = sdot4(q1.z, a1.z, s); s = sdot4(q1.w, a1.w, s);
      s = sdot4(q2.x, a2.x, s); s = sdot4(q2.y, a2.y, s); s = sdot4(q2.z, a2.z, s); s = sdot4(q2.w, a2.w, s);
      s = sdot4(q3.x, a3.x, s); s = sdot4(q3.y, a3.y, s); s = sdot4(q3.z, a3.z, s); s = sdot4(q3.w, a3.w, s);
      key = rank_key(s, j);
    }
    keys[jj] = key;
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
  __shared__ int64_t best[32];
  wave_topk(keys, sh.chunk, kp, best);
  if (lane < kp) chunk_best[((size_t)u * sh.n_chunks + c) * kp + lane] = best[lane];
}

// One workgroup (256 threads) per (slot, unit); R = query heads per group.
template <int R>
__global__ __launch_bounds__(256) void decode_attend_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int64_t* __restrict__ chunk_best,
    int32_t* __restrict__ sel, float* __restrict__ part_o, float* __restrict__ part_ml,
    int32_t* __restrict__ counters, uint16_t* __restrict__ out, DecodeShape sh) {
  // the merge keys and the value block are never live together
  __shared__ __align__(16) char big[kMaxMergeKeys * 8];
  __shared__ int64_t best[32];
  __shared__ int sel_s[33];
  __shared__ float qs[R * kHeadDim];  // the group's query rows, fp32
  __shared__ float ps[R * 128];       // scores, then weights, [head][key]
  __shared__ float stat[R][2];
  __shared__ int last;
  int64_t* keys = reinterpret_cast<int64_t*>(big);
  uint16_t* vs = reinterpret_cast<uint16_t*>(big);

  const int slot = blockIdx.x;
  const int u = blockIdx.y;
  const int b = u / sh.G;
  const int g = u - b * sh.G;
  const int tid = threadIdx.x;
  const int kp = sh.top_k - 1;
  const int bs = sh.bs;

  // ---- final selection of this unit (every workgroup of the unit agrees)
  const int n_keys = sh.n_chunks * kp;
  for (int i = tid; i < n_keys; i += 256) keys[i] = chunk_best[(size_t)u * n_keys + i];
  __syncthreads();
  if (tid < 64) wave_topk(keys, n_keys, kp, best);
  __syncthreads();
  const int own = sh.nb - 1;
  const int n_valid = min(kp, own);
  if (tid == 0) {
    // ascending block order of the kept candidates, then the own block
    for (int i = 0; i < n_valid; ++i) {
      const int y = key_block(best[i]);
      int m = i - 1;
      while (m >= 0 && sel_s[m] > y) {
        sel_s[m + 1] = sel_s[m];
        --m;
      }
      sel_s[m + 1] = y;
    }
    for (int i = n_valid; i < sh.top_k; ++i) sel_s[i] = (i == n_valid) ? own : -1;
  }
  __syncthreads();
  if (slot == 0 && sel != nullptr && tid < sh.top_k) sel[(size_t)u * sh.top_k + tid] = sel_s[tid];

  const int j = sel_s[slot];
  float* po = part_o + ((size_t)u * sh.top_k + slot) * R * kHeadDim;
  float* pml = part_ml + ((size_t)u * sh.top_k + slot) * R * 2;
  if (j >= 0) {
    const int key0 = j * bs;
    const int nk = min(bs, sh.L - key0);
    const size_t kv_off = ((size_t)u * sh.L + key0) * kHeadDim;
    // stage q (fp32) and the value block (zero past the cache end)
    for (int i = tid; i < R * kHeadDim; i += 256) {
      const uint16_t x = q[((size_t)b * sh.Hq + g * R) * kHeadDim + i];
      qs[i] = __uint_as_float((uint32_t)x << 16);
    }
    for (int i = tid; i < bs * kHeadDim / 8; i += 256) {
      u32x4_t val = {0u, 0u, 0u, 0u};
      if (i / (kHeadDim / 8) < nk) val = reinterpret_cast<const u32x4_t*>(v_cache + kv_off)[i];
      reinterpret_cast<u32x4_t*>(vs)[i] = val;
    }
    __syncthreads();
    // scores: tpk threads split the head dim of one key
    const int tpk = 256 / bs;
    const int key = tid / tpk;
    const int part = tid - key * tpk;
    const int dpt = kHeadDim / tpk;
    float acc[R];
#pragma unroll
    for (int h = 0; h < R; ++h) acc[h] = 0.f;
    if (key < nk) {
      const uint16_t* krow = k_cache + kv_off + (size_t)key * kHeadDim + part * dpt;
      for (int d8 = 0; d8 < dpt; d8 += 8) {
        const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(krow + d8);
        const float kf[8] = {bf16_lo(kw.x), bf16_hi(kw.x), bf16_lo(kw.y), bf16_hi(kw.y),
                             bf16_lo(kw.z), bf16_hi(kw.z), bf16_lo(kw.w), bf16_hi(kw.w)};
#pragma unroll
        for (int h = 0; h < R; ++h) {
          const float* qh = qs + h * kHeadDim + part * dpt + d8;
          float a = acc[h];
#pragma unroll
          for (int e = 0; e < 8; ++e) a = fmaf(qh[e], kf[e], a);
          acc[h] = a;
        }
      }
    }
    for (int off = 1; off < tpk; off <<= 1)
#pragma unroll
      for (int h = 0; h < R; ++h) acc[h] += __shfl_xor(acc[h], off);
    if (part == 0 && key < bs)
#pragma unroll
      for (int h = 0; h < R; ++h) ps[h * 128 + key] = key < nk ? acc[h] * sh.scale_log2 : -__builtin_inff();
    __syncthreads();
    // softmax statistics per head (base 2): one wave per head in turn
    const int w = tid >> 6, lane = tid & 63;
    for (int h = w; h < R; h += 4) {
      float mx = -__builtin_inff();
      for (int kk = lane; kk < bs; kk += 64) mx = fmaxf(mx, ps[h * 128 + kk]);
      for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
      float sum = 0.f;
      for (int kk = lane; kk < bs; kk += 64) {
        const float p = fast_exp2(ps[h * 128 + kk] - mx);
        ps[h * 128 + kk] = p;
        sum += p;
      }
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      if (lane == 0) {
        stat[h][0] = mx;
        stat[h][1] = sum;
      }
    }
    __syncthreads();
    // unnormalised P.V: thread -> head dim d and heads hg, hg + 2, ...
    constexpr int HPT = (R + 1) / 2;
    const int d = tid & (kHeadDim - 1);
    const int hg = tid >> 7;
    float o[HPT];
#pragma unroll
    for (int m = 0; m < HPT; ++m) o[m] = 0.f;
    for (int kk = 0; kk < nk; ++kk) {
      const float vv = __uint_as_float((uint32_t)vs[kk * kHeadDim + d] << 16);
#pragma unroll
      for (int m = 0; m < HPT; ++m) {
        const int h = hg + 2 * m;
        if (h < R) o[m] = fmaf(ps[h * 128 + kk], vv, o[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < HPT; ++m) {
      const int h = hg + 2 * m;
      if (h < R) po[h * kHeadDim + d] = o[m];
    }
    if (tid < R) {
      pml[2 * tid] = stat[tid][0];
      pml[2 * tid + 1] = stat[tid][1];
    }
  } else if (tid < R) {
    pml[2 * tid] = -__builtin_inff();
    pml[2 * tid + 1] = 0.f;
  }

  // ---- the last workgroup of the unit to arrive merges the top_k partials
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(counters + u, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (prev == sh.top_k - 1);
  }
  __syncthreads();
  if (!last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const float* pml_u = part_ml + (size_t)u * sh.top_k * R * 2;
  const float* po_u = part_o + (size_t)u * sh.top_k * R * kHeadDim;
  for (int i = tid; i < R * kHeadDim; i += 256) {
    const int h = i / kHeadDim;
    float M = -__builtin_inff();
    for (int s = 0; s < sh.top_k; ++s) M = fmaxf(M, pml_u[(s * R + h) * 2]);
    float W = 0.f, acc = 0.f;
    for (int s = 0; s < sh.top_k; ++s) {
      const float ms = pml_u[(s * R + h) * 2];
      if (ms == -__builtin_inff()) continue;
      const float wgt = fast_exp2(ms - M);
      W += wgt * pml_u[(s * R + h) * 2 + 1];
      acc += wgt * po_u[(size_t)(s * R) * kHeadDim + i];
    }
    out[((size_t)b * sh.Hq + g * R) * kHeadDim + i] = to_bf16(acc / W);
  }
}

}  // namespace

hipError_t launch_decode_index(const DecodeShape& sh, const int8_t* q_idx, const int8_t* block_keys,
                               int64_t* chunk_best, int32_t* counters, hipStream_t st) {
  hipLaunchKernelGGL(decode_index_kernel, dim3(sh.n_chunks, sh.B * sh.G), dim3(64), 0, st, q_idx, block_keys,
                     chunk_best, counters, sh);
  return hipGetLastError();
}

hipError_t launch_decode_attend(const DecodeShape& sh, const uint16_t* q, const uint16_t* k_cache,
                                const uint16_t* v_cache, const int64_t* chunk_best, int32_t* sel,
                                float* part_o, float* part_ml, int32_t* counters, uint16_t* out,
                                hipStream_t st) {
  const dim3 grid(sh.top_k, sh.B * sh.G);
  switch (sh.r) {
    case 1:
      hipLaunchKernelGGL(decode_attend_kernel<1>, grid, dim3(256), 0, st, q, k_cache, v_cache, chunk_best, sel,
                         part_o, part_ml, counters, out, sh);
      break;
    case 2:
      hipLaunchKernelGGL(decode_attend_kernel<2>, grid, dim3(256), 0, st, q, k_cache, v_cache, chunk_best, sel,
                         part_o, part_ml, counters, out, sh);
      break;
    case 4:
      hipLaunchKernelGGL(decode_attend_kernel<4>, grid, dim3(256), 0, st, q, k_cache, v_cache, chunk_best, sel,
                         part_o, part_ml, counters, out, sh);
      break;
    case 8:
      hipLaunchKernelGGL(decode_attend_kernel<8>, grid, dim3(256), 0, st, q, k_cache, v_cache, chunk_best, sel,
                         part_o, part_ml, counters, out, sh);
      break;
    default:
      hipLaunchKernelGGL(decode_attend_kernel<16>, grid, dim3(256), 0, st, q, k_cache, v_cache, chunk_best, sel,
                         part_o, part_ml, counters, out, sh);
      break;
  }
  return hipGetLastError();
}

}  // namespace msa
