// Query -> KV-block inversion for the KV-outer main branch.
//
// The main branch walks KV blocks in the outer loop and gathers, for each
// block, the queries that selected it, so a block is read once for all of
// them (yunpan.plus article on MiniMax M3, section "百万上下文，AI 怎么从奢侈品
// 变日用品", the paragraph on the operator level: KV blocks moved to the outer
// loop, each block read once with contiguous access, queries aggregated
// inward).  Building that gather list is a counting sort: per-chunk block
// histograms in LDS, an exclusive scan, and a scatter through LDS cursors
// into a CSR matrix whose rows are (unit, block) and whose entries are
// (query token, selection slot).  Device-wide atomics are avoided on
// purpose: thousands of queries hit the same block counter.

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

// Per-chunk histograms: one workgroup per (token chunk, unit) counts, in LDS,
// how many of the chunk's queries kept each block (the own block included),
// and stores the counts as H[u][chunk][block].  LDS atomics only.
__device__ __forceinline__ void chunk_tokens(const ChunkPlan& cp, int c, int S, int* t0, int* t1) {
  const int rng = c / cp.m;
  const int i = c - rng * cp.m;
  *t0 = rng * cp.T + i * cp.tpc;
  *t1 = min(min(S, (rng + 1) * cp.T), *t0 + cp.tpc);
}

__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ H, int S, int nb,
                                                         int bs_log2, int top_k, ChunkPlan cp, int q0) {
  extern __shared__ int32_t hist[];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int n_chunks = cp.n_chunks;
  for (int j = threadIdx.x; j < nb; j += 256) hist[j] = 0;
  __syncthreads();
  int t0, t1;
  chunk_tokens(cp, c, S, &t0, &t1);
  const int kp = top_k - 1;
  for (int t = t0 + (int)threadIdx.x; t < t1; t += 256) {
    const int nv = min(kp, (q0 + t) >> bs_log2);  // slot nv holds the own block
    const int32_t* srow = sel + ((size_t)u * cp.q_stride + t) * top_k;
    for (int s = 0; s <= nv; ++s) atomicAdd(&hist[srow[s]], 1);
  }
  __syncthreads();
  int32_t* dst = H + ((size_t)u * n_chunks + c) * nb;
  for (int j = threadIdx.x; j < nb; j += 256) dst[j] = hist[j];
}

// Per row (unit, range, block): total over the range's chunks -> counts.
__global__ __launch_bounds__(256) void chunk_total_kernel(const int32_t* __restrict__ H,
                                                          int32_t* __restrict__ counts, int units, int nb,
                                                          ChunkPlan cp) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= units * cp.n_ranges * nb) return;
  const int u = i / (cp.n_ranges * nb);
  const int rem = i - u * cp.n_ranges * nb;
  const int rng = rem / nb;
  const int j = rem - rng * nb;
  const int32_t* src = H + ((size_t)u * cp.n_chunks + (size_t)rng * cp.m) * nb + j;
  int total = 0;
  for (int c = 0; c < cp.m; ++c) total += src[(size_t)c * nb];
  counts[i] = total;
}

// One workgroup: each thread scans a contiguous run of the counts, the run
// totals are scanned in LDS, then every thread writes its exclusive offsets.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ row_ptr,
                                                    int32_t* __restrict__ item_ptr, int n,
                                                    int tpi) {
  __shared__ int sa[1024];
  __shared__ int sb[1024];
  const int tid = threadIdx.x;
  const int per = (n + 1023) / 1024;
  const int i0 = min(n, tid * per);
  const int i1 = min(n, i0 + per);
  int a = 0, b = 0;
  for (int i = i0; i < i1; ++i) {
    const int c = counts[i];
    a += c;
    b += (c + tpi - 1) / tpi;
  }
  sa[tid] = a;
  sb[tid] = b;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int va = tid >= off ? sa[tid - off] : 0;
    const int vb = tid >= off ? sb[tid - off] : 0;
    __syncthreads();
    sa[tid] += va;
    sb[tid] += vb;
    __syncthreads();
  }
  int ea = sa[tid] - a;
  int eb = sb[tid] - b;
  for (int i = i0; i < i1; ++i) {
    const int c = counts[i];
    row_ptr[i] = ea;
    item_ptr[i] = eb;
    ea += c;
    eb += (c + tpi - 1) / tpi;
  }
  if (tid == 1023) {
    row_ptr[n] = sa[1023];
    item_ptr[n] = sb[1023];
  }
}

// Per row (unit, range, block): turn the range's chunk counts into the
// chunks' first positions in the row's list (in place), and write the row's
// work items {row id, first entry}.
__global__ __launch_bounds__(256) void offsets_items_kernel(int32_t* __restrict__ H,
                                                            const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ item_ptr,
                                                            int2* __restrict__ items, int units, int nb,
                                                            ChunkPlan cp, int tpi) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= units * cp.n_ranges * nb) return;
  const int u = i / (cp.n_ranges * nb);
  const int rem = i - u * cp.n_ranges * nb;
  const int rng = rem / nb;
  const int j = rem - rng * nb;
  int32_t* col = H + ((size_t)u * cp.n_chunks + (size_t)rng * cp.m) * nb + j;
  int run = row_ptr[i];
  for (int c = 0; c < cp.m; ++c) {
    const int x = col[(size_t)c * nb];
    col[(size_t)c * nb] = run;
    run += x;
  }
  const int first = item_ptr[i];
  const int ni = item_ptr[i + 1] - first;
  for (int m = 0; m < ni; ++m) items[first + m] = make_int2(i, m * tpi);
}

// One workgroup per (token chunk, unit): the chunk's entries go to its
// reserved stretch of each block's list; positions inside the stretch come
// from LDS cursors.  The order inside a list does not matter: each entry's
// result is written to its own (token, slot) place.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ H,
                                                      uint32_t* __restrict__ entries, int S, int nb,
                                                      int bs_log2, int top_k, ChunkPlan cp, int q0) {
  extern __shared__ int32_t cursor[];
  const int c = blockIdx.x;
  const int u = blockIdx.y;
  const int32_t* src = H + ((size_t)u * cp.n_chunks + c) * nb;
  for (int j = threadIdx.x; j < nb; j += 256) cursor[j] = src[j];
  __syncthreads();
  int t0, t1;
  chunk_tokens(cp, c, S, &t0, &t1);
  const int kp = top_k - 1;
  for (int t = t0 + (int)threadIdx.x; t < t1; t += 256) {
    const int nv = min(kp, (q0 + t) >> bs_log2);  // slot nv holds the own block
    const int32_t* srow = sel + ((size_t)u * cp.q_stride + t) * top_k;
    for (int s = 0; s <= nv; ++s) {
      const int pos = atomicAdd(&cursor[srow[s]], 1);
      entries[pos] = ((uint32_t)t << 5) | (uint32_t)s;
    }
  }
}

}  // namespace

hipError_t launch_chunk_hist(const int32_t* sel, int32_t* H, int units, int S, int nb, int bs, int top_k,
                             const ChunkPlan& cp, int q0, hipStream_t st) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const size_t lds = (size_t)nb * 4;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunk_hist_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kMaxInvertBlocks * 4);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(chunk_hist_kernel, dim3(cp.n_chunks, units), dim3(256), lds, st, sel, H, S, nb, bs_log2,
                     top_k, cp, q0);
  return hipGetLastError();
}

hipError_t launch_chunk_total(const int32_t* H, int32_t* counts, int units, int nb, const ChunkPlan& cp,
                              hipStream_t st) {
  const int n = units * cp.n_ranges * nb;
  hipLaunchKernelGGL(chunk_total_kernel, dim3((n + 255) / 256), dim3(256), 0, st, H, counts, units, nb, cp);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* counts, int32_t* row_ptr, int32_t* item_ptr, int n,
                       int tokens_per_item, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, row_ptr, item_ptr, n, tokens_per_item);
  return hipGetLastError();
}

hipError_t launch_offsets_items(int32_t* H, const int32_t* row_ptr, const int32_t* item_ptr, int2* items,
                                int units, int nb, const ChunkPlan& cp, int tokens_per_item, hipStream_t st) {
  const int n = units * cp.n_ranges * nb;
  hipLaunchKernelGGL(offsets_items_kernel, dim3((n + 255) / 256), dim3(256), 0, st, H, row_ptr, item_ptr, items,
                     units, nb, cp, tokens_per_item);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* sel, const int32_t* H, uint32_t* entries, int units, int S, int nb,
                          int bs, int top_k, const ChunkPlan& cp, int q0, hipStream_t st) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const size_t lds = (size_t)nb * 4;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&scatter_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     kMaxInvertBlocks * 4);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(scatter_kernel, dim3(cp.n_chunks, units), dim3(256), lds, st, sel, H, entries, S, nb, bs_log2,
                     top_k, cp, q0);
  return hipGetLastError();
}

}  // namespace msa
