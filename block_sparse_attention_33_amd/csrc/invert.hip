// Query -> KV-block inversion for the KV-outer main branch.
//
// The main branch walks KV blocks in the outer loop and gathers, for each
// block, the queries that selected it, so a block is read once for all of
// them (yunpan.plus article on MiniMax M3, section "百万上下文，AI 怎么从奢侈品
// 变日用品", the paragraph on the operator level: KV blocks moved to the outer
// loop, each block read once with contiguous access, queries aggregated
// inward).  Building that gather list is a histogram (counted by the top-k
// kernel), an exclusive scan and a scatter: a CSR matrix whose rows are
// (unit, block) and whose entries are (query token, selection slot).

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

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

__global__ __launch_bounds__(256) void build_items_kernel(const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ item_ptr,
                                                          int2* __restrict__ items, int n, int tpi) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int first = item_ptr[i];
  const int ni = item_ptr[i + 1] - first;
  for (int m = 0; m < ni; ++m) items[first + m] = make_int2(i, m * tpi);
}

// One thread per (unit, query token): every selected block before the
// query's own block gets the entry (t << 5) | slot at a fresh position of
// that block's list.  The order inside a list does not matter: each entry's
// result is written to its own (token, slot) place.
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ row_ptr,
                                                      int32_t* __restrict__ fill,
                                                      uint32_t* __restrict__ entries, int units,
                                                      int S, int bs_log2, int top_k, int nb) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long)units * S) return;
  const int u = (int)(gid / S);
  const int t = (int)(gid - (long)u * S);
  const int nv = min(top_k - 1, t >> bs_log2);
  const int32_t* srow = sel + gid * top_k;
  for (int s = 0; s < nv; ++s) {
    const int blk = u * nb + srow[s];
    const int pos = __hip_atomic_fetch_add(fill + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    entries[row_ptr[blk] + pos] = ((uint32_t)t << 5) | (uint32_t)s;
  }
}

}  // namespace

hipError_t launch_scan(const int32_t* counts, int32_t* row_ptr, int32_t* item_ptr, int n,
                       int tokens_per_item, hipStream_t st) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, row_ptr, item_ptr, n, tokens_per_item);
  return hipGetLastError();
}

hipError_t launch_build_items(const int32_t* row_ptr, const int32_t* item_ptr, int2* items, int n,
                              int tokens_per_item, hipStream_t st) {
  hipLaunchKernelGGL(build_items_kernel, dim3((n + 255) / 256), dim3(256), 0, st, row_ptr, item_ptr, items, n,
                     tokens_per_item);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* sel, const int32_t* row_ptr, int32_t* fill,
                          uint32_t* entries, int units, int S, int bs, int top_k, int nb,
                          hipStream_t st) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const long n = (long)units * S;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, sel, row_ptr, fill,
                     entries, units, S, bs_log2, top_k, nb);
  return hipGetLastError();
}

}  // namespace msa
