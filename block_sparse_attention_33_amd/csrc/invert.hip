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

// Tokens t0 .. t1 - 1 of histogram chunk c.
__device__ __forceinline__ void chunk_tokens(const ChunkPlan& cp, int c, int S, int* t0, int* t1) {
  const int rng = c / cp.m;
  const int i = c - rng * cp.m;
  *t0 = rng * cp.T + i * cp.tpc;
  *t1 = min(min(S, (rng + 1) * cp.T), *t0 + cp.tpc);
}

// An entry holds its slot in 5 bits: at most 32 slots per selection row.
constexpr int kEntrySlots = 32;

// Slots 0 .. n - 1 (n <= kEntrySlots) of a 16-byte aligned selection row
// whose length is a multiple of 4, as 16-byte loads all issued before the
// first use (one 4-byte load per slot touches a cache line per lane of the
// wave).  4 i < n implies 4 i + 3 < the row length: every load is inside it.
__device__ __forceinline__ void load_sel_row(const int32_t* __restrict__ srow, int n,
                                             int32_t (&blk)[kEntrySlots]) {
#pragma unroll
  for (int i = 0; i < kEntrySlots / 4; ++i) {
    if (4 * i < n) {
      const i32x4_t x = reinterpret_cast<const i32x4_t*>(srow)[i];
      blk[4 * i] = x[0];
      blk[4 * i + 1] = x[1];
      blk[4 * i + 2] = x[2];
      blk[4 * i + 3] = x[3];
    }
  }
}

// Per-chunk histograms: one workgroup per (token chunk, unit) counts, in LDS,
// how many of the chunk's queries kept each block (the own block only with
// with_own: the forward attends it elsewhere, the backward through the
// lists), and stores the counts as H[u][chunk][block].  LDS atomics only.
// VEC: selection rows 16-byte aligned, read by load_sel_row.
template <bool VEC>
__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t* __restrict__ sel,
                                                         int32_t* __restrict__ H, int S, int nb,
                                                         int bs_log2, int top_k, ChunkPlan cp, int q0,
                                                         int with_own) {
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
    const int n = nv + with_own;
    if constexpr (VEC) {
      int32_t blk[kEntrySlots];
      load_sel_row(srow, n, blk);
#pragma unroll
      for (int s = 0; s < kEntrySlots; ++s)
        if (s < n) atomicAdd(&hist[blk[s]], 1);
    } else {
      for (int s = 0; s < n; ++s) atomicAdd(&hist[srow[s]], 1);
    }
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

// One workgroup scans the counts in batches of 16 rows of 1024 (thread i
// holds element i of each row, so every load and store of a row is one
// contiguous stretch, and a batch's loads are issued together): the
// inclusive sums within each wave come from lane shuffles for the 16 rows
// at once, one wave scans the batch's 256 (row, wave) totals in order, with
// the carry of the earlier batches, and every thread adds its wave's
// prefix.  Also the items: ceil(count / tpi) per row.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ row_ptr,
                                                    int32_t* __restrict__ item_ptr, int n,
                                                    int tpi) {
  constexpr int kB = 16;             // rows per batch
  __shared__ int wt[2][kB * 16];     // (row, wave) totals, then their exclusive prefixes
  __shared__ int bt[2];              // the batch's totals
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  int carry_a = 0, carry_b = 0;  // the same in every thread
  for (int base = 0; base < n; base += 1024 * kB) {
    int c[kB], ia[kB], ib[kB];
#pragma unroll
    for (int r = 0; r < kB; ++r) {
      const int i = base + 1024 * r + tid;
      c[r] = i < n ? counts[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kB; ++r) {
      ia[r] = c[r];
      ib[r] = (c[r] + tpi - 1) / tpi;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
      for (int r = 0; r < kB; ++r) {
        const int ua = __shfl_up(ia[r], off), ub = __shfl_up(ib[r], off);
        if (lane >= off) {
          ia[r] += ua;
          ib[r] += ub;
        }
      }
    }
    if (lane == 63) {
#pragma unroll
      for (int r = 0; r < kB; ++r) {
        wt[0][r * 16 + w] = ia[r];
        wt[1][r * 16 + w] = ib[r];
      }
    }
    __syncthreads();
    if (w == 0) {
      // lane l: totals 4 l .. 4 l + 3 of each kind, in (row, wave) order
#pragma unroll
      for (int kind = 0; kind < 2; ++kind) {
        int v[4], sum = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = wt[kind][4 * lane + e];
          sum += v[e];
        }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int up = __shfl_up(incl, off);
          if (lane >= off) incl += up;
        }
        int run = (kind == 0 ? carry_a : carry_b) + incl - sum;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wt[kind][4 * lane + e] = run;
          run += v[e];
        }
        if (lane == 63) bt[kind] = incl;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kB; ++r) {
      const int i = base + 1024 * r + tid;
      if (i < n) {
        row_ptr[i] = wt[0][r * 16 + w] + ia[r] - c[r];
        item_ptr[i] = wt[1][r * 16 + w] + ib[r] - (c[r] + tpi - 1) / tpi;
      }
    }
    carry_a += bt[0];
    carry_b += bt[1];
    __syncthreads();  // every thread has read the prefixes before the next batch writes them
  }
  if (tid == 0) {
    row_ptr[n] = carry_a;
    item_ptr[n] = carry_b;
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
// result is written to its own (token, slot) place.  VEC: selection rows
// are 16-byte aligned (top_k a multiple of 4, sel aligned) and read by
// load_sel_row.
template <bool VEC>
__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ sel,
                                                      const int32_t* __restrict__ H,
                                                      uint32_t* __restrict__ entries, int S, int nb,
                                                      int bs_log2, int top_k, ChunkPlan cp, int q0,
                                                      int with_own, int units) {
  extern __shared__ int32_t cursor[];
  // workgroup i runs on XCD i % 8 and takes unit i % units, chunk i / units:
  // with a multiple of 8 units every chunk of a unit -- whose segments of a
  // block's list are adjacent and share cache lines -- writes through one L2
  const int u = (int)(blockIdx.x % (unsigned)units);
  const int c = (int)(blockIdx.x / (unsigned)units);
  const int32_t* src = H + ((size_t)u * cp.n_chunks + c) * nb;
  for (int j = threadIdx.x; j < nb; j += 256) cursor[j] = src[j];
  __syncthreads();
  int t0, t1;
  chunk_tokens(cp, c, S, &t0, &t1);
  const int kp = top_k - 1;
  for (int t = t0 + (int)threadIdx.x; t < t1; t += 256) {
    const int nv = min(kp, (q0 + t) >> bs_log2);  // slot nv holds the own block
    const int32_t* srow = sel + ((size_t)u * cp.q_stride + t) * top_k;
    const int n = nv + with_own;  // n <= top_k
    if constexpr (VEC) {
      int32_t blk[kEntrySlots];
      load_sel_row(srow, n, blk);
#pragma unroll
      for (int s = 0; s < kEntrySlots; ++s) {
        if (s < n) {
          const int pos = atomicAdd(&cursor[blk[s]], 1);
          entries[pos] = ((uint32_t)t << 5) | (uint32_t)s;
        }
      }
    } else {
      for (int s = 0; s < n; ++s) {
        const int pos = atomicAdd(&cursor[srow[s]], 1);
        entries[pos] = ((uint32_t)t << 5) | (uint32_t)s;
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_hist(const int32_t* sel, int32_t* H, int units, int S, int nb, int bs, int top_k,
                             const ChunkPlan& cp, int q0, bool with_own, hipStream_t st) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const size_t lds = (size_t)nb * 4;
  if (top_k > kEntrySlots) return hipErrorInvalidValue;
  const bool vec = top_k % 4 == 0 && reinterpret_cast<uintptr_t>(sel) % 16 == 0;
  const void* fn = vec ? reinterpret_cast<const void*>(&chunk_hist_kernel<true>)
                       : reinterpret_cast<const void*>(&chunk_hist_kernel<false>);
  const hipError_t attr = ensure_dynamic_lds(fn, kMaxInvertBlocks * 4);
  if (attr != hipSuccess) return attr;
  if (vec)
    hipLaunchKernelGGL(chunk_hist_kernel<true>, dim3(cp.n_chunks, units), dim3(256), lds, st, sel, H, S, nb,
                       bs_log2, top_k, cp, q0, with_own ? 1 : 0);
  else
    hipLaunchKernelGGL(chunk_hist_kernel<false>, dim3(cp.n_chunks, units), dim3(256), lds, st, sel, H, S, nb,
                       bs_log2, top_k, cp, q0, with_own ? 1 : 0);
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
                          int bs, int top_k, const ChunkPlan& cp, int q0, bool with_own, hipStream_t st) {
  int bs_log2 = 0;
  while ((1 << bs_log2) < bs) ++bs_log2;
  const size_t lds = (size_t)nb * 4;
  if (top_k > kEntrySlots) return hipErrorInvalidValue;
  const bool vec = top_k % 4 == 0 && reinterpret_cast<uintptr_t>(sel) % 16 == 0;
  const void* fn = vec ? reinterpret_cast<const void*>(&scatter_kernel<true>)
                       : reinterpret_cast<const void*>(&scatter_kernel<false>);
  const hipError_t attr = ensure_dynamic_lds(fn, kMaxInvertBlocks * 4);
  if (attr != hipSuccess) return attr;
  if (vec)
    hipLaunchKernelGGL(scatter_kernel<true>, dim3((unsigned)(cp.n_chunks * units)), dim3(256), lds, st, sel, H,
                       entries, S, nb, bs_log2, top_k, cp, q0, with_own ? 1 : 0, units);
  else
    hipLaunchKernelGGL(scatter_kernel<false>, dim3((unsigned)(cp.n_chunks * units)), dim3(256), lds, st, sel, H,
                       entries, S, nb, bs_log2, top_k, cp, q0, with_own ? 1 : 0, units);
  return hipGetLastError();
}

}  // namespace msa
