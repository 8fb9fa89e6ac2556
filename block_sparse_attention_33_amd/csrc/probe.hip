// Measurement aid, not a step of the attention path: the bf16 matrix-core
// rate that a kernel made of nothing but MFMAs reaches on this device, to
// read beside the published dense peak when the attention kernels'
// fractions are judged (clock and power limits under load are the chip's,
// not the kernels').
//
// Every wave runs `iters` rounds of kProbeChains independent
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic inside
// the loop); four independent accumulators cover the result latency of one
// product, so a SIMD issues back to back.  One float per thread is written
// at the end so that the products are kept.

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {
namespace {

constexpr int kProbeChains = 4;

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  // small finite bf16 operands (about 1e-3): the sums stay far from overflow
  // for any iteration count the entry point accepts
  const uint32_t av = 0x3a803a80u + (uint32_t)(lane & 7);
  const uint32_t bv = 0x3a813a81u;
  const u32x4_t a = u32x4_t{av, av, av, av};
  const u32x4_t b = u32x4_t{bv, bv, bv, bv};
  f32x16_t acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = f32x16_t{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = mfma32x32x16(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int n_workgroups, int iters, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3((unsigned)n_workgroups), dim3(256), 0, st, out, iters);
  return hipGetLastError();
}

double mfma_probe_flop(int n_workgroups, int iters) {
  // 4 waves per workgroup, kProbeChains products per round, 2 * 32 * 32 * 16 FLOP each
  return (double)n_workgroups * 4.0 * (double)iters * kProbeChains * 2.0 * 32 * 32 * 16;
}

}  // namespace msa
