// bf16 MFMA rate probe: the rate the chip sustains with every CU issuing the
// prefill tile's matrix instruction, measured on the device the kernels run
// on.  Performance claims need a reproducible measurement beside them
// (ForgeLM README, "Tooling and Benchmarks"); the published dense bf16 peak
// assumes a clock that a chip with every CU busy does not hold, so the
// prefill benchmark reports this figure beside it.
//
// Each workgroup has 8 waves, two per SIMD as in the prefill tile.  A wave
// loads 8 A and 8 B operands of v_mfma_f32_32x32x16_bf16 from the caller's
// buffer (so the operands carry real data, and the power that goes with it)
// and then issues 64 MFMAs per round on 8 independent accumulators, pairing a
// different A with each B every round.  Each wave's accumulators are summed
// into one float of the sink, so nothing is dead.
#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {
namespace {

constexpr int kChains = 8;  // independent accumulators (and A/B operands) per wave

__global__ __launch_bounds__(64 * kMfmaProbeWaves) void mfma_rate_probe_kernel(const uint4* __restrict__ operands,
                                                                                int n_ops, int rounds,
                                                                                float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long gw = static_cast<long>(blockIdx.x) * kMfmaProbeWaves + (threadIdx.x >> 6);
  bf16x8_t a[kChains], b[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) {
    a[k] = __builtin_bit_cast(bf16x8_t, operands[(gw * 2 * kChains * 64 + k * 64 + lane) % n_ops]);
    b[k] = __builtin_bit_cast(bf16x8_t, operands[(gw * 2 * kChains * 64 + (kChains + k) * 64 + lane) % n_ops]);
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
  for (int r = 0; r < rounds; ++r) {
#pragma unroll
    for (int j = 0; j < kChains; ++j)
#pragma unroll
      for (int k = 0; k < kChains; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + k) % kChains], b[k], acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[k][i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) sink[gw] = s;
}

}  // namespace

hipError_t launch_mfma_rate_probe(const void* operands, int n_ops, int workgroups, int rounds, float* sink,
                                  hipStream_t stream) {
  if (workgroups == 0) return hipSuccess;
  const uint4* ops = static_cast<const uint4*>(operands);
  void* args[] = {&ops, &n_ops, &rounds, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mfma_rate_probe_kernel), dim3(static_cast<unsigned>(workgroups)),
                         dim3(64 * kMfmaProbeWaves), args, 0, stream);
}

}  // namespace fe
