// Chunked prefill over the paged cache on the bf16 MFMA units (ForgeEngine
// README, "What it implements": restricted prefill lab, and "Scheduling":
// token-budgeted batching that cuts prompts into chunks; "Make the Engine
// Talk" section 1.2: the prefill pass that primes the cache).  One workgroup
// per (sequence, KV head, query tile) runs the tile of prefill_body.h.
#include <math.h>

#include "prefill_body.h"

namespace fe {
namespace {

using namespace pre;

template <int G>
__global__ __launch_bounds__(Shape<G>::kThreads) void gqa_prefill_chunk_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[Shape<G>::kLdsBytes];
  // Workgroups are dispatched round-robin over the 8 XCDs (id mod 8).  The
  // query tile is the slowest-varying index, so all tiles of one (sequence,
  // KV head) pair share an XCD and read its K/V through one L2.
  const int pairs = p.B * p.Hkv;
  const int pair = blockIdx.x % pairs;
  prefill_tile<G>(p, lds, blockIdx.x / pairs, pair / p.Hkv, pair % p.Hkv);
}

template <int G>
hipError_t launch_g(const PrefillParams& prm, hipStream_t stream) {
  PrefillParams copy = prm;
  copy.qtiles = (prm.max_q_len + Shape<G>::QT - 1) / Shape<G>::QT;
  const long grid = static_cast<long>(copy.qtiles) * prm.Hkv * prm.B;
  if (grid == 0) return hipSuccess;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gqa_prefill_chunk_kernel<G>), dim3(static_cast<unsigned>(grid)),
                         dim3(Shape<G>::kThreads), args, 0, stream);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const PrefillParams prm = make_prefill_params(a);
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<1>(prm, stream);
    case 2: return launch_g<2>(prm, stream);
    case 3: return launch_g<3>(prm, stream);
    case 4: return launch_g<4>(prm, stream);
    case 5: return launch_g<5>(prm, stream);
    case 6: return launch_g<6>(prm, stream);
    case 7: return launch_g<7>(prm, stream);
    case 8: return launch_g<8>(prm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fe
