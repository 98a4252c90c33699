// Chunked prefill over the paged cache on the bf16 MFMA units (ForgeEngine
// README, "What it implements": restricted prefill lab, and "Scheduling":
// token-budgeted batching that cuts prompts into chunks; "Make the Engine
// Talk" section 1.2: the prefill pass that primes the cache).  One workgroup
// per (sequence, KV head, query tile) runs the tile of prefill_body.h, with
// its keys split over two wave groups or handled by one (launch_g below).
#include <math.h>

#include "prefill_body.h"

namespace fe {
namespace {

using namespace pre;

constexpr int kCuCount = 256;

// One kernel per (group size, key groups).  Both shapes use at most 256
// VGPRs, two waves per SIMD: one workgroup of two key groups per CU, or two
// single-group workgroups per CU (each takes half the LDS).
template <int G, int KSel, bool kSplitP>
__global__ __launch_bounds__((Shape<G, KSel>::kThreads)) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gqa_prefill_chunk_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[Shape<G, KSel>::kLdsBytes];
  // Workgroups are dispatched round-robin over the 8 XCDs (id mod 8).  All
  // query tiles of one (sequence, KV head) pair go to one XCD and read its
  // K/V through one L2; and they sit next to each other in dispatch order,
  // in groups of 8 pairs (one per XCD), so that on a grid larger than the
  // GPU they also run at the same time and find each other's K/V there.
  const int pairs = p.B * p.Hkv;
  const int units = gridDim.x / pairs;  // query tiles (or tile pairs) per sequence in this launch
  int pair, qt;
  if (pairs % 8 == 0) {
    const int span = 8 * units;
    const int r = blockIdx.x % span;
    pair = (blockIdx.x / span) * 8 + r % 8;
    qt = r / 8;
  } else {
    pair = blockIdx.x % pairs;
    qt = blockIdx.x / pairs;
  }
  prefill_tile<G, KSel, kSplitP>(p, lds, qt, pair / p.Hkv, pair % p.Hkv);
}

template <int G, int KSel>
hipError_t launch_shape(PrefillParams prm, long grid, bool split_p, hipStream_t stream) {
  void* args[] = {&prm};
  const void* fn = split_p ? reinterpret_cast<const void*>(&gqa_prefill_chunk_kernel<G, KSel, true>)
                           : reinterpret_cast<const void*>(&gqa_prefill_chunk_kernel<G, KSel, false>);
  return hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(Shape<G, KSel>::kThreads), args, 0, stream);
}

// Key groups per workgroup.  Two groups (8 waves, one workgroup per CU) pair
// each SIMD's MFMA phase with the other group's softmax phase; with at most
// one workgroup per CU, splitting a tile's keys between them is the faster
// shape.  A larger grid runs workgroups back to back on each CU, where a
// split key loop pays its prologue and merge per half.  There one group per
// workgroup (two resident per CU, overlapping one workgroup's prologue and
// tail with the other's loop) beat the split by 12-15% at 768 to 4096
// workgroups, and two query tiles per workgroup over one K/V stream (groups
// of 4 waves) beat one group: 394 against 476 us on 64 x (1024 + 256),
// keeping the ping-pong and reading each pair of tiles' K/V once.
template <int G>
hipError_t launch_g(const PrefillArgs& a, const PrefillParams& prm, hipStream_t stream) {
  PrefillParams copy = prm;
  copy.qtiles = (prm.max_q_len + Shape<G>::QT - 1) / Shape<G>::QT;
  const long grid = static_cast<long>(copy.qtiles) * prm.Hkv * prm.B;
  if (grid == 0) return hipSuccess;
  if constexpr (Shape<G>::KS == 2) {
    // two key groups per tile while the grid fits the CUs; beyond that, two
    // query tiles per workgroup over one K/V stream
    constexpr bool kPairs = Shape<G>::W == 4;  // (G = 3 runs groups of 3 waves)
    const int ks =
        a.key_groups != 0 ? a.key_groups : (grid > kCuCount ? (kPairs && copy.qtiles > 1 ? 3 : 1) : 2);
    if (ks == 1) return launch_shape<G, 1>(copy, grid, a.split_p, stream);
    if constexpr (kPairs) {
      if (ks == 3) {
        const long pairs_grid = static_cast<long>((copy.qtiles + 1) / 2) * prm.Hkv * prm.B;
        return launch_shape<G, 3>(copy, pairs_grid, a.split_p, stream);
      }
    } else {
      if (ks == 3) return hipErrorInvalidValue;
    }
  } else {
    if (a.key_groups >= 2) return hipErrorInvalidValue;
  }
  return launch_shape<G, 0>(copy, grid, a.split_p, stream);
}

}  // namespace

static_assert(Shape<1>::KS == 2 && Shape<3>::KS == 2 && Shape<4>::KS == 2 && Shape<5>::KS == 1,
              "two key groups exactly for Hq/Hkv <= 4");
bool prefill_two_key_groups_supported(int G) { return G >= 1 && G <= 4; }
bool prefill_query_tile_pairs_supported(int G) { return G == 1 || G == 2 || G == 4; }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const PrefillParams prm = make_prefill_params(a);
  switch (a.Hq / a.Hkv) {
    case 1: return launch_g<1>(a, prm, stream);
    case 2: return launch_g<2>(a, prm, stream);
    case 3: return launch_g<3>(a, prm, stream);
    case 4: return launch_g<4>(a, prm, stream);
    case 5: return launch_g<5>(a, prm, stream);
    case 6: return launch_g<6>(a, prm, stream);
    case 7: return launch_g<7>(a, prm, stream);
    case 8: return launch_g<8>(a, prm, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fe
