// Mixed batch in one launch: the decode rows and the prefill chunks that a
// token-budgeted continuous batcher puts into one step (ForgeEngine README,
// "Scheduling": continuous, token-budgeted batching; "What it implements":
// CUDA paged GQA kernel and restricted prefill lab; "Make the Engine Talk"
// section 1.2: prefill primes the cache, then one pass per generated token).
//
// Sequences [0, num_decode) are decode rows (one query each, at packed row
// query_start_loc[b]); sequences [num_decode, B) are prefill chunks.  One
// grid holds both kinds of workgroup: first the decode items (sequence, KV
// head, partition), run by as many waves as a prefill tile, then the prefill
// query tiles, in groups of 8 (sequence, KV head) pairs (one per XCD) with a
// group's query tiles next to each other.  A split decode
// sequence is merged in the same launch by the last of its partitions to
// finish.  Every workgroup reserves the prefill tile's LDS and registers, so
// a CU runs one workgroup of either kind at a time; the two kinds overlap
// across CUs, not within one.
#include <math.h>

#include "decode_body.h"
#include "prefill_body.h"

namespace fe {
namespace {

constexpr int kCuCount = 256;

struct MixedParams {
  pre::PrefillParams pre;
  dec::DecodeParams dec;
  int n_pre_wgs;   // prefill workgroups: query tiles x pre_pairs
  int pre_pairs;   // (B - num_decode) * Hkv
  int num_decode;
  int n_dec_wgs;   // decode workgroups: num_decode x P x Hkv
};

template <int G>
struct MixedShape {
  static constexpr int kThreads = pre::Shape<G>::kThreads;
  static constexpr int W = kThreads / 64;  // waves per decode item
  static constexpr size_t kDecLds = sizeof(dec::DecodeShared<G, W>);
  static constexpr size_t kLdsBytes =
      pre::Shape<G>::kLdsBytes > kDecLds ? static_cast<size_t>(pre::Shape<G>::kLdsBytes) : kDecLds;
};

template <int G>
__global__ __launch_bounds__(MixedShape<G>::kThreads) void gqa_mixed_kernel(MixedParams mp) {
  using M = MixedShape<G>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[M::kLdsBytes];
  // decode items first, then the prefill tiles: the decode items stream HBM
  // on every CU, and the long MFMA-bound prefill tiles fill the CUs that the
  // decode tail frees (measured faster than prefill first, and than an even
  // interleave, which splits a sequence's query tiles over several XCDs)
  const int wg = blockIdx.x;
  const bool is_pre = wg >= mp.n_dec_wgs;
  const int k = is_pre ? wg - mp.n_dec_wgs : wg;
  if (is_pre) {
    int pair, qt;
    if (mp.pre_pairs % 8 == 0) {
      // groups of 8 (sequence, KV head) pairs, one per XCD, with all query
      // tiles of a group next to each other in dispatch order: the tiles
      // that share a pair's K/V start close together and find it in L2
      const int span = 8 * mp.pre.qtiles;
      const int r = k % span;
      pair = (k / span) * 8 + r % 8;
      qt = r / 8;
    } else {
      pair = k % mp.pre_pairs;
      qt = k / mp.pre_pairs;
    }
    pre::prefill_tile<G>(mp.pre, lds, qt, mp.num_decode + pair / mp.pre.Hkv, pair % mp.pre.Hkv);
  } else {
    int d = k;
    const int g = d % mp.dec.Hkv;
    d /= mp.dec.Hkv;
    const int part = d % mp.dec.P;
    dec::decode_item<G, M::W, true>(mp.dec, *reinterpret_cast<dec::DecodeShared<G, M::W>*>(lds), d / mp.dec.P, g,
                                    part);
  }
}

template <int G>
hipError_t launch_g(MixedParams mp, int B, hipStream_t stream) {
  const int n_pre_seq = B - mp.num_decode;
  const int qtiles = n_pre_seq > 0 ? (mp.pre.max_q_len + pre::Shape<G>::QT - 1) / pre::Shape<G>::QT : 0;
  mp.pre.qtiles = qtiles;
  mp.pre_pairs = n_pre_seq * mp.pre.Hkv;
  mp.n_pre_wgs = qtiles * mp.pre_pairs;
  mp.n_dec_wgs = mp.num_decode * mp.dec.P * mp.dec.Hkv;
  const long grid = static_cast<long>(mp.n_pre_wgs) + mp.n_dec_wgs;
  if (grid == 0) return hipSuccess;
  void* args[] = {&mp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gqa_mixed_kernel<G>), dim3(static_cast<unsigned>(grid)),
                         dim3(MixedShape<G>::kThreads), args, 0, stream);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

bool plan_mixed(int num_decode, int Hq, int Hkv, int max_context_len, int num_partitions, MixedPlan* plan) {
  if (num_decode < 0 || Hq <= 0 || Hkv <= 0 || max_context_len < 0 || num_partitions < 0) return false;
  const int nblk_max = (max_context_len + kBlockSize - 1) / kBlockSize;
  MixedPlan r{1, kMaxPartBlocks, 0, 0, 0};
  if (nblk_max > 0 && num_decode > 0) {
    int P = num_partitions;
    if (P <= 0) {
      const long pairs = static_cast<long>(num_decode) * Hkv;
      const long by_items = (static_cast<long>(kMixedItemsPerCu) * kCuCount + pairs / 2) / pairs;
      const long by_len = (nblk_max + kMixedMinPartBlocks - 1) / kMixedMinPartBlocks;
      const long pa = by_items < by_len ? by_items : by_len;
      P = static_cast<int>(pa < 1 ? 1 : pa);
    }
    if (P > nblk_max) P = nblk_max;
    int part_blocks = (nblk_max + P - 1) / P;
    if (part_blocks > kMaxPartBlocks) part_blocks = kMaxPartBlocks;
    P = (nblk_max + part_blocks - 1) / part_blocks;
    r.partitions = P;
    r.part_blocks = part_blocks;
    if (P > 1) {
      const size_t rows = static_cast<size_t>(num_decode) * Hq * P;
      const size_t c_bytes = align256(static_cast<size_t>(num_decode) * Hkv * sizeof(int));
      const size_t o_bytes = align256(rows * kHeadDim * sizeof(float));
      r.o_part_offset = c_bytes;
      r.lse_part_offset = c_bytes + o_bytes;
      r.workspace_bytes = c_bytes + o_bytes + align256(rows * sizeof(float));
    }
  }
  *plan = r;
  return true;
}

hipError_t launch_mixed(const MixedArgs& a, hipStream_t stream) {
  const PrefillArgs& x = a.all;
  MixedParams mp{};
  mp.pre = pre::make_prefill_params(x);
  mp.dec = dec::make_decode_params(x.q, x.k_cache, x.v_cache, x.block_tables, x.max_blocks_per_seq, x.context_lens,
                                   x.out, x.lse, a.num_decode, x.Hq, x.Hkv, x.num_blocks, x.max_context_len, x.scale,
                                   a.plan.partitions, a.plan.part_blocks);
  mp.dec.q_rows = x.query_start_loc;
  mp.dec.q_rows_count = x.total_q;
  if (a.plan.partitions > 1) {
    char* ws = static_cast<char*>(a.workspace);
    mp.dec.arrivals = reinterpret_cast<int*>(ws);
    mp.dec.o_part = reinterpret_cast<float*>(ws + a.plan.o_part_offset);
    mp.dec.lse_part = reinterpret_cast<float*>(ws + a.plan.lse_part_offset);
  }
  mp.num_decode = a.num_decode;
  switch (x.Hq / x.Hkv) {
    case 1: return launch_g<1>(mp, x.B, stream);
    case 2: return launch_g<2>(mp, x.B, stream);
    case 3: return launch_g<3>(mp, x.B, stream);
    case 4: return launch_g<4>(mp, x.B, stream);
    case 5: return launch_g<5>(mp, x.B, stream);
    case 6: return launch_g<6>(mp, x.B, stream);
    case 7: return launch_g<7>(mp, x.B, stream);
    case 8: return launch_g<8>(mp, x.B, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fe
