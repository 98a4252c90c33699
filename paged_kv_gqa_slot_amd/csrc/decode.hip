// Paged GQA decode for gfx950: one query token per sequence attends over its
// block table (ForgeEngine README, "What it implements": CUDA paged GQA kernel
// over the paged block allocator; "Make the Engine Talk" sections 1.2-1.3: one
// pass per generated token, grouped-query attention).
//
// Pass 1 (gqa_decode_partition_kernel): one workgroup of 4 waves per
// (sequence, KV head, partition of KV blocks), each running the work item of
// decode_body.h.  With one partition the kernel writes the bf16 output and the
// LSE; otherwise every partition writes a normalised fp32 partial and its LSE,
// and pass 2 (gqa_decode_merge_kernel) combines the partitions of a row by
// log-sum-exp.  With a fused append (fe_paged_gqa_decode_append), pass 1 also
// writes each sequence's new K/V row into its slot, from the workgroup that
// holds the sequence's last block.
#include <math.h>

#include <mutex>

#include "decode_body.h"

// Split-K workspace of the allocation-free decode call, one copy per GPU,
// held until the process ends.  Host code never uses this name as an
// address: decode_scratch() looks the device address up per device.
static __device__ __align__(256) unsigned char scratch[fe::kDecodeScratchBytes];

namespace fe {
namespace {

using namespace dec;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// Automatic split-K (measured on MI355X, 256 CUs):
//  * at least kAutoMinParts partitions of the longest context, which keeps
//    ragged batches balanced (partitions of ~1K tokens at 8K contexts);
//  * at least kAutoFillWgs pass-1 workgroups (two per CU), rounded up to a
//    whole number of CU rounds when the grid is small, since uniform
//    contexts run best when every CU gets the same number of workgroups;
//  * no partition shorter than kAutoMinPartBlocks blocks (256 tokens).
constexpr int kCuCount = 256;
constexpr int kAutoMinParts = 8;
constexpr int kAutoFillWgs = 2 * kCuCount;
constexpr int kAutoMinPartBlocks = 16;

// Pass 1, one workgroup per item (grid B * P * Hkv, Hkv fastest); kNormRope:
// the fused per-head RMSNorm + rotary of q and the new k rows.
template <int G, bool kNormRope>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 3 : 2))) void gqa_decode_partition_kernel(
    DecodeParams p) {
  __shared__ DecodeShared<G, kWaves> sh;
  int wg = blockIdx.x;
  const int g = wg % p.Hkv;
  wg /= p.Hkv;
  const int part = wg % p.P;
  decode_item<G, kWaves, false, kNormRope>(p, sh, wg / p.P, g, part);
}

// Pass 2: one wave per (sequence, query head); lane k owns dims 2k, 2k + 1.
__global__ __launch_bounds__(256) void gqa_decode_merge_kernel(const float* __restrict__ o_part,
                                                               const float* __restrict__ lse_part,
                                                               const int32_t* __restrict__ context_lens,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse,
                                                               int B, int Hq, int P, int part_blocks, int ctx_cap) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= B * Hq) return;
  const int b = row / Hq;
  const int L = clamp_len(context_lens[b], ctx_cap);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int np = (nblk + part_blocks - 1) / part_blocks;
  const float* lp = lse_part + static_cast<size_t>(row) * P;
  const float2* op = reinterpret_cast<const float2*>(o_part + static_cast<size_t>(row) * P * kHeadDim) + lane;
  // Partitions in chunks of kMergeChunk: every load of a chunk (its LSEs and
  // this lane's partial words) is issued at once, so a row of up to
  // kMergeChunk partitions costs one memory round trip; chunks after the
  // first rescale the running sums to the new maximum.
  constexpr int kMergeChunk = 16;
  float M = -INFINITY, z = 0.f, a0 = 0.f, a1 = 0.f;
  for (int i0 = 0; i0 < np; i0 += kMergeChunk) {
    float lv[kMergeChunk];
    float2 ov[kMergeChunk];
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) {
      const int i = i0 + k;
      lv[k] = i < np ? lp[i] : -INFINITY;
      ov[k] = i < np ? op[static_cast<size_t>(i) * (kHeadDim / 2)] : make_float2(0.f, 0.f);
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) Mc = fmaxf(Mc, lv[k]);
    if (!(Mc > -INFINITY)) continue;  // every partition so far is empty
    const float f = fast_exp2((M - Mc) * kLog2e);  // 0 while nothing was summed
    z *= f;
    a0 *= f;
    a1 *= f;
#pragma unroll
    for (int k = 0; k < kMergeChunk; ++k) {
      const float w = fast_exp2((lv[k] - Mc) * kLog2e);
      z += w;
      a0 = fmaf(w, ov[k].x, a0);
      a1 = fmaf(w, ov[k].y, a1);
    }
    M = Mc;
  }
  const bool empty = !(z > 0.f);
  reinterpret_cast<uint32_t*>(out + static_cast<size_t>(row) * kHeadDim)[lane] =
      empty ? 0u : pack_bf16x2(a0 / z, a1 / z);
  if (lane == 0 && lse) lse[row] = empty ? -INFINITY : M + logf(z);
}

template <int G>
hipError_t launch_g(const DecodeParams& prm, hipStream_t stream) {
  const long items = static_cast<long>(prm.B) * prm.P * prm.Hkv;
  DecodeParams copy = prm;
  void* args[] = {&copy};
  const void* kernel = prm.q_norm_w ? reinterpret_cast<const void*>(&gqa_decode_partition_kernel<G, true>)
                                    : reinterpret_cast<const void*>(&gqa_decode_partition_kernel<G, false>);
  return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(items)), dim3(kThreads), args, 0, stream);
}

}  // namespace

bool plan_decode(int B, int Hq, int Hkv, int max_context_len, int num_partitions, DecodePlan* plan) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_context_len < 0 || num_partitions < 0) return false;
  const int nblk_max = (max_context_len + kBlockSize - 1) / kBlockSize;
  DecodePlan r{1, kMaxPartBlocks, 0, 0, 0};
  if (nblk_max > 0 && B > 0) {
    int P;
    if (num_partitions > 0) {
      P = num_partitions;
    } else {
      const long pairs = static_cast<long>(B) * Hkv;
      long pa = (kAutoFillWgs + pairs - 1) / pairs;
      if (pa < kAutoMinParts) pa = kAutoMinParts;
      if (pairs * pa <= 8L * kCuCount) {  // small grid: whole CU rounds
        const long wgs = (pairs * pa + kCuCount - 1) / kCuCount * kCuCount;
        pa = (wgs + pairs - 1) / pairs;
      }
      const long pmax = (nblk_max + kAutoMinPartBlocks - 1) / kAutoMinPartBlocks;
      if (pa > pmax) pa = pmax;
      P = static_cast<int>(pa < 1 ? 1 : pa);
    }
    if (P > nblk_max) P = nblk_max;
    int part_blocks = (nblk_max + P - 1) / P;
    if (part_blocks > kMaxPartBlocks) part_blocks = kMaxPartBlocks;
    P = (nblk_max + part_blocks - 1) / part_blocks;
    r.partitions = P;
    r.part_blocks = part_blocks;
    if (P > 1) {  // [o_part fp32 rows x D][lse_part fp32 rows]
      const size_t rows = static_cast<size_t>(B) * Hq * P;
      const size_t o_bytes = (rows * kHeadDim * sizeof(float) + 255) & ~static_cast<size_t>(255);
      r.o_part_offset = 0;
      r.lse_part_offset = o_bytes;
      r.workspace_bytes = o_bytes + ((rows * sizeof(float) + 255) & ~static_cast<size_t>(255));
    }
  }
  *plan = r;
  return true;
}

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the array's address on device `dev`, looked up with that device current
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  DecodeParams prm = make_decode_params(a.q, a.k_cache, a.v_cache, a.block_tables, a.max_blocks_per_seq,
                                        a.context_lens, a.out, a.lse, a.B, a.Hq, a.Hkv, a.num_blocks,
                                        a.max_context_len, a.scale, a.plan.partitions, a.plan.part_blocks);
  if (a.k_new) {
    prm.k_new = static_cast<const uint16_t*>(a.k_new);
    prm.v_new = static_cast<const uint16_t*>(a.v_new);
    prm.new_slots = a.new_slots;
    prm.k_cache_w = static_cast<uint16_t*>(const_cast<void*>(a.k_cache));
    prm.v_cache_w = static_cast<uint16_t*>(const_cast<void*>(a.v_cache));
    prm.num_slots = static_cast<int64_t>(a.num_blocks) * kBlockSize;
    if (a.q_norm_w) {
      prm.q_norm_w = static_cast<const uint16_t*>(a.q_norm_w);
      prm.k_norm_w = static_cast<const uint16_t*>(a.k_norm_w);
      prm.cos_sin = a.cos_sin;
      prm.positions = a.positions;
      prm.max_pos = a.max_pos;
      prm.eps = a.eps;
    }
  }
  if (prm.P > 1) {
    prm.o_part = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + a.plan.o_part_offset);
    prm.lse_part = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + a.plan.lse_part_offset);
  }
  hipError_t e;
  switch (a.Hq / a.Hkv) {
    case 1: e = launch_g<1>(prm, stream); break;
    case 2: e = launch_g<2>(prm, stream); break;
    case 3: e = launch_g<3>(prm, stream); break;
    case 4: e = launch_g<4>(prm, stream); break;
    case 5: e = launch_g<5>(prm, stream); break;
    case 6: e = launch_g<6>(prm, stream); break;
    case 7: e = launch_g<7>(prm, stream); break;
    case 8: e = launch_g<8>(prm, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || prm.P == 1) return e;
  const float* op = prm.o_part;
  const float* lp = prm.lse_part;
  const int32_t* cl = prm.context_lens;
  uint16_t* out = prm.out;
  float* lse = prm.lse;
  int B = prm.B, Hq = prm.Hq, P = prm.P, pb = prm.part_blocks, cap = prm.ctx_cap;
  void* args[] = {&op, &lp, &cl, &out, &lse, &B, &Hq, &P, &pb, &cap};
  const unsigned grid = static_cast<unsigned>((static_cast<long>(B) * Hq + 3) / 4);
  return hipLaunchKernel(reinterpret_cast<const void*>(&gqa_decode_merge_kernel), dim3(grid), dim3(256), args, 0,
                         stream);
}

}  // namespace fe
