// Fused per-head QK-RMSNorm + rotary embedding + KV append: the step that
// turns one batch of projected q/k/v rows into the attention inputs ("Make
// the Engine Talk" section 1.3: RMSNorm and rotary position embeddings are
// forward-pass mechanisms; ForgeEngine README, "What it implements": an
// RMSNorm kernel and the paged KV cache).  Doing it in one pass keeps the
// normed and rotated k from making a round trip through HBM before append.
//
// Each head row x (D = 128) of q and k is normalised per head and rotated
// (rotate-half embedding at table row positions[t]) as norm_rope_row.h
// defines, in fp32, rounded once to bf16.  q rows go to q_out; k rows and
// the unchanged v rows go to their cache slot.
//
// 16 lanes per 256-byte row, 16 bytes each: lane c holds dims 8c .. 8c + 7.
// The sum of squares is a DPP reduction over the 16 lanes; the rotation
// partner of dims 8c .. 8c + 7 is lane c ^ 8 of the same row (DPP row_ror:8).
#include <math.h>

#include "fe_device.h"
#include "fe_kernels.h"
#include "norm_rope_row.h"

namespace fe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Rows are read and written once: non-temporal 16-byte loads and stores.
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_nt(void* p, uint4 w) {
  const u32x4_t v = {w.x, w.y, w.z, w.w};
  __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
}

constexpr int kRowLanes = 16;
constexpr int kThreads = 256;
constexpr int kRowGroups = kThreads / kRowLanes;  // rows a workgroup holds at once

struct NormRopeParams {
  uint16_t* q_out;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* q_w;
  const uint16_t* k_w;
  const float* cos_sin;
  const int32_t* positions;
  const int32_t* slots;
  uint16_t* k_cache;
  uint16_t* v_cache;
  int T, Hq, Hkv, max_pos;
  int64_t num_slots;
  float eps;
};

// One head row as this lane sees it: which token / kind / head, its slot, and
// this lane's 16 bytes of the row.
struct Row {
  bool live;
  int t, kind, head;  // kind: 0 q, 1 k, 2 v
  int pos;            // rotary table row (q and k rows)
  int64_t slot;
  uint4 xw;
  uint4 ww;               // this lane's 8 norm weights
  RopeLane cs;            // this lane's cosines and sines
};

// Each 16-lane group handles kRows rows, kRowGroups rows apart (a workgroup
// covers kRowGroups * kRows consecutive rows, every load instruction of a
// wave reading 4 consecutive 256-byte rows).  All of a thread's loads are
// issued before any of them is used, so a CU keeps more bytes in flight than
// with one row per thread, which left the launch bound by bytes in flight.
// Measured on the 16384-token step (us): 1 row 111, 2 rows 87-88 (78 VGPRs,
// 6 waves/SIMD), 3 rows 90, 4 rows 94-97 (136 VGPRs, 3 waves/SIMD), 8 rows
// 105-108; capping the registers for more waves spills and runs slower.
template <int kRows>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(NormRopeParams p) {
  const int c = threadIdx.x & (kRowLanes - 1);
  // 32-bit row arithmetic: the entry point keeps a launch below 2^32
  // work-items, so there are fewer than 2^28 rows.
  const uint32_t rows_per_tok = p.Hq + 2 * p.Hkv;
  const uint32_t total = static_cast<uint32_t>(p.T) * rows_per_tok;
  const uint32_t R0 = blockIdx.x * (kRowGroups * kRows) + threadIdx.x / kRowLanes;
  const uint32_t t0 = R0 / rows_per_tok;
  const uint32_t r0 = R0 - t0 * rows_per_tok;

  // Every load below is issued unconditionally at a clamped, valid address
  // (token 0 for rows past the end): a load under a branch makes the
  // compiler wait for it where the paths join.  Slots and positions go
  // first, so that the rotary-table loads, which need the position, do not
  // wait for the row loads issued after them.
  Row row[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    Row& w = row[k];
    uint32_t r = r0 + k * kRowGroups;
    const uint32_t dt = r / rows_per_tok;
    r -= dt * rows_per_tok;
    // Rows past the end still run the row-wide DPP reductions so that every
    // lane of a row takes the same path; they store nothing.
    w.live = R0 + k * kRowGroups < total;
    w.t = w.live ? static_cast<int>(t0 + dt) : 0;
    w.kind = static_cast<int>(r) < p.Hq ? 0 : (static_cast<int>(r) < p.Hq + p.Hkv ? 1 : 2);
    w.head = w.kind == 0 ? r : (w.kind == 1 ? r - p.Hq : r - p.Hq - p.Hkv);
    w.slot = p.slots[w.t];
    const int pos = p.positions[w.t];
    w.pos = pos < 0 ? 0 : (pos >= p.max_pos ? p.max_pos - 1 : pos);
  }
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    Row& w = row[k];
    const uint16_t* src = w.kind == 0
                              ? p.q + (static_cast<size_t>(w.t) * p.Hq + w.head) * kHeadDim
                              : (w.kind == 1 ? p.k : p.v) + (static_cast<size_t>(w.t) * p.Hkv + w.head) * kHeadDim;
    w.xw = load_nt(reinterpret_cast<const uint4*>(src) + c);
    w.ww = reinterpret_cast<const uint4*>(w.kind == 0 ? p.q_w : p.k_w)[c];
  }
  // keep the table-address arithmetic (which waits for the positions) after
  // the row loads are issued
  __builtin_amdgcn_sched_barrier(0);
  // the rotary rows (one dependent round trip, under the row loads in flight)
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    Row& w = row[k];
    w.cs = rope_lane(p.cos_sin, w.pos, c);
  }

#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const Row& w = row[k];
    const bool slot_ok = w.kind != 0 && w.slot >= 0 && w.slot < p.num_slots;
    const size_t cache_off =
        slot_ok ? ((static_cast<size_t>(w.slot / kBlockSize) * p.Hkv + w.head) * kBlockSize + w.slot % kBlockSize) *
                      kHeadDim
                : 0;
    if (w.kind == 2) {  // v: bit copy into the pool
      if (w.live && slot_ok) store_nt(reinterpret_cast<uint4*>(p.v_cache + cache_off) + c, w.xw);
      continue;
    }

    const uint4 ow = norm_rope_row(w.xw, w.ww, w.cs, p.eps, c);
    if (!w.live) continue;
    if (w.kind == 0)
      store_nt(reinterpret_cast<uint4*>(p.q_out + (static_cast<size_t>(w.t) * p.Hq + w.head) * kHeadDim) + c, ow);
    else if (slot_ok)
      store_nt(reinterpret_cast<uint4*>(p.k_cache + cache_off) + c, ow);
  }
}

// Rows per 16-lane group: kDeepRows once the launch has at least kDeepMinWgs
// such workgroups (two per CU), else 1 (small launches are latency-bound and
// want every row on its own lane group).
constexpr int kDeepRows = 2;
constexpr int64_t kDeepMinWgs = 512;

}  // namespace

hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t stream) {
  NormRopeParams p{};
  p.q_out = static_cast<uint16_t*>(a.q_out);
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.q_w = static_cast<const uint16_t*>(a.q_norm_w);
  p.k_w = static_cast<const uint16_t*>(a.k_norm_w);
  p.cos_sin = a.cos_sin;
  p.positions = a.positions;
  p.slots = a.slot_mapping;
  p.k_cache = static_cast<uint16_t*>(a.k_cache);
  p.v_cache = static_cast<uint16_t*>(a.v_cache);
  p.T = a.T;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.max_pos = a.max_pos;
  p.num_slots = static_cast<int64_t>(a.num_blocks) * kBlockSize;
  p.eps = a.eps;
  const int64_t rows = static_cast<int64_t>(a.T) * (a.Hq + 2 * a.Hkv);
  if (rows == 0) return hipSuccess;
  void* args[] = {&p};
  const int64_t deep_wgs = (rows + kRowGroups * kDeepRows - 1) / (kRowGroups * kDeepRows);
  if (deep_wgs >= kDeepMinWgs)
    return hipLaunchKernel(reinterpret_cast<const void*>(&qk_norm_rope_kernel<kDeepRows>),
                           dim3(static_cast<unsigned>(deep_wgs)), dim3(kThreads), args, 0, stream);
  const unsigned grid = static_cast<unsigned>((rows + kRowGroups - 1) / kRowGroups);
  return hipLaunchKernel(reinterpret_cast<const void*>(&qk_norm_rope_kernel<1>), dim3(grid), dim3(kThreads), args, 0,
                         stream);
}

}  // namespace fe
