// Paged GQA decode for gfx950: one query token per sequence attends over its
// block table (ForgeEngine README, "What it implements": CUDA paged GQA kernel
// over the paged block allocator; "Make the Engine Talk" sections 1.2-1.3: one
// pass per generated token, grouped-query attention).
//
// Pass 1 (gqa_decode_partition_kernel): one workgroup of 4 waves per
// (sequence, KV head, partition of KV blocks).  Each wave takes every 4th
// block of the partition and streams its K and V tiles (4 KiB each, one
// contiguous run per (block, KV head)) straight into registers with
// non-temporal loads, one tile ahead of the math.  A wave holds all G query
// heads of the group, so each K/V byte is read from HBM once and used G times
// from registers.
//
//   lane layout inside a wave: lane = 16 * r + c.  Load instruction j of a
//   tile reads token rows 4j .. 4j + 3 as one contiguous 1 KiB run, so lane
//   (r, c) holds dims [8c, 8c + 8) of tokens r, r + 4, r + 8, r + 12.
//   QK^T: v_dot2_f32_bf16 on packed bf16 pairs, then a 4-step DPP sum over the
//   16 lanes of a row.  Each row keeps its own online-softmax state (running
//   max m, sum l, acc[G][8]) in the log2 domain; the max is only raised when
//   it grows by more than 8 (so exp2 stays <= 256 and the rescale of acc is
//   rare).  PV: v_dot2_f32_bf16 with the softmax weights of two tokens
//   packed as a bf16 pair against the matching V words (fp32
//   accumulation).  A partially filled last
//   block is handled after the main loop by a masked variant of the same step.
//
// At the end the 4 rows and 4 waves are merged (max-shifted sums) through
// cross-lane shuffles and LDS.  With one partition the kernel writes the
// bf16 output and the LSE; otherwise it writes a normalised fp32 partial and
// its LSE, and pass 2 (gqa_decode_merge_kernel) combines the partitions of a
// row by log-sum-exp.
#include <math.h>

#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kEmptyMax = -1.0e30f;   // running max before the first valid token
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
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
#ifndef FE_DECODE_PREFETCH
#define FE_DECODE_PREFETCH 1
#endif
constexpr int kPrefetch = FE_DECODE_PREFETCH;  // tiles in flight per wave beyond the one being consumed

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint16_t* out;
  float* lse;
  float* o_part;
  float* lse_part;
  int max_blocks, B, Hq, Hkv, num_blocks, ctx_cap;
  int P, part_blocks;
  float scale_log2;  // |scale| * log2(e)
  int negate_q;      // scale < 0
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

struct Tile {
  uint4 k[4];  // k[j]: dims [8c, 8c + 8) of token 4j + r
  uint4 v[4];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor over one 4 KiB (block, KV head) tile.  Loads at offsets
// >= num_bytes return zeros without touching memory, which masks whole
// out-of-range tiles (num_bytes = 0) and the unused rows of a partial last
// block (num_bytes = valid_tokens * 256) while every load instruction is
// still issued unconditionally.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), static_cast<short>(0), num_bytes,
                                           0x00020000);
}

// Cache policy of the K/V loads: non-temporal (streamed, read once).
constexpr int kLoadPolicyNT = 2;

// Lane reads uint4 number lane + 64 j of the tile: instruction j fetches
// token rows 4j .. 4j + 3 as one contiguous 1 KiB run.
__device__ __forceinline__ void load_tile(Tile& t, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int lane) {
  const int off = lane * 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(kr, off + 1024 * j, 0, kLoadPolicyNT);
    t.k[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(vr, off + 1024 * j, 0, kLoadPolicyNT);
    t.v[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

__device__ __forceinline__ void words4(const uint4& a, uint32_t (&w)[4]) {
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
}

// Sum over each aligned group of 16 lanes (a DPP row); every lane gets it.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  x += dpp<kDppRowMirror>(x);
  return x;
}

template <int G>
struct State {
  float m[G];   // running max (log2 units), uniform within a row
  float l[G];   // running sum of exp2(s - m), uniform within a row
  float acc[G][8];
};

// Consume one 16-token tile.  With kTail, tokens at or beyond `rem` (the
// number of valid tokens in this block) are masked: their scores become -inf.
// Their K/V words were already zeroed by the load's buffer range, so no slot
// contents (NaN included) can reach acc through 0 * x.
template <int G, bool kTail>
__device__ __forceinline__ void consume(State<G>& st, const Tile& t, const uint32_t (&qw)[G][4], float scale_log2,
                                        int r, int rem) {
  // raw scores q.k (scale_log2 > 0: a negative scale was folded into q's sign)
  float s[4][G];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t kw[4];
    words4(t.k[j], kw);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) a = dot2_bf16(qw[h][i], kw[i], a);
      s[j][h] = sum16(a);
    }
  }
  if (kTail) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * j + r >= rem)
#pragma unroll
        for (int h = 0; h < G; ++h) s[j][h] = -INFINITY;
  }
  bool need = false;
  float mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h])) * scale_log2;
    need |= mx[h] > st.m[h] + kRescaleSlack;
  }
  if (__any(need)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (mx[h] > st.m[h] + kRescaleSlack) {
        const float a = fast_exp2(st.m[h] - mx[h]);
        st.m[h] = mx[h];
        st.l[h] *= a;
#pragma unroll
        for (int i = 0; i < 8; ++i) st.acc[h][i] *= a;
      }
    }
  }
  // p = 2^(s * scale_log2 - m); the PV product takes p in bf16 pairs
  // (tokens r + 8 u and r + 8 u + 4 share a pair) with fp32 accumulation
  uint32_t pp[2][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = fast_exp2(fmaf(s[j][h], scale_log2, -st.m[h]));
    st.l[h] += (p[0] + p[1]) + (p[2] + p[3]);
    pp[0][h] = pack_bf16x2(p[0], p[1]);
    pp[1][h] = pack_bf16x2(p[2], p[3]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    uint32_t va[4], vb[4];
    words4(t.v[2 * u], va);
    words4(t.v[2 * u + 1], vb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (dim 2i of both tokens) and (dim 2i + 1 of both tokens) as bf16 pairs
      const uint32_t even = (va[i] & 0xffffu) | (vb[i] << 16);
      const uint32_t odd = (va[i] >> 16) | (vb[i] & 0xffff0000u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        st.acc[h][2 * i] = dot2_bf16(pp[u][h], even, st.acc[h][2 * i]);
        st.acc[h][2 * i + 1] = dot2_bf16(pp[u][h], odd, st.acc[h][2 * i + 1]);
      }
    }
  }
}

template <int G>
struct DecodeShared {
  float o[kWaves][G][kHeadDim];
  float m[kWaves][G];
  float l[kWaves][G];
};

// One work item: (sequence b, KV head g, partition part).
template <int G>
__device__ __forceinline__ void decode_item(const DecodeParams& p, DecodeShared<G>& sh, int b, int g, int part) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane >> 4, c = lane & 15;

  const int blk0 = part * p.part_blocks;

  // Issued together, before the context length is known: the length, this
  // wave's block ids (lane k <- local block wave + 4 k, i.e. the wave's tile
  // k; a partition has at most kMaxPartBlocks = 4 * 64 blocks) and q.
  const int Lraw = p.context_lens[b];
  const int row_blocks = min(p.part_blocks, p.max_blocks - blk0);  // table entries this partition may use
  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks + blk0;
  int ids = wave + kWaves * lane < row_blocks ? bt[wave + kWaves * lane] : 0;
  const size_t row0 = static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G;  // first q head of the group
  uint32_t qw[G][4];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + row0 * kHeadDim) + c;
#pragma unroll
    for (int h = 0; h < G; ++h) words4(qp[h * (kHeadDim / 8)], qw[h]);
    if (p.negate_q) {  // scale < 0: flip q's signs (exact) and use |scale|
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) qw[h][i] ^= 0x80008000u;
    }
  }
  ids = min(max(ids, 0), p.num_blocks - 1);

  const int L = clamp_len(Lraw, p.ctx_cap);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  if (blk0 >= nblk && p.P > 1) return;  // nothing here; pass 2 never reads this partition
  const int blk1 = min(nblk, blk0 + p.part_blocks);
  const int nb = max(0, blk1 - blk0);
  // tokens in the sequence's last block; that block is masked if partial
  const int rem = L - (nblk - 1) * kBlockSize;
  const bool has_tail = nb > 0 && blk1 == nblk && rem < kBlockSize;
  const int nfull = nb - (has_tail ? 1 : 0);

  State<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kEmptyMax;
    st.l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) st.acc[h][i] = 0.f;
  }

  const size_t blk_stride = static_cast<size_t>(p.Hkv) * kTileElems;
  const uint16_t* kg = p.k_cache + static_cast<size_t>(g) * kTileElems;
  const uint16_t* vg = p.v_cache + static_cast<size_t>(g) * kTileElems;

  // This wave's full tiles are local blocks wave, wave + 4, ... (n of them).
  // A ring of kPrefetch + 1 register tiles keeps kPrefetch tiles in flight
  // while one is consumed.  Every load is issued unconditionally (tiles past
  // n are masked by their buffer range), so the compiler's vmcnt bookkeeping
  // sees one straight-line schedule and waits only for the oldest tile.
  const int n = nfull > wave ? (nfull - wave + kWaves - 1) / kWaves : 0;
  auto issue = [&](Tile& dst, int t) {
    const bool ok = t < n;
    const size_t o = ok ? static_cast<size_t>(__builtin_amdgcn_readlane(ids, t)) * blk_stride : 0;
    const int bytes = ok ? kTileElems * 2 : 0;
    load_tile(dst, tile_rsrc(kg + o, bytes), tile_rsrc(vg + o, bytes), lane);
  };
  Tile ring[kPrefetch + 1];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) issue(ring[k], k);
  for (int t = 0; t < n; t += kPrefetch + 1) {
#pragma unroll
    for (int k = 0; k <= kPrefetch; ++k) {
      issue(ring[(k + kPrefetch) % (kPrefetch + 1)], t + k + kPrefetch);
      if (t + k < n) consume<G, false>(st, ring[k], qw, p.scale_log2, r, kBlockSize);
    }
  }
  if (has_tail && wave == (nb - 1) % kWaves) {
    const size_t o = static_cast<size_t>(__builtin_amdgcn_readlane(ids, (nb - 1) / kWaves)) * blk_stride;
    const int bytes = rem * kHeadDim * 2;
    load_tile(ring[0], tile_rsrc(kg + o, bytes), tile_rsrc(vg + o, bytes), lane);
    consume<G, true>(st, ring[0], qw, p.scale_log2, r, rem);
  }

  // merge the 4 rows of this wave: lanes c, c+16, c+32, c+48 hold the same dims
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = st.m[h];
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = fast_exp2(st.m[h] - M);
    float l = st.l[h] * f;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = st.acc[h][k] * f;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      st.acc[h][k] = a;
    }
    st.m[h] = M;
    st.l[h] = l;
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&sh.o[wave][h][8 * c]);
      dst[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
      dst[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
    }
    if (c == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sh.m[wave][h] = st.m[h];
        sh.l[wave][h] = st.l[h];
      }
    }
  }
  __syncthreads();

  // merge the 4 waves and write
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    float M = sh.m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sh.m[w][h]);
    float lsum = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(sh.m[w][h] - M);
      lsum = fmaf(sh.l[w][h], f, lsum);
      val = fmaf(sh.o[w][h][d], f, val);
    }
    const bool empty = !(lsum > 0.f);
    const float res = empty ? 0.f : val / lsum;
    const float lse_nat = empty ? -INFINITY : (M + log2f(lsum)) * kLn2;
    const size_t row = row0 + h;
    if (p.P == 1) {
      p.out[row * kHeadDim + d] = to_bf16(res);
      if (d == 0 && p.lse) p.lse[row] = lse_nat;
    } else {
      p.o_part[(row * p.P + part) * kHeadDim + d] = res;
      if (d == 0) p.lse_part[row * p.P + part] = lse_nat;
    }
  }
}

// Pass 1, one workgroup per item (grid B * P * Hkv, Hkv fastest).
template <int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 3 : 2))) void gqa_decode_partition_kernel(
    DecodeParams p) {
  __shared__ DecodeShared<G> sh;
  int wg = blockIdx.x;
  const int g = wg % p.Hkv;
  wg /= p.Hkv;
  const int part = wg % p.P;
  decode_item<G>(p, sh, wg / p.P, g, part);
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
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, lp[i]);
  float z = 0.f, a0 = 0.f, a1 = 0.f;
  if (M > -INFINITY) {
    const float2* op = reinterpret_cast<const float2*>(o_part + static_cast<size_t>(row) * P * kHeadDim) + lane;
    for (int i = 0; i < np; ++i) {
      const float w = fast_exp2((lp[i] - M) * kLog2e);
      const float2 v = op[static_cast<size_t>(i) * (kHeadDim / 2)];
      z += w;
      a0 = fmaf(w, v.x, a0);
      a1 = fmaf(w, v.y, a1);
    }
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
  return hipLaunchKernel(reinterpret_cast<const void*>(&gqa_decode_partition_kernel<G>),
                         dim3(static_cast<unsigned>(items)), dim3(kThreads), args, 0, stream);
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

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  DecodeParams prm{};
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k_cache = static_cast<const uint16_t*>(a.k_cache);
  prm.v_cache = static_cast<const uint16_t*>(a.v_cache);
  prm.block_tables = a.block_tables;
  prm.context_lens = a.context_lens;
  prm.out = static_cast<uint16_t*>(a.out);
  prm.lse = a.lse;
  prm.max_blocks = a.max_blocks_per_seq;
  prm.B = a.B;
  prm.Hq = a.Hq;
  prm.Hkv = a.Hkv;
  prm.num_blocks = a.num_blocks;
  const long cap_bt = static_cast<long>(a.max_blocks_per_seq) * kBlockSize;
  prm.ctx_cap = static_cast<int>(a.max_context_len < cap_bt ? a.max_context_len : cap_bt);
  prm.P = a.plan.partitions;
  prm.part_blocks = a.plan.part_blocks;
  prm.scale_log2 = fabsf(a.scale) * kLog2e;
  prm.negate_q = a.scale < 0.f;
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
