// Paged GQA decode for gfx950: one query token per sequence attends over its
// block table (ForgeEngine README, "What it implements": CUDA paged GQA kernel
// over the paged block allocator; "Make the Engine Talk" sections 1.2-1.3: one
// pass per generated token, grouped-query attention).
//
// Pass 1 (gqa_decode_partition_kernel): one workgroup of 4 waves per
// (sequence, KV head, partition of KV blocks).  Each wave takes every 4th
// block of the partition and streams its K and V tiles (4 KiB each, one
// contiguous run per (block, KV head)) straight into registers, one tile ahead
// of the math.  A wave holds all G query heads of the group, so each K/V byte
// is read from HBM once and used G times from registers.
//
//   lane layout inside a wave: lane = 8 * grp + c.  The 8 lanes of a group
//   share tokens grp and grp + 8 of every block; lane c holds dims
//   [16c, 16c + 16).  QK^T: v_dot2_f32_bf16 on packed bf16 pairs, then a
//   3-step DPP sum over the 8 lanes.  Each group keeps its own online-softmax
//   state (running max m, sum l, acc[G][16]) in the log2 domain; the max is
//   only raised when it grows by more than 8 (so exp2 stays <= 256 and the
//   rescale of acc is rare).  PV: fp32 FMA on the unpacked V row.
//
// At the end the 8 groups and 4 waves are merged (max-shifted sums) through
// DPP, cross-lane shuffles and LDS.  With one partition the kernel writes the
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
constexpr int kTargetWorkgroups = 2048;  // automatic split-K aims for this many pass-1 workgroups
constexpr int kMinPartBlocks = 8;        // ... but no partition shorter than 128 tokens

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
  float scale_log2;
};

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

struct Tile {
  uint4 k[4];  // tokens grp (k[0..1]) and grp + 8 (k[2..3]), dims [16c, 16c + 16)
  uint4 v[4];
};

__device__ __forceinline__ void load_tile(Tile& t, const uint16_t* kbase, const uint16_t* vbase, int lane_vec) {
  const uint4* kp = reinterpret_cast<const uint4*>(kbase) + lane_vec;
  const uint4* vp = reinterpret_cast<const uint4*>(vbase) + lane_vec;
  // token grp + 8 is 8 rows = 8 * 128 bf16 = 128 uint4 further on
  t.k[0] = kp[0];
  t.k[1] = kp[1];
  t.k[2] = kp[128];
  t.k[3] = kp[129];
  t.v[0] = vp[0];
  t.v[1] = vp[1];
  t.v[2] = vp[128];
  t.v[3] = vp[129];
}

__device__ __forceinline__ void words(const uint4& a, const uint4& b, uint32_t (&w)[8]) {
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

template <int G>
struct State {
  float m[G];
  float l[G];
  float acc[G][16];
};

// Consume one 16-token tile.  `valid` holds, per token j of this lane's group
// (t = grp + 8 j), whether it lies inside the context; `tail` is wave-uniform
// and true only for a partially filled last block.
template <int G>
__device__ __forceinline__ void consume(State<G>& st, const Tile& t, const uint32_t (&qw)[G][8], float scale_log2,
                                        bool tail, bool valid0, bool valid1) {
  float s[2][G];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t kw[8];
    words(t.k[2 * j], t.k[2 * j + 1], kw);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = dot2_bf16(qw[h][i], kw[i], a);
      s[j][h] = a;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < G; ++h) s[j][h] = sum8(s[j][h]) * scale_log2;
  if (tail) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!valid0) s[0][h] = -INFINITY;
      if (!valid1) s[1][h] = -INFINITY;
    }
  }
  bool need = false;
  float mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    mx[h] = fmaxf(s[0][h], s[1][h]);
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
        for (int i = 0; i < 16; ++i) st.acc[h][i] *= a;
      }
    }
  }
  float p[2][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    p[0][h] = fast_exp2(s[0][h] - st.m[h]);
    p[1][h] = fast_exp2(s[1][h] - st.m[h]);
    st.l[h] += p[0][h] + p[1][h];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t vw[8];
    words(t.v[2 * j], t.v[2 * j + 1], vw);
    if (tail && !(j ? valid1 : valid0)) {
      // never let a masked slot's contents (possibly NaN) reach acc via 0 * x
#pragma unroll
      for (int i = 0; i < 8; ++i) vw[i] = 0u;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v0 = bf16_lo(vw[i]), v1 = bf16_hi(vw[i]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        st.acc[h][2 * i] = fmaf(p[j][h], v0, st.acc[h][2 * i]);
        st.acc[h][2 * i + 1] = fmaf(p[j][h], v1, st.acc[h][2 * i + 1]);
      }
    }
  }
}

template <int G>
__global__ __launch_bounds__(kThreads) void gqa_decode_partition_kernel(DecodeParams p) {
  __shared__ int s_bt[kMaxPartBlocks];
  __shared__ float s_o[kWaves][G][kHeadDim];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int grp = lane >> 3, c = lane & 7;

  int wg = blockIdx.x;
  const int g = wg % p.Hkv;
  wg /= p.Hkv;
  const int part = wg % p.P;
  const int b = wg / p.P;
  const int L = clamp_len(p.context_lens[b], p.ctx_cap);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int blk0 = part * p.part_blocks;
  if (blk0 >= nblk && p.P > 1) return;  // nothing here; pass 2 never reads this partition
  const int blk1 = min(nblk, blk0 + p.part_blocks);
  const int nb = max(0, blk1 - blk0);

  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks + blk0;
  for (int i = tid; i < nb; i += kThreads) s_bt[i] = min(max(bt[i], 0), p.num_blocks - 1);

  const size_t row0 = static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G;  // first q head of the group
  uint32_t qw[G][8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + row0 * kHeadDim) + 2 * c;
#pragma unroll
    for (int h = 0; h < G; ++h) words(qp[h * 16], qp[h * 16 + 1], qw[h]);
  }
  __syncthreads();

  State<G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = kEmptyMax;
    st.l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) st.acc[h][i] = 0.f;
  }

  const size_t blk_stride = static_cast<size_t>(p.Hkv) * kTileElems;
  const uint16_t* kg = p.k_cache + static_cast<size_t>(g) * kTileElems;
  const uint16_t* vg = p.v_cache + static_cast<size_t>(g) * kTileElems;
  const int lane_vec = grp * (kHeadDim / 8) + 2 * c;  // uint4 index of this lane's first K/V word
  const int tail_blk = (L % kBlockSize) ? nblk - 1 : -1;
  const int t0 = grp, t1 = grp + 8;
  const int rem = L - (nblk - 1) * kBlockSize;  // tokens in the last block

  Tile A, B;
  int i = wave;
  if (i < nb) {
    const size_t o = static_cast<size_t>(uniform(s_bt[i])) * blk_stride;
    load_tile(A, kg + o, vg + o, lane_vec);
  }
  for (; i < nb; i += 2 * kWaves) {
    const int i2 = i + kWaves;
    if (i2 < nb) {
      const size_t o = static_cast<size_t>(uniform(s_bt[i2])) * blk_stride;
      load_tile(B, kg + o, vg + o, lane_vec);
    }
    consume<G>(st, A, qw, p.scale_log2, blk0 + i == tail_blk, t0 < rem, t1 < rem);
    if (i2 >= nb) break;
    const int i3 = i2 + kWaves;
    if (i3 < nb) {
      const size_t o = static_cast<size_t>(uniform(s_bt[i3])) * blk_stride;
      load_tile(A, kg + o, vg + o, lane_vec);
    }
    consume<G>(st, B, qw, p.scale_log2, blk0 + i2 == tail_blk, t0 < rem, t1 < rem);
  }

  // merge the 8 groups of this wave: lanes c, c+8, ..., c+56 hold the same dims
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = st.m[h];
    M = fmaxf(M, dpp<kDppRowRor8>(M));
    M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = fast_exp2(st.m[h] - M);
    float l = st.l[h] * f;
    l += dpp<kDppRowRor8>(l);
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a = st.acc[h][k] * f;
      a += dpp<kDppRowRor8>(a);
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      st.acc[h][k] = a;
    }
    st.m[h] = M;
    st.l[h] = l;
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(&s_o[wave][h][16 * c]);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        dst[k] = make_float4(st.acc[h][4 * k], st.acc[h][4 * k + 1], st.acc[h][4 * k + 2], st.acc[h][4 * k + 3]);
    }
    if (c == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        s_m[wave][h] = st.m[h];
        s_l[wave][h] = st.l[h];
      }
    }
  }
  __syncthreads();

  // merge the 4 waves and write
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float lsum = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = fast_exp2(s_m[w][h] - M);
      lsum = fmaf(s_l[w][h], f, lsum);
      val = fmaf(s_o[w][h][d], f, val);
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
  const unsigned grid = static_cast<unsigned>(prm.B) * prm.P * prm.Hkv;
  DecodeParams copy = prm;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gqa_decode_partition_kernel<G>), dim3(grid),
                         dim3(kThreads), args, 0, stream);
}

}  // namespace

bool plan_decode(int B, int Hq, int Hkv, int max_context_len, int num_partitions, DecodePlan* plan) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || max_context_len < 0 || num_partitions < 0) return false;
  const int nblk_max = (max_context_len + kBlockSize - 1) / kBlockSize;
  DecodePlan r{1, kMaxPartBlocks, 0, 0};
  if (nblk_max > 0 && B > 0) {
    int P;
    if (num_partitions > 0) {
      P = num_partitions;
    } else {
      const long pairs = static_cast<long>(B) * Hkv;
      P = static_cast<int>((kTargetWorkgroups + pairs - 1) / pairs);
      const int pmax = (nblk_max + kMinPartBlocks - 1) / kMinPartBlocks;
      if (P > pmax) P = pmax;
      if (P < 1) P = 1;
    }
    if (P > nblk_max) P = nblk_max;
    int part_blocks = (nblk_max + P - 1) / P;
    if (part_blocks > kMaxPartBlocks) part_blocks = kMaxPartBlocks;
    P = (nblk_max + part_blocks - 1) / part_blocks;
    r.partitions = P;
    r.part_blocks = part_blocks;
    if (P > 1) {
      const size_t rows = static_cast<size_t>(B) * Hq * P;
      const size_t o_bytes = (rows * kHeadDim * sizeof(float) + 255) & ~static_cast<size_t>(255);
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
  prm.scale_log2 = a.scale * kLog2e;
  if (prm.P > 1) {
    prm.o_part = static_cast<float*>(a.workspace);
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
