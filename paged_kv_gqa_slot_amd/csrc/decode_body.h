// Paged GQA decode work item for gfx950, shared by the decode kernel and the
// mixed decode/prefill kernel (ForgeEngine README, "What it implements": CUDA
// paged GQA kernel over the paged block allocator; "Make the Engine Talk"
// sections 1.2-1.3: one pass per generated token, grouped-query attention).
//
// One item is (sequence, KV head, partition of KV blocks), run by W waves.
// Each wave takes every W-th block of the partition and streams its K and V
// tiles (4 KiB each, one contiguous run per (block, KV head)) straight into
// registers with non-temporal loads, one tile ahead of the math.  A wave
// holds all G query heads of the group, so each K/V byte is read from HBM
// once and used G times from registers.
//
//   lane layout inside a wave: lane = 16 * r + c.  Load instruction j of a
//   tile reads token rows 4j .. 4j + 3 as one contiguous 1 KiB run, so lane
//   (r, c) holds dims [8c, 8c + 8) of tokens r, r + 4, r + 8, r + 12.
//   QK^T: v_dot2_f32_bf16 on packed bf16 pairs, then a 4-step DPP sum over the
//   16 lanes of a row.  Each row keeps its own online-softmax state (running
//   max m, sum l, acc[G][8]) in the log2 domain; the max is only raised when
//   it grows by more than 8 (so exp2 stays <= 256 and the rescale of acc is
//   rare).  PV in fp32: each V element is widened from bf16 (exact) and
//   accumulated with the fp32 softmax weight by one fma, so the weights that
//   enter the numerator are the ones summed into l.  A partially filled last block is handled after the main
//   loop by a masked variant of the same step; with a fused append the last
//   block always goes that way, and there the new token's row is written to
//   the cache and patched into the loaded tile.  That form can also
//   normalise and rotate q and the new k row first (norm_rope_row.h), which
//   takes the whole per-token attention input step into one launch.
//
// At the end the 4 rows and W waves are merged (max-shifted sums) through
// cross-lane shuffles and LDS.  An unsplit sequence gets its bf16 output and
// LSE directly; a split one leaves a normalised fp32 partial and its LSE per
// partition, merged by log-sum-exp either by a second pass or, fused, by the
// last partition to finish.
#pragma once

#include <math.h>

#include "fe_device.h"
#include "fe_kernels.h"
#include "norm_rope_row.h"

namespace fe {
namespace dec {

constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr float kEmptyMax = -1.0e30f;   // running max before the first valid token
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kWaitVmcnt0 = 0x0F70;     // s_waitcnt vmcnt(0) (expcnt, lgkmcnt unconstrained)
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
  int* arrivals;          // fused merge: [B][Hkv] partitions finished so far (zero between calls)
  const int32_t* q_rows;  // row of sequence b in q / out / lse (nullptr: row b)
  int q_rows_count;       // rows of q / out / lse when q_rows is used (rows are clamped into it)
  // Fused append (nullptr k_new: none): sequence b's new K/V rows
  // k_new/v_new [B][Hkv][D] go to cache slot new_slots[b], the slot of its
  // position L_b - 1, written by the workgroup that holds that block.
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* new_slots;
  uint16_t* k_cache_w;  // the pools again, writable (fused append only)
  uint16_t* v_cache_w;
  int64_t num_slots;
  // Fused per-head RMSNorm + rotary of q and of the appended k (the
  // kNormRope instance of decode_item; only with a fused append): weights
  // [D] bf16, table [max_pos][D] fp32 at row positions[b], clamped into
  // [0, max_pos)
  const uint16_t* q_norm_w;
  const uint16_t* k_norm_w;
  const float* cos_sin;
  const int32_t* positions;
  int max_pos;
  float eps;
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
  // p = 2^(s * scale_log2 - m)
  // PV in fp32: acc += p * v, v widened from bf16 (exact), one fma per
  // (token, dim, head); the same p enters l and the numerator.
  float pf[4][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pf[j][h] = fast_exp2(fmaf(s[j][h], scale_log2, -st.m[h]));
    st.l[h] += (pf[0][h] + pf[1][h]) + (pf[2][h] + pf[3][h]);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t vw[4];
    words4(t.v[j], vw);  // dims 8c .. 8c + 7 of token 4 j + r
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ve = __uint_as_float(vw[i] << 16);
      const float vo = __uint_as_float(vw[i] & 0xffff0000u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        st.acc[h][2 * i] = fmaf(pf[j][h], ve, st.acc[h][2 * i]);
        st.acc[h][2 * i + 1] = fmaf(pf[j][h], vo, st.acc[h][2 * i + 1]);
      }
    }
  }
}

template <int G, int W>
struct DecodeShared {
  float o[W][G][kHeadDim];
  float m[W][G];
  float l[W][G];
  int last;  // fused merge: this workgroup combines the partitions of its (sequence, KV head)
};

// One work item: (sequence b, KV head g, partition part), run by W waves.
// Without kFused, a split sequence's partitions leave fp32 partials for a
// separate merge pass.  With kFused, each partition counts its arrival and
// the last one of the (sequence, KV head) to arrive merges them in place.
template <int G, int W, bool kFused, bool kNormRope = false>
__device__ __forceinline__ void decode_item(const DecodeParams& p, DecodeShared<G, W>& sh, int b, int g, int part) {
  constexpr int kThreads = 64 * W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int r = lane >> 4, c = lane & 15;

  const int blk0 = part * p.part_blocks;

  // Issued together, before the context length is known: the length, this
  // wave's block ids (lane k <- local block wave + W k, i.e. the wave's tile
  // k; a partition has at most 64 W blocks) and q.
  const int Lraw = p.context_lens[b];
  const int row_blocks = min(p.part_blocks, p.max_blocks - blk0);  // table entries this partition may use
  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks + blk0;
  int ids = wave + W * lane < row_blocks ? bt[wave + W * lane] : 0;
  const size_t row0 = static_cast<size_t>(b) * p.Hq + static_cast<size_t>(g) * G;  // partial rows of the group
  const int qrow = p.q_rows ? min(max(p.q_rows[b], 0), p.q_rows_count - 1) : b;
  const size_t qrow0 = static_cast<size_t>(qrow) * p.Hq + static_cast<size_t>(g) * G;
  uint32_t qw[G][4];
  // fused norm/rotary: the position arrives with q; the table row and the
  // weights are loaded once the tile loads can be issued, and q is
  // normalised and rotated after them, so neither adds a round trip
  int nr_pos = 0;
  if constexpr (kNormRope) nr_pos = p.positions[b];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + qrow0 * kHeadDim) + c;
#pragma unroll
    for (int h = 0; h < G; ++h) words4(qp[h * (kHeadDim / 8)], qw[h]);
    if (p.negate_q && !kNormRope) {  // scale < 0: flip q's signs (exact) and use |scale|
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) qw[h][i] ^= 0x80008000u;
    }
  }
  ids = min(max(ids, 0), p.num_blocks - 1);

  const int L = clamp_len(Lraw, p.ctx_cap);
  const int nblk = (L + kBlockSize - 1) / kBlockSize;
  const int np = (nblk + p.part_blocks - 1) / p.part_blocks;  // partitions this sequence has
  if (blk0 >= nblk && p.P > 1) {  // nothing here; the merge never reads this partition
    if (kFused && part == 0) {  // empty context: out 0, lse -inf
      for (int o = tid; o < G * kHeadDim; o += kThreads) {
        const size_t row = qrow0 + o / kHeadDim;
        p.out[row * kHeadDim + o % kHeadDim] = 0;
        if (o % kHeadDim == 0 && p.lse) p.lse[row] = -INFINITY;
      }
    }
    return;
  }
  const int blk1 = min(nblk, blk0 + p.part_blocks);
  const int nb = max(0, blk1 - blk0);
  // tokens in the sequence's last block; that block is masked if partial
  const int rem = L - (nblk - 1) * kBlockSize;
  // With a fused append the sequence's last block always takes the tail path
  // below (full or not), which writes the new row and patches it in.
  const bool fuse = p.k_new != nullptr && nb > 0 && blk1 == nblk;
  const bool has_tail = nb > 0 && blk1 == nblk && (rem < kBlockSize || fuse);
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

  // This wave's full tiles are local blocks wave, wave + W, ... (n of them).
  // A ring of kPrefetch + 1 register tiles keeps kPrefetch tiles in flight
  // while one is consumed.  Every load is issued unconditionally (tiles past
  // n are masked by their buffer range), so the compiler's vmcnt bookkeeping
  // sees one straight-line schedule and waits only for the oldest tile.
  const int n = nfull > wave ? (nfull - wave + W - 1) / W : 0;
  auto issue = [&](Tile& dst, int t) {
    const bool ok = t < n;
    const size_t o = ok ? static_cast<size_t>(__builtin_amdgcn_readlane(ids, t)) * blk_stride : 0;
    const int bytes = ok ? kTileElems * 2 : 0;
    load_tile(dst, tile_rsrc(kg + o, bytes), tile_rsrc(vg + o, bytes), lane);
  };
  RopeLane q_cs;
  uint4 q_ww;
  if constexpr (kNormRope) {
    q_cs = rope_lane(p.cos_sin, min(max(nr_pos, 0), p.max_pos - 1), c);
    q_ww = reinterpret_cast<const uint4*>(p.q_norm_w)[c];
  }
  Tile ring[kPrefetch + 1];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) issue(ring[k], k);
  if constexpr (kNormRope) {  // per-head RMSNorm + rotary of q, as the fused norm/rotary/append call computes it
#pragma unroll
    for (int h = 0; h < G; ++h) {
      words4(norm_rope_row(make_uint4(qw[h][0], qw[h][1], qw[h][2], qw[h][3]), q_ww, q_cs, p.eps, c), qw[h]);
      if (p.negate_q)
#pragma unroll
        for (int i = 0; i < 4; ++i) qw[h][i] ^= 0x80008000u;
    }
  }
  for (int t = 0; t < n; t += kPrefetch + 1) {
#pragma unroll
    for (int k = 0; k <= kPrefetch; ++k) {
      issue(ring[(k + kPrefetch) % (kPrefetch + 1)], t + k + kPrefetch);
      if (t + k < n) consume<G, false>(st, ring[k], qw, p.scale_log2, r, kBlockSize);
    }
  }
  if (has_tail && wave == (nb - 1) % W) {
    const int id = __builtin_amdgcn_readlane(ids, (nb - 1) / W);
    const size_t o = static_cast<size_t>(id) * blk_stride;
    const int bytes = rem * kHeadDim * 2;
    load_tile(ring[0], tile_rsrc(kg + o, bytes), tile_rsrc(vg + o, bytes), lane);
    if (fuse) {
      // The new token: row rem - 1 of this block.  Write it into its slot (as
      // fe_paged_kv_append does: skipped unless 0 <= slot < num_slots) and,
      // when the slot is that row's, take its K/V from registers: the tile
      // load above may or may not have seen the store.
      const int64_t slot = p.new_slots[b];
      const size_t nrow = (static_cast<size_t>(b) * p.Hkv + g) * kHeadDim;
      uint4 kn = reinterpret_cast<const uint4*>(p.k_new + nrow)[c];
      const uint4 vn = reinterpret_cast<const uint4*>(p.v_new + nrow)[c];
      if constexpr (kNormRope)  // the new k row normalised and rotated first (all 64 lanes: wave-uniform branch)
        kn = norm_rope_row(kn, reinterpret_cast<const uint4*>(p.k_norm_w)[c],
                           rope_lane(p.cos_sin, min(max(p.positions[b], 0), p.max_pos - 1), c), p.eps, c);
      if (slot >= 0 && slot < p.num_slots) {
        if (r == 0) {
          const size_t dst = ((static_cast<size_t>(slot / kBlockSize) * p.Hkv + g) * kBlockSize + slot % kBlockSize) *
                             kHeadDim;
          reinterpret_cast<uint4*>(p.k_cache_w + dst)[c] = kn;
          reinterpret_cast<uint4*>(p.v_cache_w + dst)[c] = vn;
        }
        const int row = rem - 1;
        if (slot == static_cast<int64_t>(id) * kBlockSize + row && r == (row & 3)) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j == (row >> 2)) {
              ring[0].k[j] = kn;
              ring[0].v[j] = vn;
            }
        }
      }
    }
    consume<G, true>(st, ring[0], qw, p.scale_log2, r, rem);
  }

  // merge the 4 rows of this wave: lanes c, c+16, c+32, c+48 hold the same
  // dims (permlane swaps on the VALU, not LDS permutes)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = xor_max<32>(xor_max<16>(st.m[h]));
    const float f = fast_exp2(st.m[h] - M);
    st.l[h] = xor_sum<32>(xor_sum<16>(st.l[h] * f));
#pragma unroll
    for (int k = 0; k < 8; ++k) st.acc[h][k] = xor_sum<32>(xor_sum<16>(st.acc[h][k] * f));
    st.m[h] = M;
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

  // merge the W waves and write
  const bool split = kFused ? np > 1 : p.P > 1;
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    float M = sh.m[0][h];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sh.m[w][h]);
    float lsum = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float f = fast_exp2(sh.m[w][h] - M);
      lsum = fmaf(sh.l[w][h], f, lsum);
      val = fmaf(sh.o[w][h][d], f, val);
    }
    const bool empty = !(lsum > 0.f);
    const float res = empty ? 0.f : val / lsum;
    const float lse_nat = empty ? -INFINITY : (M + log2f(lsum)) * kLn2;
    const size_t row = row0 + h;
    if (!split) {
      const size_t orow = qrow0 + h;
      p.out[orow * kHeadDim + d] = to_bf16(res);
      if (d == 0 && p.lse) p.lse[orow] = lse_nat;
    } else if (kFused) {
      // device-scope stores: coherent across the XCDs' L2s once complete
      __hip_atomic_store(&p.o_part[(row * p.P + part) * kHeadDim + d], res, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      if (d == 0) __hip_atomic_store(&p.lse_part[row * p.P + part], lse_nat, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      p.o_part[(row * p.P + part) * kHeadDim + d] = res;
      if (d == 0) p.lse_part[row * p.P + part] = lse_nat;
    }
  }
  if (!kFused || !split) return;

  // Fused split-K merge: the last of the sequence's np partitions to arrive
  // combines all of them by log-sum-exp.  The partials travel through
  // agent-scope atomic stores and loads (sc1 on gfx950: performed at the
  // device's coherence point, past the XCDs' non-coherent L2s), so the
  // release / acquire that orders them needs no L2 write-back or invalidate
  // (those exist for non-atomic data): every wave waits until its partial
  // stores are acknowledged (s_waitcnt vmcnt(0)) before the barrier, the
  // arrival count is taken after it, and the last arriver reads the partials
  // only after the count has returned.  An acq_rel counter adds exactly the
  // L2 write-back / invalidate pair, which costs the mixed launch ~27%.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid == 0) {
    int* cnt = p.arrivals + static_cast<size_t>(b) * p.Hkv + g;
    const int before = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = before == np - 1;
    // every partition has arrived: the counter is ready for the next call
    if (sh.last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!sh.last) return;
  for (int o = tid; o < G * kHeadDim; o += kThreads) {
    const int h = o / kHeadDim, d = o % kHeadDim;
    const size_t row = row0 + h;
    float* lp = p.lse_part + row * p.P;
    float* op = p.o_part + row * p.P * kHeadDim + d;
    float M = -INFINITY;
    for (int i = 0; i < np; ++i) M = fmaxf(M, __hip_atomic_load(&lp[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    float z = 0.f, a = 0.f;
    for (int i = 0; i < np; ++i) {
      const float w =
          fast_exp2((__hip_atomic_load(&lp[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - M) * kLog2e);
      z += w;
      a = fmaf(w, __hip_atomic_load(&op[static_cast<size_t>(i) * kHeadDim], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
               a);
    }
    const bool empty = !(z > 0.f);
    const size_t orow = qrow0 + h;
    p.out[orow * kHeadDim + d] = to_bf16(empty ? 0.f : a / z);
    if (d == 0 && p.lse) p.lse[orow] = empty ? -INFINITY : M + logf(z);
  }
}

// Kernel parameters of a decode launch (host side); split-K buffers and the
// per-sequence q rows are left for the caller.
inline DecodeParams make_decode_params(const void* q, const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, int max_blocks_per_seq,
                                       const int32_t* context_lens, void* out, float* lse, int B, int Hq, int Hkv,
                                       int num_blocks, int max_context_len, float scale, int P, int part_blocks) {
  DecodeParams prm{};
  prm.q = static_cast<const uint16_t*>(q);
  prm.k_cache = static_cast<const uint16_t*>(k_cache);
  prm.v_cache = static_cast<const uint16_t*>(v_cache);
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.out = static_cast<uint16_t*>(out);
  prm.lse = lse;
  prm.max_blocks = max_blocks_per_seq;
  prm.B = B;
  prm.Hq = Hq;
  prm.Hkv = Hkv;
  prm.num_blocks = num_blocks;
  const long cap_bt = static_cast<long>(max_blocks_per_seq) * kBlockSize;
  prm.ctx_cap = static_cast<int>(max_context_len < cap_bt ? max_context_len : cap_bt);
  prm.P = P;
  prm.part_blocks = part_blocks;
  prm.scale_log2 = fabsf(scale) * kLog2e;
  prm.negate_q = scale < 0.f;
  return prm;
}

}  // namespace dec
}  // namespace fe
