// Chunked-prefill query tile over the paged cache on the bf16 MFMA units,
// shared by the prefill kernel and the mixed decode/prefill kernel
// (ForgeEngine README, "What it implements": restricted prefill lab, and
// "Scheduling": token-budgeted batching that cuts prompts into chunks; "Make
// the Engine Talk" section 1.2: the prefill pass that primes the cache).
//
// A chunk of C queries sits at the end of its sequence: query i is at
// position L - C + i and attends to keys 0 .. L - C + i.
//
// One workgroup per (sequence, KV head, tile of QT query rows).  W waves
// each own 32 (query row, query head) pairs of the group -- one head per wave
// when G >= 4 -- so every K/V tile staged in LDS is shared by all G heads.
// When W <= 4 the workgroup has KS = 2 such wave groups that split the key
// range in two halves (two waves per SIMD instead of one) and merge their
// (max, sum, O) by log-sum-exp through LDS at the end.
// Per 64-key tile each wave computes
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, A = K rows from LDS,
//                      B = Q^T held in registers (32 queries x 128 dims)
//   online softmax     the D layout puts query (lane % 32) in every lane, so
//                      the row max/sum are lane-local plus one permlane32 swap
//   O^T += V^T P^T     B = P^T packed to bf16 straight from the S^T registers;
//                      A = V^T read from the row-major V tile with
//                      ds_read_b64_tr_b16 (two 4-key transposed reads).
// The MFMA sums over keys in any order as long as A and B agree, so the
// k-slot -> key order of each PV step is chosen to match the keys the S^T
// accumulator layout leaves in each lane (no data movement for P).
// K and V tiles go from global memory straight into LDS (buffer loads with
// the LDS bit, no registers on the way), in 256-byte rows whose 16-byte
// chunks are XOR-swizzled so that the K row reads of 16 consecutive keys and
// the transposed V reads are free of bank conflicts on the 64 banks; every
// LDS offset is a per-lane base plus a constant.
//
// Schedule.  A tile's work is split into two phases separated by workgroup
// barriers: an MFMA phase (S^T of tile i, then O^T += V^T P^T of tile i - 1),
// run at the highest wave priority, and a VALU/memory phase (the copies of V
// of tile i + 1 and K of tile i + 2 into the buffers the MFMA phase just
// finished reading, then the softmax of tile i into P).  Each group has two
// K and two V buffers in LDS.  With two groups the second runs one phase
// behind the first, so on every SIMD one wave's MFMAs overlap the other
// wave's softmax instead of both waves contending for the same unit at the
// same time.
#pragma once

#include <math.h>

#include <type_traits>

#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {
namespace pre {

constexpr int kKeysPerTile = 64;
constexpr int kRowBytes = kHeadDim * 2;                 // 256 bytes of one K/V row
constexpr int kTileBytes = kKeysPerTile * kRowBytes;    // one K or V tile in LDS: 16 KiB, rows unpadded
constexpr int kGroupBytes = 4 * kTileBytes;             // a key group's two K and two V tiles
constexpr float kRescaleSlack = 8.0f;
constexpr float kLazyLimit = 65536.0f;  // a lane's tile sum that makes the softmax look for a new max
constexpr float kEmptyMax = -1.0e30f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct PrefillParams {
  const uint16_t* q;
  const int32_t* query_start_loc;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  uint16_t* out;
  float* lse;
  int max_blocks, B, total_q, max_q_len, Hq, Hkv, num_blocks, ctx_cap, qtiles;
  float scale_log2;  // |scale| * log2(e)
  int negate_q;      // scale < 0: q's signs are flipped on load (exact)
};

// KSel = 0 takes the default number of key groups (two when a group has at
// most 4 waves); KSel = 1 forces one group, half the LDS of two; KSel = 2
// forces two.  KSel = 3 (kPair) also has two groups, but they take two
// consecutive query tiles over one shared stream of K/V tiles instead of
// splitting the keys (for grids with more tiles than CUs).
template <int G, int KSel = 0>
struct Shape {
  static constexpr int W = (G <= 4 && 4 % G == 0) ? 4 : G;  // waves per group
  static constexpr bool kPair = KSel == 3;
  static constexpr int KS = kPair ? 2 : (KSel != 0 ? KSel : (W <= 4 ? 2 : 1));  // wave groups
  static constexpr int QT = 32 * W / G;                     // query rows per group
  static constexpr int kThreads = 64 * W * KS;
  // a 64-key tile is 4 KV blocks; wave w of a group stages blocks w, w + W, ...
  static constexpr int kStageBlocks = (4 + W - 1) / W;
  // K and V buffers: two per group, or three shared ones (kPair: a tile is
  // read by both groups, one phase apart, so a buffer frees one phase later)
  static constexpr int kBufs = kPair ? 3 : 2;
  static constexpr int kLdsBytes = kPair ? 2 * kBufs * kTileBytes : KS * kGroupBytes;
  // tiles ahead of the current one whose V and K copies a step issues
  static constexpr int kLeadV = kPair ? 2 : 1;
  static constexpr int kLeadK = kPair ? 3 : 2;
  static_assert(!kPair || W == 4, "paired query tiles are built for groups of 4 waves");
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// One 4 KiB (block, KV head) tile straight from global memory into LDS:
// four buffer loads with the LDS bit, each writing 64 lanes x 16 bytes
// contiguously at LDS byte address m0 + 1024 j (the instruction offset moves
// the global address by the same 1024 j).  Lane i's voffset v_j picks which
// 16 bytes of its 256-byte row it fetches, which is how the LDS rows get
// their XOR swizzle.  Bytes at or past `bytes` read as zeros without a memory
// access.  Written as asm because the compiler's builtin makes every later
// LDS read wait for all such loads in flight; the caller waits for them with
// s_waitcnt vmcnt (the loads count there, completing in issue order).  M0 is
// saved and restored around the loads, with the wait state that an M0 write
// before an LDS-direct load needs.
__device__ __forceinline__ void lds_direct_tile(const uint16_t* base, int bytes, uint32_t m0, uint32_t v0,
                                                uint32_t v1, uint32_t v2, uint32_t v3) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), static_cast<short>(0), bytes, 0x00020000);
  uint32_t save;
  asm volatile(
      "s_mov_b32 %[save], m0\n\t"
      "s_mov_b32 m0, %[m0]\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %[v0], %[r], 0 offen offset:0 lds\n\t"
      "buffer_load_dwordx4 %[v1], %[r], 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %[v2], %[r], 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %[v3], %[r], 0 offen offset:3072 lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %[save]"
      : [save] "=&s"(save)
      : [m0] "s"(m0), [r] "s"(r), [v0] "v"(v0), [v1] "v"(v1), [v2] "v"(v2), [v3] "v"(v3)
      : "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Query tile qt of sequence b against KV head g, run by the whole workgroup
// (Shape<G, KSel>::kThreads threads); lds holds Shape<G, KSel>::kLdsBytes bytes.
// kSplitP: the softmax weights enter the PV product as two bf16 parts, the
// rounded weight and the rounded remainder, so the product sees each weight
// to within 2^-16 instead of 2^-8 (half again the MFMA work of a step).
template <int G, int KSel = 0, bool kSplitP = false>
__device__ __forceinline__ void prefill_tile(const PrefillParams& p, unsigned char* lds, int qt, int b, int g) {
  using S = Shape<G, KSel>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = uniform(tid >> 6);
  const int grp = wave_all / S::W;  // which half of the key range (kPair: which query tile)
  const int wave = wave_all % S::W;
  const int col = lane & 31;   // this lane's query within the wave's 32
  const int half = lane >> 5;  // which 8-dim / 4-key half of an MFMA operand

  const int q0 = p.query_start_loc[b];
  int C = p.query_start_loc[b + 1] - q0;
  C = C < 0 ? 0 : (C > p.max_q_len ? p.max_q_len : C);
  // first query of the workgroup and of this group (kPair: tiles 2 qt and 2 qt + 1)
  const int wg_i0 = (S::kPair ? 2 * qt : qt) * S::QT;
  const int i0 = wg_i0 + (S::kPair ? grp * S::QT : 0);
  if (wg_i0 >= C) return;  // (kPair: a second tile past the chunk still stages the first one's K/V)
  int L = p.context_lens[b];
  L = L < 0 ? 0 : (L > p.ctx_cap ? p.ctx_cap : L);

  // this wave's (head, query) rows: head h_loc, queries i0 + qoff .. + 31
  const int h_loc = (wave * 32) / S::QT;
  const int qoff = (wave * 32) % S::QT;
  const int qi = i0 + qoff + col;              // this lane's query index in the chunk
  const bool q_valid = qi < C && q0 + qi < p.total_q;
  const int pos = L - C + qi;                  // its position; keys 0..pos are visible
  const int head = g * G + h_loc;

  // Q^T operand: k-step kk covers dims 16 kk .. 16 kk + 15; this lane holds 8.
  bf16x8_t qb[8];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(p.q + (static_cast<size_t>(q0 + qi) * p.Hq + head) * kHeadDim);
    const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      uint4 w = q_valid ? qp[2 * kk + half] : make_uint4(0, 0, 0, 0);
      w.x ^= flip;
      w.y ^= flip;
      w.z ^= flip;
      w.w ^= flip;
      qb[kk] = as_bf16x8(w);
    }
  }

  // keys this workgroup needs: 0 .. last visible position of its last query
  const int last_q = min(wg_i0 + (S::kPair ? 2 : 1) * S::QT, C) - 1;
  const int kv_end = max(0, min(L, L - C + last_q + 1));
  const int n_tiles = (kv_end + kKeysPerTile - 1) / kKeysPerTile;
  const int diag_from = max(0, L - C + i0 + 1);  // keys beyond this need the causal mask for some row
  const int n_plain = min(n_tiles, diag_from / kKeysPerTile);  // tiles needing no mask
  // group 0 takes tiles [0, nA), group 1 tiles [nA, n_tiles) (kPair: both take all)
  const int nA = S::KS == 2 && !S::kPair ? (n_tiles + 1) / 2 : n_tiles;
  const int t_first = S::kPair ? 0 : grp * nA;
  const int t_end = grp == 0 || S::kPair ? nA : n_tiles;

  const int32_t* bt = p.block_tables + static_cast<size_t>(b) * p.max_blocks;
  const size_t blk_stride = static_cast<size_t>(p.Hkv) * kTileElems;
  const uint16_t* kg = p.k_cache + static_cast<size_t>(g) * kTileElems;
  const uint16_t* vg = p.v_cache + static_cast<size_t>(g) * kTileElems;
  // this group's K tiles, then its V tiles (kPair: the shared ones)
  const int grp_base = S::kPair ? 0 : grp * kGroupBytes;
  const int n_g = t_end - t_first;         // this group's tiles

  // Staging: wave w copies blocks w, w + W, ... of each 64-key tile, each a
  // contiguous 4 KiB (block, KV head) run, straight into LDS (no registers).
  // Rows past the context come back as zeros from the buffer range (never
  // NaN, so masked keys stay inert in the PV product).  LDS rows are 256
  // bytes, unpadded; their 16-byte chunks are XOR-swizzled so that both read
  // patterns below are free of bank conflicts on the 64 banks:
  //   K row r holds logical chunk c at chunk c ^ (r & 15)  (16 rows read at
  //     one chunk hit 16 different chunks),
  //   V row r holds logical chunk c at chunk c ^ 4 (r & 3)  (the transposed
  //     reads of 4 rows x 64 bytes hit 4 different 64-byte groups).
  const int nblk_seq = (L + kBlockSize - 1) / kBlockSize;
  // Block ids of the blocks this wave stages, held in VGPRs so a fetch needs
  // no dependent scalar load: lane j of ids[i] holds the (clamped) id of
  // block wave + i W of local tile 64 chunk + j, or 0 past the context.
  int ids[S::kStageBlocks];
  int ids_chunk = -1;
  auto load_ids = [&](int chunk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::kStageBlocks; ++i) {
      const int bl = wave + i * S::W;
      const int lt = 64 * chunk + lane;
      const int gb = 4 * (t_first + lt) + bl;
      int v = 0;
      if (bl < 4 && lt < n_g && gb < nblk_seq) v = min(max(bt[gb], 0), p.num_blocks - 1);
      ids[i] = v;
    }
    ids_chunk = chunk;
  };
  // blocks this wave stages per tile, and the LDS-direct loads that makes
  // (kPair: the second group stages the shared tiles, the first stages none)
  const bool stager = !S::kPair || grp == 1;
  int n_stage = 0;
#pragma unroll
  for (int i = 0; i < S::kStageBlocks; ++i) n_stage += stager && wave + i * S::W < 4 ? 1 : 0;
  // Global byte offsets of this lane's 16 bytes within the j-th 1 KiB run
  // (rows 4 j .. 4 j + 3 of a block; the 1024 j itself is the instruction
  // offset), for the swizzles above: a block's rows are rows 16 bl + r of
  // the tile, and 16 bl changes neither r & 15 nor r & 3.
  uint32_t kvo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) kvo[j] = (lane >> 4) * kRowBytes + (((lane & 15) ^ ((4 * j + (lane >> 4)) & 15)) << 4);
  const uint32_t vvo = (lane >> 4) * kRowBytes + (((lane & 15) ^ (4 * (lane >> 4))) << 4);
  const uint32_t lds_addr = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds)) + grp_base;
  // where tile t's blocks come from (offset into the pools, valid bytes);
  // the V copy of a tile runs one phase after its K copy and reuses these
  size_t src_off[S::kStageBlocks];
  int src_bytes[S::kStageBlocks];
  auto locate = [&](int t) __attribute__((always_inline)) {
    const int lt = t - t_first;
    if (lt < n_g && (lt >> 6) != ids_chunk) {
      load_ids(lt >> 6);
      wait_vm<0>();
    }
#pragma unroll
    for (int i = 0; i < S::kStageBlocks; ++i) {
      const int bl = wave + i * S::W;
      const int gb = 4 * t + bl;  // block index within the sequence
      const bool ok = lt < n_g && gb < nblk_seq;
      src_off[i] = static_cast<size_t>(__builtin_amdgcn_readlane(ids[i], lt & 63)) * blk_stride;
      src_bytes[i] = ok ? min(kBlockSize, L - gb * kBlockSize) * kRowBytes : 0;
    }
  };
  // K of tile t into K buffer kb, from the locations just looked up
  auto stage_k = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::kStageBlocks; ++i) {
      const int bl = wave + i * S::W;
      if (bl < 4)
        lds_direct_tile(kg + src_off[i], src_bytes[i], lds_addr + kb * kTileBytes + bl * 4096, kvo[0], kvo[1],
                        kvo[2], kvo[3]);
    }
  };
  // V of the tile located by the previous locate() into V buffer vb
  auto stage_v = [&](int vb, const size_t (&off)[S::kStageBlocks], const int (&bytes)[S::kStageBlocks])
      __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < S::kStageBlocks; ++i) {
      const int bl = wave + i * S::W;
      if (bl < 4)
        lds_direct_tile(vg + off[i], bytes[i], lds_addr + (S::kBufs + vb) * kTileBytes + bl * 4096, vvo, vvo, vvo,
                        vvo);
    }
  };
  // every copy this wave issued before its latest 2 n_stage tiles has landed
  auto wait_previous = [&]() __attribute__((always_inline)) {
    if (n_stage == 1) wait_vm<8>();
    else if (n_stage == 2) wait_vm<16>();
  };

  // per-lane LDS read addresses (the buffer, key block and tau parts are
  // compile-time offsets)
  // K rows for S^T: key 32 blk + col, logical chunk 2 kk + half
  int kra[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kra[kk] = grp_base + col * kRowBytes + (((2 * kk + half) ^ (col & 15)) << 4);
  // transposed V reads: k-slots of step (blk, tau) are keys 32 blk + 16 tau +
  // {0-3, 8-11, 4-7, 12-15}; 16-lane group gq holds slots 8 (gq / 2) .. + 7 of
  // dims 16 (gq % 2) .. + 15 of each 32-dim block d; source lane src points at
  // row key0 + src / 4 (so row & 3 = src / 4), dims + 4 (src % 4): logical
  // chunk 2 (gq % 2) + (src % 4) / 2 + 4 d, byte 8 (src % 2) within it
  const int gq = lane >> 4, src = lane & 15;
  int vra[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
    vra[d] = grp_base + S::kBufs * kTileBytes + (4 * (gq >> 1) + (src >> 2)) * kRowBytes +
             ((2 * (gq & 1) + ((src & 3) >> 1) + 4 * (d ^ (src >> 2))) << 4) + 8 * (src & 1);

  f32x16_t o_acc[4];  // O^T, dim block d: lane holds query col, dims 32 d + 8 (i / 4) + 4 half + i % 4
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o_acc[d][i] = 0.f;
  float m = kEmptyMax, lsum = 0.f;
  const float sc = p.scale_log2;  // > 0

  f32x16_t s[2];      // S^T of the current tile: keys 32 blk + 8 (i / 4) + 4 half + i % 4, query col
  bf16x8_t pb[2][2];  // P^T of the previous tile, k-step (blk, tau): S^T entries 8 tau .. 8 tau + 7
  bf16x8_t pl[2][2];  // kSplitP: the remainders P^T - pb, rounded to bf16

  // S^T = K Q^T for the tile in LDS buffer `buf`
  auto qk = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    f32x16_t acc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) acc[blk][i2] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const uint4 kv = *reinterpret_cast<const uint4*>(&lds[kra[kk] + buf * kTileBytes + blk * 32 * kRowBytes]);
        acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kv), qb[kk], acc[blk], 0, 0, 0);
      }
    s[0] = acc[0];
    s[1] = acc[1];
  };

  // O^T += V^T P^T for the tile in LDS buffer `buf`
  auto pv = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    bf16x8_t va[4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int o = vra[d] + buf * kTileBytes + (32 * blk + 16 * tau) * kRowBytes;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(&lds[o]));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(&lds[o + 8 * kRowBytes]));
          // move whole dwords: element-wise 16-bit extraction here is lowered
          // into half-word shuffles that drop the upper dword of each read
          const uint2 l2 = __builtin_bit_cast(uint2, lo);
          const uint2 h2 = __builtin_bit_cast(uint2, hi);
          va[d] = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
          o_acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[d], pb[blk][tau], o_acc[d], 0, 0, 0);
        }
        if constexpr (kSplitP) {
          // the remainders, each accumulator four MFMAs after its last use
#pragma unroll
          for (int d = 0; d < 4; ++d)
            o_acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[d], pl[blk][tau], o_acc[d], 0, 0, 0);
        }
      }
  };

  // causal mask and P = 2^(S sc - m) for absolute tile t.  The running max
  // m is raised lazily: the weights are first taken against the current m;
  // only when some lane's sum over the tile leaves [0, kLazyLimit] (the first
  // tile, with m still at kEmptyMax, always does) is the tile's true max
  // taken, m raised where it grew by more than kRescaleSlack, and the weights
  // taken again.  Between raises a weight can reach about kLazyLimit, far
  // inside fp32 and bf16 range; the max search costs nothing on the tiles
  // that do not raise it.
  auto softmax = [&](int t) __attribute__((always_inline)) {
    if (t >= n_plain) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) {
          const int key = t * kKeysPerTile + 32 * blk + 8 * (i2 / 4) + 4 * half + (i2 % 4);
          if (key > pos || !q_valid) s[blk][i2] = -INFINITY;
        }
    }
    auto weights = [&]() __attribute__((always_inline)) {
      float part[4];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          float e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) e[j] = fast_exp2(fmaf(s[blk][8 * tau + j], sc, -m));
          // pairwise sums: short dependency chains in the critical VALU phase
          part[2 * blk + tau] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
          uint4 w;
          w.x = pack_bf16x2(e[0], e[1]);
          w.y = pack_bf16x2(e[2], e[3]);
          w.z = pack_bf16x2(e[4], e[5]);
          w.w = pack_bf16x2(e[6], e[7]);
          pb[blk][tau] = as_bf16x8(w);
          if constexpr (kSplitP) {
            // e - bf16(e) is exact in fp32; its own rounding leaves at most 2^-16 of e
            uint4 r;
            r.x = pack_bf16x2(e[0] - bf16_lo(w.x), e[1] - bf16_hi(w.x));
            r.y = pack_bf16x2(e[2] - bf16_lo(w.y), e[3] - bf16_hi(w.y));
            r.z = pack_bf16x2(e[4] - bf16_lo(w.z), e[5] - bf16_hi(w.z));
            r.w = pack_bf16x2(e[6] - bf16_lo(w.w), e[7] - bf16_hi(w.w));
            pl[blk][tau] = as_bf16x8(r);
          }
        }
      return (part[0] + part[1]) + (part[2] + part[3]);
    };
    float ts = weights();
    if (__any(!(ts <= kLazyLimit))) {  // also true for inf / NaN
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) mx = fmaxf(mx, s[blk][i2]);
      mx *= sc;
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      if (mx > m + kRescaleSlack) {
        const float a = fast_exp2(m - mx);
        m = mx;
        lsum *= a;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
          for (int i2 = 0; i2 < 16; ++i2) o_acc[d][i2] *= a;
      }
      ts = weights();
    }
    lsum += ts;
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  // MFMA phase of local tile i (K buffer bufc = i mod kBufs): S^T of tile i
  // and, when pvc, O^T += V^T P^T of tile i - 1 (the V buffer before bufc,
  // cyclically).  One basic block; the
  // scheduling groups keep four MFMA operands in flight from LDS so the read
  // latency hides behind the MFMAs (16 K reads of 16 bytes for S^T, then two
  // 8-byte transposed V reads per PV MFMA, or per pair of them with kSplitP).
  auto mphase = [&](auto bufc, auto pvc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    using Other = std::integral_constant<int, (buf + S::kBufs - 1) % S::kBufs>;
    qk(bufc);
    if constexpr (decltype(pvc)::value) {
      pv(Other{});
      constexpr int kPvPer = kSplitP ? 2 : 1;  // MFMAs per pair of transposed V reads
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int j = 0; j < 12; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, kPvPer, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // One local tile i (K buffer i % 2 == bufc, V buffer of tile i - 1 the
  // other): MFMA phase, barrier, then the VALU/memory phase: V of tile i + 1
  // into the V buffer the MFMA phase just finished reading (tile i - 1's),
  // K of tile i + 2 into the K buffer it just finished reading (tile i's),
  // the softmax of tile i, and a wait for the previous phase's copies (K of
  // tile i + 1, V of tile i), which the next MFMA phase reads after the
  // barrier.  A copy thus has a phase and a half to land.  The O rescale in
  // the softmax sees O with tile i - 1 already accumulated, as the online
  // softmax requires.
  // kPair: the three shared buffers of each kind hold tiles i mod 3.  Group 0
  // reads a tile one phase before group 1, so a buffer frees after group 1's
  // MFMA phase; group 1 (the stager) then copies V of tile i + 2 and K of
  // tile i + 3 in its VALU phase of tile i, into the buffers of tiles i - 1
  // and i, and waits for the copies of the step before, two phases ahead of
  // group 0's first read of them.
  size_t v_off[S::kStageBlocks];
  int v_bytes[S::kStageBlocks];
  auto step = [&](auto bufc, auto pvc, int i) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    // the MFMA phase runs at the highest wave priority: on each SIMD its
    // MFMAs and operand reads then go first, and the other group's softmax
    // fills the issue cycles between them (the second-created wave of a SIMD
    // otherwise lost the arbitration in both phases)
    __builtin_amdgcn_s_setprio(3);
    mphase(bufc, pvc);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    if (stager) {
      stage_v((buf + S::kLeadV) % S::kBufs, v_off, v_bytes);  // tile i + kLeadV (located with its K copy)
      locate(t_first + i + S::kLeadK);
#pragma unroll
      for (int k = 0; k < S::kStageBlocks; ++k) {
        v_off[k] = src_off[k];
        v_bytes[k] = src_bytes[k];
      }
      stage_k(buf);  // tile i + kLeadK, into the buffer of tile i
    }
    softmax(t_first + i);
    wait_previous();
    __syncthreads();
  };

  // Prologue.  Q and the block ids of the first 64 tiles arrive in one
  // memory round trip, settled on every path here so that no later barrier
  // waits on memory.  Each key group then copies K of its tiles 0 and 1 and V
  // of tile 0 and waits for K of tile 0 before the barriers, so the two
  // groups' first round trips overlap (kPair: the stager copies K of tiles
  // 0 - 2 and V of tiles 0 - 1 and waits for all of them).  Group 1 then
  // takes one extra barrier, which puts it one phase behind group 0.  Copies
  // of tiles past a group's range read nothing and write zeros into a buffer
  // nobody reads.
  if (stager) {
    load_ids(0);
    wait_vm<0>();
#pragma unroll
    for (int t = 0; t < S::kLeadK; ++t) {
      locate(t_first + t);
      stage_k(t);
      if (t < S::kLeadV) stage_v(t, src_off, src_bytes);
      if (t == S::kLeadV) {
#pragma unroll
        for (int k = 0; k < S::kStageBlocks; ++k) {
          v_off[k] = src_off[k];
          v_bytes[k] = src_bytes[k];
        }
      }
    }
    if (S::kPair)
      wait_vm<0>();
    else
      wait_previous();
  }
  if (S::KS == 2 && grp == 1) __syncthreads();
  __syncthreads();
  using B2 = std::integral_constant<int, 2>;
  if (n_g > 0) step(B0{}, std::false_type{}, 0);  // the first tile has no PV of a previous one
  int i = 1;
  if constexpr (S::kBufs == 2) {
    for (; i + 1 < n_g; i += 2) {
      step(B1{}, std::true_type{}, i);
      step(B0{}, std::true_type{}, i + 1);
    }
    if (i < n_g) step(B1{}, std::true_type{}, i);
  } else {
    for (; i + 2 < n_g; i += 3) {
      step(B1{}, std::true_type{}, i);
      step(B2{}, std::true_type{}, i + 1);
      step(B0{}, std::true_type{}, i + 2);
    }
    if (i < n_g) step(B1{}, std::true_type{}, i++);
    if (i < n_g) step(B2{}, std::true_type{}, i++);
  }
  // the last tile's PV
  if (n_g > 0) {
    const int lb = (n_g - 1) % S::kBufs;
    if (lb == 0)
      pv(B0{});
    else if (lb == 1)
      pv(B1{});
    else if constexpr (S::kBufs == 3)
      pv(B2{});
  }
  // the copies past the range land before LDS is reused below
  wait_vm<0>();
  if (S::KS == 2 && grp == 0) __syncthreads();
  // equal barrier counts: group 1 may have one tile fewer than group 0
  for (int k = 2 * n_g; k < 2 * nA; ++k) __syncthreads();

  // combine the two lane halves of each query's sum
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if (S::KS == 2 && !S::kPair) {
    // group 1 hands (m, lsum, O^T) to group 0 through LDS (tiles are done)
    float* xs = reinterpret_cast<float*>(lds) + (wave * 64 + lane) * 66;
    if (grp == 1) {
      xs[0] = m;
      xs[1] = lsum;
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i2 = 0; i2 < 16; ++i2) xs[2 + 16 * d + i2] = o_acc[d][i2];
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xs[0], l1 = xs[1];
    const float M = fmaxf(m, m1);
    const float f0 = fast_exp2(m - M), f1 = fast_exp2(m1 - M);
    lsum = lsum * f0 + l1 * f1;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i2 = 0; i2 < 16; ++i2) o_acc[d][i2] = o_acc[d][i2] * f0 + xs[2 + 16 * d + i2] * f1;
    m = M;
  }

  if (!q_valid) return;
  const bool empty = !(lsum > 0.f);
  const float inv = empty ? 0.f : 1.f / lsum;
  const size_t row = static_cast<size_t>(q0 + qi) * p.Hq + head;
  uint16_t* orow = p.out + row * kHeadDim;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int dim = 32 * d + 8 * r4 + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(o_acc[d][4 * r4] * inv, o_acc[d][4 * r4 + 1] * inv);
      w.y = pack_bf16x2(o_acc[d][4 * r4 + 2] * inv, o_acc[d][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + dim) = w;
    }
  if (half == 0 && p.lse) p.lse[row] = empty ? -INFINITY : (m + log2f(lsum)) * kLn2;
}

// Kernel parameters of a prefill launch (host side).
inline PrefillParams make_prefill_params(const PrefillArgs& a) {
  PrefillParams prm{};
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.query_start_loc = a.query_start_loc;
  prm.k_cache = static_cast<const uint16_t*>(a.k_cache);
  prm.v_cache = static_cast<const uint16_t*>(a.v_cache);
  prm.block_tables = a.block_tables;
  prm.context_lens = a.context_lens;
  prm.out = static_cast<uint16_t*>(a.out);
  prm.lse = a.lse;
  prm.max_blocks = a.max_blocks_per_seq;
  prm.B = a.B;
  prm.total_q = a.total_q;
  prm.max_q_len = a.max_q_len;
  prm.Hq = a.Hq;
  prm.Hkv = a.Hkv;
  prm.num_blocks = a.num_blocks;
  const long cap_bt = static_cast<long>(a.max_blocks_per_seq) * kBlockSize;
  prm.ctx_cap = static_cast<int>(a.max_context_len < cap_bt ? a.max_context_len : cap_bt);
  prm.scale_log2 = fabsf(a.scale) * kLog2e;
  prm.negate_q = a.scale < 0.f;
  return prm;
}

}  // namespace pre
}  // namespace fe
