// Host-side launch interface between the C ABI (fe_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace fe {

constexpr int kHeadDim = 128;   // D, the only head_dim built
constexpr int kBlockSize = 16;  // BS, tokens per KV block
constexpr int kTileElems = kBlockSize * kHeadDim;  // one (block, KV head) tile: 2048 bf16 = 4 KiB

// Decode launch plan: the longest context is cut into `partitions` ranges of
// `part_blocks` KV blocks each.  partitions == 1 means a single pass that
// writes the final output directly.
struct DecodePlan {
  int partitions;
  int part_blocks;
  size_t workspace_bytes;
  size_t o_part_offset;    // byte offsets in the workspace of the fp32 partial outputs
  size_t lse_part_offset;  // ... and of their LSEs
};

// Largest decode partition: 256 KV blocks (4096 tokens), i.e. at most 64
// tiles per wave, whose block ids one VGPR holds.
constexpr int kMaxPartBlocks = 256;

// Returns false for sizes the decode kernel cannot plan (non-positive sizes).
bool plan_decode(int B, int Hq, int Hkv, int max_context_len, int num_partitions, DecodePlan* plan);

// Allocation-free decode (fe_paged_gqa_decode_noalloc): the split-K
// workspace is a file-scope device array of this many bytes in decode.hip,
// one copy per GPU.  decode_scratch() returns its address on the device of
// `stream` (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = static_cast<size_t>(32) << 20;
hipError_t decode_scratch(hipStream_t stream, void** ptr);

struct DecodeArgs {
  void* out;
  float* lse;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int B, Hq, Hkv, num_blocks, max_context_len;
  float scale;
  DecodePlan plan;
  void* workspace;
  // fused append (fe_paged_gqa_decode_append): nullptr k_new means none
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* new_slots = nullptr;
  // fused norm/rotary of q and the new k (fe_paged_gqa_decode_norm_rope_append):
  // nullptr q_norm_w means none
  const void* q_norm_w = nullptr;
  const void* k_norm_w = nullptr;
  const float* cos_sin = nullptr;
  const int32_t* positions = nullptr;
  int max_pos = 0;
  float eps = 0.f;
};

struct PrefillArgs {
  void* out;
  float* lse;
  const void* q;
  const int32_t* query_start_loc;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int max_blocks_per_seq;
  const int32_t* context_lens;
  int B, total_q, max_q_len, Hq, Hkv, num_blocks, max_context_len;
  float scale;
  int key_groups = 0;  // prefill tile: 0 automatic, 1 or 2 key groups, 3 two query tiles over one K/V stream
  bool split_p = false;  // softmax weights into the PV product as two bf16 parts (rounded value + remainder)
};

// Mixed decode/prefill launch plan.  The decode sequences are split into
// `partitions` ranges of `part_blocks` blocks; their partials are merged in
// the same launch by the last partition to finish, counted in the workspace:
// [arrival counters int num_decode x Hkv][o_part fp32][lse_part fp32].
struct MixedPlan {
  int partitions;
  int part_blocks;
  size_t workspace_bytes;
  size_t o_part_offset;
  size_t lse_part_offset;
};

// Automatic decode partitions of a mixed launch: ranges of at least
// kMixedMinPartBlocks blocks (1024 tokens), and no more partitions than
// about kMixedItemsPerCu decode items per CU.  The launch runs one workgroup
// per CU (every workgroup reserves the prefill tile's LDS and registers), so
// each decode item's fixed start and split-merge cost is paid in series on
// its CU; with many decode rows, fewer and longer items pay it less often.
constexpr int kMixedMinPartBlocks = 64;
constexpr int kMixedItemsPerCu = 6;

bool plan_mixed(int num_decode, int Hq, int Hkv, int max_context_len, int num_partitions, MixedPlan* plan);

struct MixedArgs {
  PrefillArgs all;  // the whole batch: sequences [0, num_decode) decode, the rest prefill chunks
  int num_decode;
  MixedPlan plan;
  void* workspace;
};

struct NormRopeArgs {
  void* q_out;
  const void* q;
  const void* k;
  const void* v;
  const void* q_norm_w;
  const void* k_norm_w;
  const float* cos_sin;
  int max_pos;
  const int32_t* positions;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int T, Hq, Hkv, num_blocks;
  float eps;
};

// Sampler plan.  Two forms:
//  * ranges (two launches): each row of V logits is cut into `chunks` ranges
//    of `chunk_units` 8-logit units; the workspace holds one 16-byte partial
//    per (row, range);
//  * one workgroup per row (one launch): the row stays in the registers of
//    kSamplerRowThreads threads, at most kSamplerRowUnits units each, and is
//    read once.  One CU moves a row at only a few tens of GB/s, and one such
//    workgroup fills a CU, so this form needs rows that cover the CUs: the
//    automatic choice takes it when every round of kSamplerRowRound
//    workgroups (one per CU) holds at least kSamplerRowMinBatch rows.
// workspace_bytes is the ranges form's size whichever form runs, so that a
// workspace sized by the query serves either.
struct SamplerPlan {
  int chunks;
  int chunk_units;
  size_t workspace_bytes;
  bool row_per_workgroup;
};
constexpr int kSamplerTargetWgs = 1024;  // about 4 workgroups per CU
constexpr int kSamplerMinUnits = 512;    // ranges of at least 4096 logits
constexpr int kSamplerMaxUnits = 2048;   // ... and at most 16384 (8 units per thread)
constexpr int kSamplerRowThreads = 1024;
constexpr int kSamplerRowUnits = 20;     // rows of up to 163,840 logits
constexpr int kSamplerRowMinBatch = 160;
constexpr int kSamplerRowRound = 256;
// form: 0 automatic, 1 ranges, 2 one workgroup per row.  Returns false for a
// form this V cannot take (2 with V beyond the registers' reach).
bool plan_sampler(int B, int V, int form, SamplerPlan* plan);

struct SamplerArgs {
  float* probs;
  float* lse;
  int32_t* argmax;
  const void* logits;
  const float* inv_temperature;
  int B, V;
  SamplerPlan plan;
  void* workspace;
};

// HBM read probe (hbm_probe.hip): each wave reads kProbeTilesPerWave tiles
// of 4 KiB and writes one word of sink.
constexpr int kProbeTilesPerWave = 16;
hipError_t launch_hbm_read_probe(const void* base, int64_t num_tiles, const int32_t* tile_ids, int n, uint32_t* sink,
                                 hipStream_t stream);

// bf16 MFMA rate probe (mfma_probe.hip): workgroups of kMfmaProbeWaves waves,
// each issuing kMfmaProbeRoundMfmas MFMAs per round and writing one float of
// sink.
constexpr int kMfmaProbeWaves = 8;
constexpr int kMfmaProbeRoundMfmas = 64;
hipError_t launch_mfma_rate_probe(const void* operands, int n_ops, int workgroups, int rounds, float* sink,
                                  hipStream_t stream);

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_cache,
                            void* v_cache, int T, int num_blocks, int Hkv, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
bool prefill_two_key_groups_supported(int G);    // key_groups = 2 is valid for this Hq / Hkv
bool prefill_query_tile_pairs_supported(int G);  // key_groups = 3 is valid for this Hq / Hkv
hipError_t launch_mixed(const MixedArgs& a, hipStream_t stream);
hipError_t launch_qk_norm_rope(const NormRopeArgs& a, hipStream_t stream);
hipError_t launch_sampler(const SamplerArgs& a, hipStream_t stream);

}  // namespace fe
