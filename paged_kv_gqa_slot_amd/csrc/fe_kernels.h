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
};

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_cache,
                            void* v_cache, int T, int num_blocks, int Hkv, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace fe
