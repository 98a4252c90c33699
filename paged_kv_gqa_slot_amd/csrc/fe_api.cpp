// C ABI of libfe.so (declared in include/fe.h): synchronous argument checks,
// then asynchronous kernel launches on the caller's stream.  Nothing here
// allocates, and no C++ exception leaves these functions.
#include "fe.h"

#include <math.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "fe_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* func, const char* what) {
  char buf[512];
  std::snprintf(buf, sizeof buf, "%s: %s", func, what);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* func) {
  char buf[512];
  std::snprintf(buf, sizeof buf, "%s: HIP error %d (%s)", func, static_cast<int>(e), hipGetErrorString(e));
  g_last_error = buf;
  return FE_ERR_HIP;
}

// Shape checks shared by the attention calls.  Returns FE_OK or an error
// status (with the message recorded).
int check_heads(const char* func, int Hq, int Hkv, int D, int BS) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0) return fail(FE_ERR_INVALID_ARG, func, "Hq, Hkv, D and BS must be positive");
  if (Hq % Hkv != 0) return fail(FE_ERR_INVALID_ARG, func, "Hq must be a multiple of Hkv");
  if (D != fe::kHeadDim) return fail(FE_ERR_UNSUPPORTED, func, "only head_dim 128 is built");
  if (BS != fe::kBlockSize) return fail(FE_ERR_UNSUPPORTED, func, "only KV block size 16 is built");
  if (Hq / Hkv > 8) return fail(FE_ERR_UNSUPPORTED, func, "group size Hq/Hkv above 8 is not built");
  return FE_OK;
}

// The kernels move 16-byte units; every tensor pointer must allow that.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A launch's work-items (workgroups x threads) must stay below 2^32.
bool launch_fits(double workgroups, int threads) { return workgroups * threads < 4294967296.0; }
constexpr const char* kTooLarge = "sizes need a launch of 2^32 or more work-items";

}  // namespace

extern "C" {

const char* fe_status_string(int status) {
  switch (status) {
    case FE_OK: return "FE_OK";
    case FE_ERR_NULL: return "FE_ERR_NULL";
    case FE_ERR_INVALID_ARG: return "FE_ERR_INVALID_ARG";
    case FE_ERR_UNSUPPORTED: return "FE_ERR_UNSUPPORTED";
    case FE_ERR_WORKSPACE: return "FE_ERR_WORKSPACE";
    case FE_ERR_HIP: return "FE_ERR_HIP";
    case FE_ERR_INTERNAL: return "FE_ERR_INTERNAL";
    case FE_ERR_CAPACITY: return "FE_ERR_CAPACITY";
    default: return "FE_ERR_UNKNOWN";
  }
}

const char* fe_last_error(void) { return g_last_error.c_str(); }

int fe_paged_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_cache,
                       void* v_cache, int T, int num_blocks, int Hkv, int D, int BS, hipStream_t stream) {
  static const char* fn = "fe_paged_kv_append";
  try {
    if (T < 0 || num_blocks <= 0 || Hkv <= 0 || D <= 0 || BS <= 0)
      return fail(FE_ERR_INVALID_ARG, fn, "T must be >= 0 and num_blocks, Hkv, D, BS positive");
    if (D != fe::kHeadDim) return fail(FE_ERR_UNSUPPORTED, fn, "only head_dim 128 is built");
    if (BS != fe::kBlockSize) return fail(FE_ERR_UNSUPPORTED, fn, "only KV block size 16 is built");
    if (!k_cache || !v_cache) return fail(FE_ERR_NULL, fn, "k_cache and v_cache must not be NULL");
    if (T == 0) return FE_OK;
    if (!k_new || !v_new || !slot_mapping) return fail(FE_ERR_NULL, fn, "k_new, v_new, slot_mapping must not be NULL");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
      return fail(FE_ERR_INVALID_ARG, fn, "k_new, v_new, k_cache, v_cache must be 16-byte aligned");
    if (!launch_fits(static_cast<double>(T) * Hkv * 32 / 256, 256)) return fail(FE_ERR_UNSUPPORTED, fn, kTooLarge);
    const hipError_t e = fe::launch_kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, T, num_blocks, Hkv, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

size_t fe_paged_gqa_decode_workspace_size(int B, int Hq, int Hkv, int D, int max_context_len, int num_partitions) {
  fe::DecodePlan plan;
  if (D != fe::kHeadDim || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return static_cast<size_t>(-1);
  if (!fe::plan_decode(B, Hq, Hkv, max_context_len, num_partitions, &plan)) return static_cast<size_t>(-1);
  return plan.workspace_bytes;
}

int fe_paged_gqa_decode_num_partitions(int B, int Hq, int Hkv, int D, int max_context_len, int num_partitions) {
  fe::DecodePlan plan;
  if (D != fe::kHeadDim || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return -1;
  if (!fe::plan_decode(B, Hq, Hkv, max_context_len, num_partitions, &plan)) return -1;
  return plan.partitions;
}

namespace {

// The norm/rotary inputs of fe_paged_gqa_decode_norm_rope_append.
struct NormRopeIn {
  const void* q_norm_w;
  const void* k_norm_w;
  const float* cos_sin;
  int max_pos;
  const int32_t* positions;
  float eps;
};

int decode_call(const char* fn, void* out, float* lse, const void* q, const void* k_new, const void* v_new,
                const int32_t* slot_mapping, bool fused, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens, int B, int Hq,
                int Hkv, int D, int BS, int num_blocks, int max_context_len, float scale, int num_partitions,
                void* workspace, size_t workspace_bytes, hipStream_t stream, bool use_scratch = false,
                const NormRopeIn* nr = nullptr) {
  try {
    if (nr) {
      if (nr->max_pos <= 0) return fail(FE_ERR_INVALID_ARG, fn, "max_pos must be positive");
      if (!isfinite(nr->eps) || nr->eps < 0.f) return fail(FE_ERR_INVALID_ARG, fn, "eps must be finite and >= 0");
      if (B > 0 && (!nr->q_norm_w || !nr->k_norm_w || !nr->cos_sin || !nr->positions))
        return fail(FE_ERR_NULL, fn, "q_norm_w, k_norm_w, cos_sin, positions must not be NULL");
      if (!aligned16(nr->q_norm_w) || !aligned16(nr->k_norm_w) || !aligned16(nr->cos_sin))
        return fail(FE_ERR_INVALID_ARG, fn, "the norm weights and cos_sin must be 16-byte aligned");
    }
    if (B < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 || num_partitions < 0)
      return fail(FE_ERR_INVALID_ARG, fn,
                  "B, max_context_len, num_partitions must be >= 0; num_blocks, max_blocks_per_seq positive");
    if (int rc = check_heads(fn, Hq, Hkv, D, BS)) return rc;
    if (!isfinite(scale)) return fail(FE_ERR_INVALID_ARG, fn, "scale must be finite");
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
      return fail(FE_ERR_NULL, fn, "out, q, k_cache, v_cache, block_tables, context_lens must not be NULL");
    if (fused && (!k_new || !v_new || !slot_mapping))
      return fail(FE_ERR_NULL, fn, "k_new, v_new, slot_mapping must not be NULL");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
      return fail(FE_ERR_INVALID_ARG, fn, "out, q, k_cache, v_cache, workspace must be 16-byte aligned");
    if (fused && (!aligned16(k_new) || !aligned16(v_new)))
      return fail(FE_ERR_INVALID_ARG, fn, "k_new, v_new must be 16-byte aligned");
    fe::DecodePlan plan;
    if (!fe::plan_decode(B, Hq, Hkv, max_context_len, num_partitions, &plan))
      return fail(FE_ERR_INVALID_ARG, fn, "cannot plan these sizes");
    if (use_scratch) {
      if (plan.workspace_bytes > fe::kDecodeScratchBytes) {
        char msg[384];
        std::snprintf(msg, sizeof msg,
                      "these sizes need %zu bytes of split-K workspace, above the %zu bytes of device scratch the "
                      "allocation-free call holds (use fe_paged_gqa_decode with a workspace, or fewer partitions)",
                      plan.workspace_bytes, fe::kDecodeScratchBytes);
        return fail(FE_ERR_WORKSPACE, fn, msg);
      }
    } else if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes)) {
      return fail(FE_ERR_WORKSPACE, fn, "workspace missing or smaller than fe_paged_gqa_decode_workspace_size()");
    }
    if (B == 0) return FE_OK;
    if (!launch_fits(static_cast<double>(B) * plan.partitions * Hkv, 256) ||
        !launch_fits(static_cast<double>(B) * Hq / 4, 256))
      return fail(FE_ERR_UNSUPPORTED, fn, kTooLarge);
    if (use_scratch && plan.workspace_bytes > 0) {
      const hipError_t e = fe::decode_scratch(stream, &workspace);
      if (e != hipSuccess) return hip_fail(e, fn);
    }
    fe::DecodeArgs a{out, lse, q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, B, Hq, Hkv,
                     num_blocks, max_context_len, scale, plan, workspace};
    if (fused) {
      a.k_new = k_new;
      a.v_new = v_new;
      a.new_slots = slot_mapping;
    }
    if (nr) {
      a.q_norm_w = nr->q_norm_w;
      a.k_norm_w = nr->k_norm_w;
      a.cos_sin = nr->cos_sin;
      a.positions = nr->positions;
      a.max_pos = nr->max_pos;
      a.eps = nr->eps;
    }
    const hipError_t e = fe::launch_decode(a, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

}  // namespace

int fe_paged_gqa_decode(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens, int B,
                        int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len, float scale,
                        int num_partitions, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_call("fe_paged_gqa_decode", out, lse, q, nullptr, nullptr, nullptr, false, k_cache, v_cache,
                     block_tables, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, num_blocks, max_context_len,
                     scale, num_partitions, workspace, workspace_bytes, stream);
}

int fe_paged_gqa_decode_noalloc(void* out, float* lse, const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                                int B, int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len,
                                float scale, int num_partitions, hipStream_t stream) {
  return decode_call("fe_paged_gqa_decode_noalloc", out, lse, q, nullptr, nullptr, nullptr, false, k_cache, v_cache,
                     block_tables, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, num_blocks, max_context_len,
                     scale, num_partitions, nullptr, 0, stream, true);
}

int fe_paged_gqa_decode_append(void* out, float* lse, const void* q, const void* k_new, const void* v_new,
                               const int32_t* slot_mapping, void* k_cache, void* v_cache,
                               const int32_t* block_tables, int max_blocks_per_seq, const int32_t* context_lens,
                               int B, int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len,
                               float scale, int num_partitions, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return decode_call("fe_paged_gqa_decode_append", out, lse, q, k_new, v_new, slot_mapping, true, k_cache, v_cache,
                     block_tables, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, num_blocks, max_context_len,
                     scale, num_partitions, workspace, workspace_bytes, stream);
}

int fe_paged_gqa_decode_norm_rope_append(void* out, float* lse, const void* q, const void* k_new, const void* v_new,
                                         const void* q_norm_w, const void* k_norm_w, const float* cos_sin,
                                         int max_pos, const int32_t* positions, const int32_t* slot_mapping,
                                         void* k_cache, void* v_cache, const int32_t* block_tables,
                                         int max_blocks_per_seq, const int32_t* context_lens, int B, int Hq, int Hkv,
                                         int D, int BS, int num_blocks, int max_context_len, float scale, float eps,
                                         int num_partitions, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  const NormRopeIn nr{q_norm_w, k_norm_w, cos_sin, max_pos, positions, eps};
  return decode_call("fe_paged_gqa_decode_norm_rope_append", out, lse, q, k_new, v_new, slot_mapping, true, k_cache,
                     v_cache, block_tables, max_blocks_per_seq, context_lens, B, Hq, Hkv, D, BS, num_blocks,
                     max_context_len, scale, num_partitions, workspace, workspace_bytes, stream, false, &nr);
}

namespace {

int prefill_chunk(const char* fn, void* out, float* lse, const void* q, const int32_t* query_start_loc,
                  const void* k_cache, const void* v_cache, const int32_t* block_tables, int max_blocks_per_seq,
                  const int32_t* context_lens, int B, int total_q, int max_q_len, int Hq, int Hkv, int D, int BS,
                  int num_blocks, int max_context_len, float scale, int key_groups, int split_weights,
                  hipStream_t stream) {
  try {
    if (key_groups < 0 || key_groups > 3) return fail(FE_ERR_INVALID_ARG, fn, "key_groups must be 0, 1, 2 or 3");
    if (split_weights != 0 && split_weights != 1) return fail(FE_ERR_INVALID_ARG, fn, "split_weights must be 0 or 1");
    if (B < 0 || total_q < 0 || max_q_len < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0)
      return fail(FE_ERR_INVALID_ARG, fn,
                  "B, total_q, max_q_len, max_context_len must be >= 0; num_blocks, max_blocks_per_seq positive");
    if (int rc = check_heads(fn, Hq, Hkv, D, BS)) return rc;
    if (!isfinite(scale)) return fail(FE_ERR_INVALID_ARG, fn, "scale must be finite");
    if (key_groups == 2 && !fe::prefill_two_key_groups_supported(Hq / Hkv))
      return fail(FE_ERR_UNSUPPORTED, fn, "key_groups 2 needs Hq/Hkv <= 4");
    if (key_groups == 3 && !fe::prefill_query_tile_pairs_supported(Hq / Hkv))
      return fail(FE_ERR_UNSUPPORTED, fn, "key_groups 3 needs Hq/Hkv in {1, 2, 4}");
    if (B == 0 || total_q == 0) return FE_OK;
    if (!out || !q || !query_start_loc || !k_cache || !v_cache || !block_tables || !context_lens)
      return fail(FE_ERR_NULL, fn,
                  "out, q, query_start_loc, k_cache, v_cache, block_tables, context_lens must not be NULL");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
      return fail(FE_ERR_INVALID_ARG, fn, "out, q, k_cache, v_cache must be 16-byte aligned");
    if (!launch_fits((max_q_len / 32.0 + 1) * Hkv * B, 512)) return fail(FE_ERR_UNSUPPORTED, fn, kTooLarge);
    fe::PrefillArgs a{out, lse, q, query_start_loc, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                      B, total_q, max_q_len, Hq, Hkv, num_blocks, max_context_len, scale, key_groups,
                      split_weights != 0};
    const hipError_t e = fe::launch_prefill(a, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

}  // namespace

int fe_paged_gqa_prefill_chunk(void* out, float* lse, const void* q, const int32_t* query_start_loc,
                               const void* k_cache, const void* v_cache, const int32_t* block_tables,
                               int max_blocks_per_seq, const int32_t* context_lens, int B, int total_q, int max_q_len,
                               int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len, float scale,
                               hipStream_t stream) {
  return prefill_chunk("fe_paged_gqa_prefill_chunk", out, lse, q, query_start_loc, k_cache, v_cache, block_tables,
                       max_blocks_per_seq, context_lens, B, total_q, max_q_len, Hq, Hkv, D, BS, num_blocks,
                       max_context_len, scale, 0, 0, stream);
}

int fe_paged_gqa_prefill_chunk_ex(void* out, float* lse, const void* q, const int32_t* query_start_loc,
                                  const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                  int max_blocks_per_seq, const int32_t* context_lens, int B, int total_q,
                                  int max_q_len, int Hq, int Hkv, int D, int BS, int num_blocks, int max_context_len,
                                  float scale, int key_groups, int split_weights, hipStream_t stream) {
  return prefill_chunk("fe_paged_gqa_prefill_chunk_ex", out, lse, q, query_start_loc, k_cache, v_cache,
                       block_tables, max_blocks_per_seq, context_lens, B, total_q, max_q_len, Hq, Hkv, D, BS,
                       num_blocks, max_context_len, scale, key_groups, split_weights, stream);
}

size_t fe_paged_gqa_mixed_workspace_size(int num_decode, int Hq, int Hkv, int D, int max_context_len,
                                         int num_partitions) {
  fe::MixedPlan plan;
  if (D != fe::kHeadDim || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0) return static_cast<size_t>(-1);
  if (!fe::plan_mixed(num_decode, Hq, Hkv, max_context_len, num_partitions, &plan)) return static_cast<size_t>(-1);
  return plan.workspace_bytes;
}

int fe_paged_gqa_mixed(void* out, float* lse, const void* q, const int32_t* query_start_loc, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables, int max_blocks_per_seq,
                       const int32_t* context_lens, int B, int num_decode, int total_q, int max_q_len, int Hq,
                       int Hkv, int D, int BS, int num_blocks, int max_context_len, float scale, int num_partitions,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "fe_paged_gqa_mixed";
  try {
    if (B < 0 || total_q < 0 || max_q_len < 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_context_len < 0 ||
        num_partitions < 0)
      return fail(FE_ERR_INVALID_ARG, fn,
                  "B, total_q, max_q_len, max_context_len, num_partitions must be >= 0; num_blocks, "
                  "max_blocks_per_seq positive");
    if (num_decode < 0 || num_decode > B) return fail(FE_ERR_INVALID_ARG, fn, "num_decode must be in [0, B]");
    if (num_decode > total_q) return fail(FE_ERR_INVALID_ARG, fn, "every decode row needs a query row (total_q)");
    if (int rc = check_heads(fn, Hq, Hkv, D, BS)) return rc;
    if (!isfinite(scale)) return fail(FE_ERR_INVALID_ARG, fn, "scale must be finite");
    fe::MixedPlan plan;
    if (!fe::plan_mixed(num_decode, Hq, Hkv, max_context_len, num_partitions, &plan))
      return fail(FE_ERR_INVALID_ARG, fn, "cannot plan these sizes");
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
      return fail(FE_ERR_WORKSPACE, fn, "workspace missing or smaller than fe_paged_gqa_mixed_workspace_size()");
    if (B == 0 || total_q == 0) return FE_OK;
    if (!out || !q || !query_start_loc || !k_cache || !v_cache || !block_tables || !context_lens)
      return fail(FE_ERR_NULL, fn,
                  "out, q, query_start_loc, k_cache, v_cache, block_tables, context_lens must not be NULL");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(workspace))
      return fail(FE_ERR_INVALID_ARG, fn, "out, q, k_cache, v_cache, workspace must be 16-byte aligned");
    if (!launch_fits((max_q_len / 32.0 + 1) * Hkv * B + static_cast<double>(num_decode) * plan.partitions * Hkv, 512))
      return fail(FE_ERR_UNSUPPORTED, fn, kTooLarge);
    fe::MixedArgs a{{out, lse, q, query_start_loc, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                     B, total_q, max_q_len, Hq, Hkv, num_blocks, max_context_len, scale},
                    num_decode, plan, workspace};
    const hipError_t e = fe::launch_mixed(a, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

int fe_qk_norm_rope_append(void* q_out, const void* q, const void* k, const void* v, const void* q_norm_w,
                           const void* k_norm_w, const float* cos_sin, int max_pos, const int32_t* positions,
                           const int32_t* slot_mapping, void* k_cache, void* v_cache, int T, int Hq, int Hkv, int D,
                           int BS, int num_blocks, float eps, hipStream_t stream) {
  static const char* fn = "fe_qk_norm_rope_append";
  try {
    if (T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || num_blocks <= 0 || max_pos <= 0)
      return fail(FE_ERR_INVALID_ARG, fn, "T must be >= 0; Hq, Hkv, D, BS, num_blocks, max_pos positive");
    if (D != fe::kHeadDim) return fail(FE_ERR_UNSUPPORTED, fn, "only head_dim 128 is built");
    if (BS != fe::kBlockSize) return fail(FE_ERR_UNSUPPORTED, fn, "only KV block size 16 is built");
    if (!isfinite(eps) || eps < 0.f) return fail(FE_ERR_INVALID_ARG, fn, "eps must be finite and >= 0");
    if (T == 0) return FE_OK;
    if (!q_out || !q || !k || !v || !q_norm_w || !k_norm_w || !cos_sin || !positions || !slot_mapping || !k_cache ||
        !v_cache)
      return fail(FE_ERR_NULL, fn, "no pointer may be NULL when T > 0");
    if (!aligned16(q_out) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_norm_w) ||
        !aligned16(k_norm_w) || !aligned16(cos_sin) || !aligned16(k_cache) || !aligned16(v_cache))
      return fail(FE_ERR_INVALID_ARG, fn, "q_out, q, k, v, the norm weights, cos_sin and the pools must be 16-byte aligned");
    if (!launch_fits(static_cast<double>(T) * (Hq + 2.0 * Hkv) / 16 + 1, 256))
      return fail(FE_ERR_UNSUPPORTED, fn, kTooLarge);
    const fe::NormRopeArgs a{q_out, q, k, v, q_norm_w, k_norm_w, cos_sin, max_pos, positions, slot_mapping, k_cache,
                             v_cache, T, Hq, Hkv, num_blocks, eps};
    const hipError_t e = fe::launch_qk_norm_rope(a, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

size_t fe_sampler_workspace_size(int B, int V) {
  if (B < 0 || V <= 0 || V % 8 != 0) return static_cast<size_t>(-1);
  fe::SamplerPlan plan;
  fe::plan_sampler(B, V, 0, &plan);  // form 0 always plans; the size is the ranges form's, for every form
  return plan.workspace_bytes;
}

int fe_sampler_form(int B, int V) {
  if (B < 0 || V <= 0 || V % 8 != 0) return -1;
  fe::SamplerPlan plan;
  fe::plan_sampler(B, V, 0, &plan);
  return plan.row_per_workgroup ? 2 : 1;
}

int fe_sampler_softmax_argmax_ex(float* probs, float* lse, int32_t* argmax, const void* logits,
                                 const float* inv_temperature, int B, int V, int form, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "fe_sampler_softmax_argmax";
  try {
    if (B < 0 || V <= 0) return fail(FE_ERR_INVALID_ARG, fn, "B must be >= 0 and V positive");
    if (form < 0 || form > 2) return fail(FE_ERR_INVALID_ARG, fn, "form must be 0, 1 or 2");
    if (V % 8 != 0) return fail(FE_ERR_UNSUPPORTED, fn, "V must be a multiple of 8");
    if (B == 0) return FE_OK;
    if (!argmax || !logits) return fail(FE_ERR_NULL, fn, "argmax and logits must not be NULL");
    if (!aligned16(logits) || !aligned16(probs))
      return fail(FE_ERR_INVALID_ARG, fn, "logits and probs must be 16-byte aligned");
    fe::SamplerPlan plan;
    if (!fe::plan_sampler(B, V, form, &plan))
      return fail(FE_ERR_UNSUPPORTED, fn, "form 2 (one workgroup per row) holds rows of at most 163,840 logits");
    if (!launch_fits(plan.row_per_workgroup ? static_cast<double>(B) : static_cast<double>(B) * plan.chunks,
                     plan.row_per_workgroup ? fe::kSamplerRowThreads : 256))
      return fail(FE_ERR_UNSUPPORTED, fn, kTooLarge);
    if (!workspace || workspace_bytes < plan.workspace_bytes)
      return fail(FE_ERR_WORKSPACE, fn, "workspace missing or smaller than fe_sampler_workspace_size()");
    const fe::SamplerArgs a{probs, lse, argmax, logits, inv_temperature, B, V, plan, workspace};
    const hipError_t e = fe::launch_sampler(a, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

int fe_sampler_softmax_argmax(float* probs, float* lse, int32_t* argmax, const void* logits,
                              const float* inv_temperature, int B, int V, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  return fe_sampler_softmax_argmax_ex(probs, lse, argmax, logits, inv_temperature, B, V, 0, workspace,
                                      workspace_bytes, stream);
}

int fe_hbm_read_probe(const void* base, int64_t num_tiles, const int32_t* tile_ids, int n, uint32_t* sink,
                      hipStream_t stream) {
  static const char* fn = "fe_hbm_read_probe";
  try {
    if (num_tiles <= 0 || n < 0) return fail(FE_ERR_INVALID_ARG, fn, "num_tiles must be positive and n >= 0");
    if (n == 0) return FE_OK;
    if (!base || !tile_ids || !sink) return fail(FE_ERR_NULL, fn, "base, tile_ids and sink must not be NULL");
    if (!aligned16(base)) return fail(FE_ERR_INVALID_ARG, fn, "base must be 16-byte aligned");
    const hipError_t e = fe::launch_hbm_read_probe(base, num_tiles, tile_ids, n, sink, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

int fe_mfma_rate_probe(const void* operands, int n_ops, int workgroups, int rounds, float* sink, hipStream_t stream) {
  static const char* fn = "fe_mfma_rate_probe";
  try {
    if (n_ops <= 0 || workgroups < 0 || rounds < 0)
      return fail(FE_ERR_INVALID_ARG, fn, "n_ops must be positive, workgroups and rounds >= 0");
    if (workgroups == 0) return FE_OK;
    if (!operands || !sink) return fail(FE_ERR_NULL, fn, "operands and sink must not be NULL");
    if (!aligned16(operands)) return fail(FE_ERR_INVALID_ARG, fn, "operands must be 16-byte aligned");
    if (static_cast<long>(workgroups) * fe::kMfmaProbeWaves * 64 >= (1L << 31))
      return fail(FE_ERR_UNSUPPORTED, fn, "too many workgroups for one launch");
    const hipError_t e = fe::launch_mfma_rate_probe(operands, n_ops, workgroups, rounds, sink, stream);
    return e == hipSuccess ? FE_OK : hip_fail(e, fn);
  } catch (...) {
    return fail(FE_ERR_INTERNAL, fn, "unexpected exception");
  }
}

}  // extern "C"
