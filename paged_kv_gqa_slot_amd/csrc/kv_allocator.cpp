// Host-side paged KV block allocator (ForgeEngine README, "What it
// implements": the KV cache is a paged block allocator with deterministic
// cleanup; "Loading": one scheduler worker owns KV-cache mutation; its
// measurements table reports zero allocated KV blocks after a workload with
// finished and cancelled requests).
//
// Blocks are handed out from a stack.  It starts as 0, 1, 2, ... from the
// top, and a released sequence pushes its blocks back in reverse token order,
// so its first block is on top again: which block a call gets depends only on
// the sequence of calls, never on timing.  Appends are all or nothing.  The
// allocator is owned by one thread (the scheduler); calls on one allocator
// must not overlap.
#include <cstdint>
#include <new>
#include <vector>

#include "fe.h"

struct fe_kv_allocator {
  int num_blocks, block_size, max_seqs, max_blocks_per_seq;
  std::vector<int32_t> free_stack;             // top = back()
  std::vector<std::vector<int32_t>> blocks;    // per sequence, in token order
  std::vector<int> len;                        // per sequence, tokens
};

namespace {

bool valid_seq(const fe_kv_allocator* a, int seq) { return a && seq >= 0 && seq < a->max_seqs; }

long blocks_for(long tokens, int bs) { return (tokens + bs - 1) / bs; }

}  // namespace

extern "C" {

fe_kv_allocator* fe_kv_allocator_create(int num_blocks, int block_size, int max_seqs, int max_blocks_per_seq) {
  if (num_blocks <= 0 || block_size <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0) return nullptr;
  if (static_cast<int64_t>(num_blocks) * block_size > INT32_MAX) return nullptr;  // slots are int32
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX) return nullptr;
  try {
    fe_kv_allocator* a = new fe_kv_allocator;
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->max_seqs = max_seqs;
    a->max_blocks_per_seq = max_blocks_per_seq;
    a->free_stack.resize(num_blocks);
    for (int i = 0; i < num_blocks; ++i) a->free_stack[i] = num_blocks - 1 - i;  // block 0 on top
    a->blocks.resize(max_seqs);
    a->len.assign(max_seqs, 0);
    return a;
  } catch (...) {
    return nullptr;
  }
}

void fe_kv_allocator_destroy(fe_kv_allocator* a) { delete a; }

int fe_kv_allocator_append(fe_kv_allocator* a, int seq, int n, int32_t* slots_out) {
  if (!valid_seq(a, seq) || n < 0) return FE_ERR_INVALID_ARG;
  if (n == 0) return FE_OK;
  if (!slots_out) return FE_ERR_NULL;
  const long L = a->len[seq];
  const long L2 = L + n;
  if (L2 > static_cast<long>(a->max_blocks_per_seq) * a->block_size) return FE_ERR_CAPACITY;
  const long need = blocks_for(L2, a->block_size) - blocks_for(L, a->block_size);
  if (need > static_cast<long>(a->free_stack.size())) return FE_ERR_CAPACITY;
  std::vector<int32_t>& mine = a->blocks[seq];
  try {
    mine.reserve(mine.size() + need);
  } catch (...) {
    return FE_ERR_INTERNAL;
  }
  for (long i = 0; i < need; ++i) {
    mine.push_back(a->free_stack.back());
    a->free_stack.pop_back();
  }
  for (long t = L; t < L2; ++t)
    slots_out[t - L] = mine[t / a->block_size] * a->block_size + static_cast<int32_t>(t % a->block_size);
  a->len[seq] = static_cast<int>(L2);
  return FE_OK;
}

int fe_kv_allocator_release(fe_kv_allocator* a, int seq) {
  if (!valid_seq(a, seq)) return FE_ERR_INVALID_ARG;
  std::vector<int32_t>& mine = a->blocks[seq];
  for (auto it = mine.rbegin(); it != mine.rend(); ++it) a->free_stack.push_back(*it);
  mine.clear();
  a->len[seq] = 0;
  return FE_OK;
}

int fe_kv_allocator_seq_len(const fe_kv_allocator* a, int seq) {
  if (!valid_seq(a, seq)) return FE_ERR_INVALID_ARG;
  return a->len[seq];
}

int fe_kv_allocator_num_free(const fe_kv_allocator* a) {
  return a ? static_cast<int>(a->free_stack.size()) : FE_ERR_NULL;
}

int fe_kv_allocator_num_allocated(const fe_kv_allocator* a) {
  return a ? a->num_blocks - static_cast<int>(a->free_stack.size()) : FE_ERR_NULL;
}

int fe_kv_allocator_batch(const fe_kv_allocator* a, const int* seqs, int n, int32_t* block_tables, int row_len,
                          int32_t pad_block, int32_t* context_lens) {
  if (!a) return FE_ERR_NULL;
  if (n < 0 || row_len <= 0) return FE_ERR_INVALID_ARG;
  if (n == 0) return FE_OK;
  if (!seqs || !block_tables || !context_lens) return FE_ERR_NULL;
  for (int i = 0; i < n; ++i) {
    if (!valid_seq(a, seqs[i])) return FE_ERR_INVALID_ARG;
    if (static_cast<long>(a->blocks[seqs[i]].size()) > row_len) return FE_ERR_CAPACITY;
  }
  for (int i = 0; i < n; ++i) {
    const std::vector<int32_t>& mine = a->blocks[seqs[i]];
    int32_t* row = block_tables + static_cast<size_t>(i) * row_len;
    for (int j = 0; j < row_len; ++j) row[j] = j < static_cast<int>(mine.size()) ? mine[j] : pad_block;
    context_lens[i] = a->len[seqs[i]];
  }
  return FE_OK;
}

}  // extern "C"
