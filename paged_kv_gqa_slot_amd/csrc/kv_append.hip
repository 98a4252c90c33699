// KV append: scatter new K/V rows into their cache slots through the slot
// mapping (ForgeEngine README, "What it implements": paged KV cache; its
// architecture flowchart's write edge from the prefill/decode step into the
// cache).  Pure data movement: each thread moves one 16-byte quarter-row.
#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {
namespace {

// One 16-byte unit = 8 bf16; a 128-dim row is 16 units.  Unit u covers
// (token i, tensor K/V, KV head g, unit c) with c fastest, so the 16 threads of
// a row write one contiguous 256-byte run.
__global__ __launch_bounds__(256) void kv_append_kernel(const uint4* __restrict__ k_new,
                                                        const uint4* __restrict__ v_new,
                                                        const int32_t* __restrict__ slot_mapping,
                                                        uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                                        int T, int Hkv, int64_t num_slots) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(Hkv) * 32;  // 2 tensors x Hkv heads x 16 units
  if (u >= per_token * T) return;
  const int i = static_cast<int>(u / per_token);
  int r = static_cast<int>(u - static_cast<int64_t>(i) * per_token);
  const int is_v = r >= Hkv * 16;
  if (is_v) r -= Hkv * 16;
  const int g = r >> 4, c = r & 15;
  const int64_t s = slot_mapping[i];
  if (s < 0 || s >= num_slots) return;  // padding, or outside the pool
  const int64_t blk = s / kBlockSize, off = s % kBlockSize;
  const int64_t src = (static_cast<int64_t>(i) * Hkv + g) * 16 + c;
  const int64_t dst = ((blk * Hkv + g) * kBlockSize + off) * 16 + c;
  if (is_v)
    v_cache[dst] = v_new[src];
  else
    k_cache[dst] = k_new[src];
}

}  // namespace

hipError_t launch_kv_append(const void* k_new, const void* v_new, const int32_t* slot_mapping, void* k_cache,
                            void* v_cache, int T, int num_blocks, int Hkv, hipStream_t stream) {
  const int64_t units = static_cast<int64_t>(T) * Hkv * 32;
  const unsigned grid = static_cast<unsigned>((units + 255) / 256);
  const uint4* kn = static_cast<const uint4*>(k_new);
  const uint4* vn = static_cast<const uint4*>(v_new);
  uint4* kc = static_cast<uint4*>(k_cache);
  uint4* vc = static_cast<uint4*>(v_cache);
  int64_t num_slots = static_cast<int64_t>(num_blocks) * kBlockSize;
  void* args[] = {&kn, &vn, &slot_mapping, &kc, &vc, &T, &Hkv, &num_slots};
  return hipLaunchKernel(reinterpret_cast<const void*>(&kv_append_kernel), dim3(grid), dim3(256), args, 0,
                         stream);
}

}  // namespace fe
