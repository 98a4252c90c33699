// In-bounds HBM read probe: the read ceiling of the decode kernel's own load
// form, measured on the device the kernels run on.  Performance claims need a
// reproducible measurement beside them (ForgeLM README, "Tooling and
// Benchmarks"); this gives the attention benchmarks a same-run ceiling that
// uses exactly the loads decode uses: whole 4 KiB tiles, each fetched by one
// wave as four 1 KiB runs of non-temporal 16-byte buffer loads, in an order
// the caller chooses (a random permutation models the block tables).
//
// Each wave reads 16 tiles: their ids come in with one load (lane k holds
// id k), then four groups of four tiles, the next group's 16 loads issued
// before the current group is folded.  The data is XOR-folded into one word
// per wave, so nothing is dead and the only stores are 4 bytes per 64 KiB.
#include "fe_device.h"

namespace fe {
namespace {

constexpr int kProbeWaves = 4;
constexpr int kProbeTileBytes = 4096;
constexpr int kGroupTiles = 4;
constexpr int kGroups = kProbeTilesPerWave / kGroupTiles;
constexpr int kLoadPolicyNT = 2;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct Group {
  u32x4_t w[kGroupTiles][4];
};

__global__ __launch_bounds__(64 * kProbeWaves) void hbm_read_probe_kernel(const unsigned char* __restrict__ base,
                                                                           int64_t num_tiles,
                                                                           const int32_t* __restrict__ ids, int n,
                                                                           uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const long first = (static_cast<long>(blockIdx.x) * kProbeWaves + wave) * kProbeTilesPerWave;
  if (first >= n) return;
  // lane k < 16: the id of this wave's tile k, or -1 past the list or the buffer
  int id = -1;
  if (lane < kProbeTilesPerWave && first + lane < n) {
    const int v = ids[first + lane];
    id = (v >= 0 && v < num_tiles) ? v : -1;
  }
  auto load = [&](Group& gr, int grp) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < kGroupTiles; ++t) {
      const int tid = __builtin_amdgcn_readlane(id, grp * kGroupTiles + t);
      const unsigned char* p = base + static_cast<size_t>(tid < 0 ? 0 : tid) * kProbeTileBytes;
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(p), static_cast<short>(0), tid < 0 ? 0 : kProbeTileBytes, 0x00020000);
#pragma unroll
      for (int j = 0; j < 4; ++j) gr.w[t][j] = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16 + 1024 * j, 0, kLoadPolicyNT);
    }
  };
  uint32_t x = 0;
  Group ring[2];
  load(ring[0], 0);
#pragma unroll
  for (int grp = 0; grp < kGroups; ++grp) {
    if (grp + 1 < kGroups) load(ring[(grp + 1) & 1], grp + 1);
#pragma unroll
    for (int t = 0; t < kGroupTiles; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4_t& w = ring[grp & 1].w[t][j];
        x ^= w[0] ^ w[1] ^ w[2] ^ w[3];
      }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0) sink[first / kProbeTilesPerWave] = x;
}

}  // namespace

hipError_t launch_hbm_read_probe(const void* base, int64_t num_tiles, const int32_t* tile_ids, int n, uint32_t* sink,
                                 hipStream_t stream) {
  const long waves = (static_cast<long>(n) + kProbeTilesPerWave - 1) / kProbeTilesPerWave;
  const long grid = (waves + kProbeWaves - 1) / kProbeWaves;
  if (grid == 0) return hipSuccess;
  const unsigned char* b = static_cast<const unsigned char*>(base);
  void* args[] = {&b, &num_tiles, &tile_ids, &n, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&hbm_read_probe_kernel), dim3(static_cast<unsigned>(grid)),
                         dim3(64 * kProbeWaves), args, 0, stream);
}

}  // namespace fe
