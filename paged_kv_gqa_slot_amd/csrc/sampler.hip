// The sampler's hot step: fp32 softmax, log-sum-exp and greedy argmax over
// each row of vocabulary logits ("Make the Engine Talk" section 1.3: the
// sampler -- greedy, temperature and top-p decoding -- runs its softmax in
// fp32 over the whole vocabulary; ForgeEngine README, "What it implements":
// sampling policies).  Bandwidth-bound: the logits are read, the
// probabilities written.
//
// A row of V logits is cut into `chunks` ranges so that a small batch still
// fills the GPU.  Pass 1, one workgroup per (row, range): online max / sum of
// 2^(s x log2 e - m) and the first maximal logit, as a partial in the
// workspace.  Pass 2, one workgroup per (row, range): merge the row's
// partials (a few dozen bytes, one load per lane), then write the range's
// probabilities; range 0 also writes the argmax and the LSE.  Each thread reads 8 bf16 logits per
// 16-byte load.
//
// With enough rows to cover the CUs, one workgroup of 1024 threads per row
// instead: the row stays in registers, so the logits are read once and one
// launch does both passes, with the row's merge in LDS.
#include <math.h>

#include "fe_device.h"
#include "fe_kernels.h"

namespace fe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnitsPerThread = kSamplerMaxUnits / kThreads;  // a range's units per thread, loaded at once
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

struct Partial {  // one (row, range): running max m (log2 units), sum of 2^(y - m), first maximal logit
  float m, sum, best_v;
  int best_i;
};

struct SamplerParams {
  const uint16_t* logits;
  const float* inv_temp;
  float* probs;
  float* lse;
  int32_t* argmax;
  Partial* part;
  int B, V, chunks, chunk_units;  // chunk_units: 8-logit units per range
};

__device__ __forceinline__ void merge_ms(float& m, float& sum, float m2, float sum2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;  // both empty
  sum = (m == -INFINITY ? 0.f : sum * fast_exp2(m - M)) + (m2 == -INFINITY ? 0.f : sum2 * fast_exp2(m2 - M));
  m = M;
}

__device__ __forceinline__ void merge_best(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

// Exchange (m, sum, best value, best index) with one partner lane and merge:
// kCtrl is a DPP control within 16-lane rows, or 16 / 32 for the permlane
// swaps across rows.  Both lanes of a pair compute the same merge (both
// merges are symmetric), so after quad xor 1, quad xor 2, the half-row and
// row mirrors and the two swaps every lane holds the wave's result.
template <int kCtrl>
__device__ __forceinline__ void exchange(float& m, float& sum, float& best_v, int& best_i) {
  float m2, sum2, v2;
  int i2;
  if constexpr (kCtrl == 16 || kCtrl == 32) {
    m2 = xor_partner<kCtrl>(m);
    sum2 = xor_partner<kCtrl>(sum);
    v2 = xor_partner<kCtrl>(best_v);
    i2 = __float_as_int(xor_partner<kCtrl>(__int_as_float(best_i)));
  } else {
    m2 = dpp<kCtrl>(m);
    sum2 = dpp<kCtrl>(sum);
    v2 = dpp<kCtrl>(best_v);
    i2 = __float_as_int(dpp<kCtrl>(__int_as_float(best_i)));
  }
  merge_ms(m, sum, m2, sum2);
  merge_best(best_v, best_i, v2, i2);
}

__device__ __forceinline__ void wave_merge(float& m, float& sum, float& best_v, int& best_i) {
  exchange<kDppQuadXor1>(m, sum, best_v, best_i);
  exchange<kDppQuadXor2>(m, sum, best_v, best_i);
  exchange<kDppRowHalfMirror>(m, sum, best_v, best_i);
  exchange<kDppRowMirror>(m, sum, best_v, best_i);
  exchange<16>(m, sum, best_v, best_i);
  exchange<32>(m, sum, best_v, best_i);
}

__device__ __forceinline__ float row_scale(const SamplerParams& p, int b) {
  return (p.inv_temp ? p.inv_temp[b] : 1.0f) * kLog2e;
}

__global__ __launch_bounds__(kThreads) void sampler_partial_kernel(SamplerParams p) {
  const int c = blockIdx.x % p.chunks;
  const int b = blockIdx.x / p.chunks;
  const float sc = row_scale(p, b);
  const int u0 = c * p.chunk_units;
  const int u1 = min(u0 + p.chunk_units, p.V / 8);
  const uint4* row = reinterpret_cast<const uint4*>(p.logits + static_cast<size_t>(b) * p.V);
  float m = -INFINITY, sum = 0.f, best_v = -INFINITY;
  int best_i = 0x7fffffff;
  // all of this thread's loads first (at most kUnitsPerThread units)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t w[kUnitsPerThread];
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const int u = u0 + threadIdx.x + k * kThreads;
    // plain loads: non-temporal ones were 1-2% slower; pass 2 fetches the
    // logits past the L2 either way (it does not keep them across launches)
    w[k] = u < u1 ? *reinterpret_cast<const u32x4_t*>(&row[u]) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const int u = u0 + threadIdx.x + k * kThreads;
    if (u >= u1) break;
    const float x[8] = {bf16_lo(w[k][0]), bf16_hi(w[k][0]), bf16_lo(w[k][1]), bf16_hi(w[k][1]),
                        bf16_lo(w[k][2]), bf16_hi(w[k][2]), bf16_lo(w[k][3]), bf16_hi(w[k][3])};
    float um = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      um = fmaxf(um, x[j] * sc);
      if (x[j] > best_v) {  // indices grow along a thread's walk: the first maximum stays
        best_v = x[j];
        best_i = 8 * u + j;
      }
    }
    const float M = fmaxf(m, um);
    if (M == -INFINITY) continue;  // everything so far is masked
    float t = m == -INFINITY ? 0.f : sum * fast_exp2(m - M);
#pragma unroll
    for (int j = 0; j < 8; ++j) t += fast_exp2(x[j] * sc - M);
    m = M;
    sum = t;
  }
  // wave, then workgroup
  wave_merge(m, sum, best_v, best_i);
  __shared__ Partial sh[kWaves];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[wave] = Partial{m, sum, best_v, best_i};
  __syncthreads();
  if (threadIdx.x == 0) {
    Partial r = sh[0];
    for (int w = 1; w < kWaves; ++w) {
      merge_ms(r.m, r.sum, sh[w].m, sh[w].sum);
      merge_best(r.best_v, r.best_i, sh[w].best_v, sh[w].best_i);
    }
    p.part[static_cast<size_t>(b) * p.chunks + c] = r;
  }
}

// Every wave merges the row's partials (a few dozen): lane k loads partials
// k, k + 64, ... (one round trip for up to 64 ranges, where a serial walk took
// one per range), then a butterfly over the wave.  Range 0 writes the argmax
// and the LSE.
struct RowTotals {
  float M, Z;
  bool empty;
};

__device__ __forceinline__ RowTotals merge_row(const SamplerParams& p, int b, int c) {
  const Partial* pr = p.part + static_cast<size_t>(b) * p.chunks;
  float M = -INFINITY, Z = 0.f, best_v = -INFINITY;
  int best_i = 0x7fffffff;
  for (int k = threadIdx.x & 63; k < p.chunks; k += 64) {
    const Partial q = pr[k];
    merge_ms(M, Z, q.m, q.sum);
    merge_best(best_v, best_i, q.best_v, q.best_i);
  }
  wave_merge(M, Z, best_v, best_i);
  const bool empty = M == -INFINITY;
  if (c == 0 && threadIdx.x == 0) {
    p.argmax[b] = empty ? 0 : best_i;
    if (p.lse) p.lse[b] = empty ? -INFINITY : (M + log2f(Z)) * kLn2;
  }
  return RowTotals{M, Z, empty};
}

__global__ __launch_bounds__(kThreads) void sampler_write_kernel(SamplerParams p) {
  const int c = blockIdx.x % p.chunks;
  const int b = blockIdx.x / p.chunks;
  if (!p.probs) {  // argmax and LSE only: the logits are not read again
    merge_row(p, b, c);
    return;
  }
  const float sc = row_scale(p, b);
  const int u0 = c * p.chunk_units;
  const int u1 = min(u0 + p.chunk_units, p.V / 8);
  const uint4* row = reinterpret_cast<const uint4*>(p.logits + static_cast<size_t>(b) * p.V);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  // This thread's logits are loaded first, so their round trip overlaps the
  // partial merge.  Every load is issued, at a unit clamped into the row (a
  // load under a branch would make the compiler wait for it early); units
  // past the range are not used.
  u32x4_t w[kUnitsPerThread];
  const int last = max(u1 - 1, 0);
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const int u = min(u0 + static_cast<int>(threadIdx.x) + k * kThreads, last);
    w[k] = *reinterpret_cast<const u32x4_t*>(&row[u]);
  }
  const RowTotals t = merge_row(p, b, c);
  const float invZ = t.empty ? 0.f : 1.0f / t.Z;
  float4* out = reinterpret_cast<float4*>(p.probs + static_cast<size_t>(b) * p.V);
#pragma unroll
  for (int k = 0; k < kUnitsPerThread; ++k) {
    const int u = u0 + threadIdx.x + k * kThreads;
    if (u >= u1) break;
    const float x[8] = {bf16_lo(w[k][0]), bf16_hi(w[k][0]), bf16_lo(w[k][1]), bf16_hi(w[k][1]),
                        bf16_lo(w[k][2]), bf16_hi(w[k][2]), bf16_lo(w[k][3]), bf16_hi(w[k][3])};
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = t.empty ? 0.f : fast_exp2(x[j] * sc - t.M) * invZ;
    const f32x4_t lo = {e[0], e[1], e[2], e[3]}, hi = {e[4], e[5], e[6], e[7]};
    *reinterpret_cast<f32x4_t*>(&out[2 * u]) = lo;
    *reinterpret_cast<f32x4_t*>(&out[2 * u + 1]) = hi;
  }
}

// One workgroup per row: every thread issues all of its loads (units
// clamped into the row; those past it are not used), folds them into an
// online (max, sum, first maximum) as pass 1 does, the 16 waves' results
// merge through LDS, and the probabilities are written from the registers.
constexpr int kRowWaves = kSamplerRowThreads / 64;

__global__ __launch_bounds__(kSamplerRowThreads) void sampler_row_kernel(SamplerParams p) {
  const int b = blockIdx.x;
  const float sc = row_scale(p, b);
  const int units = p.V / 8;
  const uint4* row = reinterpret_cast<const uint4*>(p.logits + static_cast<size_t>(b) * p.V);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t w[kSamplerRowUnits];
  const int last = units - 1;
#pragma unroll
  for (int k = 0; k < kSamplerRowUnits; ++k) {
    const int u = min(static_cast<int>(threadIdx.x) + k * kSamplerRowThreads, last);
    w[k] = *reinterpret_cast<const u32x4_t*>(&row[u]);
  }
  float m = -INFINITY, sum = 0.f, best_v = -INFINITY;
  int best_i = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kSamplerRowUnits; ++k) {
    const int u = threadIdx.x + k * kSamplerRowThreads;
    if (u >= units) break;
    const float x[8] = {bf16_lo(w[k][0]), bf16_hi(w[k][0]), bf16_lo(w[k][1]), bf16_hi(w[k][1]),
                        bf16_lo(w[k][2]), bf16_hi(w[k][2]), bf16_lo(w[k][3]), bf16_hi(w[k][3])};
    float um = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      um = fmaxf(um, x[j] * sc);
      if (x[j] > best_v) {  // indices grow along a thread's walk: the first maximum stays
        best_v = x[j];
        best_i = 8 * u + j;
      }
    }
    const float M = fmaxf(m, um);
    if (M == -INFINITY) continue;  // everything so far is masked
    float t = m == -INFINITY ? 0.f : sum * fast_exp2(m - M);
#pragma unroll
    for (int j = 0; j < 8; ++j) t += fast_exp2(x[j] * sc - M);
    m = M;
    sum = t;
  }
  wave_merge(m, sum, best_v, best_i);
  __shared__ Partial sh[kRowWaves];
  const int lane = threadIdx.x & 63;
  if (lane == 0) sh[threadIdx.x >> 6] = Partial{m, sum, best_v, best_i};
  __syncthreads();
  // every wave merges the 16 partials (lanes past them hold empty ones, which
  // merge as nothing)
  Partial q = lane < kRowWaves ? sh[lane] : Partial{-INFINITY, 0.f, -INFINITY, 0x7fffffff};
  wave_merge(q.m, q.sum, q.best_v, q.best_i);
  const bool empty = q.m == -INFINITY;
  if (threadIdx.x == 0) {
    p.argmax[b] = empty ? 0 : q.best_i;
    if (p.lse) p.lse[b] = empty ? -INFINITY : (q.m + log2f(q.sum)) * kLn2;
  }
  if (!p.probs) return;
  const float invZ = empty ? 0.f : 1.0f / q.sum;
  float4* out = reinterpret_cast<float4*>(p.probs + static_cast<size_t>(b) * p.V);
#pragma unroll
  for (int k = 0; k < kSamplerRowUnits; ++k) {
    const int u = threadIdx.x + k * kSamplerRowThreads;
    if (u >= units) break;
    const float x[8] = {bf16_lo(w[k][0]), bf16_hi(w[k][0]), bf16_lo(w[k][1]), bf16_hi(w[k][1]),
                        bf16_lo(w[k][2]), bf16_hi(w[k][2]), bf16_lo(w[k][3]), bf16_hi(w[k][3])};
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = empty ? 0.f : fast_exp2(x[j] * sc - q.m) * invZ;
    const f32x4_t lo = {e[0], e[1], e[2], e[3]}, hi = {e[4], e[5], e[6], e[7]};
    *reinterpret_cast<f32x4_t*>(&out[2 * u]) = lo;
    *reinterpret_cast<f32x4_t*>(&out[2 * u + 1]) = hi;
  }
}

}  // namespace

bool plan_sampler(int B, int V, int form, SamplerPlan* plan) {
  SamplerPlan r{1, 0, 0, false};
  *plan = r;
  if (B <= 0 || V <= 0) return true;
  const int units = V / 8;
  // ranges: about 4 workgroups per CU over the batch, ranges of at least 512
  // units, and never more than kSamplerMaxUnits units (what the threads load
  // at once)
  int chunks = (kSamplerTargetWgs + B - 1) / B;
  const int max_chunks = (units + kSamplerMinUnits - 1) / kSamplerMinUnits;
  if (chunks > max_chunks) chunks = max_chunks;
  const int min_chunks = (units + kSamplerMaxUnits - 1) / kSamplerMaxUnits;
  if (chunks < min_chunks) chunks = min_chunks;
  if (chunks < 1) chunks = 1;
  r.chunks = chunks;
  r.chunk_units = (units + chunks - 1) / chunks;
  r.workspace_bytes = static_cast<size_t>(B) * chunks * sizeof(Partial);
  const bool row_fits = units <= kSamplerRowThreads * kSamplerRowUnits;
  if (form == 2 && !row_fits) return false;
  // automatic: rows in the last round of workgroups (one per CU); a round
  // with fewer than kSamplerRowMinBatch rows leaves most CUs idle through a
  // row's whole time
  const int last_round = B % kSamplerRowRound == 0 ? kSamplerRowRound : B % kSamplerRowRound;
  const bool row_pays = B >= kSamplerRowMinBatch && last_round >= kSamplerRowMinBatch;
  r.row_per_workgroup = form == 2 || (form == 0 && row_fits && row_pays);
  *plan = r;
  return true;
}

hipError_t launch_sampler(const SamplerArgs& a, hipStream_t stream) {
  SamplerParams p{};
  p.logits = static_cast<const uint16_t*>(a.logits);
  p.inv_temp = a.inv_temperature;
  p.probs = a.probs;
  p.lse = a.lse;
  p.argmax = a.argmax;
  p.part = static_cast<Partial*>(a.workspace);
  p.B = a.B;
  p.V = a.V;
  p.chunks = a.plan.chunks;
  p.chunk_units = a.plan.chunk_units;
  void* args[] = {&p};
  if (a.plan.row_per_workgroup) {
    if (a.B == 0) return hipSuccess;
    return hipLaunchKernel(reinterpret_cast<const void*>(&sampler_row_kernel), dim3(static_cast<unsigned>(a.B)),
                           dim3(kSamplerRowThreads), args, 0, stream);
  }
  const unsigned grid = static_cast<unsigned>(static_cast<long>(a.B) * p.chunks);
  if (grid == 0) return hipSuccess;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&sampler_partial_kernel), dim3(grid), dim3(kThreads),
                                 args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&sampler_write_kernel), dim3(grid), dim3(kThreads), args, 0,
                         stream);
}

}  // namespace fe
