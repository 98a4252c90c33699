// Reference oracle for paged grouped-query attention over a block-allocated
// KV cache.  TEST INFRASTRUCTURE ONLY: it exists so that tests/, the smoke
// check and the benchmark's CPU-baseline leg can compare the HIP kernels with
// an obviously correct CPU computation.  Nothing in the product path may load,
// link or call it, and it shares no source with the HIP library.
//
// What it computes, and where the pages state it:
//   * ForgeEngine README (github.com/marcoharuni/forge-engine), table "What it
//     implements": the KV cache is a paged block allocator, and the kernels
//     include a CUDA paged GQA kernel and a restricted prefill lab.  Its
//     architecture flowchart puts the paged KV cache in a two-way exchange with
//     the explicit prefill/decode step: each step writes the new tokens' K/V
//     into the cache, then attends over it.
//   * "Make the Engine Talk" (inference-engine book, chapter 1), section 1.2:
//     one forward pass over the prompt primes the cache, then one pass per new
//     token; section 1.3 names grouped-query attention as one of the forward
//     pass's mechanisms.
// The pages print no formulas, layouts or values; the readings used here are:
//   * query head h uses KV head h / G, G = Hq / Hkv (contiguous groups);
//   * cache pools are [num_blocks][Hkv][BS][D] bf16, a slot is block*BS + off,
//     a negative slot is padding;
//   * attention is softmax(scale * q.K^T) V over the first L tokens of the
//     sequence (L counts the token appended this step), with the natural-log
//     log-sum-exp lse = log sum_t exp(scale * q.k_t);
//   * a prefill chunk of C queries ends at the sequence end: its row i sits at
//     position L - C + i and sees keys 0 .. L - C + i (bottom-right causal);
//   * L = 0 gives out = 0 and lse = -inf.
//
// The step before attention (the NEXT row after it): "Make the Engine Talk"
// section 1.3 names RMSNorm and rotary position embeddings among the forward
// pass's mechanisms, and the ForgeEngine README's "What it implements" table
// lists an RMSNorm kernel.  The pages give no formula; the readings here are
// per-head RMSNorm y = x w / sqrt(mean_d x^2 + eps) of each q and k head row
// (one weight vector of D entries for q, one for k), then the rotate-half
// rotary embedding: dims d and d + D/2 (d < D/2) turn by the angle whose
// cosine and sine the caller's table holds at [position][d] and
// [position][D/2 + d]; the result is rounded once to bf16 (nearest even).
//
// The sampler's hot step ("Make the Engine Talk" section 1.3: the sampler,
// greedy, temperature and top-p decoding, with its softmax in fp32 over the
// whole vocabulary; ForgeEngine README, "What it implements": sampling
// policies): per row of bf16 logits x and inverse temperature s,
// p_i = exp(s x_i - m) / sum_j exp(s x_j - m) with m = max_j s x_j, the
// natural-log lse = m + log sum_j exp(s x_j - m), and the greedy token
// argmax_i x_i (the lowest index among equal maxima; -inf entries are
// masked tokens; a row of only -inf gives p = 0, lse = -inf, argmax 0).
//
// Arithmetic: every bf16 value widens exactly to double; scale is the caller's
// value; dot products sum in increasing d, softmax sums in increasing t; the
// softmax is the two-pass max-shifted definition.  No blocking or reordering.
//
// Parity pins (tests/test_oracle.py) for the norm/rotary step: identity
// rotation gives unit mean square; a quarter turn and a half turn are exact
// permutations/negations of the identity result; scaling x by 2 changes
// nothing and scaling w by 2 doubles the result exactly; heads are
// independent; a one-hot row matches its closed form (tests/golden); and the
// bf16 rounding matches torch's float32 -> bfloat16 conversion where the value
// is a float32.
//
// Parity pins (tests/test_oracle.py): brute force on contiguous copies and
// torch's scaled_dot_product_attention in float64; block-table permutation
// invariance (bit-identical); weights summing to one; identical keys -> mean
// of V; q = 0 -> uniform; L = 1; a dominant key; equal queries in a group;
// prefill rows against decode and against masked SDPA; the split/merge
// identity; append against a NumPy scatter.
#include <cmath>
#include <cstdint>
#include <algorithm>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

// bf16 is the upper half of an IEEE binary32; widening is exact.
double widen_bf16(uint16_t bits) {
  uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, sizeof f);
  return static_cast<double>(f);
}

// Nearest-even bf16 of a double, rounded once from the double's value: 8
// significant bits in the normal range, spacing 2^-133 below it, infinity
// beyond the largest finite bf16.
uint16_t narrow_bf16(double v) {
  if (std::isnan(v)) return 0x7FC0;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);  // a = m 2^e, 0.5 <= m < 1
  const int shift = e - 1 >= -126 ? 8 - e : 133;  // units of the last kept bit
  const double r = std::nearbyint(std::ldexp(a, shift)) ;  // default rounding: nearest even
  const double q = std::ldexp(r, -shift);
  if (q >= 0x1p128) return sign | 0x7F80;
  const float f = static_cast<float>(q);  // exact: at most 8 significant bits
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return static_cast<uint16_t>(sign | ((u >> 16) & 0x7FFF));
}

struct Cache {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* block_table;  // one sequence's row
  int Hkv, D, BS;
  // element offset of token t of KV head g: block = table[t / BS], off = t % BS
  size_t offset(int t, int g) const {
    const int64_t blk = block_table[t / BS];
    const int off = t % BS;
    return ((static_cast<size_t>(blk) * Hkv + g) * BS + off) * static_cast<size_t>(D);
  }
};

// Attention of one query vector over tokens [t0, t1) of one sequence and one
// KV head.  Writes D outputs and the natural-log LSE.  An empty range gives
// out = 0, lse = -inf.
void attend(double* out, double* lse, const uint16_t* qrow, const Cache& c, int g, int t0, int t1,
            double scale) {
  const int D = c.D;
  if (t1 <= t0) {
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    *lse = -std::numeric_limits<double>::infinity();
    return;
  }
  std::vector<double> s(static_cast<size_t>(t1 - t0));
  for (int t = t0; t < t1; ++t) {
    const uint16_t* k = c.k + c.offset(t, g);
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += widen_bf16(qrow[d]) * widen_bf16(k[d]);
    s[t - t0] = scale * dot;
  }
  double m = s[0];
  for (int t = t0 + 1; t < t1; ++t)
    if (s[t - t0] > m) m = s[t - t0];
  double Z = 0.0;
  for (int t = t0; t < t1; ++t) {
    s[t - t0] = std::exp(s[t - t0] - m);  // s now holds the unnormalised weights
    Z += s[t - t0];
  }
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int t = t0; t < t1; ++t) {
    const uint16_t* v = c.v + c.offset(t, g);
    const double w = s[t - t0];
    for (int d = 0; d < D; ++d) out[d] += w * widen_bf16(v[d]);
  }
  for (int d = 0; d < D; ++d) out[d] /= Z;
  *lse = m + std::log(Z);
}

// Runs fn(i) for i in [0, n) over nthreads threads; each i is independent and
// its arithmetic does not depend on the thread count.
template <class F>
void parallel_for(int n, int nthreads, F fn) {
  if (nthreads <= 1 || n <= 1) {
    for (int i = 0; i < n; ++i) fn(i);
    return;
  }
  if (nthreads > n) nthreads = n;
  std::vector<std::thread> pool;
  pool.reserve(static_cast<size_t>(nthreads));
  for (int w = 0; w < nthreads; ++w)
    pool.emplace_back([=]() {
      for (int i = w; i < n; i += nthreads) fn(i);
    });
  for (auto& th : pool) th.join();
}

int check_shape(int Hq, int Hkv, int D, int BS) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0) return -2;
  if (Hq % Hkv != 0) return -2;
  return 0;
}

}  // namespace

extern "C" {

// KV append: for each new token i with slot s = slot_mapping[i] >= 0, copy the
// D-element rows k_new[i][g][:] and v_new[i][g][:] of every KV head g into
// block s / BS, offset s % BS of the pools.  Pure bit copy; every other byte of
// the pools is left as it was.  Slots at or beyond num_blocks*BS are ignored.
void oracle_append(const uint16_t* k_new, const uint16_t* v_new, const int32_t* slot_mapping, int T,
                   uint16_t* k_cache, uint16_t* v_cache, int num_blocks, int Hkv, int D, int BS) {
  const int64_t nslots = static_cast<int64_t>(num_blocks) * BS;
  for (int i = 0; i < T; ++i) {
    const int64_t s = slot_mapping[i];
    if (s < 0 || s >= nslots) continue;
    const int64_t blk = s / BS;
    const int off = static_cast<int>(s % BS);
    for (int g = 0; g < Hkv; ++g) {
      const size_t dst = ((static_cast<size_t>(blk) * Hkv + g) * BS + off) * static_cast<size_t>(D);
      const size_t src = (static_cast<size_t>(i) * Hkv + g) * static_cast<size_t>(D);
      for (int d = 0; d < D; ++d) {
        k_cache[dst + d] = k_new[src + d];
        v_cache[dst + d] = v_new[src + d];
      }
    }
  }
}

// Decode: one query token per sequence.  out [B][Hq][D] and lse [B][Hq] are
// double; q is bf16 [B][Hq][D]; block_tables is [B][max_blocks_per_seq].
// Sequence b attends over its first context_lens[b] tokens.
int oracle_decode(double* out, double* lse, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* block_tables, int max_blocks_per_seq,
                  const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS, double scale,
                  int nthreads) {
  if (int rc = check_shape(Hq, Hkv, D, BS)) return rc;
  const int G = Hq / Hkv;
  parallel_for(B * Hq, nthreads, [&](int i) {
    const int b = i / Hq, h = i % Hq;
    const Cache c{k_cache, v_cache, block_tables + static_cast<size_t>(b) * max_blocks_per_seq, Hkv, D,
                  BS};
    const size_t row = static_cast<size_t>(b) * Hq + h;
    attend(out + row * D, lse + row, q + row * D, c, h / G, 0, context_lens[b], scale);
  });
  return 0;
}

// Decode restricted to the token ranges [p*S, min((p+1)*S, L)) for p in
// [0, P): out_part [B][Hq][P][D], lse_part [B][Hq][P].  Used only to check the
// split-K merge rule against the unsplit definition.
int oracle_decode_split(double* out_part, double* lse_part, const uint16_t* q, const uint16_t* k_cache,
                        const uint16_t* v_cache, const int32_t* block_tables, int max_blocks_per_seq,
                        const int32_t* context_lens, int B, int Hq, int Hkv, int D, int BS, double scale,
                        int S, int P, int nthreads) {
  if (int rc = check_shape(Hq, Hkv, D, BS)) return rc;
  if (S <= 0 || P <= 0) return -2;
  const int G = Hq / Hkv;
  parallel_for(B * Hq * P, nthreads, [&](int i) {
    const int p = i % P, bh = i / P;
    const int b = bh / Hq, h = bh % Hq;
    const Cache c{k_cache, v_cache, block_tables + static_cast<size_t>(b) * max_blocks_per_seq, Hkv, D,
                  BS};
    const int L = context_lens[b];
    int t0 = p * S, t1 = (p + 1) * S;
    if (t1 > L) t1 = L;
    if (t0 > L) t0 = L;
    attend(out_part + static_cast<size_t>(i) * D, lse_part + i, q + static_cast<size_t>(bh) * D, c, h / G,
           t0, t1, scale);
  });
  return 0;
}

// Log-sum-exp merge of P partial results per row: lse = M + log sum_p
// exp(lse_p - M) with M = max_p lse_p, out = sum_p exp(lse_p - lse) out_p.
// Partials with lse_p = -inf carry weight 0; all rows empty -> out 0, lse -inf.
void oracle_merge(double* out, double* lse, const double* out_part, const double* lse_part, int rows, int P,
                  int D) {
  const double ninf = -std::numeric_limits<double>::infinity();
  for (int r = 0; r < rows; ++r) {
    const double* lp = lse_part + static_cast<size_t>(r) * P;
    double M = ninf;
    for (int p = 0; p < P; ++p)
      if (lp[p] > M) M = lp[p];
    double* o = out + static_cast<size_t>(r) * D;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (M == ninf) {
      lse[r] = ninf;
      continue;
    }
    double Z = 0.0;
    for (int p = 0; p < P; ++p)
      if (lp[p] != ninf) Z += std::exp(lp[p] - M);
    lse[r] = M + std::log(Z);
    for (int p = 0; p < P; ++p) {
      if (lp[p] == ninf) continue;
      const double w = std::exp(lp[p] - lse[r]);
      const double* op = out_part + (static_cast<size_t>(r) * P + p) * D;
      for (int d = 0; d < D; ++d) o[d] += w * op[d];
    }
  }
}

// Prefill chunk: q is bf16 [total_q][Hq][D], packed by query_start_loc [B+1].
// Sequence b owns rows qsl[b] .. qsl[b+1]-1 (C_b rows); row qsl[b] + i attends
// over tokens 0 .. L_b - C_b + i, i.e. as a decode with L = L_b - C_b + i + 1.
// If rows is non-null only those n_rows packed rows are computed (out and lse
// are then [n_rows][Hq][D] and [n_rows][Hq]); otherwise every row.
int oracle_prefill_chunk(double* out, double* lse, const uint16_t* q, const int32_t* query_start_loc,
                         const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* block_tables,
                         int max_blocks_per_seq, const int32_t* context_lens, int B, int total_q, int Hq,
                         int Hkv, int D, int BS, double scale, const int32_t* rows, int n_rows,
                         int nthreads) {
  if (int rc = check_shape(Hq, Hkv, D, BS)) return rc;
  const int G = Hq / Hkv;
  const int nr = rows ? n_rows : total_q;
  // sequence of each packed row
  std::vector<int> seq_of(static_cast<size_t>(total_q), -1);
  for (int b = 0; b < B; ++b)
    for (int r = query_start_loc[b]; r < query_start_loc[b + 1] && r < total_q; ++r)
      if (r >= 0) seq_of[static_cast<size_t>(r)] = b;
  parallel_for(nr * Hq, nthreads, [&](int i) {
    const int k = i / Hq, h = i % Hq;
    const int r = rows ? rows[k] : k;
    double* o = out + static_cast<size_t>(i) * D;
    const int b = (r >= 0 && r < total_q) ? seq_of[static_cast<size_t>(r)] : -1;
    if (b < 0) {
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      lse[i] = -std::numeric_limits<double>::infinity();
      return;
    }
    const int C = query_start_loc[b + 1] - query_start_loc[b];
    const int pos = context_lens[b] - C + (r - query_start_loc[b]);
    const Cache c{k_cache, v_cache, block_tables + static_cast<size_t>(b) * max_blocks_per_seq, Hkv, D,
                  BS};
    attend(o, lse + i, q + (static_cast<size_t>(r) * Hq + h) * D, c, h / G, 0, pos + 1, scale);
  });
  return 0;
}

// Per-head RMSNorm and rotary embedding of rows x [T][H][D] (bf16), written
// as bf16 to out [T][H][D].  w: [D] bf16 norm weights; cos_sin: [max_pos][D]
// fp32 (cosines of the D/2 angles, then their sines); positions: [T], each
// clamped into [0, max_pos).  Returns 0, or -1 for odd D or bad sizes.
int oracle_qk_norm_rope(uint16_t* out, const uint16_t* x, const uint16_t* w, const float* cos_sin, int max_pos,
                        const int32_t* positions, int T, int H, int D, double eps, int nthreads) {
  if (T < 0 || H <= 0 || D <= 0 || D % 2 != 0 || max_pos <= 0) return -1;
  const int half = D / 2;
  parallel_for(T * H, nthreads, [&](int th) {
    const int t = th / H;
    const uint16_t* row = x + static_cast<size_t>(th) * D;
    double ss = 0.0;
    for (int d = 0; d < D; ++d) {
      const double v = widen_bf16(row[d]);
      ss += v * v;
    }
    const double inv_rms = 1.0 / std::sqrt(ss / D + eps);
    std::vector<double> y(D);
    for (int d = 0; d < D; ++d) y[d] = widen_bf16(row[d]) * inv_rms * widen_bf16(w[d]);
    int p = positions[t];
    p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
    const float* cs = cos_sin + static_cast<size_t>(p) * D;
    uint16_t* o = out + static_cast<size_t>(th) * D;
    for (int d = 0; d < half; ++d) {
      const double c = cs[d], s = cs[half + d];
      o[d] = narrow_bf16(y[d] * c - y[half + d] * s);
      o[half + d] = narrow_bf16(y[half + d] * c + y[d] * s);
    }
  });
  return 0;
}

// Softmax, log-sum-exp and greedy argmax of each row of bf16 logits
// [B][V] at inverse temperature inv_temp[b] (> 0; NULL = 1).  probs may be
// NULL.  Returns 0, or -1 for bad sizes.
int oracle_sampler(double* probs, double* lse, int32_t* argmax, const uint16_t* logits, const float* inv_temp, int B,
                   int V, int nthreads) {
  if (B < 0 || V <= 0) return -1;
  parallel_for(B, nthreads, [&](int b) {
    const uint16_t* x = logits + static_cast<size_t>(b) * V;
    const double s = inv_temp ? static_cast<double>(inv_temp[b]) : 1.0;
    int best = 0;
    double bestv = widen_bf16(x[0]);
    for (int i = 1; i < V; ++i) {
      const double v = widen_bf16(x[i]);
      if (v > bestv) {
        bestv = v;
        best = i;
      }
    }
    argmax[b] = best;
    double m = -std::numeric_limits<double>::infinity();
    for (int i = 0; i < V; ++i) m = std::max(m, s * widen_bf16(x[i]));
    if (m == -std::numeric_limits<double>::infinity()) {  // every token masked
      lse[b] = m;
      if (probs)
        for (int i = 0; i < V; ++i) probs[static_cast<size_t>(b) * V + i] = 0.0;
      return;
    }
    double Z = 0.0;
    for (int i = 0; i < V; ++i) Z += std::exp(s * widen_bf16(x[i]) - m);
    lse[b] = m + std::log(Z);
    if (probs)
      for (int i = 0; i < V; ++i) probs[static_cast<size_t>(b) * V + i] = std::exp(s * widen_bf16(x[i]) - m) / Z;
  });
  return 0;
}

// The narrowing used above, exposed for its pin.
uint16_t oracle_narrow_bf16(double v) { return narrow_bf16(v); }

}  // extern "C"
