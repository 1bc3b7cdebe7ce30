// The App. A measurements of one frame (paperlayer.ai, App. A.1-A.3), on a
// layer that keeps every token, from the importance its last frame computed.
//
// The pages run unmodified full attention frame by frame and aggregate the
// current frame's video-only attention over the layer's heads and queries.
// A layer whose budget covers the whole history never evicts, so its step is
// exactly that full attention and its importance rows are those aggregates
// per KV head; summed over the KV heads they give the layer-wide importance s
// of every token through the frame (tokens [0, c) from earlier frames).  For
// each budget b one workgroup computes
//   A.1  the share of the historical mass sum_{j<c} s_j held by the b largest
//        historical s_j (ties do not matter: equal values, equal mass);
//   A.3  the share held by the b most recent historical tokens;
//   A.2  the kept set S_n = top-b of all tokens (ties to the lower position),
//        and the share of its mass inside the candidate pool S_{n-1} + frame,
//        S_{n-1} being the set the previous call stored; then stores S_n.
// Thresholds come from a bitwise search for the b-th largest key (scores are
// non-negative fp32, so their bit patterns order like the values); every sum
// runs in a fixed order, so the results are reproducible.  Not on the
// per-frame path: one call per frame when the diagnostics are wanted.
#include "../skv_internal.h"

namespace skv {

constexpr int kDiagThreads = 1024;
constexpr int kDiagWaves = kDiagThreads / 64;

__device__ inline uint32_t diag_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return u > 0x7F800000u ? 0u : u;  // NaN, -0 and negatives rank lowest
}

// Sum over the workgroup of one value per thread, in a fixed order (DPP-free:
// waves add their lanes in a fixed butterfly, thread 0 adds the waves in order).
template <class V>
__device__ inline V block_sum(V x, V* sh) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w] = x;
  __syncthreads();
  V t = sh[0];
  for (int i = 1; i < kDiagWaves; ++i) t += sh[i];
  __syncthreads();
  return t;
}

// Exclusive prefix sum (index order of the threads) and total.
__device__ inline uint32_t block_scan(uint32_t x, uint32_t* sh, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t v = x;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int i = 0; i < kDiagWaves; ++i) {
    if (i < w) base += sh[i];
    tot += sh[i];
  }
  __syncthreads();
  *total = tot;
  return base + v - x;
}

__global__ __launch_bounds__(kDiagThreads) void attention_mass_kernel(MassArgs m) {
  extern __shared__ float s[];  // layer-wide importance of the pool
  __shared__ uint32_t kept_bits[kMaxPool / 32];
  __shared__ float shf[kDiagWaves];
  __shared__ uint32_t shu[kDiagWaves];
  const int tid = threadIdx.x;
  const int pool = m.pool, c = m.c;
  const int b = m.budgets[blockIdx.x];

  for (int j = tid; j < pool; j += kDiagThreads) {
    float v = m.scores[j];
    for (int h = 1; h < m.Hkv; ++h) v += m.scores[(int64_t)h * m.ldscores + j];
    s[j] = v;
  }
  for (int w = tid; w < (pool + 31) / 32; w += kDiagThreads) kept_bits[w] = 0u;
  __syncthreads();

  // contiguous chunk per thread: sums and ranks in index order
  const int per = (pool + kDiagThreads - 1) / kDiagThreads;
  const int j0 = min(pool, tid * per), j1 = min(pool, j0 + per);
  auto sum_range = [&](int lo, int hi) {  // sum of s over [lo, hi)
    float acc = 0.f;
    for (int j = max(j0, lo); j < min(j1, hi); ++j) acc += s[j];
    return block_sum(acc, shf);
  };
  auto count_ge = [&](int hi, uint32_t t) {  // #{j < hi : key_j >= t}
    uint32_t n = 0;
    for (int j = j0; j < min(j1, hi); ++j) n += diag_key(s[j]) >= t;
    return block_sum(n, shu);
  };
  // the bb-th largest key over [0, hi), bb >= 1
  auto kth_key = [&](int hi, int bb) {
    uint32_t t = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (count_ge(hi, cand) >= (uint32_t)bb) t = cand;
    }
    return t;
  };
  auto sum_above = [&](int hi, uint32_t t) {  // sum of s_j, j < hi, key_j > t
    float acc = 0.f;
    for (int j = j0; j < min(j1, hi); ++j)
      if (diag_key(s[j]) > t) acc += s[j];
    return block_sum(acc, shf);
  };

  float topb = __builtin_nanf(""), recency = __builtin_nanf("");
  if (c > 0) {
    const int bb = min(b, c);
    const float total = sum_range(0, c);
    const uint32_t t1 = kth_key(c, bb);
    const uint32_t gt = t1 == 0xFFFFFFFFu ? 0u : count_ge(c, t1 + 1u);
    const float above = t1 == 0xFFFFFFFFu ? 0.f : sum_above(c, t1);
    const float top = above + (float)(bb - (int)gt) * __builtin_bit_cast(float, t1);
    const float recent = sum_range(c - bb, c);
    if (total > 0.f) {
      topb = top / total;
      recency = recent / total;
    }
  }

  // A.2: S_n = top-b of the whole pool, ties to the lower position
  const int bb2 = min(b, pool);
  const uint32_t t2 = kth_key(pool, bb2);
  const uint32_t gt2 = t2 == 0xFFFFFFFFu ? 0u : count_ge(pool, t2 + 1u);
  const uint32_t take = (uint32_t)bb2 - gt2;  // keys equal to t2 to keep
  uint32_t neq = 0;
  for (int j = j0; j < j1; ++j) neq += diag_key(s[j]) == t2;
  uint32_t eq_total;
  uint32_t eqr = block_scan(neq, shu, &eq_total);
  const uint32_t* prev = m.sets + (int64_t)blockIdx.x * m.ldsets;
  float kept_mass = 0.f, recalled = 0.f;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = diag_key(s[j]);
    bool kept = u > t2;
    if (u == t2) kept = eqr++ < take;
    if (!kept) continue;
    atomicOr(&kept_bits[j >> 5], 1u << (j & 31));
    kept_mass += s[j];
    const bool in_pool = j >= c || !m.have_prev || ((prev[j >> 5] >> (j & 31)) & 1u);
    if (in_pool) recalled += s[j];
  }
  kept_mass = block_sum(kept_mass, shf);   // its barriers also order the bit writes
  recalled = block_sum(recalled, shf);
  uint32_t* dst = m.sets + (int64_t)blockIdx.x * m.ldsets;
  for (int w = tid; w < (pool + 31) / 32; w += kDiagThreads) dst[w] = kept_bits[w];
  if (tid == 0) {
    float* o = m.out + 3 * blockIdx.x;
    o[0] = topb;
    o[1] = recency;
    o[2] = kept_mass > 0.f ? recalled / kept_mass : __builtin_nanf("");
  }
}

hipError_t launch_attention_mass(const MassArgs& m, int n_budgets, const Stream& st) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(attention_mass_kernel), kMaxPool * (int)sizeof(float), lds_set);
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL(attention_mass_kernel, dim3(n_budgets), dim3(kDiagThreads),
                        (size_t)m.pool * sizeof(float), st.st, st.start, st.stop, 0, m);
  return hipGetLastError();
}

}  // namespace skv
