// Top-B selection over the candidate pool, one workgroup per KV head.
//
// StateKV refreshes the compressed state by keeping the B candidates of the
// pool (previous state plus the frame's tokens) with the largest importance
// (paper.rainbus.top, method-steps section; paperlayer.ai section 3.3).  Ties
// go to the lower original position; because the pool is ordered by
// ascending position, that is the lower pool index.
//
// Scores are non-negative fp32, so their bit patterns order like the values
// (NaN and negative patterns are mapped to 0).  The threshold tau = the B-th
// largest key is found by an MSB-first radix select (four 8-bit digits, LDS
// histograms, a descending exclusive scan per digit).  The kept set is every
// key > tau plus the first k keys == tau in pool order, compacted with one
// block-wide scan so the output lists pool indices in ascending order.  Only
// integer operations decide the result, so it is exact and deterministic.
#include "../skv_internal.h"

namespace skv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ inline uint32_t score_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return u > 0x7F800000u ? 0u : u;  // NaN, -0 and negatives rank lowest
}

// Exclusive prefix sum over the workgroup (all threads must call it).
__device__ inline uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  if (w == 0) {
    uint32_t t = lane < kSelWaves ? sh[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kSelWaves; o <<= 1) {
      const uint32_t y = __shfl_up(t, o);
      if (lane >= o) t += y;
    }
    if (lane < kSelWaves) sh[lane] = t;
  }
  __syncthreads();
  const uint32_t base = w ? sh[w - 1] : 0u;
  __syncthreads();
  return base + v - x;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* sig_part, int rt,
                                                             int ldsig, int pool, int budget,
                                                             float* scores, int ldscores,
                                                             int32_t* sel, int ldsel) {
  extern __shared__ uint32_t keys[];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_sh[kSelWaves];
  __shared__ uint32_t found_digit, found_excl;
  const int h = blockIdx.x, tid = threadIdx.x;
  const float* sp = sig_part + (int64_t)h * rt * ldsig;
  int32_t* out = sel + (int64_t)h * ldsel;

  // importance = sum of the row tiles' partial column sums, in tile order
  for (int j = tid; j < pool; j += kSelThreads) {
    float acc = sp[j];
    for (int r = 1; r < rt; ++r) acc += sp[(int64_t)r * ldsig + j];
    if (scores) scores[(int64_t)h * ldscores + j] = acc;
    keys[j] = score_key(acc);
  }
  if (pool <= budget) {
    for (int j = tid; j < pool; j += kSelThreads) out[j] = j;
    return;
  }
  __syncthreads();

  uint32_t prefix = 0u, pmask = 0u;
  uint32_t k = (uint32_t)budget;  // rank (from the top) still to place
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int j = tid; j < pool; j += kSelThreads) {
      const uint32_t u = keys[j];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t cnt = tid < 256 ? hist[255 - tid] : 0u;  // descending digits
    const uint32_t excl = block_exclusive_scan(cnt, scan_sh);
    if (tid < 256 && excl < k && k <= excl + cnt) {
      found_digit = 255u - tid;
      found_excl = excl;
    }
    __syncthreads();
    prefix |= found_digit << shift;
    pmask |= 0xFFu << shift;
    k -= found_excl;
    __syncthreads();
  }
  // keep keys > tau, and the first k keys == tau in pool order
  const int per = (pool + kSelThreads - 1) / kSelThreads;
  const int j0 = min(pool, tid * per), j1 = min(pool, j0 + per);
  uint32_t ngt = 0u, neq = 0u;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = keys[j];
    ngt += u > prefix;
    neq += u == prefix;
  }
  const uint32_t packed = block_exclusive_scan(ngt | (neq << 16), scan_sh);
  const uint32_t gt_before = packed & 0xFFFFu, eq_before = packed >> 16;
  uint32_t slot = gt_before + min(eq_before, k);
  uint32_t eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = keys[j];
    if (u > prefix) {
      out[slot++] = j;
    } else if (u == prefix) {
      if (eqr < k) out[slot++] = j;
      ++eqr;
    }
  }
}

hipError_t launch_select(const float* sig_part, int rt, int ldsig, int hkv, int pool,
                         int budget, float* scores, int ldscores, int32_t* sel, int ldsel,
                         hipStream_t st) {
  static bool attr_set = false;
  const size_t lds = (size_t)pool * sizeof(uint32_t);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       kMaxPool * (int)sizeof(uint32_t));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(select_kernel, dim3(hkv), dim3(kSelThreads), lds, st, sig_part, rt, ldsig,
                     pool, budget, scores, ldscores, sel, ldsel);
  return hipGetLastError();
}

}  // namespace skv
