// Top-B selection over the candidate pool, one workgroup per KV head, in the
// same launch as the fixed-order sum of the attention's split O partials.
//
// StateKV refreshes the compressed state by keeping the B candidates of the
// pool (previous state plus the frame's tokens) with the largest importance
// (paper.rainbus.top, method-steps section; paperlayer.ai section 3.3).  Ties
// go to the lower original position; because the pool is ordered by
// ascending position, that is the lower pool index.
//
// Scores are non-negative fp32, so their bit patterns order like the values
// (NaN and negative patterns are mapped to 0).  The threshold is found by an
// MSB-first radix select over the bits below the highest bit in which the
// pool's keys differ (so the first 12-bit digit already spreads the keys over
// the histogram), with one 4096-bin LDS histogram per digit: each thread
// owns four bins, reads and clears them after the counting, and one
// workgroup scan over the bins finds the boundary bin (three barriers per
// digit; at most three digits).  After each digit, if every key of the
// boundary bin is needed the search stops early.  The kept set is every key above the boundary plus the
// first k keys of the boundary bin in pool order, compacted with one
// workgroup scan so the output lists pool indices in ascending order.  Only
// integer operations decide the result: exact and deterministic.
//
// With the in-place (slot-stable) state update the state rows are in no
// position order.  Exact ties at the boundary are then broken by a second
// radix select over keys that rank the tied candidates by age (older = lower
// position = preferred) above everything dropped and below everything kept
// outright; the output is the list of rows to refill (evicted rows in row
// order, then the unused rows while C fills) and the kept frame tokens in
// frame order.  The recency window ranks the candidates by position the same
// way.  The selecting workgroup then copies those frame tokens into their
// rows itself (at most T rows per head), and extra workgroups of the launch
// append the frame to the detailed cache, so the in-place step needs no
// separate state-update launch.
#include "../skv_internal.h"

namespace skv {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline uint32_t score_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return u > 0x7F800000u ? 0u : u;  // NaN, -0 and negatives rank lowest
}

// Workgroup barrier that orders LDS only.  __syncthreads also makes each
// wave's global stores visible first, i.e. waits for them to complete (the
// importance row written right after the score sums would hold up the next
// barrier by a memory round trip); nothing in the selecting workgroup reads
// back global memory that another thread of it wrote, except the move lists
// when they do not fit in LDS (that barrier stays a full one).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wave-level primitives on DPP (every lane of the wave active).
// Inclusive prefix sum over the 64 lanes: Hillis-Steele within each 16-lane
// row (row_shr 1, 2, 4, 8, zero fill), then row 0 / 2 totals into rows 1 / 3
// (row_bcast:15) and the rows-0-1 total into rows 2-3 (row_bcast:31).
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, true);
}
__device__ inline uint32_t wave_inclusive_sum(uint32_t v) {
  v += dpp_u32<0x111, 0xF>(v);
  v += dpp_u32<0x112, 0xF>(v);
  v += dpp_u32<0x114, 0xF>(v);
  v += dpp_u32<0x118, 0xF>(v);
  v += dpp_u32<0x142, 0xA>(v);
  v += dpp_u32<0x143, 0xC>(v);
  return v;
}
// Minimum and maximum over the 64 lanes (result read from lane 63); lanes
// without a DPP source keep their own value.
template <int CTRL, int ROWS>
__device__ inline uint32_t dpp_keep(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xF, false);
}
__device__ inline void wave_min_max(uint32_t& mn, uint32_t& mx) {
#define SKV_STEP(C, R)            \
  mn = min(mn, dpp_keep<C, R>(mn)); \
  mx = max(mx, dpp_keep<C, R>(mx));
  SKV_STEP(0x111, 0xF)
  SKV_STEP(0x112, 0xF)
  SKV_STEP(0x114, 0xF)
  SKV_STEP(0x118, 0xF)
  SKV_STEP(0x142, 0xA)
  SKV_STEP(0x143, 0xC)
#undef SKV_STEP
  mn = (uint32_t)__builtin_amdgcn_readlane((int)mn, 63);
  mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
}

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ inline uint32_t block_exclusive_scan(uint32_t x, uint32_t* sh, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t v = wave_inclusive_sum(x);
  if (lane == 63) sh[w] = v;
  lds_barrier();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSelWaves; ++i) {
    const uint32_t s = sh[i];
    if (i < w) base += s;
    tot += s;
  }
  lds_barrier();
  if (total) *total = tot;
  return base + v - x;
}

__device__ inline uint32_t block_min_max(uint32_t mn, uint32_t mx, uint32_t* sh, uint32_t* out_max) {
  wave_min_max(mn, mx);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh[w] = mn;
    sh[kSelWaves + w] = mx;
  }
  lds_barrier();
  uint32_t a = sh[0], b = sh[kSelWaves];
#pragma unroll
  for (int i = 1; i < kSelWaves; ++i) {
    a = min(a, sh[i]);
    b = max(b, sh[kSelWaves + i]);
  }
  lds_barrier();
  *out_max = b;
  return a;
}

struct SelectJob {
  const float* sig_part;  // [Hkv][rt][ldsig] partial scores (rt = 1: plain scores)
  int rt, ldsig, pool, budget;
  float* scores;          // [Hkv][ldscores] summed scores (may be null)
  int ldscores;
  int32_t* sel;           // [Hkv][ldsel] kept pool indices, ascending
  int ldsel;
  int recent;             // keep the last min(pool, budget) entries (most recent)
  InPlace ip;             // ip.pos null: the pool is in position order
  int all_heads;          // the layer-wide job: its selection serves every head
  int groups;             // row groups summed in turn (the layer-wide job: one per KV head,
                          // rt rows each, consecutive), 1 otherwise
};

// In place, the move lists live in LDS past the pool's keys when they fit.
__host__ __device__ inline bool in_place_lds_fits(int pool, int T) {
  return (int64_t)pool + 2 * (int64_t)T <= kMaxPool;
}

// In place: copies M moved frame tokens of heads [h0, h1) into their state
// rows (K and V rows, 16-byte chunks, up to kMoveU loads in flight per
// thread) and writes their positions.  Move r goes to row mv[r] and comes
// from frame token mv[T + r]; mv null: rows c + r from token r (the frame is
// appended while C fills).  A move whose row or token lies outside C or the
// frame is skipped: the lists never hold one, and a broken list must not turn
// into stores outside the state.
constexpr int kMoveU = 8;
__device__ void apply_moves(const InPlace& ip, const int32_t* mv, int M, int h0, int h1) {
  const int tid = threadIdx.x;
  const int nh = h1 - h0;
  auto dst_of = [&](int r) { return mv ? mv[r] : ip.c + r; };
  auto src_of = [&](int r) { return mv ? mv[ip.T + r] : r; };
  auto valid = [&](int d, int t) {
    return (unsigned)d < (unsigned)ip.ldpos && (unsigned)t < (unsigned)ip.T;
  };
  for (int i = tid; i < nh * M; i += kSelThreads) {
    const int h = h0 + i / M, r = i % M;
    const int d = dst_of(r), t = src_of(r);
    if (valid(d, t)) ip.pos[(int64_t)h * ip.ldpos + d] = ip.frame_pos0 + t;
  }
  if (!ip.kc) return;  // the state is kept as positions into D
  const int CH = ip.D / 8;
  const int64_t items = (int64_t)nh * M * 2 * CH;  // (head, move, K/V, chunk), chunk fastest
  for (int64_t base = 0; base < items; base += kMoveU * kSelThreads) {
    u32x4 buf[kMoveU];
    uint16_t* dst[kMoveU];
#pragma unroll
    for (int u = 0; u < kMoveU; ++u) {
      const int64_t it = base + u * kSelThreads + tid;
      dst[u] = nullptr;
      if (it < items) {
        const int ch = (int)(it % CH);
        const int64_t rest = it / CH;
        const int which = (int)(rest & 1);
        const int64_t mr = rest >> 1;
        const int h = h0 + (int)(mr / M), r = (int)(mr % M);
        const int d = dst_of(r), t = src_of(r);
        if (valid(d, t)) {
          const int64_t src = ((int64_t)t * ip.Hkv + h) * ip.D + ch * 8;
          buf[u] = *reinterpret_cast<const u32x4*>((which ? ip.vf : ip.kf) + src);
          dst[u] = (which ? ip.vc : ip.kc) + ((int64_t)h * ip.ldpos + d) * ip.D + ch * 8;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kMoveU; ++u)
      if (dst[u]) *reinterpret_cast<u32x4*>(dst[u]) = buf[u];
  }
}

struct SumJob {
  const f32x4* part;      // [S][n4] split partials (already unscaled)
  void* out;              // [n4] f32x4, or [n4] x 4 bf16 when bf16
  int64_t n4;
  int S;
  int bf16;
  int delay;  // s_sleep(32) rounds (about 0.85 us each at 2.4 GHz) before the sum starts
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ void select_one_head(const SelectJob& J, int h) {
  extern __shared__ uint32_t keys[];
  // one digit histogram of 12-bit digits for the whole workgroup
  constexpr int kDigitBits = 12;
  constexpr int kBins = 1 << kDigitBits;
  constexpr int kBinsPerThread = kBins / kSelThreads;
  static_assert(kBinsPerThread * kSelThreads == kBins, "bins split evenly");
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t red[2 * kSelWaves];
  __shared__ uint32_t found[3];
  const int tid = threadIdx.x, w = tid >> 6;
  const int pool = J.pool, budget = J.budget;
  const float* sp = J.sig_part + (int64_t)h * J.rt * J.ldsig;
  const bool in_place = J.sel && J.ip.pos != nullptr;
  const bool lists_lds = in_place && in_place_lds_fits(pool, J.ip.T);

  // importance = sum of the row tiles' partial column sums, in tile order
  // (fp32); the layer-wide job adds the KV heads' sums in head order, so its
  // value is exactly the fp32 sum of the per-head importances.  Every load of
  // a batch (kLoad candidates x kRows row tiles per thread) is in flight at
  // once.
  constexpr int kLoad = 5;  // 5 * 1024 >= 4352: one round at the 8B-like shape
  constexpr int kRows = 8;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int j0 = 0; j0 < pool; j0 += kLoad * kSelThreads) {
    float tot[kLoad];
    for (int g = 0; g < J.groups; ++g) {
      const float* gp = sp + (int64_t)g * J.rt * J.ldsig;
      float acc[kLoad];
#pragma unroll
      for (int q = 0; q < kLoad; ++q) acc[q] = 0.f;
      for (int r0 = 0; r0 < J.rt; r0 += kRows) {
        float part[kRows][kLoad];
#pragma unroll
        for (int u = 0; u < kRows; ++u) {
          // the row's base is uniform, each lane adds a 32-bit byte offset
          const char* row =
              reinterpret_cast<const char*>(gp + (int64_t)min(r0 + u, J.rt - 1) * J.ldsig);
#pragma unroll
          for (int q = 0; q < kLoad; ++q) {
            const uint32_t j = (uint32_t)min(j0 + tid + q * kSelThreads, pool - 1);
            part[u][q] = *reinterpret_cast<const float*>(row + j * 4u);
          }
        }
#pragma unroll
        for (int u = 0; u < kRows; ++u)
#pragma unroll
          for (int q = 0; q < kLoad; ++q)
            if (r0 + u < J.rt) acc[q] = r0 + u == 0 ? part[u][q] : acc[q] + part[u][q];
      }
#pragma unroll
      for (int q = 0; q < kLoad; ++q) tot[q] = g == 0 ? acc[q] : tot[q] + acc[q];
    }
    float* acc = tot;
#pragma unroll
    for (int q = 0; q < kLoad; ++q) {
      const int j = j0 + tid + q * kSelThreads;
      if (j < pool) {
        if (J.scores) J.scores[(int64_t)h * J.ldscores + j] = acc[q];
        const uint32_t u = score_key(acc[q]);
        keys[j] = u;
        mn = min(mn, u);
        mx = max(mx, u);
      }
    }
  }
  if (!J.sel) return;  // scores only (per-head rows of the SHARED mode)
  int32_t* out = J.sel + (int64_t)h * J.ldsel;
  // heads whose rows this job updates (the layer-wide job: every head)
  const int mh0 = J.all_heads ? 0 : h, mh1 = J.all_heads ? J.ip.Hkv : h + 1;
  if (pool <= budget) {  // nothing is dropped
    if (!in_place)
      for (int j = tid; j < pool; j += kSelThreads) out[j] = j;
    else
      apply_moves(J.ip, nullptr, J.ip.T, mh0, mh1);  // the frame joins C at rows c..
    return;
  }
  if (J.recent && !in_place) {  // the pool is in position order: the newest entries are last
    const int keepn = min(pool, budget);
    for (int s = tid; s < keepn; s += kSelThreads) out[s] = pool - keepn + s;
    return;
  }
  // age of pool entry j in positions (0: the frame's last token), clamped so
  // that 1 + age fits below the all-ones key
  const int64_t* hpos = in_place ? J.ip.pos + (int64_t)h * J.ip.ldpos : nullptr;
  const int64_t newest = J.ip.frame_pos0 + J.ip.T - 1;
  auto age = [&](int j) -> uint32_t {
    const int64_t p = j < J.ip.c ? hpos[j] : J.ip.frame_pos0 + (j - J.ip.c);
    const uint64_t a = (uint64_t)(newest - p);
    return a < 0xFFFFFFFDull ? (uint32_t)a : 0xFFFFFFFDu;
  };
  if (J.recent) {  // in place: rank by position, newest first (same thread owns key j)
    mn = 0xFFFFFFFFu;
    mx = 0u;
    for (int j = tid; j < pool; j += kSelThreads) {
      const uint32_t u = 0xFFFFFFFEu - age(j);
      keys[j] = u;
      mn = min(mn, u);
      mx = max(mx, u);
    }
  }
  // the histogram starts cleared (the min/max barrier orders the clears)
  for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0u;
  uint32_t kmax;
  uint32_t kmin = block_min_max(mn, mx, red, &kmax);  // also orders keys[] writes

  const int lane = tid & 63;
  uint32_t prefix, pmask, k;
  // MSB-first radix select below the common prefix of all keys, 12-bit
  // digits.  Per pass: count the keys that match the prefix by digit; thread
  // tid owns the digits dmask - 4 tid - e (e < 4, highest first), reads and
  // clears them (so every bin is zero again when the pass ends) and a
  // workgroup scan of the owners' sums finds the boundary digit.  Returns the
  // boundary bin's size; k is then the number of its keys to keep.
  auto radix = [&]() -> uint32_t {
    prefix = kmin;
    pmask = 0xFFFFFFFFu;
    k = (uint32_t)budget;  // rank (from the top) still to place
    int hb = kmin == kmax ? -1 : 31 - __builtin_clz(kmin ^ kmax);
    if (hb >= 0) {
      pmask = hb == 31 ? 0u : ~((2u << hb) - 1u);
      prefix = kmin & pmask;
    }
    uint32_t bin = (uint32_t)pool;
    while (hb >= 0) {
      const int shift = hb >= kDigitBits - 1 ? hb - (kDigitBits - 1) : 0;
      const uint32_t dmask = (2u << (hb - shift)) - 1u;  // digit bits [shift, hb]
      for (int j = tid; j < pool; j += kSelThreads) {
        const uint32_t u = keys[j];
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & dmask], 1u);
      }
      lds_barrier();
      uint32_t cnt[kBinsPerThread], tsum = 0;
#pragma unroll
      for (int e = 0; e < kBinsPerThread; ++e) {
        const int d = (int)dmask - kBinsPerThread * tid - e;
        cnt[e] = 0;
        if (d >= 0) {
          cnt[e] = hist[d];
          hist[d] = 0u;
        }
        tsum += cnt[e];
      }
      const uint32_t incl = wave_inclusive_sum(tsum);
      if (lane == 63) red[w] = incl;
      lds_barrier();
      uint32_t excl = incl - tsum;
      for (int i = 0; i < w; ++i) excl += red[i];
#pragma unroll
      for (int e = 0; e < kBinsPerThread; ++e) {
        if (cnt[e] && excl < k && k <= excl + cnt[e]) {
          found[0] = dmask - (uint32_t)(kBinsPerThread * tid + e);
          found[1] = excl;
          found[2] = cnt[e];
        }
        excl += cnt[e];
      }
      lds_barrier();
      prefix |= found[0] << shift;
      pmask |= dmask << shift;
      k -= found[1];
      bin = found[2];
      if (bin == k) break;  // the whole boundary bin is kept: no tie to break
      hb = shift - 1;
    }
    return bin;
  };
  uint32_t bin = radix();
  if (in_place && bin > k) {
    // exact ties at the boundary (every key bit resolved): keep the k oldest
    // of them, by a second select over 0 (dropped) < 1 + age (tied) < ~0 (kept)
    mn = 0xFFFFFFFFu;
    mx = 0u;
    for (int j = tid; j < pool; j += kSelThreads) {
      const uint32_t u = keys[j];
      const uint32_t v = u > prefix ? 0xFFFFFFFFu : u < prefix ? 0u : 1u + age(j);
      keys[j] = v;
      mn = min(mn, v);
      mx = max(mx, v);
    }
    kmin = block_min_max(mn, mx, red, &kmax);
    bin = radix();
  }

  // keep (u & pmask) > prefix, and the first k keys with (u & pmask) == prefix
  const int per = (pool + kSelThreads - 1) / kSelThreads;
  const int j0 = min(pool, tid * per), j1 = min(pool, j0 + per);
  // ranks among the keys above / at the boundary before this thread's range:
  // in place, only needed when the boundary bin is kept in part (otherwise
  // every boundary key is kept and ranks do not matter)
  uint32_t gt_before = 0u, eq_before = 0u;
  if (!in_place || bin != k) {
    uint32_t ngt = 0u, neq = 0u;
    for (int j = j0; j < j1; ++j) {
      const uint32_t u = keys[j] & pmask;
      ngt += u > prefix;
      neq += u == prefix;
    }
    const uint32_t packed = block_exclusive_scan(ngt | (neq << 16), red, nullptr);
    gt_before = packed & 0xFFFFu;
    eq_before = packed >> 16;
  }
  if (!in_place) {
    uint32_t slot = gt_before + min(eq_before, k);
    uint32_t eqr = eq_before;
    for (int j = j0; j < j1; ++j) {
      const uint32_t u = keys[j] & pmask;
      if (u > prefix) {
        out[slot++] = j;
      } else if (u == prefix) {
        if (eqr < k) out[slot++] = j;
        ++eqr;
      }
    }
    return;
  }
  // in place: rows to refill and the kept frame tokens, both ascending
  const int c = J.ip.c, T = J.ip.T;
  auto kept = [&](int j, uint32_t& eqr) -> bool {
    const uint32_t u = keys[j] & pmask;
    if (u > prefix) return true;
    if (u < prefix) return false;
    return eqr++ < k;
  };
  uint32_t nev = 0u, nkf = 0u, eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const bool keep = kept(j, eqr);
    if (j < c) nev += !keep;
    else nkf += keep;
  }
  uint32_t tot;
  const uint32_t packed2 = block_exclusive_scan(nev | (nkf << 16), red, &tot);
  uint32_t e = packed2 & 0xFFFFu, f = packed2 >> 16;
  // the lists: freed rows at [0, T), kept frame tokens at [T, 2T) -- in LDS
  // past the keys when they fit, else in the selection row (global)
  int32_t* lst = lists_lds ? reinterpret_cast<int32_t*>(keys) + pool : out;
  eqr = eq_before;
  for (int j = j0; j < j1; ++j) {
    const bool keep = kept(j, eqr);
    if (j < c) {
      if (!keep) lst[e++] = j;
    } else if (keep) {
      lst[T + f++] = j - c;
    }
  }
  const uint32_t evicted = tot & 0xFFFFu;
  for (int r = tid; r < budget - c; r += kSelThreads) lst[evicted + r] = c + r;
  const int M = min((int)(tot >> 16), T);
  if (tid == 0) out[2 * T] = M;
  // the lists are read back by other threads of this workgroup: the barrier
  // makes the writes above visible to them (global lists need the full one)
  if (lists_lds)
    lds_barrier();
  else
    __syncthreads();
  apply_moves(J.ip, lst, M, mh0, mh1);
}

// Detailed-cache append over the append workgroups (grid-stride over
// (token, head, K/V, chunk), chunk fastest).
__device__ void append_frame(const AppendJob& A, int blk, int nblk) {
  const int CH = A.D / 8;
  const int64_t items = (int64_t)A.T * A.Hkv * 2 * CH;
  const int64_t stride = (int64_t)nblk * kSelThreads;
  for (int64_t base = (int64_t)blk * kSelThreads; base < items; base += kMoveU * stride) {
    u32x4 buf[kMoveU];
    uint16_t* dst[kMoveU];
#pragma unroll
    for (int u = 0; u < kMoveU; ++u) {
      const int64_t it = base + u * stride + threadIdx.x;
      dst[u] = nullptr;
      if (it < items) {
        const int ch = (int)(it % CH);
        const int64_t rest = it / CH;
        const int which = (int)(rest & 1);
        const int64_t th = rest >> 1;
        const int h = (int)(th % A.Hkv);
        const int64_t t = th / A.Hkv;
        buf[u] = *reinterpret_cast<const u32x4*>((which ? A.vf : A.kf) +
                                                 (t * A.Hkv + h) * A.D + ch * 8);
        int64_t slot = A.frame_base + t;
        if (A.ring) slot %= A.cap;
        dst[u] = (which ? A.vd : A.kd) + ((int64_t)h * A.cap + slot) * A.D + ch * 8;
      }
    }
#pragma unroll
    for (int u = 0; u < kMoveU; ++u)
      if (dst[u]) *reinterpret_cast<u32x4*>(dst[u]) = buf[u];
  }
}

// Blocks [0, n_select) handle one KV head each (scores, and the selection
// unless J.sel is null); block n_select, when n_shared is 1, selects once for
// the whole layer from the scores summed over every KV head (J2: the
// Hkv x rt partial rows read as one list, h-major); the next n_append blocks
// append the frame to the detailed cache; the remaining blocks sum the split
// O partials (grid-stride over their share; with a short sleep first when a
// selection runs beside them, see launch_select).
__global__ __launch_bounds__(kSelThreads) void select_sum_kernel(SelectJob J, int n_select,
                                                                 SelectJob J2, int n_shared,
                                                                 AppendJob A, int n_append,
                                                                 SumJob Sj) {
  if ((int)blockIdx.x < n_select) {
    select_one_head(J, blockIdx.x);
    return;
  }
  if ((int)blockIdx.x < n_select + n_shared) {
    select_one_head(J2, 0);
    return;
  }
  n_select += n_shared;
  if ((int)blockIdx.x < n_select + n_append) {
    append_frame(A, blockIdx.x - n_select, n_append);
    return;
  }
  n_select += n_append;
  for (int i = 0; i < Sj.delay; ++i) __builtin_amdgcn_s_sleep(32);
  const int64_t nb = gridDim.x - n_select;
  for (int64_t i = (int64_t)(blockIdx.x - n_select) * kSelThreads + threadIdx.x; i < Sj.n4;
       i += nb * kSelThreads) {
    // every split's load in flight, then the sum in split order
    constexpr int kMaxSplitsInFlight = 16;
    f32x4 pv[kMaxSplitsInFlight];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < Sj.S; s0 += kMaxSplitsInFlight) {
#pragma unroll
      for (int u = 0; u < kMaxSplitsInFlight; ++u)
        if (s0 + u < Sj.S) pv[u] = Sj.part[(s0 + u) * Sj.n4 + i];
#pragma unroll
      for (int u = 0; u < kMaxSplitsInFlight; ++u)
        if (s0 + u < Sj.S) acc += pv[u];
    }
    if (Sj.bf16)
      static_cast<bf16x4*>(Sj.out)[i] = __builtin_convertvector(acc, bf16x4);
    else
      static_cast<f32x4*>(Sj.out)[i] = acc;
  }
}

namespace {
hipError_t launch_select_sum(const SelectJob& J, int n_select, const SelectJob& J2, int n_shared,
                             const AppendJob& A, int n_append, const SumJob& Sj, int sum_blocks,
                             const Stream& st) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(select_sum_kernel), kMaxPool * (int)sizeof(uint32_t), lds_set);
  if (e != hipSuccess) return e;
  size_t words = (size_t)J.pool;
  if ((J.ip.pos || J2.ip.pos) && in_place_lds_fits(J.pool, J.ip.T))
    words = (size_t)J.pool + 2 * (size_t)J.ip.T;
  const size_t lds = words * sizeof(uint32_t);
  hipExtLaunchKernelGGL(select_sum_kernel, dim3(n_select + n_shared + n_append + sum_blocks),
                        dim3(kSelThreads), lds, st.st, st.start, st.stop, 0, J, n_select, J2,
                        n_shared, A, n_append, Sj);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_select(const float* sig_part, int rt, int ldsig, int hkv, int pool, int budget,
                         float* scores, int ldscores, int32_t* sel, int ldsel,
                         const float* o_part, int S, int64_t o_elems, void* o, bool o_bf16,
                         bool shared,
                         bool recent, const InPlace& ip, const AppendJob* app,
                         const Stream& st) {
  shared = shared && !recent;  // the recency window is the same for every head
  SelectJob J = {sig_part, rt, ldsig, pool, budget, scores, ldscores, shared ? nullptr : sel,
                 ldsel, recent ? 1 : 0, ip, 0, 1};
  // the layer-wide job: every head holds the same rows, so head 0's positions serve
  SelectJob J2 = {sig_part, rt, ldsig, pool, budget, nullptr, 0, sel, ldsel, 0, ip, 1, hkv};
  // When a selection runs and the O sum has slack, the sum starts one sleep
  // round late: the selecting workgroups first read their heads' partial
  // column sums, and the sum's tens of megabytes of split partials would
  // otherwise fill the memory queues under those reads.  The slack is judged
  // by the split partials per pool candidate: 7.6 KB at the 8B-like shape
  // (the launch takes 12.2 us instead of 12.9; two rounds are no better,
  // three make the sum the long pole), 12.3 KB in the 2B-like 28-layer
  // stream, where starting late already makes it the long pole (+1.5 %).
  const double part_per_candidate = (double)S * (double)o_elems * 4.0 / (double)pool;
  const int delay = (pool > budget && !recent && part_per_candidate < 10240.0) ? 1 : 0;
  SumJob Sj = {reinterpret_cast<const f32x4*>(o_part), o, o_elems / 4, S, o_bf16 ? 1 : 0, delay};
  // The O sum runs beside the selection: enough workgroups that it ends
  // before the selection (about 18 partial loads per thread: two f32x4
  // outputs of 9 splits at the 8B-like shape, one output when there are more
  // splits), few enough to leave the selecting workgroups most of the memory
  // system.
  int sum_blocks = 0;
  if (o_part && S > 1 && o_elems > 0) {
    const int64_t per_thread = S >= 18 ? 1 : 18 / S;
    const int64_t want = (Sj.n4 + per_thread * kSelThreads - 1) / (per_thread * kSelThreads);
    sum_blocks = (int)(want < 32 ? 32 : want > 1024 ? 1024 : want);
  }
  AppendJob A = {};
  int n_append = 0;
  if (app) {
    A = *app;
    const int64_t items = (int64_t)A.T * A.Hkv * 2 * (A.D / 8);
    const int64_t want = (items + kSelThreads - 1) / kSelThreads;
    n_append = (int)(want < 256 ? want : 256);
  }
  return launch_select_sum(J, hkv, J2, shared ? 1 : 0, A, n_append, Sj, sum_blocks, st);
}

}  // namespace skv
