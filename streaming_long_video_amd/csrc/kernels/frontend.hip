// The frame's query/key/value projection with the rotary embedding in its
// epilogue, for gfx950.
//
// For frame n the backbone forms Q_n = X_n W_Q, K_n = X_n W_K, V_n = X_n W_V
// from the hidden states X_n of the frame's visual tokens (paper.rainbus.top,
// method-steps section), and queries and keys are rotated at the tokens'
// original positions with the one RoPE configuration that cache building and
// text generation share (paperlayer.ai section 3.3; rainbus prerequisites,
// RoPE scaling).  These kernels do both and write q, k, v in the token-major
// layouts the prefill step reads.
//
// GEMM shape: M = T tokens, N = (Hq + 2 Hkv) d output features, K = hidden.
// At T = 256 the weights (N x K bf16, 33 MB at the 8B shape) are the only
// large operand, so the HBM floor is reading them once.  What binds a tiled
// kernel here is the volume staged from L2 into LDS: every tile re-reads its
// rows of X and W, (BM + BN) K elements for BM x BN outputs.
//
// Tiling.  A workgroup (8 waves) owns 128 tokens x 128 output features: the
// 64 rotation pairs (i, i + d/2) of one head (d = 128) or of two (d = 64), so
// the epilogue holds both members of every pair.  Wave (wm, wn) computes
// tokens 32 wm.. x the pairs' first (wn = 0) or second (wn = 1) members as
// two 32 x 32 blocks of v_mfma_f32_32x32x16_bf16 (tokens on M, features on N,
// fp32 accumulation).  Hidden features stream through LDS in 64-wide chunks
// (16 KB of X, 16 KB of W) by direct global-to-LDS loads
// (global_load_lds_dwordx4, no registers), in a ring of three stages: two
// chunks in flight while one is computed, one barrier per chunk and waits
// counted per chunk (a barrier without a fence, so the loads still in flight
// are not drained).  In LDS a staged row is 128 bytes with its 16-byte
// pieces XOR-swizzled by (row / 2) mod 8 -- chosen on the global side, since
// a direct load writes its 64 lanes' pieces contiguously -- so the operand
// reads are free of bank conflicts.
//
// 128 x 128 tiles leave few workgroups (72 at the 8B shape), so the hidden
// dimension is split S ways (216 workgroups, one per CU).  With S = 1 the
// GEMM kernel rotates and rounds its own tile (fp64, an angle recurrence
// over each thread's 16 consecutive tokens); otherwise it stores fp32
// partial tiles plus a few entries of a (cos, sin) table per (token, pair
// index) -- shared by every rotated head -- and qkv_combine_kernel sums the
// S partials of each output in split order (deterministic), rotates by the
// table in fp64 and rounds.  Each output is rounded to bf16 once; the
// rotation frequencies come from the host.  Workgroup ids are renumbered so
// the token tiles of one (feature tile, split) run on the same XCD and share
// its weight rows in that XCD's L2.
//
#include "../skv_internal.h"
#include "bf16_device.h"

namespace skv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFeM = 128;             // tokens per tile
constexpr int kFePairs = 64;          // rotation pairs per tile
constexpr int kFeN = 2 * kFePairs;    // output features per tile
constexpr int kFeK = 64;              // hidden features per staged chunk (128-byte rows)
constexpr int kFeThreads = 512;       // 8 waves
constexpr int kFeStages = 3;          // LDS ring: two chunks in flight + the one computed
constexpr int kFeOld = kFeN + 1;      // floats per row of the epilogue tile
constexpr int kFeRows = kFeM + kFeN;  // staged rows per chunk (X rows, then W rows)
constexpr int kFeStage = kFeRows * kFeK;  // bf16 per stage (32 KB)
// direct loads per wave per chunk: a load covers 8 rows (64 lanes x 16 B)
constexpr int kFeLoads = kFeRows / 8 / (kFeThreads / 64);
static_assert(kFeLoads * 8 * (kFeThreads / 64) == kFeRows, "rows split evenly over the waves");
static_assert(kFeM * kFeOld * 4 <= kFeStages * kFeStage * 2, "epilogue tile fits in the ring");
// s_waitcnt operands: vmcnt(n) with expcnt and lgkmcnt left alone (n < 16)
constexpr int kWaitVm = 0x0F70;
static_assert(kFeLoads < 16, "vmcnt immediate");
// tokens rotated per thread in the epilogues
constexpr int kFeRun = kFeM * kFePairs / kFeThreads;  // 16

#define FE_GLOBAL(p) ((const void __attribute__((address_space(1)))*)(p))
#define FE_LDS(p) ((void __attribute__((address_space(3)))*)(p))

// 16-byte piece `c` of staged row `r` sits in slot c ^ ((r / 2) mod 8)
__device__ inline int fe_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so each XCD
// gets a contiguous range of logical ids.
__device__ inline int fe_logical_id(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Row of W (output feature) of member `m` (0: i, 1: i + d/2) of global
// rotation pair P, pairs numbered head by head.
template <int D>
__device__ inline int fe_feature(int P, int m) {
  constexpr int HALF = D / 2;
  return (P / HALF) * D + m * HALF + P % HALF;
}

// Rotate and round kFeRun consecutive tokens of one pair.  x(u) yields the
// unrotated (first, second) member values of token t0 + u.
template <int D, class Load>
__device__ inline void fe_rotate_store(const FrontArgs& a, int P, int t0, Load x) {
  constexpr int HALF = D / 2;
  const int hh = P / HALF, i = P % HALF;
  const bool is_q = hh < a.Hq, is_k = !is_q && hh < a.Hq + a.Hkv;
  const bool rotate = (is_q || is_k) && a.theta > 0.0;
  double cs = 1.0, sn = 0.0, dc = 1.0, ds = 0.0;
  if (rotate) {
    const double inv_freq = a.inv_freq[i];
    const double step = inv_freq / a.scaling;
    sincos((double)(a.first_position + t0) / a.scaling * inv_freq, &sn, &cs);
    sincos(step, &ds, &dc);
  }
  uint16_t* out;
  int nh, head;
  if (is_q) {
    out = a.q; nh = a.Hq; head = hh;
  } else if (is_k) {
    out = a.k; nh = a.Hkv; head = hh - a.Hq;
  } else {
    out = a.v; nh = a.Hkv; head = hh - a.Hq - a.Hkv;
  }
#pragma unroll 4
  for (int u = 0; u < kFeRun; ++u) {
    const int t = t0 + u;
    if (t >= a.T) break;
    double x0, x1;
    x(u, x0, x1);
    double y0 = x0, y1 = x1;
    if (rotate) {
      y0 = fma(x0, cs, -(x1 * sn));
      y1 = fma(x0, sn, x1 * cs);
      // advance the angle by one position: (cs, sn) <- (cs, sn) * (dc, ds)
      const double nc = fma(cs, dc, -(sn * ds));
      sn = fma(sn, dc, cs * ds);
      cs = nc;
    }
    uint16_t* dst = out + ((int64_t)t * nh + head) * D;
    dst[i] = f64_to_bf16_rne(y0);
    dst[i + HALF] = f64_to_bf16_rne(y1);
  }
}

template <int D>
__global__ __launch_bounds__(kFeThreads, 1) void qkv_rope_kernel(FrontArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ring[kFeStages * kFeStage];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int mtiles = (a.T + kFeM - 1) / kFeM;
  const int lid = fe_logical_id(blockIdx.x, gridDim.x);
  const int mt = lid % mtiles;
  const int s = (lid / mtiles) % a.S;
  const int nt = lid / mtiles / a.S;
  const int m0 = mt * kFeM;
  const int npairs = (a.Hq + 2 * a.Hkv) * (D / 2);
  const int nchunks = a.hidden / kFeK;
  const int kc0 = (int)((int64_t)s * nchunks / a.S);
  const int kc1 = (int)((int64_t)(s + 1) * nchunks / a.S);

  // this lane's source row and piece for each of the wave's direct loads:
  // staged row r < 128 is token m0 + r (clamped past T: those results are
  // dropped), row 128 + j is the W row of tile feature j (member j / 64 of
  // the tile's pair j mod 64; pairs past the last are clamped and dropped)
  const uint16_t* src[kFeLoads];
#pragma unroll
  for (int u = 0; u < kFeLoads; ++u) {
    const int r = (w * kFeLoads + u) * 8 + (lane >> 3);
    const int c = fe_slot(r, lane & 7);  // the slot this lane fills holds piece c
    if (r < kFeM) {
      src[u] = a.x + (int64_t)min(m0 + r, a.T - 1) * a.hidden + c * 8;
    } else {
      const int j = r - kFeM;
      const int P = min(nt * kFePairs + (j & (kFePairs - 1)), npairs - 1);
      src[u] = a.w + (int64_t)fe_feature<D>(P, j / kFePairs) * a.hidden + c * 8;
    }
  }
  auto issue = [&](int kc) __attribute__((always_inline)) {
    uint16_t* stage = ring + (kc % kFeStages) * kFeStage;
#pragma unroll
    for (int u = 0; u < kFeLoads; ++u)
      __builtin_amdgcn_global_load_lds(FE_GLOBAL(src[u] + kc * kFeK),
                                       FE_LDS(stage + (w * kFeLoads + u) * 8 * kFeK), 16, 0, 0);
  };
#pragma unroll
  for (int kc = kc0; kc < kc0 + kFeStages - 1; ++kc)
    if (kc < kc1) issue(kc);

  // operand rows of this lane: token 32 wm + l32; features 64 wn + 32 f + l32
  const int ra = 32 * wm + l32, rb = kFeM + 64 * wn + l32;
  f32x16 acc[2] = {};
  for (int kc = kc0; kc < kc1; ++kc) {
    // chunk kc has landed once at most the next chunk's loads are in flight
    if (kc + 1 < kc1) __builtin_amdgcn_s_waitcnt(kWaitVm | kFeLoads);
    else __builtin_amdgcn_s_waitcnt(kWaitVm);
    // every wave's loads of chunk kc are in, and every wave is done with the
    // stage the next load overwrites (no fence: later loads stay in flight)
    __builtin_amdgcn_s_barrier();
    if (kc + kFeStages - 1 < kc1) issue(kc + kFeStages - 1);
    const uint16_t* stage = ring + (kc % kFeStages) * kFeStage;
    // every operand fragment of the chunk is read before its MFMAs
    bf16x8 av[kFeK / 16], bv[2][kFeK / 16];
#pragma unroll
    for (int kk = 0; kk < kFeK / 16; ++kk) {
      const int c = 2 * kk + half;
      av[kk] = *reinterpret_cast<const bf16x8*>(stage + ra * kFeK + fe_slot(ra, c) * 8);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int rf = rb + 32 * f;
        bv[f][kk] = *reinterpret_cast<const bf16x8*>(stage + rf * kFeK + fe_slot(rf, c) * 8);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
    for (int kk = 0; kk < kFeK / 16; ++kk)
#pragma unroll
      for (int f = 0; f < 2; ++f)
        acc[f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk], bv[f][kk], acc[f], 0, 0, 0);
  }

  // -- epilogue: tile[token][feature column] through LDS ----------------------
  __builtin_amdgcn_s_waitcnt(kWaitVm);
  __syncthreads();  // every operand read is done: the ring is free
  float* tile = reinterpret_cast<float*>(ring);
  // lane holds feature column 64 wn + 32 f + l32 and tokens
  // 32 wm + 8(r/4) + 4 half + r%4
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * wm + 8 * (r >> 2) + 4 * half + (r & 3);
      tile[m * kFeOld + 64 * wn + 32 * f + l32] = acc[f][r];
    }
  __syncthreads();
  if (a.S == 1) {
    // thread: pair p of the tile, tokens r0 .. r0 + kFeRun - 1
    const int p = tid & (kFePairs - 1);
    const int r0 = (tid / kFePairs) * kFeRun;
    const int P = nt * kFePairs + p;
    if (P < npairs)
      fe_rotate_store<D>(a, P, m0 + r0, [&](int u, double& x0, double& x1) {
        x0 = tile[(r0 + u) * kFeOld + p];
        x1 = tile[(r0 + u) * kFeOld + kFePairs + p];
      });
  } else {
    // fp32 partial tile: part[s][nt][t][128], rows of 512 bytes, one 16-byte
    // piece per thread
    const int ntiles = (npairs + kFePairs - 1) / kFePairs;
    float* part = a.part + ((int64_t)s * ntiles + nt) * a.T * kFeN;
    const int c4 = tid & (kFeN / 4 - 1);
    for (int m = tid / (kFeN / 4); m < kFeM; m += kFeThreads / (kFeN / 4)) {
      if (m0 + m >= a.T) break;
      const float* rowp = tile + m * kFeOld + 4 * c4;
      const f32x4 v = {rowp[0], rowp[1], rowp[2], rowp[3]};
      *reinterpret_cast<f32x4*>(part + (int64_t)(m0 + m) * kFeN + 4 * c4) = v;
    }
    // the rotation table rot[t][i] = (cos, sin) of token t's angle for pair
    // index i, shared by every rotated head: a few entries per workgroup
    if (a.theta > 0.0) {
      constexpr int HALF = D / 2;
      for (int e = lid + (int)gridDim.x * tid; e < a.T * HALF; e += (int)gridDim.x * kFeThreads) {
        const int t = e / HALF, i = e % HALF;
        const double inv_freq = a.inv_freq[i];
        double sn, cs;
        sincos((double)(a.first_position + t) / a.scaling * inv_freq, &sn, &cs);
        a.rot[2 * e] = cs;
        a.rot[2 * e + 1] = sn;
      }
    }
  }
}

// Sum of the S partial tiles of each output in split order, rotation by the
// table and rounding.  Block: one feature tile x 16 tokens; thread: pair p,
// kCbRun consecutive tokens, with every load of the thread issued before the
// arithmetic (one memory round trip).
constexpr int kCbRun = 4;
constexpr int kCbThreads = 256;
constexpr int kCbTokens = kCbThreads / kFePairs * kCbRun;  // 16
constexpr int kFeMaxSplits = 8;

template <int D>
__global__ __launch_bounds__(kCbThreads) void qkv_combine_kernel(FrontArgs a) {
  constexpr int HALF = D / 2;
  const int npairs = (a.Hq + 2 * a.Hkv) * HALF;
  const int ntiles = (npairs + kFePairs - 1) / kFePairs;
  const int ttiles = (a.T + kCbTokens - 1) / kCbTokens;
  const int nt = blockIdx.x / ttiles;
  const int tt = blockIdx.x % ttiles;
  const int p = threadIdx.x & (kFePairs - 1);
  const int t0 = tt * kCbTokens + (threadIdx.x / kFePairs) * kCbRun;
  const int P = nt * kFePairs + p;
  if (P >= npairs || t0 >= a.T) return;
  const int n = min(kCbRun, a.T - t0);
  const int hh = P / HALF, i = P % HALF;
  const bool is_q = hh < a.Hq, is_k = !is_q && hh < a.Hq + a.Hkv;
  const bool rotate = (is_q || is_k) && a.theta > 0.0;

  const int64_t split = (int64_t)ntiles * a.T * kFeN;
  const float* base = a.part + ((int64_t)nt * a.T + t0) * kFeN + p;
  float v0[kFeMaxSplits][kCbRun], v1[kFeMaxSplits][kCbRun];
  double cs[kCbRun], sn[kCbRun];
#pragma unroll
  for (int s = 0; s < kFeMaxSplits; ++s)
#pragma unroll
    for (int u = 0; u < kCbRun; ++u)
      if (s < a.S && u < n) {
        v0[s][u] = base[s * split + u * kFeN];
        v1[s][u] = base[s * split + u * kFeN + kFePairs];
      }
#pragma unroll
  for (int u = 0; u < kCbRun; ++u)
    if (rotate && u < n) {
      cs[u] = a.rot[2 * ((int64_t)(t0 + u) * HALF + i)];
      sn[u] = a.rot[2 * ((int64_t)(t0 + u) * HALF + i) + 1];
    }
  uint16_t* out;
  int nh, head;
  if (is_q) {
    out = a.q; nh = a.Hq; head = hh;
  } else if (is_k) {
    out = a.k; nh = a.Hkv; head = hh - a.Hq;
  } else {
    out = a.v; nh = a.Hkv; head = hh - a.Hq - a.Hkv;
  }
#pragma unroll
  for (int u = 0; u < kCbRun; ++u) {
    if (u >= n) break;
    float s0 = v0[0][u], s1 = v1[0][u];
#pragma unroll
    for (int s = 1; s < kFeMaxSplits; ++s)
      if (s < a.S) {
        s0 += v0[s][u];
        s1 += v1[s][u];
      }
    double y0 = s0, y1 = s1;
    if (rotate) {
      y0 = fma((double)s0, cs[u], -((double)s1 * sn[u]));
      y1 = fma((double)s0, sn[u], (double)s1 * cs[u]);
    }
    uint16_t* dst = out + ((int64_t)(t0 + u) * nh + head) * D;
    dst[i] = f64_to_bf16_rne(y0);
    dst[i + HALF] = f64_to_bf16_rne(y1);
  }
}

}  // namespace

int qkv_rope_splits(int T, int hidden, int heads, int D) {
  const int mtiles = (T + kFeM - 1) / kFeM;
  const int ntiles = (heads * (D / 2) + kFePairs - 1) / kFePairs;
  const int tiles = mtiles * ntiles;
  const int nchunks = hidden / kFeK;
  // one workgroup per CU (256), at least 8 chunks per split, at most
  // kFeMaxSplits splits
  const int s = std::min({256 / std::max(tiles, 1), nchunks / 8, kFeMaxSplits});
  return std::max(1, s);
}

size_t qkv_rope_workspace_bytes(int T, int hidden, int heads, int D) {
  const int S = qkv_rope_splits(T, hidden, heads, D);
  if (S == 1) return 0;
  const int ntiles = (heads * (D / 2) + kFePairs - 1) / kFePairs;
  // partial tiles, then the rotation table (T x D/2 (cos, sin) pairs)
  return (size_t)S * ntiles * T * kFeN * sizeof(float) + (size_t)T * (D / 2) * 2 * sizeof(double);
}

hipError_t launch_qkv_rope(const FrontArgs& a, int D, const Stream& st) {
  const int heads = a.Hq + 2 * a.Hkv;
  const int mtiles = (a.T + kFeM - 1) / kFeM;
  const int ntiles = (heads * (D / 2) + kFePairs - 1) / kFePairs;
  const dim3 grid((unsigned)(mtiles * ntiles * a.S));
  hipEvent_t stop = a.S == 1 ? st.stop : nullptr;
  if (D == 128)
    hipExtLaunchKernelGGL((qkv_rope_kernel<128>), grid, dim3(kFeThreads), 0, st.st, st.start,
                          stop, 0, a);
  else
    hipExtLaunchKernelGGL((qkv_rope_kernel<64>), grid, dim3(kFeThreads), 0, st.st, st.start,
                          stop, 0, a);
  if (a.S == 1) return hipGetLastError();
  const dim3 cgrid((unsigned)(ntiles * ((a.T + kCbTokens - 1) / kCbTokens)));
  if (D == 128)
    hipExtLaunchKernelGGL((qkv_combine_kernel<128>), cgrid, dim3(kCbThreads), 0, st.st, nullptr,
                          st.stop, 0, a);
  else
    hipExtLaunchKernelGGL((qkv_combine_kernel<64>), cgrid, dim3(kCbThreads), 0, st.st, nullptr,
                          st.stop, 0, a);
  return hipGetLastError();
}

}  // namespace skv
