// The frame's query/key/value projection with the rotary embedding in its
// epilogue, for gfx950.
//
// For frame n the backbone forms Q_n = X_n W_Q, K_n = X_n W_K, V_n = X_n W_V
// from the hidden states X_n of the frame's visual tokens (paper.rainbus.top,
// method-steps section), and queries and keys are rotated at the tokens'
// original positions with the one RoPE configuration that cache building and
// text generation share (paperlayer.ai section 3.3; rainbus prerequisites,
// RoPE scaling).  This kernel does both in one pass and writes q, k, v in the
// token-major layouts the prefill step reads.
//
// GEMM shape: M = T tokens, N = (Hq + 2 Hkv) d output features, K = hidden.
// At T = 256 the weights (N x K bf16, 33 MB at the 8B shape) are the only
// large operand: the kernel is bound by reading them once from HBM.
//
// Tiling.  A workgroup (4 waves) owns 64 tokens x 64 output features of one
// head: the 32 rotation pairs (i, i + d/2) for i in [c0, c0 + 32), so the
// epilogue holds both members of every pair.  Wave (wm, wn) computes tokens
// 32 wm.. x the pair's first (wn = 0) or second (wn = 1) members with
// v_mfma_f32_32x32x16_bf16 (tokens on M, features on N, fp32 accumulation).
// Hidden features are staged in 64-wide chunks through LDS, double-buffered
// (next chunk's global loads in registers while the current one is
// computed).  Workgroup ids are renumbered so the token tiles of one feature
// tile run on the same XCD and share its weight rows in that XCD's L2.
//
// Epilogue.  The accumulators go through LDS so that each thread holds one
// pair index j for 8 consecutive tokens; cos/sin of the angle
// (p / scaling) * theta^(-2i/d) are formed in double precision (p reaches
// 1e5 and beyond: a float angle would be off by ~1e-2 rad) for the first
// token and stepped by an exact-angle rotation for the next ones; the
// rotation is done in double from the fp32 accumulators and rounded once to
// bf16 (nearest, ties to even).  V heads are rounded without rotation.
#include "../skv_internal.h"
#include "bf16_device.h"

namespace skv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFeM = 64;         // tokens per tile
constexpr int kFeN = 64;         // output features per tile (32 rotation pairs)
constexpr int kFeK = 64;         // hidden features per staged chunk
constexpr int kFeThreads = 256;  // 4 waves
constexpr int kFeLd = kFeK + 8;  // bf16 per staged row (conflict-free 16-byte reads)
constexpr int kFeOld = kFeN + 1; // floats per row of the epilogue tile
constexpr int kFePieces = kFeM * kFeK / 8 / kFeThreads;  // 16-byte pieces / thread / operand
static_assert(kFePieces * kFeThreads * 8 == kFeM * kFeK, "X chunk splits evenly");
static_assert(kFeN == kFeM, "one piece count serves both operands");

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so each XCD
// gets a contiguous range of logical ids (the token tiles of a feature tile
// are consecutive ids).
__device__ inline int fe_logical_id(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <int D>
__global__ __launch_bounds__(kFeThreads) void qkv_rope_kernel(FrontArgs a) {
  constexpr int HALF = D / 2;
  constexpr int TPH = HALF / 32;  // feature tiles per head
  constexpr int kStageBytes = 2 * 2 * kFeM * kFeLd * 2;
  constexpr int kTileBytes = kFeM * kFeOld * 4;
  static_assert(kTileBytes <= kStageBytes, "epilogue tile fits in the staging buffers");
  __shared__ __attribute__((aligned(16))) char smem[kStageBytes];
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);        // [2][kFeM][kFeLd]
  uint16_t* ws = xs + 2 * kFeM * kFeLd;                    // [2][kFeN][kFeLd]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int mtiles = (a.T + kFeM - 1) / kFeM;
  const int lid = fe_logical_id(blockIdx.x, gridDim.x);
  const int mt = lid % mtiles, nt = lid / mtiles;
  const int hh = nt / TPH;             // head among Q heads, K heads, V heads
  const int c0 = (nt % TPH) * 32;      // first pair index of the tile
  const int m0 = mt * kFeM;

  // staged rows: X token rows (clamped past T: those results are dropped) and
  // W feature rows (tile column j: the pair's first member for j < 32)
  const uint16_t* xrow[kFePieces];
  const uint16_t* wrow[kFePieces];
  int pcol[kFePieces], prow[kFePieces];
#pragma unroll
  for (int u = 0; u < kFePieces; ++u) {
    const int p = tid + u * kFeThreads;
    prow[u] = p / (kFeK / 8);
    pcol[u] = (p % (kFeK / 8)) * 8;
    const int t = min(m0 + prow[u], a.T - 1);
    xrow[u] = a.x + (int64_t)t * a.hidden + pcol[u];
    const int j = prow[u];
    const int feat = hh * D + (j < 32 ? c0 + j : HALF + c0 + (j - 32));
    wrow[u] = a.w + (int64_t)feat * a.hidden + pcol[u];
  }
  u32x4 xr[kFePieces], wr[kFePieces];
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kFePieces; ++u) {
      xr[u] = *reinterpret_cast<const u32x4*>(xrow[u] + k0);
      wr[u] = *reinterpret_cast<const u32x4*>(wrow[u] + k0);
    }
  };
  auto store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kFePieces; ++u) {
      *reinterpret_cast<u32x4*>(&xs[(buf * kFeM + prow[u]) * kFeLd + pcol[u]]) = xr[u];
      *reinterpret_cast<u32x4*>(&ws[(buf * kFeN + prow[u]) * kFeLd + pcol[u]]) = wr[u];
    }
  };

  const int nchunks = a.hidden / kFeK;
  load(0);
  store(0);
  __syncthreads();
  f32x16 acc = {};
  for (int kc = 0; kc < nchunks; ++kc) {
    const int cur = kc & 1;
    const bool more = kc + 1 < nchunks;
    if (more) load((kc + 1) * kFeK);
    const uint16_t* xa = &xs[(cur * kFeM + 32 * wm + l32) * kFeLd + half * 8];
    const uint16_t* wb = &ws[(cur * kFeN + 32 * wn + l32) * kFeLd + half * 8];
#pragma unroll
    for (int kk = 0; kk < kFeK / 16; ++kk) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(xa + kk * 16);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(wb + kk * 16);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    }
    if (more) store(cur ^ 1);
    __syncthreads();
  }

  // -- epilogue: tile[token][feature column] through LDS ----------------------
  float* tile = reinterpret_cast<float*>(smem);
  // lane holds feature column 32 wn + l32 and tokens 8(r/4) + 4 half + r%4
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 32 * wm + 8 * (r >> 2) + 4 * half + (r & 3);
    tile[m * kFeOld + 32 * wn + l32] = acc[r];
  }
  __syncthreads();
  const int j = tid & 31;            // pair of the tile
  const int r0 = (tid >> 5) * 8;     // first of this thread's 8 tokens
  const int i = c0 + j;              // pair index within the head
  const bool is_q = hh < a.Hq, is_k = !is_q && hh < a.Hq + a.Hkv;
  const bool rotate = (is_q || is_k) && a.theta > 0.0;
  double cs = 1.0, sn = 0.0, dc = 1.0, ds = 0.0;
  if (rotate) {
    const double inv_freq = pow(a.theta, -2.0 * i / D);
    const double step = inv_freq / a.scaling;
    sincos((double)(a.first_position + m0 + r0) / a.scaling * inv_freq, &sn, &cs);
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
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = r0 + u;
    const double x0 = tile[r * kFeOld + j];
    const double x1 = tile[r * kFeOld + 32 + j];
    double y0 = x0, y1 = x1;
    if (rotate) {
      y0 = fma(x0, cs, -(x1 * sn));
      y1 = fma(x0, sn, x1 * cs);
      // advance the angle by one position: (cs, sn) <- (cs, sn) * (dc, ds)
      const double nc = fma(cs, dc, -(sn * ds));
      sn = fma(sn, dc, cs * ds);
      cs = nc;
    }
    const int t = m0 + r;
    if (t < a.T) {
      uint16_t* dst = out + ((int64_t)t * nh + head) * D;
      dst[i] = f64_to_bf16_rne(y0);
      dst[i + HALF] = f64_to_bf16_rne(y1);
    }
  }
}

}  // namespace

hipError_t launch_qkv_rope(const FrontArgs& a, int D, const Stream& st) {
  const int mtiles = (a.T + kFeM - 1) / kFeM;
  const int heads = a.Hq + 2 * a.Hkv;
  const dim3 grid((unsigned)(mtiles * heads * (D / 64)));
  if (D == 128)
    hipExtLaunchKernelGGL((qkv_rope_kernel<128>), grid, dim3(kFeThreads), 0, st.st, st.start,
                          st.stop, 0, a);
  else
    hipExtLaunchKernelGGL((qkv_rope_kernel<64>), grid, dim3(kFeThreads), 0, st.st, st.start,
                          st.stop, 0, a);
  return hipGetLastError();
}

}  // namespace skv
