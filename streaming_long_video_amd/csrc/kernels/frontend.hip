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
// Hidden features stream through LDS in 64-wide chunks (8 KB of X, 8 KB of
// W) by direct global-to-LDS loads (global_load_lds_dwordx4, no registers),
// in a ring of kFeStages stages: kFeStages - 1 chunks are in flight while one
// is computed, with one barrier per chunk and waits counted per chunk (a
// barrier without a fence, so the loads still in flight are not drained).
// In LDS a staged row is 128 bytes with its 16-byte pieces XOR-swizzled by
// (row / 2) mod 8 -- chosen on the global side, since a direct load writes
// its 64 lanes' pieces contiguously -- so the operand reads are free of bank
// conflicts.  Workgroup ids are renumbered so the token tiles of one feature
// tile run on the same XCD and share its weight rows in that XCD's L2.
//
#include "../skv_internal.h"
#include "bf16_device.h"

namespace skv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kFeM = 64;          // tokens per tile
constexpr int kFeN = 64;          // output features per tile (32 rotation pairs)
constexpr int kFeK = 64;          // hidden features per staged chunk (128-byte rows)
constexpr int kFeThreads = 256;   // 4 waves
constexpr int kFeStages = 4;      // LDS ring: chunks in flight + the one computed
constexpr int kFeOld = kFeN + 1;  // floats per row of the epilogue tile
constexpr int kFeRows = kFeM + kFeN;  // staged rows per chunk (X rows, then W rows)
constexpr int kFeStage = kFeRows * kFeK;  // bf16 per stage (16 KB)
// direct loads per wave per chunk: a load covers 8 rows (64 lanes x 16 B)
constexpr int kFeLoads = kFeRows / 8 / (kFeThreads / 64);
static_assert(kFeLoads * 8 * (kFeThreads / 64) == kFeRows, "rows split evenly over the waves");
// s_waitcnt operand: vmcnt(n) with expcnt and lgkmcnt left alone
constexpr int kWaitVm = 0x0F70;

#define FE_GLOBAL(p) ((const void __attribute__((address_space(1)))*)(p))
#define FE_LDS(p) ((void __attribute__((address_space(3)))*)(p))

// 16-byte piece `c` of staged row `r` sits in slot c ^ ((r / 2) mod 8)
__device__ inline int fe_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so each XCD
// gets a contiguous range of logical ids (the token tiles of a feature tile
// are consecutive ids).
__device__ inline int fe_logical_id(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <int D>
__global__ __launch_bounds__(kFeThreads, 2) void qkv_rope_kernel(FrontArgs a) {
  constexpr int HALF = D / 2;
  constexpr int TPH = HALF / 32;  // feature tiles per head
  static_assert(kFeM * kFeOld * 4 <= kFeStages * kFeStage * 2, "epilogue tile fits");
  __shared__ __attribute__((aligned(16))) uint16_t ring[kFeStages * kFeStage];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int mtiles = (a.T + kFeM - 1) / kFeM;
  const int lid = fe_logical_id(blockIdx.x, gridDim.x);
  const int mt = lid % mtiles, nt = lid / mtiles;
  const int hh = nt / TPH;             // head among Q heads, K heads, V heads
  const int c0 = (nt % TPH) * 32;      // first pair index of the tile
  const int m0 = mt * kFeM;

  // this lane's source row and piece for each of the wave's direct loads:
  // staged row r < 64 is token m0 + r (clamped past T: those results are
  // dropped), row 64 + j is the W row of tile feature j (the pair's first
  // member for j < 32, its second for j >= 32)
  const uint16_t* src[kFeLoads];
#pragma unroll
  for (int u = 0; u < kFeLoads; ++u) {
    const int r = (w * kFeLoads + u) * 8 + (lane >> 3);
    const int c = fe_slot(r, lane & 7);  // the slot this lane fills holds piece c
    if (r < kFeM) {
      src[u] = a.x + (int64_t)min(m0 + r, a.T - 1) * a.hidden + c * 8;
    } else {
      const int j = r - kFeM;
      const int feat = hh * D + (j < 32 ? c0 + j : HALF + c0 + (j - 32));
      src[u] = a.w + (int64_t)feat * a.hidden + c * 8;
    }
  }
  const int nchunks = a.hidden / kFeK;
  auto issue = [&](int kc) __attribute__((always_inline)) {
    uint16_t* stage = ring + (kc % kFeStages) * kFeStage;
#pragma unroll
    for (int u = 0; u < kFeLoads; ++u)
      __builtin_amdgcn_global_load_lds(FE_GLOBAL(src[u] + kc * kFeK),
                                       FE_LDS(stage + (w * kFeLoads + u) * 8 * kFeK), 16, 0, 0);
  };
#pragma unroll
  for (int kc = 0; kc < kFeStages - 1; ++kc)
    if (kc < nchunks) issue(kc);

  // operand rows of this lane: token 32 wm + l32, feature 32 wn + l32
  const int ra = 32 * wm + l32, rb = kFeM + 32 * wn + l32;
  f32x16 acc = {};
  for (int kc = 0; kc < nchunks; ++kc) {
    // chunk kc has landed once at most the later chunks' loads are in flight
    const int later = min(nchunks - 1, kc + kFeStages - 2) - kc;
    if (later >= 2) __builtin_amdgcn_s_waitcnt(kWaitVm | (2 * kFeLoads));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(kWaitVm | kFeLoads);
    else __builtin_amdgcn_s_waitcnt(kWaitVm);
    // every wave's loads of chunk kc are in, and every wave is done with the
    // stage the next load overwrites (no fence: later loads stay in flight)
    __builtin_amdgcn_s_barrier();
    if (kc + kFeStages - 1 < nchunks) issue(kc + kFeStages - 1);
    const uint16_t* stage = ring + (kc % kFeStages) * kFeStage;
    // every operand fragment of the chunk is read before its MFMAs
    bf16x8 av[kFeK / 16], bv[kFeK / 16];
#pragma unroll
    for (int kk = 0; kk < kFeK / 16; ++kk) {
      const int c = 2 * kk + half;
      av[kk] = *reinterpret_cast<const bf16x8*>(stage + ra * kFeK + fe_slot(ra, c) * 8);
      bv[kk] = *reinterpret_cast<const bf16x8*>(stage + rb * kFeK + fe_slot(rb, c) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
    for (int kk = 0; kk < kFeK / 16; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk], bv[kk], acc, 0, 0, 0);
  }
  static_assert(kFeStages - 2 <= 2, "the waits above cover at most two later chunks");

  // -- epilogue: tile[token][feature column] through LDS ----------------------
  __builtin_amdgcn_s_waitcnt(kWaitVm);
  __syncthreads();  // every operand read is done: the ring is free
  float* tile = reinterpret_cast<float*>(ring);
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
  static_assert(kFeThreads == 256, "launch shape");
  if (D == 128)
    hipExtLaunchKernelGGL((qkv_rope_kernel<128>), grid, dim3(kFeThreads), 0, st.st, st.start,
                          st.stop, 0, a);
  else
    hipExtLaunchKernelGGL((qkv_rope_kernel<64>), grid, dim3(kFeThreads), 0, st.st, st.start,
                          st.stop, 0, a);
  return hipGetLastError();
}

}  // namespace skv
