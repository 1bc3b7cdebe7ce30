// Decoding attention over the detailed state D for gfx950.
//
// Once every frame is in, text generation attends over D_N, the cache that
// keeps every original video token (gist.science/nl, "Het Proces", decoding
// item; rainbus summary, core method: ordinary text decoding over all video
// tokens after the incremental build).  The text follows the video, so every
// D token is visible to every text query.  This step reads all of D once per
// decoding step and is bound by HBM bandwidth.
//
// Work layout.  For KV head h the G query heads x M text tokens form at most
// 32 rows (row r: query head h*G + r % G, token r / G), one MFMA block.  The
// live D tokens of head h are cut into NS contiguous splits; one wave owns one
// split (four waves per workgroup, independent until the end) and streams it
// in 32-key blocks:
//   * K rows go straight from HBM into the A operand of S^T = K Q^T
//     (v_mfma_f32_32x32x16_bf16, keys on M, rows on N; 16 bytes per lane per
//     d-step), the next block's loads in flight while the current block is
//     computed;
//   * V rows are loaded coalesced, converted to fp16 and transposed into a
//     wave-private LDS tile, from which the A operand of O^T = V^T P^T
//     (v_mfma_f32_32x32x16_f16) is read;
//   * online softmax per row (max over the two half-waves that hold a row's
//     keys), P formed as fp16 * 2^12 exactly as in the prefill kernels.
// The four waves of a workgroup merge their (max, sum, O) through LDS in wave
// order and write one partial per workgroup; a second kernel merges the
// workgroups' partials of each row, every sum in a fixed order
// (deterministic).
#include "../skv_internal.h"

namespace skv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kVtLd = 36;                  // fp16 per V^T row (32 keys + pad): conflict-free
constexpr float kPScaleUnscale = 1.f / 4096.f;  // P is formed as 2^12 * P

__device__ inline float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ inline int as_i(float x) { return __builtin_bit_cast(int, x); }
__device__ inline float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ inline uint32_t pack_f16(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

template <int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode_kernel(DecodeArgs a) {
  constexpr int NKK = D / 16;           // d-steps of QK^T
  constexpr int NMB = D / 32;           // 32-row blocks of O^T
  constexpr int VITEMS = 16 * (D / 8);  // (key pair, 8-column chunk) items of a V block
  constexpr int VIT = VITEMS / 64;      // per lane
  static_assert(VIT * 64 == VITEMS, "V block splits evenly over a wave");
  // wave-private V^T tiles during the sweep; the merge of the waves' O after it
  constexpr int kOxLd = D + 4;  // floats per row of the O exchange (padded)
  constexpr int kVtBytes = kDecWaves * D * kVtLd * 2;
  constexpr int kOxBytes = (kDecWaves - 1) * 32 * kOxLd * 4;
  __shared__ __attribute__((aligned(16))) char smem[kVtBytes > kOxBytes ? kVtBytes : kOxBytes];
  __shared__ float cm[kDecWaves][32], cl[kDecWaves][32];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int per_head = (a.NS + kDecWaves - 1) / kDecWaves;
  const int h = blockIdx.x / per_head;
  const int wg = blockIdx.x % per_head;  // this workgroup's partial of head h
  const int split = wg * kDecWaves + w;  // splits past NS are empty
  _Float16* vt = reinterpret_cast<_Float16*>(smem) + w * D * kVtLd;
  const int64_t k_lo = split < a.NS ? (int64_t)split * a.len / a.NS : 0;
  const int64_t k_hi = split < a.NS ? (int64_t)(split + 1) * a.len / a.NS : 0;
  const uint16_t* kbase_ptr = a.kd + (int64_t)h * a.cap * D;
  const uint16_t* vbase_ptr = a.vd + (int64_t)h * a.cap * D;
  const float sl2 = a.scale_log2;

  // this lane's row: query head h*G + r % G, text token r / G
  const int rows = a.G * a.M;
  const bool row_ok = l32 < rows;
  const int qhead = h * a.G + (row_ok ? l32 % a.G : 0);
  const int qtok = row_ok ? l32 / a.G : 0;
  bf16x8 qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row_ok)
      v = *reinterpret_cast<const u32x4*>(a.q + ((int64_t)qtok * a.Hq + qhead) * D + kk * 16 +
                                          half * 8);
    qreg[kk] = __builtin_bit_cast(bf16x8, v);
  }

  // K block kb0 .. kb0+31 as the A operand (row = key, clamped into the split;
  // keys at or past k_hi are masked below)
  auto load_k = [&](int64_t kb0, bf16x8 (&kr)[NKK]) __attribute__((always_inline)) {
    const int64_t key = min(kb0 + l32, k_hi - 1);
    const uint16_t* row = kbase_ptr + key * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      kr[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(row + kk * 16));
  };
  // V block: item it = (key pair kp, column chunk cc); two 16-byte rows per item
  auto load_v = [&](int64_t kb0, u32x4 (&v0)[VIT], u32x4 (&v1)[VIT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = lane + 64 * i;
      const int kp = it % 16, cc = it / 16;
      const int64_t key0 = min(kb0 + 2 * kp, k_hi - 1), key1 = min(kb0 + 2 * kp + 1, k_hi - 1);
      v0[i] = *reinterpret_cast<const u32x4*>(vbase_ptr + key0 * D + cc * 8);
      v1[i] = *reinterpret_cast<const u32x4*>(vbase_ptr + key1 * D + cc * 8);
    }
  };
  // V^T[d][key] in fp16 (keys 2kp, 2kp+1 share one 32-bit word)
  auto store_vt = [&](const u32x4 (&v0)[VIT], const u32x4 (&v1)[VIT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = lane + 64 * i;
      const int kp = it % 16, cc = it / 16;
      uint32_t* col = reinterpret_cast<uint32_t*>(&vt[(cc * 8) * kVtLd + 2 * kp]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        col[(2 * e) * (kVtLd / 2)] = pack_f16(bf16lo(v0[i][e]), bf16lo(v1[i][e]));
        col[(2 * e + 1) * (kVtLd / 2)] = pack_f16(bf16hi(v0[i][e]), bf16hi(v1[i][e]));
      }
    }
  };

  f32x16 oacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) oacc[mb] = f32x16{};
  float mrun = -INFINITY, lrun = 0.f;

  bf16x8 kr[NKK];
  u32x4 v0[VIT], v1[VIT];
  if (k_lo < k_hi) {
    load_k(k_lo, kr);
    load_v(k_lo, v0, v1);
  }
  for (int64_t kb0 = k_lo; kb0 < k_hi; kb0 += 32) {
    const bool more = kb0 + 32 < k_hi;
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk], qreg[kk], sacc, 0, 0, 0);
    store_vt(v0, v1);
    if (more) {
      load_k(kb0 + 32, kr);
      load_v(kb0 + 32, v0, v1);
    }
    // register r holds key kb0 + 8(r/4) + 4 half + r%4 of this lane's row
    const int64_t lim = k_hi - kb0 - 4 * half;  // visible iff offset < lim
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      z[r] = (8 * (r >> 2) + (r & 3) < lim) ? sacc[r] : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
    {  // both half-waves hold the same row
      const auto sw = __builtin_amdgcn_permlane32_swap(as_i(mx), as_i(mx), false, false);
      mx = fmaxf(as_f(sw[0]), as_f(sw[1]));
    }
    const float mnew = fmaxf(mrun, mx);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f((mrun - msafe) * sl2);
    const float ms = fmaf(msafe, sl2, -12.f);
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(z[r], sl2, -ms));
    u32x4 ph[2];
#pragma unroll
    for (int slab = 0; slab < 2; ++slab)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        ph[slab][m] = pack_f16(e[slab * 8 + 2 * m], e[slab * 8 + 2 * m + 1]);
#pragma unroll
    for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
      for (int r = 0; r < st; ++r) e[r] += e[r + st];
    lrun = lrun * alpha + e[0];
    mrun = mnew;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      oacc[mb] *= alpha;
#pragma unroll
      for (int slab = 0; slab < 2; ++slab) {
        const _Float16* vrow = &vt[(mb * 32 + l32) * kVtLd + slab * 16 + 4 * half];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
        const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
        oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, av),
                                                          __builtin_bit_cast(f16x8, ph[slab]),
                                                          oacc[mb], 0, 0, 0);
      }
    }
  }

  // merge the four waves (all rows; rows past G*M carry zeros), then wave 0
  // writes the workgroup's partial: row max of the raw logits, row sum and
  // O, both relative to that max
  const float lt = lrun + __shfl_xor(lrun, 32);  // both halves of the row
  if (half == 0) {
    cm[w][l32] = mrun;
    cl[w][l32] = lt;
  }
  __syncthreads();  // every wave is past its last V^T read: smem is free
  float mx = cm[0][l32];
#pragma unroll
  for (int i = 1; i < kDecWaves; ++i) mx = fmaxf(mx, cm[i][l32]);
  const float msafe = mx == -INFINITY ? 0.f : mx;
  const float f = mrun == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mrun - msafe) * sl2);
  float* ox = reinterpret_cast<float*>(smem);
  if (w > 0) {
    float* row = ox + ((w - 1) * 32 + l32) * kOxLd;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = {oacc[mb][4 * q4], oacc[mb][4 * q4 + 1], oacc[mb][4 * q4 + 2],
                         oacc[mb][4 * q4 + 3]};
        *reinterpret_cast<f32x4*>(row + mb * 32 + 8 * q4 + 4 * half) = v * f;
      }
  }
  __syncthreads();
  if (w != 0) return;
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < kDecWaves; ++i) {
    const float mi = cm[i][l32];
    if (mi > -INFINITY) L += cl[i][l32] * __builtin_amdgcn_exp2f((mi - msafe) * sl2);
  }
  if (!row_ok) return;
  float* dst = a.o_part + (((int64_t)wg * a.M + qtok) * a.Hq + qhead) * D;
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int col = mb * 32 + 8 * q4 + 4 * half;
      f32x4 v = {oacc[mb][4 * q4], oacc[mb][4 * q4 + 1], oacc[mb][4 * q4 + 2],
                 oacc[mb][4 * q4 + 3]};
      v *= f;
#pragma unroll
      for (int i = 1; i < kDecWaves; ++i)
        v += *reinterpret_cast<const f32x4*>(ox + ((i - 1) * 32 + l32) * kOxLd + col);
      *reinterpret_cast<f32x4*>(dst + col) = v * kPScaleUnscale;
    }
  if (half == 0) {
    const int64_t idx = ((int64_t)wg * a.Hq + qhead) * a.M + qtok;
    a.m_part[idx] = mx;
    a.l_part[idx] = L * kPScaleUnscale;
  }
}

// Merge of the workgroup partials of one output row (text token t, query head
// g) over a 32-column slice: M = max_p m_p, w_p = 2^((m_p - M) c),
// O = sum_p w_p O_p / sum_p w_p l_p.  Thread (column, part) sums every 8th
// partial; all reductions run in a fixed order.  The row's m and l partials
// and each thread's first kEarly O partials are loaded together, before the
// weights are known, so the merge waits for one memory round trip rather
// than three.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a, int parts, float* o) {
  constexpr int kParts = 8;   // 256 threads = 32 columns x 8
  constexpr int kEarly = 24;  // O partials per thread loaded with m and l
  constexpr int kMl = kMaxDecodeParts / 256;  // m and l partials per thread
  static_assert(kMl * 256 == kMaxDecodeParts, "m and l partials split evenly");
  __shared__ float wsh[kMaxDecodeParts];
  __shared__ float red[8];
  __shared__ float osum[kParts][32];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int chunk = blockIdx.x % (D / 32);
  const int row = blockIdx.x / (D / 32);
  const int g = row % a.Hq, t = row / a.Hq;
  const float sl2 = a.scale_log2;
  const int c = tid % 32, part = tid / 32;
  const float* src = a.o_part + ((int64_t)t * a.Hq + g) * D + chunk * 32 + c;
  const int64_t pstride = (int64_t)a.M * a.Hq * D;
  float early[kEarly], mv[kMl], lv[kMl];
#pragma unroll
  for (int u = 0; u < kEarly; ++u) {
    const int p = part + u * kParts;
    early[u] = p < parts ? src[p * pstride] : 0.f;
  }
#pragma unroll
  for (int u = 0; u < kMl; ++u) {
    const int p = tid + 256 * u;
    const int64_t i = ((int64_t)p * a.Hq + g) * a.M + t;
    mv[u] = p < parts ? a.m_part[i] : -INFINITY;
    lv[u] = p < parts ? a.l_part[i] : 0.f;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < kMl; ++u) mloc = fmaxf(mloc, mv[u]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, off));
  if (lane == 0) red[wv] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float msafe = M == -INFINITY ? 0.f : M;
  float lloc = 0.f;
#pragma unroll
  for (int u = 0; u < kMl; ++u) {
    const int p = tid + 256 * u;
    if (p < parts) {
      const float wp = mv[u] == -INFINITY ? 0.f : exp2f((mv[u] - msafe) * sl2);
      wsh[p] = wp;
      lloc += wp * lv[u];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lloc += __shfl_xor(lloc, off);
  if (lane == 0) red[4 + wv] = lloc;
  __syncthreads();
  const float L = (red[4] + red[5]) + (red[6] + red[7]);
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kEarly; ++u) {
    const int p = part + u * kParts;
    if (p < parts) acc += wsh[p] * early[u];
  }
  // the rest (more than 8 kEarly partials): groups of 8 independent loads,
  // summed in partial order
  for (int p0 = part + kEarly * kParts; p0 < parts; p0 += 8 * kParts) {
    float vals[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * kParts;
      vals[u] = p < parts ? src[p * pstride] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * kParts;
      if (p < parts) acc += wsh[p] * vals[u];
    }
  }
  osum[part][c] = acc;
  __syncthreads();
  if (part == 0) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < kParts; ++i) sum += osum[i][c];
    o[((int64_t)t * a.Hq + g) * D + chunk * 32 + c] = sum / L;
  }
}

}  // namespace

int decode_parts(int ns) { return (ns + kDecWaves - 1) / kDecWaves; }

hipError_t launch_decode(const DecodeArgs& a, int D, const Stream& st) {
  const int per_head = decode_parts(a.NS);
  const dim3 grid(a.Hkv * per_head);
  if (D == 128)
    hipExtLaunchKernelGGL((decode_kernel<128>), grid, dim3(kDecThreads), 0, st.st, st.start,
                          st.stop, 0, a);
  else
    hipExtLaunchKernelGGL((decode_kernel<64>), grid, dim3(kDecThreads), 0, st.st, st.start,
                          st.stop, 0, a);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, float* o, int D, const Stream& st) {
  const int parts = decode_parts(a.NS);
  if (parts > kMaxDecodeParts) return hipErrorInvalidValue;
  const dim3 grid(a.M * a.Hq * (D / 32));
  if (D == 128)
    hipExtLaunchKernelGGL((decode_merge_kernel<128>), grid, dim3(256), 0, st.st, st.start, st.stop,
                          0, a, parts, o);
  else
    hipExtLaunchKernelGGL((decode_merge_kernel<64>), grid, dim3(256), 0, st.st, st.start, st.stop,
                          0, a, parts, o);
  return hipGetLastError();
}

}  // namespace skv
