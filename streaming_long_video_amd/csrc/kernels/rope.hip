// Rotary position embedding at the tokens' original positions.
//
// The compressed state is physically shorter than the video, yet its keys
// keep the positions they arrived with, and cache building and text generation
// share one RoPE configuration (paperlayer summary, section 3.3; rainbus
// summary, prerequisites, RoPE scaling).  With rope_theta > 0 the library
// rotates each frame's q and k itself, before attention, so the keys stored in
// C and D are rotated once, at their original position.
//
// Pair (x_i, x_{i+d/2}) of a token at position p turns by the angle
// (p / scaling) * theta^(-2i/d).  Everything is computed in double precision
// -- the angle (p reaches 1e5 and beyond, where a float angle would be off by
// ~1e-2 rad), its cosine and sine and the rotation (when the two products
// nearly cancel, float cosines would move a small result by several bf16
// units) -- and the result is rounded once, straight from double, to bf16
// (nearest, ties to even).
// One thread owns one (token, pair) in kRopeHeads consecutive heads (a
// second grid dimension covers the heads): the trigonometry is shared by
// those heads, and every load of the thread is in flight at once.  The
// frequencies theta^(-2i/d) come from the host.
#include "../skv_internal.h"
#include "bf16_device.h"

namespace skv {

namespace {

constexpr int kRopeHeads = 4;  // heads per thread

template <int D>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs r) {
  constexpr int HALF = D / 2;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (int64_t)r.n_tokens * HALF) return;
  const int t = (int)(item / HALF), i = (int)(item % HALF);
  const int rows = r.n_rows + r.n_rows2;
  const int hd0 = (int)blockIdx.y * kRopeHeads;
  // rows of the first tensor, then of the second (if any)
  const uint16_t* src[kRopeHeads];
  uint16_t* dst[kRopeHeads];
  float x0[kRopeHeads], x1[kRopeHeads];
#pragma unroll
  for (int u = 0; u < kRopeHeads; ++u) {
    const int hd = min(hd0 + u, rows - 1);
    const bool first = hd < r.n_rows;
    const int row = first ? hd : hd - r.n_rows;
    const int nr = first ? r.n_rows : r.n_rows2;
    const int64_t base = ((int64_t)t * nr + row) * D + i;
    src[u] = (first ? r.x : r.x2) + base;
    dst[u] = (first ? r.y : r.y2) + base;
    x0[u] = bf16_bits_to_f32(src[u][0]);
    x1[u] = bf16_bits_to_f32(src[u][HALF]);
  }
  const double ang = ((double)(r.first_position + t) / r.scaling) * r.inv_freq[i];
  double s, c;
  sincos(ang, &s, &c);
#pragma unroll
  for (int u = 0; u < kRopeHeads; ++u) {
    if (hd0 + u >= rows) break;
    const double a0 = x0[u], a1 = x1[u];
    dst[u][0] = f64_to_bf16_rne(fma(a0, c, -(a1 * s)));
    dst[u][HALF] = f64_to_bf16_rne(fma(a0, s, a1 * c));
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& args, int D, const Stream& st) {
  const int64_t items = (int64_t)args.n_tokens * (D / 2);
  const int rows = args.n_rows + args.n_rows2;
  if (items == 0 || rows == 0) return hipSuccess;
  RopeArgs r = args;
  for (int i = 0; i < D / 2; ++i) r.inv_freq[i] = pow(r.theta, -2.0 * i / D);
  const dim3 grid((unsigned)((items + 255) / 256), (unsigned)((rows + kRopeHeads - 1) / kRopeHeads));
  if (D == 128)
    hipExtLaunchKernelGGL((rope_kernel<128>), grid, dim3(256), 0, st.st, st.start, st.stop, 0, r);
  else
    hipExtLaunchKernelGGL((rope_kernel<64>), grid, dim3(256), 0, st.st, st.start, st.stop, 0, r);
  return hipGetLastError();
}

}  // namespace skv
