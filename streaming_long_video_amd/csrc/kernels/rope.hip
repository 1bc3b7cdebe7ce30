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
// One thread owns one (token, pair) and rotates it in every head, so the
// trigonometry is done once per (token, pair).
#include "../skv_internal.h"
#include "bf16_device.h"

namespace skv {

namespace {

template <int D>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs r) {
  constexpr int HALF = D / 2;
  const int64_t item = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (item >= (int64_t)r.n_tokens * HALF) return;
  const int t = (int)(item / HALF), i = (int)(item % HALF);
  const double inv_freq = pow(r.theta, -2.0 * i / D);
  const double ang = ((double)(r.first_position + t) / r.scaling) * inv_freq;
  double s, c;
  sincos(ang, &s, &c);
  // rows of the first tensor, then of the second (if any)
  for (int hd = 0; hd < r.n_rows + r.n_rows2; ++hd) {
    const bool first = hd < r.n_rows;
    const int row = first ? hd : hd - r.n_rows;
    const int nr = first ? r.n_rows : r.n_rows2;
    const uint16_t* x = first ? r.x : r.x2;
    uint16_t* y = first ? r.y : r.y2;
    const int64_t base = ((int64_t)t * nr + row) * D;
    const double x0 = bf16_bits_to_f32(x[base + i]);
    const double x1 = bf16_bits_to_f32(x[base + i + HALF]);
    y[base + i] = f64_to_bf16_rne(fma(x0, c, -(x1 * s)));
    y[base + i + HALF] = f64_to_bf16_rne(fma(x0, s, x1 * c));
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& r, int D, const Stream& st) {
  const int64_t items = (int64_t)r.n_tokens * (D / 2);
  if (items == 0) return hipSuccess;
  const dim3 grid((unsigned)((items + 255) / 256));
  if (D == 128)
    hipExtLaunchKernelGGL((rope_kernel<128>), grid, dim3(256), 0, st.st, st.start, st.stop, 0, r);
  else
    hipExtLaunchKernelGGL((rope_kernel<64>), grid, dim3(256), 0, st.st, st.start, st.stop, 0, r);
  return hipGetLastError();
}

}  // namespace skv
