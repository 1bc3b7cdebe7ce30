// State update and detailed-cache append.
//
//   gather: C_n[h][s] = pool[h][sel[h][s]] for s < |C_n|, where the pool is
//     [C_{n-1}[h] ; frame tokens of KV head h] -- key row, value row and the
//     original position (paper.rainbus.top, method-steps section: the top-B
//     candidates of previous state plus frame become the new compressed state;
//     paperlayer.ai section 3.3: virtual positions are kept although the
//     state is physically shorter);
//   append: D[h][slot(p)] = frame token p for every token of the frame
//     (rainbus method steps: after frame n the frame's keys/values join the
//     detailed state, which keeps every video token for decoding).
//
// Both are row copies of d bf16 (128 or 256 bytes): 16-byte vector loads and
// stores, consecutive threads on consecutive 16-byte chunks of a row.
#include "../skv_internal.h"

namespace skv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kRowsPerBlock = 32;

template <int D>
__global__ __launch_bounds__(kCopyThreads) void gather_append_kernel(GatherArgs g,
                                                                     int gather_blocks) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  if (b < gather_blocks) {
    const int per_h = (g.newc + kRowsPerBlock - 1) / kRowsPerBlock;
    const int h = b / per_h;
    const int s0 = (b % per_h) * kRowsPerBlock;
    const int rows = min(kRowsPerBlock, g.newc - s0);
    for (int it = tid; it < 2 * rows * CH; it += kCopyThreads) {
      const int which = it / (rows * CH);  // 0: keys, 1: values
      const int rem = it % (rows * CH);
      const int s = s0 + rem / CH, col = (rem % CH) * 8;
      const int j = g.keep_all ? s : g.sel[(int64_t)h * g.B + s];
      const uint16_t* src;
      if (j < g.c)
        src = (which ? g.vc_prev : g.kc_prev) + ((int64_t)h * g.B + j) * D + col;
      else
        src = (which ? g.vf : g.kf) + ((int64_t)(j - g.c) * g.Hkv + h) * D + col;
      uint16_t* dst = (which ? g.vc_next : g.kc_next) + ((int64_t)h * g.B + s) * D + col;
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    }
    if (tid < rows) {
      const int s = s0 + tid;
      const int j = g.keep_all ? s : g.sel[(int64_t)h * g.B + s];
      g.pos_next[(int64_t)h * g.B + s] =
          j < g.c ? g.pos_prev[(int64_t)h * g.B + j] : g.pos_offset + g.frame_base + (j - g.c);
    }
    return;
  }
  // append the frame to the detailed cache
  const int ab = b - gather_blocks;
  const int per_h = (g.T + kRowsPerBlock - 1) / kRowsPerBlock;
  const int h = ab / per_h;
  const int t0 = (ab % per_h) * kRowsPerBlock;
  const int rows = min(kRowsPerBlock, g.T - t0);
  for (int it = tid; it < 2 * rows * CH; it += kCopyThreads) {
    const int which = it / (rows * CH);
    const int rem = it % (rows * CH);
    const int t = t0 + rem / CH, col = (rem % CH) * 8;
    int64_t slot = g.frame_base + t;
    if (g.ring) slot %= g.cap;
    const uint16_t* src = (which ? g.vf : g.kf) + ((int64_t)t * g.Hkv + h) * D + col;
    uint16_t* dst = (which ? g.vd : g.kd) + ((int64_t)h * g.cap + slot) * D + col;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

namespace {
hipError_t launch(const GatherArgs& g, int D, int gather_blocks, int append_blocks,
                  hipStream_t st) {
  const int blocks = gather_blocks + append_blocks;
  if (blocks == 0) return hipSuccess;
  if (D == 128)
    hipLaunchKernelGGL((gather_append_kernel<128>), dim3(blocks), dim3(kCopyThreads), 0, st, g,
                       gather_blocks);
  else
    hipLaunchKernelGGL((gather_append_kernel<64>), dim3(blocks), dim3(kCopyThreads), 0, st, g,
                       gather_blocks);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gather_append(const GatherArgs& g, int D, hipStream_t st) {
  const int gather_blocks = g.Hkv * ((g.newc + kRowsPerBlock - 1) / kRowsPerBlock);
  const int append_blocks = g.kd ? g.Hkv * ((g.T + kRowsPerBlock - 1) / kRowsPerBlock) : 0;
  return launch(g, D, gather_blocks, append_blocks, st);
}

hipError_t launch_append_only(const GatherArgs& g, int D, hipStream_t st) {
  return launch(g, D, 0, g.Hkv * ((g.T + kRowsPerBlock - 1) / kRowsPerBlock), st);
}

}  // namespace skv
