// State update and detailed-cache append.
//
//   gather: C_n[h][s] = pool[h][sel[h][s]] for s < |C_n| (the positions only,
//     when the state is kept as positions into D), where the pool is
//     [C_{n-1}[h] ; frame tokens of KV head h] -- key row, value row and the
//     original position (paper.rainbus.top, method-steps section: the top-B
//     candidates of previous state plus frame become the new compressed state;
//     paperlayer.ai section 3.3: virtual positions are kept although the
//     state is physically shorter);
//   append: D[h][slot(p)] = frame token p for every token of the frame
//     (rainbus method steps: after frame n the frame's keys/values join the
//     detailed state, which keeps every video token for decoding).
//
// Both are copies of d-element bf16 rows.  A workgroup moves 32 rows (K and
// V); every thread issues all of its 16-byte loads before its stores (4 in
// flight per thread at d = 128), consecutive threads on consecutive 16-byte
// chunks of a row.
#include "../skv_internal.h"

namespace skv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kRowsPerBlock = 32;

template <int D>
__global__ __launch_bounds__(kCopyThreads) void gather_append_kernel(GatherArgs g,
                                                                     int gather_blocks) {
  constexpr int CH = D / 8;                                    // 16-byte chunks per row
  constexpr int PER = 2 * kRowsPerBlock * CH / kCopyThreads;  // chunks per thread (K and V)
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  u32x4 buf[PER];
  if (b < gather_blocks) {
    const int per_h = (g.newc + kRowsPerBlock - 1) / kRowsPerBlock;
    const int h = b / per_h;
    const int s0 = (b % per_h) * kRowsPerBlock;
    const int rows = min(kRowsPerBlock, g.newc - s0);
    const int32_t* sel = g.sel + (int64_t)h * g.sel_stride + s0;
    if (tid < rows) {
      const int j = g.keep_all ? s0 + tid : sel[tid];
      g.pos_next[(int64_t)h * g.B + s0 + tid] =
          j < g.c ? g.pos_prev[(int64_t)h * g.B + j] : g.pos_offset + g.frame_base + (j - g.c);
    }
    if (!g.kc_next) return;  // the state is kept as positions into D: no row copy
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = tid + i * kCopyThreads;
      const int which = it / (kRowsPerBlock * CH);  // 0: keys, 1: values
      const int r = (it / CH) % kRowsPerBlock, col = (it % CH) * 8;
      if (r < rows) {
        const int j = g.keep_all ? s0 + r : sel[r];
        const uint16_t* p =
            j < g.c ? (which ? g.vc_prev : g.kc_prev) + ((int64_t)h * g.B + j) * D + col
                    : (which ? g.vf : g.kf) + ((int64_t)(j - g.c) * g.Hkv + h) * D + col;
        buf[i] = *reinterpret_cast<const u32x4*>(p);
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int it = tid + i * kCopyThreads;
      const int which = it / (kRowsPerBlock * CH);
      const int r = (it / CH) % kRowsPerBlock, col = (it % CH) * 8;
      if (r < rows)
        *reinterpret_cast<u32x4*>((which ? g.vc_next : g.kc_next) +
                                  ((int64_t)h * g.B + s0 + r) * D + col) = buf[i];
    }
    return;
  }
  // append the frame to the detailed cache
  const int ab = b - gather_blocks;
  const int per_h = (g.T + kRowsPerBlock - 1) / kRowsPerBlock;
  const int h = ab / per_h;
  const int t0 = (ab % per_h) * kRowsPerBlock;
  const int rows = min(kRowsPerBlock, g.T - t0);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int it = tid + i * kCopyThreads;
    const int which = it / (kRowsPerBlock * CH);
    const int r = (it / CH) % kRowsPerBlock, col = (it % CH) * 8;
    if (r < rows)
      buf[i] = *reinterpret_cast<const u32x4*>((which ? g.vf : g.kf) +
                                               ((int64_t)(t0 + r) * g.Hkv + h) * D + col);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int it = tid + i * kCopyThreads;
    const int which = it / (kRowsPerBlock * CH);
    const int r = (it / CH) % kRowsPerBlock, col = (it % CH) * 8;
    if (r < rows) {
      int64_t slot = g.frame_base + t0 + r;
      if (g.ring) slot %= g.cap;
      *reinterpret_cast<u32x4*>((which ? g.vd : g.kd) + ((int64_t)h * g.cap + slot) * D + col) =
          buf[i];
    }
  }
}

namespace {
hipError_t launch(const GatherArgs& g, int D, int gather_blocks, int append_blocks,
                  const Stream& st) {
  const int blocks = gather_blocks + append_blocks;
  if (blocks == 0) return hipSuccess;
  if (D == 128)
    hipExtLaunchKernelGGL((gather_append_kernel<128>), dim3(blocks), dim3(kCopyThreads), 0, st.st, st.start, st.stop, 0, g,
                       gather_blocks);
  else
    hipExtLaunchKernelGGL((gather_append_kernel<64>), dim3(blocks), dim3(kCopyThreads), 0, st.st, st.start, st.stop, 0, g,
                       gather_blocks);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_gather_append(const GatherArgs& g, int D, const Stream& st) {
  const int gather_blocks = g.Hkv * ((g.newc + kRowsPerBlock - 1) / kRowsPerBlock);
  const int append_blocks = g.kd ? g.Hkv * ((g.T + kRowsPerBlock - 1) / kRowsPerBlock) : 0;
  return launch(g, D, gather_blocks, append_blocks, st);
}

hipError_t launch_append_only(const GatherArgs& g, int D, const Stream& st) {
  return launch(g, D, 0, g.Hkv * ((g.T + kRowsPerBlock - 1) / kRowsPerBlock), st);
}

}  // namespace skv
