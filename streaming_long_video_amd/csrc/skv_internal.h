// Internal interface between the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "plan.h"

namespace skv {

// A launch's stream and, when set, two events that the dispatch itself
// timestamps at the kernel's start and end (hipExtLaunchKernel).
struct Stream {
  hipStream_t st;
  hipEvent_t start = nullptr, stop = nullptr;
  Stream(hipStream_t s) : st(s) {}  // NOLINT: plain streams convert implicitly
  Stream(hipStream_t s, hipEvent_t a, hipEvent_t b) : st(s), start(a), stop(b) {}
};

// Raises the dynamic-LDS limit of kernel `fn` to `bytes` on the current
// device, once per device (safe to call from several host threads).
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Arguments of the two attention passes over the pool [C_{n-1} ; frame].
struct AttnArgs {
  const uint16_t* q;   // [T][Hq][D] bf16
  const uint16_t* kf;  // [T][Hkv][D] bf16, frame keys
  const uint16_t* vf;  // [T][Hkv][D] bf16, frame values
  const uint16_t* kc;  // [Hkv][ldc][D] bf16, state keys (rows [0, c) live)
  const uint16_t* vc;  // [Hkv][ldc][D] bf16, state values
  float* m_part;       // statistics pass: [Sst][Hq][tpad] per-split row log-sum-exp of the
                       // logits scaled by scale_log2 (base 2); full attention: [S][Hq][tpad]
                       // per-split row max of raw logits
  float* l_part;       // full attention: [S][Hq][tpad] per-split sum of exp relative to m
  float* o_out;        // [T][Hq][D] fp32 when S == 1, else [S][T][Hq][D] partials
  int out_bf16;        // S == 1: o_out holds [T][Hq][D] bf16 instead
  float* sig_part;     // [Hkv][rt][ldsig] per-row-tile score partials
  int64_t ldc;         // state rows per KV head (B)
  const int64_t* cpos;  // null, or [Hkv][ldcp] positions of the state tokens: state token
                        // j of head h is then row cpos[h*ldcp + j] - cpos_base of kc/vc
  int64_t cpos_base;
  int ldcp;
  int T, Hq, Hkv, G;
  int c;               // live state rows; pool = c + T
  int ntblk, nqblk, rt, tpad;
  int S;               // key splits of this launch
  int Sst;             // splits of the statistics pass (read by the output pass)
  int ldsig;
  float scale_log2;    // softmax scale * log2(e)
  int causal;
};

hipError_t launch_attn_stats(const AttnArgs& a, int D, const Stream& st);
// In-place (slot-stable) state update: positions of the state rows ([Hkv][ldpos]),
// live rows c, frame tokens T and the frame's first position.  pos null: the
// pool is in position order and the selection lists kept pool indices.  The
// selecting workgroup also moves the kept frame tokens (kf, vf: [T][Hkv][D])
// into their rows of kc, vc ([Hkv][ldpos][D]; null: positions only) and
// writes their positions.
struct InPlace {
  int64_t* pos;
  int ldpos, c, T;
  int64_t frame_pos0;
  const uint16_t* kf;
  const uint16_t* vf;
  uint16_t* kc;
  uint16_t* vc;
  int Hkv, D;
};
// Detailed-cache append done by extra workgroups of the select launch:
// D[h][slot(frame_base + t)] = frame token t.
struct AppendJob {
  const uint16_t* kf;  // [T][Hkv][D]
  const uint16_t* vf;
  uint16_t* kd;        // [Hkv][cap][D]
  uint16_t* vd;
  int64_t cap, frame_base;
  int T, Hkv, D, ring;
};
hipError_t launch_attn_out(const AttnArgs& a, int D, const Stream& st);
// The output pass forms P scaled by 2^12 (fp16 range) and removes the scale
// (exactly: a power of 2) before it writes O or its split partials.
constexpr float kOPartUnscale = 1.f / 4096.f;
// One launch: per KV head, sums the score partials (scores may be null),
// selects the top-B or keeps all (sel); concurrently, when o_part is given
// and S > 1, o[i] = sum_{s<S} o_part[s*o_elems + i] in split order (o fp32,
// or bf16 rounded to nearest even when o_bf16).
// Standalone mode: rt = 1 and sig_part holds the scores.  In place (ip.pos
// set), each selection row holds the rows to refill at [0, T), the kept frame
// tokens at [T, 2T) and their count at 2T, and the launch applies the moves;
// app (may be null) adds the detailed-cache append to the same launch.
hipError_t launch_select(const float* sig_part, int rt, int ldsig, int hkv, int pool,
                         int budget, float* scores, int ldscores, int32_t* sel, int ldsel,
                         const float* o_part, int S, int64_t o_elems, void* o, bool o_bf16,
                         bool shared,
                         bool recent, const InPlace& ip, const AppendJob* app,
                         const Stream& st);

struct GatherArgs {
  const uint16_t* kc_prev;  // [Hkv][B][D]
  const uint16_t* vc_prev;
  const int64_t* pos_prev;  // [Hkv][B]
  const uint16_t* kf;       // [T][Hkv][D]
  const uint16_t* vf;
  const int32_t* sel;       // [Hkv][sel_stride] pool indices, ascending (ignored if
                            // keep_all)
  int sel_stride;           // selection row stride, or 0 when one kept set serves
                            // every head (SHARED)
  uint16_t* kc_next;        // null: positions only (state kept as positions into D)
  uint16_t* vc_next;
  int64_t* pos_next;
  uint16_t* kd;             // [Hkv][cap][D] detailed cache (null: no append)
  uint16_t* vd;
  int64_t cap;
  int64_t frame_base;       // n*T: frame index of token 0 (relative to the offset)
  int64_t pos_offset;
  int B, T, Hkv, c, newc;
  int keep_all;             // pool <= B: C_n = [C_{n-1} ; frame]
  int ring;
};
hipError_t launch_gather_append(const GatherArgs& g, int D, const Stream& st);
hipError_t launch_append_only(const GatherArgs& g, int D, const Stream& st);

// Full-attention baseline (single online-softmax pass): the pool is
// [D[0:c) ; frame], causal within the frame.  With S == 1 it writes the
// normalised O to o_out; otherwise unnormalised partials plus (m, l).
hipError_t launch_full_attn(const AttnArgs& a, int D, const Stream& st);
// Combines the unnormalised split partials of the full-attention baseline.
// Decoding over the detailed state: one wave per (KV head, split); the four
// waves of a workgroup write one merged partial ([parts][...] below).
struct DecodeArgs {
  const uint16_t* q;   // [M][Hq][D] bf16 text queries
  const uint16_t* kd;  // [Hkv][cap][D] bf16 detailed keys
  const uint16_t* vd;  // [Hkv][cap][D] bf16 detailed values
  float* m_part;       // [parts][Hq][M] row max of raw logits per workgroup partial
  float* l_part;       // [parts][Hq][M] row sum (relative to m)
  float* o_part;       // [parts][M][Hq][D] unnormalised O
  int64_t cap;         // D rows per KV head
  int64_t len;         // live D rows per KV head (slots [0, len))
  int M, Hq, Hkv, G, NS;
  float scale_log2;
};
hipError_t launch_decode(const DecodeArgs& a, int D, const Stream& st);
// Workgroup partials the decode launch writes per KV head for NS splits.
int decode_parts(int ns);
constexpr int kMaxDecodeParts = 1024;
// o[M][Hq][D] from the workgroup partials, in a fixed order.
hipError_t launch_decode_merge(const DecodeArgs& a, float* o, int D, const Stream& st);

// Rotary embedding of n_tokens x n_rows rows of D bf16 values (x -> y; y may
// be x) at positions first_position + token; optionally a second tensor of
// the same tokens with n_rows2 rows (x2 -> y2) in the same launch.
struct RopeArgs {
  const uint16_t* x;
  uint16_t* y;
  const uint16_t* x2;
  uint16_t* y2;
  int n_tokens, n_rows, n_rows2;
  int64_t first_position;
  double theta, scaling;
  double inv_freq[64];  // theta^(-2i/D), filled by launch_rope
};
hipError_t launch_rope(const RopeArgs& r, int D, const Stream& st);

hipError_t launch_full_combine(const AttnArgs& a, float* o, int D, const Stream& st);

// The frame's q/k/v projection with RoPE (front end): q = rope(X W_Q),
// k = rope(X W_K), v = X W_V.
struct FrontArgs {
  const uint16_t* x;  // [T][hidden] bf16 hidden states
  const uint16_t* w;  // [(Hq + 2 Hkv) D][hidden] bf16, rows: Q heads, K heads, V heads
  uint16_t* q;        // [T][Hq][D] bf16
  uint16_t* k;        // [T][Hkv][D] bf16
  uint16_t* v;        // [T][Hkv][D] bf16
  int T, hidden, Hq, Hkv;
  int64_t first_position;  // position of token 0
  double theta, scaling;   // theta <= 0: no rotation
  double inv_freq[64];     // theta^(-2i/D) for pair index i < D/2 (host-computed)
  int S;                   // splits of the hidden dimension
  float* part;             // S > 1: [S][feature tiles][T][128] fp32 partial sums
  double* rot;             // S > 1: [T][D/2] (cos, sin) of each token's angle per pair index
};
// splits of the hidden dimension the front end uses, and the bytes of its
// partial sums (0 when it does not split)
int qkv_rope_splits(int T, int hidden, int heads, int D);
size_t qkv_rope_workspace_bytes(int T, int hidden, int heads, int D);
hipError_t launch_qkv_rope(const FrontArgs& a, int D, const Stream& st);

// App. A diagnostics of the last frame (one workgroup per budget).
constexpr int kMaxMassBudgets = 64;
struct MassArgs {
  const float* scores;  // [Hkv][ldscores] per-KV-head importance of the pool
  int ldscores, Hkv;
  int pool;             // tokens through the frame
  int c;                // tokens of earlier frames
  int have_prev;        // sets hold the previous frame's kept sets
  uint32_t* sets;       // [n_budgets][ldsets] bit j of word j/32: token j kept
  int ldsets;
  float* out;           // [n_budgets][3]
  int32_t budgets[kMaxMassBudgets];
};
hipError_t launch_attention_mass(const MassArgs& m, int n_budgets, const Stream& st);

}  // namespace skv
