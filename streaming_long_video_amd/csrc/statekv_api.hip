// C ABI of the StateKV streaming video-prefill library (declared in statekv.h).
//
// Host side of the per-frame step: argument checks, the workspace carve-up
// (plan.cpp), the launch sequence on the caller's stream, and the host mirror
// of the layer's progress (frames seen, live state size, detailed-cache
// length, which compressed-state buffer is current).  Every quantity the
// launches need is known on the host ahead of time, so nothing is read back
// from the device.
#include <math.h>

#include <mutex>
#include <new>
#include <vector>

#include "plan.h"
#include "skv_internal.h"

// Timing hook state: one (kernel, before, after) event triple per recorded launch.
struct ProfRecord {
  int kernel;
  hipEvent_t before, after;
};

struct statekv_layer {
  skv::Plan plan;
  char* ws;          // device workspace base
  int device;        // device current at init (the workspace's)
  int64_t n;         // frames seen
  int32_t c;         // live compressed-state rows
  int32_t cur;       // index (0/1) of the buffer holding C_n
  int32_t last_pool; // pool size of the last frame
  int32_t mode;      // 0 unused, 1 StateKV, 2 full attention
  // timing hooks
  uint32_t prof_mask;
  std::vector<ProfRecord> prof;  // pre-created events
  size_t prof_used;
};

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Device scratch of statekv_decode_attention_noalloc: the decoding kernels'
// split partials (row max, row sum, O) for callers that cannot allocate.
// Every GPU holds its own copy for the life of the process; host code never
// passes the array's name to a kernel (on the host it only names the
// symbol), only the per-device address resolved below.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
bool scratch_done[kMaxDevices];
hipError_t scratch_status[kMaxDevices];
void* scratch_ptr[kMaxDevices];

// Resolves the device address of `scratch` once per device, with that device
// current (the caller's).  Returns the cached status of that one call.
hipError_t resolve_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_done[dev]) {
    void* ptr = nullptr;
    scratch_status[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_status[dev] == hipSuccess ? ptr : nullptr;
    scratch_done[dev] = true;
  }
  return scratch_status[dev];
}

template <class T>
T* at(const statekv_layer* L, size_t off) {
  return reinterpret_cast<T*>(L->ws + off);
}

int hip_status(hipError_t e) { return e == hipSuccess ? STATEKV_OK : STATEKV_ERR_HIP; }

skv::AttnArgs attn_args(const statekv_layer* L, const void* q, const void* k, const void* v) {
  const skv::Plan& p = L->plan;
  skv::AttnArgs a = {};
  a.q = static_cast<const uint16_t*>(q);
  a.kf = static_cast<const uint16_t*>(k);
  a.vf = static_cast<const uint16_t*>(v);
  a.m_part = at<float>(L, p.off_m);
  a.l_part = at<float>(L, p.off_l);
  a.sig_part = at<float>(L, p.off_sig);
  a.T = p.T;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.ntblk = p.ntblk;
  a.nqblk = p.nqblk;
  a.rt = p.rt;
  a.tpad = p.tpad;
  a.ldsig = p.ldsig;
  a.scale_log2 = p.scale * kLog2e;
  a.causal = (p.flags & STATEKV_FLAG_NONCAUSAL_FRAME) ? 0 : 1;
  return a;
}

bool aligned16(const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; }

// Runs one kernel launch; when the timing hook asks for it, the dispatch
// itself timestamps two events at the kernel's start and end.
template <class F>
hipError_t timed(statekv_layer* L, int kernel, hipStream_t st, F&& launch) {
  if ((L->prof_mask >> kernel) & 1u && L->prof_used < L->prof.size()) {
    ProfRecord* r = &L->prof[L->prof_used++];
    r->kernel = kernel;
    return launch(skv::Stream(st, r->before, r->after));
  }
  return launch(skv::Stream(st));
}

// With in-library RoPE: rotate the frame's q and k into the workspace at the
// frame's original positions and hand back the rotated copies.
hipError_t rotate_frame(statekv_layer* L, hipStream_t st, const void** q, const void** k) {
  const skv::Plan& p = L->plan;
  if (!(p.rope_theta > 0.0)) return hipSuccess;
  skv::RopeArgs r = {};
  r.x = static_cast<const uint16_t*>(*q);
  r.y = at<uint16_t>(L, p.off_qrot);
  r.x2 = static_cast<const uint16_t*>(*k);
  r.y2 = at<uint16_t>(L, p.off_krot);
  r.n_tokens = p.T;
  r.n_rows = p.Hq;
  r.n_rows2 = p.Hkv;
  r.first_position = p.offset + L->n * (int64_t)p.T;
  r.theta = p.rope_theta;
  r.scaling = p.rope_scaling;
  *q = r.y;
  *k = r.y2;
  return timed(L, STATEKV_KERNEL_ROPE, st,
               [&](const skv::Stream& ks) { return skv::launch_rope(r, p.D, ks); });
}

}  // namespace

extern "C" {

int statekv_workspace_bytes(const statekv_layer_config* cfg, size_t* bytes) {
  if (!bytes) return STATEKV_ERR_INVALID_ARGUMENT;
  skv::Plan p;
  const int st = skv::make_plan(cfg, &p);
  if (st != STATEKV_OK) return st;
  *bytes = p.total;
  return STATEKV_OK;
}

int statekv_init_layer(const statekv_layer_config* cfg, void* d_workspace, size_t workspace_bytes,
                       statekv_layer** out) {
  if (!out || !d_workspace) return STATEKV_ERR_INVALID_ARGUMENT;
  skv::Plan p;
  const int st = skv::make_plan(cfg, &p);
  if (st != STATEKV_OK) return st;
  if (workspace_bytes < p.total) return STATEKV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(d_workspace) & 255u) return STATEKV_ERR_WORKSPACE;
  // the no-allocation decoding entry point's scratch on the current device
  // (the workspace's); a failure here only affects that entry point, which
  // reports it, and without a device the address is resolved on its first call
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess) (void)resolve_scratch(dev);
  else dev = -1;
  statekv_layer* L = new (std::nothrow) statekv_layer();
  if (!L) return STATEKV_ERR_INVALID_ARGUMENT;
  L->plan = p;
  L->ws = static_cast<char*>(d_workspace);
  L->device = dev;
  L->n = 0;
  L->c = 0;
  L->cur = 0;
  L->last_pool = 0;
  L->mode = 0;
  L->prof_mask = 0;
  L->prof_used = 0;
  *out = L;
  return STATEKV_OK;
}

int statekv_prefill_frame(statekv_layer* L, const void* q, const void* k, const void* v, void* o,
                          void* stream) {
  if (!L || !q || !k || !v || !o) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (L->mode == 2) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  const bool ring = p.flags & STATEKV_FLAG_D_RING;
  const bool shared = p.flags & STATEKV_FLAG_SELECT_SHARED;
  const bool c_in_d = p.flags & STATEKV_FLAG_C_IN_D;
  const bool in_place = p.flags & STATEKV_FLAG_SLOT_STABLE;
  const int64_t next_len = (L->n + 1) * (int64_t)p.T;
  if (!ring && next_len > p.cap) return STATEKV_ERR_CAPACITY;
  if (L->n * (int64_t)p.T + p.T + p.offset > ((int64_t)1 << 62)) return STATEKV_ERR_CAPACITY;
  hipStream_t st = static_cast<hipStream_t>(stream);
  L->mode = 1;

  const int cur = L->cur, nxt = in_place ? cur : cur ^ 1;
  const int c = L->c;
  const int pool = c + p.T;
  const int newc = pool < p.B ? pool : p.B;

  hipError_t e = rotate_frame(L, st, &q, &k);
  skv::AttnArgs a = attn_args(L, q, k, v);
  if (c_in_d) {  // state rows are D rows, found through the state's positions
    a.kc = at<uint16_t>(L, p.off_dk);
    a.vc = at<uint16_t>(L, p.off_dv);
    a.ldc = p.cap;
    a.cpos = at<int64_t>(L, p.off_cpos[cur]);
    a.cpos_base = p.offset;
    a.ldcp = p.B;
  } else {
    a.kc = at<uint16_t>(L, p.off_ck[cur]);
    a.vc = at<uint16_t>(L, p.off_cv[cur]);
    a.ldc = p.B;
  }
  a.c = c;
  a.S = skv::splits_for_pool(p, pool);
  float* opart = at<float>(L, p.off_o);
  const bool out_bf16 = p.flags & STATEKV_FLAG_OUT_BF16;
  a.o_out = a.S == 1 ? static_cast<float*>(o) : opart;  // S == 1: written as is (fp32 or bf16)
  a.out_bf16 = out_bf16 ? 1 : 0;

  a.Sst = skv::stat_splits_for_pool(p, pool);
  skv::AttnArgs a1 = a;
  a1.S = a.Sst;
  if (e == hipSuccess)
    e = timed(L, STATEKV_KERNEL_ATTN_STATS, st,
              [&](const skv::Stream& ks) { return skv::launch_attn_stats(a1, p.D, ks); });
  if (e == hipSuccess)
    e = timed(L, STATEKV_KERNEL_ATTN_OUT, st, [&](const skv::Stream& ks) { return skv::launch_attn_out(a, p.D, ks); });
  // in place, the select launch also moves the kept frame tokens into C and
  // appends the frame to D: no state-update launch follows
  skv::InPlace ip = {};
  skv::AppendJob app = {};
  if (in_place) {
    ip.pos = at<int64_t>(L, p.off_cpos[cur]);
    ip.ldpos = p.B;
    ip.c = c;
    ip.T = p.T;
    ip.frame_pos0 = p.offset + L->n * (int64_t)p.T;
    ip.kf = a.kf;
    ip.vf = a.vf;
    ip.kc = c_in_d ? nullptr : at<uint16_t>(L, p.off_ck[cur]);
    ip.vc = c_in_d ? nullptr : at<uint16_t>(L, p.off_cv[cur]);
    ip.Hkv = p.Hkv;
    ip.D = p.D;
    app.kf = a.kf;
    app.vf = a.vf;
    app.kd = at<uint16_t>(L, p.off_dk);
    app.vd = at<uint16_t>(L, p.off_dv);
    app.cap = p.cap;
    app.frame_base = L->n * (int64_t)p.T;
    app.T = p.T;
    app.Hkv = p.Hkv;
    app.D = p.D;
    app.ring = ring;
  }
  if (e == hipSuccess)
    e = timed(L, STATEKV_KERNEL_SELECT, st, [&](const skv::Stream& ks) {
      return skv::launch_select(a.sig_part, p.rt, p.ldsig, p.Hkv, pool, p.B,
                                at<float>(L, p.off_scores), p.ldsig, at<int32_t>(L, p.off_sel),
                                p.ldsel, a.S > 1 ? opart : nullptr, a.S,
                                (int64_t)p.T * p.Hq * p.D, o, out_bf16, shared,
                                (p.flags & STATEKV_FLAG_SELECT_RECENT) != 0, ip,
                                in_place ? &app : nullptr, ks);
    });
  if (e == hipSuccess && !in_place) {
    skv::GatherArgs g = {};
    g.kc_prev = c_in_d ? nullptr : a.kc;
    g.vc_prev = c_in_d ? nullptr : a.vc;
    g.pos_prev = at<int64_t>(L, p.off_cpos[cur]);
    g.kf = a.kf;
    g.vf = a.vf;
    g.sel = at<int32_t>(L, p.off_sel);
    g.sel_stride = (shared && !(p.flags & STATEKV_FLAG_SELECT_RECENT)) ? 0 : p.ldsel;
    g.kc_next = c_in_d ? nullptr : at<uint16_t>(L, p.off_ck[nxt]);
    g.vc_next = c_in_d ? nullptr : at<uint16_t>(L, p.off_cv[nxt]);
    g.pos_next = at<int64_t>(L, p.off_cpos[nxt]);
    g.kd = at<uint16_t>(L, p.off_dk);
    g.vd = at<uint16_t>(L, p.off_dv);
    g.cap = p.cap;
    g.frame_base = L->n * (int64_t)p.T;
    g.pos_offset = p.offset;
    g.B = p.B;
    g.T = p.T;
    g.Hkv = p.Hkv;
    g.c = c;
    g.newc = newc;
    g.keep_all = pool <= p.B;
    g.ring = ring;
    e = timed(L, STATEKV_KERNEL_GATHER, st,
              [&](const skv::Stream& ks) { return skv::launch_gather_append(g, p.D, ks); });
  }
  if (e != hipSuccess) return hip_status(e);
  L->cur = nxt;
  L->c = newc;
  L->last_pool = pool;
  L->n += 1;
  return STATEKV_OK;
}

int statekv_full_attention_frame(statekv_layer* L, const void* q, const void* k, const void* v,
                                 float* o, void* stream) {
  if (!L || !q || !k || !v || !o) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (L->mode == 1) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  if (p.flags & STATEKV_FLAG_OUT_BF16) return STATEKV_ERR_INVALID_ARGUMENT;  // fp32 output only
  if (p.flags & STATEKV_FLAG_D_RING) return STATEKV_ERR_UNSUPPORTED;
  const int64_t hist = L->n * (int64_t)p.T;
  if (hist + p.T > p.cap) return STATEKV_ERR_CAPACITY;
  if (hist + p.T > (int64_t)0x7FFFFFFF) return STATEKV_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  L->mode = 2;

  hipError_t e = rotate_frame(L, st, &q, &k);
  skv::GatherArgs g = {};
  g.kf = static_cast<const uint16_t*>(k);
  g.vf = static_cast<const uint16_t*>(v);
  g.kd = at<uint16_t>(L, p.off_dk);
  g.vd = at<uint16_t>(L, p.off_dv);
  g.cap = p.cap;
  g.frame_base = hist;
  g.B = p.B;
  g.T = p.T;
  g.Hkv = p.Hkv;
  if (e == hipSuccess)
    e = timed(L, STATEKV_KERNEL_GATHER, st,
              [&](const skv::Stream& ks) { return skv::launch_append_only(g, p.D, ks); });

  skv::AttnArgs a = attn_args(L, q, k, v);
  a.kc = at<uint16_t>(L, p.off_dk);
  a.vc = at<uint16_t>(L, p.off_dv);
  a.ldc = p.cap;
  a.c = (int)hist;
  const int tiles = (int)((hist + p.T + skv::kKeyTile - 1) / skv::kKeyTile);
  a.S = p.full_splits < tiles ? p.full_splits : tiles;
  a.Sst = a.S;
  a.o_out = a.S == 1 ? o : at<float>(L, p.off_o);
  if (e == hipSuccess)
    e = timed(L, STATEKV_KERNEL_ATTN_OUT, st, [&](const skv::Stream& ks) { return skv::launch_full_attn(a, p.D, ks); });
  if (e == hipSuccess && a.S > 1)
    e = timed(L, STATEKV_KERNEL_SPLIT_SUM, st,
              [&](const skv::Stream& ks) { return skv::launch_full_combine(a, o, p.D, ks); });
  if (e != hipSuccess) return hip_status(e);
  L->n += 1;
  return STATEKV_OK;
}

}  // extern "C"

namespace {
// Decoding over D with the split partials at m_part / l_part ([parts][Hq][M]
// floats each) and o_part ([parts][M][Hq][D] floats), room for max_parts
// workgroup partials.
int decode_into(statekv_layer* L, const void* q, int32_t n_queries, float* o, void* stream,
                float* m_part, float* l_part, float* o_part, int64_t max_parts) {
  const skv::Plan& p = L->plan;
  const int64_t hist = L->n * (int64_t)p.T;
  const int64_t len = hist < p.cap ? hist : p.cap;
  if (len <= 0) return STATEKV_ERR_INVALID_ARGUMENT;
  hipStream_t st = static_cast<hipStream_t>(stream);

  // splits (one wave each): about two waves per SIMD over all KV heads, at
  // least 32 keys per wave, at most four per workgroup partial
  const int64_t want = (2048 + p.Hkv - 1) / p.Hkv;
  const int64_t by_len = (len + 31) / 32;
  if (max_parts > skv::kMaxDecodeParts) max_parts = skv::kMaxDecodeParts;
  int64_t ns = want < by_len ? want : by_len;
  if (ns > 4 * max_parts) ns = 4 * max_parts;
  if (ns < 1) ns = 1;
  skv::DecodeArgs d = {};
  d.q = static_cast<const uint16_t*>(q);
  d.kd = at<uint16_t>(L, p.off_dk);
  d.vd = at<uint16_t>(L, p.off_dv);
  d.m_part = m_part;
  d.l_part = l_part;
  d.o_part = o_part;
  d.cap = p.cap;
  d.len = len;
  d.M = n_queries;
  d.Hq = p.Hq;
  d.Hkv = p.Hkv;
  d.G = p.G;
  d.NS = (int)ns;
  d.scale_log2 = p.scale * kLog2e;
  hipError_t e = timed(L, STATEKV_KERNEL_DECODE, st,
                       [&](const skv::Stream& ks) { return skv::launch_decode(d, p.D, ks); });
  if (e == hipSuccess)
    e = timed(L, STATEKV_KERNEL_SPLIT_SUM, st,
              [&](const skv::Stream& ks) { return skv::launch_decode_merge(d, o, p.D, ks); });
  return hip_status(e);
}

int check_decode_args(const statekv_layer* L, const void* q, int32_t n_queries, const float* o) {
  if (!L || !q || !o || n_queries < 1) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(o)) return STATEKV_ERR_INVALID_ARGUMENT;
  if (L->plan.G * (int64_t)n_queries > 32) return STATEKV_ERR_UNSUPPORTED;
  if (L->n < 1) return STATEKV_ERR_INVALID_ARGUMENT;
  return STATEKV_OK;
}
}  // namespace

extern "C" {

int statekv_decode_attention(statekv_layer* L, const void* q, int32_t n_queries, float* o,
                             void* stream) {
  const int chk = check_decode_args(L, q, n_queries, o);
  if (chk != STATEKV_OK) return chk;
  const skv::Plan& p = L->plan;
  // the workgroup partials live in the workspace's split-partial regions
  const int64_t opart = p.splits > p.full_splits ? p.splits : p.full_splits;
  const int64_t parts_o = opart * p.T / n_queries;
  const int64_t parts_ml = (int64_t)p.part_splits * p.tpad / n_queries;
  const int64_t max_parts = parts_o < parts_ml ? parts_o : parts_ml;
  return decode_into(L, q, n_queries, o, stream, at<float>(L, p.off_m), at<float>(L, p.off_l),
                     at<float>(L, p.off_o), max_parts);
}

int statekv_decode_attention_noalloc(statekv_layer* L, const void* q, int32_t n_queries,
                                     float* o, void* stream) {
  const int chk = check_decode_args(L, q, n_queries, o);
  if (chk != STATEKV_OK) return chk;
  const skv::Plan& p = L->plan;
  if (L->device < 0) {  // no device was current at init: take the current one now
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return STATEKV_ERR_HIP;
    L->device = dev;
  }
  if (resolve_scratch(L->device) != hipSuccess) return STATEKV_ERR_HIP;
  char* base = static_cast<char*>(scratch_ptr[L->device]);
  // carve [parts][Hq][M] row maxima, the same for row sums, then
  // [parts][M][Hq][D] O partials out of the fixed scratch
  const size_t rows = (size_t)p.Hq * (size_t)n_queries;
  const size_t per_part = rows * (2 + (size_t)p.D) * sizeof(float);
  const size_t room = kNoAllocScratchBytes - 2 * 256;
  const int64_t max_parts = (int64_t)(room / per_part);
  if (max_parts < 1) return STATEKV_ERR_UNSUPPORTED;  // cannot happen for G*M <= 32, Hkv < 500
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t ml_bytes = up((size_t)max_parts * rows * sizeof(float));
  float* m_part = reinterpret_cast<float*>(base);
  float* l_part = reinterpret_cast<float*>(base + ml_bytes);
  float* o_part = reinterpret_cast<float*>(base + 2 * ml_bytes);
  if (2 * ml_bytes + (size_t)max_parts * rows * p.D * sizeof(float) > kNoAllocScratchBytes)
    return STATEKV_ERR_UNSUPPORTED;
  return decode_into(L, q, n_queries, o, stream, m_part, l_part, o_part, max_parts);
}

int statekv_rope(statekv_layer* L, void* x, int32_t n_tokens, int32_t n_heads,
                 int64_t first_position, void* stream) {
  if (!L || !x || n_tokens < 1 || n_heads < 1 || first_position < 0)
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(x)) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  if (!(p.rope_theta > 0.0)) return STATEKV_ERR_INVALID_ARGUMENT;
  skv::RopeArgs r = {};
  r.x = static_cast<const uint16_t*>(x);
  r.y = static_cast<uint16_t*>(x);
  r.n_tokens = n_tokens;
  r.n_rows = n_heads;
  r.first_position = first_position;
  r.theta = p.rope_theta;
  r.scaling = p.rope_scaling;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(timed(L, STATEKV_KERNEL_ROPE, st, [&](const skv::Stream& ks) {
    return skv::launch_rope(r, p.D, ks);
  }));
}

int statekv_state(const statekv_layer* L, statekv_state_view* out) {
  if (!L || !out) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  statekv_state_view v = {};
  const bool c_in_d = p.flags & STATEKV_FLAG_C_IN_D;
  v.k = c_in_d ? nullptr : at<uint16_t>(L, p.off_ck[L->cur]);
  v.v = c_in_d ? nullptr : at<uint16_t>(L, p.off_cv[L->cur]);
  v.pos = at<int64_t>(L, p.off_cpos[L->cur]);
  v.last_scores = at<float>(L, p.off_scores);
  v.count = L->c;
  v.capacity = p.B;
  v.n_kv_heads = p.Hkv;
  v.head_dim = p.D;
  v.last_pool = L->mode == 1 ? L->last_pool : 0;
  v.scores_stride = p.ldsig;
  v.frames_seen = L->n;
  *out = v;
  return STATEKV_OK;
}

int statekv_detailed_cache(const statekv_layer* L, statekv_cache_view* out) {
  if (!L || !out) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  statekv_cache_view v = {};
  v.k = at<uint16_t>(L, p.off_dk);
  v.v = at<uint16_t>(L, p.off_dv);
  const int64_t total = L->n * (int64_t)p.T;
  v.length = total < p.cap ? total : p.cap;
  v.capacity = p.cap;
  v.start = p.offset + (total > p.cap ? total - p.cap : 0);
  v.n_kv_heads = p.Hkv;
  v.head_dim = p.D;
  *out = v;
  return STATEKV_OK;
}

int statekv_reset_layer(statekv_layer* L) {
  if (!L) return STATEKV_ERR_INVALID_ARGUMENT;
  L->n = 0;
  L->c = 0;
  L->cur = 0;
  L->last_pool = 0;
  L->mode = 0;
  return STATEKV_OK;
}

int statekv_restore_layer(statekv_layer* L, int64_t frames_seen, int32_t count) {
  if (!L || frames_seen < 0 || count < 0) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  const int64_t hist = frames_seen * (int64_t)p.T;
  if (count != (hist < p.B ? hist : (int64_t)p.B)) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(p.flags & STATEKV_FLAG_D_RING) && hist > p.cap) return STATEKV_ERR_CAPACITY;
  L->n = frames_seen;
  L->c = count;
  L->last_pool = 0;
  L->mode = frames_seen > 0 ? 1 : 0;
  return STATEKV_OK;
}

int statekv_launch_plan_for(const statekv_layer* L, int32_t pool, statekv_launch_plan* out) {
  if (!L || !out || pool < 1 || pool > L->plan.max_pool) return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  out->out_splits = skv::splits_for_pool(p, pool);
  out->stat_splits = skv::stat_splits_for_pool(p, pool);
  out->row_tiles = p.rt;
  out->key_tiles = (pool + skv::kKeyTile - 1) / skv::kKeyTile;
  return STATEKV_OK;
}

int statekv_mass_set_words(const statekv_layer* L, int32_t* words) {
  if (!L || !words) return STATEKV_ERR_INVALID_ARGUMENT;
  *words = (L->plan.max_pool + 31) / 32;
  return STATEKV_OK;
}

int statekv_attention_mass(statekv_layer* L, const int32_t* budgets, int32_t n_budgets,
                           uint32_t* sets, float* out, void* stream) {
  if (!L || !budgets || !sets || !out) return STATEKV_ERR_INVALID_ARGUMENT;
  if (n_budgets < 1 || n_budgets > skv::kMaxMassBudgets) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(out) || (reinterpret_cast<uintptr_t>(sets) & 3u))
    return STATEKV_ERR_INVALID_ARGUMENT;
  const skv::Plan& p = L->plan;
  // the last frame must have seen every token: no eviction so far
  if (L->mode != 1 || L->n < 1 || L->last_pool <= 0) return STATEKV_ERR_INVALID_ARGUMENT;
  if ((int64_t)L->last_pool != L->n * (int64_t)p.T) return STATEKV_ERR_INVALID_ARGUMENT;
  skv::MassArgs m = {};
  for (int i = 0; i < n_budgets; ++i) {
    if (budgets[i] < 1) return STATEKV_ERR_INVALID_ARGUMENT;
    m.budgets[i] = budgets[i];
  }
  m.scores = at<float>(L, p.off_scores);
  m.ldscores = p.ldsig;
  m.Hkv = p.Hkv;
  m.pool = L->last_pool;
  m.c = L->last_pool - p.T;
  m.have_prev = L->n > 1;
  m.sets = sets;
  m.ldsets = (p.max_pool + 31) / 32;
  m.out = out;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(timed(L, STATEKV_KERNEL_MASS, st, [&](const skv::Stream& ks) {
    return skv::launch_attention_mass(m, n_budgets, ks);
  }));
}

namespace {
void destroy_profile_events(statekv_layer* L) {
  // teardown: a failed destroy leaves nothing to recover
  for (ProfRecord& r : L->prof) {
    (void)hipEventDestroy(r.before);
    (void)hipEventDestroy(r.after);
  }
  L->prof.clear();
  L->prof_used = 0;
  L->prof_mask = 0;
}
}  // namespace

int statekv_profile_start(statekv_layer* L, uint32_t kernel_mask, int32_t max_records) {
  if (!L || max_records < 0 || (kernel_mask >> STATEKV_NUM_KERNELS))
    return STATEKV_ERR_INVALID_ARGUMENT;
  destroy_profile_events(L);
  L->prof.reserve((size_t)max_records);
  for (int32_t i = 0; i < max_records; ++i) {
    ProfRecord r = {0, nullptr, nullptr};
    if (hipEventCreate(&r.before) != hipSuccess) {
      destroy_profile_events(L);
      return STATEKV_ERR_HIP;
    }
    if (hipEventCreate(&r.after) != hipSuccess) {
      (void)hipEventDestroy(r.before);
      destroy_profile_events(L);
      return STATEKV_ERR_HIP;
    }
    L->prof.push_back(r);
  }
  L->prof_mask = kernel_mask;
  return STATEKV_OK;
}

int statekv_profile_stop(statekv_layer* L, double* total_ms, int64_t* launches) {
  if (!L) return STATEKV_ERR_INVALID_ARGUMENT;
  double ms[STATEKV_NUM_KERNELS] = {0};
  int64_t cnt[STATEKV_NUM_KERNELS] = {0};
  int status = STATEKV_OK;
  for (size_t i = 0; i < L->prof_used; ++i) {
    const ProfRecord& r = L->prof[i];
    float t = 0.f;
    if (hipEventSynchronize(r.after) != hipSuccess ||
        hipEventElapsedTime(&t, r.before, r.after) != hipSuccess) {
      status = STATEKV_ERR_HIP;
      break;
    }
    ms[r.kernel] += t;
    cnt[r.kernel] += 1;
  }
  destroy_profile_events(L);
  for (int k = 0; k < STATEKV_NUM_KERNELS; ++k) {
    if (total_ms) total_ms[k] = ms[k];
    if (launches) launches[k] = cnt[k];
  }
  return status;
}

int statekv_free_layer(statekv_layer* L) {
  if (!L) return STATEKV_ERR_INVALID_ARGUMENT;
  destroy_profile_events(L);
  delete L;
  return STATEKV_OK;
}

const char* statekv_status_string(int status) {
  switch (status) {
    case STATEKV_OK: return "ok";
    case STATEKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case STATEKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case STATEKV_ERR_WORKSPACE: return "workspace too small or misaligned";
    case STATEKV_ERR_CAPACITY: return "detailed cache capacity exceeded";
    case STATEKV_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int statekv_select_topb(const float* d_scores, int32_t n, int32_t budget, int32_t* d_out_idx,
                        void* stream) {
  if (!d_scores || !d_out_idx) return STATEKV_ERR_INVALID_ARGUMENT;
  if (n < 1 || budget < 1) return STATEKV_ERR_INVALID_ARGUMENT;
  if (n > skv::kMaxPool) return STATEKV_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return hip_status(skv::launch_select(d_scores, 1, n, 1, n, budget, nullptr, 0, d_out_idx,
                                       budget, nullptr, 1, 0, nullptr, false, false, false,
                                       skv::InPlace{}, nullptr, st));
}

}  // extern "C"
