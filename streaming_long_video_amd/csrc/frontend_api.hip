// C ABI of the frame front end (declared in statekv.h): argument checks, the
// workspace of the hidden-dimension splits, and the launches of the fused
// projection + rotary-embedding kernels.
#include <math.h>

#include "plan.h"
#include "skv_internal.h"

namespace {

// the size checks shared by both entry points
int check_sizes(int32_t n_tokens, int32_t hidden, int32_t n_q_heads, int32_t n_kv_heads,
                int32_t head_dim) {
  if (n_tokens < 1 || hidden < 1 || n_q_heads < 1 || n_kv_heads < 1)
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (n_q_heads % n_kv_heads) return STATEKV_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return STATEKV_ERR_UNSUPPORTED;
  if (hidden % 64) return STATEKV_ERR_UNSUPPORTED;
  if (n_tokens > (1 << 20) || hidden > (1 << 20) || n_q_heads + 2 * n_kv_heads > 4096)
    return STATEKV_ERR_UNSUPPORTED;
  return STATEKV_OK;
}

}  // namespace

extern "C" {

int statekv_qkv_rope_workspace_size(int32_t n_tokens, int32_t hidden, int32_t n_q_heads,
                                    int32_t n_kv_heads, int32_t head_dim, uint64_t* bytes) {
  if (!bytes) return STATEKV_ERR_INVALID_ARGUMENT;
  const int rc = check_sizes(n_tokens, hidden, n_q_heads, n_kv_heads, head_dim);
  if (rc != STATEKV_OK) return rc;
  *bytes = skv::qkv_rope_workspace_bytes(n_tokens, hidden, n_q_heads + 2 * n_kv_heads, head_dim);
  return STATEKV_OK;
}

int statekv_qkv_rope(const void* x, const void* w, int32_t n_tokens, int32_t hidden,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int64_t first_position, double rope_theta, double rope_scaling, void* q,
                     void* k, void* v, void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!x || !w || !q || !k || !v) return STATEKV_ERR_INVALID_ARGUMENT;
  for (const void* p : {x, w, static_cast<const void*>(q), static_cast<const void*>(k),
                        static_cast<const void*>(v)})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return STATEKV_ERR_INVALID_ARGUMENT;
  const int rc = check_sizes(n_tokens, hidden, n_q_heads, n_kv_heads, head_dim);
  if (rc != STATEKV_OK) return rc;
  if (first_position < 0) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(rope_theta >= 0.0) || isinf(rope_theta) || rope_theta == 1.0)
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(rope_scaling == rope_scaling) || isinf(rope_scaling)) return STATEKV_ERR_INVALID_ARGUMENT;
  if (first_position > ((int64_t)1 << 52) - n_tokens) return STATEKV_ERR_UNSUPPORTED;
  const int heads = n_q_heads + 2 * n_kv_heads;
  const size_t need = skv::qkv_rope_workspace_bytes(n_tokens, hidden, heads, head_dim);
  if (workspace && need > 0 &&
      ((reinterpret_cast<uintptr_t>(workspace) & 255u) || workspace_bytes < need))
    return STATEKV_ERR_WORKSPACE;

  skv::FrontArgs a = {};
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.q = static_cast<uint16_t*>(q);
  a.k = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.T = n_tokens;
  a.hidden = hidden;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.first_position = first_position;
  a.theta = rope_theta;
  a.scaling = rope_scaling > 0.0 ? rope_scaling : 1.0;
  if (rope_theta > 0.0)
    for (int i = 0; i < head_dim / 2; ++i) a.inv_freq[i] = pow(rope_theta, -2.0 * i / head_dim);
  a.S = skv::qkv_rope_splits(n_tokens, hidden, heads, head_dim);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  bool owned = false;
  if (need > 0) {
    if (workspace) {
      a.part = static_cast<float*>(workspace);
    } else {
      void* p = nullptr;
      if (hipMallocAsync(&p, need, st) != hipSuccess) return STATEKV_ERR_HIP;
      a.part = static_cast<float*>(p);
      owned = true;
    }
  }
  if (need > 0) {
    const int ntiles = (heads * (head_dim / 2) + 63) / 64;
    a.rot = reinterpret_cast<double*>(a.part + (size_t)a.S * ntiles * n_tokens * 128);
  }
  hipError_t e = skv::launch_qkv_rope(a, head_dim, skv::Stream(st));
  if (owned) {
    const hipError_t f = hipFreeAsync(a.part, st);
    if (e == hipSuccess) e = f;
  }
  return e == hipSuccess ? STATEKV_OK : STATEKV_ERR_HIP;
}

}  // extern "C"
