// C ABI of the frame front end (declared in statekv.h): argument checks and
// the launch of the fused projection + rotary-embedding kernel.
#include <math.h>

#include "plan.h"
#include "skv_internal.h"

extern "C" {

int statekv_qkv_rope(const void* x, const void* w, int32_t n_tokens, int32_t hidden,
                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     int64_t first_position, double rope_theta, double rope_scaling, void* q,
                     void* k, void* v, void* stream) {
  if (!x || !w || !q || !k || !v) return STATEKV_ERR_INVALID_ARGUMENT;
  for (const void* p : {x, w, static_cast<const void*>(q), static_cast<const void*>(k),
                        static_cast<const void*>(v)})
    if (reinterpret_cast<uintptr_t>(p) & 15u) return STATEKV_ERR_INVALID_ARGUMENT;
  if (n_tokens < 1 || hidden < 1 || n_q_heads < 1 || n_kv_heads < 1 || first_position < 0)
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (n_q_heads % n_kv_heads) return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(rope_theta >= 0.0) || isinf(rope_theta) || rope_theta == 1.0)
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(rope_scaling == rope_scaling) || isinf(rope_scaling)) return STATEKV_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return STATEKV_ERR_UNSUPPORTED;
  if (hidden % 64) return STATEKV_ERR_UNSUPPORTED;
  if (n_tokens > (1 << 20) || hidden > (1 << 20) || n_q_heads + 2 * n_kv_heads > 4096)
    return STATEKV_ERR_UNSUPPORTED;
  if (first_position > ((int64_t)1 << 52) - n_tokens) return STATEKV_ERR_UNSUPPORTED;
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
  const hipError_t e =
      skv::launch_qkv_rope(a, head_dim, skv::Stream(static_cast<hipStream_t>(stream)));
  return e == hipSuccess ? STATEKV_OK : STATEKV_ERR_HIP;
}

}  // extern "C"
