// Host-side layer plan (see plan.h).
#include "plan.h"

#include <math.h>

namespace skv {

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace

int make_plan(const statekv_layer_config* cfg, Plan* p) {
  if (!cfg || !p) return STATEKV_ERR_INVALID_ARGUMENT;
  const int32_t Hq = cfg->n_q_heads, Hkv = cfg->n_kv_heads, D = cfg->head_dim;
  const int32_t T = cfg->frame_tokens, B = cfg->state_budget;
  if (Hq <= 0 || Hkv <= 0 || T <= 0 || B <= 0) return STATEKV_ERR_INVALID_ARGUMENT;
  if (Hq % Hkv) return STATEKV_ERR_INVALID_ARGUMENT;
  if (cfg->detailed_capacity < T) return STATEKV_ERR_INVALID_ARGUMENT;
  if (cfg->position_offset < 0) return STATEKV_ERR_INVALID_ARGUMENT;
  if (cfg->num_splits < 0) return STATEKV_ERR_INVALID_ARGUMENT;
  if (cfg->flags & ~(uint32_t)(STATEKV_FLAG_SELECT_SHARED | STATEKV_FLAG_D_RING |
                               STATEKV_FLAG_NONCAUSAL_FRAME | STATEKV_FLAG_C_IN_D |
                               STATEKV_FLAG_SELECT_RECENT | STATEKV_FLAG_SLOT_STABLE |
                               STATEKV_FLAG_OUT_BF16))
    return STATEKV_ERR_INVALID_ARGUMENT;
  if ((cfg->flags & STATEKV_FLAG_C_IN_D) && (cfg->flags & STATEKV_FLAG_D_RING))
    return STATEKV_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return STATEKV_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return STATEKV_ERR_UNSUPPORTED;
  if (T > 4096) return STATEKV_ERR_UNSUPPORTED;
  if ((int64_t)B + T > kMaxPool) return STATEKV_ERR_UNSUPPORTED;
  if (cfg->detailed_capacity > ((int64_t)1 << 40)) return STATEKV_ERR_UNSUPPORTED;
  if (!(cfg->softmax_scale == cfg->softmax_scale) || isinf(cfg->softmax_scale))
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(cfg->rope_theta >= 0.f) || isinf(cfg->rope_theta) || cfg->rope_theta == 1.f)
    return STATEKV_ERR_INVALID_ARGUMENT;
  if (!(cfg->rope_scaling == cfg->rope_scaling) || isinf(cfg->rope_scaling))
    return STATEKV_ERR_INVALID_ARGUMENT;

  Plan q = {};
  q.Hq = Hq;
  q.Hkv = Hkv;
  q.G = Hq / Hkv;
  q.D = D;
  q.T = T;
  q.B = B;
  q.cap = cfg->detailed_capacity;
  q.offset = cfg->position_offset;
  q.scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : (float)(1.0 / sqrt((double)D));
  q.flags = cfg->flags;
  q.rope_theta = cfg->rope_theta;
  q.rope_scaling = cfg->rope_scaling > 0.f ? cfg->rope_scaling : 1.0;
  q.ntblk = ceil_div(T, kTokBlk);
  q.nqblk = q.G * q.ntblk;
  q.rt = ceil_div(q.nqblk, kRowBlk);
  q.tpad = q.ntblk * kTokBlk;
  q.max_pool = B + T;
  q.max_tiles = ceil_div(q.max_pool, kKeyTile);
  const int per_split = Hkv * q.rt;
  int s = cfg->num_splits;
  if (s == 0) {
    // one workgroup per CU, but at least kMinTilesPerSplit key tiles per
    // split: each split costs a fixed prologue and epilogue and one O partial
    // of T*Hq*d floats, which small pools cannot amortise
    s = per_split >= kTargetWGs ? 1 : kTargetWGs / per_split;
    const int by_tiles = q.max_tiles / kMinTilesPerSplit;
    if (s > by_tiles) s = by_tiles;
  }
  if (s > q.max_tiles) s = q.max_tiles;
  if (s < 1) s = 1;
  q.splits = s;
  // the statistics pass writes only two floats per row and split: with the
  // automatic choice it takes twice the splits (two workgroups per CU)
  int ss = cfg->num_splits ? s : 2 * s;
  if (ss > q.max_tiles) ss = q.max_tiles;
  q.stat_splits = ss;
  q.ldsig = ceil_div(q.max_pool, kKeyTile) * kKeyTile;
  // full-attention baseline: the pool grows to the whole detailed cache
  int64_t full_tiles = (q.cap + kKeyTile - 1) / kKeyTile;
  int fs = cfg->num_splits ? cfg->num_splits
                           : (per_split >= 2 * kTargetWGs ? 1 : 2 * kTargetWGs / per_split);
  if (fs > kMaxFullSplits) fs = kMaxFullSplits;
  if (fs > full_tiles) fs = (int)full_tiles;
  if (fs < 1) fs = 1;
  q.full_splits = fs;
  q.part_splits = q.splits > q.full_splits ? q.splits : q.full_splits;
  if (q.stat_splits > q.part_splits) q.part_splits = q.stat_splits;

  const size_t A = 256;
  size_t off = 0;
  const size_t c_rows = (size_t)Hkv * B;
  const size_t d_rows = (size_t)Hkv * (size_t)q.cap;
  const size_t c_kv = (cfg->flags & STATEKV_FLAG_C_IN_D) ? 0 : c_rows * D * 2;
  // two state buffers (ping-pong), one when the state is updated in place
  const bool in_place = cfg->flags & STATEKV_FLAG_SLOT_STABLE;
  for (int i = 0; i < 2; ++i) {
    const size_t rows = (i == 1 && in_place) ? 0 : c_rows;
    q.off_ck[i] = off; off = align_up(off + (rows ? c_kv : 0), A);
    q.off_cv[i] = off; off = align_up(off + (rows ? c_kv : 0), A);
    q.off_cpos[i] = off; off = align_up(off + rows * 8, A);
  }
  q.off_dk = off; off = align_up(off + d_rows * D * 2, A);
  q.off_dv = off; off = align_up(off + d_rows * D * 2, A);
  const size_t stat = (size_t)q.part_splits * Hq * q.tpad * 4;
  const size_t opart = (size_t)(q.splits > q.full_splits ? q.splits : q.full_splits);
  q.off_m = off; off = align_up(off + stat, A);
  q.off_l = off; off = align_up(off + stat, A);
  q.off_o = off; off = align_up(off + opart * T * Hq * D * 4, A);
  q.off_sig = off; off = align_up(off + (size_t)Hkv * q.rt * q.ldsig * 4, A);
  q.off_scores = off; off = align_up(off + (size_t)Hkv * q.ldsig * 4, A);
  // selection rows: kept pool indices, or with the in-place update the move
  // lists (freed rows [0, T), frame tokens [T, 2T), move count at 2T)
  q.ldsel = in_place ? (B > 2 * T + 1 ? B : 2 * T + 1) : B;
  q.off_sel = off; off = align_up(off + (size_t)Hkv * q.ldsel * 4, A);
  const bool rope = q.rope_theta > 0.0;
  q.off_qrot = off; off = align_up(off + (rope ? (size_t)T * Hq * D * 2 : 0), A);
  q.off_krot = off; off = align_up(off + (rope ? (size_t)T * Hkv * D * 2 : 0), A);
  q.total = off;
  *p = q;
  return STATEKV_OK;
}

int splits_for_pool(const Plan& p, int pool) {
  int tiles = ceil_div(pool, kKeyTile);
  return p.splits < tiles ? p.splits : tiles;
}

int stat_splits_for_pool(const Plan& p, int pool) {
  int tiles = ceil_div(pool, kKeyTile);
  return p.stat_splits < tiles ? p.stat_splits : tiles;
}

}  // namespace skv
