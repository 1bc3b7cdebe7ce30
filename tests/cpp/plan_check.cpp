// Host-only checks of the layer plan (built with g++ and sanitizers, no HIP):
// regions are 256-byte aligned, disjoint and inside the total; sizes follow
// the configuration; invalid configurations are rejected.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "plan.h"

static int failures = 0;
#define CHECK(x)                                                  \
  do {                                                            \
    if (!(x)) {                                                   \
      fprintf(stderr, "%s:%d: CHECK failed: %s\n", __FILE__, __LINE__, #x); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static statekv_layer_config cfg(int hq, int hkv, int d, int t, int b, long long cap) {
  statekv_layer_config c = {};
  c.n_q_heads = hq;
  c.n_kv_heads = hkv;
  c.head_dim = d;
  c.frame_tokens = t;
  c.state_budget = b;
  c.detailed_capacity = cap;
  return c;
}

static void check_layout(const statekv_layer_config& c) {
  skv::Plan p;
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK);
  const size_t cr = (size_t)p.Hkv * p.B, dr = (size_t)p.Hkv * p.cap;
  std::vector<std::pair<size_t, size_t>> r = {
      {p.off_ck[0], cr * p.D * 2}, {p.off_cv[0], cr * p.D * 2}, {p.off_cpos[0], cr * 8},
      {p.off_ck[1], cr * p.D * 2}, {p.off_cv[1], cr * p.D * 2}, {p.off_cpos[1], cr * 8},
      {p.off_dk, dr * p.D * 2},     {p.off_dv, dr * p.D * 2},
      {p.off_m, (size_t)p.part_splits * p.Hq * p.tpad * 4},
      {p.off_l, (size_t)p.part_splits * p.Hq * p.tpad * 4},
      {p.off_o, (size_t)std::max(p.splits, p.full_splits) * p.T * p.Hq * p.D * 4},
      {p.off_sig, (size_t)p.Hkv * p.rt * p.ldsig * 4},
      {p.off_scores, (size_t)p.Hkv * p.ldsig * 4},
      {p.off_sel, (size_t)p.Hkv * p.B * 4},
      {p.off_qrot, p.rope_theta > 0 ? (size_t)p.T * p.Hq * p.D * 2 : 0},
      {p.off_krot, p.rope_theta > 0 ? (size_t)p.T * p.Hkv * p.D * 2 : 0}};
  std::sort(r.begin(), r.end());
  for (size_t i = 0; i < r.size(); ++i) {
    CHECK(r[i].first % 256 == 0);
    CHECK(r[i].first + r[i].second <= p.total);
    if (i + 1 < r.size()) CHECK(r[i].first + r[i].second <= r[i + 1].first);
  }
  CHECK(p.G * p.Hkv == p.Hq);
  CHECK(p.ntblk * skv::kTokBlk >= p.T && (p.ntblk - 1) * skv::kTokBlk < p.T);
  CHECK(p.rt * skv::kRowBlk >= p.nqblk);
  CHECK(p.ldsig >= p.B + p.T && p.ldsig % skv::kKeyTile == 0);
  CHECK(p.splits >= 1 && p.splits <= p.max_tiles);
  CHECK(p.Hkv * p.rt * p.splits <= skv::kTargetWGs || p.splits == 1);
  CHECK(p.stat_splits >= p.splits && p.stat_splits <= p.max_tiles);
  CHECK(p.part_splits >= p.stat_splits && p.part_splits >= p.full_splits);
  for (int pool = 1; pool <= p.B + p.T; pool += 97) {
    const int s = skv::splits_for_pool(p, pool);
    CHECK(s >= 1 && s <= (pool + skv::kKeyTile - 1) / skv::kKeyTile);
    const int s1 = skv::stat_splits_for_pool(p, pool);
    CHECK(s1 >= s && s1 <= (pool + skv::kKeyTile - 1) / skv::kKeyTile);
  }
}

int main() {
  check_layout(cfg(28, 4, 128, 256, 4096, 131072));
  check_layout(cfg(14, 2, 64, 256, 1024, 16384));
  check_layout(cfg(12, 2, 128, 256, 2048, 65536));
  check_layout(cfg(2, 1, 64, 16, 32, 128));
  check_layout(cfg(6, 2, 128, 17, 50, 102));
  check_layout(cfg(16, 1, 64, 4096, 28672, 4096));
  {
    statekv_layer_config r = cfg(28, 4, 128, 256, 4096, 131072);
    r.rope_theta = 1e6f;
    check_layout(r);
    skv::Plan p;
    CHECK(skv::make_plan(&r, &p) == STATEKV_OK && p.rope_theta == 1e6 && p.rope_scaling == 1.0);
    r.rope_scaling = 4.f;
    CHECK(skv::make_plan(&r, &p) == STATEKV_OK && p.rope_scaling == 4.0);
    r.rope_theta = 1.f;  // every frequency would be 1
    CHECK(skv::make_plan(&r, &p) == STATEKV_ERR_INVALID_ARGUMENT);
    r.rope_theta = -5.f;
    CHECK(skv::make_plan(&r, &p) == STATEKV_ERR_INVALID_ARGUMENT);
  }
  skv::Plan p;
  statekv_layer_config c = cfg(28, 4, 128, 256, 4096, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK && p.splits == 9 && p.stat_splits == 18 && p.rt == 7);
  // small pools: at least 2 key tiles per output split (2B-like: 36 tiles;
  // 1B-like at B = 1024: 20 tiles); the statistics pass takes twice as many,
  // at most one per key tile
  c = cfg(12, 2, 128, 256, 2048, 65536);
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK && p.splits == 18 && p.stat_splits == 36 && p.rt == 6);
  c = cfg(14, 2, 64, 256, 1024, 16384);
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK && p.splits == 10 && p.stat_splits == 20);
  c = cfg(28, 4, 96, 256, 4096, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_UNSUPPORTED);
  c = cfg(28, 5, 128, 256, 4096, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_INVALID_ARGUMENT);
  c = cfg(28, 4, 128, 256, 4096, 100);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_INVALID_ARGUMENT);
  c = cfg(28, 4, 128, 256, 32600, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_UNSUPPORTED);
  c = cfg(28, 4, 128, 256, 32512, 131072);  // B + T = 32768: the largest pool
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK && p.max_pool == 32768);
  c = cfg(28, 4, 128, 256, 32513, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_UNSUPPORTED);
  c = cfg(34, 2, 128, 256, 4096, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_UNSUPPORTED);
  c = cfg(28, 4, 128, 0, 4096, 131072);
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_INVALID_ARGUMENT);
  c = cfg(28, 4, 128, 256, 4096, 131072);
  c.flags = 1u << 7;
  CHECK(skv::make_plan(&c, &p) == STATEKV_ERR_INVALID_ARGUMENT);
  c.flags = STATEKV_FLAG_SELECT_SHARED;
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK);
  {
    // in-place update: one state buffer, selection rows wide enough for the
    // move lists (2T + 1 when that exceeds B)
    skv::Plan a, b;
    c.flags = 0;
    CHECK(skv::make_plan(&c, &a) == STATEKV_OK && a.ldsel == 4096);
    c.flags = STATEKV_FLAG_SLOT_STABLE;
    CHECK(skv::make_plan(&c, &b) == STATEKV_OK && b.ldsel == 4096);
    CHECK(a.total - b.total >= (size_t)4 * 4096 * (128 * 2 * 2 + 8));
    CHECK(b.off_ck[1] == b.off_cv[1] && b.off_cv[1] == b.off_cpos[1]);
    statekv_layer_config s = cfg(4, 2, 64, 300, 100, 3000);
    s.flags = STATEKV_FLAG_SLOT_STABLE;
    CHECK(skv::make_plan(&s, &b) == STATEKV_OK && b.ldsel == 601);
    CHECK(b.off_qrot - b.off_sel >= (size_t)2 * 601 * 4);
  }
  c.flags = 0;
  c.num_splits = 3;
  CHECK(skv::make_plan(&c, &p) == STATEKV_OK && p.splits == 3 && p.stat_splits == 3);
  CHECK(skv::make_plan(nullptr, &p) == STATEKV_ERR_INVALID_ARGUMENT);
  if (failures) return 1;
  printf("plan checks passed\n");
  return 0;
}
