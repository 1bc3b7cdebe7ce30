// Host-side layer plan: configuration checks, derived sizes and the carve-up
// of the caller's device workspace.  Plain C++ (no HIP), so it is also built
// and tested with the host compiler alone.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "statekv.h"

namespace skv {

// Kernel tiling shared by the host plan and the kernels.
constexpr int kTokBlk = 32;     // query tokens per MFMA block (MFMA n dimension)
constexpr int kRowBlk = 8;      // query blocks per attention row tile (256 rows)
constexpr int kKeyTile = 64;    // keys staged in LDS per step
constexpr int kTargetWGs = 256; // one workgroup per compute unit on MI355X
constexpr int kMinTilesPerSplit = 2;  // key tiles per output-pass split (automatic plan)
constexpr int kMaxPool = 32768; // B + T limit (select keeps the pool in LDS)
constexpr int kMaxFullSplits = 64;

struct Plan {
  // configuration
  int32_t Hq, Hkv, G, D, T, B;
  int64_t cap, offset;
  float scale;        // softmax scale applied to the logits
  double rope_theta;  // > 0: the library rotates q and k (else they arrive rotated)
  double rope_scaling;
  uint32_t flags;
  // attention grid
  int32_t ntblk;      // ceil(T / kTokBlk): token blocks per query head
  int32_t nqblk;      // G * ntblk: query blocks per KV head
  int32_t rt;         // row tiles per KV head = ceil(nqblk / kRowBlk)
  int32_t tpad;       // ntblk * kTokBlk
  int32_t max_pool;   // B + T
  int32_t max_tiles;  // ceil(max_pool / kKeyTile)
  int32_t splits;     // key splits of the StateKV output pass
  int32_t stat_splits;  // key splits of the StateKV statistics pass
  int32_t ldsig;      // row stride (floats) of score partials / scores
  int32_t full_splits;  // key splits of the full-attention baseline
  int32_t part_splits;  // largest of the split counts: partial buffers sized for it
  int32_t ldsel;      // row stride (int32) of the selection region
  // workspace offsets (bytes, 256-aligned)
  size_t off_ck[2], off_cv[2], off_cpos[2];
  size_t off_dk, off_dv;
  size_t off_m, off_l, off_o;
  size_t off_sig, off_scores, off_sel;
  size_t off_qrot, off_krot;  // rotated frame q / k (only with rope_theta > 0)
  size_t total;
};

// Fills *plan from *cfg.  Returns STATEKV_OK or an error status.
int make_plan(const statekv_layer_config* cfg, Plan* plan);

// Splits actually used for a pool of `pool` candidates (never more than tiles):
// output pass, and statistics pass.
int splits_for_pool(const Plan& p, int pool);
int stat_splits_for_pool(const Plan& p, int pool);

}  // namespace skv
