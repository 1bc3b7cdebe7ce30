// Fused GQA attention over the StateKV candidate pool [C_{n-1} ; frame n] for
// gfx950.  One kernel template, three passes sharing one tiling:
//
//   pass 1 (statistics): per query row, the log-sum-exp of the logits over
//     this workgroup's key split (a running max and sum per 32-key block,
//     stored as one float);
//   pass 2 (output + scores): combines the split statistics into the row
//     log-sum-exp, recomputes the logits, forms the normalised probabilities
//     P, accumulates O = P V and the column sums of P (the candidates'
//     importance, summed over the queries of every query head that shares the
//     KV head);
//   pass 3 (quadratic baseline): plain online-softmax attention of the frame
//     over the whole detailed cache, no scores.
//
// What passes 1-2 implement is the attention and importance part of the
// StateKV step (paper.rainbus.top, method-steps section: softmax over the
// concatenated compressed memory and frame keys; a candidate's importance is
// the sum over queries of its attention weight; paperlayer.ai App. A.3: cache
// building needs the attention weights or sufficient statistics, which fused
// attention kernels normally do not expose -- the row statistics of pass 1
// are exactly those statistics).
//
// Work layout: the G query heads that share KV head h and the T frame tokens
// form G*T query rows, cut into 32-token blocks of one head.  A workgroup (8
// waves, two per SIMD) owns 8 such blocks (a 256-row tile, one per wave) and
// one contiguous split of the pool's 64-key tiles.  Key tiles are staged through
// LDS double-buffered: the next tile's global loads are in flight in
// registers while the current tile is computed, then written to the other
// buffer (one barrier per tile).  Logits are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (keys on M, queries on N): each
// lane holds one query and 16 keys, so row statistics need no cross-lane
// work, the probabilities feed O^T = V^T P^T (v_mfma_f32_32x32x16_f16)
// straight from registers (A and B use the same permutation of the 16 key
// slots), and the column sums are a reduce-scatter across the 32 lanes of each
// half-wave (v_permlane16_swap, then bank-masked DPP).  P enters PV as fp16
// scaled by 2^12 (11 significant bits, clear of fp16 subnormals); V is
// converted bf16 -> fp16 (exact for |v| in [2^-17, 65504]) while it is
// transposed into LDS.  Key blocks entirely inside the visible region take a
// branch-free path; only blocks that reach the frame's causal triangle or the
// pool's end are masked.  Scores and O partials are written per split / row
// tile and reduced in a fixed order elsewhere: no atomics, bitwise
// reproducible results.
#include "../skv_internal.h"

namespace skv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;        // two waves per SIMD
constexpr int kQBlkPerWave = 1;  // 32-token query blocks per wave
constexpr int kThreads = kWaves * 64;

// Keeps the compiler's scheduler from moving instructions across phase
// boundaries of the block step (operand reads / softmax / MFMA issue).
#define SKV_FENCE() __builtin_amdgcn_sched_barrier(0)
constexpr int kKPad = 8;  // bf16 padding per K row in LDS (conflict-free b128 reads)
constexpr int kVPad = 8;  // fp16 padding per V^T row (conflict-free b128 reads)
constexpr int kScoreTiles = 64;  // key tiles of scores buffered in LDS per flush
// s_waitcnt operand for vmcnt(0) with the other counters left alone
// (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

// Position of key k of a tile within a V^T row in LDS: in every 16-key slab
// the key groups 4-7 and 8-11 trade places, so that the 8 keys one lane feeds
// to the PV MFMA (slots 8(r/4) + 4 half + r%4, r < 8) are contiguous.
__host__ __device__ constexpr int vt_pos(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}
constexpr float kPUnscale = kOPartUnscale;  // P is formed as 2^12 * P

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so that each
// XCD gets a contiguous range of logical ids (consecutive ids then share
// operands in that XCD's L2).
__device__ inline int xcd_logical_id(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// The same ranges with the dispatch order inside each XCD changed so that
// the logical ids of the last key split (lid % S == S - 1, the split holding
// the frame's masked tiles, the slowest) come first, then the others in
// order: workgroups start over about 2 us in dispatch order.
__device__ inline int xcd_logical_id_last_split_first(int b, int n, int S) {
  const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
  const int L0 = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  const int len = x < r ? q + 1 : q;
  const int o = (S - 1 - L0 % S) % S;  // first last-split id: L0 + o
  const int nf = len > o ? (len - o - 1) / S + 1 : 0;
  if (i < nf) return L0 + o + i * S;
  const int j = i - nf;  // the j-th of the other ids (S > 1 here)
  return L0 + (j < o ? j : j + 1 + (j - o) / (S - 1));
}
__device__ inline float as_f(int x) { return __builtin_bit_cast(float, x); }
__device__ inline int as_i(float x) { return __builtin_bit_cast(int, x); }

// DPP move of `src` into the lanes of `BANKS`; other lanes keep `old`.
template <int CTRL, int BANKS>
__device__ inline float dpp_into(float old, float src) {
  return as_f(__builtin_amdgcn_update_dpp(as_i(old), as_i(src), CTRL, 0xF, BANKS, false));
}
template <int CTRL>
__device__ inline float dpp_all(float src) {
  return as_f(__builtin_amdgcn_update_dpp(0, as_i(src), CTRL, 0xF, 0xF, true));
}

// Sum of v[r] over the 32 lanes of each half-wave (the 32 queries of a block),
// reduce-scatter style.  Lane l ends with the total of register r = (l>>1)&15
// (both lanes of a pair hold it).  Each stage halves the registers a lane
// keeps: the lane picks its own half and the partner's copy of it arrives by
// one DPP read folded into the add.
//   xor 16: v_permlane16_swap pairs (v[k], v[k+8]) across 16-lane rows;
//   bit 3:  row_ror:8 (lane i <-> i^8 in a row), keep w[k + 4 b3];
//   bit 2:  row_half_mirror (lane i <-> 7-i in 8 lanes), keep x[k + 2 b2];
//   bit 1, bit 0: quad_perm xor 2, xor 1.
__device__ inline float colsum_reduce(const float (&v)[16], int l32) {
  const bool b3 = l32 & 8, b2 = l32 & 4, b1 = l32 & 2;
  float w[8], x[4], y[2];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto s = __builtin_amdgcn_permlane16_swap(as_i(v[k]), as_i(v[k + 8]), false, false);
    w[k] = as_f(s[0]) + as_f(s[1]);  // r = 8*b4 + k
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b3 ? w[k + 4] : w[k], give = b3 ? w[k] : w[k + 4];
    x[k] = keep + dpp_all<0x128>(give);  // r = 8*b4 + 4*b3 + k
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b2 ? x[k + 2] : x[k], give = b2 ? x[k] : x[k + 2];
    y[k] = keep + dpp_all<0x141>(give);  // r = 8*b4 + 4*b3 + 2*b2 + k
  }
  const float keep = b1 ? y[1] : y[0], give = b1 ? y[0] : y[1];
  const float z = keep + dpp_all<0x4E>(give);
  return z + dpp_all<0xB1>(z);
}

__device__ inline float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__device__ inline uint32_t pack_f16(float a, float b) {
  const f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Row of the state buffer that holds state token j of KV head h: j itself, or
// (with the state kept as positions into D) the D row of its position.
template <bool CIND>
__device__ inline int64_t state_row(const AttnArgs& a, int h, int j) {
  if constexpr (CIND) return a.cpos[(int64_t)h * a.ldcp + j] - a.cpos_base;
  return (int64_t)j;
}

// One 16-byte chunk (8 bf16) of pool row j, columns [col, col+8).  Rows past
// the pool read the last pool row instead: every such key is masked (its
// weight is exactly 0), and a finite stand-in keeps 0 * value at 0.  One load
// from a selected address, so the staged registers have a single source.
template <int D, bool CIND>
__device__ inline u32x4 pool_chunk(const AttnArgs& a, const uint16_t* state,
                                   const uint16_t* frame, int h, int pool, int j, int col) {
  const int jj = min(j, pool - 1);
  const uint16_t* p =
      jj < a.c ? state + ((int64_t)h * a.ldc + state_row<CIND>(a, h, jj)) * D + col
               : frame + ((int64_t)(jj - a.c) * a.Hkv + h) * D + col;
  return *reinterpret_cast<const u32x4*>(p);
}

// Registers staging one key tile between its global loads and its LDS stores.
template <int D, bool WITH_V>
struct TileStage {
  static constexpr int KCH = kKeyTile * (D / 8) / kThreads;  // 16-B K chunks / thread
  // (key pair, 8-column chunk) items of the V tile; at d = 64 there are fewer
  // items than threads and the upper threads stage no V
  static constexpr int VITEMS = (kKeyTile / 2) * (D / 8);
  static constexpr int VIT = (VITEMS + kThreads - 1) / kThreads;  // items / thread
  static constexpr bool VPART = VITEMS % kThreads != 0;
  static_assert(KCH * kThreads == kKeyTile * (D / 8), "K tile must split evenly");
  u32x4 k[KCH];
  u32x4 v0[WITH_V ? VIT : 1], v1[WITH_V ? VIT : 1];

  template <bool CIND>
  __device__ inline void load(const AttnArgs& a, int h, int pool, int key0, int tid) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * kThreads;
      k[i] = pool_chunk<D, CIND>(a, a.kc, a.kf, h, pool, key0 + ch / (D / 8), (ch % (D / 8)) * 8);
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < VIT; ++i) {
        const int it = tid + i * kThreads;
        if (VPART && it >= VITEMS) continue;
        const int kp = it % (kKeyTile / 2), dc = (it / (kKeyTile / 2)) * 8;
        v0[i] = pool_chunk<D, CIND>(a, a.vc, a.vf, h, pool, key0 + 2 * kp, dc);
        v1[i] = pool_chunk<D, CIND>(a, a.vc, a.vf, h, pool, key0 + 2 * kp + 1, dc);
      }
    }
  }

  // Tile wholly inside the state: no per-chunk source choice, no bounds.
  __device__ inline void load_state(const AttnArgs& a, int h, int key0, int tid) {
    const uint16_t* kb = a.kc + ((int64_t)h * a.ldc + key0) * D;
    const uint16_t* vb = a.vc + ((int64_t)h * a.ldc + key0) * D;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * kThreads;
      k[i] = *reinterpret_cast<const u32x4*>(kb + ch * 8);
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < VIT; ++i) {
        const int it = tid + i * kThreads;
        if (VPART && it >= VITEMS) continue;
        const int kp = it % (kKeyTile / 2), dc = (it / (kKeyTile / 2)) * 8;
        v0[i] = *reinterpret_cast<const u32x4*>(vb + (2 * kp) * D + dc);
        v1[i] = *reinterpret_cast<const u32x4*>(vb + (2 * kp + 1) * D + dc);
      }
    }
  }

  // State tile kept as positions into D: the rows come from the D rows in
  // `rows` (looked up one tile ahead, see StateRows).
  template <class Rows>
  __device__ inline void load_state_rows(const AttnArgs& a, int h, const Rows& rows, int tid) {
    const uint16_t* kb = a.kc + (int64_t)h * a.ldc * D;
    const uint16_t* vb = a.vc + (int64_t)h * a.ldc * D;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * kThreads;
      k[i] = *reinterpret_cast<const u32x4*>(kb + (int64_t)rows.k[i] * D + (ch % (D / 8)) * 8);
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < VIT; ++i) {
        const int it = tid + i * kThreads;
        if (VPART && it >= VITEMS) continue;
        const int dc = (it / (kKeyTile / 2)) * 8;
        v0[i] = *reinterpret_cast<const u32x4*>(vb + (int64_t)rows.v0[i] * D + dc);
        v1[i] = *reinterpret_cast<const u32x4*>(vb + (int64_t)rows.v1[i] * D + dc);
      }
    }
  }

  // K rows as they are; V transposed to [d][key] and converted to fp16.
  __device__ inline void store(uint16_t* Ks, _Float16* Vt, int tid) const {
    constexpr int KLD = D + kKPad, VLD = kKeyTile + kVPad;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = tid + i * kThreads;
      *reinterpret_cast<u32x4*>(&Ks[(ch / (D / 8)) * KLD + (ch % (D / 8)) * 8]) = k[i];
    }
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < VIT; ++i) {
        const int it = tid + i * kThreads;
        if (VPART && it >= VITEMS) continue;
        const int kp = it % (kKeyTile / 2), dc = (it / (kKeyTile / 2)) * 8;
        uint32_t* col = reinterpret_cast<uint32_t*>(&Vt[dc * VLD + vt_pos(2 * kp)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          col[(2 * e) * (VLD / 2)] = pack_f16(bf16lo(v0[i][e]), bf16lo(v1[i][e]));
          col[(2 * e + 1) * (VLD / 2)] = pack_f16(bf16hi(v0[i][e]), bf16hi(v1[i][e]));
        }
      }
    }
  }
};

// D rows of the state tokens one thread stages for a state tile (same
// row assignment as TileStage), when the state is kept as positions into D.
template <int D, bool WITH_V>
struct StateRows {
  using TS = TileStage<D, WITH_V>;
  int32_t k[TS::KCH];
  int32_t v0[WITH_V ? TS::VIT : 1], v1[WITH_V ? TS::VIT : 1];

  __device__ inline void load(const AttnArgs& a, int h, int key0, int tid) {
#pragma unroll
    for (int i = 0; i < TS::KCH; ++i)
      k[i] = (int32_t)state_row<true>(a, h, key0 + (tid + i * kThreads) / (D / 8));
    if constexpr (WITH_V) {
#pragma unroll
      for (int i = 0; i < TS::VIT; ++i) {
        const int it = tid + i * kThreads;
        if (TS::VPART && it >= TS::VITEMS) continue;
        const int kp = it % (kKeyTile / 2);
        v0[i] = (int32_t)state_row<true>(a, h, key0 + 2 * kp);
        v1[i] = (int32_t)state_row<true>(a, h, key0 + 2 * kp + 1);
      }
    }
  }
};

// Second launch bound = minimum waves per SIMD: the statistics pass runs two
// workgroups per CU (four waves per SIMD, at most 128 registers), the other
// passes one (two waves per SIMD).
// CIND: the state is kept as positions into D (a.cpos set).
template <int D, int PASS, bool CIND>
__global__ __launch_bounds__(kThreads, PASS == 1 ? 4 : 2) void attn_kernel(AttnArgs a) {
  constexpr int QB = kQBlkPerWave;
  constexpr int KT = kKeyTile;
  constexpr int NKK = D / 16;  // k-steps of the QK^T MFMA
  constexpr int NMB = D / 32;  // 32-row blocks of O^T
  constexpr int KLD = D + kKPad;
  constexpr int VLD = KT + kVPad;
  static_assert(VLD % 8 == 0, "16-byte aligned V^T rows");
  constexpr bool WITH_V = PASS >= 2;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[WITH_V ? 2 : 1][WITH_V ? D * VLD : 8];
  __shared__ float sigw[PASS == 2 ? 2 : 1][PASS == 2 ? kWaves * KT : 1];
  // the row tile's finished scores of up to kScoreTiles key tiles, stored to
  // global memory in bursts (a store inside the tile loop would make the next
  // tile's loads wait for it)
  __shared__ float sbuf[PASS == 2 ? kScoreTiles * KT : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int lid = PASS == 2 ? xcd_logical_id_last_split_first(blockIdx.x, gridDim.x, a.S)
                            : xcd_logical_id(blockIdx.x, gridDim.x);
  // The statistics pass gives consecutive logical ids the row tiles of one
  // key split (they share K tiles in L2).  The output pass gives them the key
  // splits of one row tile instead: its prologue reads the row tile's queries
  // and every split's statistics, a burst that then stays within one XCD
  // (1.3 us faster at the 8B shape; the same order makes the statistics pass
  // slower).  In both passes the last key split (the frame's masked tiles,
  // the slowest workgroups) is dispatched first: 0.8 % off the 2B-like
  // 28-layer stream, neutral at the 8B-like shape.
  int rtile, s, h;
  if (PASS == 2) {
    s = lid % a.S;
    const int hr = lid / a.S;
    rtile = hr % a.rt;
    h = hr / a.rt;
  } else {
    rtile = lid % a.rt;
    const int hs = lid / a.rt;
    s = a.S - 1 - hs % a.S;  // splits in reverse: each head's last split first
    h = hs / a.S;
  }
  const int c = a.c;
  const int pool = c + a.T;
  const int ntiles = (pool + KT - 1) / KT;
  const int tile_lo = (int)((int64_t)s * ntiles / a.S);
  const int tile_hi = (int)((int64_t)(s + 1) * ntiles / a.S);
  const float sl2 = a.scale_log2;

  // This wave's query blocks: block b = tb*G + gl holds tokens [32tb, 32tb+32)
  // of query head h*G + gl.  Lane l32 owns token 32tb + l32 of each block.
  const int b0 = rtile * kRowBlk;
  int qtok[QB], qhead[QB], qlim[QB];
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    const int b = b0 + w * QB + i;
    qtok[i] = -1;
    qhead[i] = h * a.G;
    if (b < a.nqblk) {
      const int tb = b / a.G;
      const int t = tb * kTokBlk + l32;
      qtok[i] = t < a.T ? t : -1;
      qhead[i] = h * a.G + b % a.G;
    }
    // frame key t' is visible to this lane's query iff t' <= qlim
    qlim[i] = qtok[i] < 0 ? -1 : (a.causal ? qtok[i] : a.T - 1);
  }
  const int blast = min(b0 + kRowBlk, a.nqblk) - 1;
  const int wg_tmax = min(a.T - 1, (blast / a.G) * kTokBlk + kTokBlk - 1);
  const int wg_klim = a.causal ? c + wg_tmax + 1 : pool;
  const int tile_end = max(tile_lo, min(tile_hi, (wg_klim + KT - 1) / KT));

  // the first key tile's global loads go out first, so that their latency
  // overlaps the Q and row-statistics loads below
  TileStage<D, WITH_V> stage;
  // With the state kept as positions into D, the D rows of the next state
  // tile are looked up one tile before its K/V loads go out.
  StateRows<D, WITH_V> rows;
  auto stage_load = [&](int key0) __attribute__((always_inline)) {
    if (key0 + KT <= c) {
      if constexpr (CIND) {
        stage.load_state_rows(a, h, rows, tid);
        if (key0 + 2 * KT <= c) rows.load(a, h, key0 + KT, tid);
      } else {
        stage.load_state(a, h, key0, tid);
      }
    } else {
      stage.template load<CIND>(a, h, pool, key0, tid);
    }
  };
  if (CIND && (tile_lo + 1) * KT <= c) rows.load(a, h, tile_lo * KT, tid);
  if (tile_end > tile_lo) stage_load(tile_lo * KT);

  bf16x8 qreg[QB][NKK];
#pragma unroll
  for (int i = 0; i < QB; ++i) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qtok[i] >= 0)
        v = *reinterpret_cast<const u32x4*>(
            a.q + ((int64_t)qtok[i] * a.Hq + qhead[i]) * D + kk * 16 + half * 8);
      qreg[i][kk] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float mrun[QB], lrun[QB], lse2[QB];
  f32x16 oacc[WITH_V ? QB : 1][WITH_V ? NMB : 1];
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
    lse2[i] = INFINITY;
  }
  if constexpr (WITH_V) {
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[i][mb] = f32x16{};
  }
  if constexpr (PASS == 2) {
    // Row log-sum-exp (base 2, scaled logits) of the row tile's 256 rows from
    // the statistics pass's per-split log-sum-exps (one float per row and
    // split: half the bytes of a (max, sum) pair, and this prologue's loads
    // are what it waits for).  Thread pair (r, r + 256) takes row r, each
    // half of the splits (even / odd index), every load of a group in flight
    // at once; the halves merge through LDS.  12 is subtracted so that P
    // comes out * 2^12.
    {
      static_assert(kThreads == 2 * kRowBlk * kTokBlk, "two threads per row");
      constexpr int kGrp = 16;
      __shared__ float mh[2][kRowBlk * kTokBlk], lh[2][kRowBlk * kTokBlk];
      // par is uniform over a wave: the split offsets below are scalar
      const int r = tid % (kRowBlk * kTokBlk);
      const int par = __builtin_amdgcn_readfirstlane(tid / (kRowBlk * kTokBlk));
      const int b = b0 + r / kTokBlk;
      const int t = (b / a.G) * kTokBlk + r % kTokBlk;
      float M = -INFINITY, L = 0.f;
      if (b < a.nqblk && t < a.T) {
        // 32-bit offsets (the partials hold Sst * Hq * tpad floats); loads
        // past the last split re-read it and are then replaced, so no load is
        // conditional; exp2 of -inf (an empty split) is 0
        const int stride = a.Hq * a.tpad, last = a.Sst - 1;
        const uint32_t rbytes = (uint32_t)((h * a.G + b % a.G) * a.tpad + t) * 4u;
        // M: the largest split log-sum-exp so far, L: sum of 2^(lse - M)
        for (int s0 = par; s0 < a.Sst; s0 += 2 * kGrp) {
          float mv[kGrp];
#pragma unroll
          for (int u = 0; u < kGrp; ++u) {
            const int sp = s0 + 2 * u;
            const int o = min(sp, last) * stride;
            // scalar base + 32-bit lane offset: one address register for all loads
            const float mr = *reinterpret_cast<const float*>(
                reinterpret_cast<const char*>(a.m_part + o) + rbytes);
            mv[u] = sp <= last ? mr : -INFINITY;
          }
          float Mg = M;
#pragma unroll
          for (int u = 0; u < kGrp; ++u) Mg = fmaxf(Mg, mv[u]);
          const float Ms = Mg == -INFINITY ? 0.f : Mg;
          L = L * __builtin_amdgcn_exp2f(M - Ms);
#pragma unroll
          for (int u = 0; u < kGrp; ++u) L += __builtin_amdgcn_exp2f(mv[u] - Ms);
          M = Mg;
        }
      }
      mh[par][r] = M;
      lh[par][r] = L;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < QB; ++i) {
        if (qtok[i] < 0) continue;
        const int rr = (w * QB + i) * kTokBlk + l32;
        const float m0 = mh[0][rr], m1 = mh[1][rr];
        const float Mx = fmaxf(m0, m1);
        float Lx = 0.f;
        if (m0 > -INFINITY) Lx += lh[0][rr] * exp2f(m0 - Mx);
        if (m1 > -INFINITY) Lx += lh[1][rr] * exp2f(m1 - Mx);
        lse2[i] = Mx + log2f(Lx) - 12.f;
      }
    }
  }

  // -- per-32-key-block work -----------------------------------------------
  // register r of query block i holds frame offset kbase - c + 8(r/4) + 4 half
  // + r%4 of its key, visible iff that offset does not exceed qlim[i]
  auto visible = [&](int kbase, int i, int r) __attribute__((always_inline)) {
    return 8 * (r >> 2) + (r & 3) <= qlim[i] - (kbase - c + 4 * half);
  };

  // K rows of block kb as the A operand of S^T = K Q^T: 8 consecutive d per
  // lane, one 16-wide d step per fragment
  auto read_k = [&](const uint16_t* K, int kb, bf16x8 (&kf)[NKK]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(&K[(kb * 32 + l32) * KLD + kk * 16 + half * 8]);
  };
  auto mfma_qk = [&](const bf16x8 (&kf)[NKK], f32x16 (&sacc)[QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < QB; ++i) sacc[i] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int i = 0; i < QB; ++i)
        sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qreg[i][kk], sacc[i], 0, 0, 0);
  };
  // V^T rows (d) of block kb as the A operand of O^T = V^T P^T, key slots in
  // the order of the logits' registers (8(r/4) + 4 half + r%4): one 16-byte
  // read, the rows being stored in vt_pos order
  auto read_v = [&](const _Float16* V, int kb, u32x4 (&vf)[NMB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int slab = 0; slab < 2; ++slab)
        vf[mb][slab] = *reinterpret_cast<const u32x4*>(
            &V[(mb * 32 + l32) * VLD + kb * 32 + slab * 16 + 8 * half]);
  };
  auto mfma_pv = [&](const u32x4 (&vf)[NMB][2], const u32x4 (&ph)[QB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int slab = 0; slab < 2; ++slab)
#pragma unroll
        for (int i = 0; i < QB; ++i)
          oacc[i][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              __builtin_bit_cast(f16x8, vf[mb][slab]), __builtin_bit_cast(f16x8, ph[i][slab]),
              oacc[i][mb], 0, 0, 0);
  };

  // pass 1: row sum of exp over this block relative to a reference maximum
  // mrun.  The reference only moves when a block's sum shows it was exceeded
  // by more than 2^32 (or before the row has seen a visible key): then the
  // block's maximum is taken exactly and the running sum rescaled.  Logits
  // below the reference only shrink their terms, so the (reference, sum)
  // pair describes the same log-sum-exp as the exact running maximum would.
  auto stats_block = [&](const f32x16 (&sacc)[QB], int kbase, bool masked) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      float z[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        z[r] = (!masked || visible(kbase, i, r)) ? sacc[i][r] : -INFINITY;
      auto block_sum = [&](float ms) __attribute__((always_inline)) {
        float e[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(z[r], sl2, -ms));
#pragma unroll
        for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
          for (int r = 0; r < st; ++r) e[r] += e[r + st];
        return e[0];
      };
      const float sum = block_sum(mrun[i] == -INFINITY ? 0.f : mrun[i] * sl2);
      if (mrun[i] == -INFINITY || !(sum <= 0x1p32f)) {
        float m8[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) m8[r] = fmaxf(z[2 * r], z[2 * r + 1]);
        const float mx = fmaxf(fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3])),
                               fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7])));
        const float mnew = fmaxf(mrun[i], mx);
        // nothing visible yet for this lane: every exp below is exp2(-inf) = 0
        const float ms = (mnew == -INFINITY ? 0.f : mnew) * sl2;
        lrun[i] = lrun[i] * __builtin_amdgcn_exp2f(fmaf(mrun[i], sl2, -ms)) + block_sum(ms);
        mrun[i] = mnew;
      } else {
        lrun[i] += sum;
      }
    }
  };

  // pass 2: normalised P (x 2^12) -> fp16 pairs, column sums -> LDS
  auto scores_block = [&](const f32x16 (&sacc)[QB], int kbase, bool masked, int kb,
                          float* sw, u32x4 (&ph)[QB][2]) __attribute__((always_inline)) {
    float p[QB][16];
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[i][r], sl2, -lse2[i]));
        p[i][r] = (!masked || visible(kbase, i, r)) ? e : 0.f;
      }
#pragma unroll
    for (int i = 0; i < QB; ++i)
#pragma unroll
      for (int slab = 0; slab < 2; ++slab)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          ph[i][slab][m] = pack_f16(p[i][slab * 8 + 2 * m], p[i][slab * 8 + 2 * m + 1]);
    // the column-sum swaps overwrite their operands: the packs are formed first
    // (an empty asm that reads them), so no copies of P are needed
#pragma unroll
    for (int i = 0; i < QB; ++i) asm volatile("" ::"v"(ph[i][0]), "v"(ph[i][1]));
    float cs[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      cs[r] = p[0][r];
#pragma unroll
      for (int i = 1; i < QB; ++i) cs[r] += p[i][r];
    }
    const float tot = colsum_reduce(cs, l32);
    if (!(l32 & 1)) {
      const int r = l32 >> 1;
      sw[w * KT + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = tot * kPUnscale;
    }
  };

  // pass 3: online softmax with rescaled O (quadratic baseline)
  auto online_block = [&](const f32x16 (&sacc)[QB], int kbase, bool masked,
                          u32x4 (&ph)[QB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      float z[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        z[r] = (!masked || visible(kbase, i, r)) ? sacc[i][r] : -INFINITY;
        mx = fmaxf(mx, z[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));  // both half-waves hold the same query
      const float mnew = fmaxf(mrun[i], mx);
      // nothing visible yet for this query: every exp below is exp2(-inf) = 0
      const float msafe = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f((mrun[i] - msafe) * sl2);
      const float ms = fmaf(msafe, sl2, -12.f);
      float e[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(z[r], sl2, -ms));
#pragma unroll
      for (int slab = 0; slab < 2; ++slab)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          ph[i][slab][m] = pack_f16(e[slab * 8 + 2 * m], e[slab * 8 + 2 * m + 1]);
#pragma unroll
      for (int st = 8; st >= 1; st >>= 1)
#pragma unroll
        for (int r = 0; r < st; ++r) e[r] += e[r + st];
      lrun[i] = lrun[i] * alpha + e[0];
      mrun[i] = mnew;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[i][mb] *= alpha;
    }
  };

  // Thread tid < KT owns key tid of every tile: it sums the waves' column sums
  // of a finished tile into sbuf and later stores its own entries, so no
  // barrier orders the two.
  auto emit_scores = [&](int tile, const float* sw) __attribute__((always_inline)) {
    if constexpr (PASS == 2) {
      if (tid < KT) {
        float acc = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) acc += sw[ww * KT + tid];
        sbuf[((tile - tile_lo) % kScoreTiles) * KT + tid] = acc;
      }
    }
  };
  auto flush_scores = [&](int t0, int t1) __attribute__((always_inline)) {  // tiles [t0, t1]
    if constexpr (PASS == 2) {
      if (tid < KT) {
        float* dst = a.sig_part + ((int64_t)h * a.rt + rtile) * a.ldsig;
        for (int t = t0; t <= t1; ++t) {
          const int j = t * KT + tid;
          if (j < pool) dst[j] = sbuf[((t - tile_lo) % kScoreTiles) * KT + tid];
        }
      }
    }
  };

  // -- the tile loop (double-buffered LDS, one barrier per tile) -------------
  if (tile_end > tile_lo) {
    stage.store(Ks[0], Vt[0], tid);
    __syncthreads();
  }
  // nothing loaded before the loop is still in flight: otherwise the wait for
  // it (on a path the compiler cannot rule out) would sit inside the loop and
  // hold up every tile's prefetch
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  for (int tile = tile_lo; tile < tile_end; ++tile) {
    const int cur = (tile - tile_lo) & 1;
    const int key0 = tile * KT;
    const bool more = tile + 1 < tile_end;
    // the previous tile's score store goes out before the next tile's loads,
    // so that no wait for the store holds the loads up
    if constexpr (PASS == 2) {
      if (tile > tile_lo) emit_scores(tile - 1, sigw[cur ^ 1]);
    }
    if (more) stage_load(key0 + KT);
    bf16x8 kf[NKK];
    read_k(Ks[cur], 0, kf);
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
      const int kbase = key0 + kb * 32;
      // blocks inside the state (or, without the causal mask, inside the
      // pool) are fully visible to every query
      const bool masked = a.causal ? (kbase + 32 > c) : (kbase + 32 > pool);
      f32x16 sacc[QB];
      mfma_qk(kf, sacc);
      if constexpr (PASS == 1) {
        if (kb + 1 < KT / 32) read_k(Ks[cur], kb + 1, kf);
        SKV_FENCE();
        if (masked) stats_block(sacc, kbase, true);
        else stats_block(sacc, kbase, false);
      } else {
        u32x4 vf[NMB][2];
        read_v(Vt[cur], kb, vf);
        SKV_FENCE();
        u32x4 ph[QB][2];
        if constexpr (PASS == 2) {
          if (masked) scores_block(sacc, kbase, true, kb, sigw[cur], ph);
          else scores_block(sacc, kbase, false, kb, sigw[cur], ph);
        } else {
          if (masked) online_block(sacc, kbase, true, ph);
          else online_block(sacc, kbase, false, ph);
        }
        SKV_FENCE();
        mfma_pv(vf, ph);
        if (kb + 1 < KT / 32) read_k(Ks[cur], kb + 1, kf);
        SKV_FENCE();
      }
    }
    if constexpr (PASS == 2) {
      // the buffer is full: store it, and wait here (rarely) rather than
      // leave stores in flight into the next tile
      if (tile > tile_lo && (tile - 1 - tile_lo) % kScoreTiles == kScoreTiles - 1) {
        flush_scores(tile - kScoreTiles, tile - 1);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      }
    }
    if (more) stage.store(Ks[cur ^ 1], Vt[WITH_V ? cur ^ 1 : 0], tid);
    __syncthreads();
  }

  if constexpr (PASS == 2) {
    if (tile_end > tile_lo) {
      emit_scores(tile_end - 1, sigw[(tile_end - 1 - tile_lo) & 1]);
      const int t1 = tile_end - 1;
      flush_scores(max(tile_lo, t1 - (t1 - tile_lo) % kScoreTiles), t1);
    }
    // key tiles of this split that no query of the row tile can see
    for (int j = tile_end * KT + tid; j < min(tile_hi * KT, pool); j += kThreads)
      a.sig_part[((int64_t)h * a.rt + rtile) * a.ldsig + j] = 0.f;
    // O^T[d = 32mb + 8(r/4) + 4 half + r%4][query] -> O[t][g][d], P's 2^12
    // removed (exactly: a power of 2).  A single split is the output itself;
    // several write fp32 partials [S][T][Hq][d] that the select launch sums
    // in split order
#pragma unroll
    for (int i = 0; i < QB; ++i) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) oacc[i][mb] *= kPUnscale;
      if (a.S > 1) {
        // this split's partial [S][T][Hq][d], stored row-major through a
        // wave-private slice of the idle K (waves 0-3) or V^T (waves 4-7)
        // tile buffers: a lane holds one query's d values column-wise, so
        // direct stores would write 32-byte pieces of 32 rows each; via LDS
        // every store instruction writes whole rows.  Non-temporal: the lines
        // stream out instead of staying dirty in L2 until the kernel ends.
        // kCR d values per round.
        // Every lane of the wave takes part (a lane stores pieces of other
        // lanes' rows); the block's validity is uniform over the wave.
        constexpr int kCR = D == 128 ? 64 : 32;
        constexpr int kOLd = kCR + 4;  // floats per staged row (16-byte aligned)
        constexpr int kPerRow = kCR / 4;  // 16-byte pieces per row and round
        static_assert(4 * 32 * kOLd * 4 <= (int)sizeof(Ks), "K tile buffers hold 4 slices");
        static_assert(4 * 32 * kOLd * 4 <= (int)sizeof(Vt), "V tile buffers hold 4 slices");
        static_assert(32 * kPerRow % 64 == 0, "whole store instructions per round");
        const int b = b0 + w * QB + i;
        if (b >= a.nqblk) continue;
        const int tok0 = (b / a.G) * kTokBlk;  // the block's tokens: tok0 + lane row
        const int qh = h * a.G + b % a.G;
        float* ot = reinterpret_cast<float*>(w < 4 ? (void*)&Ks[0][0] : (void*)&Vt[0][0]) +
                    (w & 3) * 32 * kOLd;
        float* dst = a.o_out + ((int64_t)s * a.T * a.Hq + qh) * D;
#pragma unroll
        for (int h2 = 0; h2 < D / kCR; ++h2) {
#pragma unroll
          for (int m2 = 0; m2 < kCR / 32; ++m2) {
            const int mb = (kCR / 32) * h2 + m2;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                         oacc[i][mb][4 * q4 + 3]};
              *reinterpret_cast<f32x4*>(ot + l32 * kOLd + m2 * 32 + 8 * q4 + 4 * half) = v;
            }
          }
          // LDS accesses of one wave complete in order; keep the compiler
          // from moving the reads above the writes (or the next round's
          // writes above these reads)
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int u = 0; u < 32 * kPerRow / 64; ++u) {
            const int p = u * 64 + lane;
            const int r = p / kPerRow, c4 = p % kPerRow;
            const f32x4 v = *reinterpret_cast<const f32x4*>(ot + r * kOLd + c4 * 4);
            if (tok0 + r < a.T)
              __builtin_nontemporal_store(
                  v, reinterpret_cast<f32x4*>(dst + (int64_t)(tok0 + r) * a.Hq * D + kCR * h2 + c4 * 4));
          }
          __builtin_amdgcn_wave_barrier();
        }
        continue;
      }
      if (qtok[i] < 0) continue;
      float* dst = a.o_out + ((int64_t)qtok[i] * a.Hq + qhead[i]) * D;
      if (a.out_bf16) {  // the output itself, as bf16 (same element offsets)
        __bf16* dst16 = reinterpret_cast<__bf16*>(a.o_out) + ((int64_t)qtok[i] * a.Hq + qhead[i]) * D;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                       oacc[i][mb][4 * q4 + 3]};
            *reinterpret_cast<bf16x4*>(dst16 + mb * 32 + 8 * q4 + 4 * half) =
                __builtin_convertvector(v, bf16x4);
          }
        continue;
      }
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                     oacc[i][mb][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * q4 + 4 * half) = v;
        }
    }
  } else if constexpr (PASS == 3) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const float lt = lrun[i] + __shfl_xor(lrun[i], 32);  // both halves: same running max
      if (qtok[i] < 0) continue;
      const int64_t row = (int64_t)qtok[i] * a.Hq + qhead[i];
      const bool direct = a.S == 1;
      const float scale = direct ? 1.f / lt : kPUnscale;
      float* dst = a.o_out + ((direct ? 0 : (int64_t)s * a.T * a.Hq) + row) * D;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                     oacc[i][mb][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * q4 + 4 * half) = v * scale;
        }
      if (!direct && half == 0) {
        const int64_t idx = ((int64_t)s * a.Hq + qhead[i]) * a.tpad + qtok[i];
        a.m_part[idx] = mrun[i];
        a.l_part[idx] = lt * kPUnscale;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const float mo = __shfl_xor(mrun[i], 32);
      const float lo = __shfl_xor(lrun[i], 32);
      const float M = fmaxf(mrun[i], mo);
      float L = 0.f;
      if (mrun[i] > -INFINITY) L += lrun[i] * exp2f((mrun[i] - M) * sl2);
      if (mo > -INFINITY) L += lo * exp2f((mo - M) * sl2);
      if (half == 0 && qtok[i] >= 0) {
        // the split's log-sum-exp (base 2, scaled logits); -inf: no key of
        // the split is visible to the row
        const int64_t idx = ((int64_t)s * a.Hq + qhead[i]) * a.tpad + qtok[i];
        a.m_part[idx] = L > 0.f ? M * sl2 + log2f(L) : -INFINITY;
      }
    }
  }
}

// Full-attention split combine: O = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^((m_s - M) * scale_log2), splits in order.
template <int D>
__global__ __launch_bounds__(256) void full_combine_kernel(AttnArgs a, float* o) {
  const int64_t n4 = (int64_t)a.T * a.Hq * (D / 4);
  const int64_t stride = (int64_t)a.Hq * a.tpad;
  const int64_t ostride = (int64_t)a.T * a.Hq * D;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n4;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tg = idx / (D / 4);
    const int d4 = (int)(idx % (D / 4));
    const int g = (int)(tg % a.Hq), t = (int)(tg / a.Hq);
    const int64_t row = (int64_t)g * a.tpad + t;
    float M = -INFINITY;
    for (int sp = 0; sp < a.S; ++sp) M = fmaxf(M, a.m_part[sp * stride + row]);
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < a.S; ++sp) {
      const float ms = a.m_part[sp * stride + row];
      if (ms > -INFINITY) {
        const float wgt = exp2f((ms - M) * a.scale_log2);
        L += wgt * a.l_part[sp * stride + row];
        acc += wgt * reinterpret_cast<const f32x4*>(a.o_out + sp * ostride + tg * D)[d4];
      }
    }
    reinterpret_cast<f32x4*>(o + tg * D)[d4] = acc / L;
  }
}

namespace {
int attn_grid(const AttnArgs& a) { return a.Hkv * a.S * a.rt; }

template <int PASS, bool CIND>
hipError_t launch_pass_as(const AttnArgs& a, int D, const Stream& st) {
  if (D == 128)
    hipExtLaunchKernelGGL((attn_kernel<128, PASS, CIND>), dim3(attn_grid(a)), dim3(kThreads), 0,
                          st.st, st.start, st.stop, 0, a);
  else
    hipExtLaunchKernelGGL((attn_kernel<64, PASS, CIND>), dim3(attn_grid(a)), dim3(kThreads), 0,
                          st.st, st.start, st.stop, 0, a);
  return hipGetLastError();
}

template <int PASS>
hipError_t launch_pass(const AttnArgs& a, int D, const Stream& st) {
  if constexpr (PASS == 3) {
    return launch_pass_as<3, false>(a, D, st);  // the baseline's state is D itself
  } else {
    return a.cpos ? launch_pass_as<PASS, true>(a, D, st) : launch_pass_as<PASS, false>(a, D, st);
  }
}
}  // namespace

hipError_t launch_attn_stats(const AttnArgs& a, int D, const Stream& st) {
  return launch_pass<1>(a, D, st);
}

hipError_t launch_attn_out(const AttnArgs& a, int D, const Stream& st) {
  return launch_pass<2>(a, D, st);
}

hipError_t launch_full_attn(const AttnArgs& a, int D, const Stream& st) {
  return launch_pass<3>(a, D, st);
}

hipError_t launch_full_combine(const AttnArgs& a, float* o, int D, const Stream& st) {
  const int64_t n4 = (int64_t)a.T * a.Hq * (D / 4);
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (D == 128)
    hipExtLaunchKernelGGL((full_combine_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st.st, st.start, st.stop, 0, a, o);
  else
    hipExtLaunchKernelGGL((full_combine_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st.st, st.start, st.stop, 0, a, o);
  return hipGetLastError();
}

}  // namespace skv
