// Fused GQA attention over the StateKV candidate pool [C_{n-1} ; frame n] for
// gfx950, in two passes that share one tiling:
//
//   pass 1 (statistics): per query row, the max and the sum of exp of the
//     logits over this workgroup's key split (online, per 32-key block);
//   pass 2 (output + scores): combines the split statistics into the row
//     log-sum-exp, recomputes the logits, forms the normalised probabilities
//     P, accumulates O = P V and the column sums of P (the candidates'
//     importance, summed over the queries of every query head that shares the
//     KV head).
//
// The per-frame step these passes implement is the attention and importance
// part of StateKV (paper.rainbus.top, method-steps section: softmax over the
// concatenated compressed memory and frame keys; a candidate's importance is
// the sum over queries of its attention weight; paperlayer.ai App. A.3: cache
// building needs the attention weights or sufficient statistics, which fused
// attention kernels normally do not expose -- the row statistics of pass 1
// are exactly those statistics).
//
// Layout of the work: the G query heads that share KV head h and the T frame
// tokens form G*T query rows, cut into 32-token blocks of one head.  A
// workgroup (4 waves) owns 8 such blocks (a row tile) and one contiguous split
// of the pool's key tiles.  Logits are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16 (keys on M, queries on N): each lane then holds one
// query and 16 keys, so the row statistics need no cross-lane work, the
// probabilities feed the PV product O^T = V^T P^T
// (v_mfma_f32_32x32x16_f16) straight from registers, and the column sums are
// a short butterfly across the 32 lanes of each half-wave.  P enters PV as
// fp16 scaled by 2^12 (11 significant bits, kept clear of fp16 subnormals);
// V is converted bf16 -> fp16 (exact for |v| in [2^-17, 65504]) while it is
// transposed into LDS.  Scores and O partials are written per split / row
// tile and reduced in a fixed order elsewhere: no atomics, bitwise
// reproducible results.
#include "../skv_internal.h"

namespace skv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = kWaves * 64;
constexpr int kKPad = 8;  // bf16 padding per K row in LDS (conflict-free b128 reads)
constexpr int kVPad = 4;  // fp16 padding per V^T row (conflict-free b64 reads)
constexpr float kPUnscale = 1.f / 4096.f;

// Workgroups are dealt to the 8 XCDs round-robin; renumber them so that each
// XCD gets a contiguous range of logical ids (consecutive ids share a KV head
// and key split, hence the same K/V tiles in that XCD's L2).
__device__ inline int xcd_logical_id(int b, int n) {
  const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

__device__ inline float swizzle_xor16(float x) {
  // ds_swizzle bit mode: and_mask 0x1F, or_mask 0, xor_mask 0x10 (32-lane groups)
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

// Sum of v[r] over the 32 lanes of each half-wave, one key per lane pair.
// Reduce-scatter butterfly: partners lane^16, lane^8 (row_ror:8), lane^7
// (row_half_mirror), lane^2, lane^1 (quad_perm).  Lane l ends with the total
// of register r = (l >> 1) & 15 (both lanes of a pair hold it).
__device__ inline float colsum_reduce(float (&v)[16], int l32) {
  const bool b4 = l32 & 16, b3 = l32 & 8, b2 = l32 & 4, b1 = l32 & 2;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float send = b4 ? v[k] : v[k + 8];
    const float keep = b4 ? v[k + 8] : v[k];
    v[k] = keep + swizzle_xor16(send);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float send = b3 ? v[k] : v[k + 4];
    const float keep = b3 ? v[k + 4] : v[k];
    v[k] = keep + dpp<0x128>(send);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float send = b2 ? v[k] : v[k + 2];
    const float keep = b2 ? v[k + 2] : v[k];
    v[k] = keep + dpp<0x141>(send);
  }
  {
    const float send = b1 ? v[0] : v[1];
    const float keep = b1 ? v[1] : v[0];
    v[0] = keep + dpp<0x4E>(send);
  }
  return v[0] + dpp<0xB1>(v[0]);
}

__device__ inline float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// One 16-byte chunk (8 bf16) of pool row j, columns [col, col+8); zero past the pool.
template <int D>
__device__ inline u32x4 pool_chunk(const uint16_t* state, const uint16_t* frame, int64_t ldc,
                                   int Hkv, int h, int c, int pool, int j, int col) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (j < c)
    v = *reinterpret_cast<const u32x4*>(state + ((int64_t)h * ldc + j) * D + col);
  else if (j < pool)
    v = *reinterpret_cast<const u32x4*>(frame + ((int64_t)(j - c) * Hkv + h) * D + col);
  return v;
}

template <int D, int PASS>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  constexpr int QB = kQBlkPerWave;
  constexpr int KT = kKeyTile;
  constexpr int NKK = D / 16;  // k-steps of the QK^T MFMA
  constexpr int NMB = D / 32;  // 32-row blocks of O^T
  constexpr int KLD = D + kKPad;
  constexpr int VLD = KT + kVPad;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KLD];
  __shared__ __attribute__((aligned(16))) _Float16 Vt[PASS >= 2 ? D * VLD : 8];
  __shared__ float sigw[PASS == 2 ? kWaves * KT : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
  const int rtile = lid % a.rt;
  const int hs = lid / a.rt;
  const int s = hs % a.S;
  const int h = hs / a.S;
  const int c = a.c;
  const int pool = c + a.T;
  const int ntiles = (pool + KT - 1) / KT;
  const int tile_lo = (int)((int64_t)s * ntiles / a.S);
  const int tile_hi = (int)((int64_t)(s + 1) * ntiles / a.S);
  const float sl2 = a.scale_log2;

  // This wave's query blocks: block b = tb*G + gl holds tokens [32tb, 32tb+32)
  // of query head h*G + gl.  Lane l32 owns token 32tb + l32 of each block.
  const int b0 = rtile * kRowBlk;
  int qtok[QB], qhead[QB];
  int wave_tmax = -1;
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
      wave_tmax = max(wave_tmax, min(a.T - 1, tb * kTokBlk + kTokBlk - 1));
    }
  }
  const int blast = min(b0 + kRowBlk, a.nqblk) - 1;
  const int wg_tmax = min(a.T - 1, (blast / a.G) * kTokBlk + kTokBlk - 1);
  const int wg_klim = a.causal ? c + wg_tmax + 1 : pool;
  const int wave_klim = wave_tmax < 0 ? 0 : (a.causal ? c + wave_tmax + 1 : pool);
  const int tile_end = max(tile_lo, min(tile_hi, (wg_klim + KT - 1) / KT));

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
  f32x16 oacc[QB][NMB];
#pragma unroll
  for (int i = 0; i < QB; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
    lse2[i] = INFINITY;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) oacc[i][mb] = f32x16{};
  }
  if constexpr (PASS == 2) {
    // Row log-sum-exp (base 2, scaled logits) from the split statistics,
    // combined in split order; 12 is subtracted so that P comes out * 2^12.
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      if (qtok[i] < 0) continue;
      const int64_t row = (int64_t)qhead[i] * a.tpad + qtok[i];
      const int64_t stride = (int64_t)a.Hq * a.tpad;
      float M = -INFINITY;
      for (int sp = 0; sp < a.S; ++sp) M = fmaxf(M, a.m_part[sp * stride + row]);
      float L = 0.f;
      for (int sp = 0; sp < a.S; ++sp) {
        const float ms = a.m_part[sp * stride + row];
        if (ms > -INFINITY) L += a.l_part[sp * stride + row] * exp2f((ms - M) * sl2);
      }
      lse2[i] = M * sl2 + log2f(L) - 12.f;
    }
  }

  auto emit_scores = [&](int tile) {
    if constexpr (PASS == 2) {
      if (tid < KT) {
        const int j = tile * KT + tid;
        if (j < pool) {
          float acc = 0.f;
#pragma unroll
          for (int ww = 0; ww < kWaves; ++ww) acc += sigw[ww * KT + tid];
          a.sig_part[((int64_t)h * a.rt + rtile) * a.ldsig + j] = acc;
        }
      }
    }
  };

  for (int tile = tile_lo; tile < tile_end; ++tile) {
    const int key0 = tile * KT;
    __syncthreads();  // LDS tiles free; previous tile's sigw complete
    if (tile > tile_lo) emit_scores(tile - 1);
    for (int ch = tid; ch < KT * (D / 8); ch += kThreads) {
      const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&Ks[row * KLD + col]) =
          pool_chunk<D>(a.kc, a.kf, a.ldc, a.Hkv, h, c, pool, key0 + row, col);
    }
    if constexpr (PASS >= 2) {
      for (int it = tid; it < (KT / 2) * (D / 8); it += kThreads) {
        const int kp = it % (KT / 2), dc = (it / (KT / 2)) * 8;
        const u32x4 v0 = pool_chunk<D>(a.vc, a.vf, a.ldc, a.Hkv, h, c, pool, key0 + 2 * kp, dc);
        const u32x4 v1 =
            pool_chunk<D>(a.vc, a.vf, a.ldc, a.Hkv, h, c, pool, key0 + 2 * kp + 1, dc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f16x2 lo = {(_Float16)bf16lo(v0[e]), (_Float16)bf16lo(v1[e])};
          f16x2 hi = {(_Float16)bf16hi(v0[e]), (_Float16)bf16hi(v1[e])};
          *reinterpret_cast<f16x2*>(&Vt[(dc + 2 * e) * VLD + 2 * kp]) = lo;
          *reinterpret_cast<f16x2*>(&Vt[(dc + 2 * e + 1) * VLD + 2 * kp]) = hi;
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
      const int kbase = key0 + kb * 32;
      float cs[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) cs[r] = 0.f;
      if (kbase < wave_klim) {
        f32x16 sacc[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) sacc[i] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 ak =
              *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + l32) * KLD + kk * 16 + half * 8]);
#pragma unroll
          for (int i = 0; i < QB; ++i)
            sacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[i][kk], sacc[i], 0, 0, 0);
        }
        // lane holds S^T[key = kbase + 8(r/4) + 4 half + r%4][query qtok]
        if constexpr (PASS == 1) {
#pragma unroll
          for (int i = 0; i < QB; ++i) {
            float z[16];
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = kbase + 8 * (r >> 2) + 4 * half + (r & 3);
              const bool vis = j < pool && (j < c || !a.causal || j - c <= qtok[i]);
              z[r] = vis ? sacc[i][r] : -INFINITY;
              mx = fmaxf(mx, z[r]);
            }
            if (mx > -INFINITY) {
              const float mnew = fmaxf(mrun[i], mx);
              const float ms = mnew * sl2;
              float sum = 0.f;
#pragma unroll
              for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(z[r], sl2, -ms));
              lrun[i] = lrun[i] * __builtin_amdgcn_exp2f(fmaf(mrun[i], sl2, -ms)) + sum;
              mrun[i] = mnew;
            }
          }
        } else {
          f16x8 ph[QB][2];
          if constexpr (PASS == 2) {
#pragma unroll
            for (int i = 0; i < QB; ++i) {
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int j = kbase + 8 * (r >> 2) + 4 * half + (r & 3);
                const bool vis = j < pool && (j < c || !a.causal || j - c <= qtok[i]);
                const float p =
                    vis ? __builtin_amdgcn_exp2f(fmaf(sacc[i][r], sl2, -lse2[i])) : 0.f;
                cs[r] += p;
                ph[i][r >> 3][r & 7] = (_Float16)p;
              }
            }
          } else {
            // online softmax: running max shared by the two half-waves that
            // hold the same query; O^T and l rescaled when the max grows
#pragma unroll
            for (int i = 0; i < QB; ++i) {
              float z[16];
              float mx = -INFINITY;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int j = kbase + 8 * (r >> 2) + 4 * half + (r & 3);
                const bool vis = j < pool && (j < c || !a.causal || j - c <= qtok[i]);
                z[r] = vis ? sacc[i][r] : -INFINITY;
                mx = fmaxf(mx, z[r]);
              }
              mx = fmaxf(mx, __shfl_xor(mx, 32));
              const float mnew = fmaxf(mrun[i], mx);
              if (mnew == -INFINITY) {
#pragma unroll
                for (int r = 0; r < 16; ++r) ph[i][r >> 3][r & 7] = (_Float16)0.f;
                continue;
              }
              const float alpha = __builtin_amdgcn_exp2f((mrun[i] - mnew) * sl2);
              const float ms = fmaf(mnew, sl2, -12.f);
              float sum = 0.f;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(z[r], sl2, -ms));
                sum += p;
                ph[i][r >> 3][r & 7] = (_Float16)p;
              }
              lrun[i] = lrun[i] * alpha + sum;
              mrun[i] = mnew;
#pragma unroll
              for (int mb = 0; mb < NMB; ++mb) oacc[i][mb] *= alpha;
            }
          }
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
            for (int slab = 0; slab < 2; ++slab) {
              const _Float16* vrow = &Vt[(mb * 32 + l32) * VLD + kb * 32 + slab * 16 + 4 * half];
              const f16x4 lo = *reinterpret_cast<const f16x4*>(vrow);
              const f16x4 hi = *reinterpret_cast<const f16x4*>(vrow + 8);
              const f16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
              for (int i = 0; i < QB; ++i)
                oacc[i][mb] =
                    __builtin_amdgcn_mfma_f32_32x32x16_f16(av, ph[i][slab], oacc[i][mb], 0, 0, 0);
            }
          }
        }
      }
      if constexpr (PASS == 2) {
        const float tot = colsum_reduce(cs, l32);
        if (!(l32 & 1)) {
          const int r = l32 >> 1;
          sigw[w * KT + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3)] = tot * kPUnscale;
        }
      }
    }
  }

  if constexpr (PASS == 2) {
    __syncthreads();
    if (tile_end > tile_lo) emit_scores(tile_end - 1);
    // key tiles of this split that no query of the row tile can see
    for (int j = tile_end * KT + tid; j < min(tile_hi * KT, pool); j += kThreads)
      a.sig_part[((int64_t)h * a.rt + rtile) * a.ldsig + j] = 0.f;
    // O^T[d = 32mb + 8(r/4) + 4 half + r%4][query] -> O[t][g][d]
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      if (qtok[i] < 0) continue;
      float* dst = a.o_out + ((int64_t)(a.S == 1 ? 0 : s) * a.T + qtok[i]) * a.Hq * D +
                   (int64_t)qhead[i] * D;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                     oacc[i][mb][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * q4 + 4 * half) = v * kPUnscale;
        }
    }
  } else if constexpr (PASS == 3) {
#pragma unroll
    for (int i = 0; i < QB; ++i) {
      const float lt = lrun[i] + __shfl_xor(lrun[i], 32);  // both halves: same running max
      if (qtok[i] < 0) continue;
      const int64_t row = (int64_t)qtok[i] * a.Hq + qhead[i];
      if (a.S == 1) {
        const float inv = 1.f / lt;
        float* dst = a.o_out + row * D;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                       oacc[i][mb][4 * q4 + 3]};
            *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * q4 + 4 * half) = v * inv;
          }
      } else {
        float* dst = a.o_out + ((int64_t)s * a.T * a.Hq + row) * D;
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v = {oacc[i][mb][4 * q4], oacc[i][mb][4 * q4 + 1], oacc[i][mb][4 * q4 + 2],
                       oacc[i][mb][4 * q4 + 3]};
            *reinterpret_cast<f32x4*>(dst + mb * 32 + 8 * q4 + 4 * half) = v * kPUnscale;
          }
        if (half == 0) {
          const int64_t idx = ((int64_t)s * a.Hq + qhead[i]) * a.tpad + qtok[i];
          a.m_part[idx] = mrun[i];
          a.l_part[idx] = lt * kPUnscale;
        }
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
        const int64_t idx = ((int64_t)s * a.Hq + qhead[i]) * a.tpad + qtok[i];
        a.m_part[idx] = M;
        a.l_part[idx] = L;
      }
    }
  }
}

__global__ __launch_bounds__(256) void split_sum_kernel(const f32x4* part, int S, int64_t n4,
                                                        f32x4* o) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    f32x4 acc = part[i];
    for (int sp = 1; sp < S; ++sp) acc += part[sp * n4 + i];
    o[i] = acc;
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
}  // namespace

hipError_t launch_full_attn(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL((attn_kernel<128, 3>), dim3(attn_grid(a)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<64, 3>), dim3(attn_grid(a)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_full_combine(const AttnArgs& a, float* o, int D, hipStream_t st) {
  const int64_t n4 = (int64_t)a.T * a.Hq * (D / 4);
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (D == 128)
    hipLaunchKernelGGL((full_combine_kernel<128>), dim3((unsigned)blocks), dim3(256), 0, st, a, o);
  else
    hipLaunchKernelGGL((full_combine_kernel<64>), dim3((unsigned)blocks), dim3(256), 0, st, a, o);
  return hipGetLastError();
}

hipError_t launch_attn_stats(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL((attn_kernel<128, 1>), dim3(attn_grid(a)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<64, 1>), dim3(attn_grid(a)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_out(const AttnArgs& a, int D, hipStream_t st) {
  if (D == 128)
    hipLaunchKernelGGL((attn_kernel<128, 2>), dim3(attn_grid(a)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<64, 2>), dim3(attn_grid(a)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_split_sum(const float* part, int S, int64_t n, float* o, hipStream_t st) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     reinterpret_cast<const f32x4*>(part), S, n4, reinterpret_cast<f32x4*>(o));
  return hipGetLastError();
}

}  // namespace skv
