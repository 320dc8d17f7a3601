// Backward pass of the causal Parallax prefill in bf16 on CDNA4 matrix cores.
//
// The pages (page "Parallax - Parameterized Local Linear Attention for Language
// Modeling") describe the forward pass only (section "Core mechanism", Eq. 2);
// the backward pass is its exact derivative.  With S = scale Q K^T (causal),
// W = rowsoftmax(S), R = rho K^T, rbar = rowsum(W*R), the correction
// C = (W*R) V - (W V) rbar and O = W V - g C, the gradients of sum(O * dO) are
//     Delta = dO V^T,  D = rowsum(dO * (O + g C)),  F = rowsum(dO * O)
//     dV   = (W * (1 - g (R - rbar)))^T dO
//     dR   = g W * (D - Delta)
//     dS'  = scale W * (Delta * (1 - g (R - rbar)) + g (R - rbar) D - F)
//     dQ   = dS' K,   dK = dS'^T Q + dR^T rho,   drho = dR K
//     dg   = -sum over rows of <dO, C>
// W is recomputed from the scores and the saved log partition function; rbar
// and C come from the training forward pass.
//
// Kernels (one stream, in this order):
//   bwd_prep_kernel   dO -> bf16 (row-major copy), per-row constants of the
//                     elementwise step and per-tile partials of <dO, C>.
//   stage_v_kernel    (bf16 output) transposed 64-key tiles of K, the K^T
//                     operand of the query-stationary kernel.
//   bwd_dkdv_kernel   key-stationary: a workgroup owns 16*KB*NW keys, each wave
//                     16*KB of them with their K and V fragments in registers;
//                     it streams the later queries through LDS in steps of 32
//                     and accumulates dK^T and dV^T on the matrix cores.
//   bwd_dq_kernel     query-stationary: a workgroup owns 16*NW queries (16 per
//                     wave), streams the causal key range through LDS in tiles
//                     of 64 and accumulates dQ^T and drho^T.
//   bwd_dgate_kernel  sums the <dO, C> partials per head in a fixed order.
// Both main kernels recompute S, R and Delta (three products) and add two or
// three more, so no gradient needs atomics and the result is deterministic.
// The elementwise products W~, dS' and dR are rounded to bf16 for the second
// set of MFMAs, as are dO and every input; all sums are fp32.

#include <type_traits>

#include "plx_common.h"

namespace plx {

constexpr int BW_T = 64;    // keys per tile of the query-stationary kernel (the forward's tile)
constexpr int BW_BQ = 32;   // queries per step of the key-stationary kernel

// Launch shapes (waves per workgroup, 16-key blocks per wave), per head dimension.
// At d = 128 the key-stationary kernel is bound by LDS bandwidth: every wave
// reads each step's query tiles twice (score fragments and transposed halves),
// 56 KB of LDS reads per wave and 32-query step for 48 MFMAs.  Two 16-key blocks
// per wave would halve that, but the dK and dV accumulators of 32 keys need 128
// VGPRs and the kernel then no longer fits two waves per SIMD.
// Grid order of the dK/dV and dQ kernels, per head dimension: 0 = the tiles of
// all heads in order of work with heads fastest; G > 0 = the same within groups
// of G heads, group after group (more tiles of fewer heads share each XCD's L2).
// Measured against 0 (bit-identical results): G = 32 at d = 128, -3.2 % on
// B4 H16 L4096; G = 16 at d = 64, -6.7 % on B2 H32 L16384.
#ifndef PLX_BW_HEAD_GROUP_D128
#define PLX_BW_HEAD_GROUP_D128 32
#endif
#ifndef PLX_BW_HEAD_GROUP_D64
#define PLX_BW_HEAD_GROUP_D64 16
#endif
#ifndef PLX_BW_KV_NW_D128
#define PLX_BW_KV_NW_D128 8
#endif
#ifndef PLX_BW_KV_KB_D128
#define PLX_BW_KV_KB_D128 1
#endif
#ifndef PLX_BW_KV_NW_D64
#define PLX_BW_KV_NW_D64 4
#endif
#ifndef PLX_BW_KV_KB_D64
#define PLX_BW_KV_KB_D64 2
#endif
#ifndef PLX_BW_Q_NW_D128
#define PLX_BW_Q_NW_D128 8
#endif
#ifndef PLX_BW_Q_NW_D64
#define PLX_BW_Q_NW_D64 8
#endif

// Row-major tile, D bf16 features per row.  16-byte chunk c of row r sits at
// physical chunk c ^ rm_swz<D>(r), chosen so that both fragment reads are free
// of bank conflicts:
//   * 16-byte reads of one chunk in 16 consecutive rows (each 16-lane phase),
//     the score products' operands: the swizzle is a bijection over 16 rows
//     (over the 8 rows of each parity for D = 64, two rows per bank line);
//   * 8-byte transposed reads (ds_read_b64_tr_b16), the accumulation products'
//     operands: 16-lane group a reads chunks 2m and 2m+1 of rows 4a .. 4a+3
//     (mod 16), and two groups share a cycle, as (0,1) and (2,3) or as (0,2)
//     and (1,3).  A row's two chunks land on the slot pair p = rm_swz >> 1, so
//     the pairs of rows in groups sharing a cycle must differ: groups 0 and 3
//     take one half of the pair indices, groups 1 and 2 the other (a Gray-code
//     split), and the low bit separates 0 from 3 and 1 from 2.
// D = 128: row r = 4a + i, p = 4 [a in {1,2}] + i, swizzle 2p + [a >= 2].
// D = 64: row r = 4a + 2i + parity, p = 2 [a in {1,2}] + i, swizzle 2p + [a >= 2].
template <int D>
__device__ __forceinline__ int rm_swz(int r) {
  const int a = (r >> 2) & 3;
  const int mid = (a ^ (a >> 1)) & 1;            // a is 1 or 2
  if constexpr (D == 128) return 2 * (4 * mid + (r & 3)) + (a >> 1);
  else return 2 * (2 * mid + ((r >> 1) & 1)) + (a >> 1);
}
template <int D>
__device__ __forceinline__ int rm_off(int r, int c) {
  return r * D + ((c ^ rm_swz<D>(r)) << 3);
}

// The query-stationary kernel's K and V tiles: 16-byte chunks XOR-swizzled by
// row (its fragment reads are all 16-byte reads of 16 consecutive rows), and
// its K^T operand comes from a staged transposed tile (one row of W = 64
// positions per feature) with the forward's V^T swizzle c ^ (f & 7), so that
// eight lanes at a time hit eight different 16-byte slots of a bank line.  (A
// transposed LDS read of K would save the staging but needs eight more live
// address registers, which push this kernel past 256 VGPRs at d = 128.)
template <int D>
__device__ __forceinline__ int rm_off_q(int r, int c) {
  return r * D + ((c ^ (r & (D / 8 - 1))) << 3);
}
__device__ __forceinline__ int tr_off64(int f, int c) { return f * 64 + ((c ^ (f & 7)) << 3); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed fragment of a row-major tile: for lane (c16, g4), feature f0 + c16
// of rows r0 + 4 g4 + 0..3 and r0 + 16 + 4 g4 + 0..3, the order in which a lane
// holds rows of two stacked 16-row score blocks.  ds_read_b64_tr_b16 (measured
// on gfx950): in each 16-lane group, lane i receives element i mod 4 of the
// 8-byte chunks addressed by lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12; so lane j
// addresses features f0 + 4 (j mod 4) .. +3 of row (j / 4) of the 4-row block.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int r0, int f0, int c16, int g4) {
  const int c = (f0 >> 3) + ((c16 & 3) >> 1);    // logical chunk of features f0 + 4 (c16 & 3)
  const int e = 4 * (c16 & 1);                   // their first element within the chunk
  const int r = r0 + 4 * g4 + (c16 >> 2);
  // rm_swz repeats every 16 rows: the second block is the same offset 16 rows on
  const uint16_t* p = tile + rm_off<D>(r, c) + e;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 16 * D));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------------------- prep
// 64 rows per workgroup.  Each lane handles 4 consecutive features of a row,
// so one wave instruction reads 64 / (D/4) whole rows of each fp32 input.
template <int D>
__global__ __launch_bounds__(256)
void bwd_prep_kernel(const float* __restrict__ dout, const float* __restrict__ out,
                     const float* __restrict__ corr, const float* __restrict__ lse,
                     const float* __restrict__ rbar, const float* __restrict__ gate,
                     __bf16* __restrict__ do16, f32x4* __restrict__ stats,
                     float* __restrict__ gpart, int H, int L, int n_t) {
  constexpr int LPR = D / 4;                 // lanes per row
  constexpr int RPW = 64 / LPR;              // rows per wave instruction
  constexpr int ITER = 16 / RPW;             // 16 rows per wave
  __shared__ float red[4];
  const int bh = blockIdx.x / n_t, t = blockIdx.x % n_t;
  const int h = bh % H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int sub = lane % LPR;
  const float g = gate[h];
  float gsum = 0.f;
  f32x4 dx[ITER], ox[ITER], cx[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int row = t * 64 + wave * 16 + it * RPW + lane / LPR;
    if (row < L) {
      const size_t o = ((size_t)bh * L + row) * D + 4 * sub;
      dx[it] = *reinterpret_cast<const f32x4*>(dout + o);
      ox[it] = *reinterpret_cast<const f32x4*>(out + o);
      cx[it] = *reinterpret_cast<const f32x4*>(corr + o);
    } else {
      dx[it] = ox[it] = cx[it] = f32x4{};
    }
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int row = t * 64 + wave * 16 + it * RPW + lane / LPR;
    float fo = 0.f, fc = 0.f, gx = 0.f;
    __bf16 pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pk[e] = (__bf16)dx[it][e];
      const float dr = (float)pk[e];
      fo = fmaf(dr, ox[it][e], fo);
      fc = fmaf(dr, cx[it][e], fc);
      gx = fmaf(dx[it][e], cx[it][e], gx);
    }
    fo = group_sum<LPR>(fo);
    fc = group_sum<LPR>(fc);
    gx = group_sum<LPR>(gx);
    if (row < L) {
      const size_t o = ((size_t)bh * L + row) * D + 4 * sub;
      uint2 w;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, pk[0]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, pk[1]) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, pk[2]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, pk[3]) << 16);
      *reinterpret_cast<uint2*>(do16 + o) = w;
      if (sub == 0) {
        // D uses o_sa = o + g C; both D and F come from the rounded dO that the
        // products Delta = dO V^T see, so that the dS rows sum to zero.  Stored
        // as the constants of the elementwise step (bwd_elt).
        const float rb = rbar[(size_t)bh * L + row];
        const float gD = g * fmaf(g, fc, fo);
        stats[(size_t)bh * L + row] = f32x4{-lse[(size_t)bh * L + row] * kLog2e,
                                            fmaf(g, rb, 1.f), gD, -fmaf(gD, rb, fo)};
        gsum += gx;                          // exact fp32 dO; row order fixed
      }
    }
  }
  // tile partial of sum <dO, C>: lanes, then waves, in a fixed order
  gsum = group_sum<32>(gsum);
  gsum += __shfl_xor(gsum, 32);
  if (lane == 0) red[wave] = gsum;
  __syncthreads();
  if (tid == 0) gpart[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// dgate[h] = -sum over b and tiles of the partials: one wave per head, each
// lane a fixed strided subset, then a fixed reduction tree.
__global__ __launch_bounds__(64)
void bwd_dgate_kernel(const float* __restrict__ gpart, float* __restrict__ dgate, int B, int H,
                      int n_t) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x;
  float s = 0.f;
  for (int b = 0; b < B; ++b)
    for (int t = lane; t < n_t; t += 64) s += gpart[((size_t)b * H + h) * n_t + t];
  s = group_sum<32>(s);
  s += __shfl_xor(s, 32);
  if (lane == 0) dgate[h] = -s;
}

// Elementwise step shared by both main kernels, for one (query i, key j):
// score s (the raw <q,k>), r = <rho,k>, dl = <dO,v>, and the row's constants
//   st = {-lse_i log2e, 1 + g rbar_i, g D_i, -(g D_i rbar_i + F_i)}.
// Returns W~ = w (1 - g (r - rbar)), dS/scale = w (dl (1 - g (r - rbar)) +
// g D (r - rbar) - F) and dR = g w (D - dl); the factor `scale` of dS is applied
// to the accumulated products instead of to every element.
struct BwdElt {
  float wt, ds, dr;
};
template <bool MASK>
__device__ __forceinline__ BwdElt bwd_elt(bool keep, float s, float r, float dl, f32x4 st,
                                          float ng, float sl2) {
  float w = __builtin_amdgcn_exp2f(fmaf(s, sl2, st[0]));
  if constexpr (MASK) w = keep ? w : 0.f;      // a masked score contributes exact zeros
  const float t1 = fmaf(ng, r, st[1]);
  BwdElt e;
  e.wt = w * t1;
  e.ds = w * fmaf(dl, t1, fmaf(st[2], r, st[3]));
  e.dr = w * fmaf(ng, dl, st[2]);
  return e;
}

// ------------------------------------------------------- key-stationary dK, dV
// Block b of a BH * n_t grid -> (tile rank t, head bh) in the grid order above.
template <int G>
__device__ __forceinline__ void bwd_grid_order(int b, int BH, int n_t, int* t, int* bh) {
  if constexpr (G > 0) {
    const int full = BH / G;
    const int g = b / (G * n_t);
    const int gs = g < full ? G : BH - full * G;
    const int r = b - g * G * n_t;
    *t = r / gs;
    *bh = g * G + r % gs;
  } else {
    *t = b / BH;
    *bh = b % BH;
  }
}

// At least two waves per SIMD (8 waves per CU): with four-wave workgroups the
// bound asks for two workgroups, which keeps the compiler from trading
// occupancy for accumulator registers (AGPRs).
template <int D, int NW, int KB>
__global__ __launch_bounds__(64 * NW, 8 / NW)
void bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, const __bf16* __restrict__ rho,
                     const __bf16* __restrict__ do16, const f32x4* __restrict__ stats,
                     const float* __restrict__ gate, float* __restrict__ dk,
                     float* __restrict__ dv, int H, int L, int BH,
                     int n_kblk, float sl2, float scale) {
  static_assert(NW == 4 || NW == 8, "the launch bounds ask for 8 / NW workgroups per CU");
  constexpr int KSTEPS = D / 32;
  constexpr int FB = D / 16;
  constexpr int BK = 16 * KB * NW;                 // keys per workgroup
  constexpr int RM = BW_BQ * D;                    // elements of a row-major step tile
  constexpr int STAGE = 3 * RM + 64 * 8;           // + 64 stats records (1 KB)
  constexpr int RMBLK = RM * 2 / 1024;             // 1-KB blocks per tile
  static_assert(RMBLK % NW == 0, "tile blocks per wave");
  __shared__ __align__(16) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;
  int kblk, bh;                                         // lowest key blocks (most work) first
  bwd_grid_order<D == 64 ? PLX_BW_HEAD_GROUP_D64 : PLX_BW_HEAD_GROUP_D128>(
      (int)blockIdx.x, BH, n_kblk, &kblk, &bh);
  const int h = bh % H;
  const int k0 = kblk * BK;
  const int kw0 = k0 + 16 * KB * wave;
  const size_t head = (size_t)bh * L * D;
  const float ng = -gate[h];
  const float inv_scale = 1.0f / scale;

  // B-operand fragments of this wave's keys: key kw0 + 16 kb + c16, features
  // 32 kk + 8 g4 .. +7
  bf16x8 kf[KB][KSTEPS], vf[KB][KSTEPS];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = kw0 + 16 * kb + c16;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      if (key < L) {
        kf[kb][kk] = *reinterpret_cast<const bf16x8*>(k + head + (size_t)key * D + 32 * kk + 8 * g4);
        vf[kb][kk] = *reinterpret_cast<const bf16x8*>(v + head + (size_t)key * D + 32 * kk + 8 * g4);
      } else {
        kf[kb][kk] = bf16x8{};
        vf[kb][kk] = bf16x8{};
      }
    }
  }
  f32x4 dk_acc[KB][FB], dv_acc[KB][FB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      dk_acc[kb][fb] = f32x4{};
      dv_acc[kb][fb] = f32x4{};
    }
  }

  // per-lane byte offsets of this wave's 1-KB blocks (swizzle included)
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t rmoff[RMBLK / NW];
#pragma unroll
  for (int i = 0; i < RMBLK / NW; ++i) {
    // physical chunk pc of LDS row r holds logical chunk pc ^ rm_swz(r)
    const int e = (i * NW + wave) * 512 + 8 * lane;
    const int r = e / D, pc = (e % D) / 8;
    rmoff[i] = (uint32_t)((r * D + ((pc ^ rm_swz<D>(r)) << 3)) * 2);
  }
  const int n_qs = (L + BW_BQ - 1) / BW_BQ;
  const int qs0 = k0 / BW_BQ;
  auto load_stage = [&](int qs, int buf) {
    uint16_t* st = smem + buf * STAGE;
    const int q0 = qs * BW_BQ;
    const int rows = min(BW_BQ, L - q0);
    const size_t roff = head + (size_t)q0 * D;
    const __bf16* srcs[3] = {q + roff, rho + roff, do16 + roff};
#pragma unroll
    for (int m = 0; m < 3; ++m) {
#pragma unroll
      for (int i = 0; i < RMBLK / NW; ++i)
        buffer_load_lds16(srcs[m], rows * D * 2, st + m * RM + (i * NW + wave_u) * 512, rmoff[i]);
    }
    // statistics of rows q0 .. q0+63 (the second half is not used)
    if (wave_u == 0)
      buffer_load_lds16(stats + (size_t)bh * L + q0, (L - q0) * 16, st + 3 * RM,
                        (uint32_t)(16 * lane));
  };

  // MASK: the step holds a query before one of this wave's keys, or past L
  auto compute = [&](int qs, auto par, auto mask_c) {
    constexpr bool MASK = decltype(mask_c)::value;
    const uint16_t* st = smem + decltype(par)::value * STAGE;
    const uint16_t* Qs = st;
    const uint16_t* Rs = st + RM;
    const uint16_t* Os = st + 2 * RM;
    const f32x4* Ss = reinterpret_cast<const f32x4*>(st + 3 * RM);
    const int q0 = qs * BW_BQ;
    // S = Q K^T, R = rho K^T, Delta = dO V^T for 32 queries x 16*KB keys; lane
    // holds key kw0 + 16 kb + c16 and queries q0 + 16 qb + 4 g4 + j
    f32x4 sa[KB][2], ra[KB][2], da[KB][2];
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int off = rm_off<D>(c16, 4 * kk + g4) + 16 * qb * D;   // rm_swz repeats every 16 rows
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + off);
        const bf16x8 ar = *reinterpret_cast<const bf16x8*>(Rs + off);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(Os + off);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const f32x4 zs = kk == 0 ? f32x4{} : sa[kb][qb];
          const f32x4 zr = kk == 0 ? f32x4{} : ra[kb][qb];
          const f32x4 zd = kk == 0 ? f32x4{} : da[kb][qb];
          sa[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, kf[kb][kk], zs, 0, 0, 0);
          ra[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, kf[kb][kk], zr, 0, 0, 0);
          da[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, vf[kb][kk], zd, 0, 0, 0);
        }
      }
    }
    // W~, dS/scale, dR/scale in bf16 (dK = scale (Q^T dS/scale + rho^T dR/scale)):
    // element e = 4 qb + j of a key's 8 queries, the row order of tr_frag
    bf16x8 wtp[KB], dsp[KB], drp[KB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int qr = 16 * qb + 4 * g4 + j;
        const f32x4 sv = Ss[qr];
        const int qq = q0 + qr;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int key = kw0 + 16 * kb + c16;
          const bool keep = qq >= key && qq < L;
          const BwdElt el = bwd_elt<MASK>(keep, sa[kb][qb][j], ra[kb][qb][j], da[kb][qb][j], sv,
                                          ng, sl2);
          wtp[kb][4 * qb + j] = (__bf16)el.wt;
          dsp[kb][4 * qb + j] = (__bf16)el.ds;
          drp[kb][4 * qb + j] = (__bf16)(el.dr * inv_scale);
        }
      }
    }
    // dV^T += dO^T W~,  dK^T += Q^T dS' + rho^T dR
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      const bf16x8 ao = tr_frag<D>(Os, 0, 16 * fb, c16, g4);
      const bf16x8 aq = tr_frag<D>(Qs, 0, 16 * fb, c16, g4);
      const bf16x8 ar = tr_frag<D>(Rs, 0, 16 * fb, c16, g4);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        dv_acc[kb][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, wtp[kb], dv_acc[kb][fb], 0, 0, 0);
        dk_acc[kb][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, dsp[kb], dk_acc[kb][fb], 0, 0, 0);
        dk_acc[kb][fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ar, drp[kb], dk_acc[kb][fb], 0, 0, 0);
      }
    }
  };

  if (qs0 < n_qs) {
    load_stage(qs0, 0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  }
  // step qs reads buffer P = (qs - qs0) & 1, a compile-time parity
  auto step = [&](int qs, auto par) {
    constexpr int P = decltype(par)::value;
    // staging is unconditional: past the last step the loads re-read it into
    // the buffer no wave reads again
    load_stage(min(qs + 1, n_qs - 1), 1 - P);
    // a wave whose keys all follow the step's last query has nothing to add
    const int q0 = qs * BW_BQ;
    if (q0 + BW_BQ - 1 >= kw0) {
      if (q0 < kw0 + 16 * KB || q0 + BW_BQ > L) compute(qs, par, std::true_type{});
      else compute(qs, par, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  for (int qs = qs0; qs < n_qs; qs += 2) {
    step(qs, std::integral_constant<int, 0>{});
    if (qs + 1 < n_qs) step(qs + 1, std::integral_constant<int, 1>{});
  }

#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int key = kw0 + 16 * kb + c16;
    if (key < L) {
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        *reinterpret_cast<f32x4*>(dk + head + (size_t)key * D + 16 * fb + 4 * g4) =
            dk_acc[kb][fb] * scale;
        *reinterpret_cast<f32x4*>(dv + head + (size_t)key * D + 16 * fb + 4 * g4) = dv_acc[kb][fb];
      }
    }
  }
}

// ---------------------------------------------------- query-stationary dQ, drho
template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 1)
void bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                   const __bf16* __restrict__ v, const __bf16* __restrict__ rho,
                   const __bf16* __restrict__ do16, const __bf16* __restrict__ kT,
                   const f32x4* __restrict__ stats, const float* __restrict__ gate,
                   float* __restrict__ dq, float* __restrict__ drho, int H, int L, int BH,
                   int n_qt, float sl2, float scale) {
  constexpr int KSTEPS = D / 32;
  constexpr int FB = D / 16;
  constexpr int BR = 16 * NW;                      // queries per workgroup
  constexpr int TE = BW_T * D;                     // elements of one 64-key tile
  constexpr int STAGE = 3 * TE;                    // K, V (row-major) and K^T
  constexpr int TBLK = TE * 2 / 1024;
  static_assert(TBLK % NW == 0, "tile blocks per wave");
  __shared__ __align__(16) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;
  int qt, bh;                                           // longest rows first
  bwd_grid_order<D == 64 ? PLX_BW_HEAD_GROUP_D64 : PLX_BW_HEAD_GROUP_D128>(
      (int)blockIdx.x, BH, n_qt, &qt, &bh);
  qt = n_qt - 1 - qt;
  const int h = bh % H;
  const int q0 = qt * BR;
  const int qw0 = q0 + wave * 16;
  const int qi = qw0 + c16;
  const size_t head = (size_t)bh * L * D;
  const int n64 = (L + BW_T - 1) / BW_T;
  const float ng = -gate[h];

  bf16x8 qf[KSTEPS], rf[KSTEPS], df[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    if (qi < L) {
      const size_t o = head + (size_t)qi * D + 32 * kk + 8 * g4;
      qf[kk] = *reinterpret_cast<const bf16x8*>(q + o);
      rf[kk] = *reinterpret_cast<const bf16x8*>(rho + o);
      df[kk] = *reinterpret_cast<const bf16x8*>(do16 + o);
    } else {
      qf[kk] = bf16x8{};
      rf[kk] = bf16x8{};
      df[kk] = bf16x8{};
    }
  }
  const f32x4 sv = (qi < L) ? stats[(size_t)bh * L + qi] : f32x4{};
  f32x4 dq_acc[FB], dr_acc[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) {
    dq_acc[fb] = f32x4{};
    dr_acc[fb] = f32x4{};
  }

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t rmoff[TBLK / NW], troff[TBLK / NW];
#pragma unroll
  for (int i = 0; i < TBLK / NW; ++i) {
    const int e = (i * NW + wave) * 512 + 8 * lane;
    {
      const int r = e / D, pc = (e % D) / 8;
      rmoff[i] = (uint32_t)((r * D + ((pc ^ (r & (D / 8 - 1))) << 3)) * 2);
    }
    {
      const int f = e / BW_T, pc = (e % BW_T) / 8;
      troff[i] = (uint32_t)((f * BW_T + ((pc ^ (f & 7)) << 3)) * 2);
    }
  }
  const int last_q = min(q0 + BR, L) - 1;
  const int n_kt = last_q / BW_T + 1;
  const int n_w = (qw0 < L) ? min(qw0 + 15, L - 1) / BW_T + 1 : 0;
  auto load_stage = [&](int kt, int buf) {
    uint16_t* st = smem + buf * STAGE;
    const int rows = min(BW_T, L - kt * BW_T);
    const size_t roff = head + (size_t)kt * BW_T * D;
    const __bf16* srcs[2] = {k + roff, v + roff};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int i = 0; i < TBLK / NW; ++i)
        buffer_load_lds16(srcs[m], rows * D * 2, st + m * TE + (i * NW + wave_u) * 512, rmoff[i]);
    }
    const __bf16* kts = kT + ((size_t)bh * n64 + kt) * (size_t)(D * BW_T);
#pragma unroll
    for (int i = 0; i < TBLK / NW; ++i)
      buffer_load_lds16(kts, TE * 2, st + 2 * TE + (i * NW + wave_u) * 512, troff[i]);
  };

  auto compute = [&](int kt, auto par, auto diag_c) {
    const uint16_t* st = smem + decltype(par)::value * STAGE;
    const uint16_t* Ks = st;
    const uint16_t* Vs = st + TE;
    const uint16_t* KTs = st + 2 * TE;
    // S^T = K Q^T, R^T = K rho^T, Delta^T = V dO^T; lane holds query qi and
    // keys kt*64 + 16 kb + 4 g4 + j
    f32x4 sa[4], ra[4], da[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int off = rm_off_q<D>(16 * kb + c16, 4 * kk + g4);
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Ks + off);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(Vs + off);
        if (kk == 0) {
          sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qf[0], f32x4{}, 0, 0, 0);
          ra[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, rf[0], f32x4{}, 0, 0, 0);
          da[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, df[0], f32x4{}, 0, 0, 0);
        } else {
          sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, qf[kk], sa[kb], 0, 0, 0);
          ra[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, rf[kk], ra[kb], 0, 0, 0);
          da[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, df[kk], da[kb], 0, 0, 0);
        }
      }
    }
    const int lim = qi - kt * BW_T - 4 * g4;   // key offset 16 kb + j is causal iff <= lim
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bf16x8 dsp, drp;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int kb = 2 * t + hh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool keep = 16 * kb + j <= lim;
          const BwdElt el = bwd_elt<decltype(diag_c)::value>(keep, sa[kb][j], ra[kb][j], da[kb][j],
                                                             sv, ng, sl2);
          dsp[4 * hh + j] = (__bf16)el.ds;
          drp[4 * hh + j] = (__bf16)el.dr;
        }
      }
      // dQ^T += K^T (dS/scale)^T,  drho^T += K^T dR^T over the 32 keys of group t
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(KTs + tr_off64(16 * fb + c16, 4 * t + g4));
        dq_acc[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dsp, dq_acc[fb], 0, 0, 0);
        dr_acc[fb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, drp, dr_acc[fb], 0, 0, 0);
      }
    }
  };

  load_stage(0, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  // tile kt reads buffer kt & 1, a compile-time parity
  auto step = [&](int kt, auto par) {
    load_stage(min(kt + 1, n_kt - 1), 1 - decltype(par)::value);
    if (kt < n_w) {
      if (kt + 1 == n_w) compute(kt, par, std::true_type{});
      else compute(kt, par, std::false_type{});
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
  };
  for (int kt = 0; kt < n_kt; kt += 2) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < n_kt) step(kt + 1, std::integral_constant<int, 1>{});
  }

  if (qi < L) {
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      *reinterpret_cast<f32x4*>(dq + head + (size_t)qi * D + 16 * fb + 4 * g4) = dq_acc[fb] * scale;
      *reinterpret_cast<f32x4*>(drho + head + (size_t)qi * D + 16 * fb + 4 * g4) = dr_acc[fb];
    }
  }
}

// ------------------------------------------------------------------ launches
hipError_t launch_stage_t_bf16(const void* x, void* xt, int BH, int L, int d, hipStream_t s);

// Scratch layout of one backward call, in bytes from the workspace start.
hipError_t launch_stage_t_bf16(const void* x, void* xt, int BH, int L, int d, hipStream_t s);

struct BwdScratch {
  size_t do16, kT, stats, gpart, total;
};
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
BwdScratch bwd_scratch(int B, int H, int L, int d) {
  const size_t BH = (size_t)B * H;
  const size_t n64 = (size_t)((L + BW_T - 1) / BW_T);
  const size_t rm = align256(BH * L * d * 2);
  const size_t tr = align256(BH * n64 * BW_T * d * 2);
  BwdScratch w;
  w.do16 = 0;
  w.kT = w.do16 + rm;
  w.stats = w.kT + tr;
  w.gpart = w.stats + align256(BH * L * 16);
  w.total = w.gpart + align256(BH * n64 * 4);
  return w;
}

template <int D, int NW, int KB>
static void launch_dkdv_t(const void* q, const void* k, const void* v, const void* rho,
                          const void* do16, const void* stats, const float* gate, float* dk,
                          float* dv, int BH,
                          int H, int L, float sl2, float scale, hipStream_t s) {
  constexpr int BK = 16 * KB * NW;
  const int n_kblk = (L + BK - 1) / BK;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, KB>), dim3((unsigned)(BH * n_kblk)), dim3(64 * NW),
                     0, s, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (const __bf16*)rho, (const __bf16*)do16, (const f32x4*)stats, gate, dk, dv,
                     H, L, BH, n_kblk, sl2, scale);
}

template <int D, int NW>
static void launch_dq_t(const void* q, const void* k, const void* v, const void* rho,
                        const void* do16, const void* kT, const void* stats, const float* gate,
                        float* dq, float* drho, int BH, int H, int L, float sl2, float scale,
                        hipStream_t s) {
  const int n_qt = (L + 16 * NW - 1) / (16 * NW);
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)(BH * n_qt)), dim3(64 * NW), 0, s,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)rho,
                     (const __bf16*)do16, (const __bf16*)kT, (const f32x4*)stats, gate, dq, drho,
                     H, L, BH, n_qt, sl2, scale);
}

hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const void* rho,
                                   const float* gate, const float* out, const float* corr,
                                   const float* lse, const float* rbar, const float* dout,
                                   float* dq, float* dk, float* dv, float* drho, float* dgate,
                                   int B, int H, int L, int d, float scale, void* ws,
                                   hipStream_t s) {
  const int BH = B * H;
  const int n64 = (L + BW_T - 1) / BW_T;
  const BwdScratch w = bwd_scratch(B, H, L, d);
  char* base = static_cast<char*>(ws);
  void* do16 = base + w.do16;
  void* kT = base + w.kT;
  f32x4* stats = reinterpret_cast<f32x4*>(base + w.stats);
  float* gpart = reinterpret_cast<float*>(base + w.gpart);
  const float sl2 = scale * kLog2e;

  if (d == 128)
    hipLaunchKernelGGL(bwd_prep_kernel<128>, dim3((unsigned)(BH * n64)), dim3(256), 0, s, dout,
                       out, corr, lse, rbar, gate, (__bf16*)do16, stats, gpart, H, L, n64);
  else
    hipLaunchKernelGGL(bwd_prep_kernel<64>, dim3((unsigned)(BH * n64)), dim3(256), 0, s, dout,
                       out, corr, lse, rbar, gate, (__bf16*)do16, stats, gpart, H, L, n64);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // K^T tiles for the query-stationary kernel (the key-stationary one reads its
  // transposed operands straight from its row-major tiles)
  e = launch_stage_t_bf16(k, kT, BH, L, d, s);
  if (e != hipSuccess) return e;
  if (d == 128) {
    launch_dkdv_t<128, PLX_BW_KV_NW_D128, PLX_BW_KV_KB_D128>(q, k, v, rho, do16, stats, gate, dk,
                                                              dv, BH, H, L, sl2, scale, s);
    launch_dq_t<128, PLX_BW_Q_NW_D128>(q, k, v, rho, do16, kT, stats, gate, dq, drho, BH, H, L,
                                       sl2, scale, s);
  } else {
    launch_dkdv_t<64, PLX_BW_KV_NW_D64, PLX_BW_KV_KB_D64>(q, k, v, rho, do16, stats, gate, dk,
                                                          dv, BH, H, L, sl2, scale, s);
    launch_dq_t<64, PLX_BW_Q_NW_D64>(q, k, v, rho, do16, kT, stats, gate, dq, drho, BH, H, L,
                                     sl2, scale, s);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dgate_kernel, dim3((unsigned)H), dim3(64), 0, s, gpart, dgate, B, H,
                     n64);
  return hipGetLastError();
}

size_t bwd_workspace_bytes(int B, int H, int L, int d) { return bwd_scratch(B, H, L, d).total; }

}  // namespace plx
