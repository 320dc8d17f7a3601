// Split-KV Parallax decode on gfx950.
//
// One query per (b,h) attends every cached key of its sequence (page "Parallax -
// Parameterized Local Linear Attention for Language Modeling", section "Core
// mechanism", Eq. 2).  Both branches, softmax and covariance, consume the same
// single pass over K and V (section "Hardware-aware algorithm"): the kernel is
// bound by HBM bandwidth, so the design goal is one coalesced read of every
// valid cache byte and nothing else.
//
// decode_split_kernel: grid (S, B*H), S = ceil(Lmax / C).  Workgroup s of a
//   stream covers keys [s*C, min((s+1)*C, L_b)) and exits at once when that range
//   is empty.  Inside a wave a key row is spread over LPR lanes, 16 bytes each,
//   so one load instruction covers KPW consecutive rows of contiguous memory.
//   Each lane keeps U row-loads of K and U of V in flight.  The partial dot
//   products <q,k> and <rho,k> of a row are summed across its lanes with DPP;
//   every lane group keeps its own online-softmax state (m, l, c) and the
//   accumulators sum p v and sum p r v for its features.  At the end the
//   groups of all four waves merge through LDS into one partial record.
// decode_combine_kernel: one workgroup per (b,h) merges the records of its
//   splits, rescaling by 2^(m_s - M), with the splits spread over the lanes of
//   the workgroup (butterfly reductions across lanes, then across waves), and
//   applies the output formula.
//
// CORR = false compiles the covariance branch out of both kernels (no rho
// reads, no <rho,k>, c or sum p r v; records of d+4 floats): plain softmax
// decode over the same stream, the baseline for the cost of the correction.

#include "plx_common.h"

namespace plx {

template <typename T, int D>
struct DecCfg {
  static constexpr int EPL = 16 / (int)sizeof(T);   // elements per lane per row load
  static constexpr int LPR = D / EPL;                // lanes per key row
  static constexpr int KPW = 64 / LPR;               // rows per wave load
  static constexpr int U = 16;                       // row loads in flight per lane
  static constexpr int CHUNK = KPW * U;              // keys per wave iteration
  static constexpr int NG = 4 * KPW;                 // lane groups per workgroup
};

// floats per split record: m, l, c, pad, sum p v [D] and, with the correction, sum p r v [D]
template <int D, bool CORR>
constexpr int rec_floats() { return (CORR ? 2 * D : D) + 4; }

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

template <typename T, int D, bool CORR>
__global__ __launch_bounds__(256)
void decode_split_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                         const T* __restrict__ vc, const T* __restrict__ rho,
                         const int* __restrict__ seqlens, float* __restrict__ part,
                         int H, int Lmax, int C, int S, float sl2) {
  using CF = DecCfg<T, D>;
  constexpr int EPL = CF::EPL, LPR = CF::LPR, KPW = CF::KPW, U = CF::U, NG = CF::NG;
  __shared__ float s_m[NG], s_l[NG], s_c[NG];
  constexpr int RF = rec_floats<D, CORR>();
  __shared__ float s_a[NG][D], s_b[CORR ? NG : 1][D];

  const int s = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / H;
  const int Lb = min(max(seqlens[b], 0), Lmax);
  const int k_begin = s * C;
  if (k_begin >= Lb) return;                    // uniform over the workgroup
  const int k_end = min(k_begin + C, Lb);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = lane / LPR;
  const int sub = lane % LPR;
  const size_t head = (size_t)bh * Lmax * D;

  // this lane's slice of q and rho: features sub*EPL .. +EPL-1
  const u32x4 qw = *reinterpret_cast<const u32x4*>(q + (size_t)bh * D + sub * EPL);
  u32x4 rw = u32x4{0u, 0u, 0u, 0u};
  if constexpr (CORR) rw = *reinterpret_cast<const u32x4*>(rho + (size_t)bh * D + sub * EPL);

  float A[EPL], Bv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) { A[e] = 0.f; Bv[e] = 0.f; }
  float m_run = kMinit, l_run = 0.f, c_run = 0.f;

  const T* kb = kc + head + sub * EPL;
  const T* vb = vc + head + sub * EPL;

  for (int c0 = k_begin + wave * CF::CHUNK; c0 < k_end; c0 += 4 * CF::CHUNK) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = c0 + u * KPW + grp;
      if (key < k_end) {
        // streamed once: non-temporal loads keep the cache stream out of L2
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (size_t)key * D));
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (size_t)key * D));
      } else {
        kr[u] = u32x4{0u, 0u, 0u, 0u};
        vr[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float sv[U], rv[U];
    float mx = kMinit;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float sp = 0.f, rp = 0.f;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          sp = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw[w]), as_bf16x2(kr[u][w]), sp, false);
          if constexpr (CORR)
            rp = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(rw[w]), as_bf16x2(kr[u][w]), rp, false);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float kx = __uint_as_float(kr[u][w]);
          sp = fmaf(__uint_as_float(qw[w]), kx, sp);
          if constexpr (CORR) rp = fmaf(__uint_as_float(rw[w]), kx, rp);
        }
      }
      sp = group_sum<LPR>(sp);
      if constexpr (CORR) rp = group_sum<LPR>(rp);
      const int key = c0 + u * KPW + grp;
      sv[u] = (key < k_end) ? sp : -INFINITY;
      rv[u] = rp;
      mx = fmaxf(mx, sv[u]);
    }
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if constexpr (CORR) c_run *= alpha;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      A[e] *= alpha;
      if constexpr (CORR) Bv[e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sv[u], sl2, -m_new));
      const float t = p * rv[u];
      l_run += p;
      if constexpr (CORR) c_run += t;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float v0 = bf16lo_to_f32(vr[u][w]);
          const float v1 = bf16hi_to_f32(vr[u][w]);
          A[2 * w] = fmaf(p, v0, A[2 * w]);
          A[2 * w + 1] = fmaf(p, v1, A[2 * w + 1]);
          if constexpr (CORR) {
            Bv[2 * w] = fmaf(t, v0, Bv[2 * w]);
            Bv[2 * w + 1] = fmaf(t, v1, Bv[2 * w + 1]);
          }
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float vx = __uint_as_float(vr[u][w]);
          A[w] = fmaf(p, vx, A[w]);
          if constexpr (CORR) Bv[w] = fmaf(t, vx, Bv[w]);
        }
      }
    }
  }

  // merge the lane groups of all waves
  const int gi = wave * KPW + grp;
  if (sub == 0) {
    s_m[gi] = m_run;
    s_l[gi] = l_run;
    s_c[gi] = c_run;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    s_a[gi][sub * EPL + e] = A[e];
    if constexpr (CORR) s_b[gi][sub * EPL + e] = Bv[e];
  }
  __syncthreads();
  float M = kMinit;
#pragma unroll
  for (int i = 0; i < NG; ++i) M = fmaxf(M, s_m[i]);
  float* rec = part + ((size_t)bh * S + s) * RF;
  for (int t = tid; t < RF - 4; t += 256) {
    const int f = t % D;
    float acc = 0.f;
    if (t < D) {
#pragma unroll
      for (int i = 0; i < NG; ++i) acc += __builtin_amdgcn_exp2f(s_m[i] - M) * s_a[i][f];
    } else if constexpr (CORR) {
#pragma unroll
      for (int i = 0; i < NG; ++i) acc += __builtin_amdgcn_exp2f(s_m[i] - M) * s_b[i][f];
    }
    rec[4 + t] = acc;
  }
  if (tid == 0) {
    float lt = 0.f, ct = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const float w = __builtin_amdgcn_exp2f(s_m[i] - M);
      lt += w * s_l[i];
      ct += w * s_c[i];
    }
    rec[0] = M;
    rec[1] = lt;
    rec[2] = ct;
    rec[3] = 0.f;
  }
}

// Merge of (m, l, c) triples in the base-2 log domain: both sides rescaled to
// the larger running max.
struct Mlc {
  float m, l, c;
};
__device__ __forceinline__ Mlc mlc_merge(Mlc a, Mlc b) {
  const float M = fmaxf(a.m, b.m);
  const float wa = __builtin_amdgcn_exp2f(a.m - M), wb = __builtin_amdgcn_exp2f(b.m - M);
  return Mlc{M, a.l * wa + b.l * wb, a.c * wa + b.c * wb};
}
__device__ __forceinline__ Mlc mlc_xor(Mlc x, int mask) {
  return Mlc{__shfl_xor(x.m, mask), __shfl_xor(x.l, mask), __shfl_xor(x.c, mask)};
}

// Merge the split records of one (b,h) and write o = o_sa - g (u - o_sa rbar)
// (o = o_sa without the correction).  One workgroup of 256 threads per stream,
// splits spread over lanes:
//   1. every thread folds the (m, l, c) of splits tid, tid+256, ... into one
//      triple, and the triples of the workgroup meet in a butterfly across the
//      64 lanes of each wave and then across the 4 waves (LDS): the stream's
//      max M, l and c;
//   2. the 2D (D without the correction) feature sums are split into float4
//      columns; NSG groups of threads take every NSG-th split, so each thread
//      issues all its 16-byte record loads at once (unrolled) and accumulates
//      2^(m_s - M) times them;
//   3. the groups' column sums meet in LDS, in a fixed order.
// The merge order is fixed, so results are deterministic.
template <int D, bool CORR>
__global__ __launch_bounds__(256)
void decode_combine_kernel(const float* __restrict__ part, const float* __restrict__ gate,
                           const int* __restrict__ seqlens, float* __restrict__ out,
                           int H, int Lmax, int C, int S) {
  constexpr int RF = rec_floats<D, CORR>();
  constexpr int NF = RF - 4;                 // feature floats per record
  // float4 columns of the correction's record layout, used by both variants so
  // that the softmax-only twin sums sum p v in the same order (its columns past
  // NF / 4 stay idle): a zero probe then gives bit-identical outputs
  constexpr int NC = (2 * D) / 4;
  constexpr int NSG = 256 / NC;              // split groups
  static_assert(NC * NSG == 256, "columns x groups must cover the workgroup");
  __shared__ Mlc s_w[4];
  __shared__ f32x4 s_acc[NSG][NC];

  const int bh = blockIdx.x;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int Lb = min(max(seqlens[b], 0), Lmax);
  const int ns = (Lb + C - 1) / C;
  float* o = out + (size_t)bh * D;
  if (ns == 0) {                              // uniform over the workgroup
    if (tid < D) o[tid] = 0.f;
    return;
  }
  const float* rec = part + (size_t)bh * S * RF;

  // Thread (group sg, column cc) sums splits sg, sg + NSG, ... of feature
  // column cc, UNR at a time, in split order.  Its first UNR splits are loaded
  // before the stream's (M, l, c) is known, so that both rounds of record loads
  // are in flight together.
  const int cc = tid % NC, sg = tid / NC;
  const bool col = cc < NF / 4;
  constexpr int UNR = 8;
  f32x4 v[UNR];
  float w[UNR];
  auto load = [&](int s0) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int sp = s0 + u * NSG;
      if (col && sp < ns) {
        const float* r = rec + (size_t)sp * RF;
        w[u] = r[0];
        v[u] = *reinterpret_cast<const f32x4*>(r + 4 + 4 * cc);
      } else {
        w[u] = -INFINITY;
        v[u] = f32x4{};
      }
    }
  };
  load(sg);

  // 1. (M, l, c) of the stream
  Mlc t{kMinit, 0.f, 0.f};
  for (int sp = tid; sp < ns; sp += 256) {
    const f32x4 hd = *reinterpret_cast<const f32x4*>(rec + (size_t)sp * RF);
    t = mlc_merge(t, Mlc{hd[0], hd[1], CORR ? hd[2] : 0.f});
  }
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) t = mlc_merge(t, mlc_xor(t, mask));
  if (lane == 0) s_w[wave] = t;
  __syncthreads();
  const Mlc tot = mlc_merge(mlc_merge(s_w[0], s_w[1]), mlc_merge(s_w[2], s_w[3]));
  const float M = tot.m;

  // 2. weighted feature sums
  f32x4 acc = {};
  for (int s0 = sg;;) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) acc += __builtin_amdgcn_exp2f(w[u] - M) * v[u];
    s0 += UNR * NSG;
    if (!col || s0 >= ns) break;
    load(s0);
  }
  s_acc[sg][cc] = acc;
  __syncthreads();

  // 3. column sums over the groups, then the output formula
  if (tid < D) {
    const int f = tid;
    float a = 0.f, bv = 0.f;
#pragma unroll
    for (int g = 0; g < NSG; ++g) {
      a += s_acc[g][f >> 2][f & 3];
      if constexpr (CORR) bv += s_acc[g][(D + f) >> 2][(D + f) & 3];
    }
    const float inv = 1.0f / tot.l;
    const float osa = a * inv;
    if constexpr (CORR) {
      const float uu = bv * inv;
      o[f] = osa - gate[h] * (uu - osa * (tot.c * inv));
    } else {
      o[f] = osa;
    }
  }
}

template <typename T, int D, bool CORR>
static hipError_t launch_split_t(const void* q, const void* kc, const void* vc,
                                 const void* rho, const int* seqlens, float* part, int B,
                                 int H, int Lmax, int C, float sl2, hipStream_t s) {
  const int S = (Lmax + C - 1) / C;
  hipLaunchKernelGGL((decode_split_kernel<T, D, CORR>), dim3((unsigned)S, (unsigned)(B * H)),
                     dim3(256), 0, s, (const T*)q, (const T*)kc, (const T*)vc,
                     (const T*)rho, seqlens, part, H, Lmax, C, S, sl2);
  return hipGetLastError();
}

template <bool CORR>
static hipError_t launch_split_c(const void* q, const void* kc, const void* vc, const void* rho,
                                 const int* seqlens, float* part, int B, int H, int Lmax, int d,
                                 int C, float sl2, bool bf16, hipStream_t s) {
  if (bf16) {
    if (d == 128)
      return launch_split_t<__bf16, 128, CORR>(q, kc, vc, rho, seqlens, part, B, H, Lmax, C, sl2, s);
    return launch_split_t<__bf16, 64, CORR>(q, kc, vc, rho, seqlens, part, B, H, Lmax, C, sl2, s);
  }
  if (d == 128)
    return launch_split_t<float, 128, CORR>(q, kc, vc, rho, seqlens, part, B, H, Lmax, C, sl2, s);
  return launch_split_t<float, 64, CORR>(q, kc, vc, rho, seqlens, part, B, H, Lmax, C, sl2, s);
}

hipError_t launch_decode_split(const void* q, const void* kc, const void* vc, const void* rho,
                               const int* seqlens, float* part, int B, int H, int Lmax, int d,
                               int C, float scale, bool bf16, bool corr, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  if (corr) return launch_split_c<true>(q, kc, vc, rho, seqlens, part, B, H, Lmax, d, C, sl2, bf16, s);
  return launch_split_c<false>(q, kc, vc, rho, seqlens, part, B, H, Lmax, d, C, sl2, bf16, s);
}

template <int D, bool CORR>
static void launch_combine_t(const float* part, const float* gate, const int* seqlens,
                             float* out, int B, int H, int Lmax, int C, int S, hipStream_t s) {
  hipLaunchKernelGGL((decode_combine_kernel<D, CORR>), dim3((unsigned)(B * H)), dim3(256), 0, s,
                     part, gate, seqlens, out, H, Lmax, C, S);
}

hipError_t launch_decode_combine(const float* part, const float* gate, const int* seqlens,
                                 float* out, int B, int H, int Lmax, int d, int C, bool corr,
                                 hipStream_t s) {
  const int S = (Lmax + C - 1) / C;
  if (d == 128) {
    if (corr) launch_combine_t<128, true>(part, gate, seqlens, out, B, H, Lmax, C, S, s);
    else launch_combine_t<128, false>(part, gate, seqlens, out, B, H, Lmax, C, S, s);
  } else {
    if (corr) launch_combine_t<64, true>(part, gate, seqlens, out, B, H, Lmax, C, S, s);
    else launch_combine_t<64, false>(part, gate, seqlens, out, B, H, Lmax, C, S, s);
  }
  return hipGetLastError();
}

}  // namespace plx
