// Causal Parallax prefill with fp32 inputs (vector ALU path, gfx950).
//
// Same operation as the bf16 kernel (page "Parallax - Parameterized Local Linear
// Attention for Language Modeling", section "Core mechanism", Eq. 2), computed
// entirely in fp32 on the vector units: this is the high-precision mode.
//
// A workgroup owns 64 queries of one head; each query is served by 4
// consecutive lanes, each holding a quarter of the features (float4 groups
// 16*j + 4*part).  Keys stream through LDS in tiles of 32; per tile the 4 lanes
// form the partial dot products <q,k_j> and <rho,k_j>, reduce them with DPP,
// update the online-softmax state once per tile, and accumulate sum p v and
// sum p r v for their features.  CORR = false compiles the covariance branch
// out: plain causal softmax attention on the same schedule.

#include "plx_common.h"

namespace plx {

constexpr int PF32_QB = 64;
constexpr int PF32_KB = 32;

template <int D, bool CORR>
__global__ __launch_bounds__(256)
void prefill_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                        const float* __restrict__ v, const float* __restrict__ rho,
                        const float* __restrict__ gate, float* __restrict__ out,
                        int H, int L, int BH, int n_qt, float sl2) {
  constexpr int NJ = D / 16;            // float4 groups per lane
  __shared__ __align__(16) float ks[PF32_KB * D];
  __shared__ __align__(16) float vs[PF32_KB * D];

  const int tid = threadIdx.x;
  const int part = tid & 3;
  const int qt = n_qt - 1 - (int)(blockIdx.x / (unsigned)BH);
  const int bh = (int)(blockIdx.x % (unsigned)BH);
  const int h = bh % H;
  const int q0 = qt * PF32_QB;
  const int qi = q0 + (tid >> 2);
  const size_t head = (size_t)bh * L * D;

  f32x4 qr[NJ], rr[NJ], A[NJ], Bv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (qi < L) {
      qr[j] = *reinterpret_cast<const f32x4*>(q + head + (size_t)qi * D + 16 * j + 4 * part);
      rr[j] = CORR ? *reinterpret_cast<const f32x4*>(rho + head + (size_t)qi * D + 16 * j + 4 * part)
                   : f32x4{};
    } else {
      qr[j] = f32x4{};
      rr[j] = f32x4{};
    }
    A[j] = f32x4{};
    Bv[j] = f32x4{};
  }
  float m_run = kMinit, l_run = 0.f, c_run = 0.f;

  const int last_q = min(q0 + PF32_QB, L) - 1;
  const int n_kt = last_q / PF32_KB + 1;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * PF32_KB;
    __syncthreads();
    for (int ch = tid; ch < PF32_KB * D / 4; ch += 256) {
      const int row = ch / (D / 4), col = (ch % (D / 4)) * 4;
      f32x4 kv = f32x4{}, vv = f32x4{};
      if (k0 + row < L) {
        kv = *reinterpret_cast<const f32x4*>(k + head + (size_t)(k0 + row) * D + col);
        vv = *reinterpret_cast<const f32x4*>(v + head + (size_t)(k0 + row) * D + col);
      }
      *reinterpret_cast<f32x4*>(ks + row * D + col) = kv;
      *reinterpret_cast<f32x4*>(vs + row * D + col) = vv;
    }
    __syncthreads();

    float s[PF32_KB], r[PF32_KB];
    float mx = kMinit;
#pragma unroll
    for (int j = 0; j < PF32_KB; ++j) {
      float sp = 0.f, rp = 0.f;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(ks + j * D + 16 * jj + 4 * part);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sp = fmaf(qr[jj][e], kv[e], sp);
          if constexpr (CORR) rp = fmaf(rr[jj][e], kv[e], rp);
        }
      }
      sp = group_sum<4>(sp);
      if constexpr (CORR) rp = group_sum<4>(rp);
      s[j] = (k0 + j <= qi) ? sp : -INFINITY;
      r[j] = rp;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx * sl2);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
    if constexpr (CORR) c_run *= alpha;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      A[jj] *= alpha;
      if constexpr (CORR) Bv[jj] *= alpha;
    }
#pragma unroll
    for (int j = 0; j < PF32_KB; ++j) {
      const float p = exp2f(fmaf(s[j], sl2, -m_new));
      const float t = p * r[j];
      l_run += p;
      if constexpr (CORR) c_run += t;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const f32x4 vv = *reinterpret_cast<const f32x4*>(vs + j * D + 16 * jj + 4 * part);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          A[jj][e] = fmaf(p, vv[e], A[jj][e]);
          if constexpr (CORR) Bv[jj][e] = fmaf(t, vv[e], Bv[jj][e]);
        }
      }
    }
  }

  if (qi < L) {
    const float inv = 1.0f / l_run;
    const float rbar = c_run * inv;
    const float gh = CORR ? gate[h] : 0.f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float osa = A[jj][e] * inv;
        if constexpr (CORR) {
          const float uu = Bv[jj][e] * inv;
          o[e] = osa - gh * (uu - osa * rbar);
        } else {
          o[e] = osa;
        }
      }
      *reinterpret_cast<f32x4*>(out + head + (size_t)qi * D + 16 * jj + 4 * part) = o;
    }
  }
}

template <int D, bool CORR>
static void launch_f32_t(const void* q, const void* k, const void* v, const void* rho,
                         const float* gate, float* out, int H, int L, int BH, int n_qt,
                         float sl2, hipStream_t s) {
  hipLaunchKernelGGL((prefill_f32_kernel<D, CORR>), dim3((unsigned)(BH * n_qt)), dim3(256), 0,
                     s, (const float*)q, (const float*)k, (const float*)v, (const float*)rho,
                     gate, out, H, L, BH, n_qt, sl2);
}

hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, const void* rho,
                              const float* gate, float* out, int B, int H, int L, int d,
                              float scale, bool corr, hipStream_t s) {
  const int BH = B * H;
  const int n_qt = (L + PF32_QB - 1) / PF32_QB;
  const float sl2 = scale * kLog2e;
  if (d == 128) {
    if (corr) launch_f32_t<128, true>(q, k, v, rho, gate, out, H, L, BH, n_qt, sl2, s);
    else launch_f32_t<128, false>(q, k, v, rho, gate, out, H, L, BH, n_qt, sl2, s);
  } else {
    if (corr) launch_f32_t<64, true>(q, k, v, rho, gate, out, H, L, BH, n_qt, sl2, s);
    else launch_f32_t<64, false>(q, k, v, rho, gate, out, H, L, BH, n_qt, sl2, s);
  }
  return hipGetLastError();
}

}  // namespace plx
