// Causal Parallax prefill in bf16 on CDNA4 matrix cores (gfx950).
//
// Computes, for every query i of every (b,h) head (page "Parallax - Parameterized
// Local Linear Attention for Language Modeling", section "Core mechanism", Eq. 2):
//     o_i = o^SA_i - g_h ( sum_j w_ij r_ij v_j - o^SA_i sum_j w_ij r_ij ),   j <= i
// with w_ij the causal softmax weights of scale <q_i,k_j> and r_ij = <rho_i,k_j>,
// in one streaming pass over the keys shared by both branches (section
// "Hardware-aware algorithm").
//
// Work decomposition
//   * A workgroup owns 16*NW consecutive queries of one head (NW waves x 16 rows)
//     and walks the causal key range in tiles of 64 keys.  Every K tile (bf16)
//     and V^T tile (fp16, pre-staged by stage_v) is copied from HBM to LDS once
//     per workgroup by buffer loads that write LDS directly, double-buffered,
//     and read by all waves.
//   * Each wave computes the transposed score blocks S^T = K Q^T and R^T = K rho^T
//     with v_mfma_f32_16x16x32_bf16, 16 keys x 16 queries per block.  One K
//     fragment read from LDS feeds both MFMAs (the joint QK / RK product).  Q
//     and rho fragments stay in registers.
//   * In the transposed layout a lane owns one query and 4 keys per block, so
//     the online-softmax row max is lane-local except for two exchanges across
//     the four lanes that share a query.
//   * P = exp2(S*scale*log2e - m) and R are rounded to fp16 (RNE) and T = P*R is
//     formed from the rounded values by packed fp16 multiplies (half the vector
//     instructions of an fp32 product followed by a conversion).  P and T are fed,
//     as B operands, to v_mfma_f32_16x16x32_f16 against the V^T fragment:
//     O^T += V^T P^T and A_r^T += V^T T^T, fp32 accumulators in registers.  The
//     row sums l = sum P and c = sum T come from the same rounded values, by one
//     more MFMA each against an all-ones A block (every row of that product holds
//     the per-query sums), so a single key reproduces v exactly and the vector
//     ALU, the scarcer resource here, is spared 16 instructions per tile.
//   * stage_v stores the keys of every 32-key group of V^T in the order in which
//     the score accumulators of a lane group come out of two consecutive 16-key
//     blocks, so P and T go from the score MFMA output straight into the value
//     MFMA input without any data movement.
//   * The running max moves lazily: only when some row's tile max exceeds it by
//     more than kRescaleSlack (log2 units), which makes the rescale of the
//     accumulators rare after the first tile.
//   * R has no bound (rho is an input).  The tile walk converts it to fp16
//     unchecked; a row whose R or T overflowed fp16 ends with a non-finite c, and
//     its wave then walks its keys once more with a per-tile range check that
//     scales the row's R by a power of two (exact: Eq. 2 is linear in rho).
//   * The register footprint stays within 256 per lane so that two waves share
//     each SIMD and one wave's MFMAs overlap the other's softmax arithmetic.
//   * Grid order: the longest (last) query tiles of every head first; heads
//     cycle fastest so that the 8 XCDs each receive a fixed subset of heads.

#include <type_traits>

#include "plx_common.h"

namespace plx {

constexpr int PF_BC = 64;       // keys per tile
// s_waitcnt immediate for "lgkmcnt(0)" with vmcnt and expcnt left unconstrained
constexpr int kWaitLgkm0 = 0xC07F;
// waves per workgroup (16 queries each), per head dimension
#ifndef PLX_PF_NW_D128
#define PLX_PF_NW_D128 4
#endif
#ifndef PLX_PF_NW_D64
#define PLX_PF_NW_D64 8
#endif
// software-pipelined schedule (next tile's scores overlap this tile's softmax)
#ifndef PLX_PF_PIPE_D128
#define PLX_PF_PIPE_D128 1
#endif
#ifndef PLX_PF_PIPE_D64
#define PLX_PF_PIPE_D64 0
#endif
// minimum waves per SIMD the register allocation must allow, per head dimension
#ifndef PLX_PF_MINW_D128
#define PLX_PF_MINW_D128 2
#endif
#ifndef PLX_PF_MINW_D64
#define PLX_PF_MINW_D64 4
#endif
// Prefill grid order, per head dimension: 0 = the query tiles of all heads
// longest first with heads fastest; G > 0 = the same within groups of G heads,
// group after group.  Groups put more query tiles of fewer heads on each XCD at
// once, so a K/V tile fetched into its L2 serves more workgroups: HBM reads of
// the B4 H16 L4096 d128 launch drop from 1.22 GB to 0.53 GB (G = 32) and 0.35 GB
// (G = 16).  Measured: d = 64 gains 2.6-2.9 % with G = 16; d = 128 loses 0-3 %
// with either, so it keeps the plain order.
#ifndef PLX_PF_HEAD_GROUP_D128
#define PLX_PF_HEAD_GROUP_D128 0
#endif
#ifndef PLX_PF_HEAD_GROUP_D64
#define PLX_PF_HEAD_GROUP_D64 16
#endif
// Chunked prefill on a staged V cache whose chunks fit one query tile (no
// workgroup re-reads a K/V tile): K and V tiles are loaded with the
// non-temporal cache policy (1), like decode's stream, or with the default one
// (0).  Measured on 16-query chunks over 8192 cached keys: -8 to -12 %; with
// 512-query chunks, whose 8 query tiles share each K/V tile through L2, it cost
// +13 %.
#ifndef PLX_CHUNK_NT
#define PLX_CHUNK_NT 1
#endif
// Per-call chunked prefill at d = 128 with at most 64 queries per chunk (one
// query tile): convert the raw V tiles in the kernel (1) instead of a staging
// pass (0).
#ifndef PLX_CHUNK_FUSEV
#define PLX_CHUNK_FUSEV 1
#endif
// The same three choices for the softmax-only variant (correction compiled out),
// tuned on their own: without R, T and their accumulators the d=128 kernel
// needs 104 VGPRs un-pipelined, so two 8-wave workgroups share a CU (four waves
// per SIMD), which beats the pipelined 4-wave shape by about 20%.
#ifndef PLX_SM_NW_D128
#define PLX_SM_NW_D128 8
#endif
#ifndef PLX_SM_NW_D64
#define PLX_SM_NW_D64 PLX_PF_NW_D64
#endif
#ifndef PLX_SM_PIPE_D128
#define PLX_SM_PIPE_D128 0
#endif
#ifndef PLX_SM_PIPE_D64
#define PLX_SM_PIPE_D64 PLX_PF_PIPE_D64
#endif
#ifndef PLX_SM_MINW_D128
#define PLX_SM_MINW_D128 PLX_PF_MINW_D128
#endif
#ifndef PLX_SM_MINW_D64
#define PLX_SM_MINW_D64 PLX_PF_MINW_D64
#endif
// Rescale slack in log2 units: P = 2^(s - m) may grow to 2^kRescaleSlack before
// the running max m is moved, so fp16 P <= 16.
constexpr float kRescaleSlack = 4.0f;
// Largest |R| a row may feed to the fp16 products in the checked pass: with
// P <= 16, T = P*R stays below 2^15, inside fp16's range.  A row whose R exceeds
// it is scaled by a power of two (exactly; Eq. 2 is linear in rho), see rescale_r.
constexpr float kRMax = 2048.0f;
static_assert(16.0f * kRMax < 65504.0f, "T = P*R must fit fp16");

// LDS tiles have no padding; 16-byte chunks are XOR-swizzled by row instead,
// which keeps every fragment read and tile store free of bank conflicts
// (measured on gfx950: a conflict-free ds_read_b128 occupies the LDS for 8
// cycles, and twice as long with a 16-byte row padding).
template <int D>
struct PfLayout {
  static constexpr int KCHUNKS = D / 8;        // 16-byte chunks per K row
  static constexpr int K_ELEMS = PF_BC * D;    // bf16 elements per K tile
  static constexpr int V_ELEMS = D * PF_BC;    // fp16 elements per V^T tile
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  // element offset of logical 16-byte chunk c of K row r / V^T row r
  static __device__ __forceinline__ int k_off(int r, int c) {
    return r * D + ((c ^ (r & (KCHUNKS - 1))) << 3);
  }
  static __device__ __forceinline__ int v_off(int r, int c) {
    return r * PF_BC + ((c ^ (r & 7)) << 3);
  }
};

// V goes to the fp16 value products through this: fp16 holds |v| <= 65504
// exactly (bf16 values up to 65280), and larger magnitudes, which fp16 cannot
// represent, are clamped to +-65504 instead of becoming infinite, so that a key
// a row never attends (a masked key in its diagonal tile, P = 0) cannot turn
// the row into NaN through 0 * inf.  NaN stays NaN.
__device__ __forceinline__ _Float16 v_to_f16(float x) {
  return (_Float16)(fabsf(x) > 65504.0f ? __builtin_copysignf(65504.0f, x) : x);
}

// Key stored at position p of a 32-key group of a staged V^T tile.  Position
// 8*g + 4*h + j holds key 16*h + 4*g + j: lane group g of a 16x16 score block
// owns keys 4g..4g+3 of each block, and two consecutive blocks h = 0, 1 form
// the 32-key step of the value MFMA.
__host__ __device__ constexpr int vt_key_of_pos(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}

// Chunked prefill against a KV cache: sequence b owns token rows
// cu_q[b] .. cu_q[b+1]-1 of q, rho and out ([T, H, D], token-major) and puts
// them at cache positions ctx[b] + j; its keys are cache rows 0 .. ctx[b]+n_b-1
// of K [B, H, Lmax, D] and of the staged V^T.  The device clamps every length so
// that no access leaves q (T rows) or the cache (Lmax rows).
struct ChunkArgs {
  const int* cu_q;
  const int* ctx;
  int T;        // rows of q, rho and out
  int Lmax;     // cache rows per (b, h)
  int max_q;    // largest chunk: the grid covers ceil(max_q / queries per workgroup)
  int n64max;   // staged V^T tiles per (b, h): ceil(Lmax / 64)
  int new_rows_only;   // staging: only the tiles that hold cache rows >= ctx[b]
  // split-KV chunked prefill: split s of every query tile covers key tiles
  // s*split_tiles .. (s+1)*split_tiles - 1; its partial records go to part
  // ([T*H][n_split][2D+4] floats, row index token*H + head)
  int split_tiles;
  int n_split;
  float* part;
};
// (first row, queries, position of query 0) of sequence b, clamped
__device__ __forceinline__ void chunk_geometry(const ChunkArgs& ca, int b, int* c0, int* n_q,
                                               int* pos0) {
  const int a = min(max(ca.cu_q[b], 0), ca.T);
  const int e = min(max(ca.cu_q[b + 1], a), ca.T);
  *c0 = a;
  *n_q = min(e - a, min(ca.max_q, ca.Lmax));
  *pos0 = min(max(ca.ctx[b], 0), ca.Lmax - *n_q);
}

// Second launch bound: at least two waves per SIMD, which caps the register
// budget at 256 per lane and keeps every MFMA operand in VGPRs.
// CORR = false compiles the covariance branch out (no R, T, A_r or c): plain
// causal softmax attention through the same staging, tiling and schedule, the
// baseline for the cost of the correction.  SAVE = true (training) also writes
// what the backward pass needs: the natural-log partition function of every
// row, rbar = c / l and the correction vector (u - o_sa rbar).  VARLEN = true
// is the chunked prefill (ChunkArgs): the same tile loop with the causal mask
// offset by the chunk's cache position.  SPLIT (with VARLEN) walks only the key
// tiles of one split and writes the unnormalised state of every row (m, l, c,
// sum p v, sum p r v) to ca.part for chunk_combine_kernel.  NT loads the K and
// V tiles with the non-temporal cache policy.  FUSEV > 0 (chunks of at most
// 16 * FUSEV queries, so only waves 0 .. FUSEV-1 have queries; plain schedule)
// reads V straight from the bf16 cache: each raw tile is staged in LDS like K,
// and the remaining waves convert it to the fp16 V^T tile layout (the layout
// stage_v writes, the same values) while the busy waves compute its scores.
template <int D, int NW, bool PIPE, bool CORR, bool SAVE, bool VARLEN, bool SPLIT, bool NT,
          int FUSEV>
__global__ __launch_bounds__(64 * NW, CORR ? (D == 64 ? PLX_PF_MINW_D64 : PLX_PF_MINW_D128)
                                          : (D == 64 ? PLX_SM_MINW_D64 : PLX_SM_MINW_D128))
void prefill_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                         const _Float16* __restrict__ vt, const __bf16* __restrict__ rho,
                         const float* __restrict__ gate, float* __restrict__ out,
                         float* __restrict__ lse_out, float* __restrict__ rbar_out,
                         float* __restrict__ corr_out, int H, int L, int BH, int n_qt,
                         float sl2, ChunkArgs ca) {
  static_assert(CORR || !SAVE, "the training statistics belong to the Parallax kernel");
  static_assert(!(SAVE && VARLEN), "the training statistics are for whole sequences");
  static_assert(!SPLIT || (VARLEN && CORR), "key splits are for the chunked prefill");
  static_assert(FUSEV == 0 || (VARLEN && !PIPE &&
                               (FUSEV == NW ? 64 * NW >= 2 * (D / 8) * (PF_BC / 8)
                                            : 64 * (NW - FUSEV) >= (D / 8) * (PF_BC / 8))),
                "fused V conversion: chunks, plain schedule, a converting thread per block "
                "(per half block when every wave is busy)");
  using LY = PfLayout<D>;
  constexpr int PF_BR = 16 * NW;                         // queries per workgroup
  constexpr int PF_THREADS = 64 * NW;
  constexpr int KSTEPS = D / 32;                         // MFMA steps over features
  constexpr int FB = D / 16;                             // 16-feature output blocks

  // FUSEV: K and raw V double-buffered, one V^T tile
  constexpr int SMEM = FUSEV > 0 ? 4 * LY::K_ELEMS + LY::V_ELEMS : 2 * LY::STAGE;
  __shared__ __align__(16) uint16_t smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c16 = lane & 15;
  const int g4 = lane >> 4;

  // heads in groups of G: each group's query tiles run longest first, heads
  // fastest, before the next group's (a partial last group has BH mod G heads)
  constexpr int G = D == 64 ? PLX_PF_HEAD_GROUP_D64 : PLX_PF_HEAD_GROUP_D128;
  int qt, bh;
  if constexpr (!VARLEN && G > 0) {
    const int full = BH / G;
    const int b = (int)blockIdx.x;
    const int g = b / (G * n_qt);
    const int gs = g < full ? G : BH - full * G;
    const int r = b - g * G * n_qt;
    qt = n_qt - 1 - r / gs;
    bh = g * G + r % gs;
  } else {
    qt = n_qt - 1 - (int)(blockIdx.x / (unsigned)BH);
    bh = (int)(blockIdx.x % (unsigned)BH);
  }
  int sp = 0;                                    // key split (SPLIT)
  if constexpr (SPLIT) {
    const int rest = (int)(blockIdx.x / (unsigned)BH);
    qt = n_qt - 1 - rest % n_qt;
    sp = rest / n_qt;
  }
  const int h = bh % H;
  const int q0 = qt * PF_BR;
  const int qw0 = q0 + wave * 16;
  const int qi = qw0 + c16;
  const size_t head = (size_t)bh * L * D;
  const int n_kt_all = (L + PF_BC - 1) / PF_BC;

  // Geometry of this head.  Prefill: L queries at positions 0 .. L-1 against
  // the same L keys.  Chunk: n_q queries at positions pos0 + j against the first
  // pos0 + n_q cache keys, rows token-major (stride H*D).
  int n_q = L, pos0 = 0;
  size_t qbase = head, qstride = D;
  const __bf16* kh = k + head;
  const _Float16* vth = vt + (size_t)bh * n_kt_all * (D * PF_BC);
  int c0 = 0;
  if constexpr (VARLEN) {
    chunk_geometry(ca, bh / H, &c0, &n_q, &pos0);
    if (q0 >= n_q) return;                       // uniform over the workgroup
    qbase = ((size_t)c0 * H + h) * D;
    qstride = (size_t)H * D;
    kh = k + (size_t)bh * ca.Lmax * D;
    // staged V^T tiles; FUSEV > 0: the raw bf16 cache rows of this head, like K
    vth = FUSEV > 0 ? vt + (size_t)bh * ca.Lmax * D : vt + (size_t)bh * ca.n64max * (D * PF_BC);
  }
  const int n_k = pos0 + n_q;

  // B-operand fragments: query qi, features 32*kk + 8*g4 .. +7
  bf16x8 qf[KSTEPS], rf[KSTEPS];
  if (qi < n_q) {
    const bf16x8* qp = reinterpret_cast<const bf16x8*>(q + qbase + (size_t)qi * qstride);
    const bf16x8* rp = CORR ? reinterpret_cast<const bf16x8*>(rho + qbase + (size_t)qi * qstride)
                            : nullptr;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qf[kk] = qp[4 * kk + g4];
      if constexpr (CORR) rf[kk] = rp[4 * kk + g4];
      else rf[kk] = bf16x8{};
    }
  } else {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      qf[kk] = bf16x8{};
      rf[kk] = bf16x8{};
    }
  }

  f32x4 acc_o[FB], acc_r[FB];
#pragma unroll
  for (int fb = 0; fb < FB; ++fb) {
    acc_o[fb] = f32x4{};
    acc_r[fb] = f32x4{};
  }
  float m_run = kMinit;
  // The row's R enters the fp16 products as R * 2^-r_exp (r_exp = 0 until some
  // |R| of the row exceeds kRMax); acc_r and c carry the same factor, removed in
  // the epilogue.  The four lanes of a query hold the same value.
  float r_exp = 0.f;
  // l = sum_j P_ij and c = sum_j T_ij, accumulated on the matrix cores: the
  // product of an all-ones 16x32 block with P^T (or T^T) holds the per-query
  // sums in every row, so each lane's four values are copies of its query's.
  f32x4 acc_l = {}, acc_c = {};
  f16x8 ones8;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones8[e] = (_Float16)1.0f;

  const int last_pos = pos0 + min(q0 + PF_BR, n_q) - 1;
  const int n_kt = last_pos / PF_BC + 1;
  // Key tiles this workgroup walks: 0 .. n_kt-1, or with SPLIT those of split
  // sp.  A split that starts past n_kt holds no key of these queries (and no
  // combine reads its records).
  int t_beg = 0, t_end = n_kt;
  if constexpr (SPLIT) {
    t_beg = sp * ca.split_tiles;
    if (t_beg >= n_kt) return;                   // uniform over the workgroup
    t_end = min(n_kt, t_beg + ca.split_tiles);
  }
  const int wave_last_pos = pos0 + min(qw0 + 15, n_q - 1);

  // Tiles move HBM -> LDS with buffer_load_dwordx4 ... lds: each lane's 16
  // bytes land at (wave-uniform base) + 16 * lane, so one wave instruction
  // fills 1 KB of LDS; the lane's offset into the tile picks which logical
  // chunk goes there, which implements the XOR swizzle without touching
  // registers.  The per-lane byte offsets of this wave's 1-KB blocks (swizzle
  // included) are the same for every tile: computed once, one 32-bit register
  // each.  Each load takes a scalar buffer descriptor based at the tile and
  // sized to the bytes that exist, so K rows past L come back as zeros from
  // the hardware range check (they only meet masked, future keys).
  constexpr int KBLK = LY::K_ELEMS * 2 / 1024;   // 1-KB blocks per K tile
  constexpr int VBLK = LY::V_ELEMS * 2 / 1024;   // 1-KB blocks per V^T tile
  static_assert(KBLK % NW == 0 && VBLK % NW == 0, "tile blocks per wave");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t koff[KBLK / NW], voff[VBLK / NW];
#pragma unroll
  for (int i = 0; i < KBLK / NW; ++i) {
    const int e = (i * NW + wave) * 512 + 8 * lane;   // element offset in the tile
    const int r = e / D, pc = (e % D) / 8;
    koff[i] = (uint32_t)((r * D + ((pc ^ (r & (LY::KCHUNKS - 1))) << 3)) * 2);
  }
#pragma unroll
  for (int i = 0; i < VBLK / NW; ++i) {
    const int e = (i * NW + wave) * 512 + 8 * lane;
    const int r = e / PF_BC, pc = (e % PF_BC) / 8;
    voff[i] = (uint32_t)((r * PF_BC + ((pc ^ (r & 7)) << 3)) * 2);
  }
  // cache policy of the K / V tile loads: non-temporal for chunks (streamed)
  constexpr int kTileAux = NT ? 2 : 0;
  auto tile_load16 = [&](const void* base, int bytes, void* lds, uint32_t voff) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(base), (short)0, bytes, kBufferRsrcWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds, 16, voff, 0, 0, kTileAux);
  };
  const char* kbase = reinterpret_cast<const char*>(kh);
  // blocks [i0, i1) of this wave's share of a K tile
  auto load_k = [&](int kt, int buf, auto i0, auto i1) {
    const int rows = min(PF_BC, n_k - kt * PF_BC);
    const char* tile = kbase + (size_t)kt * PF_BC * D * 2;
#pragma unroll
    for (int i = decltype(i0)::value; i < decltype(i1)::value; ++i)
      tile_load16(tile, rows * D * 2, smem + buf * LY::K_ELEMS + (i * NW + wave_u) * 512, koff[i]);
  };
  const char* vbase = reinterpret_cast<const char*>(vth);
  auto load_v = [&](int kt, int buf) {
    if constexpr (FUSEV > 0) {
      // raw bf16 rows of the cache, laid out like K
      const int rows = min(PF_BC, n_k - kt * PF_BC);
      const char* tile = vbase + (size_t)kt * PF_BC * D * 2;
#pragma unroll
      for (int i = 0; i < KBLK / NW; ++i)
        tile_load16(tile, rows * D * 2,
                    smem + 2 * LY::K_ELEMS + buf * LY::K_ELEMS + (i * NW + wave_u) * 512, koff[i]);
      return;
    }
    const char* tile = vbase + (size_t)kt * (D * PF_BC) * 2;
#pragma unroll
    for (int i = 0; i < VBLK / NW; ++i)
      tile_load16(tile, D * PF_BC * 2,
                  smem + 2 * LY::K_ELEMS + buf * LY::V_ELEMS + (i * NW + wave_u) * 512, voff[i]);
  };
  // this wave's tile loads have landed in LDS (then a barrier publishes them)
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); };
  // S^T = K Q^T and R^T = K rho^T of one tile; lane holds keys 16*kb + 4*g4 + j.
  // kfrag(kb, kk): the K fragment of key 16*kb + c16, features 32*kk + 8*g4 .. +7.
  // The checked pass after the tile walk reads its fragments through this; the
  // walk keeps its own copy with the LDS reads written out (`scores`), because
  // routing them through the fragment functor changed the register allocation
  // of the kernels that run at 250-256 VGPRs and made some of them spill.
  auto scores_of = [&](auto kfrag, f32x4 (&sa)[4], f32x4 (&ra)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 a[KSTEPS];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) a[kk] = kfrag(kb, kk);
      sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], qf[0], f32x4{}, 0, 0, 0);
      if constexpr (CORR)
        ra[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], rf[0], f32x4{}, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk) {
        sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], qf[kk], sa[kb], 0, 0, 0);
        if constexpr (CORR)
          ra[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], rf[kk], ra[kb], 0, 0, 0);
      }
    }
  };
  // the same with K tile `buf` in LDS
  auto scores = [&](auto buf, f32x4 (&sa)[4], f32x4 (&ra)[4]) {
    const uint16_t* ks = smem + (int)buf * LY::K_ELEMS;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 a[KSTEPS];
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk)
        a[kk] = *reinterpret_cast<const bf16x8*>(ks + LY::k_off(16 * kb + c16, 4 * kk + g4));
      sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], qf[0], f32x4{}, 0, 0, 0);
      if constexpr (CORR)
        ra[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], rf[0], f32x4{}, 0, 0, 0);
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk) {
        sa[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], qf[kk], sa[kb], 0, 0, 0);
        if constexpr (CORR)
          ra[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kk], rf[kk], ra[kb], 0, 0, 0);
      }
    }
  };

  // tiles this wave computes: 0 .. n_w-1 (a row always sees key 0 of tile 0);
  // a tile needs the causal mask when its last key follows the wave's first
  // query (for a whole-sequence prefill, only the wave's last tile)
  const int n_w = (qw0 < n_q) ? wave_last_pos / PF_BC + 1 : 0;
  const int w_end = SPLIT ? min(n_w, t_end) : n_w;   // this wave computes tiles t_beg .. w_end-1
  auto needs_mask = [&](int t) { return t * PF_BC + PF_BC - 1 > pos0 + qw0; };

  // K and V tiles are double-buffered.  Pipelined schedule: K runs one tile
  // ahead of V; in iteration kt the waves read K of tile kt+1 and V of tile kt
  // while K of tile kt+2 and V of tile kt+1 are written into the buffers read in
  // iteration kt-1.  Plain schedule: iteration kt reads K and V of tile kt and
  // writes tile kt+1 into the other buffers.
  using KAll0 = std::integral_constant<int, 0>;
  using KHalf = std::integral_constant<int, KBLK / NW / 2>;
  using KAll1 = std::integral_constant<int, KBLK / NW>;
  load_k(t_beg, 0, KAll0{}, KAll1{});
  load_v(t_beg, 0);
  if (PIPE && t_end - t_beg > 1) load_k(t_beg + 1, 1, KAll0{}, KAll1{});
  wait_loads();
  __syncthreads();

  f32x4 sc[4], rc[4];     // scores of the tile being finished

  // Rare path of the R range check: some row of the wave has |R| > kRMax in the
  // tile whose R is `ra`.  Each such row takes the smallest power of two that
  // brings its largest |R| to at most kRMax and applies it, exactly, to what
  // the fp16 products of its later tiles see (its rho fragments), to this
  // tile's R and to the r-weighted sums gathered so far (acc_r, acc_c).
  auto rescale_r = [&](f32x4 (&ra)[4], float rm) {
    // keeps this path behind its branch: without the barrier the compiler
    // speculates it into every tile with a factor of one
    asm volatile("" ::: "memory");
    float rr = lane_xor16(rm, Max{});
    rr = lane_xor32(rr, Max{});
    // rr in [2^e, 2^(e+1)) with e >= 11: scaling by 2^-(e-10) lands in [2^10, 2^11)
    const int de = rr > kRMax ? __builtin_amdgcn_frexp_expf(rr) - 11 : 0;
    const float f = __builtin_ldexpf(1.0f, -de);
    r_exp += (float)de;
    acc_c *= f;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) acc_r[fb] *= f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) ra[kb] *= f;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) rf[kk][e] = (__bf16)((float)rf[kk][e] * f);
    }
  };
  // The tile walk checks |R| per tile only with the in-kernel V conversion
  // (FUSEV); the other kernels check each row once, after the walk (below).
  using kHotCheck = std::integral_constant<bool, (FUSEV > 0)>;
  using kLanes = std::true_type;    // tile_max: the lane's own maximum
  using kRows = std::false_type;    // tile_max: the row maximum (lanes exchanged)
  // Causal mask (the wave's last tile is its only diagonal tile) and the scaled
  // row max of one tile's scores; the four lanes that share a query combine.
  // With the correction, masked keys also get R = 0 (they never reach a row's
  // sums: neither their |R| nor an fp16 overflow of it may touch the row).  In
  // the checked walk (`chk`) the tile's |R| is held to kRMax before its fp16
  // conversion.
  // (With `lanes`, the lane's own maximum, scaled, without the exchange.)
  auto tile_max = [&](f32x4 (&sa)[4], f32x4 (&ra)[4], int kt_, auto diag_c,
                      auto chk, auto lanes) -> float {
    if constexpr (decltype(diag_c)::value) {
      const int lim = pos0 + qi - kt_ * PF_BC - 4 * g4;   // key offset 16*kb + j kept iff <= lim
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (16 * kb + j > lim) {
            sa[kb][j] = -INFINITY;
            if constexpr (CORR) ra[kb][j] = 0.f;
          }
        }
      }
    }
    float mx = kMinit;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sa[kb][j]);
    }
    if constexpr (CORR && decltype(chk)::value) {
      float rm = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) rm = fmaxf(rm, fabsf(ra[kb][j]));
      }
      if (__any(rm > kRMax)) rescale_r(ra, rm);
    }
    if constexpr (!decltype(lanes)::value) {
      mx = lane_xor16(mx, Max{});
      mx = lane_xor32(mx, Max{});
    }
    return mx * sl2;
  };
  // The lazy rescale of a tile from its lanes' own (scaled) maxima, before the
  // exchange between the four lanes of a query: a row's maximum passes the
  // running max by more than the slack exactly when one of its lanes' does, so
  // the exchange (two lane swaps) is needed only when a rescale is due.
  auto rescale_lanes = [&](float m_lane) {
    if (__any(m_lane > m_run + kRescaleSlack)) {
      float mx = lane_xor16(m_lane, Max{});
      mx = lane_xor32(mx, Max{});
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      acc_l *= alpha;
      if constexpr (CORR) acc_c *= alpha;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        acc_o[fb] *= alpha;
        if constexpr (CORR) acc_r[fb] *= alpha;
      }
    }
  };
  // Lazy rescale: the running max only moves when some row's tile max exceeds
  // it by more than the slack, so P stays below 2^slack.
  auto rescale_to = [&](float m_tile) {
    if (__any(m_tile > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      acc_l *= alpha;
      if constexpr (CORR) acc_c *= alpha;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        acc_o[fb] *= alpha;
        if constexpr (CORR) acc_r[fb] *= alpha;
      }
    }
  };
  // P = 2^(S*scale*log2e - m) and T = P*R in fp16, their row sums, and the
  // value products O^T += V^T P^T, A_r^T += V^T T^T of one tile.
  // vfrag(fb, t): the V^T fragment of feature 16*fb + c16, positions 8*(4t + g4) .. +7.
  // (For the checked pass; the walk's copy, `softmax_pv`, reads LDS directly, as
  // `scores` does.)
  auto softmax_pv_of = [&](auto vfrag, f32x4 (&sa)[4], f32x4 (&ra)[4]) {
    const float m_use = m_run;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f16x8 pf, rf, tf;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pf[4 * hh + j] =
              (_Float16)__builtin_amdgcn_exp2f(fmaf(sa[2 * t + hh][j], sl2, -m_use));
          if constexpr (CORR) rf[4 * hh + j] = (_Float16)ra[2 * t + hh][j];
        }
      }
      if constexpr (CORR) tf = pf * rf;
      acc_l = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, pf, acc_l, 0, 0, 0);
      if constexpr (CORR)
        acc_c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, tf, acc_c, 0, 0, 0);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        const f16x8 va = vfrag(fb, t);
        acc_o[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, acc_o[fb], 0, 0, 0);
        if constexpr (CORR)
          acc_r[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, tf, acc_r[fb], 0, 0, 0);
      }
    }
  };
  // the same with V^T tile `vbuf` in LDS
  auto softmax_pv = [&](auto vbuf, f32x4 (&sa)[4], f32x4 (&ra)[4]) {
    const float m_use = m_run;
    const uint16_t* vs = FUSEV > 0 ? smem + 4 * LY::K_ELEMS
                               : smem + 2 * LY::K_ELEMS + (int)vbuf * LY::V_ELEMS;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f16x8 pf, rf, tf;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pf[4 * hh + j] =
              (_Float16)__builtin_amdgcn_exp2f(fmaf(sa[2 * t + hh][j], sl2, -m_use));
          if constexpr (CORR) rf[4 * hh + j] = (_Float16)ra[2 * t + hh][j];
        }
      }
      if constexpr (CORR) tf = pf * rf;
      acc_l = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, pf, acc_l, 0, 0, 0);
      if constexpr (CORR)
        acc_c = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones8, tf, acc_c, 0, 0, 0);
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        const f16x8 va =
            *reinterpret_cast<const f16x8*>(vs + LY::v_off(16 * fb + c16, 4 * t + g4));
        acc_o[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pf, acc_o[fb], 0, 0, 0);
        if constexpr (CORR)
          acc_r[fb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, tf, acc_r[fb], 0, 0, 0);
      }
    }
  };
  // FUSEV: raw V tile `buf` (bf16, K's layout) -> the fp16 V^T tile, in 8 x 8
  // blocks: features 8 fc .. 8 fc + 7 (one 16-byte chunk of each raw row) of
  // the keys vt_key_of_pos(8c .. 8c+7) that chunk c of the V^T rows holds.
  // 16-byte LDS reads, a transpose in registers, bf16 -> fp32 -> fp16 (RNE) as
  // stage_v converts, 16- (or 8-) byte LDS writes.  The waves past the busy
  // ones take a block per thread; when every wave is busy, all threads take
  // half a block (4 of the 8 keys) each.
  auto convert_v = [&](int buf) {
    constexpr bool ALL = FUSEV == NW;
    constexpr int KP = ALL ? 4 : 8;                      // keys per thread
    typedef _Float16 f16xkp __attribute__((ext_vector_type(KP)));
    const uint16_t* raw = smem + 2 * LY::K_ELEMS + buf * LY::K_ELEMS;
    uint16_t* vtl = smem + 4 * LY::K_ELEMS;
    const int item = ALL ? tid >> 1 : tid - 64 * FUSEV;
    const int e0 = ALL ? 4 * (tid & 1) : 0;
    if (item >= (D / 8) * (PF_BC / 8)) return;
    const int c = item & 7, fc = item >> 3;
    u32x4 in[KP];
#pragma unroll
    for (int e = 0; e < KP; ++e)
      in[e] = *reinterpret_cast<const u32x4*>(raw + LY::k_off(vt_key_of_pos(8 * c + e0 + e), fc));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16xkp o;
#pragma unroll
      for (int e = 0; e < KP; ++e) {
        const uint32_t w = in[e][j >> 1];
        o[e] = v_to_f16(__uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16)));
      }
      *reinterpret_cast<f16xkp*>(vtl + LY::v_off(8 * fc + j, c) + e0) = o;
    }
  };
  // Pipelined step: the score MFMAs of tile kt_+1, the softmax and value MFMAs
  // of tile kt_, then the mask and max of tile kt_+1 form one basic block, so
  // the scheduler can overlap MFMA work with the softmax arithmetic and with
  // the latency of the cross-lane max.  Returns the scaled max of tile kt_+1.
  // `par` is the parity of kt_: it names the buffers at compile time, and the
  // loop below alternates the two score register sets instead of copying.
  auto pipe_step = [&](int kt_, auto par, auto diag_next, f32x4 (&cs)[4], f32x4 (&cr)[4],
                       f32x4 (&ns)[4], f32x4 (&nr)[4]) -> float {
    constexpr int P = decltype(par)::value;
    scores(std::integral_constant<int, 1 - P>{}, ns, nr);
    // The second half of the K tile two steps ahead and the V tile of the next
    // step are staged here rather than at the top of the iteration: the wave's
    // vector-memory issue then overlaps its score MFMAs instead of delaying them.
    load_k(min(kt_ + 2, t_end - 1), P, KHalf{}, KAll1{});
    load_v(min(kt_ + 1, t_end - 1), 1 - P);
    softmax_pv(par, cs, cr);
    return tile_max(ns, nr, kt_ + 1, diag_next, kHotCheck{}, kLanes{});
  };

  f32x4 sn[4], rn[4];     // the other score register set of the pipelined loop
  if constexpr (PIPE) {
    if (w_end > t_beg) {
      scores(std::integral_constant<int, 0>{}, sc, rc);
      m_run = needs_mask(t_beg) ? tile_max(sc, rc, t_beg, std::true_type{}, kHotCheck{}, kRows{})
                                : tile_max(sc, rc, t_beg, std::false_type{}, kHotCheck{}, kRows{});
    }
    // iteration 0 overwrites K buffer 0: every wave must be done reading it
    __syncthreads();
  }

  // One iteration of the tile loop; kt has parity P.
  auto iteration = [&](int kt, auto par, f32x4 (&cs)[4], f32x4 (&cr)[4], f32x4 (&ns)[4],
                       f32x4 (&nr)[4]) {
    constexpr int P = decltype(par)::value;
    // Staging is unconditional: past the last tile the loads re-read tile
    // n_kt-1 into buffers no wave reads again.
    const int k_ahead = PIPE ? kt + 2 : kt + 1;
    const bool in_step = PIPE && kt + 1 < w_end;   // pipe_step stages the rest itself
    if (in_step) {
      load_k(min(k_ahead, t_end - 1), P, KAll0{}, KHalf{});
    } else {
      load_k(min(k_ahead, t_end - 1), PIPE ? P : 1 - P, KAll0{}, KAll1{});
      load_v(min(kt + 1, t_end - 1), 1 - P);
    }
    if (kt < w_end) {
      if constexpr (PIPE) {
        if (kt + 1 < w_end) {
          const float m_next =
              needs_mask(kt + 1) ? pipe_step(kt, par, std::true_type{}, cs, cr, ns, nr)
                                 : pipe_step(kt, par, std::false_type{}, cs, cr, ns, nr);
          rescale_lanes(m_next);
        } else {
          softmax_pv(par, cs, cr);
        }
      } else if constexpr (FUSEV == 0) {
        scores(par, cs, cr);
        // (the first tile always rescales: from m_run = kMinit to the row
        // maxima, with zero accumulators)
        rescale_lanes(needs_mask(kt) ? tile_max(cs, cr, kt, std::true_type{}, kHotCheck{}, kLanes{})
                                     : tile_max(cs, cr, kt, std::false_type{}, kHotCheck{}, kLanes{}));
        softmax_pv(par, cs, cr);
      }
    }
    if constexpr (FUSEV > 0) {
      // the busy waves: the scores of tile kt; the other waves: its V^T tile
      // (every wave busy: each converts its share first, then its scores)
      if constexpr (FUSEV == NW) convert_v(P);
      if (wave_u < FUSEV) {
        if (kt < w_end) {
          scores(par, cs, cr);
          const float m_tile =
              needs_mask(kt) ? tile_max(cs, cr, kt, std::true_type{}, kHotCheck{}, kRows{})
                             : tile_max(cs, cr, kt, std::false_type{}, kHotCheck{}, kRows{});
          if (kt == t_beg) m_run = m_tile;      // accumulators are still zero
          rescale_to(m_tile);
        }
      } else if constexpr (FUSEV < NW) {
        convert_v(P);
      }
      // V^T complete: this wave's LDS writes are done (lgkmcnt); a bare barrier,
      // since __syncthreads() would also wait for the loads of tile kt+1
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (kt < w_end) softmax_pv(par, cs, cr);
    }
    wait_loads();
    __syncthreads();
  };
  for (int kt = t_beg; kt < t_end; kt += 2) {
    iteration(kt, std::integral_constant<int, 0>{}, sc, rc, sn, rn);
    if (kt + 1 < t_end) iteration(kt + 1, std::integral_constant<int, 1>{}, sn, rn, sc, rc);
  }

  // Without FUSEV the walk above holds no |R| check.  fp16 carries R and T = P*R
  // with the same relative precision at any magnitude it can represent; past its
  // range R or T becomes infinite, and then the row's c (the sum of its T on the
  // matrix cores) can only end as +-inf or NaN.  A wave with such a row walks its
  // key tiles again, with the check, reading K and V^T straight from memory (its
  // own pass, no LDS and no barrier): the check scales a row's R by a power of two
  // before it can overflow, exactly, since Eq. 2 is linear in rho.
  if constexpr (CORR && FUSEV == 0) {
    if (__any(!__builtin_isfinite(acc_c[0]))) {
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        acc_o[fb] = f32x4{};
        acc_r[fb] = f32x4{};
      }
      acc_l = f32x4{};
      acc_c = f32x4{};
      m_run = kMinit;
      r_exp = 0.f;
      for (int kt = t_beg; kt < w_end; ++kt) {
        // key rows past the end read as zeros, as the tile loads give them
        scores_of([&](int kb, int kk) {
          const int row = kt * PF_BC + 16 * kb + c16;
          return row < n_k ? *reinterpret_cast<const bf16x8*>(kh + (size_t)row * D + 32 * kk + 8 * g4)
                           : bf16x8{};
        }, sc, rc);
        const float m_tile =
            needs_mask(kt) ? tile_max(sc, rc, kt, std::true_type{}, std::true_type{}, kRows{})
                           : tile_max(sc, rc, kt, std::false_type{}, std::true_type{}, kRows{});
        if (kt == t_beg) m_run = m_tile;          // accumulators are still zero
        rescale_to(m_tile);
        softmax_pv_of([&](int fb, int t) {
          // staged V^T tile kt: [D][64] fp16, unswizzled in memory
          return *reinterpret_cast<const f16x8*>(vth + (size_t)kt * (D * PF_BC) +
                                                 (size_t)(16 * fb + c16) * PF_BC + 8 * (4 * t + g4));
        }, sc, rc);
      }
    }
  }

  // epilogue: o = o_sa - g (u - o_sa * rbar), o_sa = O/l, u = A_r/l, rbar = c/l
  // (A_r and c times 2^r_exp: the row's R scale comes off here)
  const float l_tot = acc_l[0];
  const float c_tot = acc_c[0];
  if constexpr (SPLIT) {
    // the split's unnormalised state, relative to 2^m_run, with c and sum p r v
    // relative to 2^-r_exp; a row whose keys all precede this split leaves a
    // record no combine reads
    if (qi < n_q) {
      constexpr int RF = 2 * D + 4;
      float* rec = ca.part + (((size_t)(c0 + qi) * H + h) * ca.n_split + sp) * RF;
#pragma unroll
      for (int fb = 0; fb < FB; ++fb) {
        *reinterpret_cast<f32x4*>(rec + 4 + 16 * fb + 4 * g4) = acc_o[fb];
        *reinterpret_cast<f32x4*>(rec + 4 + D + 16 * fb + 4 * g4) = acc_r[fb];
      }
      if (g4 == 0) *reinterpret_cast<f32x4*>(rec) = f32x4{m_run, l_tot, c_tot, r_exp};
    }
    return;
  }
  if (qi < n_q) {
    const float inv = 1.0f / l_tot;
    const float inv_r = CORR ? __builtin_ldexpf(inv, (int)r_exp) : inv;
    const float rbar = c_tot * inv_r;
    const float gh = CORR ? gate[h] : 0.f;
    float* orow = out + qbase + (size_t)qi * qstride;
#pragma unroll
    for (int fb = 0; fb < FB; ++fb) {
      f32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float osa = acc_o[fb][j] * inv;
        if constexpr (CORR) {
          const float uu = acc_r[fb][j] * inv_r;
          o[j] = osa - gh * (uu - osa * rbar);
        } else {
          o[j] = osa;
        }
      }
      *reinterpret_cast<f32x4*>(orow + 16 * fb + 4 * g4) = o;
      if constexpr (SAVE) {
        f32x4 cv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float osa = acc_o[fb][j] * inv;
          cv[j] = acc_r[fb][j] * inv_r - osa * rbar;
        }
        *reinterpret_cast<f32x4*>(corr_out + head + (size_t)qi * D + 16 * fb + 4 * g4) = cv;
      }
    }
    if constexpr (SAVE) {
      // l sums 2^(s*scale*log2e - m) over the row, so log2 of the partition
      // function is m + log2(l); the four lanes of a query hold the same values
      if (g4 == 0) {
        lse_out[(size_t)bh * L + qi] = (m_run + __log2f(l_tot)) * kLn2;
        rbar_out[(size_t)bh * L + qi] = rbar;
      }
    }
  }
}

// X [BH, L, D] bf16 -> X^T tiles [BH][ceil(L/64)][D][64] of TOUT (fp16 for the
// forward's V^T, bf16 for the backward's transposed operands), zero past L, with
// the rows of each 32-row group in vt_key_of_pos order.
// One workgroup per (head, 64-row tile): coalesced 16-B loads into LDS, then
// each thread gathers 8 rows of one feature, converts and stores 16 B.
// VARLEN: v is the cache [B, H, L = Lmax, D]; only the tiles holding keys
// 0 .. ctx[b] + n_b - 1 of each head are written (the ones the chunk reads).
template <int D, typename TOUT, bool VARLEN = false>
__global__ __launch_bounds__(256)
void stage_v_kernel(const __bf16* __restrict__ v, TOUT* __restrict__ vt, int L, int n_kt,
                    ChunkArgs ca = {}, int H = 1, int span = 0) {
  typedef TOUT outx8 __attribute__((ext_vector_type(8)));
  constexpr int PITCH = D + 2;     // odd dword pitch spreads the column reads over banks
  __shared__ uint16_t tile[PF_BC * PITCH];
  // workgroups per head: every tile, or (new rows only) the `span` tiles from
  // the one holding the chunk's first row
  const int per = (VARLEN && ca.new_rows_only) ? span : n_kt;
  const int bh = blockIdx.x / per;
  int kt = blockIdx.x % per;
  const int tid = threadIdx.x;
  int n_valid = L;                      // rows of this head that exist
  if constexpr (VARLEN) {
    int c0, n_q, pos0;
    chunk_geometry(ca, bh / H, &c0, &n_q, &pos0);
    n_valid = pos0 + n_q;
    if (ca.new_rows_only) kt += pos0 / PF_BC;
    if (kt * PF_BC >= n_valid) return;  // uniform over the workgroup
  }
  const __bf16* src = v + ((size_t)bh * L + (size_t)kt * PF_BC) * D;
  constexpr int CH = PF_BC * D / 8;
  constexpr int PER = CH / 256;         // 16-byte chunks per thread
  // all global loads in flight before the first LDS store
  u32x4 w[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + 256 * i;
    const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
    w[i] = (kt * PF_BC + row < n_valid)
               ? *reinterpret_cast<const u32x4*>(src + (size_t)row * D + col)
               : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int ch = tid + 256 * i;
    const int row = ch / (D / 8), col = (ch % (D / 8)) * 8;
    uint32_t* dst = reinterpret_cast<uint32_t*>(tile + row * PITCH + col);
    dst[0] = w[i][0]; dst[1] = w[i][1]; dst[2] = w[i][2]; dst[3] = w[i][3];
  }
  __syncthreads();
  TOUT* dst = vt + ((size_t)bh * n_kt + kt) * (size_t)(D * PF_BC);
  for (int ch = tid; ch < CH; ch += 256) {
    const int f = ch / (PF_BC / 8), key0 = (ch % (PF_BC / 8)) * 8;
    outx8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = vt_key_of_pos(key0 + e);
      const float x = __uint_as_float((uint32_t)tile[key * PITCH + f] << 16);
      if constexpr (std::is_same<TOUT, _Float16>::value) o[e] = v_to_f16(x);
      else o[e] = (TOUT)x;
    }
    *reinterpret_cast<outx8*>(dst + (size_t)ch * 8) = o;
  }
}

template <typename TOUT>
static hipError_t launch_stage_t(const void* v, void* vt, int BH, int L, int d, hipStream_t s) {
  const int n_kt = (L + PF_BC - 1) / PF_BC;
  const dim3 grid((unsigned)(BH * n_kt));
  if (d == 128)
    hipLaunchKernelGGL((stage_v_kernel<128, TOUT>), grid, dim3(256), 0, s, (const __bf16*)v,
                       (TOUT*)vt, L, n_kt);
  else
    hipLaunchKernelGGL((stage_v_kernel<64, TOUT>), grid, dim3(256), 0, s, (const __bf16*)v,
                       (TOUT*)vt, L, n_kt);
  return hipGetLastError();
}

hipError_t launch_stage_v(const void* v, void* vt, int BH, int L, int d, hipStream_t s) {
  return launch_stage_t<_Float16>(v, vt, BH, L, d, s);
}

hipError_t launch_stage_t_bf16(const void* x, void* xt, int BH, int L, int d, hipStream_t s) {
  return launch_stage_t<__bf16>(x, xt, BH, L, d, s);
}

// Pointers a training forward writes besides the output (all null otherwise).
struct TrainOut {
  float* lse;
  float* rbar;
  float* corr;
};

template <int D, int NW, bool PIPE, bool CORR, bool SAVE = false, bool VARLEN = false,
          bool SPLIT = false, bool NT = false, int FUSEV = 0>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* vt,
                                   const void* rho, const float* gate, float* out, int B,
                                   int H, int L, float sl2, hipStream_t s, TrainOut tr = {},
                                   ChunkArgs ca = {}) {
  const int BH = B * H;
  const int n_qt = ((VARLEN ? ca.max_q : L) + 16 * NW - 1) / (16 * NW);
  const unsigned n_blocks = (unsigned)BH * (unsigned)n_qt * (SPLIT ? (unsigned)ca.n_split : 1u);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, PIPE, CORR, SAVE, VARLEN, SPLIT, NT, FUSEV>),
                     dim3(n_blocks), dim3(64 * NW), 0, s, (const __bf16*)q,
                     (const __bf16*)k, (const _Float16*)vt, (const __bf16*)rho, gate, out, tr.lse,
                     tr.rbar, tr.corr, H, L, BH, n_qt, sl2, ca);
  return hipGetLastError();
}

template <bool CORR>
static hipError_t launch_prefill_c(const void* q, const void* k, const void* vt, const void* rho,
                                   const float* gate, float* out, int B, int H, int L, int d,
                                   float sl2, hipStream_t s) {
  constexpr int nw128 = CORR ? PLX_PF_NW_D128 : PLX_SM_NW_D128;
  constexpr int nw64 = CORR ? PLX_PF_NW_D64 : PLX_SM_NW_D64;
  constexpr bool pipe128 = CORR ? (PLX_PF_PIPE_D128 != 0) : (PLX_SM_PIPE_D128 != 0);
  constexpr bool pipe64 = CORR ? (PLX_PF_PIPE_D64 != 0) : (PLX_SM_PIPE_D64 != 0);
  if (d == 128)
    return launch_prefill_t<128, nw128, pipe128, CORR>(q, k, vt, rho, gate, out, B, H, L, sl2, s);
  return launch_prefill_t<64, nw64, pipe64, CORR>(q, k, vt, rho, gate, out, B, H, L, sl2, s);
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* vt, const void* rho,
                               const float* gate, float* out, int B, int H, int L, int d,
                               float scale, bool corr, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  if (corr) return launch_prefill_c<true>(q, k, vt, rho, gate, out, B, H, L, d, sl2, s);
  return launch_prefill_c<false>(q, k, vt, rho, gate, out, B, H, L, d, sl2, s);
}

// V^T tiles of the cache rows the chunks read (all of them, or with
// new_rows_only only the tiles holding rows ctx[b] .. ctx[b]+n_b-1); rows at or
// past ctx[b]+n_b of a written tile are zero.
hipError_t launch_stage_v_rows(const void* vc, void* vt, const int* cu_q, const int* ctx, int B,
                               int H, int T, int Lmax, int max_q, int d, bool new_rows_only,
                               hipStream_t s) {
  const int n64 = (Lmax + PF_BC - 1) / PF_BC;
  const ChunkArgs ca{cu_q, ctx, T, Lmax, max_q, n64, new_rows_only ? 1 : 0};
  // new rows only: a chunk of n <= min(max_q, Lmax) rows spans at most
  // floor((n + 62) / 64) + 1 tiles, so the grid covers only those of each head
  const int mq = min(max_q, Lmax);
  const int span = new_rows_only ? min(n64, (mq + PF_BC - 2) / PF_BC + 1) : n64;
  const dim3 grid((unsigned)(B * H * span));
  if (d == 128)
    hipLaunchKernelGGL((stage_v_kernel<128, _Float16, true>), grid, dim3(256), 0, s,
                       (const __bf16*)vc, (_Float16*)vt, Lmax, n64, ca, H, span);
  else
    hipLaunchKernelGGL((stage_v_kernel<64, _Float16, true>), grid, dim3(256), 0, s,
                       (const __bf16*)vc, (_Float16*)vt, Lmax, n64, ca, H, span);
  return hipGetLastError();
}

// Merge the split records of every chunk row over the splits that start at or
// before the row's cache position (each holds at least one of its keys; later
// splits hold none) and write o = o_sa - g (u - o_sa rbar).  One workgroup of D
// threads per (chunk query j, head b*H + h), heads fastest; the merge order is
// fixed.
template <int D>
__global__ __launch_bounds__(D)
void chunk_combine_kernel(const float* __restrict__ gate, float* __restrict__ out, int H, int BH,
                          ChunkArgs ca) {
  const int j = (int)(blockIdx.x / (unsigned)BH);
  const int bh = (int)(blockIdx.x % (unsigned)BH);
  const int b = bh / H, h = bh % H;
  int c0, n_q, pos0;
  chunk_geometry(ca, b, &c0, &n_q, &pos0);
  if (j >= n_q) return;
  const int f = threadIdx.x;
  constexpr int RF = 2 * D + 4;
  const int ns = (pos0 + j) / (ca.split_tiles * PF_BC) + 1;
  const size_t row = (size_t)(c0 + j) * H + h;
  const float* rec = ca.part + row * ca.n_split * RF;
  // unrolled so that several records' loads are in flight at once (the sums
  // keep their order)
  float M = kMinit;
#pragma unroll 8
  for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, rec[(size_t)sp * RF]);
  float l = 0.f, c = 0.f, a = 0.f, bv = 0.f;
#pragma unroll 8
  for (int sp = 0; sp < ns; ++sp) {
    const float* r = rec + (size_t)sp * RF;
    const float w = __builtin_amdgcn_exp2f(r[0] - M);
    // c and sum p r v of a split are relative to 2^-r_exp (record slot 3)
    const float wr = __builtin_ldexpf(w, (int)r[3]);
    l += w * r[1];
    c += wr * r[2];
    a += w * r[4 + f];
    bv += wr * r[4 + D + f];
  }
  const float inv = 1.0f / l;
  const float osa = a * inv;
  out[row * D + f] = osa - gate[h] * (bv * inv - osa * (c * inv));
}

// Keys per split the chunked prefill uses by default: none (one split of the
// whole cache) once the query tiles alone give PLX_CHUNK_SPLIT_BELOW
// workgroups (one per CU), else enough splits for PLX_CHUNK_SPLIT_TARGET
// workgroups, each at least PLX_CHUNK_SPLIT_MIN_TILES tiles long.  Measured:
// splitting 256 - 384 query tiles (one or two workgroups per CU already) costs
// 4 - 9 % in record traffic; below 256 it gains up to 8x.
#ifndef PLX_CHUNK_SPLIT_BELOW
#define PLX_CHUNK_SPLIT_BELOW 256
#endif
#ifndef PLX_CHUNK_SPLIT_TARGET
#define PLX_CHUNK_SPLIT_TARGET 512
#endif
#ifndef PLX_CHUNK_SPLIT_MIN_TILES
#define PLX_CHUNK_SPLIT_MIN_TILES 4
#endif
constexpr int kChunkMinSplitTiles = PLX_CHUNK_SPLIT_MIN_TILES;
constexpr int kChunkTargetBlocks = PLX_CHUNK_SPLIT_TARGET;
int chunk_default_split(int B, int H, int Lmax, int max_q, int d) {
  const int qpb = 16 * (d == 128 ? PLX_PF_NW_D128 : PLX_PF_NW_D64);
  const int n64 = (Lmax + PF_BC - 1) / PF_BC;
  const long long base = (long long)B * H * ((min(max_q, Lmax) + qpb - 1) / qpb);
  if (base <= 0 || base >= PLX_CHUNK_SPLIT_BELOW) return n64 * PF_BC;
  const int want = (int)((kChunkTargetBlocks + base - 1) / base);
  const int tiles = max(kChunkMinSplitTiles, (n64 + want - 1) / want);
  return min(tiles, n64) * PF_BC;
}

// Splits of split_keys keys over a cache of Lmax rows (1: no split).
int chunk_num_splits(int Lmax, int split_keys) {
  const int n64 = (Lmax + PF_BC - 1) / PF_BC;
  const int st = split_keys / PF_BC;
  return (n64 + st - 1) / st;
}

// Workgroups of the larger of the two split-KV launches (the API keeps it
// within a 1-D grid).
long long chunk_split_blocks(int B, int H, int Lmax, int max_q, int d, int split_keys) {
  const int qpb = 16 * (d == 128 ? PLX_PF_NW_D128 : PLX_PF_NW_D64);
  const long long mq = min(max_q, Lmax);
  const long long attend = (long long)B * H * ((mq + qpb - 1) / qpb) *
                           chunk_num_splits(Lmax, split_keys);
  const long long combine = (long long)B * H * mq;
  return attend > combine ? attend : combine;
}

// Bytes of split records a chunked prefill over T query rows needs (0 without
// a split).
size_t chunk_part_bytes(int T, int H, int Lmax, int d, int split_keys) {
  const int ns = chunk_num_splits(Lmax, split_keys);
  return ns > 1 ? (size_t)T * H * ns * (2 * d + 4) * sizeof(float) : 0;
}

// Whether a per-call chunked prefill reads V straight from the bf16 cache and
// converts its tiles in the kernel (no staging pass, no staged V^T workspace):
// d = 128 with chunks of at most 64 queries, one query tile.  (At d = 64 the
// kernel's 128-register budget spills in this form; it keeps the staging pass.)
bool chunk_fuses_v(int d, int max_q) { return PLX_CHUNK_FUSEV && d == 128 && max_q <= 64; }

// The fused-V chunk kernel (d = 128, four waves, plain schedule, non-temporal
// tile loads: a chunk of at most 64 queries is one query tile, so no workgroup
// re-reads a tile).  A tile is 128 blocks of 8 x 8.  Chunks of at most 16
// queries: wave 0 computes while waves 1-2 convert a block per thread; at most
// 32: waves 0-1 compute, waves 2-3 convert; else every wave converts half a
// block per thread and then computes.
template <bool SPLIT>
static hipError_t launch_fused_t(int max_q, const void* q, const void* kc, const void* vc,
                                 const void* rho, const float* gate, float* out, int B, int H,
                                 int Lmax, float sl2, hipStream_t s, const ChunkArgs& ca) {
  constexpr bool NT = PLX_CHUNK_NT != 0;
  if (max_q <= 16)
    return launch_prefill_t<128, 4, false, true, false, true, SPLIT, NT, 1>(
        q, kc, vc, rho, gate, out, B, H, Lmax, sl2, s, {}, ca);
  if (max_q <= 32)
    return launch_prefill_t<128, 4, false, true, false, true, SPLIT, NT, 2>(
        q, kc, vc, rho, gate, out, B, H, Lmax, sl2, s, {}, ca);
  return launch_prefill_t<128, 4, false, true, false, true, SPLIT, NT, 4>(
      q, kc, vc, rho, gate, out, B, H, Lmax, sl2, s, {}, ca);
}

// The chunked-prefill kernel at head dimension D (split-KV or not, NT cache policy).
template <int D, bool SPLIT, bool NT>
static hipError_t launch_chunk_t(const void* q, const void* kc, const void* vt, const void* rho,
                                 const float* gate, float* out, int B, int H, int Lmax, float sl2,
                                 hipStream_t s, const ChunkArgs& ca) {
  constexpr int NW = D == 128 ? PLX_PF_NW_D128 : PLX_PF_NW_D64;
  constexpr bool PIPE = (D == 128 ? PLX_PF_PIPE_D128 : PLX_PF_PIPE_D64) != 0;
  return launch_prefill_t<D, NW, PIPE, true, false, true, SPLIT, NT>(q, kc, vt, rho, gate, out, B,
                                                                     H, Lmax, sl2, s, {}, ca);
}

// Chunked prefill: unless the caller keeps the V cache staged (vc == null),
// stage V^T of the cache rows each chunk reads into vt; then attend, over the
// whole cache prefix or, with more than one split of split_keys keys (a
// multiple of 64), split by split into part and then combined.
hipError_t launch_prefill_chunk(const void* q, const void* kc, const void* vc, const void* rho,
                                const float* gate, float* out, const int* cu_q, const int* ctx,
                                int B, int H, int T, int Lmax, int max_q, int d, float scale,
                                int split_keys, void* vt, float* part, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  const int n64 = (Lmax + PF_BC - 1) / PF_BC;
  ChunkArgs ca{cu_q, ctx, T, Lmax, max_q, n64, 0};
  // Per-call V with short chunks: the kernel converts the raw V tiles itself
  // (no staging pass, and vt is not used).
  const bool fuse = vc != nullptr && chunk_fuses_v(d, max_q);
  if (vc && !fuse) {
    hipError_t e = launch_stage_v_rows(vc, vt, cu_q, ctx, B, H, T, Lmax, max_q, d, false, s);
    if (e != hipSuccess) return e;
  }
  // Non-temporal tile loads when each sequence's chunk fits one query tile (no
  // workgroup re-reads a K/V tile) and V comes from the caller's staged cache
  // or, fused, straight from the V cache.  With per-call staging the V^T tiles
  // were written just before and the default policy measured as fast or faster.
  const bool nt = PLX_CHUNK_NT && (vc == nullptr || fuse) &&
                  max_q <= 16 * (d == 128 ? PLX_PF_NW_D128 : PLX_PF_NW_D64);
  const int n_split = chunk_num_splits(Lmax, split_keys);
  if (n_split > 1) {
    ca.split_tiles = split_keys / PF_BC;
    ca.n_split = n_split;
    ca.part = part;
    hipError_t e;
    if (fuse)
      e = launch_fused_t<true>(max_q, q, kc, vc, rho, gate, out, B, H, Lmax, sl2, s, ca);
    else if (d == 128)
      e = nt ? launch_chunk_t<128, true, true>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca)
             : launch_chunk_t<128, true, false>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca);
    else
      e = nt ? launch_chunk_t<64, true, true>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca)
             : launch_chunk_t<64, true, false>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)min(max_q, Lmax) * (unsigned)(B * H));
    if (d == 128)
      hipLaunchKernelGGL((chunk_combine_kernel<128>), grid, dim3(128), 0, s, gate, out, H, B * H,
                         ca);
    else
      hipLaunchKernelGGL((chunk_combine_kernel<64>), grid, dim3(64), 0, s, gate, out, H, B * H,
                         ca);
    return hipGetLastError();
  }
  if (fuse)
    return launch_fused_t<false>(max_q, q, kc, vc, rho, gate, out, B, H, Lmax, sl2, s, ca);
  if (d == 128)
    return nt ? launch_chunk_t<128, false, true>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca)
              : launch_chunk_t<128, false, false>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca);
  return nt ? launch_chunk_t<64, false, true>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca)
            : launch_chunk_t<64, false, false>(q, kc, vt, rho, gate, out, B, H, Lmax, sl2, s, ca);
}

hipError_t launch_prefill_bf16_train(const void* q, const void* k, const void* vt,
                                     const void* rho, const float* gate, float* out,
                                     float* lse, float* rbar, float* corr, int B, int H, int L,
                                     int d, float scale, hipStream_t s) {
  const float sl2 = scale * kLog2e;
  const TrainOut tr{lse, rbar, corr};
  if (d == 128)
    return launch_prefill_t<128, PLX_PF_NW_D128, (PLX_PF_PIPE_D128 != 0), true, true>(
        q, k, vt, rho, gate, out, B, H, L, sl2, s, tr);
  return launch_prefill_t<64, PLX_PF_NW_D64, (PLX_PF_PIPE_D64 != 0), true, true>(
      q, k, vt, rho, gate, out, B, H, L, sl2, s, tr);
}

}  // namespace plx
