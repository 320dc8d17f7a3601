/*
 * parallax.h - C ABI of the Parallax attention forward pass on AMD CDNA4 (gfx950).
 *
 * The operation is defined on the page "Parallax - Parameterized Local Linear
 * Attention for Language Modeling" (technical summary; section "Core
 * mechanism", Eq. 2):
 *
 *     o_i = o^SA_i - g_h * Sigma_KV^(i) rho_i
 *
 * o^SA_i is causal softmax attention with weights w_ij = softmax_j(scale <q_i,k_j>),
 * Sigma_KV^(i) is the d x d cross-covariance of (v_j, k_j) under those weights
 * (centred, weights summing to one), rho_i is the probe (Eq. 1, rho_i = W_R x_i,
 * supplied here as an input), the boundary factor eta_i is zero and no solver
 * is involved (same section, design choices), and g_h is a per-head gate on
 * the correction branch (section "Results").  The kernels evaluate the
 * covariance term without forming the matrix, through
 *     Sigma^(i) rho_i = sum_j w_ij r_ij v_j - o^SA_i sum_j w_ij r_ij,  r_ij = <rho_i,k_j>,
 * in one streaming pass over K and V shared by both branches (section
 * "Hardware-aware algorithm").
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major arrays,
 *     16-byte aligned.  The caller owns every buffer; the library keeps no
 *     pointer after a call returns and never frees caller memory.
 *   - d (head dimension, d_k = d_v) must be 64 or 128.
 *   - dtype is PLX_BF16 (inputs stored as bfloat16) or PLX_F32.  Outputs are
 *     always fp32.  scale multiplies <q,k> only; pass scale <= 0 for 1/sqrt(d).
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; device faults surface at the caller's
 *     next synchronisation.
 *   - Arguments are validated before anything is enqueued.  On a bad argument
 *     the call returns an error status, enqueues nothing and sets the text of
 *     parallax_last_error().  A failed launch or allocation returns PLX_EHIP /
 *     PLX_ENOMEM.  The library never aborts, prints or throws across the ABI.
 *   - Apart from the per-thread error text and the per-device address of the
 *     scratch array of parallax_decode_noalloc (looked up once per device,
 *     under a once-flag), the library has no mutable global state; calls from
 *     several host threads are safe.
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARALLAX_ABI_VERSION 7

typedef enum {
  PLX_OK = 0,
  PLX_EINVAL = 1,        /* null pointer, non-positive size, workspace too small */
  PLX_EUNSUPPORTED = 2,  /* d not in {64,128}, unknown dtype */
  PLX_ENOMEM = 3,        /* the library could not allocate its own workspace */
  PLX_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} plx_status;

typedef enum { PLX_F32 = 0, PLX_BF16 = 1 } plx_dtype;

/* ABI version of the loaded library (PARALLAX_ABI_VERSION at build time). */
int parallax_abi_version(void);

/* Text of the last error on the calling thread ("" if none).  Valid until the
 * next library call on the same thread. */
const char* parallax_last_error(void);

/* ------------------------------------------------------------------ prefill
 * Causal prefill (page section "Core mechanism", Eq. 2, with query i attending
 * keys 0..i).
 *   q, k, v, rho : [B, H, L, d] in dtype
 *   gate         : [H] fp32, the correction gate g_h
 *   out          : [B, H, L, d] fp32
 * workspace: device scratch of at least parallax_prefill_workspace_bytes()
 * bytes (0 for PLX_F32).  If workspace is NULL the library allocates and frees
 * it on `stream` (stream-ordered allocation).  In PLX_BF16 mode the workspace
 * holds V converted to fp16 in a per-64-key-tile transposed layout (see
 * parallax_prefill_stage_v).  Range of the bf16 path:
 *   - V: fp16 holds every bf16 value with |v| <= 65280 exactly (subnormal fp16
 *     below 2^-14, absolute error < 2^-25).  fp16 cannot represent larger
 *     magnitudes: they are clamped to +-65504, so a row that attends such a
 *     value gets the clamped value, while rows that do not attend it are
 *     unaffected (in particular, never NaN).  |v| <= 65280 is the exact range.
 *   - rho: no limit.  The softmax numerators P (kept <= 16) and
 *     r_ij = <rho_i,k_j> are rounded to fp16 and T = P*r is formed in fp16 for
 *     the value products.  When r or T of some row leaves fp16's range, the
 *     16-row block holding that row is computed again with every row whose
 *     |r_ij| exceeds 2048 scaled by a power of two before that rounding and
 *     unscaled in fp32 at the end, which is exact because Eq. 2 is linear in
 *     rho; the block's other rows come out bit-identical to the single pass.
 *     (Only an element of rho_i whose magnitude falls below 2^-126 after that
 *     scaling loses bits.)  Such a block costs a second pass over its keys. */
size_t parallax_prefill_workspace_bytes(int B, int H, int L, int d, int dtype);

int parallax_prefill(const void* q, const void* k, const void* v, const void* rho,
                     const float* gate, float* out,
                     int B, int H, int L, int d, float scale, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of a PLX_BF16 prefill, for callers that keep the staged V
 * (for example across several calls over the same keys).
 * stage_v: v [B,H,L,d] bf16 -> vt16, fp16, laid out [B*H][ceil(L/64)][d][64]
 *          (the 64 keys of one tile and one feature contiguous); inside each
 *          group of 32 keys, position 8a+4b+c (a<4, b<2, c<4) holds key
 *          16b+4a+c, the order in which the attend kernel's score blocks
 *          produce them.  Keys past L are zero.
 *          vt16 must hold parallax_prefill_workspace_bytes(B,H,L,d,PLX_BF16).
 * attend : the fused causal forward pass reading V from vt16. */
int parallax_prefill_stage_v(const void* v, void* vt16, int B, int H, int L, int d,
                             void* stream);

int parallax_prefill_attend(const void* q, const void* k, const void* vt16,
                            const void* rho, const float* gate, float* out,
                            int B, int H, int L, int d, float scale, void* stream);

/* ------------------------------------------------------------------- decode
 * One decode step per sequence (page section "Core mechanism", Eq. 2, the
 * query attending every cached key of its sequence; section "Hardware-aware
 * algorithm": both branches share one pass over the KV stream).
 *   q, rho         : [B, H, d] in dtype
 *   kcache, vcache : [B, H, Lmax, d] in dtype
 *   gate           : [H] fp32
 *   seqlens        : [B] int32 in device memory; sequence b attends cache
 *                    positions 0..seqlens[b]-1.  Values are clamped to
 *                    [0, Lmax] on the device; length 0 yields a zero row.
 *                    Cache positions at or past seqlens[b] are never read.
 *   out            : [B, H, d] fp32
 * split_keys: keys per split of the split-KV pass (a multiple of 64, or 0 for
 * the library's choice).  workspace: at least
 * parallax_decode_workspace_bytes() bytes, or NULL to let the library allocate
 * on `stream`. */
size_t parallax_decode_workspace_bytes(int B, int H, int Lmax, int d, int split_keys);

int parallax_decode(const void* q, const void* kcache, const void* vcache, const void* rho,
                    const float* gate, float* out, const int32_t* seqlens,
                    int B, int H, int Lmax, int d, float scale, int dtype, int split_keys,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of a decode step.  They are also the merge point for a
 * sequence whose keys are spread over several devices: partial states over
 * disjoint key ranges combine exactly.
 * partials: for each (b,h) and split s < ceil(seqlens[b]/split_keys), a record
 *   of 2d+4 floats at partials + ((b*H+h)*S + s)*(2d+4), S = ceil(Lmax/split_keys):
 *   [0] m = max_j scale*log2(e)*<q,k_j>       (base-2 log domain)
 *   [1] l = sum_j 2^(scale*log2(e)*<q,k_j> - m)
 *   [2] c = sum_j 2^(...) r_j,  r_j = <rho,k_j>
 *   [3] unused
 *   [4 .. 4+d)      sum_j 2^(...) v_j
 *   [4+d .. 4+2d)   sum_j 2^(...) r_j v_j
 *   split_keys must be given explicitly (no 0) and the same in both calls. */
int parallax_decode_partials(const void* q, const void* kcache, const void* vcache,
                             const void* rho, const int32_t* seqlens, float* partials,
                             int B, int H, int Lmax, int d, float scale, int dtype,
                             int split_keys, void* stream);

int parallax_decode_combine(const float* partials, const float* gate, const int32_t* seqlens,
                            float* out, int B, int H, int Lmax, int d, int split_keys,
                            void* stream);

/* The split size parallax_decode uses when split_keys is 0. */
int parallax_decode_default_split(int B, int H, int Lmax, int d);

/* parallax_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  It
 * takes no workspace and calls no allocator: the split records live in a
 * fixed scratch array that the library's code object carries on every device
 * it runs on (parallax_decode_noalloc_max_bytes() bytes, 32 MiB, held until
 * the process ends).  Its device address is looked up once per device, on the
 * first call with that device current.  Arguments, layouts and results are
 * those of parallax_decode, which it matches bit for bit at the same
 * split_keys.  A call whose records
 * (parallax_decode_workspace_bytes(B, H, Lmax, d, split_keys)) exceed the
 * scratch returns PLX_EINVAL without enqueuing anything: pass a larger
 * split_keys.  The scratch is shared by every call on the same device and
 * keeps the last call's records; calls that overlap in time on one device
 * (different streams or host threads) race on it and must be ordered by the
 * caller.  The calling thread's current device must be the device of
 * `stream`. */
size_t parallax_decode_noalloc_max_bytes(void);

int parallax_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const void* rho, const float* gate, float* out,
                            const int32_t* seqlens, int B, int H, int Lmax, int d, float scale,
                            int dtype, int split_keys, void* stream);

/* ----------------------------------------------------------- chunked prefill
 * The step between prefill and decode (the pages' kernels target every batch
 * size and context length, section "Contributions"): sequence b holds ctx[b]
 * keys in its cache and appends a chunk of n_b = cu_q[b+1] - cu_q[b] queries,
 * whose keys and values the caller has already written to cache positions
 * ctx[b] .. ctx[b]+n_b-1.  Chunk query j sits at position ctx[b] + j and
 * attends cache positions 0 .. ctx[b] + j (Eq. 2 over that prefix).
 *   q, rho  : [T, H, d] bf16, packed and token-major: sequence b owns rows
 *             cu_q[b] .. cu_q[b+1]-1
 *   kcache, vcache : [B, H, Lmax, d] bf16
 *   gate    : [H] fp32
 *   cu_q    : [B+1] int32 device, non-decreasing row offsets into q
 *   ctx     : [B] int32 device, cached keys before each chunk
 *   out     : [T, H, d] fp32; rows of the chunks are written, others untouched
 * max_q must be at least the largest n_b (it sizes the grid).  The device
 * clamps cu_q to [0, T], n_b to min(max_q, Lmax) and ctx[b] to
 * [0, Lmax - n_b], so no access leaves q or the cache.  Cache rows at or past
 * ctx[b] + n_b are never read.  PLX_BF16 only.
 * split_keys: with fewer query tiles than the GPU has room for (few sequences,
 * short chunks), the cache prefix of every query tile is split into ranges of
 * split_keys keys, attended by separate workgroups into partial states that a
 * second kernel merges per query row in a fixed order (split-KV; exact up to
 * fp32 rounding order).  0 picks the library's split
 * (parallax_prefill_chunk_default_split); otherwise a positive multiple of 64,
 * where split_keys >= Lmax means no split.  Other values are PLX_EINVAL.
 * The workspace (at least parallax_prefill_chunk_workspace_bytes(B, H, T,
 * Lmax, max_q, d, split_keys) bytes, or NULL to let the library allocate on
 * `stream` when it needs any) holds the fp16 V^T tiles of the cache rows the
 * chunks read and, when split, the partial states (T*H*S records of 2d+4
 * floats, S = ceil(ceil(Lmax/64) / (split_keys/64))).  At d = 128 with
 * max_q <= 64 the kernel converts the bf16 V tiles itself, so there are no
 * V^T tiles and, without a split, the size is 0. */
size_t parallax_prefill_chunk_workspace_bytes(int B, int H, int T, int Lmax, int max_q, int d,
                                              int split_keys);

int parallax_prefill_chunk(const void* q, const void* kcache, const void* vcache,
                           const void* rho, const float* gate, float* out,
                           const int32_t* cu_q, const int32_t* ctx, int B, int H, int T,
                           int Lmax, int max_q, int d, float scale, int dtype, int split_keys,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Keys per split parallax_prefill_chunk uses for split_keys = 0: a multiple of
 * 64, at least Lmax when it does not split (0 for invalid sizes). */
int parallax_prefill_chunk_default_split(int B, int H, int Lmax, int max_q, int d);

/* A serving loop can keep the V cache's staged copy and skip the per-call
 * staging, which for short chunks is most of the traffic: vt_cache
 * ([B, H, ceil(Lmax/64), d, 64] fp16, parallax_prefill_workspace_bytes(B, H,
 * Lmax, d, PLX_BF16) bytes, the layout of parallax_prefill_stage_v applied to
 * the cache) holds V^T of every cache row.
 * parallax_stage_v_rows: after the chunks' values are written to vcache,
 *   re-stages only the 64-row tiles that hold rows ctx[b] .. ctx[b]+n_b-1
 *   (arguments and clamping as in parallax_prefill_chunk); rows at or past
 *   ctx[b]+n_b of those tiles are written as zeros.
 * parallax_prefill_chunk_vt: parallax_prefill_chunk reading V from vt_cache,
 *   whose tiles must hold rows 0 .. ctx[b]+n_b-1 of each sequence (after
 *   parallax_stage_v_rows for every append, or one parallax_prefill_stage_v of
 *   a cache whose rows are all finite).  Results are bit-identical to
 *   parallax_prefill_chunk with the same split_keys.  Its workspace holds only
 *   the partial states of a split: at least
 *   parallax_prefill_chunk_vt_workspace_bytes(B, H, T, Lmax, max_q, d,
 *   split_keys) bytes (0 without a split), or NULL to let the library allocate
 *   on `stream` when it needs any. */
int parallax_stage_v_rows(const void* vcache, void* vt_cache, const int32_t* cu_q,
                          const int32_t* ctx, int B, int H, int T, int Lmax, int max_q, int d,
                          void* stream);

size_t parallax_prefill_chunk_vt_workspace_bytes(int B, int H, int T, int Lmax, int max_q, int d,
                                                 int split_keys);

int parallax_prefill_chunk_vt(const void* q, const void* kcache, const void* vt_cache,
                              const void* rho, const float* gate, float* out,
                              const int32_t* cu_q, const int32_t* ctx, int B, int H, int T,
                              int Lmax, int max_q, int d, float scale, int dtype, int split_keys,
                              void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------- softmax baseline
 * Plain causal softmax attention, o_i = o^SA_i (Eq. 2 without the correction
 * branch), computed by the same kernels as the Parallax calls above with the
 * covariance branch removed at compile time: same staging, tiling, launch
 * shapes and precision, no rho reads, no <rho,k> products, no r-weighted
 * accumulators.  The page's efficiency claim (section "Key contributions")
 * compares Parallax kernels with softmax-attention kernels over batch sizes and
 * context lengths, and section "Hardware-aware algorithm" puts the extra work
 * at about twice the compute over a shared KV stream; these entry points are
 * the like-for-like softmax side of that comparison on this hardware.
 * Arguments, layouts, workspaces and error rules are those of the matching
 * Parallax call with rho and gate left out:
 *   parallax_softmax_prefill        <-> parallax_prefill
 *                                       (workspace: parallax_prefill_workspace_bytes)
 *   parallax_softmax_prefill_attend <-> parallax_prefill_attend
 *                                       (vt16 from parallax_prefill_stage_v)
 *   parallax_softmax_decode         <-> parallax_decode
 *                                       (workspace: parallax_decode_workspace_bytes,
 *                                        which also covers this call's smaller records) */
int parallax_softmax_prefill(const void* q, const void* k, const void* v, float* out,
                             int B, int H, int L, int d, float scale, int dtype,
                             void* workspace, size_t workspace_bytes, void* stream);

int parallax_softmax_prefill_attend(const void* q, const void* k, const void* vt16, float* out,
                                    int B, int H, int L, int d, float scale, void* stream);

int parallax_softmax_decode(const void* q, const void* kcache, const void* vcache, float* out,
                            const int32_t* seqlens, int B, int H, int Lmax, int d, float scale,
                            int dtype, int split_keys, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ----------------------------------------------------------------- training
 * The pages describe the forward pass only; pretraining (section "Results")
 * needs its gradient.  These calls give the exact derivative of Eq. 2 of the
 * causal prefill with respect to q, k, v, rho and the per-head gate, for
 * PLX_BF16 inputs (PLX_F32 returns PLX_EUNSUPPORTED).
 *
 * parallax_prefill_train: parallax_prefill that also writes, per row,
 *   lse  : [B, H, L] fp32, natural log of sum_j exp(scale <q_i,k_j>), j <= i
 *   rbar : [B, H, L] fp32, sum_j w_ij <rho_i,k_j>
 *   corr : [B, H, L, d] fp32, the correction Sigma^(i) rho_i
 *          (out = o^SA - gate[h] * corr).
 * out alone does not determine o^SA when the gate is non-zero, so the
 * backward pass needs corr.  Workspace: parallax_prefill_workspace_bytes().
 *
 * parallax_prefill_backward: given out, corr, lse and rbar from
 * parallax_prefill_train on the same inputs, and dout = dL/dout ([B,H,L,d]
 * fp32), writes the gradients of L:
 *   dq, dk, dv, drho : [B, H, L, d] fp32
 *   dgate            : [H] fp32, summed over the batch
 * Every output element is written; nothing is accumulated into the outputs.
 * dout is rounded to bf16 for the matrix products (as are the softmax-weight
 * gradients); all sums are fp32.  The result is deterministic (no atomics).
 * Workspace: at least parallax_prefill_backward_workspace_bytes() bytes
 * (about 5 * B*H*L*d*2 bytes), or NULL to let the library allocate on `stream`. */
int parallax_prefill_train(const void* q, const void* k, const void* v, const void* rho,
                           const float* gate, float* out, float* lse, float* rbar, float* corr,
                           int B, int H, int L, int d, float scale, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

size_t parallax_prefill_backward_workspace_bytes(int B, int H, int L, int d);

int parallax_prefill_backward(const void* q, const void* k, const void* v, const void* rho,
                              const float* gate, const float* out, const float* corr,
                              const float* lse, const float* rbar, const float* dout,
                              float* dq, float* dk, float* dv, float* drho, float* dgate,
                              int B, int H, int L, int d, float scale, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
