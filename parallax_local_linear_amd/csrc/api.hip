// Host side of the Parallax C ABI: argument checks, workspace handling, launches.
// Declarations, layouts and error rules are in include/parallax.h.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/parallax.h"

namespace plx {
hipError_t launch_stage_v(const void* v, void* vt, int BH, int L, int d, hipStream_t s);
// corr = false: the same kernels with the covariance branch compiled out
hipError_t launch_prefill_bf16(const void* q, const void* k, const void* vt, const void* rho,
                               const float* gate, float* out, int B, int H, int L, int d,
                               float scale, bool corr, hipStream_t s);
hipError_t launch_prefill_f32(const void* q, const void* k, const void* v, const void* rho,
                              const float* gate, float* out, int B, int H, int L, int d,
                              float scale, bool corr, hipStream_t s);
hipError_t launch_decode_split(const void* q, const void* kc, const void* vc, const void* rho,
                               const int* seqlens, float* part, int B, int H, int Lmax, int d,
                               int C, float scale, bool bf16, bool corr, hipStream_t s);
hipError_t launch_decode_combine(const float* part, const float* gate, const int* seqlens,
                                 float* out, int B, int H, int Lmax, int d, int C, bool corr,
                                 hipStream_t s);
hipError_t launch_prefill_bf16_train(const void* q, const void* k, const void* vt,
                                     const void* rho, const float* gate, float* out,
                                     float* lse, float* rbar, float* corr, int B, int H, int L,
                                     int d, float scale, hipStream_t s);
hipError_t launch_prefill_backward(const void* q, const void* k, const void* v, const void* rho,
                                   const float* gate, const float* out, const float* corr,
                                   const float* lse, const float* rbar, const float* dout,
                                   float* dq, float* dk, float* dv, float* drho, float* dgate,
                                   int B, int H, int L, int d, float scale, void* ws,
                                   hipStream_t s);
size_t bwd_workspace_bytes(int B, int H, int L, int d);
hipError_t launch_prefill_chunk(const void* q, const void* kc, const void* vc, const void* rho,
                                const float* gate, float* out, const int* cu_q, const int* ctx,
                                int B, int H, int T, int Lmax, int max_q, int d, float scale,
                                int split_keys, void* vt, float* part, hipStream_t s);
int chunk_default_split(int B, int H, int Lmax, int max_q, int d);
int chunk_num_splits(int Lmax, int split_keys);
size_t chunk_part_bytes(int T, int H, int Lmax, int d, int split_keys);
bool chunk_fuses_v(int d, int max_q);
long long chunk_split_blocks(int B, int H, int Lmax, int max_q, int d, int split_keys);
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_stage_v_rows(const void* vc, void* vt, const int* cu_q, const int* ctx, int B,
                               int H, int T, int Lmax, int max_q, int d, bool new_rows_only,
                               hipStream_t s);
}  // namespace plx

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return PLX_OK;
}

int hip_fail(const char* what, hipError_t e) {
  return fail(PLX_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int launch_fail(const char* fn, const char* kernel, hipError_t e) {
  return fail(PLX_EHIP, "%s: %s launch: %s", fn, kernel, hipGetErrorString(e));
}

constexpr int kTileKeys = 64;
constexpr long long kMaxElems = (1LL << 40);   // guard against size_t overflow of products

bool dims_ok(int B, int H, int L, int d, const char* fn, const char* lname, int* status) {
  if (B <= 0 || H <= 0 || L <= 0) {
    *status = fail(PLX_EINVAL, "%s: B, H and %s must be positive (got %d, %d, %d)", fn, lname,
                   B, H, L);
    return false;
  }
  if (d != 64 && d != 128) {
    *status = fail(PLX_EUNSUPPORTED, "%s: d must be 64 or 128 (got %d)", fn, d);
    return false;
  }
  if ((long long)B * H * (long long)L * d > kMaxElems || (long long)L * d > (1LL << 31)) {
    *status = fail(PLX_EINVAL, "%s: tensor too large", fn);
    return false;
  }
  return true;
}

// Checks shared by the chunked-prefill calls.
bool chunk_args_ok(int B, int H, int T, int Lmax, int max_q, int d, const char* fn, int* st) {
  if (!dims_ok(B, H, Lmax, d, fn, "Lmax", st)) return false;
  if (T <= 0 || max_q <= 0) {
    *st = fail(PLX_EINVAL, "%s: T and max_q must be positive (got %d, %d)", fn, T, max_q);
    return false;
  }
  if ((long long)T * H * d > kMaxElems) {
    *st = fail(PLX_EINVAL, "%s: tensor too large", fn);
    return false;
  }
  return true;
}

// split_keys of a chunked prefill: 0 picks the library's split, else a positive
// multiple of 64 (at least Lmax: no split).  The split launches must fit a 1-D
// grid.
bool chunk_split_ok(int split_keys, int B, int H, int Lmax, int max_q, int d, const char* fn,
                    int* st, int* keys) {
  if (split_keys < 0 || split_keys % 64 != 0) {
    *st = fail(PLX_EINVAL, "%s: split_keys must be 0 or a positive multiple of 64 (got %d)", fn,
               split_keys);
    return false;
  }
  *keys = split_keys ? split_keys : plx::chunk_default_split(B, H, Lmax, max_q, d);
  if (plx::chunk_num_splits(Lmax, *keys) > 1 &&
      plx::chunk_split_blocks(B, H, Lmax, max_q, d, *keys) > 0x7fffffffLL) {
    *st = fail(PLX_EINVAL, "%s: split_keys %d gives too many workgroups", fn, *keys);
    return false;
  }
  return true;
}

// Split records follow the staged V^T in a chunk workspace, 256-byte aligned.
size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// The decode grid puts the B*H streams on its second dimension.
bool streams_ok(int B, int H, const char* fn, int* status) {
  if ((long long)B * H > 65535) {
    *status = fail(PLX_EINVAL, "%s: B*H must not exceed 65535 (got %lld)", fn, (long long)B * H);
    return false;
  }
  return true;
}

bool dtype_ok(int dtype, const char* fn, int* status) {
  if (dtype != PLX_F32 && dtype != PLX_BF16) {
    *status = fail(PLX_EUNSUPPORTED, "%s: unknown dtype %d", fn, dtype);
    return false;
  }
  return true;
}

float eff_scale(float scale, int d) { return scale > 0.f ? scale : 1.0f / std::sqrt((float)d); }

size_t vt_bytes(int B, int H, int L, int d) {
  const size_t n_kt = (size_t)((L + kTileKeys - 1) / kTileKeys);
  return (size_t)B * H * n_kt * kTileKeys * d * 2;
}

// Bytes ahead of the split records in a per-call chunk workspace: the staged
// V^T tiles, unless the kernel converts the raw V tiles itself.
size_t chunk_vt_off(int B, int H, int Lmax, int max_q, int d) {
  return plx::chunk_fuses_v(d, max_q) ? 0 : align256(vt_bytes(B, H, Lmax, d));
}

size_t part_bytes(int B, int H, int Lmax, int d, int C) {
  const size_t S = (size_t)((Lmax + C - 1) / C);
  return (size_t)B * H * S * (2 * d + 4) * sizeof(float);
}

int default_split(int B, int H, int Lmax) {
  // aim at ~8k workgroups for the split pass (32 per CU), with at least 512 keys
  // per split: two passes of the workgroup's 256-key loop, so a workgroup's fixed
  // work (its q and rho loads, the merge of its lane groups, its record) stays
  // small beside its share of the cache.  Measured on small batches (B 1 and 8,
  // H 16, 8192-32768 keys): 512 keys beat 256 by 7-9 %.
  long long target = 8192;
  long long c = ((long long)Lmax * B * H + target - 1) / target;
  int C = 512;
  while (C < c && C < 16384) C <<= 1;
  return C;
}

bool split_ok(int C, const char* fn, int* status) {
  if (C <= 0 || C % kTileKeys != 0) {
    *status = fail(PLX_EINVAL, "%s: split_keys must be a positive multiple of 64 (got %d)",
                   fn, C);
    return false;
  }
  return true;
}

// Stream-ordered scratch used when the caller passes no workspace.
struct Scratch {
  void* ptr = nullptr;
  hipStream_t stream = nullptr;
  ~Scratch() {
    if (ptr) (void)hipFreeAsync(ptr, stream);
  }
};

// The caller's workspace when it is large enough, else stream-ordered scratch.
bool get_workspace(void* workspace, size_t workspace_bytes, size_t need, hipStream_t s,
                   Scratch* scratch, void** ws, const char* fn, int* status) {
  if (workspace) {
    if (workspace_bytes < need) {
      *status = fail(PLX_EINVAL, "%s: workspace of %zu bytes is smaller than the %zu required",
                     fn, workspace_bytes, need);
      return false;
    }
    *ws = workspace;
    return true;
  }
  hipError_t e = hipMallocAsync(&scratch->ptr, need, s);
  if (e != hipSuccess) {
    *status = fail(PLX_ENOMEM, "%s: hipMallocAsync(%zu): %s", fn, need, hipGetErrorString(e));
    return false;
  }
  scratch->stream = s;
  *ws = scratch->ptr;
  return true;
}

// Whole prefill; rho and gate are ignored (may be null) when corr is false.
int prefill_impl(const char* fn, const void* q, const void* k, const void* v, const void* rho,
                 const float* gate, float* out, int B, int H, int L, int d, float scale,
                 int dtype, void* workspace, size_t workspace_bytes, hipStream_t s, bool corr) {
  int st = PLX_OK;
  if (!dims_ok(B, H, L, d, fn, "L", &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (!q || !k || !v || !out || (corr && (!rho || !gate)))
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  const float sc = eff_scale(scale, d);
  if (dtype == PLX_F32) {
    hipError_t e = plx::launch_prefill_f32(q, k, v, rho, gate, out, B, H, L, d, sc, corr, s);
    if (e != hipSuccess) return launch_fail(fn, "fp32 prefill", e);
    return ok();
  }
  Scratch scratch;
  void* ws = nullptr;
  if (!get_workspace(workspace, workspace_bytes, vt_bytes(B, H, L, d), s, &scratch, &ws, fn,
                     &st))
    return st;
  hipError_t e = plx::launch_stage_v(v, ws, B * H, L, d, s);
  if (e != hipSuccess) return launch_fail(fn, "stage_v", e);
  e = plx::launch_prefill_bf16(q, k, ws, rho, gate, out, B, H, L, d, sc, corr, s);
  if (e != hipSuccess) return launch_fail(fn, "attend", e);
  return ok();
}

int attend_impl(const char* fn, const void* q, const void* k, const void* vt16, const void* rho,
                const float* gate, float* out, int B, int H, int L, int d, float scale,
                hipStream_t s, bool corr) {
  int st = PLX_OK;
  if (!dims_ok(B, H, L, d, fn, "L", &st)) return st;
  if (!q || !k || !vt16 || !out || (corr && (!rho || !gate)))
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  hipError_t e = plx::launch_prefill_bf16(q, k, vt16, rho, gate, out, B, H, L, d,
                                          eff_scale(scale, d), corr, s);
  if (e != hipSuccess) return launch_fail(fn, "attend", e);
  return ok();
}

// Whole decode step; rho and gate are ignored (may be null) when corr is false.
int decode_impl(const char* fn, const void* q, const void* kcache, const void* vcache,
                const void* rho, const float* gate, float* out, const int32_t* seqlens, int B,
                int H, int Lmax, int d, float scale, int dtype, int split_keys, void* workspace,
                size_t workspace_bytes, hipStream_t s, bool corr) {
  int st = PLX_OK;
  if (!dims_ok(B, H, Lmax, d, fn, "Lmax", &st)) return st;
  if (!streams_ok(B, H, fn, &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (split_keys < 0) return fail(PLX_EINVAL, "%s: split_keys must be >= 0", fn);
  const int C = split_keys > 0 ? split_keys : default_split(B, H, Lmax);
  if (!split_ok(C, fn, &st)) return st;
  if (!q || !kcache || !vcache || !out || !seqlens || (corr && (!rho || !gate)))
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  Scratch scratch;
  void* ws = nullptr;
  if (!get_workspace(workspace, workspace_bytes, part_bytes(B, H, Lmax, d, C), s, &scratch, &ws,
                     fn, &st))
    return st;
  float* part = static_cast<float*>(ws);
  hipError_t e = plx::launch_decode_split(q, kcache, vcache, rho, seqlens, part, B, H, Lmax, d,
                                          C, eff_scale(scale, d), dtype == PLX_BF16, corr, s);
  if (e != hipSuccess) return launch_fail(fn, "split", e);
  e = plx::launch_decode_combine(part, gate, seqlens, out, B, H, Lmax, d, C, corr, s);
  if (e != hipSuccess) return launch_fail(fn, "combine", e);
  return ok();
}

}  // namespace

extern "C" {

int parallax_abi_version(void) { return PARALLAX_ABI_VERSION; }

const char* parallax_last_error(void) { return g_err; }

size_t parallax_prefill_workspace_bytes(int B, int H, int L, int d, int dtype) {
  if (B <= 0 || H <= 0 || L <= 0 || (d != 64 && d != 128) || dtype != PLX_BF16) return 0;
  return vt_bytes(B, H, L, d);
}

int parallax_prefill_stage_v(const void* v, void* vt16, int B, int H, int L, int d,
                             void* stream) {
  int st = PLX_OK;
  if (!dims_ok(B, H, L, d, "parallax_prefill_stage_v", "L", &st)) return st;
  if (!v || !vt16) return fail(PLX_EINVAL, "parallax_prefill_stage_v: null pointer");
  hipError_t e = plx::launch_stage_v(v, vt16, B * H, L, d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("parallax_prefill_stage_v launch", e);
  return ok();
}

int parallax_prefill_attend(const void* q, const void* k, const void* vt16, const void* rho,
                            const float* gate, float* out, int B, int H, int L, int d,
                            float scale, void* stream) {
  return attend_impl("parallax_prefill_attend", q, k, vt16, rho, gate, out, B, H, L, d, scale,
                     (hipStream_t)stream, true);
}

int parallax_prefill(const void* q, const void* k, const void* v, const void* rho,
                     const float* gate, float* out, int B, int H, int L, int d, float scale,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl("parallax_prefill", q, k, v, rho, gate, out, B, H, L, d, scale, dtype,
                      workspace, workspace_bytes, (hipStream_t)stream, true);
}

int parallax_decode_default_split(int B, int H, int Lmax, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || Lmax <= 0) return 0;
  return default_split(B, H, Lmax);
}

size_t parallax_decode_workspace_bytes(int B, int H, int Lmax, int d, int split_keys) {
  if (B <= 0 || H <= 0 || Lmax <= 0 || (d != 64 && d != 128)) return 0;
  const int C = split_keys > 0 ? split_keys : default_split(B, H, Lmax);
  if (C % kTileKeys) return 0;
  return part_bytes(B, H, Lmax, d, C);
}

int parallax_decode_partials(const void* q, const void* kcache, const void* vcache,
                             const void* rho, const int32_t* seqlens, float* partials, int B,
                             int H, int Lmax, int d, float scale, int dtype, int split_keys,
                             void* stream) {
  const char* fn = "parallax_decode_partials";
  int st = PLX_OK;
  if (!dims_ok(B, H, Lmax, d, fn, "Lmax", &st)) return st;
  if (!streams_ok(B, H, fn, &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (!split_ok(split_keys, fn, &st)) return st;
  if (!q || !kcache || !vcache || !rho || !seqlens || !partials)
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  hipError_t e = plx::launch_decode_split(q, kcache, vcache, rho, seqlens, partials, B, H, Lmax,
                                          d, split_keys, eff_scale(scale, d),
                                          dtype == PLX_BF16, true, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("parallax_decode_partials launch", e);
  return ok();
}

int parallax_decode_combine(const float* partials, const float* gate, const int32_t* seqlens,
                            float* out, int B, int H, int Lmax, int d, int split_keys,
                            void* stream) {
  const char* fn = "parallax_decode_combine";
  int st = PLX_OK;
  if (!dims_ok(B, H, Lmax, d, fn, "Lmax", &st)) return st;
  if (!split_ok(split_keys, fn, &st)) return st;
  if (!partials || !gate || !seqlens || !out) return fail(PLX_EINVAL, "%s: null pointer", fn);
  hipError_t e = plx::launch_decode_combine(partials, gate, seqlens, out, B, H, Lmax, d,
                                            split_keys, true, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail("parallax_decode_combine launch", e);
  return ok();
}

int parallax_decode(const void* q, const void* kcache, const void* vcache, const void* rho,
                    const float* gate, float* out, const int32_t* seqlens, int B, int H,
                    int Lmax, int d, float scale, int dtype, int split_keys, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_impl("parallax_decode", q, kcache, vcache, rho, gate, out, seqlens, B, H, Lmax,
                     d, scale, dtype, split_keys, workspace, workspace_bytes,
                     (hipStream_t)stream, true);
}

size_t parallax_decode_noalloc_max_bytes(void) { return plx::noalloc_scratch_bytes(); }

int parallax_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const void* rho, const float* gate, float* out,
                            const int32_t* seqlens, int B, int H, int Lmax, int d, float scale,
                            int dtype, int split_keys, void* stream) {
  const char* fn = "parallax_decode_noalloc";
  int st = PLX_OK;
  if (!dims_ok(B, H, Lmax, d, fn, "Lmax", &st)) return st;
  if (!streams_ok(B, H, fn, &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (split_keys < 0) return fail(PLX_EINVAL, "%s: split_keys must be >= 0", fn);
  const int C = split_keys > 0 ? split_keys : default_split(B, H, Lmax);
  if (!split_ok(C, fn, &st)) return st;
  if (!q || !kcache || !vcache || !rho || !gate || !out || !seqlens)
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  const size_t need = part_bytes(B, H, Lmax, d, C);
  if (need > plx::noalloc_scratch_bytes())
    return fail(PLX_EINVAL,
                "%s: the split records need %zu bytes, more than the %zu-byte scratch; pass a "
                "larger split_keys or call parallax_decode with a workspace",
                fn, need, plx::noalloc_scratch_bytes());
  void* ws = nullptr;
  hipError_t se = plx::noalloc_scratch(&ws);
  if (se != hipSuccess) return hip_fail("parallax_decode_noalloc: scratch address", se);
  hipStream_t s = (hipStream_t)stream;
  float* part = static_cast<float*>(ws);
  hipError_t e = plx::launch_decode_split(q, kcache, vcache, rho, seqlens, part, B, H, Lmax, d,
                                          C, eff_scale(scale, d), dtype == PLX_BF16, true, s);
  if (e != hipSuccess) return launch_fail(fn, "split", e);
  e = plx::launch_decode_combine(part, gate, seqlens, out, B, H, Lmax, d, C, true, s);
  if (e != hipSuccess) return launch_fail(fn, "combine", e);
  return ok();
}

int parallax_softmax_prefill(const void* q, const void* k, const void* v, float* out, int B,
                             int H, int L, int d, float scale, int dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return prefill_impl("parallax_softmax_prefill", q, k, v, nullptr, nullptr, out, B, H, L, d,
                      scale, dtype, workspace, workspace_bytes, (hipStream_t)stream, false);
}

int parallax_softmax_prefill_attend(const void* q, const void* k, const void* vt16, float* out,
                                    int B, int H, int L, int d, float scale, void* stream) {
  return attend_impl("parallax_softmax_prefill_attend", q, k, vt16, nullptr, nullptr, out, B,
                     H, L, d, scale, (hipStream_t)stream, false);
}

size_t parallax_prefill_backward_workspace_bytes(int B, int H, int L, int d) {
  if (B <= 0 || H <= 0 || L <= 0 || (d != 64 && d != 128)) return 0;
  if ((long long)B * H * (long long)L * d > kMaxElems) return 0;
  return plx::bwd_workspace_bytes(B, H, L, d);
}

int parallax_prefill_train(const void* q, const void* k, const void* v, const void* rho,
                           const float* gate, float* out, float* lse, float* rbar, float* corr,
                           int B, int H, int L, int d, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const char* fn = "parallax_prefill_train";
  int st = PLX_OK;
  if (!dims_ok(B, H, L, d, fn, "L", &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (dtype != PLX_BF16) return fail(PLX_EUNSUPPORTED, "%s: only PLX_BF16 is supported", fn);
  if (!q || !k || !v || !rho || !gate || !out || !lse || !rbar || !corr)
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch;
  void* ws = nullptr;
  if (!get_workspace(workspace, workspace_bytes, vt_bytes(B, H, L, d), s, &scratch, &ws, fn, &st))
    return st;
  hipError_t e = plx::launch_stage_v(v, ws, B * H, L, d, s);
  if (e != hipSuccess) return launch_fail(fn, "stage_v", e);
  e = plx::launch_prefill_bf16_train(q, k, ws, rho, gate, out, lse, rbar, corr, B, H, L, d,
                                     eff_scale(scale, d), s);
  if (e != hipSuccess) return launch_fail(fn, "attend", e);
  return ok();
}

int parallax_prefill_backward(const void* q, const void* k, const void* v, const void* rho,
                              const float* gate, const float* out, const float* corr,
                              const float* lse, const float* rbar, const float* dout, float* dq,
                              float* dk, float* dv, float* drho, float* dgate, int B, int H,
                              int L, int d, float scale, int dtype, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const char* fn = "parallax_prefill_backward";
  int st = PLX_OK;
  if (!dims_ok(B, H, L, d, fn, "L", &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (dtype != PLX_BF16) return fail(PLX_EUNSUPPORTED, "%s: only PLX_BF16 is supported", fn);
  if (!q || !k || !v || !rho || !gate || !out || !corr || !lse || !rbar || !dout || !dq || !dk ||
      !dv || !drho || !dgate)
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch;
  void* ws = nullptr;
  if (!get_workspace(workspace, workspace_bytes, plx::bwd_workspace_bytes(B, H, L, d), s,
                     &scratch, &ws, fn, &st))
    return st;
  hipError_t e = plx::launch_prefill_backward(q, k, v, rho, gate, out, corr, lse, rbar, dout, dq,
                                              dk, dv, drho, dgate, B, H, L, d,
                                              eff_scale(scale, d), ws, s);
  if (e != hipSuccess) return launch_fail(fn, "backward", e);
  return ok();
}

size_t parallax_prefill_chunk_workspace_bytes(int B, int H, int T, int Lmax, int max_q, int d,
                                              int split_keys) {
  if (B <= 0 || H <= 0 || T <= 0 || Lmax <= 0 || max_q <= 0 || (d != 64 && d != 128)) return 0;
  if (split_keys < 0 || split_keys % 64 != 0) return 0;
  const int keys = split_keys ? split_keys : plx::chunk_default_split(B, H, Lmax, max_q, d);
  return chunk_vt_off(B, H, Lmax, max_q, d) + plx::chunk_part_bytes(T, H, Lmax, d, keys);
}

size_t parallax_prefill_chunk_vt_workspace_bytes(int B, int H, int T, int Lmax, int max_q, int d,
                                                 int split_keys) {
  if (B <= 0 || H <= 0 || T <= 0 || Lmax <= 0 || max_q <= 0 || (d != 64 && d != 128)) return 0;
  if (split_keys < 0 || split_keys % 64 != 0) return 0;
  const int keys = split_keys ? split_keys : plx::chunk_default_split(B, H, Lmax, max_q, d);
  return plx::chunk_part_bytes(T, H, Lmax, d, keys);
}

int parallax_prefill_chunk_default_split(int B, int H, int Lmax, int max_q, int d) {
  if (B <= 0 || H <= 0 || Lmax <= 0 || max_q <= 0 || (d != 64 && d != 128)) return 0;
  return plx::chunk_default_split(B, H, Lmax, max_q, d);
}

int parallax_prefill_chunk(const void* q, const void* kcache, const void* vcache, const void* rho,
                           const float* gate, float* out, const int32_t* cu_q,
                           const int32_t* ctx, int B, int H, int T, int Lmax, int max_q, int d,
                           float scale, int dtype, int split_keys, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const char* fn = "parallax_prefill_chunk";
  int st = PLX_OK;
  if (!chunk_args_ok(B, H, T, Lmax, max_q, d, fn, &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (dtype != PLX_BF16) return fail(PLX_EUNSUPPORTED, "%s: only PLX_BF16 is supported", fn);
  if (!q || !kcache || !vcache || !rho || !gate || !out || !cu_q || !ctx)
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  int keys = 0;
  if (!chunk_split_ok(split_keys, B, H, Lmax, max_q, d, fn, &st, &keys)) return st;
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch;
  void* ws = nullptr;
  const size_t vt_off = chunk_vt_off(B, H, Lmax, max_q, d);
  const size_t need = vt_off + plx::chunk_part_bytes(T, H, Lmax, d, keys);
  if (need > 0 && !get_workspace(workspace, workspace_bytes, need, s, &scratch, &ws, fn, &st))
    return st;
  float* part = ws ? reinterpret_cast<float*>(static_cast<char*>(ws) + vt_off) : nullptr;
  hipError_t e = plx::launch_prefill_chunk(q, kcache, vcache, rho, gate, out, cu_q, ctx, B, H, T,
                                           Lmax, max_q, d, eff_scale(scale, d), keys, ws, part,
                                           s);
  if (e != hipSuccess) return launch_fail(fn, "chunk", e);
  return ok();
}

int parallax_stage_v_rows(const void* vcache, void* vt_cache, const int32_t* cu_q,
                          const int32_t* ctx, int B, int H, int T, int Lmax, int max_q, int d,
                          void* stream) {
  const char* fn = "parallax_stage_v_rows";
  int st = PLX_OK;
  if (!chunk_args_ok(B, H, T, Lmax, max_q, d, fn, &st)) return st;
  if (!vcache || !vt_cache || !cu_q || !ctx) return fail(PLX_EINVAL, "%s: null pointer", fn);
  hipError_t e = plx::launch_stage_v_rows(vcache, vt_cache, cu_q, ctx, B, H, T, Lmax, max_q, d,
                                          true, (hipStream_t)stream);
  if (e != hipSuccess) return launch_fail(fn, "stage_v", e);
  return ok();
}

int parallax_prefill_chunk_vt(const void* q, const void* kcache, const void* vt_cache,
                              const void* rho, const float* gate, float* out,
                              const int32_t* cu_q, const int32_t* ctx, int B, int H, int T,
                              int Lmax, int max_q, int d, float scale, int dtype, int split_keys,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "parallax_prefill_chunk_vt";
  int st = PLX_OK;
  if (!chunk_args_ok(B, H, T, Lmax, max_q, d, fn, &st)) return st;
  if (!dtype_ok(dtype, fn, &st)) return st;
  if (dtype != PLX_BF16) return fail(PLX_EUNSUPPORTED, "%s: only PLX_BF16 is supported", fn);
  if (!q || !kcache || !vt_cache || !rho || !gate || !out || !cu_q || !ctx)
    return fail(PLX_EINVAL, "%s: null pointer", fn);
  int keys = 0;
  if (!chunk_split_ok(split_keys, B, H, Lmax, max_q, d, fn, &st, &keys)) return st;
  hipStream_t s = (hipStream_t)stream;
  Scratch scratch;
  void* ws = nullptr;
  const size_t need = plx::chunk_part_bytes(T, H, Lmax, d, keys);
  if (need > 0 && !get_workspace(workspace, workspace_bytes, need, s, &scratch, &ws, fn, &st))
    return st;
  hipError_t e = plx::launch_prefill_chunk(q, kcache, nullptr, rho, gate, out, cu_q, ctx, B, H, T,
                                           Lmax, max_q, d, eff_scale(scale, d), keys,
                                           const_cast<void*>(vt_cache), static_cast<float*>(ws),
                                           s);
  if (e != hipSuccess) return launch_fail(fn, "chunk", e);
  return ok();
}

int parallax_softmax_decode(const void* q, const void* kcache, const void* vcache, float* out,
                            const int32_t* seqlens, int B, int H, int Lmax, int d, float scale,
                            int dtype, int split_keys, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return decode_impl("parallax_softmax_decode", q, kcache, vcache, nullptr, nullptr, out,
                     seqlens, B, H, Lmax, d, scale, dtype, split_keys, workspace,
                     workspace_bytes, (hipStream_t)stream, false);
}

}  // extern "C"
