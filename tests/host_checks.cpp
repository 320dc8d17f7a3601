// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer around the library's host code (tests/test_host_sanitized.py).
//
// Every call here is rejected by argument validation before anything touches a
// device pointer, except the "no device" block, which only runs when the HIP
// runtime reports no device: there the launch and allocation failures must come
// back as PLX_EHIP / PLX_ENOMEM with an error text.  Exit status = number of
// failed checks.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <thread>

#include "parallax.h"

namespace {

int g_failed = 0;

void check(bool cond, const char* what) {
  if (!cond) {
    std::printf("FAIL: %s (last error: \"%s\")\n", what, parallax_last_error());
    ++g_failed;
  }
}

// status matches and the error text names the entry point
void expect(int st, int want, const char* fn, const char* what) {
  const std::string msg = parallax_last_error();
  if (st != want || msg.find(fn) == std::string::npos) {
    std::printf("FAIL: %s: status %d (want %d), error \"%s\"\n", what, st, want, msg.c_str());
    ++g_failed;
  }
}

// Distinct non-null addresses that are never dereferenced by the rejected calls.
char g_dummy[64];
void* P(int i) { return g_dummy + i; }
float* F(int i) { return reinterpret_cast<float*>(g_dummy + 4 * i); }
const int32_t* I(int i) { return reinterpret_cast<const int32_t*>(g_dummy + 4 * i); }

size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

void workspace_sizes() {
  for (int d : {64, 128})
    for (int L : {1, 63, 64, 65, 4096}) {
      const size_t want = (size_t)3 * 5 * ceil_div(L, 64) * 64 * d * 2;
      check(parallax_prefill_workspace_bytes(3, 5, L, d, PLX_BF16) == want,
            "prefill workspace = B*H*ceil(L/64)*64*d*2 bytes");
      check(parallax_prefill_workspace_bytes(3, 5, L, d, PLX_F32) == 0,
            "fp32 prefill needs no workspace");
    }
  check(parallax_prefill_workspace_bytes(0, 1, 64, 64, PLX_BF16) == 0, "B=0 workspace is 0");
  check(parallax_prefill_workspace_bytes(1, 1, 64, 96, PLX_BF16) == 0, "d=96 workspace is 0");
  for (int d : {64, 128})
    for (int Lmax : {1, 1000, 8192, 131072}) {
      const size_t want = (size_t)2 * 3 * ceil_div(Lmax, 1024) * (2 * d + 4) * 4;
      check(parallax_decode_workspace_bytes(2, 3, Lmax, d, 1024) == want,
            "decode workspace = B*H*ceil(Lmax/C)*(2d+4)*4 bytes");
      const int C = parallax_decode_default_split(2, 3, Lmax, d);
      check(C >= 256 && C % 64 == 0, "default split is a multiple of 64, at least 256");
      check(parallax_decode_workspace_bytes(2, 3, Lmax, d, 0) ==
                parallax_decode_workspace_bytes(2, 3, Lmax, d, C),
            "split 0 sizes the workspace for the default split");
    }
  check(parallax_decode_workspace_bytes(1, 1, 1024, 128, 100) == 0,
        "split not a multiple of 64 gives 0");
}

void prefill_rejections() {
  const char* fn = "parallax_prefill";
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 0, 1, 64, 64, 0.f, PLX_BF16,
                          nullptr, 0, nullptr), PLX_EINVAL, fn, "prefill B=0");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 0, 64, 0.f, PLX_BF16,
                          nullptr, 0, nullptr), PLX_EINVAL, fn, "prefill L=0");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 96, 0.f, PLX_BF16,
                          nullptr, 0, nullptr), PLX_EUNSUPPORTED, fn, "prefill d=96");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 64, 0.f, 7, nullptr, 0,
                          nullptr), PLX_EUNSUPPORTED, fn, "prefill dtype 7");
  expect(parallax_prefill(nullptr, P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 64, 0.f, PLX_BF16,
                          nullptr, 0, nullptr), PLX_EINVAL, fn, "prefill null q");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), nullptr, F(5), 1, 1, 64, 64, 0.f, PLX_F32,
                          nullptr, 0, nullptr), PLX_EINVAL, fn, "prefill null gate");
  const size_t need = parallax_prefill_workspace_bytes(2, 2, 100, 128, PLX_BF16);
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 2, 2, 100, 128, 0.f, PLX_BF16,
                          P(6), need - 1, nullptr), PLX_EINVAL, fn, "prefill workspace too small");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 65535, 65535, 1 << 20, 128, 0.f,
                          PLX_BF16, nullptr, 0, nullptr), PLX_EINVAL, fn, "prefill too large");
  expect(parallax_prefill_stage_v(nullptr, P(1), 1, 1, 64, 64, nullptr), PLX_EINVAL,
         "parallax_prefill_stage_v", "stage_v null v");
  expect(parallax_prefill_stage_v(P(0), P(1), 1, -2, 64, 64, nullptr), PLX_EINVAL,
         "parallax_prefill_stage_v", "stage_v H<0");
  expect(parallax_prefill_attend(P(0), P(1), P(2), P(3), F(4), nullptr, 1, 1, 64, 128, 0.f,
                                 nullptr), PLX_EINVAL, "parallax_prefill_attend",
         "attend null out");
  expect(parallax_prefill_attend(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 32, 0.f, nullptr),
         PLX_EUNSUPPORTED, "parallax_prefill_attend", "attend d=32");
}

void decode_rejections() {
  const char* fn = "parallax_decode";
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 1, 1, 0, 128, 0.f, PLX_BF16,
                         0, nullptr, 0, nullptr), PLX_EINVAL, fn, "decode Lmax=0");
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 300, 300, 64, 128, 0.f,
                         PLX_BF16, 0, nullptr, 0, nullptr), PLX_EINVAL, fn, "decode B*H > 65535");
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 1, 1, 64, 128, 0.f, PLX_BF16,
                         100, nullptr, 0, nullptr), PLX_EINVAL, fn, "decode split 100");
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 1, 1, 64, 128, 0.f, PLX_BF16,
                         -64, nullptr, 0, nullptr), PLX_EINVAL, fn, "decode split -64");
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), nullptr, 1, 1, 64, 128, 0.f,
                         PLX_BF16, 0, nullptr, 0, nullptr), PLX_EINVAL, fn, "decode null seqlens");
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 1, 1, 64, 128, 0.f, 3, 0,
                         nullptr, 0, nullptr), PLX_EUNSUPPORTED, fn, "decode dtype 3");
  const size_t need = parallax_decode_workspace_bytes(4, 2, 5000, 64, 512);
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 4, 2, 5000, 64, 0.f, PLX_BF16,
                         512, P(7), need - 4, nullptr), PLX_EINVAL, fn,
         "decode workspace too small");
  expect(parallax_decode_partials(P(0), P(1), P(2), P(3), I(4), F(5), 1, 1, 64, 64, 0.f,
                                  PLX_BF16, 0, nullptr), PLX_EINVAL, "parallax_decode_partials",
         "partials need an explicit split");
  expect(parallax_decode_combine(nullptr, F(1), I(2), F(3), 1, 1, 64, 64, 64, nullptr),
         PLX_EINVAL, "parallax_decode_combine", "combine null partials");
  expect(parallax_decode_combine(F(0), F(1), I(2), F(3), 1, 1, 64, 64, 96, nullptr), PLX_EINVAL,
         "parallax_decode_combine", "combine split 96");
}

// The softmax-only entry points share the Parallax calls' validation; they take
// no rho or gate.
void softmax_rejections() {
  const char* fp = "parallax_softmax_prefill";
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 0, 64, 64, 0.f, PLX_BF16, nullptr, 0,
                                  nullptr), PLX_EINVAL, fp, "softmax prefill H=0");
  expect(parallax_softmax_prefill(P(0), P(1), nullptr, F(3), 1, 1, 64, 64, 0.f, PLX_F32, nullptr,
                                  0, nullptr), PLX_EINVAL, fp, "softmax prefill null v");
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 1, 64, 256, 0.f, PLX_BF16, nullptr,
                                  0, nullptr), PLX_EUNSUPPORTED, fp, "softmax prefill d=256");
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 1, 64, 64, 0.f, 5, nullptr, 0,
                                  nullptr), PLX_EUNSUPPORTED, fp, "softmax prefill dtype 5");
  const size_t need = parallax_prefill_workspace_bytes(1, 2, 300, 64, PLX_BF16);
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 2, 300, 64, 0.f, PLX_BF16, P(4),
                                  need - 1, nullptr), PLX_EINVAL, fp,
         "softmax prefill workspace too small");
  expect(parallax_softmax_prefill_attend(P(0), P(1), nullptr, F(3), 1, 1, 64, 64, 0.f, nullptr),
         PLX_EINVAL, "parallax_softmax_prefill_attend", "softmax attend null vt16");
  expect(parallax_softmax_prefill_attend(P(0), P(1), P(2), F(3), 1, 1, -5, 64, 0.f, nullptr),
         PLX_EINVAL, "parallax_softmax_prefill_attend", "softmax attend L<0");
  const char* fd = "parallax_softmax_decode";
  expect(parallax_softmax_decode(P(0), P(1), P(2), F(3), nullptr, 1, 1, 64, 128, 0.f, PLX_BF16, 0,
                                 nullptr, 0, nullptr), PLX_EINVAL, fd, "softmax decode null seqlens");
  expect(parallax_softmax_decode(P(0), P(1), P(2), F(3), I(4), 1, 1, 64, 128, 0.f, PLX_BF16, 96,
                                 nullptr, 0, nullptr), PLX_EINVAL, fd, "softmax decode split 96");
  expect(parallax_softmax_decode(P(0), P(1), P(2), F(3), I(4), 65536, 1, 64, 128, 0.f, PLX_BF16, 0,
                                 nullptr, 0, nullptr), PLX_EINVAL, fd, "softmax decode B*H > 65535");
  const size_t dneed = parallax_decode_workspace_bytes(2, 2, 900, 128, 256);
  expect(parallax_softmax_decode(P(0), P(1), P(2), F(3), I(4), 2, 2, 900, 128, 0.f, PLX_F32, 256,
                                 P(5), dneed - 4, nullptr), PLX_EINVAL, fd,
         "softmax decode workspace too small");
}

// Training, backward and chunked-prefill entry points.
void training_and_chunk_rejections() {
  const char* ft = "parallax_prefill_train";
  expect(parallax_prefill_train(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), 1, 1, 64, 64,
                                0.f, PLX_F32, nullptr, 0, nullptr), PLX_EUNSUPPORTED, ft,
         "train fp32");
  expect(parallax_prefill_train(P(0), P(1), P(2), P(3), F(4), F(5), nullptr, F(7), F(8), 1, 1, 64,
                                64, 0.f, PLX_BF16, nullptr, 0, nullptr), PLX_EINVAL, ft,
         "train null lse");
  expect(parallax_prefill_train(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), 1, 1, 64, 96,
                                0.f, PLX_BF16, nullptr, 0, nullptr), PLX_EUNSUPPORTED, ft,
         "train d=96");
  const size_t tw = parallax_prefill_workspace_bytes(2, 1, 100, 64, PLX_BF16);
  expect(parallax_prefill_train(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), 2, 1, 100,
                                64, 0.f, PLX_BF16, P(9), tw - 1, nullptr), PLX_EINVAL, ft,
         "train workspace too small");
  const char* fb = "parallax_prefill_backward";
  check(parallax_prefill_backward_workspace_bytes(2, 3, 100, 128) > 0, "backward workspace > 0");
  check(parallax_prefill_backward_workspace_bytes(2, 3, 100, 80) == 0, "backward d=80 gives 0");
  check(parallax_prefill_backward_workspace_bytes(0, 3, 100, 64) == 0, "backward B=0 gives 0");
  expect(parallax_prefill_backward(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9),
                                   F(10), F(11), F(12), F(13), nullptr, 1, 1, 64, 64, 0.f,
                                   PLX_BF16, nullptr, 0, nullptr), PLX_EINVAL, fb,
         "backward null dgate");
  expect(parallax_prefill_backward(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9),
                                   F(10), F(11), F(12), F(13), F(14), 1, 1, 64, 64, 0.f, PLX_F32,
                                   nullptr, 0, nullptr), PLX_EUNSUPPORTED, fb, "backward fp32");
  const size_t bw = parallax_prefill_backward_workspace_bytes(1, 2, 70, 64);
  expect(parallax_prefill_backward(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9),
                                   F(10), F(11), F(12), F(13), F(14), 1, 2, 70, 64, 0.f,
                                   PLX_BF16, P(15), bw - 1, nullptr), PLX_EINVAL, fb,
         "backward workspace too small");
  const char* fc = "parallax_prefill_chunk";
  // 1 x 3 heads, 16-query chunks, 130 cache rows: no split when the split
  // covers the cache, else 3 splits of 64 keys for 8 query rows
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 65, 128, 192) ==
            ((parallax_prefill_workspace_bytes(2, 3, 130, 128, PLX_BF16) + 255) & ~(size_t)255),
        "chunk workspace = V^T tiles of the cache without a split");
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 65, 128, 64) ==
            ((parallax_prefill_workspace_bytes(2, 3, 130, 128, PLX_BF16) + 255) & ~(size_t)255) +
                (size_t)8 * 3 * 3 * (2 * 128 + 4) * 4,
        "chunk workspace adds T*H*S records of 2d+4 floats");
  // d = 128 chunks of at most 64 queries convert the V tiles in the kernel
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 16, 128, 192) == 0,
        "fused-V chunk workspace without a split");
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 32, 128, 192) == 0,
        "fused-V chunk workspace with two busy waves");
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 64, 128, 192) == 0,
        "fused-V chunk workspace with four busy waves");
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 16, 128, 64) ==
            (size_t)8 * 3 * 3 * (2 * 128 + 4) * 4,
        "fused-V chunk workspace = the split records");
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 16, 64, 192) ==
            ((parallax_prefill_workspace_bytes(2, 3, 130, 64, PLX_BF16) + 255) & ~(size_t)255),
        "d = 64 chunks stage V^T");
  check(parallax_prefill_chunk_vt_workspace_bytes(2, 3, 8, 130, 16, 128, 192) == 0,
        "chunk_vt workspace without a split");
  check(parallax_prefill_chunk_vt_workspace_bytes(2, 3, 8, 130, 16, 128, 64) ==
            (size_t)8 * 3 * 3 * (2 * 128 + 4) * 4,
        "chunk_vt workspace = the split records");
  check(parallax_prefill_chunk_workspace_bytes(2, 3, 8, 130, 16, 128, 100) == 0,
        "chunk workspace of a bad split size");
  // default split: one 16-query tile per head wants 512 workgroups, at least 4
  // tiles per split; 512 query tiles already fill the GPU
  check(parallax_prefill_chunk_default_split(1, 1, 8192, 16, 128) == 256, "default split, B*H=1");
  check(parallax_prefill_chunk_default_split(2, 16, 8192, 16, 128) == 512,
        "default split, B*H=32");
  check(parallax_prefill_chunk_default_split(32, 16, 8192, 16, 128) >= 8192,
        "no split for 512 query tiles");
  check(parallax_prefill_chunk_default_split(1, 1, 200, 16, 64) >= 200,
        "no split below 4 tiles of cache");
  check(parallax_prefill_chunk_default_split(0, 1, 200, 16, 64) == 0, "default split, B=0");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 0, 64, 8, 64,
                                0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EINVAL, fc, "chunk T=0");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 0, 64,
                                0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EINVAL, fc,
         "chunk max_q=0");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), nullptr, I(7), 1, 1, 8, 64, 8,
                                64, 0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EINVAL, fc,
         "chunk null cu_q");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8, 80,
                                0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EUNSUPPORTED, fc,
         "chunk d=80");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8, 64,
                                0.f, PLX_F32, 0, nullptr, 0, nullptr), PLX_EUNSUPPORTED, fc,
         "chunk fp32");
  expect(parallax_stage_v_rows(nullptr, P(1), I(2), I(3), 1, 1, 8, 64, 8, 64, nullptr), PLX_EINVAL,
         "parallax_stage_v_rows", "stage rows null vcache");
  expect(parallax_stage_v_rows(P(0), P(1), I(2), I(3), 1, 1, 0, 64, 8, 64, nullptr), PLX_EINVAL,
         "parallax_stage_v_rows", "stage rows T=0");
  expect(parallax_prefill_chunk_vt(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8,
                                   64, 0.f, PLX_F32, 0, nullptr, 0, nullptr), PLX_EUNSUPPORTED,
         "parallax_prefill_chunk_vt", "chunk_vt fp32");
  expect(parallax_prefill_chunk_vt(P(0), P(1), nullptr, P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64,
                                   8, 64, 0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EINVAL,
         "parallax_prefill_chunk_vt", "chunk_vt null vt_cache");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8, 64,
                                0.f, PLX_BF16, -64, nullptr, 0, nullptr), PLX_EINVAL, fc,
         "chunk negative split");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8, 64,
                                0.f, PLX_BF16, 96, nullptr, 0, nullptr), PLX_EINVAL, fc,
         "chunk split not a multiple of 64");
  expect(parallax_prefill_chunk_vt(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 640, 8,
                                   64, 0.f, PLX_BF16, 64, P(8), 1, nullptr), PLX_EINVAL,
         "parallax_prefill_chunk_vt", "chunk_vt split workspace too small");
  const size_t cw = parallax_prefill_chunk_workspace_bytes(2, 2, 40, 300, 20, 64, 0);
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 2, 2, 40, 300, 20,
                                64, 0.f, PLX_BF16, 0, P(8), cw - 1, nullptr), PLX_EINVAL, fc,
         "chunk workspace too small");
}

// Without a device, valid arguments reach the HIP runtime: the launch and
// allocation failures must be reported, not crash.
void no_device_failures() {
  const size_t ws = parallax_prefill_workspace_bytes(1, 1, 64, 64, PLX_BF16);
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 64, 0.f, PLX_BF16, P(6),
                          ws, nullptr), PLX_EHIP, "parallax_prefill", "prefill launch failure");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 64, 0.f, PLX_BF16,
                          nullptr, 0, nullptr), PLX_ENOMEM, "parallax_prefill",
         "prefill allocation failure");
  expect(parallax_prefill(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 64, 0.f, PLX_F32,
                          nullptr, 0, nullptr), PLX_EHIP, "parallax_prefill",
         "fp32 prefill launch failure");
  expect(parallax_prefill_stage_v(P(0), P(1), 1, 1, 64, 64, nullptr), PLX_EHIP,
         "parallax_prefill_stage_v", "stage_v launch failure");
  expect(parallax_prefill_attend(P(0), P(1), P(2), P(3), F(4), F(5), 1, 1, 64, 64, 0.f, nullptr),
         PLX_EHIP, "parallax_prefill_attend", "attend launch failure");
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 1, 1, 64, 128, 0.f, PLX_BF16,
                         0, nullptr, 0, nullptr), PLX_ENOMEM, "parallax_decode",
         "decode allocation failure");
  const size_t dws = parallax_decode_workspace_bytes(1, 1, 64, 128, 64);
  expect(parallax_decode(P(0), P(1), P(2), P(3), F(4), F(5), I(6), 1, 1, 64, 128, 0.f, PLX_BF16,
                         64, P(7), dws, nullptr), PLX_EHIP, "parallax_decode",
         "decode launch failure");
  expect(parallax_decode_partials(P(0), P(1), P(2), P(3), I(4), F(5), 1, 1, 64, 64, 0.f,
                                  PLX_F32, 64, nullptr), PLX_EHIP, "parallax_decode_partials",
         "partials launch failure");
  expect(parallax_decode_combine(F(0), F(1), I(2), F(3), 1, 1, 64, 64, 64, nullptr), PLX_EHIP,
         "parallax_decode_combine", "combine launch failure");
  // the softmax-only calls: null rho and gate are fine, the launch still fails
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 1, 64, 128, 0.f, PLX_BF16, P(6), ws * 2,
                                  nullptr), PLX_EHIP, "parallax_softmax_prefill",
         "softmax prefill launch failure");
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 1, 64, 64, 0.f, PLX_BF16, nullptr, 0,
                                  nullptr), PLX_ENOMEM, "parallax_softmax_prefill",
         "softmax prefill allocation failure");
  expect(parallax_softmax_prefill(P(0), P(1), P(2), F(3), 1, 1, 64, 64, 0.f, PLX_F32, nullptr, 0,
                                  nullptr), PLX_EHIP, "parallax_softmax_prefill",
         "softmax fp32 prefill launch failure");
  expect(parallax_softmax_prefill_attend(P(0), P(1), P(2), F(3), 1, 1, 64, 64, 0.f, nullptr),
         PLX_EHIP, "parallax_softmax_prefill_attend", "softmax attend launch failure");
  expect(parallax_softmax_decode(P(0), P(1), P(2), F(3), I(4), 1, 1, 64, 128, 0.f, PLX_F32, 64,
                                 P(7), dws, nullptr), PLX_EHIP, "parallax_softmax_decode",
         "softmax decode launch failure");
  expect(parallax_softmax_decode(P(0), P(1), P(2), F(3), I(4), 1, 1, 64, 128, 0.f, PLX_F32, 0,
                                 nullptr, 0, nullptr), PLX_ENOMEM, "parallax_softmax_decode",
         "softmax decode allocation failure");
  expect(parallax_prefill_train(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), 1, 1, 64, 64,
                                0.f, PLX_BF16, P(9), ws, nullptr), PLX_EHIP,
         "parallax_prefill_train", "train launch failure");
  const size_t bws = parallax_prefill_backward_workspace_bytes(1, 1, 64, 64);
  expect(parallax_prefill_backward(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9),
                                   F(10), F(11), F(12), F(13), F(14), 1, 1, 64, 64, 0.f,
                                   PLX_BF16, P(15), bws, nullptr), PLX_EHIP,
         "parallax_prefill_backward", "backward launch failure");
  expect(parallax_prefill_backward(P(0), P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), F(9),
                                   F(10), F(11), F(12), F(13), F(14), 1, 1, 64, 64, 0.f,
                                   PLX_BF16, nullptr, 0, nullptr), PLX_ENOMEM,
         "parallax_prefill_backward", "backward allocation failure");
  const size_t cws = parallax_prefill_chunk_workspace_bytes(1, 1, 8, 64, 8, 64, 0);
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8, 64,
                                0.f, PLX_BF16, 0, P(8), cws, nullptr), PLX_EHIP,
         "parallax_prefill_chunk", "chunk launch failure");
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8, 64,
                                0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_ENOMEM,
         "parallax_prefill_chunk", "chunk allocation failure");
  // fused V at d = 128 without a split needs no workspace: straight to the launch
  expect(parallax_prefill_chunk(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8,
                                128, 0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EHIP,
         "parallax_prefill_chunk", "fused-V chunk launch failure");
  expect(parallax_stage_v_rows(P(0), P(1), I(2), I(3), 1, 1, 8, 64, 8, 64, nullptr), PLX_EHIP,
         "parallax_stage_v_rows", "stage rows launch failure");
  expect(parallax_prefill_chunk_vt(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 64, 8,
                                   64, 0.f, PLX_BF16, 0, nullptr, 0, nullptr), PLX_EHIP,
         "parallax_prefill_chunk_vt", "chunk_vt launch failure");
  expect(parallax_prefill_chunk_vt(P(0), P(1), P(2), P(3), F(4), F(5), I(6), I(7), 1, 1, 8, 640, 8,
                                   64, 0.f, PLX_BF16, 64, nullptr, 0, nullptr), PLX_ENOMEM,
         "parallax_prefill_chunk_vt", "chunk_vt split allocation failure");
}

void error_text_is_per_thread() {
  expect(parallax_prefill_stage_v(nullptr, P(1), 1, 1, 64, 64, nullptr), PLX_EINVAL,
         "parallax_prefill_stage_v", "error on the main thread");
  std::string other = "unset";
  std::thread t([&] { other = parallax_last_error(); });
  t.join();
  check(other.empty(), "another thread does not see this thread's error text");
  check(std::strlen(parallax_last_error()) > 0, "this thread keeps its error text");
}

}  // namespace

int main() {
  check(parallax_abi_version() == PARALLAX_ABI_VERSION, "ABI version");
  workspace_sizes();
  prefill_rejections();
  decode_rejections();
  softmax_rejections();
  training_and_chunk_rejections();
  error_text_is_per_thread();
  int n_dev = 0;
  if (hipGetDeviceCount(&n_dev) != hipSuccess) n_dev = 0;
  if (n_dev == 0) no_device_failures();
  else std::printf("a device is present: the no-device failure checks are skipped\n");
  std::printf("%d failed\n", g_failed);
  return g_failed;
}
