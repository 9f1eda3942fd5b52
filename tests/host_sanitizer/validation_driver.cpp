// Host-side validation of every libqlin entry point, for a build of the
// library's host code with AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Each call either fails validation (a non-zero status, nothing launched) or
// is an empty batch that returns QLIN_OK before any HIP call.  Pointers are
// made-up addresses that are never dereferenced on the host.  Sizes far
// beyond memory check that the size arithmetic rejects them instead of
// overflowing.  The driver refuses to run when a GPU is visible: it is a test
// of host code only.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qlin.h"

namespace {

int g_failures = 0;
int g_calls = 0;

void expect(const char* what, qlin_status got, qlin_status want) {
  ++g_calls;
  const char* msg = qlin_last_error();
  const size_t len = strlen(msg);  // the message must be a terminated string
  if (got != want) {
    ++g_failures;
    printf("FAIL %s: got %s, want %s (%s)\n", what, qlin_status_string(got), qlin_status_string(want), msg);
  } else if (got != QLIN_OK && len == 0) {
    ++g_failures;
    printf("FAIL %s: %s without a message\n", what, qlin_status_string(got));
  }
}

template <class T>
T* at(uintptr_t a) {
  return reinterpret_cast<T*>(a);
}

constexpr uintptr_t kA = 0x10000, kB = 0x20000, kMis = 0x10008;
constexpr int64_t kHuge = int64_t(1) << 40;     // a multiple of 128, far beyond memory
constexpr int64_t kHuger = int64_t(1) << 62;    // products and roundings overflow int64

#define EXPECT(call, want) expect(#call, (call), (want))

void status_and_sizes() {
  if (qlin_abi_version() != QLIN_ABI_VERSION) {
    ++g_failures;
    printf("FAIL abi version %d\n", qlin_abi_version());
  }
  for (int s = -1; s <= 6; ++s)
    if (strlen(qlin_status_string(static_cast<qlin_status>(s))) == 0) ++g_failures;
  const int32_t lds[][2] = {{-5, 0}, {0, 0}, {1, 16}, {16, 16}, {17, 32}, {205, 208}};
  for (auto& c : lds)
    if (qlin_outlier_ld(c[0]) != c[1]) {
      ++g_failures;
      printf("FAIL qlin_outlier_ld(%d) = %d\n", c[0], qlin_outlier_ld(c[0]));
    }
  // Sizes: plain cases, invalid shapes, and products past int64.
  struct P { int32_t layout; int64_t K, N; size_t want; };
  const P ps[] = {
      {QLIN_LAYOUT_W8, 256, 128, 256 * 128},     {QLIN_LAYOUT_W4S, 256, 128, 256 * 64},
      {QLIN_LAYOUT_W4U, 256, 128, 256 * 64},     {QLIN_LAYOUT_WO, 205, 128, 208 * 128 * 2},
      {QLIN_LAYOUT_W8T, 128, 256, 128 * 256},    {QLIN_LAYOUT_W8, 100, 128, 0},
      {QLIN_LAYOUT_W8, 256, 100, 0},             {9, 256, 128, 0},
      {QLIN_LAYOUT_W8, kHuge, kHuge, 0},         {QLIN_LAYOUT_W4S, kHuge, kHuge, 0},
      {QLIN_LAYOUT_WO, kHuger, 128, 0},          {QLIN_LAYOUT_W8T, kHuge, kHuge, 0},
      {QLIN_LAYOUT_W8, INT64_MAX - 127, 128, 0}, {QLIN_LAYOUT_W8, -128, 128, 0},
  };
  for (const P& p : ps) {
    const size_t got = qlin_packed_bytes(p.layout, p.K, p.N);
    if (got != p.want) {
      ++g_failures;
      printf("FAIL qlin_packed_bytes(%d, %lld, %lld) = %zu, want %zu\n", p.layout, (long long)p.K,
             (long long)p.N, got, p.want);
    }
  }
  if (qlin_momentum_work_bytes(2048, 205) != 16 * 205 * 4 || qlin_momentum_work_bytes(-1, 5) != 0 ||
      qlin_momentum_work_bytes(kHuger, INT32_MAX) != size_t(16) * INT32_MAX * 4) {
    ++g_failures;
    printf("FAIL qlin_momentum_work_bytes\n");
  }
}

void activations() {
  auto qa = [](const uint16_t* x, int64_t M, int64_t K, const float* r, const int32_t* O, int32_t nO,
               const float* s, int8_t* qO, uint16_t* xO) {
    return qlin_quant_act(x, M, K, r, at<int8_t>(kB), at<float>(kA), O, nO, s, qO, xO, nullptr);
  };
  const uint16_t* x = at<uint16_t>(kA);
  EXPECT(qa(nullptr, 4, 256, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qa(x, 4, 200, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qa(x, -1, 256, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qa(at<uint16_t>(kMis), 4, 256, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_ALIGN);
  EXPECT(qa(x, 4, 256, at<float>(kMis), nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_ALIGN);
  EXPECT(qa(x, 4, 256, nullptr, at<int32_t>(kA), 0, nullptr, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qa(x, 4, 256, nullptr, at<int32_t>(kA), 3, nullptr, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qa(x, 4, 256, nullptr, at<int32_t>(kA), 3, nullptr, nullptr, at<uint16_t>(kB)), QLIN_ERR_INVALID_ARG);
  EXPECT(qa(x, 4, 256, nullptr, at<int32_t>(kA), 300, nullptr, at<int8_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qa(x, kHuger, 256, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qa(x, kHuge, kHuge, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qa(x, 0, 256, nullptr, nullptr, 0, nullptr, nullptr, nullptr), QLIN_OK);

  for (int grouped = 0; grouped < 2; ++grouped) {
    auto h = [grouped](const uint16_t* x, int64_t M, int64_t K, const int8_t* d, int32_t block, const float* t) {
      auto f = grouped ? qlin_hadamard_offset_group : qlin_hadamard_offset;
      return f(x, M, K, d, block, at<uint8_t>(kA), at<float>(kA), at<int32_t>(kA), at<int32_t>(kA),
               const_cast<float*>(t), nullptr);
    };
    const int8_t* d = at<int8_t>(kB);
    EXPECT(h(x, 4, 256, d, 64, nullptr), QLIN_ERR_UNSUPPORTED);
    EXPECT(h(x, 4, 192, d, 128, nullptr), QLIN_ERR_SHAPE);
    EXPECT(h(x, 4, 256, nullptr, 128, nullptr), QLIN_ERR_INVALID_ARG);
    EXPECT(h(x, 4, 256, d, 128, at<float>(kMis)), QLIN_ERR_ALIGN);
    EXPECT(h(x, kHuger, 256, d, 128, nullptr), QLIN_ERR_SHAPE);
    EXPECT(h(x, kHuge, kHuge, d, 128, nullptr), QLIN_ERR_SHAPE);
    EXPECT(h(x, 0, 256, d, 128, nullptr), QLIN_OK);
  }
}

void momentum() {
  const uint16_t* x = at<uint16_t>(kA);
  const int32_t* O = at<int32_t>(kA);
  const float* wm = at<float>(kA);
  float* s = at<float>(kA);
  float* r = at<float>(kB);
  EXPECT(qlin_momentum_update(x, 8, 256, O, 4, wm, 1.5f, s, r, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_momentum_update(x, 8, 256, O, 4, wm, -0.0f / 0.0f, s, r, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_momentum_update(x, 8, 256, O, 400, wm, 0.9f, s, r, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_momentum_update(x, 8, 256, nullptr, 4, wm, 0.9f, s, r, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_momentum_update(x, 8, 256, O, 4, wm, 0.9f, nullptr, r, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_momentum_update(x, -2, 256, O, 4, wm, 0.9f, s, r, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_momentum_update(x, 8, 256, O, 4, wm, 0.9f, s, r, at<float>(kA + 4), nullptr), QLIN_ERR_ALIGN);
  EXPECT(qlin_momentum_update(x, kHuger, 256, O, 4, wm, 0.9f, s, r, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_momentum_update(x, kHuge, kHuge, O, 4, wm, 0.9f, s, r, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_momentum_update_noalloc(x, 8, 256, O, 8193, wm, 0.9f, s, r, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_momentum_update_noalloc(x, 8, 256, O, 4, wm, 1.5f, s, r, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_momentum_update_noalloc(x, kHuger, 256, O, 4, wm, 0.9f, s, r, nullptr), QLIN_ERR_SHAPE);
  // The momentum update and the quantization in one call.
  int8_t* q = at<int8_t>(kA);
  float* sc = at<float>(kB);
  uint16_t* xO = at<uint16_t>(kA);
  auto mq = [&](int64_t M, int64_t K, int32_t nO, float gamma, float* work, uint16_t* xo) {
    return qlin_quaff_momentum_quant(x, M, K, O, nO, wm, gamma, s, r, work, q, sc, xo, nullptr);
  };
  EXPECT(mq(8, 256, 4, 1.5f, nullptr, xO), QLIN_ERR_INVALID_ARG);
  EXPECT(mq(8, 256, 400, 0.9f, nullptr, xO), QLIN_ERR_SHAPE);
  EXPECT(mq(8, 200, 4, 0.9f, nullptr, xO), QLIN_ERR_SHAPE);
  EXPECT(mq(-1, 256, 4, 0.9f, nullptr, xO), QLIN_ERR_INVALID_ARG);
  EXPECT(mq(8, 256, 4, 0.9f, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(mq(8, 256, 4, 0.9f, at<float>(kA + 4), xO), QLIN_ERR_ALIGN);
  EXPECT(mq(kHuger, 256, 4, 0.9f, nullptr, xO), QLIN_ERR_SHAPE);
  EXPECT(mq(kHuge, kHuge, 4, 0.9f, nullptr, xO), QLIN_ERR_SHAPE);
  if (qlin_quaff_momentum_quant_work_bytes(128, 205) != 5 * 205 * 4 ||
      qlin_quaff_momentum_quant_work_bytes(2048, 205) != 16 * 205 * 4 ||
      qlin_quaff_momentum_quant_work_bytes(-1, 7) != 0 || qlin_quaff_momentum_quant_work_bytes(kHuger, 7) != 16 * 7 * 4) {
    ++g_failures;
    printf("FAIL qlin_quaff_momentum_quant_work_bytes\n");
  }
}

void weights() {
  const uint16_t* w = at<uint16_t>(kA);
  EXPECT(qlin_quant_weight_sym(w, 256, 128, 3, at<int8_t>(kA), at<uint16_t>(kB), nullptr), QLIN_ERR_UNSUPPORTED);
  EXPECT(qlin_quant_weight_sym(w, 256, 100, 8, at<int8_t>(kA), at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_quant_weight_sym(w, kHuge, kHuge, 8, at<int8_t>(kA), at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_quant_weight_group(w, 256, 128, 64, at<int8_t>(kA), at<uint16_t>(kB), at<uint16_t>(kA),
                                 at<uint16_t>(kB), nullptr),
         QLIN_ERR_UNSUPPORTED);
  EXPECT(qlin_quant_weight_group(w, kHuge, kHuge, 128, at<int8_t>(kA), at<uint16_t>(kB), at<uint16_t>(kA),
                                 at<uint16_t>(kB), nullptr),
         QLIN_ERR_SHAPE);
  EXPECT(qlin_quant_weight_offq(w, 256, 128, nullptr, 128, at<uint8_t>(kA), at<float>(kB), at<int32_t>(kA),
                                at<int32_t>(kB), nullptr),
         QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_quant_weight_offq(w, kHuge, kHuge, at<int8_t>(kA), 128, at<uint8_t>(kA), at<float>(kB),
                                at<int32_t>(kA), at<int32_t>(kB), nullptr),
         QLIN_ERR_SHAPE);
  EXPECT(qlin_pack_weight(9, at<void>(kA), 256, 128, at<void>(kB), nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_pack_weight(QLIN_LAYOUT_W8, at<void>(kA), 256, 128, at<void>(kMis), nullptr), QLIN_ERR_ALIGN);
  EXPECT(qlin_pack_weight(QLIN_LAYOUT_WO, at<void>(kA), 0, 128, at<void>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pack_weight(QLIN_LAYOUT_W8T, at<void>(kA), 128, 200, at<void>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pack_weight(QLIN_LAYOUT_W8, at<void>(kA), kHuge, kHuge, at<void>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pack_weight(QLIN_LAYOUT_WO, at<void>(kA), kHuger, 128, at<void>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_weight_row_absmax(w, 0, 128, nullptr, nullptr), QLIN_OK);
  EXPECT(qlin_weight_row_absmax(w, kHuge, kHuge, at<float>(kA), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_weight_colsum_group(at<uint8_t>(kA), 256, 128, 64, at<int32_t>(kA), nullptr), QLIN_ERR_UNSUPPORTED);
  EXPECT(qlin_weight_colsum_group(at<uint8_t>(kA), 200, 128, 128, at<int32_t>(kA), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_weight_colsum_group(at<uint8_t>(kA), 256, 128, 128, at<int32_t>(kMis), nullptr), QLIN_ERR_ALIGN);
  EXPECT(qlin_weight_colsum_group(at<uint8_t>(kA), kHuge, kHuge, 128, at<int32_t>(kA), nullptr), QLIN_ERR_SHAPE);
}

void gemms() {
  const int8_t* qa = at<int8_t>(kA);
  const float* sa = at<float>(kA);
  const void* w = at<void>(kB);
  const uint16_t* sw = at<uint16_t>(kA);
  uint16_t* y = at<uint16_t>(kA);
  auto w8 = [&](int64_t M, int64_t N, int64_t K, const uint16_t* xO, int32_t nO, const void* WO, int32_t* acc) {
    return qlin_gemm_w8a8(qa, sa, w, sw, M, N, K, xO, nO, WO, y, acc, nullptr);
  };
  EXPECT(w8(16, 100, 256, nullptr, 0, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(w8(16, 128, 250, nullptr, 0, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_gemm_w8a8(nullptr, sa, w, sw, 16, 128, 256, nullptr, 0, nullptr, y, nullptr, nullptr),
         QLIN_ERR_INVALID_ARG);
  EXPECT(w8(16, 128, 256, at<uint16_t>(kA), 5, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(w8(16, 128, 256, at<uint16_t>(kA), 0, nullptr, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(w8(16, 128, 256, nullptr, 300, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(w8(16, 128, 256, nullptr, 0, nullptr, at<int32_t>(kMis)), QLIN_ERR_ALIGN);
  EXPECT(w8(kHuger, 128, 256, nullptr, 0, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(w8(kHuge, kHuge, kHuge, nullptr, 0, nullptr, nullptr), QLIN_ERR_SHAPE);
  EXPECT(w8(0, 128, 256, nullptr, 0, nullptr, nullptr), QLIN_OK);

  auto w4 = [&](const uint16_t* ratio, int32_t group, int64_t M, int64_t N, int64_t K) {
    return qlin_gemm_w4a8(qa, sa, w, sw, ratio, group, M, N, K, y, nullptr, nullptr, nullptr);
  };
  EXPECT(w4(nullptr, 64, 16, 128, 256), QLIN_ERR_UNSUPPORTED);
  EXPECT(w4(nullptr, 128, 16, 128, 256), QLIN_ERR_INVALID_ARG);
  EXPECT(w4(at<uint16_t>(kA), 0, 16, 128, 256), QLIN_ERR_INVALID_ARG);
  EXPECT(w4(nullptr, 0, kHuger, 128, 256), QLIN_ERR_SHAPE);
  EXPECT(w4(nullptr, 0, kHuge, kHuge, kHuge), QLIN_ERR_SHAPE);
  EXPECT(w4(nullptr, 0, 0, 128, 256), QLIN_OK);
  EXPECT(qlin_gemm_w4a8(qa, sa, w, sw, at<uint16_t>(kA), 128, 256, 128, 256, y, nullptr, at<void>(kMis), nullptr),
         QLIN_ERR_ALIGN);
  if (qlin_gemm_w4a8_work_bytes(4096, 4096, 11008, 128) != size_t(4096) * 11008 ||
      qlin_gemm_w4a8_work_bytes(128, 4096, 11008, 128) != 0 || qlin_gemm_w4a8_work_bytes(kHuger, 4096, 256, 128) != 0 ||
      qlin_gemm_w4a8_work_bytes(kHuge, kHuge, kHuge, 128) != 0) {
    ++g_failures;
    printf("FAIL qlin_gemm_w4a8_work_bytes\n");
  }

  for (int grouped = 0; grouped < 2; ++grouped) {
    auto f = grouped ? qlin_gemm_w4a4_group : qlin_gemm_w4a4;
    auto w44 = [&](const int32_t* cs, int64_t M, int64_t N, int64_t K, int32_t* acc) {
      return f(at<uint8_t>(kA), sa, at<int32_t>(kA), at<int32_t>(kA), w, at<float>(kA), at<int32_t>(kA), cs, M, N,
               K, y, acc, nullptr);
    };
    const int32_t* cs = at<int32_t>(kA);
    EXPECT(w44(nullptr, 16, 128, 256, nullptr), QLIN_ERR_INVALID_ARG);
    EXPECT(w44(cs, 16, 100, 256, nullptr), QLIN_ERR_SHAPE);
    EXPECT(w44(cs, 16, 128, 256, at<int32_t>(kA + 4)), QLIN_ERR_ALIGN);
    EXPECT(w44(cs, kHuger, 128, 256, nullptr), QLIN_ERR_SHAPE);
    EXPECT(w44(cs, kHuge, kHuge, kHuge, nullptr), QLIN_ERR_SHAPE);
    EXPECT(w44(cs, 0, 128, 256, nullptr), QLIN_OK);
  }

  EXPECT(qlin_outlier_comp(at<uint16_t>(kA), sa, 4, w, 16, 100, y, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_outlier_comp(nullptr, sa, 4, w, 16, 128, y, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_outlier_comp(at<uint16_t>(kA), sa, 4, at<void>(kMis), 16, 128, y, nullptr), QLIN_ERR_ALIGN);
  EXPECT(qlin_outlier_comp(at<uint16_t>(kA), sa, 4, w, kHuger, 128, y, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_outlier_comp(at<uint16_t>(kA), sa, 4, w, kHuge, kHuge, y, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_outlier_comp(at<uint16_t>(kA), sa, 0, w, 16, 128, y, nullptr), QLIN_OK);
}

void backward() {
  auto bw = [](int64_t M, int64_t N, int64_t K, const int32_t* O, int32_t nO, const uint16_t* wo, uint16_t* dx) {
    return qlin_quaff_backward(at<uint16_t>(kA), M, N, K, at<uint16_t>(kA), at<void>(kB), at<float>(kA),
                               at<float>(kA), O, nO, wo, at<int8_t>(kA), at<float>(kA), at<float>(kA), dx, nullptr,
                               nullptr);
  };
  const int32_t* O = at<int32_t>(kA);
  uint16_t* dx = at<uint16_t>(kA);
  EXPECT(bw(8, 192, 128, O, 3, at<uint16_t>(kA), dx), QLIN_ERR_SHAPE);
  EXPECT(bw(8, 256, 192, O, 3, at<uint16_t>(kA), dx), QLIN_ERR_SHAPE);
  EXPECT(bw(8, 256, 128, O, 200, at<uint16_t>(kA), dx), QLIN_ERR_SHAPE);
  EXPECT(bw(8, 256, 128, O, 3, nullptr, dx), QLIN_ERR_INVALID_ARG);
  EXPECT(bw(8, 256, 128, O, 3, at<uint16_t>(kA), at<uint16_t>(kMis)), QLIN_ERR_ALIGN);
  EXPECT(bw(kHuger, 256, 128, O, 3, at<uint16_t>(kA), dx), QLIN_ERR_SHAPE);
  EXPECT(bw(kHuge, kHuge, kHuge, O, 3, at<uint16_t>(kA), dx), QLIN_ERR_SHAPE);
  EXPECT(bw(0, 256, 128, O, 3, at<uint16_t>(kA), dx), QLIN_OK);
}

void pca() {
  const uint16_t* x = at<uint16_t>(kA);
  EXPECT(qlin_pca_select(x, 4, 16, 100, at<int32_t>(kA), at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_select(x, 4, 0, 128, at<int32_t>(kA), at<uint16_t>(kB), nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_pca_select(x, 4, 16, 128, nullptr, at<uint16_t>(kB), nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_pca_select(x, kHuge, kHuge, kHuge, at<int32_t>(kA), at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_select(x, 0, 16, 128, at<int32_t>(kA), at<uint16_t>(kB), nullptr), QLIN_OK);
  double* d = at<double>(kA);
  EXPECT(qlin_pca_leading_eigvec(x, 1, 128, 10, 1e-9, d, d, at<int32_t>(kA), d, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_leading_eigvec(x, 8, 128, 0, 1e-9, d, d, at<int32_t>(kA), d, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_pca_leading_eigvec(x, 8, 128, 10, -1.0, d, d, at<int32_t>(kA), d, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_pca_leading_eigvec(x, 8, 128, 10, 1e-9, d, d, at<int32_t>(kA), at<double>(kMis), nullptr),
         QLIN_ERR_ALIGN);
  EXPECT(qlin_pca_leading_eigvec(x, 8, 16384, 10, 1e-9, d, d, at<int32_t>(kA), d, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_leading_eigvec(x, kHuger, 128, 10, 1e-9, d, d, at<int32_t>(kA), d, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_fold_weight(x, 70000, 64, d, at<uint16_t>(kB), d, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_fold_weight(x, 128, 60, d, at<uint16_t>(kB), d, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_fold_weight(x, 128, 64, nullptr, at<uint16_t>(kB), d, nullptr), QLIN_ERR_INVALID_ARG);
  EXPECT(qlin_pca_fold_weight(x, 128, kHuger, d, at<uint16_t>(kB), d, nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_rotate(x, 4, 100, d, at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_rotate(x, 4, 0, d, at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_rotate(x, kHuger, 128, d, at<uint16_t>(kB), nullptr), QLIN_ERR_SHAPE);
  EXPECT(qlin_pca_rotate(x, 0, 128, d, at<uint16_t>(kB), nullptr), QLIN_OK);
}

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    printf("SKIP: a GPU is visible; this driver checks host code only\n");
    return 77;
  }
  status_and_sizes();
  activations();
  momentum();
  weights();
  gemms();
  backward();
  pca();
  printf("%d calls, %d failures\n", g_calls, g_failures);
  return g_failures == 0 ? 0 : 1;
}
