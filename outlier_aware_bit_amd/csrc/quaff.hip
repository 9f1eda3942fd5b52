// Quaff kernels of libqlin (gfx950):
//   qlin_momentum_update    targeted momentum scaling on the fixed outlier set O
//   qlin_weight_row_absmax  max_n |W_O[o, n]| for beta
//   qlin_outlier_comp       the sparse compensation term added to Y
//
// Source: "Quaff: Quantized Parameter-Efficient Fine-Tuning under Outlier
// Spatial Stability Hypothesis" (paper notes), "key design".
#include "common.hpp"
#include "comp.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

constexpr int kMomThreads = 256;

// One workgroup per outlier channel O[j]: c = max_m |x[m, O[j]]|, then
// beta = max(1, sqrt(c / wmax)), s = gamma*s + (1-gamma)*beta, r = 1/s.  The
// same workgroup writes r = 1/s for the channels between O[j-1] and O[j]
// (and after the last one), so r covers every channel in one launch.
__global__ __launch_bounds__(kMomThreads) void momentum_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int32_t* __restrict__ O, int nO,
    const float* __restrict__ wmax, float gamma, float* __restrict__ s, float* __restrict__ r) {
  __shared__ float red[kMomThreads / 64];
  const int j = blockIdx.x;
  const int o = O[j];
  const bool valid = (o >= 0 && o < K);
  float c = 0.0f;
  if (valid) {
    // Eight rows per thread per pass, all loads issued before the reduction.
    constexpr int R = 8;
    const uint16_t* col = x + o + static_cast<int64_t>(threadIdx.x) * K;
    const int64_t step = static_cast<int64_t>(kMomThreads) * K;
    for (int64_t base = threadIdx.x; base < M; base += static_cast<int64_t>(kMomThreads) * R) {
      uint16_t v[R];
#pragma unroll
      for (int i = 0; i < R; ++i) v[i] = (base + i * kMomThreads < M) ? col[i * step] : static_cast<uint16_t>(0);
#pragma unroll
      for (int i = 0; i < R; ++i) c = fmaxf(c, fabsf(h2f(v[i])));
      col += R * step;
    }
  }
  c = block_max<kMomThreads / 64>(c, red);
  if (threadIdx.x == 0 && valid) {
    const float w = wmax[j];
    float beta = 1.0f;
    if (w != 0.0f) beta = fmaxf(1.0f, sqrt_rn(div_rn(c, w)));
    const float g1 = sub_rn(1.0f, gamma);
    const float sn = add_rn(mul_rn(gamma, s[o]), mul_rn(g1, beta));
    s[o] = sn;
    r[o] = div_rn(1.0f, sn);
  }
  // Channels strictly between the previous outlier and this one.
  int64_t lo = (j == 0) ? 0 : static_cast<int64_t>(O[j - 1]) + 1;
  int64_t hi = static_cast<int64_t>(o);
  lo = lo < 0 ? 0 : (lo > K ? K : lo);
  hi = hi < 0 ? 0 : (hi > K ? K : hi);
  for (int64_t k = lo + threadIdx.x; k < hi; k += kMomThreads) r[k] = div_rn(1.0f, s[k]);
  if (j == nO - 1) {
    int64_t t0 = static_cast<int64_t>(o) + 1;
    t0 = t0 < 0 ? 0 : (t0 > K ? K : t0);
    for (int64_t k = t0 + threadIdx.x; k < K; k += kMomThreads) r[k] = div_rn(1.0f, s[k]);
  }
}

__global__ __launch_bounds__(kMomThreads) void reciprocal_kernel(const float* __restrict__ s,
                                                                 float* __restrict__ r, int64_t K) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * kMomThreads + threadIdx.x;
  if (k < K) r[k] = div_rn(1.0f, s[k]);
}

__global__ __launch_bounds__(kMomThreads) void row_absmax_kernel(const uint16_t* __restrict__ w,
                                                                 int64_t N, float* __restrict__ out) {
  __shared__ float red[kMomThreads / 64];
  const int64_t i = blockIdx.x;
  const uint16_t* row = w + i * N;
  float a = 0.0f;
  for (int64_t c = threadIdx.x; c < N / 8; c += kMomThreads) {
    const uint4 raw = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t v[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a = fmaxf(a, fabsf(h2f(static_cast<uint16_t>(v[q] & 0xffffu))));
      a = fmaxf(a, fabsf(h2f(static_cast<uint16_t>(v[q] >> 16))));
    }
  }
  a = block_max<kMomThreads / 64>(a, red);
  if (threadIdx.x == 0) out[i] = a;
}

// Standalone compensation: y = fp16(y + sa * sum_j xO[m,j] * WO[j,n]) on
// 128 x 256 tiles, four waves of 128 x 64 (no LDS: both operands arrive in
// fragment order).
constexpr int kCompTM = 4, kCompThreads = 256;

__global__ __launch_bounds__(kCompThreads) void outlier_comp_kernel(
    const uint16_t* __restrict__ xO, int ldO, const float* __restrict__ sa,
    const uint8_t* __restrict__ WOp, int64_t M, int64_t N, uint16_t* __restrict__ y) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32 * kCompTM;
  const int64_t wcol0 = static_cast<int64_t>(blockIdx.x) * 256 + 64 * wave;
  if (wcol0 >= N) return;
  v16f f[kCompTM][2];
#pragma unroll
  for (int a = 0; a < kCompTM; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) f[a][b] = v16f{};
  comp_accumulate<kCompTM, 2>(f, xO, ldO, WOp, M, N, m0, wcol0 / 32);
  // Lane l holds row (l & 31) and runs of four adjacent columns: 8-byte
  // read-modify-write of y per run.
#pragma unroll
  for (int tm = 0; tm < kCompTM; ++tm) {
    const int64_t m = m0 + 32 * tm + (lane & 31);
    if (m >= M) continue;
    const float sam = sa[m];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2* p = reinterpret_cast<uint2*>(y + m * N + wcol0 + 32 * nt + 8 * q + 4 * (lane >> 5));
        const uint2 old = *p;
        const uint16_t in[4] = {static_cast<uint16_t>(old.x & 0xffffu), static_cast<uint16_t>(old.x >> 16),
                                static_cast<uint16_t>(old.y & 0xffffu), static_cast<uint16_t>(old.y >> 16)};
        uint16_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = f2h(h2f(in[j]) + sam * f[tm][nt][4 * q + j]);
        *p = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
      }
  }
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_momentum_update(const uint16_t* x, int64_t M, int64_t K,
                                            const int32_t* O, int32_t nO, const float* wmax_O,
                                            float gamma, float* s, float* r, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  QLIN_REQUIRE(gamma >= 0.0f && gamma <= 1.0f, QLIN_ERR_INVALID_ARG, "gamma=%g must be in [0, 1]", (double)gamma);
  QLIN_PTR(s);
  QLIN_PTR(r);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_PTR(wmax_O);
    if (M > 0) QLIN_PTR(x);
    momentum_kernel<<<dim3(nO), kMomThreads, 0, as_stream(stream)>>>(x, M, K, O, nO, wmax_O, gamma, s, r);
  } else {
    reciprocal_kernel<<<dim3(static_cast<unsigned>((K + kMomThreads - 1) / kMomThreads)), kMomThreads, 0,
                        as_stream(stream)>>>(s, r, K);
  }
  QLIN_LAUNCH_CHECK("momentum_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_weight_row_absmax(const uint16_t* w_rows, int64_t R, int64_t N,
                                              float* out, void* stream) {
  QLIN_REQUIRE(R >= 0, QLIN_ERR_INVALID_ARG, "R=%lld is negative", (long long)R);
  QLIN_REQUIRE(N > 0 && N % 64 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 64", (long long)N);
  if (R == 0) return QLIN_OK;
  QLIN_PTR(w_rows);
  QLIN_PTR(out);
  QLIN_REQUIRE(R <= 0x7fffffffLL, QLIN_ERR_SHAPE, "R too large");
  row_absmax_kernel<<<dim3(static_cast<unsigned>(R)), kMomThreads, 0, as_stream(stream)>>>(w_rows, N, out);
  QLIN_LAUNCH_CHECK("row_absmax_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_outlier_comp(const uint16_t* xO, const float* sa, int32_t nO,
                                         const void* WO, int64_t M, int64_t N, uint16_t* y,
                                         void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(N > 0 && N % 64 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 64", (long long)N);
  QLIN_REQUIRE(nO >= 0, QLIN_ERR_INVALID_ARG, "nO=%d is negative", nO);
  if (M == 0 || nO == 0) return QLIN_OK;
  QLIN_PTR(xO);
  QLIN_PTR(sa);
  QLIN_PTR(WO);
  QLIN_PTR(y);
  const int64_t gy = (M + 32 * kCompTM - 1) / (32 * kCompTM);
  QLIN_REQUIRE(gy <= 65535, QLIN_ERR_SHAPE, "M too large");
  const dim3 grid(static_cast<unsigned>((N + 255) / 256), static_cast<unsigned>(gy));
  outlier_comp_kernel<<<grid, kCompThreads, 0, as_stream(stream)>>>(
      xO, static_cast<int>(outlier_ld(nO)), sa, static_cast<const uint8_t*>(WO), M, N, y);
  QLIN_LAUNCH_CHECK("outlier_comp_kernel");
  return QLIN_OK;
}
