// OffQ's concentration step, Top-1 PCA, as offline kernels of libqlin (gfx950):
//   qlin_pca_select           per calibration sequence, the token with the largest max |x|
//   qlin_pca_leading_eigvec   leading eigenvector of the extreme tokens' covariance
//   qlin_pca_fold_weight      W <- H W for the Householder reflection H with H v = e_0
//   qlin_pca_rotate           x <- x H (the activation side of the same rotation)
//
// Source: "OffQ: Taming Structured Outliers in LLM Quantization by Offsetting",
// methodology, "concentration via Top-1 PCA".  The calibration step runs once
// per layer; these kernels favour a fixed summation order (results that do
// not depend on timing) over speed.
#include "common.hpp"

namespace qlin {
namespace {

constexpr int kSelThreads = 256;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One workgroup per sequence: wave w scans tokens w, w + 4, ...; the largest
// max|x| wins, the first token on ties.  Then the winner is copied to z.
__global__ __launch_bounds__(kSelThreads) void pca_select_kernel(const uint16_t* __restrict__ x, int64_t T, int64_t K,
                                                                 int32_t* __restrict__ idx, uint16_t* __restrict__ z) {
  __shared__ float best_v[kSelThreads / 64];
  __shared__ int64_t best_t[kSelThreads / 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t s = blockIdx.x;
  const uint16_t* xs = x + s * T * K;
  float bv = -1.0f;
  int64_t bt = -1;
  for (int64_t t = wave; t < T; t += kSelThreads / 64) {
    const uint16_t* row = xs + t * K;
    float m = 0.0f;
    for (int64_t k = lane * 8; k < K; k += 64 * 8) {
      const v4i raw = *reinterpret_cast<const v4i*>(row + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = static_cast<uint32_t>(raw[i]);
        m = fmaxf(m, fabsf(h2f(static_cast<uint16_t>(w & 0xffffu))));
        m = fmaxf(m, fabsf(h2f(static_cast<uint16_t>(w >> 16))));
      }
    }
    m = wave_max(m);
    if (m > bv) {  // tokens arrive in increasing t: strict > keeps the first
      bv = m;
      bt = t;
    }
  }
  if (lane == 0) {
    best_v[wave] = bv;
    best_t[wave] = bt;
  }
  __syncthreads();
  float v = best_v[0];
  int64_t t = best_t[0];
#pragma unroll
  for (int w = 1; w < kSelThreads / 64; ++w) {
    if (best_v[w] > v || (best_v[w] == v && best_t[w] < t)) {
      v = best_v[w];
      t = best_t[w];
    }
  }
  if (threadIdx.x == 0) idx[s] = static_cast<int32_t>(t);
  const uint16_t* src = xs + t * K;
  uint16_t* dst = z + s * K;
  for (int64_t k = threadIdx.x * 8; k < K; k += kSelThreads * 8)
    *reinterpret_cast<v4i*>(dst + k) = *reinterpret_cast<const v4i*>(src + k);
}

// Power iteration for the leading eigenvector of C = Zc^T Zc / (S - 1), with
// Zc the extreme tokens centred on their mean, without forming C:
// y = Zc v, v' = Zc^T y / (S - 1), lambda = |v'|, v = v' / lambda.  One
// workgroup; every sum in a fixed order, in float64.  The start vector is the
// centred extreme token of largest norm (it holds the dominant direction
// whenever one token carries it).  Stops when successive vectors differ by
// less than tol in 2-norm, or after max_iter iterations; then v_0 <= 0.
constexpr int kPowThreads = 1024, kPowWaves = kPowThreads / 64;

__device__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < kPowWaves; ++w) r += red[w];
  return r;
}

__global__ __launch_bounds__(kPowThreads) void pca_power_kernel(const uint16_t* __restrict__ z, int64_t S, int64_t K,
                                                                int max_iter, double tol, double* __restrict__ v,
                                                                double* __restrict__ lambda_out,
                                                                int32_t* __restrict__ iters_out,
                                                                double* __restrict__ mu, double* __restrict__ vn,
                                                                double* __restrict__ y) {
  __shared__ double red[kPowWaves];
  __shared__ double sh_s[2];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // mean over the S tokens
  for (int64_t k = threadIdx.x; k < K; k += kPowThreads) {
    double acc = 0.0;
    for (int64_t s = 0; s < S; ++s) acc += static_cast<double>(h2f(z[s * K + k]));
    mu[k] = acc / static_cast<double>(S);
  }
  __syncthreads();
  // norms of the centred tokens (one wave per token), start from the largest
  for (int64_t s = wave; s < S; s += kPowWaves) {
    double acc = 0.0;
    for (int64_t k = lane; k < K; k += 64) {
      const double d = static_cast<double>(h2f(z[s * K + k])) - mu[k];
      acc += d * d;
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) y[s] = acc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t bs = 0;
    for (int64_t s = 1; s < S; ++s)
      if (y[s] > y[bs]) bs = s;
    sh_s[0] = static_cast<double>(bs);
  }
  __syncthreads();
  const int64_t s0 = static_cast<int64_t>(sh_s[0]);
  double part = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += kPowThreads) {
    const double d = static_cast<double>(h2f(z[s0 * K + k])) - mu[k];
    v[k] = d;
    part += d * d;
  }
  double nrm = sqrt(block_sum_f64(part, red));
  const double inv0 = nrm > 0.0 ? 1.0 / nrm : 0.0;
  for (int64_t k = threadIdx.x; k < K; k += kPowThreads) v[k] = nrm > 0.0 ? v[k] * inv0 : (k == 0 ? 1.0 : 0.0);
  __syncthreads();
  const double inv_s1 = 1.0 / static_cast<double>(S > 1 ? S - 1 : 1);
  double lam = 0.0;
  int it = 0;
  for (; it < max_iter; ++it) {
    // y = Zc v: one wave per token
    for (int64_t s = wave; s < S; s += kPowWaves) {
      double acc = 0.0;
      for (int64_t k = lane; k < K; k += 64) acc += (static_cast<double>(h2f(z[s * K + k])) - mu[k]) * v[k];
      acc = wave_sum_f64(acc);
      if (lane == 0) y[s] = acc;
    }
    __syncthreads();
    // v' = Zc^T y / (S - 1): one thread per channel, tokens in order
    part = 0.0;
    for (int64_t k = threadIdx.x; k < K; k += kPowThreads) {
      double acc = 0.0;
      for (int64_t s = 0; s < S; ++s) acc += (static_cast<double>(h2f(z[s * K + k])) - mu[k]) * y[s];
      acc *= inv_s1;
      vn[k] = acc;
      part += acc * acc;
    }
    lam = sqrt(block_sum_f64(part, red));
    const double inv = lam > 0.0 ? 1.0 / lam : 0.0;
    part = 0.0;
    for (int64_t k = threadIdx.x; k < K; k += kPowThreads) {
      const double nv = vn[k] * inv;
      const double d = nv - v[k];
      part += d * d;
      v[k] = nv;
    }
    const double diff = sqrt(block_sum_f64(part, red));
    if (lam == 0.0 || diff < tol) {
      ++it;
      break;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) sh_s[1] = v[0] > 0.0 ? -1.0 : 1.0;
  __syncthreads();
  const double sg = sh_s[1];
  for (int64_t k = threadIdx.x; k < K; k += kPowThreads) v[k] *= sg;
  if (threadIdx.x == 0) {
    *lambda_out = lam;
    *iters_out = it;
  }
}

// Householder reflection with H v = e_0: w = v - e_0, beta = 2 / (w^T w).
__device__ double householder_beta(const double* v, int64_t K, double* red) {
  double part = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
    const double wk = v[k] - (k == 0 ? 1.0 : 0.0);
    part += wk * wk;
  }
  part = wave_sum_f64(part);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = part;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < nw; ++w) r += red[w];
  return r > 0.0 ? 2.0 / r : 0.0;
}

constexpr int kFoldThreads = 256;

// p[n] = sum_k w[k] W[k, n] (float64, k in order): one thread per column.
__global__ __launch_bounds__(kFoldThreads) void pca_fold_dot_kernel(const uint16_t* __restrict__ wt, int64_t K,
                                                                    int64_t N, const double* __restrict__ v,
                                                                    double* __restrict__ p) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kFoldThreads + threadIdx.x;
  if (n >= N) return;
  double acc = 0.0;
  for (int64_t k = 0; k < K; ++k) acc += (v[k] - (k == 0 ? 1.0 : 0.0)) * static_cast<double>(h2f(wt[k * N + n]));
  p[n] = acc;
}

// W'[k, n] = fp16(W[k, n] - beta w[k] p[n]).
__global__ __launch_bounds__(kFoldThreads) void pca_fold_apply_kernel(const uint16_t* __restrict__ wt, int64_t K,
                                                                      int64_t N, const double* __restrict__ v,
                                                                      const double* __restrict__ p,
                                                                      uint16_t* __restrict__ out) {
  __shared__ double red[kFoldThreads / 64];
  const double beta = householder_beta(v, K, red);
  const int64_t k = blockIdx.y;
  const double wk = v[k] - (k == 0 ? 1.0 : 0.0);
  for (int64_t n = static_cast<int64_t>(blockIdx.x) * kFoldThreads + threadIdx.x; n < N;
       n += static_cast<int64_t>(gridDim.x) * kFoldThreads) {
    const double r = static_cast<double>(h2f(wt[k * N + n])) - beta * wk * p[n];
    out[k * N + n] = f2h(static_cast<float>(r));
  }
}

// x'[m, :] = fp16(x - beta (x . w) w^T): one wave per token.
constexpr int kRotWaves = 4;

__global__ __launch_bounds__(64 * kRotWaves) void pca_rotate_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                    int64_t K, const double* __restrict__ v,
                                                                    uint16_t* __restrict__ out) {
  __shared__ double red[kRotWaves];
  const double beta = householder_beta(v, K, red);
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kRotWaves + (threadIdx.x >> 6);
  if (m >= M) return;  // after the block-wide reduction above
  const uint16_t* row = x + m * K;
  double acc = 0.0;
  for (int64_t k = lane; k < K; k += 64) acc += static_cast<double>(h2f(row[k])) * (v[k] - (k == 0 ? 1.0 : 0.0));
  const double c = beta * wave_sum_f64(acc);
  for (int64_t k = lane; k < K; k += 64) {
    const double r = static_cast<double>(h2f(row[k])) - c * (v[k] - (k == 0 ? 1.0 : 0.0));
    out[m * K + k] = f2h(static_cast<float>(r));
  }
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_pca_select(const uint16_t* x, int64_t S, int64_t T, int64_t K, int32_t* idx,
                                       uint16_t* z, void* stream) {
  QLIN_REQUIRE(S >= 0 && T > 0, QLIN_ERR_INVALID_ARG, "S=%lld, T=%lld", (long long)S, (long long)T);
  QLIN_REQUIRE(K > 0 && K % 8 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 8", (long long)K);
  if (S == 0) return QLIN_OK;
  QLIN_PTR(x);
  QLIN_PTR(idx);
  QLIN_PTR(z);
  QLIN_REQUIRE(S <= 0x7fffffffLL && T <= 0x7fffffffLL, QLIN_ERR_SHAPE, "S or T too large");
  pca_select_kernel<<<dim3(static_cast<unsigned>(S)), kSelThreads, 0, as_stream(stream)>>>(x, T, K, idx, z);
  QLIN_LAUNCH_CHECK("pca_select_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_pca_leading_eigvec(const uint16_t* z, int64_t S, int64_t K, int32_t max_iter,
                                               double tol, double* v, double* lambda, int32_t* iters, double* ws,
                                               void* stream) {
  QLIN_REQUIRE(S >= 2, QLIN_ERR_SHAPE, "S=%lld: a covariance needs at least 2 tokens", (long long)S);
  QLIN_REQUIRE(K > 0, QLIN_ERR_SHAPE, "K=%lld must be positive", (long long)K);
  QLIN_REQUIRE(max_iter > 0, QLIN_ERR_INVALID_ARG, "max_iter=%d must be positive", max_iter);
  QLIN_REQUIRE(tol >= 0.0, QLIN_ERR_INVALID_ARG, "tol must be non-negative");
  QLIN_PTR(z);
  QLIN_PTR(v);
  QLIN_PTR(lambda);
  QLIN_PTR(iters);
  QLIN_PTR(ws);
  pca_power_kernel<<<dim3(1), kPowThreads, 0, as_stream(stream)>>>(z, S, K, max_iter, tol, v, lambda, iters, ws,
                                                                   ws + K, ws + 2 * K);
  QLIN_LAUNCH_CHECK("pca_power_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_pca_fold_weight(const uint16_t* w, int64_t K, int64_t N, const double* v,
                                            uint16_t* w_out, double* ws, void* stream) {
  QLIN_REQUIRE(K > 0 && N > 0, QLIN_ERR_SHAPE, "K=%lld, N=%lld must be positive", (long long)K, (long long)N);
  QLIN_REQUIRE(K <= 65535, QLIN_ERR_SHAPE, "K=%lld too large", (long long)K);
  QLIN_PTR(w);
  QLIN_PTR(v);
  QLIN_PTR(w_out);
  QLIN_PTR(ws);
  hipStream_t st = as_stream(stream);
  const unsigned gx = static_cast<unsigned>((N + kFoldThreads - 1) / kFoldThreads);
  pca_fold_dot_kernel<<<dim3(gx), kFoldThreads, 0, st>>>(w, K, N, v, ws);
  QLIN_LAUNCH_CHECK("pca_fold_dot_kernel");
  pca_fold_apply_kernel<<<dim3(gx, static_cast<unsigned>(K)), kFoldThreads, 0, st>>>(w, K, N, v, ws, w_out);
  QLIN_LAUNCH_CHECK("pca_fold_apply_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_pca_rotate(const uint16_t* x, int64_t M, int64_t K, const double* v, uint16_t* x_out,
                                       void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0, QLIN_ERR_SHAPE, "K=%lld must be positive", (long long)K);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(x);
  QLIN_PTR(v);
  QLIN_PTR(x_out);
  QLIN_REQUIRE(M / kRotWaves < 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  pca_rotate_kernel<<<dim3(static_cast<unsigned>((M + kRotWaves - 1) / kRotWaves)), 64 * kRotWaves, 0,
                      as_stream(stream)>>>(x, M, K, v, x_out);
  QLIN_LAUNCH_CHECK("pca_rotate_kernel");
  return QLIN_OK;
}
