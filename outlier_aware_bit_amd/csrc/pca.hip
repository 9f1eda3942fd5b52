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

constexpr int kSelThreads = 512, kSelWaves = kSelThreads / 64, kSelParts = 4, kSelCH = 8;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void unpack8_f64(v4i raw, double (&d)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = static_cast<uint32_t>(raw[i]);
    d[2 * i] = static_cast<double>(h2f(static_cast<uint16_t>(w & 0xffffu)));
    d[2 * i + 1] = static_cast<double>(h2f(static_cast<uint16_t>(w >> 16)));
  }
}

__device__ __forceinline__ float absmax8(v4i raw, float m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = static_cast<uint32_t>(raw[i]);
    m = fmaxf(m, fabsf(h2f(static_cast<uint16_t>(w & 0xffffu))));
    m = fmaxf(m, fabsf(h2f(static_cast<uint16_t>(w >> 16))));
  }
  return m;
}

// The extreme token in two passes.  Pass 1: workgroup (p, s) takes the p-th
// of P contiguous runs of sequence s's tokens; wave w scans tokens w,
// w + kSelWaves, ... of the run, all of a token's loads in flight at once;
// the largest max|x| wins, the first token on ties.  Its candidate (value,
// token) goes to slot p of z's row s, which pass 2 reads and then overwrites
// with the winning token.
__global__ __launch_bounds__(kSelThreads) void pca_select_part_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                                      int64_t K, int P, uint16_t* __restrict__ z) {
  __shared__ float best_v[kSelWaves];
  __shared__ int64_t best_t[kSelWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t s = blockIdx.y, run = (T + P - 1) / P;
  const int64_t t0 = blockIdx.x * run, t1 = t0 + run < T ? t0 + run : T;
  const uint16_t* xs = x + s * T * K;
  const int nch = static_cast<int>(K / 8);
  float bv = -1.0f;
  int64_t bt = -1;
  for (int64_t t = t0 + wave; t < t1; t += kSelWaves) {
    const uint16_t* row = xs + t * K;
    v4i raw[kSelCH];
#pragma unroll
    for (int i = 0; i < kSelCH; ++i) {
      const int c = lane + 64 * i;
      raw[i] = *reinterpret_cast<const v4i*>(row + 8 * (c < nch ? c : nch - 1));
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kSelCH; ++i) m = absmax8(raw[i], m);  // clamped repeats change no maximum
    for (int c = lane + 64 * kSelCH; c < nch; c += 64) m = absmax8(*reinterpret_cast<const v4i*>(row + 8 * c), m);
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
  if (threadIdx.x == 0) {
    float v = best_v[0];
    int64_t t = best_t[0];
    for (int w = 1; w < kSelWaves; ++w) {
      if (best_t[w] >= 0 && (t < 0 || best_v[w] > v || (best_v[w] == v && best_t[w] < t))) {
        v = best_v[w];
        t = best_t[w];
      }
    }
    float* slot = reinterpret_cast<float*>(z + s * K) + 2 * blockIdx.x;
    slot[0] = v;
    reinterpret_cast<int32_t*>(slot)[1] = static_cast<int32_t>(t);
  }
}

// Pass 2: the best of the P candidates (runs in increasing t: the first run
// wins ties), then the copy of the winner into z.
__global__ __launch_bounds__(kSelThreads) void pca_select_final_kernel(const uint16_t* __restrict__ x, int64_t T,
                                                                       int64_t K, int P, int32_t* __restrict__ idx,
                                                                       uint16_t* __restrict__ z) {
  __shared__ int64_t win;
  const int64_t s = blockIdx.x;
  uint16_t* dst = z + s * K;
  if (threadIdx.x == 0) {
    const float* slot = reinterpret_cast<const float*>(dst);
    float v = -1.0f;
    int64_t t = -1;
    for (int p = 0; p < P; ++p) {
      const float pv = slot[2 * p];
      const int32_t pt = reinterpret_cast<const int32_t*>(slot)[2 * p + 1];
      if (pt >= 0 && (t < 0 || pv > v)) {
        v = pv;
        t = pt;
      }
    }
    win = t;
    idx[s] = static_cast<int32_t>(t);
  }
  __syncthreads();
  const uint16_t* src = x + (s * T + win) * K;
  for (int64_t k = threadIdx.x * 8; k < K; k += kSelThreads * 8)
    *reinterpret_cast<v4i*>(dst + k) = *reinterpret_cast<const v4i*>(src + k);
}

// Power iteration for the leading eigenvector of C = Zc^T Zc / (S - 1), with
// Zc the extreme tokens centred on their mean, without forming C, run in the
// tokens' coordinates: every iterate is v = Zc^T a for a vector a of S
// token weights, and with the Gram matrix G = Zc Zc^T (S x S)
//   C v = Zc^T b,  b = G a / (S - 1),  |C v|^2 = b^T G b,  |Zc^T d|^2 = d^T G d,
// so the iteration v' = C v / |C v| is a' = b / lambda with lambda = |C v|,
// the distance of successive vectors is sqrt(da^T G da), and v = Zc^T a at
// the end.  The start vector is the centred extreme token of largest norm
// (a = e_s0 / |Zc[s0]|, the largest diagonal entry of G); the iteration
// stops when successive vectors differ by less than tol, or after max_iter;
// then v_0 <= 0.  float64 throughout, every sum in a fixed order.  Passes:
// the mean, G on the fp64 matrix cores, the iteration (one workgroup, one
// product by G per iteration), and the projection v = Zc^T a.
constexpr int kPcaThreads = 256;
constexpr int kPowThreads = 256, kPowWaves = kPowThreads / 64, kPowU = 8;
constexpr int64_t kPowMaxK = 8192, kPowMaxS = 2048, kPowLdsS = 128;  // G in LDS up to S = 128

// Column sums over the tokens, sum_s f(s) (z[s, k] - c_k) w_s: a workgroup
// takes 64 channels (8 chunks of 8); thread (chunk t & 7, token group
// t >> 3) adds the tokens s = group, group + 32, ... (8 in flight), then the
// 32 groups' sums are added in order through LDS.  kMean: c = 0, w = 1.
constexpr int kColGroups = kPcaThreads / 8;

template <bool kMean>
__device__ __forceinline__ void column_sums(const uint16_t* __restrict__ z, int64_t S, int64_t K,
                                            const double* __restrict__ cen, const double* __restrict__ w,
                                            double (&out)[8], double (*red)[8][8]) {
  const int ch = threadIdx.x & 7, grp = threadIdx.x >> 3;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 8 + ch;
  const bool ok = c < K / 8;
  const uint16_t* zc = z + 8 * (ok ? c : 0);
  double m[8], acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = (kMean || !ok) ? 0.0 : cen[8 * c + j];
  int64_t s = grp;
  for (; s + kColGroups * (kPowU - 1) < S; s += kColGroups * kPowU) {
    v4i raw[kPowU];
#pragma unroll
    for (int u = 0; u < kPowU; ++u) raw[u] = *reinterpret_cast<const v4i*>(zc + (s + kColGroups * u) * K);
#pragma unroll
    for (int u = 0; u < kPowU; ++u) {
      double d[8];
      unpack8_f64(raw[u], d);
      const double ws = kMean ? 1.0 : w[s + kColGroups * u];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += kMean ? d[j] : (d[j] - m[j]) * ws;
    }
  }
  for (; s < S; s += kColGroups) {
    double d[8];
    unpack8_f64(*reinterpret_cast<const v4i*>(zc + s * K), d);
    const double ws = kMean ? 1.0 : w[s];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] += kMean ? d[j] : (d[j] - m[j]) * ws;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[grp][ch][j] = acc[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = 0.0;
  if (grp == 0) {
    for (int g = 0; g < kColGroups; ++g)
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] += red[g][ch][j];
  }
}

// mu[k] = sum_s z[s, k] / S.
__global__ __launch_bounds__(kPcaThreads) void pca_mean_kernel(const uint16_t* __restrict__ z, int64_t S, int64_t K,
                                                               double* __restrict__ mu) {
  __shared__ double red[kColGroups][8][8];
  double sum[8];
  column_sums<true>(z, S, K, nullptr, nullptr, sum, red);
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x & 7);
  if ((threadIdx.x >> 3) == 0 && c < K / 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) mu[8 * c + j] = sum[j] / static_cast<double>(S);
  }
}

// G tile (16 tokens i) x (16 tokens j) on v_mfma_f64_16x16x4f64.  In a
// product step lane l gives the centred value of token (l & 15) at one k and
// the hardware pairs A's lane (i, g) with B's lane (j, g), g = l >> 4; a
// lane's 16-byte chunk (8 consecutive k) feeds 8 steps, so 4 lane groups
// cover 32 k per 8 steps.  The 16 waves take the 32-k blocks in turn; their
// tiles are added in order through LDS.  Result layout: lane l, register r
// holds row 4 r + (l >> 4), column l & 15.
typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kGramThreads = 1024;

__global__ __launch_bounds__(kGramThreads) void pca_gram_kernel(const uint16_t* __restrict__ z, int64_t S, int64_t K,
                                                                const double* __restrict__ mu,
                                                                double* __restrict__ G) {
  __shared__ double red[kGramThreads / 64][64][4];
  __shared__ double mul[kPowMaxK];
  for (int64_t k = threadIdx.x; k < K; k += kGramThreads) mul[k] = mu[k];
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t ti = static_cast<int64_t>(blockIdx.y) * 16 + (lane & 15);
  const int64_t tj = static_cast<int64_t>(blockIdx.x) * 16 + (lane & 15);
  const bool oki = ti < S, okj = tj < S;
  const uint16_t* zi = z + (oki ? ti : 0) * K;
  const uint16_t* zj = z + (okj ? tj : 0) * K;
  const int nch = static_cast<int>(K / 8), g = lane >> 4;
  v4d acc = v4d{0.0, 0.0, 0.0, 0.0};
  constexpr int kW = kGramThreads / 64;
  // Blocks blk = wave + kW u; two blocks' loads in flight per step.
  for (int blk = wave; 4 * blk < nch; blk += 2 * kW) {
    v4i ra[2], rb[2];
    bool okc[2];
    int cc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = 4 * (blk + kW * u) + g;  // this lane's chunk
      okc[u] = c < nch;
      cc[u] = okc[u] ? c : 0;
      ra[u] = *reinterpret_cast<const v4i*>(zi + 8 * cc[u]);
      rb[u] = *reinterpret_cast<const v4i*>(zj + 8 * cc[u]);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      double a[8], b[8];
      unpack8_f64(ra[u], a);
      unpack8_f64(rb[u], b);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double m = mul[8 * cc[u] + j];
        const double av = (oki && okc[u]) ? a[j] - m : 0.0;
        const double bv = (okj && okc[u]) ? b[j] - m : 0.0;
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) red[wave][lane][r] = acc[r];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    double t = red[0][lane][r];
#pragma unroll
    for (int w = 1; w < kGramThreads / 64; ++w) t += red[w][lane][r];
    const int64_t row = static_cast<int64_t>(blockIdx.y) * 16 + 4 * r + (lane >> 4);
    const int64_t col = static_cast<int64_t>(blockIdx.x) * 16 + (lane & 15);
    if (row < S && col < S) G[row * S + col] = t;
  }
}

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

// The iteration in token coordinates (one workgroup).  out: a [S], then
// the sign to apply to v (out[S]), lambda and the iteration count.
__global__ __launch_bounds__(kPowThreads) void pca_iter_kernel(const uint16_t* __restrict__ z, int64_t S, int64_t K,
                                                               const double* __restrict__ G,
                                                               const double* __restrict__ mu, int max_iter,
                                                               double tol, double* __restrict__ out,
                                                               double* __restrict__ lambda_out,
                                                               int32_t* __restrict__ iters_out) {
  // LDS: a, ga, b, gb (S each), then G itself when S <= kPowLdsS.
  extern __shared__ __attribute__((aligned(16))) double il[];
  __shared__ double red[kPowWaves];
  __shared__ int64_t sh_s0;
  double* const a = il;
  double* const ga = il + S;
  double* const b = il + 2 * S;
  double* const gb = il + 3 * S;
  const bool g_lds = S <= kPowLdsS;
  double* const gl = il + 4 * S;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (g_lds) {
#pragma unroll 16
    for (int64_t e = threadIdx.x; e < S * S; e += kPowThreads) gl[e] = G[e];
  } else {
#pragma unroll 2
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) gb[t] = G[t * S + t];
  }
  __syncthreads();
  const double* const gm = g_lds ? gl : G;
  // y = G x: thread t sums column t of G (G is symmetric), j in order, so
  // that the lanes read consecutive entries.
  auto matvec = [&](const double* x, double* y) {
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) {
      double acc = 0.0;
#pragma unroll 8
      for (int64_t j = 0; j < S; ++j) acc += gm[j * S + t] * x[j];
      y[t] = acc;
    }
  };
  // s0 = the first token of largest diagonal entry: each wave its stride of
  // tokens, then wave 0 over the waves' winners (both keep the first).
  {
    __shared__ double wv[kPowWaves];
    __shared__ int64_t wt[kPowWaves];
    double bv = -1.0;
    int64_t bt = S;
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) {
      const double dv = g_lds ? gl[t * S + t] : gb[t];
      if (dv > bv) {  // t increases: strict > keeps the first
        bv = dv;
        bt = t;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ov = __shfl_xor(bv, o, 64);
      const int64_t ot = __shfl_xor(bt, o, 64);
      if (ov > bv || (ov == bv && ot < bt)) {
        bv = ov;
        bt = ot;
      }
    }
    if (lane == 0) {
      wv[wave] = bv;
      wt[wave] = bt;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double v = wv[0];
      int64_t t = wt[0];
      for (int w = 1; w < kPowWaves; ++w)
        if (wv[w] > v || (wv[w] == v && wt[w] < t)) {
          v = wv[w];
          t = wt[w];
        }
      sh_s0 = t < S ? t : 0;
    }
    __syncthreads();
  }
  const int64_t s0 = sh_s0;
  const double n0 = gm[s0 * S + s0];
  const bool zero = !(n0 > 0.0);  // every centred token is zero: v = e_0
  const double inv0 = zero ? 0.0 : 1.0 / sqrt(n0);
  for (int64_t t = threadIdx.x; t < S; t += kPowThreads) {
    a[t] = t == s0 ? inv0 : 0.0;
    ga[t] = gm[t * S + s0] * inv0;
  }
  __syncthreads();
  const double inv_s1 = 1.0 / static_cast<double>(S - 1);
  double lam = 0.0;
  int it = 0;
  for (; it < max_iter; ++it) {
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) b[t] = ga[t] * inv_s1;
    __syncthreads();
    matvec(b, gb);
    __syncthreads();
    double part = 0.0;
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) part += b[t] * gb[t];
    const double l2 = block_sum_f64(part, red);
    lam = l2 > 0.0 ? sqrt(l2) : 0.0;
    if (lam == 0.0) {
      ++it;
      break;
    }
    const double inv = 1.0 / lam;
    part = 0.0;
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) {
      const double an = b[t] * inv, gan = gb[t] * inv;
      part += (an - a[t]) * (gan - ga[t]);
    }
    const double d2 = block_sum_f64(part, red);  // its barriers order the reads above before the writes below
    for (int64_t t = threadIdx.x; t < S; t += kPowThreads) {
      a[t] = b[t] * inv;
      ga[t] = gb[t] * inv;
    }
    __syncthreads();
    if (sqrt(d2 > 0.0 ? d2 : 0.0) < tol) {
      ++it;
      break;
    }
  }
  // v_0 = sum_s (z[s, 0] - mu_0) a_s decides the sign.
  double part = 0.0;
  const double m0 = mu[0];
  for (int64_t t = threadIdx.x; t < S; t += kPowThreads)
    part += (static_cast<double>(h2f(z[t * K])) - m0) * a[t];
  const double v0 = block_sum_f64(part, red);
  for (int64_t t = threadIdx.x; t < S; t += kPowThreads) out[t] = a[t];
  if (threadIdx.x == 0) {
    // zero: v = e_0, so v_0 = 1 > 0 flips it.
    out[S] = zero ? 2.0 : (v0 > 0.0 ? -1.0 : 1.0);
    *lambda_out = lam;
    *iters_out = it;
  }
}

// v[k] = sign * sum_s (z[s, k] - mu[k]) a_s.  sign == 2 marks the all-zero
// case: v = -e_0.
__global__ __launch_bounds__(kPcaThreads) void pca_project_kernel(const uint16_t* __restrict__ z, int64_t S,
                                                                  int64_t K, const double* __restrict__ mu,
                                                                  const double* __restrict__ av,
                                                                  double* __restrict__ v) {
  __shared__ double red[kColGroups][8][8];
  double sum[8];
  column_sums<false>(z, S, K, mu, av, sum, red);
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x & 7);
  if ((threadIdx.x >> 3) != 0 || c >= K / 8) return;
  const double sg = av[S];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[8 * c + j] = sg == 2.0 ? ((8 * c + j == 0) ? -1.0 : 0.0) : sum[j] * sg;
}

// Householder reflection with H v = e_0: w = v - e_0, beta = 2 / (w^T w).
__device__ double householder_beta(const double* v, int64_t K, double* red) {
  double part = 0.0;
#pragma unroll 8
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

// The weight fold in three passes, sums in a fixed order (not k in order):
//   partial: block (column block of kFoldCols, row block of kFoldRows) adds
//            u[k] W[k, n] over its rows (each wave over kFoldRows / 4
//            consecutive rows, then the four waves in order);
//   reduce:  q[n] = beta * sum over the row blocks, in order;
//   apply:   W'[k, n] = fp16(W[k, n] - u[k] q[n]).
// The row-block sums are kept in w_out (8 bytes per column and row block fit
// in the 2 bytes per element of w_out), which the apply pass then overwrites.
constexpr int kFoldThreads = 256, kFoldCols = 512, kFoldRows = 64;

__global__ __launch_bounds__(kFoldThreads) void pca_fold_partial_kernel(const uint16_t* __restrict__ wt, int64_t K,
                                                                        int64_t N, const double* __restrict__ v,
                                                                        double* __restrict__ part) {
  __shared__ double red[kFoldThreads / 64][64][8];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kFoldCols + 8 * lane;
  const int64_t kb = static_cast<int64_t>(blockIdx.y) * kFoldRows;
  constexpr int kPer = kFoldRows / (kFoldThreads / 64);
  const int64_t k0 = kb + kPer * wave;
  double acc[8] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  if (n < N) {
    v4i raw[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int64_t k = k0 + i < K ? k0 + i : K - 1;
      raw[i] = *reinterpret_cast<const v4i*>(wt + k * N + n);
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (k0 + i < K) {
        const double uk = v[k0 + i] - (k0 + i == 0 ? 1.0 : 0.0);
        double d[8];
        unpack8_f64(raw[i], d);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += uk * d[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wave][lane][j] = acc[j];
  __syncthreads();
  if (wave == 0 && n < N) {
    double* dst = part + static_cast<int64_t>(blockIdx.y) * N + n;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      double t = red[0][lane][j];
#pragma unroll
      for (int w = 1; w < kFoldThreads / 64; ++w) t += red[w][lane][j];
      dst[j] = t;
    }
  }
}

constexpr int kFoldRedThreads = 64;

__global__ __launch_bounds__(kFoldRedThreads) void pca_fold_reduce_kernel(const double* __restrict__ part, int64_t nb,
                                                                       int64_t K, int64_t N,
                                                                       const double* __restrict__ v,
                                                                       double* __restrict__ q) {
  __shared__ double red[kFoldRedThreads / 64];
  const double beta = householder_beta(v, K, red);
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kFoldRedThreads + threadIdx.x;
  if (n >= N) return;
  double acc = 0.0;
#pragma unroll 16
  for (int64_t b = 0; b < nb; ++b) acc += part[b * N + n];
  q[n] = beta * acc;
}

// Thread: 8 columns of one row; a workgroup 8 * kFoldThreads columns.
__global__ __launch_bounds__(kFoldThreads) void pca_fold_apply_kernel(const uint16_t* __restrict__ wt, int64_t K,
                                                                      int64_t N, const double* __restrict__ v,
                                                                      const double* __restrict__ q,
                                                                      uint16_t* __restrict__ out) {
  const int64_t k = blockIdx.y;
  const int64_t n = (static_cast<int64_t>(blockIdx.x) * kFoldThreads + threadIdx.x) * 8;
  if (n >= N) return;
  const double uk = v[k] - (k == 0 ? 1.0 : 0.0);
  double d[8];
  unpack8_f64(*reinterpret_cast<const v4i*>(wt + k * N + n), d);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const double r0 = d[2 * i] - uk * q[n + 2 * i];
    const double r1 = d[2 * i + 1] - uk * q[n + 2 * i + 1];
    o[i] = static_cast<uint32_t>(f2h(static_cast<float>(r0))) |
           (static_cast<uint32_t>(f2h(static_cast<float>(r1))) << 16);
  }
  *reinterpret_cast<v4i*>(out + k * N + n) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
}

// x'[m, :] = fp16(x - beta (x . u) u^T), u = v - e_0: u and beta once per
// workgroup in LDS, one wave per token, each lane 8 consecutive channels per
// 16-byte chunk (chunks lane + 64 i, the first kRotCH of them held in
// registers between the dot and the update).
constexpr int kRotWaves = 8, kRotCH = 8, kRotMaxK = 8192;

__global__ __launch_bounds__(64 * kRotWaves) void pca_rotate_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                                    int64_t K, const double* __restrict__ v,
                                                                    uint16_t* __restrict__ out) {
  __shared__ double u[kRotMaxK];
  __shared__ double red[kRotWaves];
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kRotWaves + (threadIdx.x >> 6);
  const int64_t mc = m < M ? m : M - 1;
  const uint16_t* row = x + mc * K;
  const int nch = static_cast<int>(K / 8);
  v4i raw[kRotCH];
#pragma unroll
  for (int i = 0; i < kRotCH; ++i) {
    const int c = lane + 64 * i;
    raw[i] = *reinterpret_cast<const v4i*>(row + 8 * (c < nch ? c : nch - 1));
  }
  for (int64_t k = threadIdx.x; k < K; k += 64 * kRotWaves) u[k] = v[k] - (k == 0 ? 1.0 : 0.0);
  __syncthreads();
  double part = 0.0;
  for (int64_t k = threadIdx.x; k < K; k += 64 * kRotWaves) part += u[k] * u[k];
  part = wave_sum_f64(part);
  if (lane == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  double uu = 0.0;
#pragma unroll
  for (int w = 0; w < kRotWaves; ++w) uu += red[w];
  const double beta = uu > 0.0 ? 2.0 / uu : 0.0;
  if (m >= M) return;  // after the workgroup's barriers
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kRotCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      double d[8];
      unpack8_f64(raw[i], d);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += d[j] * u[8 * c + j];
    }
  }
  for (int c = lane + 64 * kRotCH; c < nch; c += 64) {
    double d[8];
    unpack8_f64(*reinterpret_cast<const v4i*>(row + 8 * c), d);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += d[j] * u[8 * c + j];
  }
  const double cf = beta * wave_sum_f64(acc);
  uint16_t* orow = out + m * K;
  auto emit = [&](int c, v4i r) {
    double d[8];
    unpack8_f64(r, d);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double r0 = d[2 * i] - cf * u[8 * c + 2 * i];
      const double r1 = d[2 * i + 1] - cf * u[8 * c + 2 * i + 1];
      o[i] = static_cast<uint32_t>(f2h(static_cast<float>(r0))) |
             (static_cast<uint32_t>(f2h(static_cast<float>(r1))) << 16);
    }
    *reinterpret_cast<v4i*>(orow + 8 * c) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  };
#pragma unroll
  for (int i = 0; i < kRotCH; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) emit(c, raw[i]);
  }
  for (int c = lane + 64 * kRotCH; c < nch; c += 64) emit(c, *reinterpret_cast<const v4i*>(row + 8 * c));
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
  QLIN_DIMS(S, T);
  QLIN_DIMS(S * T, K);
  // P candidate slots of 8 bytes fit in a row of z (2K >= 16 bytes).
  const int P = static_cast<int>(K / 4 < kSelParts ? K / 4 : kSelParts);
  hipStream_t st = as_stream(stream);
  pca_select_part_kernel<<<dim3(static_cast<unsigned>(P), static_cast<unsigned>(S)), kSelThreads, 0, st>>>(x, T, K, P,
                                                                                                        z);
  QLIN_LAUNCH_CHECK("pca_select_part_kernel");
  pca_select_final_kernel<<<dim3(static_cast<unsigned>(S)), kSelThreads, 0, st>>>(x, T, K, P, idx, z);
  QLIN_LAUNCH_CHECK("pca_select_final_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_pca_leading_eigvec(const uint16_t* z, int64_t S, int64_t K, int32_t max_iter,
                                               double tol, double* v, double* lambda, int32_t* iters, double* ws,
                                               void* stream) {
  QLIN_REQUIRE(S >= 2 && S <= kPowMaxS, QLIN_ERR_SHAPE, "S=%lld: a covariance needs 2 to %lld tokens", (long long)S,
               (long long)kPowMaxS);
  QLIN_REQUIRE(K > 0 && K % 8 == 0 && K <= kPowMaxK, QLIN_ERR_SHAPE,
               "K=%lld must be a positive multiple of 8, at most %lld", (long long)K, (long long)kPowMaxK);
  QLIN_REQUIRE(max_iter > 0, QLIN_ERR_INVALID_ARG, "max_iter=%d must be positive", max_iter);
  QLIN_REQUIRE(tol >= 0.0, QLIN_ERR_INVALID_ARG, "tol must be non-negative");
  QLIN_PTR(z);
  QLIN_PTR(v);
  QLIN_PTR(lambda);
  QLIN_PTR(iters);
  QLIN_PTR(ws);
  // ws: G [S x S], mu [K], a [S] and the sign.
  double* const G = ws;
  double* const mu = ws + S * S;
  double* const av = mu + K;
  hipStream_t st = as_stream(stream);
  const unsigned gc = static_cast<unsigned>((K / 8 + 7) / 8);  // 64 channels per workgroup
  const unsigned gt = static_cast<unsigned>((S + 15) / 16);
  pca_mean_kernel<<<dim3(gc), kPcaThreads, 0, st>>>(z, S, K, mu);
  QLIN_LAUNCH_CHECK("pca_mean_kernel");
  pca_gram_kernel<<<dim3(gt, gt), kGramThreads, 0, st>>>(z, S, K, mu, G);
  QLIN_LAUNCH_CHECK("pca_gram_kernel");
  const size_t ilds = static_cast<size_t>(4 * S + (S <= kPowLdsS ? S * S : 0)) * sizeof(double);
  pca_iter_kernel<<<dim3(1), kPowThreads, ilds, st>>>(z, S, K, G, mu, max_iter,
                                                                                           tol, av, lambda, iters);
  QLIN_LAUNCH_CHECK("pca_iter_kernel");
  pca_project_kernel<<<dim3(gc), kPcaThreads, 0, st>>>(z, S, K, mu, av, v);
  QLIN_LAUNCH_CHECK("pca_project_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_pca_fold_weight(const uint16_t* w, int64_t K, int64_t N, const double* v,
                                            uint16_t* w_out, double* ws, void* stream) {
  QLIN_REQUIRE(K > 0 && N > 0 && N % 8 == 0, QLIN_ERR_SHAPE, "K=%lld, N=%lld: both positive, N a multiple of 8",
               (long long)K, (long long)N);
  QLIN_REQUIRE(K <= 65535, QLIN_ERR_SHAPE, "K=%lld too large", (long long)K);
  QLIN_DIMS(K, N);
  QLIN_PTR(w);
  QLIN_PTR(v);
  QLIN_PTR(w_out);
  QLIN_PTR(ws);
  hipStream_t st = as_stream(stream);
  const int64_t nb = (K + kFoldRows - 1) / kFoldRows;  // row blocks; with nb > 1, nb * N doubles fit in w_out
  // One row block (K <= kFoldRows): its sums go straight to ws, where the
  // reduce pass turns each into q in place.
  double* const part = nb == 1 ? ws : reinterpret_cast<double*>(w_out);
  pca_fold_partial_kernel<<<dim3(static_cast<unsigned>((N + kFoldCols - 1) / kFoldCols), static_cast<unsigned>(nb)),
                            kFoldThreads, 0, st>>>(w, K, N, v, part);
  QLIN_LAUNCH_CHECK("pca_fold_partial_kernel");
  pca_fold_reduce_kernel<<<dim3(static_cast<unsigned>((N + kFoldRedThreads - 1) / kFoldRedThreads)), kFoldRedThreads,
                           0, st>>>(
      part, nb, K, N, v, ws);
  QLIN_LAUNCH_CHECK("pca_fold_reduce_kernel");
  pca_fold_apply_kernel<<<dim3(static_cast<unsigned>((N / 8 + kFoldThreads - 1) / kFoldThreads),
                               static_cast<unsigned>(K)),
                          kFoldThreads, 0, st>>>(w, K, N, v, ws, w_out);
  QLIN_LAUNCH_CHECK("pca_fold_apply_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_pca_rotate(const uint16_t* x, int64_t M, int64_t K, const double* v, uint16_t* x_out,
                                       void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 8 == 0 && K <= kRotMaxK, QLIN_ERR_SHAPE,
               "K=%lld must be a positive multiple of 8, at most %d", (long long)K, kRotMaxK);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(x);
  QLIN_PTR(v);
  QLIN_PTR(x_out);
  QLIN_REQUIRE(M / kRotWaves < 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  QLIN_DIMS(M, K);
  pca_rotate_kernel<<<dim3(static_cast<unsigned>((M + kRotWaves - 1) / kRotWaves)), 64 * kRotWaves, 0,
                      as_stream(stream)>>>(x, M, K, v, x_out);
  QLIN_LAUNCH_CHECK("pca_rotate_kernel");
  return QLIN_OK;
}
