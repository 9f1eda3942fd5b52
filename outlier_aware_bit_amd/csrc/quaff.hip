// Quaff kernels of libqlin (gfx950):
//   qlin_momentum_update    targeted momentum scaling on the fixed outlier set O
//   qlin_weight_row_absmax  max_n |W_O[o, n]| for beta
//   qlin_outlier_comp       the sparse compensation term added to Y
//
// Source: "Quaff: Quantized Parameter-Efficient Fine-Tuning under Outlier
// Spatial Stability Hypothesis" (paper notes), "key design".
#include "common.hpp"
#include "comp.hpp"
#include "internal.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

constexpr int kMomThreads = 256;

// Momentum update, one workgroup per 64-channel strip of X (one 128-byte
// line per token row).  The outliers of a strip share its lines, so reading
// the whole strip once per row fetches every line of X that holds an outlier
// exactly once, with no reduction across workgroups.  Strips without an
// outlier read nothing from X.  (Splitting a strip's rows over several
// workgroups needs either a second launch to fold their maxima or
// device-scope fences, which write back and invalidate the per-XCD L2
// caches; both cost more than the extra workgroups save at 2048 tokens.)
//   c_k   = max_m |x[m, k]| for the 64 channels k of the strip
//   o in O in the strip:  beta = max(1, sqrt(c_o / wmax)) (1 if wmax == 0),
//                         s_o = gamma*s_o + (1-gamma)*beta, r_o = 1/s_o
//   other channels:       r_k = 1/s_k
constexpr int kStripThreads = 1024;
constexpr int kStripLoads = 16;                             // 16-byte loads in flight per thread
constexpr int kStripRows = kStripThreads / 8 * kStripLoads;  // rows per pass (8 lanes per row)

__global__ __launch_bounds__(kStripThreads) void momentum_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int32_t* __restrict__ O, int nO,
    const float* __restrict__ wmax, float gamma, float* __restrict__ s, float* __restrict__ r) {
  __shared__ float red[kStripThreads / 64][64];
  __shared__ int owner[64];  // 1 + index into O of the outlier at this channel, or 0
  const int64_t strip = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) owner[tid] = 0;
  __syncthreads();
  for (int j = tid; j < nO; j += kStripThreads) {
    const int o = O[j];
    if (o >= 0 && o < K && o / 64 == strip) owner[o % 64] = j + 1;
  }
  __syncthreads();
  const bool any = __syncthreads_or(tid < 64 && owner[tid] != 0);

  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // channels 8*(tid&7) + [0, 8)
  if (any) {
    const uint16_t* col = x + strip * 64 + (tid & 7) * 8;
    const int64_t row0 = tid >> 3;
    for (int64_t mb = 0; mb < M; mb += kStripRows) {
      v4i v[kStripLoads];
#pragma unroll
      for (int i = 0; i < kStripLoads; ++i) {
        const int64_t m = mb + row0 + static_cast<int64_t>(kStripThreads / 8) * i;
        v[i] = (m < M) ? *reinterpret_cast<const v4i*>(col + m * K) : v4i{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < kStripLoads; ++i)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t u = static_cast<uint32_t>(v[i][w]);
          cm[2 * w] = fmaxf(cm[2 * w], fabsf(h2f(static_cast<uint16_t>(u & 0xffffu))));
          cm[2 * w + 1] = fmaxf(cm[2 * w + 1], fabsf(h2f(static_cast<uint16_t>(u >> 16))));
        }
    }
  }
  // Lanes with equal (lane & 7) hold the same channels: combine over lane bits 3..5.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v = cm[c];
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    cm[c] = v;
  }
  if (lane < 8) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[wave][lane * 8 + c] = cm[c];
  }
  __syncthreads();
  if (tid < 64) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < kStripThreads / 64; ++w) c = fmaxf(c, red[w][tid]);
    const int64_t k = strip * 64 + tid;
    const int own = owner[tid];
    if (own != 0) {
      const float wm = wmax[own - 1];
      float beta = 1.0f;
      if (wm != 0.0f) beta = fmaxf(1.0f, sqrt_rn(div_rn(c, wm)));
      const float g1 = sub_rn(1.0f, gamma);
      const float sn = add_rn(mul_rn(gamma, s[k]), mul_rn(g1, beta));
      s[k] = sn;
      r[k] = div_rn(1.0f, sn);
    } else {
      r[k] = div_rn(1.0f, s[k]);
    }
  }
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

// STE backward, compensation part: cb[m, j] = sum_n dy[m, n] * w_o[j, n] in
// fp32 (fp16 products on the matrix cores) for j < nO, zero for
// nO <= j < ldO.  A small product (N long, ldO narrow) bound by moving the
// operands from L2 into the compute units: a workgroup takes 32 rows and
// kGradCB column blocks of 32, its kGradWaves waves take the 64-wide blocks
// of n in turn (wave w: blocks w, w + kGradWaves, ...).  A wave moves each
// block through its own LDS region: coalesced 16-byte loads (eight lanes per
// 128-byte row piece, kGradD blocks in flight), then reads in the fragment
// order of v_mfma_f32_32x32x16_f16 (lane: row l & 31, 8 consecutive n from
// 8 (l >> 5) on).  Each row's eight 16-byte chunks sit permuted by the xor
// with grad_swz(row), so that 16 lanes reading one chunk of 16 consecutive
// rows touch all 64 banks once (8 lanes of an aligned half: 32 distinct
// banks).  The waves' sums meet in LDS in a fixed pairing order (w and
// w + 4, then w and w + 2, then 0 and 1): the result does not depend on
// timing.
constexpr int kGradCB = 2, kGradWaves = 8, kGradThreads = 64 * kGradWaves, kGradD = 2;
constexpr int kGradBW = 64;                      // n per block
constexpr int kGradCPR = kGradBW / 8;            // 16-byte chunks per row
constexpr int kGradRPL = 64 / kGradCPR;          // rows per load
constexpr int kGradRows = 32 * (1 + kGradCB);    // staged rows per block: dy, then w_o
constexpr int kGradLoads = kGradRows / kGradRPL;

__device__ __forceinline__ int grad_swz(int row) { return ((row >> 1) & 3) | (((row ^ (row >> 3)) & 1) << 2); }
__device__ __forceinline__ int grad_slot(int row, int chunk) { return kGradCPR * row + (chunk ^ grad_swz(row)); }

// One wave's sweep over its blocks k = 0 .. cnt - 1 (block wave + kGradWaves k
// of n) with the first NB column blocks live.  The loop body stores block k
// from registers into LDS, refills those registers with block k + kGradD and
// multiplies block k; the steady-state loop has no branch, so that the
// compiler's load counting waits only for the block being stored.
template <int NB>
__device__ __forceinline__ void grad_sweep(const uint16_t* const* src, const int* dst, v4i* lds, int wave,
                                           int cnt, int nblk, int lane, v16f* acc) {
  constexpr int L = (32 / kGradRPL) * (1 + NB);  // loads per block: dy rows, then the live w_o rows
  v4i reg[kGradD][L];
  auto issue = [&](int k, v4i* r) {
    int blk = wave + kGradWaves * k;
    blk = blk < nblk ? blk : nblk - 1;  // the first kGradD loads of a short sweep
    const int64_t off = kGradBW * static_cast<int64_t>(blk);
#pragma unroll
    for (int t = 0; t < L; ++t) r[t] = *reinterpret_cast<const v4i*>(src[t] + off);
  };
  const int rrow = lane & 31, rchunk = lane >> 5;
  auto step = [&](v4i* r, bool refill, int next) {
#pragma unroll
    for (int t = 0; t < L; ++t) lds[dst[t]] = r[t];
    if (refill) issue(next, r);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int st = 0; st < kGradBW / 16; ++st) {
      const v8h a = __builtin_bit_cast(v8h, lds[grad_slot(rrow, 2 * st + rchunk)]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const v8h bv = __builtin_bit_cast(v8h, lds[grad_slot(32 + 32 * b + rrow, 2 * st + rchunk)]);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bv, acc[b], 0, 0, 0);
      }
    }
    // The next block's stores to this region come after these reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Unconditional, so that the loop's load counting starts from one state.
#pragma unroll
  for (int d = 0; d < kGradD; ++d) issue(d, reg[d]);
  int k0 = 0;
  for (; k0 + 2 * kGradD <= cnt; k0 += kGradD) {
#pragma unroll
    for (int d = 0; d < kGradD; ++d) step(reg[d], true, k0 + d + kGradD);
  }
  // Fewer than 2 kGradD blocks remain.
#pragma unroll
  for (int d = 0; d < kGradD; ++d) {
    if (k0 + d < cnt) {
      if (k0 + d + kGradD < cnt) step(reg[d], true, k0 + d + kGradD);
      else step(reg[d], false, 0);
    }
  }
#pragma unroll
  for (int d = 0; d < kGradD; ++d)
    if (k0 + kGradD + d < cnt) step(reg[d], false, 0);
}

__global__ __launch_bounds__(kGradThreads) void outlier_grad_kernel(const uint16_t* __restrict__ dy,
                                                                   const uint16_t* __restrict__ w_o, int64_t M,
                                                                   int64_t N, int nO, int ldO,
                                                                   float* __restrict__ cb) {
  static_assert(kGradCB == 2, "the sweep is instantiated for one or two live column blocks");
  __shared__ v4i stage[kGradWaves][kGradCPR * kGradRows];
  __shared__ float red[kGradWaves / 2][kGradCB][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int jb0 = blockIdx.y * kGradCB;
  // Load t brings rows kGradRPL t .. kGradRPL (t + 1) - 1 of the block: lane l
  // takes row kGradRPL t + l / kGradCPR, chunk l % kGradCPR.  Rows past M
  // repeat row M - 1, columns past nO repeat row nO - 1 (their sums are
  // dropped at the store); a column block wholly past nO is neither loaded
  // nor multiplied.
  const uint16_t* src[kGradLoads];
  int dst[kGradLoads];
#pragma unroll
  for (int t = 0; t < kGradLoads; ++t) {
    const int row = kGradRPL * t + lane / kGradCPR, chunk = lane % kGradCPR;
    if (row < 32) {
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      src[t] = dy + m * N + 8 * chunk;
    } else {
      int j = 32 * jb0 + row - 32;
      j = j < nO ? j : nO - 1;
      src[t] = w_o + static_cast<int64_t>(j) * N + 8 * chunk;
    }
    dst[t] = grad_slot(row, chunk);
  }
  const int nblk = static_cast<int>(N / kGradBW);
  const int cnt = nblk > wave ? (nblk - wave + kGradWaves - 1) / kGradWaves : 0;
  v16f acc[kGradCB];
#pragma unroll
  for (int b = 0; b < kGradCB; ++b) acc[b] = v16f{};
  if (32 * (jb0 + 1) < nO) grad_sweep<2>(src, dst, stage[wave], wave, cnt, nblk, lane, acc);
  else grad_sweep<1>(src, dst, stage[wave], wave, cnt, nblk, lane, acc);
  // Pairwise reduction over the waves in a fixed order.
#pragma unroll
  for (int span = kGradWaves / 2; span >= 1; span /= 2) {
    if (wave >= span && wave < 2 * span) {
#pragma unroll
      for (int b = 0; b < kGradCB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - span][b][v][lane] = acc[b][v];
    }
    __syncthreads();
    if (wave < span) {
#pragma unroll
      for (int b = 0; b < kGradCB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] += red[wave][b][v][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // Lane l holds column (l & 31) and rows frag_row(v, l) of each block.
#pragma unroll
  for (int b = 0; b < kGradCB; ++b) {
    const int j = 32 * (jb0 + b) + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + frag_row(v, lane);
      if (j < ldO && row < M) cb[row * ldO + j] = j < nO ? acc[b][v] : 0.0f;
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
  }
  QLIN_REQUIRE(K / 64 <= 0x7fffffffLL, QLIN_ERR_SHAPE, "K too large");
  momentum_kernel<<<dim3(static_cast<unsigned>(K / 64)), kStripThreads, 0, as_stream(stream)>>>(
      x, M, K, O, nO, wmax_O, gamma, s, r);
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

extern "C" qlin_status qlin_quaff_backward(const uint16_t* dy, int64_t M, int64_t N, int64_t K,
                                           const uint16_t* sw, const void* w8t, const float* s, const float* r,
                                           const int32_t* O, int32_t nO, const uint16_t* w_o, int8_t* gq,
                                           float* gs, float* cb, uint16_t* dx, int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_REQUIRE(N > 0 && N % 128 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 128", (long long)N);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(dy);
  QLIN_PTR(sw);
  QLIN_PTR(w8t);
  QLIN_PTR(s);
  QLIN_PTR(r);
  QLIN_PTR(gq);
  QLIN_PTR(gs);
  QLIN_PTR(dx);
  QLIN_OPT_PTR(acc);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_PTR(w_o);
    QLIN_PTR(cb);
  } else {
    QLIN_REQUIRE(O == nullptr && w_o == nullptr && cb == nullptr, QLIN_ERR_INVALID_ARG,
                 "O, w_o and cb must be NULL when nO == 0");
  }
  const int64_t gx = (M + 31) / 32;
  QLIN_REQUIRE(gx <= 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  hipStream_t st = as_stream(stream);
  qlin_status rc = launch_quant_grad(dy, M, N, sw, gq, gs, st);
  if (rc != QLIN_OK) return rc;
  if (nO > 0) {
    const int ldO = static_cast<int>(outlier_ld(nO));
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>((ldO + 32 * kGradCB - 1) / (32 * kGradCB)));
    outlier_grad_kernel<<<grid, kGradThreads, 0, st>>>(dy, w_o, M, N, nO, ldO, cb);
    QLIN_LAUNCH_CHECK("outlier_grad_kernel");
  }
  return launch_gemm_bwd(gq, gs, w8t, r, s, O, nO, cb, M, N, K, dx, acc, st);
}
