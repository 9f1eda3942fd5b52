// Offline weight preparation of libqlin (gfx950): quantization of frozen fp16
// weights and packing into the tiled layouts of layout.hpp.  Not on the
// per-token path; written for clarity, one thread per output column.
#include "common.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

constexpr int kColThreads = 256;  // 64 columns x 4 k slices
constexpr int kCols = 64;
constexpr int kSlices = kColThreads / kCols;

__device__ __forceinline__ int sym_weight_code(float w, float step, int lo, int hi) {
  if (step == 0.0f) return 0;
  float q = rint_f(div_rn(w, step));
  q = fminf(fmaxf(q, static_cast<float>(lo)), static_cast<float>(hi));
  return static_cast<int>(q);
}

// Symmetric per-column: step = fp16(max|W| / qmax), code = clamp(rint(W / step)).
__global__ __launch_bounds__(kColThreads) void quant_sym_kernel(const uint16_t* __restrict__ w, int64_t K,
                                                                int64_t N, int qmax, int lo,
                                                                int8_t* __restrict__ codes,
                                                                uint16_t* __restrict__ scale) {
  __shared__ float red[kSlices][kCols];
  const int c = threadIdx.x % kCols, sl = threadIdx.x / kCols;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kCols + c;
  float a = 0.0f;
  for (int64_t k = sl; k < K; k += kSlices) a = fmaxf(a, fabsf(h2f(w[k * N + n])));
  red[sl][c] = a;
  __syncthreads();
  a = red[0][c];
#pragma unroll
  for (int i = 1; i < kSlices; ++i) a = fmaxf(a, red[i][c]);
  const uint16_t step16 = f2h(div_rn(a, static_cast<float>(qmax)));
  const float step = h2f(step16);
  if (sl == 0) scale[n] = step16;
  for (int64_t k = sl; k < K; k += kSlices)
    codes[k * N + n] = static_cast<int8_t>(sym_weight_code(h2f(w[k * N + n]), step, lo, qmax));
}

// QQQ per-group: s_g = fp16(max_g|W| / 7), codes, s_c = fp16(max|W| / 127),
// ratio = fp16(s_g / s_c).  Groups of 128 along k.
__global__ __launch_bounds__(kColThreads) void quant_group_kernel(
    const uint16_t* __restrict__ w, int64_t K, int64_t N, int8_t* __restrict__ codes,
    uint16_t* __restrict__ gscale, uint16_t* __restrict__ cscale, uint16_t* __restrict__ ratio) {
  __shared__ float red[kSlices][kCols];
  const int c = threadIdx.x % kCols, sl = threadIdx.x / kCols;
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kCols + c;
  const int64_t G = K / 128;
  float amax = 0.0f;
  for (int64_t g = 0; g < G; ++g) {
    float a = 0.0f;
    for (int64_t k = g * 128 + sl; k < (g + 1) * 128; k += kSlices) a = fmaxf(a, fabsf(h2f(w[k * N + n])));
    __syncthreads();
    red[sl][c] = a;
    __syncthreads();
    a = red[0][c];
#pragma unroll
    for (int i = 1; i < kSlices; ++i) a = fmaxf(a, red[i][c]);
    amax = fmaxf(amax, a);
    const uint16_t sg16 = f2h(div_rn(a, 7.0f));
    const float sg = h2f(sg16);
    if (sl == 0) gscale[g * N + n] = sg16;
    for (int64_t k = g * 128 + sl; k < (g + 1) * 128; k += kSlices)
      codes[k * N + n] = static_cast<int8_t>(sym_weight_code(h2f(w[k * N + n]), sg, -8, 7));
  }
  if (sl == 0) {
    const uint16_t sc16 = f2h(div_rn(amax, 127.0f));
    const float sc = h2f(sc16);
    cscale[n] = sc16;
    for (int64_t g = 0; g < G; ++g)
      ratio[g * N + n] = (sc == 0.0f) ? f2h(0.0f) : f2h(div_rn(h2f(gscale[g * N + n]), sc));
  }
}

// OffQ weights: W'' = (1/128) H diag(d) W per 128-row block (exact in float64:
// fp16 inputs, sums below 2^23 with at most 47 significant bits), rounded once
// to fp32, then per-column asymmetric int4 over k.  W'' is recomputed in the
// second pass rather than stored.
constexpr int kOffCols = 32;
constexpr int kOffSlices = kColThreads / kOffCols;

__device__ void offq_block(const uint16_t* __restrict__ w, const int8_t* __restrict__ signs, int64_t N,
                           int64_t n0, int64_t k0, double (*buf)[kOffCols]) {
  // buf[i][c] = d_i * W[k0 + i, n0 + c]
  for (int idx = threadIdx.x; idx < 128 * kOffCols; idx += kColThreads) {
    const int i = idx / kOffCols, c = idx % kOffCols;
    const double v = static_cast<double>(h2f(w[(k0 + i) * N + n0 + c]));
    buf[i][c] = signs[k0 + i] < 0 ? -v : v;
  }
  __syncthreads();
  for (int h = 1; h < 128; h <<= 1) {
    for (int idx = threadIdx.x; idx < 64 * kOffCols; idx += kColThreads) {
      const int p = idx / kOffCols, c = idx % kOffCols;
      const int i = ((p / h) * 2 * h) + (p % h);  // index with bit h clear
      const double a = buf[i][c], b = buf[i + h][c];
      buf[i][c] = a + b;
      buf[i + h][c] = a - b;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kColThreads) void quant_offq_kernel(
    const uint16_t* __restrict__ w, int64_t K, int64_t N, const int8_t* __restrict__ signs,
    uint8_t* __restrict__ codes, float* __restrict__ scale, int32_t* __restrict__ zero,
    int32_t* __restrict__ colsum) {
  __shared__ double buf[128][kOffCols];
  __shared__ float rmin[kOffSlices][kOffCols], rmax[kOffSlices][kOffCols];
  __shared__ int rsum[kOffSlices][kOffCols];
  const int c = threadIdx.x % kOffCols, sl = threadIdx.x / kOffCols;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kOffCols;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t k0 = 0; k0 < K; k0 += 128) {
    offq_block(w, signs, N, n0, k0, buf);
    for (int i = sl; i < 128; i += kOffSlices) {
      const float t = static_cast<float>(buf[i][c] / 128.0);
      mn = fminf(mn, t);
      mx = fmaxf(mx, t);
    }
    __syncthreads();
  }
  rmin[sl][c] = mn;
  rmax[sl][c] = mx;
  __syncthreads();
  mn = rmin[0][c];
  mx = rmax[0][c];
#pragma unroll
  for (int i = 1; i < kOffSlices; ++i) {
    mn = fminf(mn, rmin[i][c]);
    mx = fmaxf(mx, rmax[i][c]);
  }
  const float rng = sub_rn(mx, mn);
  const float inv = (rng == 0.0f) ? 1.0f : div_rn(15.0f, rng);
  const float step = (rng == 0.0f) ? 1.0f : div_rn(rng, 15.0f);
  const int z = static_cast<int>(rint_f(mul_rn(-mn, inv)));
  int sum = 0;
  for (int64_t k0 = 0; k0 < K; k0 += 128) {
    __syncthreads();
    offq_block(w, signs, N, n0, k0, buf);
    for (int i = sl; i < 128; i += kOffSlices) {
      const float t = static_cast<float>(buf[i][c] / 128.0);
      int code = static_cast<int>(rint_f(mul_rn(t, inv))) + z;
      code = code < 0 ? 0 : (code > 15 ? 15 : code);
      sum += code;
      codes[(k0 + i) * N + n0 + c] = static_cast<uint8_t>(code);
    }
  }
  rsum[sl][c] = sum;
  __syncthreads();
  if (sl == 0) {
    int total = 0;
    for (int i = 0; i < kOffSlices; ++i) total += rsum[i][c];
    scale[n0 + c] = step;
    zero[n0 + c] = z;
    colsum[n0 + c] = total;
  }
}

// Column sums of the codes over each group of 128 k (the group-wise W4A4
// zero-point correction): one thread per (group, column), rows read
// coalesced across the columns.
__global__ __launch_bounds__(kColThreads) void colsum_group_kernel(const uint8_t* __restrict__ codes, int64_t K,
                                                                   int64_t N, int32_t* __restrict__ out) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * kColThreads + threadIdx.x;
  const int64_t g = blockIdx.y;
  if (n >= N) return;
  const uint8_t* p = codes + g * 128 * N + n;
  int sum = 0;
  for (int i = 0; i < 128; ++i) sum += p[i * N];
  out[g * N + n] = sum;
}

// ---------------------------------------------------------------- packing
// One thread writes one 16-byte lane chunk of the packed layout (layout.hpp).
// K and N are those of the packed matrix; TRANSPOSED packs the transpose of
// codes [N x K] (row-major), so that element (k, n) is codes[n * K + k].
template <bool TRANSPOSED>
__global__ void pack_w8_kernel(const int8_t* __restrict__ codes, int64_t K, int64_t N,
                               uint8_t* __restrict__ out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= K * N / 16) return;
  const int lane = static_cast<int>(q & 63);
  const int64_t nt = (q >> 6) / (K / 32);
  const int64_t s = (q >> 6) % (K / 32);
  const int64_t n = nt * 32 + (lane & 31);
  const int64_t kb = s * 32 + 16 * (lane >> 5);
  uint32_t word[4] = {0, 0, 0, 0};
  for (int j = 0; j < 16; ++j) {
    const int8_t c = TRANSPOSED ? codes[n * K + kb + j] : codes[(kb + j) * N + n];
    word[j >> 2] |= static_cast<uint32_t>(static_cast<uint8_t>(c)) << (8 * (j & 3));
  }
  *reinterpret_cast<uint4*>(out + q * 16) = make_uint4(word[0], word[1], word[2], word[3]);
}

template <bool SIGNED_SHIFT>
__global__ void pack_w4_kernel(const uint8_t* __restrict__ codes, int64_t K, int64_t N,
                               uint8_t* __restrict__ out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= K * N / 32) return;
  const int lane = static_cast<int>(q & 63);
  const int64_t nt = (q >> 6) / (K / 64);
  const int64_t p = (q >> 6) % (K / 64);
  const int64_t n = nt * 32 + (lane & 31);
  uint32_t word[4] = {0, 0, 0, 0};
  for (int half = 0; half < 2; ++half) {
    const int64_t kb = p * 64 + half * 32 + 16 * (lane >> 5);
    uint32_t nib[16];
    for (int j = 0; j < 16; ++j) nib[j] = static_cast<uint32_t>(codes[(kb + j) * N + n]) & 0xfu;
    for (int i = 0; i < 2; ++i) {
      uint32_t v = 0;
      for (int b = 0; b < 4; ++b) {
        const uint32_t byte = SIGNED_SHIFT ? (nib[8 * i + b] | (nib[8 * i + 4 + b] << 4))
                                           : (nib[8 * i + 2 * b] | (nib[8 * i + 2 * b + 1] << 4));
        v |= byte << (8 * b);
      }
      word[2 * half + i] = v;
    }
  }
  *reinterpret_cast<uint4*>(out + q * 16) = make_uint4(word[0], word[1], word[2], word[3]);
}

// W_O fp16 [nO x N] -> lane tiles of 32 columns x 16 rows (zero rows past nO).
__global__ void pack_wo_kernel(const uint16_t* __restrict__ wo, int64_t nO, int64_t ldO, int64_t N,
                               uint8_t* __restrict__ out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (q >= ldO * N / 8) return;
  const int lane = static_cast<int>(q & 63);
  const int64_t nt = (q >> 6) % (N / 32);
  const int64_t s = (q >> 6) / (N / 32);
  const int64_t n = nt * 32 + (lane & 31);
  const int64_t jb = s * 16 + 8 * (lane >> 5);
  uint32_t word[4] = {0, 0, 0, 0};
  for (int i = 0; i < 8; ++i) {
    const uint32_t v = (jb + i < nO) ? wo[(jb + i) * N + n] : 0u;
    word[i >> 1] |= v << (16 * (i & 1));
  }
  *reinterpret_cast<uint4*>(out + q * 16) = make_uint4(word[0], word[1], word[2], word[3]);
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_quant_weight_sym(const uint16_t* w, int64_t K, int64_t N, int32_t bits,
                                             int8_t* codes, uint16_t* scale, void* stream) {
  QLIN_K_N(K, N);
  QLIN_DIMS(K, N);
  QLIN_REQUIRE(bits == 8 || bits == 4, QLIN_ERR_UNSUPPORTED, "bits=%d: only 8 and 4 are provided", bits);
  QLIN_PTR(w);
  QLIN_PTR(codes);
  QLIN_PTR(scale);
  const int qmax = bits == 8 ? 127 : 7, lo = bits == 8 ? -127 : -8;
  quant_sym_kernel<<<dim3(static_cast<unsigned>(N / kCols)), kColThreads, 0, as_stream(stream)>>>(
      w, K, N, qmax, lo, codes, scale);
  QLIN_LAUNCH_CHECK("quant_sym_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_quant_weight_group(const uint16_t* w, int64_t K, int64_t N,
                                               int32_t group, int8_t* codes, uint16_t* group_scale,
                                               uint16_t* channel_scale, uint16_t* ratio,
                                               void* stream) {
  QLIN_K_N(K, N);
  QLIN_DIMS(K, N);
  QLIN_REQUIRE(group == 128, QLIN_ERR_UNSUPPORTED, "group=%d: only 128 is provided", group);
  QLIN_PTR(w);
  QLIN_PTR(codes);
  QLIN_PTR(group_scale);
  QLIN_PTR(channel_scale);
  QLIN_PTR(ratio);
  quant_group_kernel<<<dim3(static_cast<unsigned>(N / kCols)), kColThreads, 0, as_stream(stream)>>>(
      w, K, N, codes, group_scale, channel_scale, ratio);
  QLIN_LAUNCH_CHECK("quant_group_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_quant_weight_offq(const uint16_t* w, int64_t K, int64_t N,
                                              const int8_t* signs, int32_t block, uint8_t* codes,
                                              float* scale, int32_t* zero, int32_t* colsum,
                                              void* stream) {
  QLIN_K_N(K, N);
  QLIN_DIMS(K, N);
  QLIN_REQUIRE(block == 128, QLIN_ERR_UNSUPPORTED, "block=%d: only 128 is provided", block);
  QLIN_PTR(w);
  QLIN_PTR(signs);
  QLIN_PTR(codes);
  QLIN_PTR(scale);
  QLIN_PTR(zero);
  QLIN_PTR(colsum);
  quant_offq_kernel<<<dim3(static_cast<unsigned>(N / kOffCols)), kColThreads, 0, as_stream(stream)>>>(
      w, K, N, signs, codes, scale, zero, colsum);
  QLIN_LAUNCH_CHECK("quant_offq_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_weight_colsum_group(const uint8_t* codes, int64_t K, int64_t N, int32_t group,
                                                int32_t* colsum_g, void* stream) {
  QLIN_K_N(K, N);
  QLIN_DIMS(K, N);
  QLIN_REQUIRE(group == 128, QLIN_ERR_UNSUPPORTED, "group=%d: only 128 is provided", group);
  QLIN_PTR(codes);
  QLIN_PTR(colsum_g);
  QLIN_REQUIRE(K / 128 <= 65535, QLIN_ERR_SHAPE, "K=%lld too large", (long long)K);
  const dim3 grid(static_cast<unsigned>((N + kColThreads - 1) / kColThreads), static_cast<unsigned>(K / 128));
  colsum_group_kernel<<<grid, kColThreads, 0, as_stream(stream)>>>(codes, K, N, colsum_g);
  QLIN_LAUNCH_CHECK("colsum_group_kernel");
  return QLIN_OK;
}

extern "C" int32_t qlin_outlier_ld(int32_t nO) {
  return nO < 0 ? 0 : static_cast<int32_t>(outlier_ld(nO));
}

extern "C" size_t qlin_packed_bytes(int32_t layout, int64_t K, int64_t N) {
  if (!dims_ok(K, N)) return 0;
  // The transposed layout packs the [N x K] matrix: N is its reduction length.
  if (layout == QLIN_LAYOUT_W8T) return (K <= 0 || K % 64 || N <= 0 || N % 128) ? 0 : static_cast<size_t>(K * N);
  if (N <= 0 || N % 64) return 0;
  if (layout == QLIN_LAYOUT_WO) return K <= 0 ? 0 : static_cast<size_t>(outlier_ld(K) * N * 2);
  if (K <= 0 || K % 128) return 0;
  switch (layout) {
    case QLIN_LAYOUT_W8: return static_cast<size_t>(K * N);
    case QLIN_LAYOUT_W8T: return static_cast<size_t>(K * N);
    case QLIN_LAYOUT_W4S:
    case QLIN_LAYOUT_W4U: return static_cast<size_t>(K * N / 2);
    default: return 0;
  }
}

extern "C" qlin_status qlin_pack_weight(int32_t layout, const void* codes, int64_t K, int64_t N,
                                        void* packed, void* stream) {
  QLIN_REQUIRE(layout == QLIN_LAYOUT_W8 || layout == QLIN_LAYOUT_W4S || layout == QLIN_LAYOUT_W4U ||
                   layout == QLIN_LAYOUT_WO || layout == QLIN_LAYOUT_W8T,
               QLIN_ERR_INVALID_ARG, "layout=%d is not a QLIN_LAYOUT_* value", layout);
  if (layout == QLIN_LAYOUT_W8T) {
    QLIN_K_N(N, K);  // the packed matrix is [N x K]
    QLIN_DIMS(K, N);
  } else if (layout == QLIN_LAYOUT_WO) {
    QLIN_REQUIRE(K > 0, QLIN_ERR_SHAPE, "nO=%lld must be positive", (long long)K);
    QLIN_REQUIRE(N > 0 && N % 64 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 64", (long long)N);
    QLIN_DIMS(K, N);
  } else {
    QLIN_K_N(K, N);
    QLIN_DIMS(K, N);
  }
  QLIN_PTR(codes);
  QLIN_PTR(packed);
  constexpr int T = 256;
  hipStream_t st = as_stream(stream);
  if (layout == QLIN_LAYOUT_W8) {
    const int64_t total = K * N / 16;
    pack_w8_kernel<false><<<dim3(static_cast<unsigned>((total + T - 1) / T)), T, 0, st>>>(
        static_cast<const int8_t*>(codes), K, N, static_cast<uint8_t*>(packed));
  } else if (layout == QLIN_LAYOUT_W8T) {
    const int64_t total = K * N / 16;
    pack_w8_kernel<true><<<dim3(static_cast<unsigned>((total + T - 1) / T)), T, 0, st>>>(
        static_cast<const int8_t*>(codes), N, K, static_cast<uint8_t*>(packed));
  } else if (layout == QLIN_LAYOUT_WO) {
    const int64_t ldO = outlier_ld(K);
    const int64_t total = ldO * N / 8;
    pack_wo_kernel<<<dim3(static_cast<unsigned>((total + T - 1) / T)), T, 0, st>>>(
        static_cast<const uint16_t*>(codes), K, ldO, N, static_cast<uint8_t*>(packed));
  } else {
    const int64_t total = K * N / 32;
    const dim3 grid(static_cast<unsigned>((total + T - 1) / T));
    if (layout == QLIN_LAYOUT_W4S)
      pack_w4_kernel<true><<<grid, T, 0, st>>>(static_cast<const uint8_t*>(codes), K, N, static_cast<uint8_t*>(packed));
    else
      pack_w4_kernel<false><<<grid, T, 0, st>>>(static_cast<const uint8_t*>(codes), K, N, static_cast<uint8_t*>(packed));
  }
  QLIN_LAUNCH_CHECK("pack_weight");
  return QLIN_OK;
}
