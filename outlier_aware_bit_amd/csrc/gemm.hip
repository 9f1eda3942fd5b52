// Integer GEMMs of libqlin on gfx950 int8 matrix cores (v_mfma_i32_16x16x64_i8):
//   qlin_gemm_w8a8  int8 x int8, fused dequant, optional fused Quaff compensation
//   qlin_gemm_w4a8  QQQ W4A8: per channel (shift-by-4 unpack) or per group of
//                   128 (fused fp16 dequant-quant in the K loop)
//   qlin_gemm_w4a4  OffQ-style asymmetric int4 x int4 with the zero-point
//                   correction in the epilogue
//
// Two kernels serve all of them, specialised by an operand policy:
//   * gemm_tile: 128 x 128 output tiles, four waves of 64 x 64, K in stages of
//     128.  Each stage is fetched with 16-byte global loads into registers
//     (while the previous stage is multiplied), unpacked to int8 on the way
//     into LDS (double buffered, 16-byte chunks XOR-swizzled by row so the
//     fragment reads of 8 consecutive rows hit distinct banks), then read back
//     as MFMA fragments.
//   * gemm_skinny: M <= 64 (decode).  Weight bound: each workgroup owns NT
//     16-column tiles, its waves split K, every weight byte is loaded exactly
//     once straight into MFMA fragments (the packed layout is fragment
//     ordered), and the waves' int32 partial sums meet in LDS.
#include "common.hpp"
#include "comp.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

enum class BOp { W8, W4Shift, W4Group, W4U };
enum class AOp { I8, U4 };

struct GemmArgs {
  const void* a;           // int8 [M x K] or packed uint4 [M x K/2]
  const float* sa;         // [M]
  const uint8_t* b;        // packed weights
  const uint16_t* sw_h;    // fp16 [N] (W8A8, W4A8)
  const float* sw_f;       // fp32 [N] (W4A4)
  const uint16_t* ratio;   // fp16 [K/128 x N] (per group)
  const int32_t* za;       // [M]  (W4A4)
  const int32_t* rowsum;   // [M]
  const int32_t* zw;       // [N]
  const int32_t* colsum;   // [N]
  const int8_t* qO;        // compensation (W8A8)
  const int32_t* O;
  int nO;
  const float* s;
  const uint16_t* WO;
  uint16_t* y;
  int32_t* acc;
  int64_t M, N, K;
};

// ---------------------------------------------------------------- unpacking
// int4 pairs -> int8 bytes.  Shift path: the nibble lands in the high half of
// the byte, i.e. the signed byte reads 16*q4 (QQQ's INT4 -> INT8 left shift).
__device__ __forceinline__ uint32_t shift_lo(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t shift_hi(uint32_t w) { return w & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t mask_lo(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t mask_hi(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// QQQ per-group requantization of one 32-bit word of the W4S layout (8 signed
// nibbles) into 8 int8 values in natural k order (two words):
//   w8 = clamp(rint(fp16(q4 * r)), -127, 127).
// Packed fp16 arithmetic, two values per instruction:
//   nibble ^ 8 in the low mantissa bits of 1024.0 gives 1024 + q4 + 8, minus
//   1032 gives q4 exactly; one fp16 multiply by r rounds the exact product
//   once; after clamping, adding 1536.0 (spacing 1 on [1024, 2048)) rounds to
//   an integer n with ties to even and leaves n's two's complement in the low
//   byte of the fp16 pattern.
__device__ __forceinline__ void requant_word(uint32_t w, v2h rr, uint32_t& out_lo, uint32_t& out_hi) {
  const uint32_t xw = w ^ 0x88888888u;
  uint32_t pr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t bits = ((xw >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
    v2h h = __builtin_bit_cast(v2h, bits);
    h = h - v2h{static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
    h = h * rr;
    h = __builtin_elementwise_max(h, v2h{static_cast<_Float16>(-127.0f), static_cast<_Float16>(-127.0f)});
    h = __builtin_elementwise_min(h, v2h{static_cast<_Float16>(127.0f), static_cast<_Float16>(127.0f)});
    h = h + v2h{static_cast<_Float16>(1536.0f), static_cast<_Float16>(1536.0f)};
    pr[p] = __builtin_bit_cast(uint32_t, h);
  }
  // Nibble p of the word holds k = {0,4,1,5}[p] (low half) and {2,6,3,7}[p]
  // (high half) relative to the word's 8-value slice.
  out_lo = __builtin_amdgcn_perm(pr[2], pr[0], 0x06020400u);  // k 0,1,2,3
  out_hi = __builtin_amdgcn_perm(pr[3], pr[1], 0x06020400u);  // k 4,5,6,7
}

// 16 packed bytes of a W4 lane chunk -> two 16-byte int8 chunks (k steps 0, 1).
template <BOp B>
__device__ __forceinline__ void unpack_w4(uint4 raw, v2h rr, v4i& c0, v4i& c1) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (B == BOp::W4Shift) {
      o[2 * i] = shift_lo(w[i]);
      o[2 * i + 1] = shift_hi(w[i]);
    } else if constexpr (B == BOp::W4U) {
      o[2 * i] = mask_lo(w[i]);
      o[2 * i + 1] = mask_hi(w[i]);
    } else {
      requant_word(w[i], rr, o[2 * i], o[2 * i + 1]);
    }
  }
  c0 = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  c1 = v4i{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
}

// 8 packed bytes of int4 activations (natural packing) -> 16 int8 values in
// the same k order as unpack_w4<W4U>.
__device__ __forceinline__ v4i unpack_a4(uint32_t w0, uint32_t w1) {
  return v4i{(int)mask_lo(w0), (int)mask_hi(w0), (int)mask_lo(w1), (int)mask_hi(w1)};
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- epilogue
// Per output element: int32 accumulator -> fp16 (and the optional raw int32).
template <BOp B>
__device__ __forceinline__ int32_t finish_acc(int32_t raw, const GemmArgs& g, int64_t m, int64_t n) {
  if constexpr (B == BOp::W4Shift) {
    return raw >> 4;  // every product is 16 * q * q4: the division is exact
  } else if constexpr (B == BOp::W4U) {
    const int64_t za = g.za[m], zw = g.zw[n];
    const int64_t v = static_cast<int64_t>(raw) - zw * g.rowsum[m] - za * g.colsum[n] + g.K * za * zw;
    return static_cast<int32_t>(v);
  } else {
    return raw;
  }
}

template <BOp B>
__device__ __forceinline__ float col_scale(const GemmArgs& g, int64_t n) {
  if constexpr (B == BOp::W4U)
    return g.sw_f[n];
  else
    return h2f(g.sw_h[n]);
}

// ============================================================ tiled kernel
constexpr int kBM = 128, kBN = 128, kBK = 128, kTileThreads = 256;
constexpr int kTM = 4, kTN = 4;  // 16x16 fragments per wave (64 x 64)
constexpr int kStageBytes = (kBM + kBN) * kBK;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 4); }

template <BOp B, AOp A>
struct TileLoader {
  // Registers holding one stage between its global load and its LDS store.
  static constexpr int kAChunks = (A == AOp::I8) ? (kBM * 8) / kTileThreads : (kBM * 4) / kTileThreads;
  static constexpr int kBChunks = (B == BOp::W8) ? (kBN / 16 * 128) / kTileThreads : (kBN / 16 * 64) / kTileThreads;
  uint4 ra[kAChunks];
  uint4 rb[kBChunks];
  v2h rr[kBChunks];

  __device__ __forceinline__ void load(const GemmArgs& g, int64_t m0, int64_t n0, int s) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kTileThreads;
      if constexpr (A == AOp::I8) {
        const int row = q >> 3, c = q & 7;
        const int64_t m = m0 + row;
        ra[i] = (m < g.M) ? *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(g.a) + m * g.K + s * kBK + c * 16)
                          : make_uint4(0, 0, 0, 0);
      } else {
        const int row = q >> 2, c = q & 3;
        const int64_t m = m0 + row;
        ra[i] = (m < g.M) ? *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(g.a) + m * (g.K / 2) + s * (kBK / 2) + c * 16)
                          : make_uint4(0, 0, 0, 0);
      }
    }
    const int64_t ntiles = g.N / 16;
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int q = tid + i * kTileThreads;
      if constexpr (B == BOp::W8) {
        const int nt = q >> 7, ks = (q >> 6) & 1, lane = q & 63;
        const int64_t gnt = n0 / 16 + nt;
        rb[i] = (gnt < ntiles) ? *reinterpret_cast<const uint4*>(g.b + ((static_cast<int64_t>(2 * s + ks) * ntiles + gnt) << 10) + lane * 16)
                               : make_uint4(0, 0, 0, 0);
      } else {
        const int nt = q >> 6, lane = q & 63;
        const int64_t gnt = n0 / 16 + nt;
        rb[i] = (gnt < ntiles) ? *reinterpret_cast<const uint4*>(g.b + ((static_cast<int64_t>(s) * ntiles + gnt) << 10) + lane * 16)
                               : make_uint4(0, 0, 0, 0);
        if constexpr (B == BOp::W4Group) {
          const int64_t n = gnt * 16 + (lane & 15);
          const uint16_t r16 = (gnt < ntiles) ? g.ratio[static_cast<int64_t>(s) * g.N + n] : 0;
          const _Float16 r = __builtin_bit_cast(_Float16, r16);
          rr[i] = v2h{r, r};
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int tid = threadIdx.x;
    uint8_t* la = lds;
    uint8_t* lb = lds + kBM * kBK;
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int q = tid + i * kTileThreads;
      if constexpr (A == AOp::I8) {
        const int row = q >> 3, c = q & 7;
        *reinterpret_cast<uint4*>(la + swz(row, c)) = ra[i];
      } else {
        const int row = q >> 2, c = q & 3;
        *reinterpret_cast<v4i*>(la + swz(row, 2 * c)) = unpack_a4(ra[i].x, ra[i].y);
        *reinterpret_cast<v4i*>(la + swz(row, 2 * c + 1)) = unpack_a4(ra[i].z, ra[i].w);
      }
    }
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int q = tid + i * kTileThreads;
      if constexpr (B == BOp::W8) {
        const int nt = q >> 7, ks = (q >> 6) & 1, lane = q & 63;
        const int col = nt * 16 + (lane & 15);
        *reinterpret_cast<uint4*>(lb + swz(col, ks * 4 + (lane >> 4))) = rb[i];
      } else {
        const int nt = q >> 6, lane = q & 63;
        const int col = nt * 16 + (lane & 15);
        v4i c0, c1;
        unpack_w4<B>(rb[i], rr[i], c0, c1);
        *reinterpret_cast<v4i*>(lb + swz(col, lane >> 4)) = c0;
        *reinterpret_cast<v4i*>(lb + swz(col, 4 + (lane >> 4))) = c1;
      }
    }
  }
};

template <BOp B, AOp A, bool COMP>
__global__ __launch_bounds__(kTileThreads) void gemm_tile(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * kBM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kBN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wrow0 = (wave >> 1) * 64, wcol0 = (wave & 1) * 64;

  v4i acc[kTM][kTN];
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b) acc[a][b] = v4i{0, 0, 0, 0};

  const int S = static_cast<int>(g.K / kBK);
  TileLoader<B, A> ld;
  ld.load(g, m0, n0, 0);
  ld.store(lds);
  __syncthreads();
  for (int s = 0; s < S; ++s) {
    const uint8_t* cur = lds + (s & 1) * kStageBytes;
    if (s + 1 < S) ld.load(g, m0, n0, s + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v4i af[kTM], bf[kTN];
      const int chunk = ks * 4 + (lane >> 4);
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm)
        af[tm] = *reinterpret_cast<const v4i*>(cur + swz(wrow0 + tm * 16 + (lane & 15), chunk));
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn)
        bf[tn] = *reinterpret_cast<const v4i*>(cur + kBM * kBK + swz(wcol0 + tn * 16 + (lane & 15), chunk));
#pragma unroll
      for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
        for (int tn = 0; tn < kTN; ++tn) acc[tm][tn] = mfma_i8(af[tm], bf[tn], acc[tm][tn]);
    }
    if (s + 1 < S) ld.store(lds + ((s + 1) & 1) * kStageBytes);
    __syncthreads();
  }

  // Epilogue.  Fragment (tm, tn), register i of lane l holds
  // row wrow0 + 16 tm + 4 (l >> 4) + i, column wcol0 + 16 tn + (l & 15).
  v4f accf[kTM][kTN];
#pragma unroll
  for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
    for (int tn = 0; tn < kTN; ++tn) {
      const int64_t n = n0 + wcol0 + tn * 16 + (lane & 15);
      const float sw = (n < g.N) ? col_scale<B>(g, n) : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wrow0 + tm * 16 + 4 * (lane >> 4) + i;
        int32_t v = acc[tm][tn][i];
        if (m < g.M && n < g.N) {
          v = finish_acc<B>(v, g, m, n);
          if (g.acc != nullptr) g.acc[m * g.N + n] = v;
        }
        accf[tm][tn][i] = static_cast<float>(v) * sw;
      }
    }
  if constexpr (COMP) {
    comp_accumulate<kBM, kBN, kTileThreads, kTM, kTN>(accf, g.qO, g.O, g.nO, g.s, g.WO, g.M, g.N, g.K,
                                                       m0, n0, wrow0, wcol0, lds);
  }
#pragma unroll
  for (int tm = 0; tm < kTM; ++tm)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wrow0 + tm * 16 + 4 * (lane >> 4) + i;
      if (m >= g.M) continue;
      const float sam = g.sa[m];
#pragma unroll
      for (int tn = 0; tn < kTN; ++tn) {
        const int64_t n = n0 + wcol0 + tn * 16 + (lane & 15);
        if (n < g.N) g.y[m * g.N + n] = f2h(accf[tm][tn][i] * sam);
      }
    }
}

// ============================================================ skinny kernel
// M <= 16*MT.  Workgroup: WAVES waves, NT 16-column tiles; wave w takes the
// K stages s = w, w + WAVES, ...
template <BOp B, AOp A, int MT, int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny(GemmArgs g) {
  __shared__ int red[MT * NT * 4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nt0 = static_cast<int64_t>(blockIdx.x) * NT;
  const int64_t ntiles = g.N / 16;
  const int S = static_cast<int>(g.K / 128);

  for (int i = threadIdx.x; i < MT * NT * 4 * 64; i += 64 * WAVES) (&red[0][0])[i] = 0;

  v4i acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = v4i{0, 0, 0, 0};

  const int row = lane & 15, grp = lane >> 4;
  for (int s = wave; s < S; s += WAVES) {
    v4i bf[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t gnt = nt0 + nt;
      const bool ok = gnt < ntiles;
      if constexpr (B == BOp::W8) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint4 raw = ok ? *reinterpret_cast<const uint4*>(g.b + ((static_cast<int64_t>(2 * s + ks) * ntiles + gnt) << 10) + lane * 16)
                               : make_uint4(0, 0, 0, 0);
          bf[nt][ks] = v4i{(int)raw.x, (int)raw.y, (int)raw.z, (int)raw.w};
        }
      } else {
        const uint4 raw = ok ? *reinterpret_cast<const uint4*>(g.b + ((static_cast<int64_t>(s) * ntiles + gnt) << 10) + lane * 16)
                             : make_uint4(0, 0, 0, 0);
        v2h rr = v2h{static_cast<_Float16>(0.0f), static_cast<_Float16>(0.0f)};
        if constexpr (B == BOp::W4Group) {
          const uint16_t r16 = ok ? g.ratio[static_cast<int64_t>(s) * g.N + gnt * 16 + row] : 0;
          const _Float16 r = __builtin_bit_cast(_Float16, r16);
          rr = v2h{r, r};
        }
        unpack_w4<B>(raw, rr, bf[nt][0], bf[nt][1]);
      }
    }
    v4i af[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = mt * 16 + row;
      const bool ok = m < g.M;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (A == AOp::I8) {
          const uint4 raw = ok ? *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(g.a) + m * g.K + s * 128 + ks * 64 + grp * 16)
                               : make_uint4(0, 0, 0, 0);
          af[mt][ks] = v4i{(int)raw.x, (int)raw.y, (int)raw.z, (int)raw.w};
        } else {
          const uint2 raw = ok ? *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(g.a) + m * (g.K / 2) + (s * 128 + ks * 64 + grp * 16) / 2)
                               : make_uint2(0, 0);
          af[mt][ks] = unpack_a4(raw.x, raw.y);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_i8(af[mt][ks], bf[nt][ks], acc[mt][nt]);
  }

  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(&red[(mt * NT + nt) * 4 + i][lane], acc[mt][nt][i]);
  __syncthreads();

  for (int f = wave; f < MT * NT; f += WAVES) {
    const int mt = f / NT, nt = f % NT;
    const int64_t n = (nt0 + nt) * 16 + row;
    if (n >= g.N) continue;
    const float sw = col_scale<B>(g, n);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = mt * 16 + 4 * grp + i;
      if (m >= g.M) continue;
      const int32_t v = finish_acc<B>(red[f * 4 + i][lane], g, m, n);
      if (g.acc != nullptr) g.acc[m * g.N + n] = v;
      g.y[m * g.N + n] = f2h(static_cast<float>(v) * sw * g.sa[m]);
    }
  }
}

// ------------------------------------------------------------ dispatch
template <BOp B, AOp A>
qlin_status launch(const GemmArgs& g, bool comp, hipStream_t st) {
  if (!comp && g.M <= 64) {
    constexpr int NT = 2, WAVES = 8;
    const dim3 grid(static_cast<unsigned>((g.N / 16 + NT - 1) / NT));
    if (g.M <= 16)
      gemm_skinny<B, A, 1, NT, WAVES><<<grid, 64 * WAVES, 0, st>>>(g);
    else if (g.M <= 32)
      gemm_skinny<B, A, 2, NT, WAVES><<<grid, 64 * WAVES, 0, st>>>(g);
    else
      gemm_skinny<B, A, 4, NT, WAVES><<<grid, 64 * WAVES, 0, st>>>(g);
    QLIN_LAUNCH_CHECK("gemm_skinny");
    return QLIN_OK;
  }
  const int64_t gy = (g.M + kBM - 1) / kBM;
  QLIN_REQUIRE(gy <= 65535, QLIN_ERR_SHAPE, "M=%lld too large", (long long)g.M);
  const dim3 grid(static_cast<unsigned>((g.N + kBN - 1) / kBN), static_cast<unsigned>(gy));
  if constexpr (B == BOp::W8 && A == AOp::I8) {
    if (comp) {
      gemm_tile<B, A, true><<<grid, kTileThreads, 0, st>>>(g);
      QLIN_LAUNCH_CHECK("gemm_tile");
      return QLIN_OK;
    }
  }
  gemm_tile<B, A, false><<<grid, kTileThreads, 0, st>>>(g);
  QLIN_LAUNCH_CHECK("gemm_tile");
  return QLIN_OK;
}

GemmArgs base_args(int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc) {
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.y = y;
  g.acc = acc;
  return g;
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_gemm_w8a8(const int8_t* qa, const float* sa, const void* w8,
                                      const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                      const int8_t* qO, const int32_t* O, int32_t nO, const float* s,
                                      const uint16_t* WO, uint16_t* y, int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(qa);
  QLIN_PTR(sa);
  QLIN_PTR(w8);
  QLIN_PTR(sw);
  QLIN_PTR(y);
  QLIN_OPT_PTR(acc);
  if (nO > 0) {
    QLIN_PTR(qO);
    QLIN_PTR(O);
    QLIN_PTR(s);
    QLIN_PTR(WO);
  } else {
    QLIN_REQUIRE(qO == nullptr && O == nullptr && s == nullptr && WO == nullptr, QLIN_ERR_INVALID_ARG,
                 "qO, O, s and WO must be NULL when nO == 0");
  }
  GemmArgs g = base_args(M, N, K, y, acc);
  g.a = qa;
  g.sa = sa;
  g.b = static_cast<const uint8_t*>(w8);
  g.sw_h = sw;
  g.qO = qO;
  g.O = O;
  g.nO = nO;
  g.s = s;
  g.WO = WO;
  return launch<BOp::W8, AOp::I8>(g, nO > 0, as_stream(stream));
}

extern "C" qlin_status qlin_gemm_w4a8(const int8_t* qa, const float* sa, const void* w4,
                                      const uint16_t* sw, const uint16_t* ratio, int32_t group,
                                      int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc,
                                      void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  QLIN_REQUIRE(group == 0 || group == 128, QLIN_ERR_UNSUPPORTED, "group=%d: only 0 and 128 are provided", group);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(qa);
  QLIN_PTR(sa);
  QLIN_PTR(w4);
  QLIN_PTR(sw);
  QLIN_PTR(y);
  QLIN_OPT_PTR(acc);
  if (group == 128)
    QLIN_PTR(ratio);
  else
    QLIN_REQUIRE(ratio == nullptr, QLIN_ERR_INVALID_ARG, "ratio must be NULL when group == 0");
  GemmArgs g = base_args(M, N, K, y, acc);
  g.a = qa;
  g.sa = sa;
  g.b = static_cast<const uint8_t*>(w4);
  g.sw_h = sw;
  g.ratio = ratio;
  if (group == 128) return launch<BOp::W4Group, AOp::I8>(g, false, as_stream(stream));
  return launch<BOp::W4Shift, AOp::I8>(g, false, as_stream(stream));
}

extern "C" qlin_status qlin_gemm_w4a4(const uint8_t* qa4, const float* sa, const int32_t* za,
                                      const int32_t* rowsum, const void* w4, const float* sw,
                                      const int32_t* zw, const int32_t* colsum, int64_t M, int64_t N,
                                      int64_t K, uint16_t* y, int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(qa4);
  QLIN_PTR(sa);
  QLIN_PTR(za);
  QLIN_PTR(rowsum);
  QLIN_PTR(w4);
  QLIN_PTR(sw);
  QLIN_PTR(zw);
  QLIN_PTR(colsum);
  QLIN_PTR(y);
  QLIN_OPT_PTR(acc);
  GemmArgs g = base_args(M, N, K, y, acc);
  g.a = qa4;
  g.sa = sa;
  g.b = static_cast<const uint8_t*>(w4);
  g.sw_f = sw;
  g.za = za;
  g.rowsum = rowsum;
  g.zw = zw;
  g.colsum = colsum;
  return launch<BOp::W4U, AOp::U4>(g, false, as_stream(stream));
}
