// Integer GEMMs of libqlin on gfx950 matrix cores (v_mfma_i32_32x32x32_i8;
// the group-wise W4A4 product on the fp8 form, v_mfma_f32_32x32x64_f8f6f4):
//   qlin_gemm_w8a8  int8 x int8, fused dequant, optional fused Quaff compensation
//   qlin_gemm_w4a8  QQQ W4A8: per channel (shift-by-4 unpack) or per group of
//                   128 (fused fp16 dequant-quant inside the K loop)
//   qlin_gemm_w4a4  OffQ-style asymmetric int4 x int4 with the zero-point
//                   correction in the epilogue
//   qlin_gemm_w4a4_group  the same with a step and zero point per token and
//                   128-k group: each group's exact partial sum is scaled
//                   into fp32 accumulators inside the K loop
//
// Two kernels serve all of them, specialised by an operand policy.
//
// gemm_tile (M > 128, with a compensation term, or group-wise W4A4): a
// workgroup computes a (32*TM) x 256 tile with four waves side by side, each
// owning 64 distinct output columns (32*TM x 64 per wave, 2*TM accumulator
// fragments of 32 x 32), or, for 128-row int8 tiles, eight waves of 32
// columns (two per SIMD).
//   * Weights never touch LDS: the packed layout is in MFMA fragment order, so
//     each wave streams its own columns straight from memory into registers
//     with one 16-byte load per lane per fragment (int4 weights at half the
//     bytes), up to two K stages ahead of use, and unpacks them in registers.
//   * The K loop is unrolled over the period of the register rotation with no
//     branches inside (prefetch indices are clamped to the last stage), so
//     the accumulators stay in place in the accumulation registers.
//   * Activations, shared by the waves, go global -> registers -> LDS
//     (double buffered, loaded two stages of 128 k ahead), stored as 16-byte chunks
//     XOR-swizzled by row so that fragment reads and row stores are free of
//     bank conflicts.
//   * Workgroups are mapped to tiles in groups of 4 tile rows, with each
//     XCD (every 8th workgroup) given a contiguous block of tiles so the
//     operands it streams stay in its own L2.
// gemm_skinny (M <= 128: decode and small batches): bound by the weight stream.  A workgroup
// owns NT 32-column tiles, its waves split K, every weight byte is loaded
// once straight into MFMA fragments with U units of 64 k in flight per lane,
// and the waves' int32 partial sums meet in LDS.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "comp.hpp"
#include "internal.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

enum class BOp { W8, W4Shift, W4Group, W4U };
// U4G: int4 activations with a step and zero point per (token, 128-k group).
enum class AOp { I8, U4, U4G };

struct GemmArgs {
  const void* a;          // int8 [M x K] or packed uint4 [M x K/2]
  const float* sa;        // [M]
  const uint8_t* b;       // packed weights
  const uint16_t* sw_h;   // fp16 [N] (W8A8, W4A8)
  const float* sw_f;      // fp32 [N] (W4A4)
  const uint16_t* ratio;  // fp16 [K/128 x N] (per group)
  const int32_t* za;      // [M]  (W4A4); group-wise: [M x K/128], as sa and rowsum
  const int32_t* rowsum;  // [M]
  const int32_t* zw;      // [N]
  const int32_t* colsum;  // [N]; group-wise W4A4: [K/128 x N]
  const uint16_t* xO;     // fp16 [M x ldO] compensation operand (W8A8)
  const uint8_t* WOp;     // packed fp16 W_O
  int ldO;
  // STE backward (COMP == 3): s [N], outlier indices O [nO] (increasing),
  // cb fp32 [M x ldO]; sa holds the gradient steps, sw_f the column factors r.
  const float* s;
  const int32_t* O;
  int nO;
  const float* cb;
  uint16_t* y;
  int32_t* acc;
  int64_t M, N, K;
};

// ---------------------------------------------------------------- unpacking
// Shift path: the nibble lands in the high half of the byte, i.e. the signed
// byte reads 16*q4 (QQQ's INT4 -> INT8 left shift).
__device__ __forceinline__ uint32_t shift_lo(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t shift_hi(uint32_t w) { return w & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t mask_lo(uint32_t w) { return w & 0x0F0F0F0Fu; }
__device__ __forceinline__ uint32_t mask_hi(uint32_t w) { return (w >> 4) & 0x0F0F0F0Fu; }

// QQQ per-group requantization of one 32-bit word of the W4S layout (8 signed
// nibbles) into 8 int8 values in natural k order (two words):
//   w8 = clamp(rint(fp16(q4 * r)), -127, 127).
// Packed fp16 arithmetic, two values per instruction: nibble ^ 8 in the low
// mantissa bits of 1024.0 gives 1024 + q4 + 8, minus 1032 gives q4 exactly;
// one fp16 multiply by r rounds the exact product once; after clamping, adding
// 1536.0 (spacing 1 on [1024, 2048)) rounds to an integer n with ties to even
// and leaves n's two's complement in the low byte of the fp16 pattern.
__device__ __forceinline__ void requant_word(uint32_t w, v2h rr, uint32_t& out_lo, uint32_t& out_hi) {
  const v2h r2 = __builtin_shufflevector(rr, rr, 0, 0);  // the ratio is the low half of rr
  const uint32_t xw = w ^ 0x88888888u;
  const v2h off = {static_cast<_Float16>(1032.0f), static_cast<_Float16>(1032.0f)};
  const v2h lo = {static_cast<_Float16>(-127.0f), static_cast<_Float16>(-127.0f)};
  const v2h hi = {static_cast<_Float16>(127.0f), static_cast<_Float16>(127.0f)};
  const v2h magic = {static_cast<_Float16>(1536.0f), static_cast<_Float16>(1536.0f)};
  uint32_t pr[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t bits = ((xw >> (4 * p)) & 0x000F000Fu) | 0x64006400u;
    v2h h = __builtin_bit_cast(v2h, bits);
    h = h - off;
    h = h * r2;
    h = __builtin_elementwise_min(__builtin_elementwise_max(h, lo), hi);
    h = h + magic;
    pr[p] = __builtin_bit_cast(uint32_t, h);
  }
  // Nibble p of the word holds k = {0,4,1,5}[p] (low half) and {2,6,3,7}[p]
  // (high half) relative to the word's 8-value slice.
  out_lo = __builtin_amdgcn_perm(pr[2], pr[0], 0x06020400u);  // k 0,1,2,3
  out_hi = __builtin_amdgcn_perm(pr[3], pr[1], 0x06020400u);  // k 4,5,6,7
}

// 16 packed bytes of a W4 lane chunk -> the int8 B fragments of k steps 0 and 1.
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

template <BOp B>
__device__ __forceinline__ void unpack_w4v(v4i raw, v2h rr, v4i& c0, v4i& c1) {
  unpack_w4<B>(make_uint4(raw[0], raw[1], raw[2], raw[3]), rr, c0, c1);
}

// 8 packed bytes of int4 activations (natural packing) -> 16 int8 values in
// the same k order as unpack_w4<W4U>.
__device__ __forceinline__ v4i unpack_a4(uint32_t w0, uint32_t w1) {
  return v4i{(int)mask_lo(w0), (int)mask_hi(w0), (int)mask_lo(w1), (int)mask_hi(w1)};
}

__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

typedef int v8i __attribute__((ext_vector_type(8)));

// Unsigned int4 codes (0..15, one per byte) on the fp8 matrix cores.  Read
// as OCP e4m3, the byte c encodes c * 2^-9 (a subnormal for c < 8), so every
// product is c * c' * 2^-18 and a 64-deep sum, at most 64 * 225 * 2^-18, is
// exact in fp32: the int32 sum of the same bytes as int8, times 2^-18, with
// the fp32 result the group-wise fold needs and no conversion.  Slot t of
// lane half h of the first operand pairs with slot t of lane half h of the
// second, as in two int8 products over the low and high register halves.
// Zero scale operands select the unscaled instruction.
__device__ __forceinline__ v16f mfma_c4(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ---------------------------------------------------------------- epilogue
template <BOp B>
__device__ __forceinline__ float col_scale(const GemmArgs& g, int64_t n) {
  if constexpr (B == BOp::W4U)
    return g.sw_f[n];
  else
    return h2f(g.sw_h[n]);
}

// ============================================================ tiled kernel
constexpr int kBN = 256, kBK = 128, kTileThreads = 256;

// LDS byte offset of 16-byte chunk `chunk` of A row `row`.  The chunk index is
// XORed with (row >> 1) & 7: the LDS serves 16 lanes per cycle over 64 banks,
// and a fragment read has lanes 0..15 on rows 0..15 at one logical chunk, so
// rows of equal parity (which share a bank half) must land on 8 different
// chunks.
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ swz_key(row)) << 4); }

// WV waves per 32*TM x 256 tile: four waves of 64 columns, or eight of 32
// (two waves per SIMD).
template <BOp B, AOp A, int TM, int WV = 4>
struct Tile {
  static_assert(WV == 4 || WV == 8, "four or eight waves per tile");
  static constexpr int kThreads = 64 * WV;
  static constexpr int kNTW = 8 / WV;  // 32-column tiles per wave
  static constexpr int BM = 32 * TM;
  static constexpr int kStage = BM * kBK;  // LDS bytes of one A stage (int8)
  static constexpr int kAChunks = (A == AOp::I8) ? BM * 8 / kThreads : BM * 4 / kThreads;
  static constexpr int kNB = ((B == BOp::W8) ? 4 : 2) * kNTW;  // 16-byte B loads per lane per stage
  static constexpr int kARowStep = (A == AOp::I8) ? kThreads / 8 : kThreads / 4;  // rows between chunks
};

// Per-thread operand pointers, computed once.  A chunk i of a stage is row
// (r0 + i * kARowStep), 16-byte column c0; B tile t of a stage is
// bptr + t_offset (uniform) for this lane.
template <BOp B, AOp A, int TM, int WV = 4>
struct TilePtrs {
  const uint8_t* a[Tile<B, A, TM, WV>::kAChunks];  // stage 0 addresses of this thread's A chunks
  int lds_a;                                   // LDS byte offset of chunk 0 (chunk i adds i * kARowStep * kBK)
  const uint8_t* b;                            // this lane's B address in tile (0, nt32)
  const uint16_t* ratio;                       // this lane's ratio column (W4Group)
};

template <BOp B, AOp A, int TM, int WV>
__device__ __forceinline__ void tile_ptrs(const GemmArgs& g, int64_t m0, int64_t nt32, TilePtrs<B, A, TM, WV>& p) {
  using T = Tile<B, A, TM, WV>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int row0 = (A == AOp::I8) ? (tid >> 3) : (tid >> 2);
  const int c0 = (A == AOp::I8) ? (tid & 7) : (tid & 3);
  const int64_t lda = (A == AOp::I8) ? g.K : g.K / 2;
#pragma unroll
  for (int i = 0; i < T::kAChunks; ++i) {
    int64_t m = m0 + row0 + i * T::kARowStep;
    m = m < g.M ? m : g.M - 1;
    p.a[i] = static_cast<const uint8_t*>(g.a) + m * lda + c0 * 16;
  }
  p.lds_a = (A == AOp::I8) ? swz(row0, c0) : swz(row0, 2 * c0);
  const int64_t kt = (B == BOp::W8) ? g.K / 32 : g.K / 64;  // lane tiles per 32-column strip
  p.b = g.b + ((nt32 * kt) << 10) + lane * 16;
  p.ratio = g.ratio + nt32 * 32 + (lane & 31);
}

template <BOp B, AOp A, int TM, int WV>
__device__ __forceinline__ void load_a(const TilePtrs<B, A, TM, WV>& p, int s,
                                       v4i (&ra)[Tile<B, A, TM, WV>::kAChunks]) {
  constexpr int stage_bytes = (A == AOp::I8) ? kBK : kBK / 2;
#pragma unroll
  for (int i = 0; i < Tile<B, A, TM, WV>::kAChunks; ++i)
    ra[i] = *reinterpret_cast<const v4i*>(p.a[i] + static_cast<int64_t>(s) * stage_bytes);
}

template <BOp B, AOp A, int TM, int WV>
__device__ __forceinline__ void store_a(uint8_t* buf, int lds_a, const v4i (&ra)[Tile<B, A, TM, WV>::kAChunks]) {
  using T = Tile<B, A, TM, WV>;
#pragma unroll
  for (int i = 0; i < T::kAChunks; ++i) {
    // Rows of chunk i differ from chunk 0 by a multiple of 32: same swizzle key.
    uint8_t* d = buf + lds_a + i * T::kARowStep * kBK;
    if constexpr (A == AOp::I8) {
      *reinterpret_cast<v4i*>(d) = ra[i];
    } else {
      // swz(row, 2c + 1) is swz(row, 2c) with the chunk bit 0 flipped.
      const int base = lds_a + i * T::kARowStep * kBK;
      *reinterpret_cast<v4i*>(buf + base) = unpack_a4(ra[i][0], ra[i][1]);
      *reinterpret_cast<v4i*>(buf + (base ^ 16)) = unpack_a4(ra[i][2], ra[i][3]);
    }
  }
}

// Part KS (k step KS of the stage) of the B loads of stage s for this wave:
// 32-column tiles nt32 .. nt32 + kNTW - 1.  int8 weights: one tile per k step
// and column tile; int4 weights (four waves): one tile holds two k steps, so
// part KS loads tile (kp = KS >> 1, nt = KS & 1), and the per-group ratios
// come with part 0.
template <BOp B, AOp A, int TM, int KS, int WV>
__device__ __forceinline__ void load_b_part(const TilePtrs<B, A, TM, WV>& p, int64_t kt, int64_t N, int s,
                                            v4i (&rb)[Tile<B, A, TM, WV>::kNB], v2h (&rr)[2]) {
  if constexpr (B == BOp::W8) {
    constexpr int kNTW = Tile<B, A, TM, WV>::kNTW;
#pragma unroll
    for (int nt = 0; nt < kNTW; ++nt)
      rb[KS * kNTW + nt] =
          *reinterpret_cast<const v4i*>(p.b + ((static_cast<int64_t>(4 * s + KS) + nt * kt) << 10));
  } else {
    static_assert(WV == 4, "int4 weights take two column tiles per wave");
    constexpr int kp = KS >> 1, nt = KS & 1;
    rb[kp * 2 + nt] = *reinterpret_cast<const v4i*>(p.b + ((static_cast<int64_t>(2 * s + kp) + nt * kt) << 10));
    if constexpr (B == BOp::W4Group && KS == 0) {
      // The ratio stays in the low half as loaded (zero-extended, no
      // instruction): packing it into both halves here, next to its load in
      // the k step's schedule, waited for every load in flight.
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2)
        rr[n2] = __builtin_bit_cast(v2h, static_cast<uint32_t>(p.ratio[static_cast<int64_t>(s) * N + n2 * 32]));
    }
  }
}

template <BOp B, AOp A, int TM, int WV>
__device__ __forceinline__ void load_b(const TilePtrs<B, A, TM, WV>& p, int64_t kt, int64_t N, int s,
                                       v4i (&rb)[Tile<B, A, TM, WV>::kNB], v2h (&rr)[2]) {
  load_b_part<B, A, TM, 0, WV>(p, kt, N, s, rb, rr);
  load_b_part<B, A, TM, 1, WV>(p, kt, N, s, rb, rr);
  load_b_part<B, A, TM, 2, WV>(p, kt, N, s, rb, rr);
  load_b_part<B, A, TM, 3, WV>(p, kt, N, s, rb, rr);
}

// Chunks [P * n / 2, (P + 1) * n / 2) of this thread's A loads of stage s
// (with a single chunk, all of it in part 1).
template <BOp B, AOp A, int TM, int P, int WV>
__device__ __forceinline__ void load_a_half(const TilePtrs<B, A, TM, WV>& p, int s,
                                            v4i (&ra)[Tile<B, A, TM, WV>::kAChunks]) {
  constexpr int n = Tile<B, A, TM, WV>::kAChunks, stage_bytes = (A == AOp::I8) ? kBK : kBK / 2;
#pragma unroll
  for (int i = P * n / 2; i < (P + 1) * n / 2; ++i)
    ra[i] = *reinterpret_cast<const v4i*>(p.a[i] + static_cast<int64_t>(s) * stage_bytes);
}

// Group-wise W4A4: the constants of one 128-k group (one K stage) for this
// lane's TM token rows -- the step and d = rowsum - 128 za (code sum less
// the zero point's share), as sa * 2^18 and d * 2^-18 (both exact): the
// fp8 products carry a factor 2^-18 that the first cancels.
template <int TM>
struct GroupC {
  float sa[TM];
  float d[TM];
};

// The tile's per-group token constants, staged in LDS kGcChunk groups at a
// time: sa * 2^18 and (rowsum - 128 za) * 2^-18 of every (row, group), row
// pitch kGcChunk + 1 words so that the 32 rows a wave reads at one group
// fall in 32 different banks.  A token's groups are contiguous in memory,
// so these loads are coalesced; a per-stage load of one group for the
// wave's token rows touches a separate 128-byte line per row, and those
// loads, not the vector work, set the pace of the group-wise product
// (2048 x 4096 x 14336: 229 us with them, 158 us from LDS).
constexpr int kGcChunk = 48;
constexpr int kGcBatch = 6;  // entries per thread in flight when a later chunk is loaded

// kB entries per thread are loaded before they are stored: the whole share
// at kernel start, a few at a time inside the K loop, where the prefetched
// operands hold most registers.
template <int TM, int kB>
__device__ __forceinline__ void gc_stage_chunk(const GemmArgs& g, int64_t m0, int64_t c0, float* gsa, float* gd) {
  constexpr int kPer = 32 * TM * kGcChunk / kTileThreads;
  static_assert(kPer % kB == 0, "batch must divide the per-thread share");
  // The empty asm keeps the address arithmetic here: hoisted out of the K
  // loop, the per-entry offsets would hold registers for its whole length.
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const int64_t G = g.K / kBK;
#pragma unroll
  for (int k0 = 0; k0 < kPer; k0 += kB) {
    float sv[kB], dv[kB];
    // Clamped, unconditional loads (rows past M and groups past G repeat
    // the last ones; nothing reads them back).
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int i = t + kTileThreads * (k0 + k), row = i / kGcChunk, gg = i % kGcChunk;
      int64_t m = m0 + row;
      m = m < g.M ? m : g.M - 1;
      int64_t gi = c0 + gg;
      gi = gi < G ? gi : G - 1;
      const int64_t o = m * G + gi;
      sv[k] = g.sa[o] * 262144.0f;
      dv[k] = static_cast<float>(g.rowsum[o] - 128 * g.za[o]) * 0x1p-18f;
    }
#pragma unroll
    for (int k = 0; k < kB; ++k) {
      const int i = t + kTileThreads * (k0 + k), row = i / kGcChunk, gg = i % kGcChunk;
      gsa[row * (kGcChunk + 1) + gg] = sv[k];
      gd[row * (kGcChunk + 1) + gg] = dv[k];
    }
  }
}

// The constants of group s (s % kGcChunk within the staged chunk) for this
// lane's TM token rows.
template <int TM>
__device__ __forceinline__ void load_group(const float* gsa, const float* gd, int s, GroupC<TM>& c) {
  const int r = threadIdx.x & 31, gg = s % kGcChunk;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    c.sa[tm] = gsa[(32 * tm + r) * (kGcChunk + 1) + gg];
    c.d[tm] = gd[(32 * tm + r) * (kGcChunk + 1) + gg];
  }
}

// End of group s: with raw = sum over the group of qa * qw (exact; the fp8
// products give f = raw * 2^-18, and 0 <= raw <= 128 * 225),
//   cf += sa_g * fp32(raw)                        per element
//   P  += sa_g * fp32(rowsum_g - 128 * za_g)      per token row
// each one fma of the scaled constants (the same rounding as of sa_g and
// fp32(raw)), and after the last group group_zero_corr adds
//   sum_g (-sa_g za_g) * colsum_g                 per element
// so that y = sw * (cf - zw * P) is sw * sum_g sa_g * sum_{k in g} (qa - za_g)(qw - zw).
template <int TM>
__device__ __forceinline__ void group_rescale(const v16f (&accf)[TM][2], v16f (&cf)[TM][2], float (&P)[TM],
                                              const GroupC<TM>& c) {
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const float sa = c.sa[tm];
    P[tm] = fmaf(sa, c.d[tm], P[tm]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) cf[tm][nt][v] = fmaf(sa, accf[tm][nt][v], cf[tm][nt][v]);
  }
}

// The integer sum behind an fp8 product of codes (exact: f * 2^18 is an
// integer below 2^15).
__device__ __forceinline__ int32_t raw_of(float f) { return static_cast<int32_t>(f * 262144.0f); }

// Group-wise W4A4, parity output: the raw int32 sums of group s for this
// wave's fragments, raw[s, m, n] at ((s * M) + m) * N + n.  Lane l holds token
// row m0 + 32 tm + (l & 31) and, in registers 4q..4q+3 of fragment nt, the
// four adjacent columns wcol0 + 32 nt + 8 q + 4 (l >> 5) + [0, 4).
template <int TM>
__device__ __forceinline__ void store_group_sums(const GemmArgs& g, const v16f (&accf)[TM][2], int s, int64_t m0,
                                                 int64_t wcol0, bool live) {
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  if (!live) return;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t m = m0 + 32 * tm + r;
    if (m >= g.M) continue;
    int32_t* row = g.acc + (static_cast<int64_t>(s) * g.M + m) * g.N + wcol0 + 4 * h;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<v4i*>(row + 32 * nt + 8 * q) =
            v4i{raw_of(accf[tm][nt][4 * q]), raw_of(accf[tm][nt][4 * q + 1]), raw_of(accf[tm][nt][4 * q + 2]),
                raw_of(accf[tm][nt][4 * q + 3])};
  }
}

// The activation zero points' term of the group-wise W4A4 product,
// cf[tm][nt] += sum_g w_g[m] * colsum_g[n] with w_g = -(sa_g * za_g), on fp16
// matrix cores, the groups being the k dimension (16 per
// v_mfma_f32_32x32x16_f16).  colsum (the first operand, rows n) is an integer
// of at most 128 * 15, exact in fp16.  The workgroup forms w for its 32 * TM
// token rows, kCorrG groups at a time, from coalesced row segments of sa and
// za into LDS; per chunk each token's w (the second operand, columns m) is
// scaled by the power of two 2^e that puts its largest magnitude in
// [2^14, 2^15) and split into hi + lo fp16 halves, which carry it to within
// 2^-21 of that magnitude (e then only decreases over later chunks); the
// fp32 sums are scaled back by 2^-e exactly.  Lane half h takes groups 16 c + 8 h + [0, 8), as the operand
// layout assigns k.  It runs before the K loop, between the first operand
// prefetch and its LDS stores: the first chunk's sa and za are loaded ahead
// of that prefetch (CorrIn) and the colsum loads behind it, so that their
// latencies overlap.  Called by every wave (it has barriers); waves past N
// read the last 64 columns and discard the result.
constexpr int kCorrG = 32;

template <int TM>
struct CorrIn {
  static constexpr int kPer = 32 * TM * kCorrG / kTileThreads;  // entries per thread
  float sa[kPer];
  int32_t za[kPer];
};

// Entry k of thread t: token row i = (t + 256 k) / kCorrG, group c0 + (t % kCorrG);
// consecutive threads read consecutive groups of one token.
template <int TM>
__device__ __forceinline__ void corr_load(const GemmArgs& g, int64_t m0, int64_t c0, CorrIn<TM>& ci) {
  // Loads from clamped indices are unconditional (a guarded load would be a
  // branch that waits for it); entries past the last group are zeroed after.
  const int t = threadIdx.x;
  const int64_t G = g.K / kBK, gg = c0 + t % kCorrG, gc = gg < G ? gg : G - 1;
#pragma unroll
  for (int k = 0; k < CorrIn<TM>::kPer; ++k) {
    int64_t m = m0 + (t + kTileThreads * k) / kCorrG;
    m = m < g.M ? m : g.M - 1;
    ci.sa[k] = g.sa[m * G + gc];
    ci.za[k] = g.za[m * G + gc];
  }
  if (gg >= G) {
#pragma unroll
    for (int k = 0; k < CorrIn<TM>::kPer; ++k) ci.za[k] = 0;
  }
}

template <int TM>
__device__ __forceinline__ void group_zero_corr(v16f (&cf)[TM][2], const GemmArgs& g, int64_t m0, int64_t wcol0,
                                                bool live, uint8_t* lds, CorrIn<TM>& ci) {
  constexpr int kPitch = kCorrG + 1;  // the odd pitch spreads token rows over the banks
  const int t = threadIdx.x, lane = t & 63, h = lane >> 5, r = lane & 31;
  const int64_t G = g.K / kBK;
  float* const wl = reinterpret_cast<float*>(lds);
  const int32_t* csn = g.colsum + (live ? wcol0 : g.N - 64) + r;
  // cf (zero on entry) accumulates in units of 2^-e[tm]; e only decreases
  // from chunk to chunk, so rescaling cf is an exact power-of-two step down.
  int e[TM];
  for (int64_t c0 = 0; c0 < G; c0 += kCorrG) {
    if (c0 > 0) corr_load<TM>(g, m0, c0, ci);
#pragma unroll
    for (int k = 0; k < CorrIn<TM>::kPer; ++k)
      wl[((t + kTileThreads * k) / kCorrG) * kPitch + t % kCorrG] = -(ci.sa[k] * static_cast<float>(ci.za[k]));
    lds_barrier();
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const float* wr = wl + (32 * tm + r) * kPitch + 8 * h;
      float mx = 0.0f;
#pragma unroll
      for (int c = 0; c < kCorrG / 16; ++c)
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(wr[16 * c + j]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      int x;
      frexpf(mx, &x);  // mx in [2^(x-1), 2^x); x = 0 for mx = 0
      const int ec = 15 - x;
      if (c0 == 0) {
        e[tm] = ec;
      } else if (ec < e[tm]) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int v = 0; v < 16; ++v) cf[tm][nt][v] = ldexpf(cf[tm][nt][v], ec - e[tm]);
        e[tm] = ec;
      }
    }
#pragma unroll
    for (int c = 0; c < kCorrG / 16; ++c) {
      v8h ca[2], wh[TM], wo[TM];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t gg = c0 + 16 * c + 8 * h + j, gc = gg < G ? gg : G - 1;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int32_t v = csn[gc * g.N + 32 * nt];  // unconditional, from a clamped row
          ca[nt][j] = static_cast<_Float16>(static_cast<float>(gg < G ? v : 0));
        }
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float sc = ldexpf(wl[(32 * tm + r) * kPitch + 16 * c + 8 * h + j], e[tm]);
          const _Float16 hi = static_cast<_Float16>(sc);
          wh[tm][j] = hi;
          wo[tm][j] = static_cast<_Float16>(sc - static_cast<float>(hi));
        }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          cf[tm][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ca[nt], wh[tm], cf[tm][nt], 0, 0, 0);
          cf[tm][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ca[nt], wo[tm], cf[tm][nt], 0, 0, 0);
        }
    }
    lds_barrier();  // the chunk's LDS rows are read before they are refilled
  }
  if (G > 0) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int v = 0; v < 16; ++v) cf[tm][nt][v] = ldexpf(cf[tm][nt][v], -e[tm]);
  }
}

template <int TM>
__device__ __forceinline__ void read_frags(const uint8_t* buf, int ks, v4i (&af)[TM]) {
  const int lane = threadIdx.x & 63;
  const int arow = lane & 31, ahalf = lane >> 5;
  const uint8_t* abuf = buf + arow * kBK + (((2 * ks + ahalf) ^ swz_key(arow)) << 4);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) af[tm] = *reinterpret_cast<const v4i*>(abuf + tm * 32 * kBK);
}

// The same fragments into the low (HI = 0) or high (HI = 1) halves of the
// fp8 operands of the group-wise product.
template <int TM, int HI>
__device__ __forceinline__ void read_frags_half(const uint8_t* buf, int ks, v8i (&af)[TM]) {
  const int lane = threadIdx.x & 63;
  const int arow = lane & 31, ahalf = lane >> 5;
  const uint8_t* abuf = buf + arow * kBK + (((2 * ks + ahalf) ^ swz_key(arow)) << 4);
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const v4i v = *reinterpret_cast<const v4i*>(abuf + tm * 32 * kBK);
    if constexpr (HI)
      af[tm].hi = v;
    else
      af[tm].lo = v;
  }
}

template <int Mask, int N>
__device__ __forceinline__ void sched_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(Mask, N, 0);
}

// Issue order of one k step (2*TM MFMAs with four waves, TM with eight).  A
// wave issues in order (alone on its SIMD with four waves), so a burst of
// memory instructions that fills a queue stalls the matrix-core instructions
// behind it: the next k step's fragment
// reads go first (a full k step of cover), then pairs of MFMAs, each pair
// followed by its share of the global loads and LDS stores of the k step.
template <int NP, int NVM, int NDS, int P>
__device__ __forceinline__ void sched_kpair() {
  sched_group<0x008, 2>();                                       // MFMA
  sched_group<0x020, (P + 1) * NVM / NP - P * NVM / NP>();       // global load
  sched_group<0x200, (P + 1) * NDS / NP - P * NDS / NP>();       // LDS write
}

// Ps: the k step's pairs of MFMAs, 0 .. NP - 1.
template <int TM, int NVM, int NDS, int... Ps>
__device__ __forceinline__ void sched_kstep(std::integer_sequence<int, Ps...>) {
  sched_group<0x100, TM>();  // LDS fragment reads of the next k step
  (sched_kpair<static_cast<int>(sizeof...(Ps)), NVM, NDS, Ps>(), ...);
}

// The group-wise product's k steps: an even one has no matrix-core work
// (fragment reads, then loads and stores); an odd one issues its 2*TM
// products in pairs with its loads and stores, then the fragment reads that
// overwrite the low operand halves.
template <int TM, int NVM, int NDS>
__device__ __forceinline__ void sched_kstep_c4_even() {
  sched_group<0x100, TM>();
  sched_group<0x020, NVM>();
  sched_group<0x200, NDS>();
}

template <int TM, int NVM, int NDS, int... Ps>
__device__ __forceinline__ void sched_kstep_c4_odd(std::integer_sequence<int, Ps...>) {
  (sched_kpair<static_cast<int>(sizeof...(Ps)), NVM, NDS, Ps>(), ...);
  sched_group<0x100, TM>();
}

// Stage barrier.  The last TM LDS operations of the wave are the fragment
// reads of the next stage (from a buffer completed before the previous
// barrier) and may stay in flight; everything before them -- in particular
// this stage's stores of a future stage -- has completed, since LDS
// operations of a wave complete in order.
template <int TM>
__device__ __forceinline__ void stage_barrier() {
  static_assert(TM == 2 || TM == 4 || TM == 8, "lgkmcnt immediate");
  if constexpr (TM == 2)
    asm volatile("s_waitcnt lgkmcnt(2)\n\ts_barrier" ::: "memory");
  else if constexpr (TM == 4)
    asm volatile("s_waitcnt lgkmcnt(4)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt lgkmcnt(8)\n\ts_barrier" ::: "memory");
}

// Tile index -> (tile row, tile column).  Workgroup b runs on XCD b % 8, so
// the tiles of XCD x are taken from one block of the tile grid: with a
// 2 x 4 split of the grid (tile rows in 2 blocks, tile columns in 4, which
// keeps each XCD's A rows and B columns -- the operands its L2 must fetch --
// about equal in bytes for tiles twice as wide as tall), else from a
// contiguous run of the row-grouped order.  Inside a block, tiles go in
// groups of 4 tile rows so that tiles running at the same time share rows.
__device__ __forceinline__ void group_order(int64_t idx, int64_t rows, int64_t cols, int64_t& r_out,
                                            int64_t& c_out) {
  constexpr int64_t G = 4;
  const int64_t per_group = G * cols;
  const int64_t first = (idx / per_group) * G;
  const int64_t gm = (rows - first) < G ? (rows - first) : G;
  const int64_t r = idx % per_group;
  r_out = first + r % gm;
  c_out = r / gm;
}

__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tm_idx, int64_t& tn_idx) {
  const int64_t T = tiles_m * tiles_n;
  const int64_t bid = blockIdx.x;
  if (tiles_m % 2 == 0 && tiles_n % 4 == 0) {
    const int64_t x = bid % 8, l = bid / 8;  // XCD, index within it
    const int64_t br = tiles_m / 2, bc = tiles_n / 4;
    int64_t r, c;
    group_order(l, br, bc, r, c);
    tm_idx = (x % 2) * br + r;
    tn_idx = (x / 2) * bc + c;
    return;
  }
  group_order((T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid, tiles_m, tiles_n, tm_idx, tn_idx);
}

// COMP: 0 no compensation term; 1 compensation after the K loop with xO read
// from memory; 2 compensation before the K loop, while the loop's first
// operands are in flight, with the tile's xO rows staged in LDS
// (ldO <= kXOMaxLd); 3 the STE backward epilogue, where output column k is
// scaled by r[k] and, for an outlier column k = O[j], receives
// (s[k] - 1) * cb[m, j] first; 4 (group-wise W4A4 only) the int32 sums of
// every 128-k group are also written out, raw_g[g, m, n] = sum over the
// group of qa * qw, for parity checks; 5 as 2, with the tile's W_O fragments
// also staged in LDS at the start (ldO <= kXOLdsLd): every operand of the
// compensation arrives in one round trip, under the K loop's first loads.
constexpr int kXOMaxLd = 384;
constexpr int kXOLdsLd = 208;

// Group-wise W4A4 tiles carry a per-group fold of every accumulator on the
// vector ALU: two workgroups per CU, so that one wave's fold runs while the
// other's matrix-core work and loads proceed.  WV = 8 (int8 x int8
// without the compensation or with it staged in LDS): eight waves of 32
// columns, two per SIMD, so that each CU has twice the operand loads in
// flight.
template <BOp B, AOp A, int TM, int BD, int COMP, int WV = 4>
__global__ __launch_bounds__(64 * WV, (A == AOp::U4G || (A == AOp::U4 && TM == 4)) ? 2 : 1) void gemm_tile(GemmArgs g) {
  using T = Tile<B, A, TM, WV>;
  constexpr int NTW = T::kNTW;
  static_assert(WV == 4 || (B == BOp::W8 && A == AOp::I8 && (COMP == 0 || COMP == 5)),
                "eight waves only for the int8 product, plain or with the compensation staged in LDS");
  // Three activation stages, then the epilogue constants of the tile: the
  // token steps (and W4A4 zero points / row sums) of its BM rows and the
  // column steps (and W4A4 zero points / column sums) of its 256 columns.
  constexpr bool kGrp = (A == AOp::U4G);
  constexpr bool kBwd = (COMP == 3);
  constexpr bool kGrpAcc = kGrp && COMP == 4;
  static_assert(COMP != 4 || kGrp, "per-group sums exist only in the group-wise product");
  constexpr int kRowC = (B == BOp::W4U && !kGrp) ? 3 : 1, kColC = (B == BOp::W4U || kBwd) ? 3 : 1;
  // COMP == 2 stages the tile's xO rows (BM x ldO fp16, unpadded) in the
  // same space before the activation stages are first written.
  constexpr bool kComp1st = (COMP == 2 || COMP == 5);
  // COMP == 5: xO rows, then each wave's W_O lane tiles (NTW column tiles
  // per 16 rows of W_O, ldO / 16 of them; 8 column tiles per tile).
  constexpr int kXORows = (COMP == 5) ? T::BM * 2 * kXOLdsLd : T::BM * 2 * kXOMaxLd;
  constexpr int kXO = (COMP == 2) ? kXORows : (COMP == 5) ? kXORows + 8 * (kXOLdsLd / 16) * 1024 : 0;
  static_assert(!kBwd || (B == BOp::W8 && A == AOp::I8), "the backward epilogue is int8 x int8");
  static_assert(!kComp1st || (B == BOp::W8 && A == AOp::I8), "the compensation belongs to the W8A8 product");
  constexpr int kMainBytes = (kXO > 3 * T::kStage) ? kXO : 3 * T::kStage;
  constexpr int kGcBytes = kGrp ? 2 * T::BM * (kGcChunk + 1) * 4 : 0;  // group constants (sa and d)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kMainBytes + 4 * (kRowC * T::BM + kColC * kBN) + kGcBytes];
  [[maybe_unused]] uint8_t* const xlds = lds;
  float* const c_sa = reinterpret_cast<float*>(lds + kMainBytes);
  [[maybe_unused]] int32_t* const c_za = reinterpret_cast<int32_t*>(c_sa + T::BM);
  [[maybe_unused]] int32_t* const c_rs = c_za + T::BM;
  float* const c_sw = c_sa + kRowC * T::BM;
  [[maybe_unused]] int32_t* const c_zw = reinterpret_cast<int32_t*>(c_sw + kBN);
  [[maybe_unused]] int32_t* const c_cs = c_zw + kBN;
  [[maybe_unused]] float* const gsa = reinterpret_cast<float*>(lds + kMainBytes + 4 * (kRowC * T::BM + kColC * kBN));
  [[maybe_unused]] float* const gd = gsa + T::BM * (kGcChunk + 1);
  const int64_t tiles_m = (g.M + T::BM - 1) / T::BM, tiles_n = (g.N + kBN - 1) / kBN;
  int64_t tmi, tni;
  tile_coords(tiles_m, tiles_n, tmi, tni);
  const int64_t m0 = tmi * T::BM, n0 = tni * kBN;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // N % 64 == 0: a wave's 32 * NTW columns are all in range or all out.  A
  // wave out of range still streams (clamped, in-bounds) weights so that
  // every wave takes part in every barrier; it stores nothing.
  int64_t wcol0 = n0 + 32 * NTW * wave;
  const bool live = wcol0 < g.N;
  const int64_t nt32 = (live ? wcol0 : g.N - 32 * NTW) / 32;
  const int64_t b_tiles = (B == BOp::W8) ? g.K / 32 : g.K / 64;  // lane tiles per 32-column strip

  TilePtrs<B, A, TM, WV> p;
  tile_ptrs<B, A, TM, WV>(g, m0, nt32, p);

  v16i acc[TM][NTW];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[a][b] = v16i{};
  // Group-wise: fp32 sums of the fp8 products of one group, and the fp8
  // operand fragments (low half: even k step, high half: odd k step).
  [[maybe_unused]] v16f accf[TM][2];
  [[maybe_unused]] v8i af8[TM];

  const int S = static_cast<int>(g.K / kBK);
  // Stage t of K: its weights live in B register set t % NBS (NBS = BD + 1),
  // loaded BD stages ahead; its activations in LDS buffer t % 3.  Stage s
  // reads buffer s % 3 and, at its last k step, the first fragments of
  // buffer (s+1) % 3; it stores A(s+2) (held in A register set s % 2 since
  // the previous stage) into buffer (s+2) % 3, and loads A(s+3) into set
  // (s+1) % 2.  The buffer written during stage s is read only after the
  // barriers ending stages s and s+1, and the one it overwrites was last read
  // before the barrier ending stage s-1.
  constexpr int NBS = BD + 1;
  v4i ra[2][T::kAChunks];
  v4i rb[NBS][T::kNB];
  v2h rr[NBS][2];
  v4i af[2][TM];
  // The epilogue constants are fetched first, with the first operands: they
  // arrive during the prologue instead of costing a round trip at the end.
  // Thread t takes row m0 + t % BM and column n0 + t % 256 (both clamped),
  // so that every thread loads and stores them unconditionally (threads with
  // equal indices store equal values): a load used only under a condition is
  // sunk into it, and the wait for it there would drain every operand load
  // issued before it.
  float k_sa = 0.0f, k_sw;
  [[maybe_unused]] int32_t k_za = 0, k_rs = 0, k_zw = 0, k_cs = 0, k_o = -1;
  {
    const int t = threadIdx.x;
    int64_t mc = m0 + t % T::BM;
    mc = mc < g.M ? mc : g.M - 1;
    int64_t nc = n0 + t % kBN;
    nc = nc < g.N ? nc : g.N - 1;
    if constexpr (kGrp) {
      k_sw = g.sw_f[nc];
      k_zw = g.zw[nc];
    } else if constexpr (B == BOp::W4U) {
      k_sa = g.sa[mc];
      k_za = g.za[mc];
      k_rs = g.rowsum[mc];
      k_sw = g.sw_f[nc];
      k_zw = g.zw[nc];
      k_cs = g.colsum[nc];
    } else if constexpr (kBwd) {
      // Gradient step, r[k], s[k] - 1 and the first outlier index this
      // thread checks against the tile's columns.
      k_sa = g.sa[mc];
      k_sw = g.sw_f[nc];
      k_cs = __builtin_bit_cast(int32_t, sub_rn(g.s[nc], 1.0f));
      const int32_t* const Op = (g.nO > 0) ? g.O : reinterpret_cast<const int32_t*>(g.sa);  // sa: any valid word
      const int32_t o = Op[(t < g.nO) ? t : 0];
      k_o = (t < g.nO) ? o : -1;
    } else {
      k_sa = g.sa[mc];
      k_sw = h2f(g.sw_h[nc]);
    }
  }
  auto clamp_s = [S](int t) { return t < S ? t : S - 1; };
  // fp32 accumulators: the compensation term (COMP), or the scaled group sums.
  constexpr bool kCF = COMP == 1 || kComp1st || kGrp;
  [[maybe_unused]] v16f cf[kCF ? TM : 1][NTW];
  if constexpr (kCF) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < NTW; ++b) cf[a][b] = v16f{};
  }
  if constexpr (kComp1st) {
    // The tile's xO rows go straight from memory into LDS (BM * ldO / 8
    // chunks of 16 bytes in row-major order, a multiple of 256; 64
    // consecutive chunks per wave and load), ahead of the K loop's first
    // operands.
    const int xcpr = g.ldO / 8, xchunks = T::BM * xcpr;
    for (int cw = 64 * wave; cw < xchunks; cw += T::kThreads) {
      const int c = cw + lane, row = c / xcpr, cc = c - row * xcpr;
      int64_t m = m0 + row;
      m = m < g.M ? m : g.M - 1;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(g.xO + m * g.ldO + 8 * cc),
          (__attribute__((address_space(3))) void*)(xlds + cw * 16), 16, 0, 0);
    }
    if constexpr (COMP == 5) {
      // This wave's W_O lane tiles (js, nt32 + nt), js < ldO / 16, to
      // consecutive 1 KB slots of its own region.
      const int nj = g.ldO / 16;
      const int64_t tiles32 = g.N / 32;
      uint8_t* const wl = xlds + kXORows + wave * (kXOLdsLd / 16) * NTW * 1024;
      for (int js = 0; js < nj; ++js)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void*)(g.WOp + ((static_cast<int64_t>(js) * tiles32 + nt32 + nt)
                                                                       << 10) + lane * 16),
              (__attribute__((address_space(3))) void*)(wl + (NTW * js + nt) * 1024), 16, 0, 0);
    }
  }
  // Group-wise: the first chunk of group constants goes to LDS before the
  // K loop's operand loads are issued (the barrier ahead of the loop
  // publishes it).
  if constexpr (kGrp) gc_stage_chunk<TM, 32 * TM * kGcChunk / kTileThreads>(g, m0, 0, gsa, gd);
  [[maybe_unused]] CorrIn<TM> ci;
  if constexpr (kGrp) corr_load<TM>(g, m0, 0, ci);
  load_a<B, A, TM, WV>(p, 0, ra[0]);
  load_a<B, A, TM, WV>(p, clamp_s(1), ra[1]);
#pragma unroll
  for (int j = 0; j < BD; ++j) load_b<B, A, TM, WV>(p, b_tiles, g.N, clamp_s(j), rb[j], rr[j]);
  // Group-wise: the constants of group t are read from LDS at the start of
  // stage t and used at its end.
  [[maybe_unused]] GroupC<TM> gc;
  [[maybe_unused]] float P[kGrp ? TM : 1];
  if constexpr (kGrp) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) P[tm] = 0.0f;
  }
  if constexpr (kComp1st) {
    // Wait for the staged operands only: the K loop's loads issued after
    // them may stay in flight while the compensation runs.
    constexpr int younger = 2 * T::kAChunks + BD * T::kNB;
    static_assert(younger < 64, "vmcnt immediate");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(((younger >> 4) << 14) | (15 << 8) | (7 << 4) | (younger & 15));
    lds_barrier();
    if constexpr (COMP == 5)
      comp_accumulate_lds2<TM, NTW>(cf, xlds, 2 * g.ldO, g.ldO / 16,
                                    xlds + kXORows + wave * (kXOLdsLd / 16) * NTW * 1024);
    else
      comp_accumulate_lds<TM, NTW>(cf, xlds, 2 * g.ldO, g.ldO / 16, g.WOp, g.N, nt32);
    lds_barrier();  // every wave has read the staged operands
  }
  if constexpr (kGrp) {
    static_assert(32 * TM * (kCorrG + 1) * 4 <= kMainBytes, "the w chunk exceeds the LDS buffers");
    group_zero_corr<TM>(cf, g, m0, wcol0, live, lds, ci);
  }
  store_a<B, A, TM, WV>(lds, p.lds_a, ra[0]);
  store_a<B, A, TM, WV>(lds + T::kStage, p.lds_a, ra[1]);
  load_a<B, A, TM, WV>(p, clamp_s(2), ra[0]);
  {
    const int tr = threadIdx.x % T::BM, tc = threadIdx.x % kBN;
    c_sa[tr] = k_sa;
    if constexpr (B == BOp::W4U && !kGrp) {  // group-wise: no per-row constants
      c_za[tr] = k_za;
      c_rs[tr] = k_rs;
    }
    c_sw[tc] = k_sw;
    if constexpr (B == BOp::W4U) {
      c_zw[tc] = k_zw;
      c_cs[tc] = k_cs;
    }
    if constexpr (kBwd) {
      c_zw[tc] = -1;  // outlier index of the column, marked below
      c_cs[tc] = k_cs;
    }
  }
  lds_barrier();
  if constexpr (kBwd) {
    // Mark the tile's outlier columns: c_zw[O[j] - n0] = j.  The marks are
    // read only after the K loop's barriers.
    const int t = threadIdx.x;
    if (k_o >= n0 && k_o < n0 + kBN) c_zw[k_o - n0] = t;
    for (int j = t + T::kThreads; j < g.nO; j += T::kThreads) {
      const int o = g.O[j];
      if (o >= n0 && o < n0 + kBN) c_zw[o - n0] = j;
    }
  }
  if constexpr (kGrp)
    read_frags_half<TM, 0>(lds, 0, af8);
  else
    read_frags<TM>(lds, 0, af[0]);

  constexpr int kVmB = (B == BOp::W8) ? NTW : 1;                         // B loads per k step
  constexpr int kDsW = (A == AOp::I8) ? T::kAChunks : 2 * T::kAChunks;   // LDS stores in k step 2
  auto stage = [&](auto jb, auto ja, auto jl, int st) __attribute__((always_inline)) {
    constexpr int JB = decltype(jb)::value, JA = decltype(ja)::value, JL = decltype(jl)::value;
    const int sb = clamp_s(st + BD), s3 = clamp_s(st + 3);
    const uint8_t* const cur = lds + JL * T::kStage;
    const uint8_t* const nxt = lds + ((JL + 1) % 3) * T::kStage;
    uint8_t* const fut = lds + ((JL + 2) % 3) * T::kStage;
    v4i (&rbn)[T::kNB] = rb[(JB + BD) % NBS];
    v2h (&rrn)[2] = rr[(JB + BD) % NBS];
    [[maybe_unused]] v4i bq[2][2];  // int4 weights: [nt][k step & 1], unpacked two k steps at a time
    auto kstep = [&](auto ksc) __attribute__((always_inline)) {
      constexpr int KS = decltype(ksc)::value;
      if constexpr (KS < 3)
        read_frags<TM>(cur, KS + 1, af[(KS + 1) & 1]);
      else
        read_frags<TM>(nxt, 0, af[0]);
      load_b_part<B, A, TM, KS, WV>(p, b_tiles, g.N, sb, rbn, rrn);
      if constexpr (KS == 0) load_a_half<B, A, TM, 0, WV>(p, s3, ra[1 - JA]);
      if constexpr (KS == 1) load_a_half<B, A, TM, 1, WV>(p, s3, ra[1 - JA]);
      if constexpr (KS == 2) store_a<B, A, TM, WV>(fut, p.lds_a, ra[JA]);
      v4i bf[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        if constexpr (B == BOp::W8) {
          bf[nt] = rb[JB][KS * NTW + nt];
        } else {
          if constexpr ((KS & 1) == 0) unpack_w4v<B>(rb[JB][(KS >> 1) * 2 + nt], rr[JB][nt], bq[nt][0], bq[nt][1]);
          bf[nt] = bq[nt][KS & 1];
        }
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[tm][nt] = mfma_i8(bf[nt], af[KS & 1][tm], acc[tm][nt]);
      constexpr int kVmAKS = (KS == 0) ? T::kAChunks / 2 : (KS == 1) ? T::kAChunks - T::kAChunks / 2 : 0;
      constexpr int nvm = kVmB + kVmAKS + ((B == BOp::W4Group && KS == 0) ? 2 : 0);
      sched_kstep<TM, nvm, (KS == 2) ? kDsW : 0>(std::make_integer_sequence<int, TM * NTW / 2>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    // Group-wise: int4 codes on the fp8 matrix cores, two k steps per
    // product.  An even k step reads the next k step's fragments into the
    // high operand halves and unpacks the weights of both; an odd one issues
    // the products, then reads the following k step's fragments into the low
    // halves.  Every group starts its sums afresh.
    [[maybe_unused]] v8i bq8[2];
    auto kstep_c4 = [&](auto ksc) __attribute__((always_inline)) {
      constexpr int KS = decltype(ksc)::value;
      if constexpr ((KS & 1) == 0) read_frags_half<TM, 1>(cur, KS + 1, af8);
      load_b_part<B, A, TM, KS, WV>(p, b_tiles, g.N, sb, rbn, rrn);
      if constexpr (KS == 0) load_group<TM>(gsa, gd, st, gc);
      if constexpr (KS == 0) load_a_half<B, A, TM, 0, WV>(p, s3, ra[1 - JA]);
      if constexpr (KS == 1) load_a_half<B, A, TM, 1, WV>(p, s3, ra[1 - JA]);
      if constexpr (KS == 2) store_a<B, A, TM, WV>(fut, p.lds_a, ra[JA]);
      if constexpr ((KS & 1) == 0) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          v4i c0, c1;
          unpack_w4v<B>(rb[JB][(KS >> 1) * 2 + nt], rr[JB][nt], c0, c1);
          bq8[nt] = __builtin_shufflevector(c0, c1, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      } else {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) accf[tm][nt] = mfma_c4(bq8[nt], af8[tm], KS == 1 ? v16f{} : accf[tm][nt]);
        if constexpr (KS == 1)
          read_frags_half<TM, 0>(cur, 2, af8);
        else
          read_frags_half<TM, 0>(nxt, 0, af8);
      }
      constexpr int kVmAKS = (KS == 0) ? T::kAChunks / 2 : (KS == 1) ? T::kAChunks - T::kAChunks / 2 : 0;
      constexpr int nvm = kVmB + kVmAKS;
      if constexpr ((KS & 1) == 0)
        sched_kstep_c4_even<TM, nvm, (KS == 2) ? kDsW : 0>();
      else
        sched_kstep_c4_odd<TM, nvm, 0>(std::make_integer_sequence<int, TM>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (kGrp) {
      kstep_c4(std::integral_constant<int, 0>{});
      kstep_c4(std::integral_constant<int, 1>{});
      kstep_c4(std::integral_constant<int, 2>{});
      kstep_c4(std::integral_constant<int, 3>{});
    } else {
      kstep(std::integral_constant<int, 0>{});
      kstep(std::integral_constant<int, 1>{});
      kstep(std::integral_constant<int, 2>{});
      kstep(std::integral_constant<int, 3>{});
    }
    if constexpr (kGrpAcc) store_group_sums<TM>(g, accf, st, m0, wcol0, live);
    if constexpr (kGrp) group_rescale<TM>(accf, cf, P, gc);
    stage_barrier<TM>();
    __builtin_amdgcn_sched_barrier(0);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  // Group-wise: every kGcChunk stages (a multiple of the 6-stage rotation,
  // so always ahead of a rotation) the next chunk of group constants
  // replaces the last one.  The stage barrier that ended the previous stage
  // has ended every read of the old chunk.  A branch between the stages of
  // a rotation instead splits the scheduling regions and spills registers.
  static_assert(kGcChunk % 6 == 0, "group-constant chunks must align with the stage rotation");
  auto gc_next = [&](int st) __attribute__((always_inline)) {
    if constexpr (kGrp) {
      if (st > 0 && st % kGcChunk == 0) {
        gc_stage_chunk<TM, kGcBatch>(g, m0, st, gsa, gd);
        lds_barrier();
      }
    }
  };
  // The register-set and buffer rotations repeat every 6 stages.
  int s = 0;
  if constexpr (BD == 2) {
    for (; s + 5 < S; s += 6) {
      gc_next(s);
      stage(C0{}, C0{}, C0{}, s);
      stage(C1{}, C1{}, C1{}, s + 1);
      stage(C2{}, C0{}, C2{}, s + 2);
      stage(C0{}, C1{}, C0{}, s + 3);
      stage(C1{}, C0{}, C1{}, s + 4);
      stage(C2{}, C1{}, C2{}, s + 5);
    }
    const int rem = S - s;  // 0..5 stages left, uniform
    if (rem > 0) gc_next(s);
    if (rem > 0) stage(C0{}, C0{}, C0{}, s);
    if (rem > 1) stage(C1{}, C1{}, C1{}, s + 1);
    if (rem > 2) stage(C2{}, C0{}, C2{}, s + 2);
    if (rem > 3) stage(C0{}, C1{}, C0{}, s + 3);
    if (rem > 4) stage(C1{}, C0{}, C1{}, s + 4);
  } else {
    for (; s + 5 < S; s += 6) {
      gc_next(s);
      stage(C0{}, C0{}, C0{}, s);
      stage(C1{}, C1{}, C1{}, s + 1);
      stage(C0{}, C0{}, C2{}, s + 2);
      stage(C1{}, C1{}, C0{}, s + 3);
      stage(C0{}, C0{}, C1{}, s + 4);
      stage(C1{}, C1{}, C2{}, s + 5);
    }
    const int rem = S - s;
    if (rem > 0) gc_next(s);
    if (rem > 0) stage(C0{}, C0{}, C0{}, s);
    if (rem > 1) stage(C1{}, C1{}, C1{}, s + 1);
    if (rem > 2) stage(C0{}, C0{}, C2{}, s + 2);
    if (rem > 3) stage(C1{}, C1{}, C0{}, s + 3);
    if (rem > 4) stage(C0{}, C0{}, C1{}, s + 4);
  }

  // Epilogue.  The weight fragment is the first matrix-core operand, so each
  // accumulator fragment is the transposed 32 x 32 block: lane l holds token
  // row (l & 31) and, in register v, output column 8*(v>>2) + 4*(l>>5) + (v&3)
  // -- runs of four adjacent columns.  Per 32 rows the wave finishes the
  // integer accumulator, scales by the column step, adds the compensation
  // term, scales by the token step, converts to fp16, stages the 32 x 32 NTW
  // block in its own LDS rows and writes it out as whole row segments (64 NTW
  // bytes), 16 bytes per lane.
  const int r = lane & 31, h = lane >> 5;
  // COMP == 1: the (final, int8-weight) accumulators are reported if asked
  // and then continue in fp32 as acc * sw, onto which the compensation
  // products accumulate, so that one set of accumulation registers is live.
  if constexpr (COMP == 1) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int64_t m = m0 + 32 * tm + r;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4f sw = *reinterpret_cast<const v4f*>(c_sw + 32 * NTW * wave + 32 * nt + 8 * q + 4 * h);
          const v4i iv = v4i{acc[tm][nt][4 * q], acc[tm][nt][4 * q + 1], acc[tm][nt][4 * q + 2], acc[tm][nt][4 * q + 3]};
          if (g.acc != nullptr && live && m < g.M)
            *reinterpret_cast<v4i*>(g.acc + m * g.N + wcol0 + 32 * nt + 8 * q + 4 * h) = iv;
#pragma unroll
          for (int j = 0; j < 4; ++j) cf[tm][nt][4 * q + j] = static_cast<float>(iv[j]) * sw[j];
        }
    }
    comp_accumulate<TM, NTW>(cf, g.xO, g.ldO, g.WOp, g.M, g.N, m0, nt32);
  }
  lds_barrier();  // every wave has finished reading the activation stages
  // Eight waves: the two waves of a pair (2i, 2i + 1) hold the two 64-byte
  // halves of the same 128-byte row pieces.  Written by each wave on its
  // own, every line of y would be written in two halves at different times,
  // which the memory system turns into extra write traffic (23 MB instead
  // of 16.8 at q_proj); so a pair stages its 32 x 64 block in one LDS region
  // (two regions, alternating over tm) and, after a barrier, each wave
  // writes 16 of its rows as whole lines.  Dead waves (whole pairs past N)
  // stay for the barriers.
  if (WV == 4 && !live) return;
  // Bytes per staged row: 128 + 16 spreads the rows over the banks.
  constexpr int kOutPitch = 144;
  constexpr int kPairBytes = 32 * kOutPitch;
  static_assert((WV == 4 ? 4 : 8) * kPairBytes <= kMainBytes, "output staging exceeds the LDS buffers");
  const bool want_acc = g.acc != nullptr;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int64_t m = m0 + 32 * tm + r;
    // This wave's staging rows and the byte offset of its columns in them.
    uint8_t* const out_lds = (WV == 4) ? lds + wave * kPairBytes
                                       : lds + (tm & 1) * 4 * kPairBytes + (wave >> 1) * kPairBytes;
    const int out_col = (WV == 4) ? 0 : 64 * (wave & 1);
    // W4A4 zero points: acc = raw - zw*(rowsum - K*za) - za*colsum, evaluated
    // in wrapping 32-bit arithmetic (exact: the true value fits int32).
    const float sam = kGrp ? 1.0f : c_sa[32 * tm + r];
    [[maybe_unused]] uint32_t za = 0, rkt = 0;
    if constexpr (B == BOp::W4U && !kGrp) {
      za = static_cast<uint32_t>(c_za[32 * tm + r]);
      rkt = static_cast<uint32_t>(c_rs[32 * tm + r]) - static_cast<uint32_t>(g.K) * za;
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = wcol0 + 32 * nt + 8 * q + 4 * h;        // first of this lane's four columns
        const int cb = 32 * NTW * wave + 32 * nt + 8 * q + 4 * h;  // the same column within the tile
        const v4f sw = *reinterpret_cast<const v4f*>(c_sw + cb);
        [[maybe_unused]] v4i zw, cs;
        if constexpr (B == BOp::W4U) {
          zw = *reinterpret_cast<const v4i*>(c_zw + cb);
          cs = *reinterpret_cast<const v4i*>(c_cs + cb);
        }
        if constexpr (kBwd) zw = *reinterpret_cast<const v4i*>(c_zw + cb);
        v4i iv;
        uint16_t hv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int32_t val = acc[tm][nt][4 * q + j];
          if constexpr (B == BOp::W4Shift) {
            val >>= 4;  // every product is 16 * q * q4: the division is exact
          } else if constexpr (B == BOp::W4U && !kGrp) {
            val = static_cast<int32_t>(static_cast<uint32_t>(val) - static_cast<uint32_t>(zw[j]) * rkt -
                                       za * static_cast<uint32_t>(cs[j]));
          }
          iv[j] = val;
          float f;
          if constexpr (kBwd) {
            // r[k] * (gs[m] * acc + (s[k] - 1) * cb[m, o]) for outlier column k = O[o].
            f = static_cast<float>(val) * sam;
            const int o = zw[j];
            if (o >= 0) {
              const int64_t mcl = m < g.M ? m : g.M - 1;
              const float sm1 = __builtin_bit_cast(float, c_cs[cb + j]);
              f = fmaf(sm1, g.cb[mcl * g.ldO + o], f);
            }
            f = f * sw[j];
          } else if constexpr (kGrp)
            f = (cf[tm][nt][4 * q + j] - static_cast<float>(zw[j]) * P[tm]) * sw[j];
          else if constexpr (COMP == 1)
            f = cf[tm][nt][4 * q + j];  // acc * sw + compensation
          else if constexpr (kComp1st)
            f = static_cast<float>(val) * sw[j] + cf[tm][nt][4 * q + j];
          else
            f = static_cast<float>(val) * sw[j];
          hv[j] = f2h(kBwd ? f : f * sam);
        }
        if (WV == 4 || live)
          *reinterpret_cast<uint2*>(out_lds + r * kOutPitch + out_col + (32 * nt + 8 * q + 4 * h) * 2) =
              make_uint2(hv[0] | (static_cast<uint32_t>(hv[1]) << 16), hv[2] | (static_cast<uint32_t>(hv[3]) << 16));
        if (COMP != 1 && !kGrp && want_acc && live && m < g.M) *reinterpret_cast<v4i*>(g.acc + m * g.N + n) = iv;
      }
    // Four waves: each reads back only the rows it wrote; LDS operations of
    // one wave complete in order, so a compiler fence suffices.  Eight: the
    // pair's other half comes from the other wave, after a barrier.
    if constexpr (WV == 4)
      asm volatile("" ::: "memory");
    else
      lds_barrier();
    // 128-byte rows, 8 lanes per row: all 32 rows (four waves), or this
    // wave's 16 of the pair's 32 (eight waves).
    constexpr int kRows = (WV == 4) ? 32 : 16;
    const int row0 = (WV == 4) ? 0 : 16 * (wave & 1);
    const int64_t col0 = (WV == 4) ? wcol0 : n0 + 64 * (wave >> 1);
#pragma unroll
    for (int i = 0; i < kRows / 8; ++i) {
      const int row = row0 + (lane >> 3) + 8 * i, chunk = lane & 7;
      const v4i d = *reinterpret_cast<const v4i*>(out_lds + row * kOutPitch + chunk * 16);
      const int64_t mr = m0 + 32 * tm + row;
      // Streaming store: the output is not read again by this kernel.
      if (live && mr < g.M) __builtin_nontemporal_store(d, reinterpret_cast<v4i*>(g.y + mr * g.N + col0 + 8 * chunk));
    }
    asm volatile("" ::: "memory");
  }
}

// ============================================================ skinny kernel
// M <= 32*MT.  Workgroup: WAVES waves and NT 32-column tiles; wave w takes the
// 64-k units u = w, w + WAVES, ...; U units are loaded before any is used.
template <BOp B, AOp A, int MT, int NT, int WAVES, int U>
__global__ __launch_bounds__(64 * WAVES) void gemm_skinny(GemmArgs g) {
  __shared__ int red[MT * NT * 16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nt0 = static_cast<int64_t>(blockIdx.x) * NT;
  const int64_t tiles_n = g.N / 32;
  const int KU = static_cast<int>(g.K / 64);
  const int arow = lane & 31, ahalf = lane >> 5;

  for (int i = threadIdx.x; i < MT * NT * 16 * 64; i += 64 * WAVES) (&red[0][0])[i] = 0;

  v16i acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = v16i{};

  for (int base = wave; base < KU; base += WAVES * U) {
    constexpr int NBU = (B == BOp::W8) ? 2 : 1;
    uint4 rb[U][NT][NBU];
    v2h rr[U][NT];
    v4i af[U][MT][2];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int u = base + WAVES * uu;
      const bool ok_u = u < KU;
      // Weights and ratios come from clamped, in-bounds indices with no
      // condition: a unit past K meets zero activations below, and a strip
      // past N is never stored.  Under a condition, the compiler sinks the
      // per-group requantization into the branch, where it waits for each
      // load before issuing the next.
      const int uc = ok_u ? u : KU - 1;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int64_t strip = (nt0 + nt) < tiles_n ? nt0 + nt : tiles_n - 1;
#pragma unroll
        for (int h = 0; h < NBU; ++h) {
          const int64_t tile_k = (B == BOp::W8) ? (2 * static_cast<int64_t>(uc) + h) : static_cast<int64_t>(uc);
          const int64_t tix = strip * ((B == BOp::W8) ? g.K / 32 : g.K / 64) + tile_k;
          rb[uu][nt][h] = *reinterpret_cast<const uint4*>(g.b + (tix << 10) + lane * 16);
        }
        rr[uu][nt] = v2h{static_cast<_Float16>(0.0f), static_cast<_Float16>(0.0f)};
        if constexpr (B == BOp::W4Group) {
          const _Float16 r = __builtin_bit_cast(_Float16, g.ratio[static_cast<int64_t>(uc / 2) * g.N + strip * 32 + arow]);
          rr[uu][nt] = v2h{r, r};
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int64_t m = mt * 32 + arow;
        const bool ok = ok_u && m < g.M;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int64_t k = 64 * static_cast<int64_t>(u) + 32 * h + 16 * ahalf;
          if constexpr (A == AOp::I8) {
            const uint4 raw = ok ? *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(g.a) + m * g.K + k)
                                 : make_uint4(0, 0, 0, 0);
            af[uu][mt][h] = v4i{(int)raw.x, (int)raw.y, (int)raw.z, (int)raw.w};
          } else {
            const uint2 raw = ok ? *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(g.a) + m * (g.K / 2) + k / 2)
                                 : make_uint2(0, 0);
            af[uu][mt][h] = unpack_a4(raw.x, raw.y);
          }
        }
      }
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        v4i bf[2];
        if constexpr (B == BOp::W8) {
          bf[0] = v4i{(int)rb[uu][nt][0].x, (int)rb[uu][nt][0].y, (int)rb[uu][nt][0].z, (int)rb[uu][nt][0].w};
          bf[1] = v4i{(int)rb[uu][nt][NBU - 1].x, (int)rb[uu][nt][NBU - 1].y, (int)rb[uu][nt][NBU - 1].z,
                      (int)rb[uu][nt][NBU - 1].w};
        } else {
          unpack_w4<B>(rb[uu][nt][0], rr[uu][nt], bf[0], bf[1]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma_i8(af[uu][mt][h], bf[h], acc[mt][nt]);
      }
    }
  }

  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) atomicAdd(&red[(mt * NT + nt) * 16 + v][lane], acc[mt][nt][v]);
  __syncthreads();

  for (int fi = wave; fi < MT * NT; fi += WAVES) {
    const int mt = fi / NT, nt = fi % NT;
    if (nt0 + nt >= tiles_n) continue;
    const int64_t n = (nt0 + nt) * 32 + arow;
    // All constants first, in one batch (a load after a store waits for its
    // own round trip, since the store may alias it).
    const float sw = col_scale<B>(g, n);
    float sam[16];
    [[maybe_unused]] int32_t zam[16], rsm[16];
    [[maybe_unused]] int32_t zwn = 0, csn = 0;
    if constexpr (B == BOp::W4U) {
      zwn = g.zw[n];
      csn = g.colsum[n];
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int64_t m = mt * 32 + frag_row(v, lane);
      m = m < g.M ? m : g.M - 1;
      sam[v] = g.sa[m];
      if constexpr (B == BOp::W4U) {
        zam[v] = g.za[m];
        rsm[v] = g.rowsum[m];
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = mt * 32 + frag_row(v, lane);
      if (m >= g.M) continue;
      int32_t val = red[fi * 16 + v][lane];
      if constexpr (B == BOp::W4Shift) {
        val >>= 4;  // every product is 16 * q * q4: the division is exact
      } else if constexpr (B == BOp::W4U) {
        // Zero-point correction in wrapping 32-bit arithmetic (exact: the
        // true value fits int32).
        const uint32_t za = static_cast<uint32_t>(zam[v]), zw = static_cast<uint32_t>(zwn);
        val = static_cast<int32_t>(static_cast<uint32_t>(val) - zw * static_cast<uint32_t>(rsm[v]) -
                                   za * static_cast<uint32_t>(csn) + static_cast<uint32_t>(g.K) * za * zw);
      }
      if (g.acc != nullptr) g.acc[m * g.N + n] = val;
      g.y[m * g.N + n] = f2h(static_cast<float>(val) * sw * sam[v]);
    }
  }
}

// ------------------------------------------------------ skinny, LDS-staged
// gemm_skinny_lds (32 < M <= 128, int8 activations): the skinny kernel with
// its activations staged through LDS.  Loaded straight into fragments, a
// 16-byte-per-lane activation load touches 32 token rows in 32-byte pieces;
// here the workgroup loads each round's activation block (all 32 * MT rows,
// 512 * U bytes of each) as whole row segments, 16 bytes per thread and a
// row segment per 32 * U threads, stores it to LDS with the 16-byte chunks of
// row m XOR-permuted by (m & 15) (16 rows reading one logical chunk hit 16
// different bank groups), and every wave reads its fragments from there.
// Round r covers units [8U r, 8U (r + 1)) of 64 k; wave w takes units
// 8U r + w + 8j, j < U.  Activations are loaded two rounds ahead and stored
// to the other of two LDS buffers one round ahead; weights are loaded two
// rounds ahead into two register sets.  Units past K (a partial last round)
// read their weights from the last unit and their activation chunks from a
// clamped, in-bounds address; their activation fragments are zeroed, so they
// add exactly zero.  Rows past M are read from row M - 1 and their outputs
// are not stored.
template <BOp B, int MT, int U>
__global__ __launch_bounds__(512) void gemm_skinny_lds(GemmArgs g) {
  constexpr int NT = 2, WAVES = 8;
  constexpr int kRows = 32 * MT;
  constexpr int kRowB = 512 * U;         // bytes of a row per round
  constexpr int kBuf = kRows * kRowB;    // bytes of a round's block
  constexpr int kCh = kBuf / 16 / 512;   // 16-byte chunks per thread per round
  constexpr int kCpr = kRowB / 16;       // chunks per row segment
  constexpr int kRpi = 512 / kCpr;       // rows between a thread's chunks
  constexpr int NBU = (B == BOp::W8) ? 2 : 1;
  static_assert(MT * NT * 16 * 64 * 4 <= 2 * kBuf, "the reduction reuses the activation buffers");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBuf];
  int* const red = reinterpret_cast<int*>(lds);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int arow = lane & 31, ahalf = lane >> 5;
  const int64_t nt0 = static_cast<int64_t>(blockIdx.x) * NT;  // N % 64 == 0: both strips exist
  const int KU = static_cast<int>(g.K / 64);
  const int R = (KU + 8 * U - 1) / (8 * U);
  const int64_t KT = (B == BOp::W8) ? g.K / 32 : g.K / 64;

  // Chunk i of this thread in a round: row i * kRpi + tid / kCpr, chunk cc.
  const int cc = tid % kCpr, r0 = tid / kCpr;
  const int8_t* const a0 = static_cast<const int8_t*>(g.a);
  auto load_act = [&](int r, v4i (&ra)[kCh]) __attribute__((always_inline)) {
    int64_t k = static_cast<int64_t>(r) * kRowB + cc * 16;
    k = k < g.K ? k : g.K - 16;
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      int64_t m = i * kRpi + r0;
      m = m < g.M ? m : g.M - 1;
      ra[i] = *reinterpret_cast<const v4i*>(a0 + m * g.K + k);
    }
  };
  auto store_act = [&](uint8_t* buf, const v4i (&ra)[kCh]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int row = i * kRpi + r0;
      *reinterpret_cast<v4i*>(buf + row * kRowB + ((cc ^ (row & 15)) << 4)) = ra[i];
    }
  };
  auto load_w = [&](int r, uint4 (&rb)[U][NT][NBU], v2h (&rr)[U][NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      // Unconditional loads from a clamped unit: the fragments of a unit
      // past K are zeroed on the activation side instead (a select on the
      // weights becomes a branch around the load and, per group, around the
      // requantization, which then waits for each load in turn).
      const int u = 8 * U * r + wave + 8 * j;
      const int uc = u < KU ? u : KU - 1;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int h = 0; h < NBU; ++h) {
          const int64_t tix = (nt0 + nt) * KT + ((B == BOp::W8) ? 2 * static_cast<int64_t>(uc) + h : uc);
          rb[j][nt][h] = *reinterpret_cast<const uint4*>(g.b + (tix << 10) + lane * 16);
        }
        if constexpr (B == BOp::W4Group) {
          const _Float16 q = __builtin_bit_cast(
              _Float16, g.ratio[static_cast<int64_t>(uc / 2) * g.N + (nt0 + nt) * 32 + arow]);
          rr[j][nt] = v2h{q, q};
        } else {
          rr[j][nt] = v2h{};
        }
      }
    }
  };

  v16i acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = v16i{};

  v4i ra[kCh];
  uint4 rb[2][U][NT][NBU];
  v2h rr[2][U][NT];
  load_act(0, ra);
  load_w(0, rb[0], rr[0]);
  store_act(lds, ra);
  if (R > 1) {
    load_act(1, ra);
    load_w(1, rb[1], rr[1]);
  }
  __syncthreads();

  auto round = [&](auto par, int r) __attribute__((always_inline)) {
    constexpr int P = decltype(par)::value;
    const uint8_t* const cur = lds + P * kBuf;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      v4i af[MT][2];
      const bool uok = 8 * U * r + wave + 8 * j < KU;  // a unit past K adds zero
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int row = 32 * mt + arow, c = 4 * (wave + 8 * j) + 2 * h + ahalf;
          const v4i f = *reinterpret_cast<const v4i*>(cur + row * kRowB + ((c ^ (row & 15)) << 4));
          af[mt][h] = uok ? f : v4i{};
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        v4i bf[2];
        if constexpr (B == BOp::W8) {
          const uint4 w0 = rb[P][j][nt][0], w1 = rb[P][j][nt][NBU - 1];
          bf[0] = v4i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w};
          bf[1] = v4i{(int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
        } else {
          unpack_w4<B>(rb[P][j][nt][0], rr[P][j][nt], bf[0], bf[1]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma_i8(af[mt][h], bf[h], acc[mt][nt]);
      }
    }
    // The other buffer was last read in round r - 1, before its closing barrier.
    if (r + 1 < R) store_act(lds + (1 - P) * kBuf, ra);
    if (r + 2 < R) {
      load_act(r + 2, ra);
      load_w(r + 2, rb[P], rr[P]);
    }
    __syncthreads();
  };
  for (int r = 0; r < R; r += 2) {
    round(std::integral_constant<int, 0>{}, r);
    if (r + 1 < R) round(std::integral_constant<int, 1>{}, r + 1);
  }

  // The waves' int32 partial sums meet in the (now free) activation buffers.
  for (int i = tid; i < MT * NT * 16 * 64; i += 512) red[i] = 0;
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) atomicAdd(&red[((mt * NT + nt) * 16 + v) * 64 + lane], acc[mt][nt][v]);
  __syncthreads();
  for (int fi = wave; fi < MT * NT; fi += WAVES) {
    const int mt = fi / NT, nt = fi % NT;
    const int64_t n = (nt0 + nt) * 32 + arow;
    const float sw = h2f(g.sw_h[n]);
    float sam[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int64_t m = mt * 32 + frag_row(v, lane);
      m = m < g.M ? m : g.M - 1;
      sam[v] = g.sa[m];
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t m = mt * 32 + frag_row(v, lane);
      if (m >= g.M) continue;
      int32_t val = red[(fi * 16 + v) * 64 + lane];
      if constexpr (B == BOp::W4Shift) val >>= 4;  // every product is 16 * q * q4: the division is exact
      if (g.acc != nullptr) g.acc[m * g.N + n] = val;
      g.y[m * g.N + n] = f2h(static_cast<float>(val) * sw * sam[v]);
    }
  }
}

// ------------------------------------------------------ per-group requant
// The per-group requantization of a whole W4S-packed weight matrix into the
// W8 layout, once per call (QQQ review, "technical architecture": the fused
// dequant-quant of the per-group W4A8 kernel).  One thread per 16-byte lane
// chunk of a 64-k tile t of strip nt; the chunk's two int8 fragments are W8
// tiles 2t and 2t + 1 of the same strip, each value the same
// requant_word result the tiled kernel computes in its K loop.
__global__ __launch_bounds__(256) void requant_w4_group_kernel(const uint8_t* w4, const uint16_t* ratio, int64_t K,
                                                               int64_t N, uint8_t* w8) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t kt4 = K / 64;
  if (i >= kt4 * (N / 32) * 64) return;
  const int lane = static_cast<int>(i & 63);
  const int64_t nt = (i >> 6) / kt4, t = (i >> 6) % kt4;
  const uint4 raw = *reinterpret_cast<const uint4*>(w4 + i * 16);
  const _Float16 r = __builtin_bit_cast(_Float16, ratio[(t / 2) * N + nt * 32 + (lane & 31)]);
  v4i c0, c1;
  unpack_w4<BOp::W4Group>(raw, v2h{r, r}, c0, c1);
  uint8_t* const out = w8 + ((nt * (K / 32) + 2 * t) << 10) + lane * 16;
  *reinterpret_cast<v4i*>(out) = c0;
  *reinterpret_cast<v4i*>(out + 1024) = c1;
}

// Tokens above which the per-group W4A8 product, given a workspace,
// requantizes the weights once per call and runs the int8 tile on them.  At
// and below it the skinny kernels stream the int4 weights once, which beats
// reading them, writing twice the bytes and reading those again.
constexpr int64_t kRequantMinRows = 128;

// ------------------------------------------------------------ dispatch
template <BOp B, AOp A, int MT, int NT, int WAVES, int U>
void launch_skinny(const GemmArgs& g, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((g.N / 32 + NT - 1) / NT));
  gemm_skinny<B, A, MT, NT, WAVES, U><<<grid, 64 * WAVES, 0, st>>>(g);
}

template <BOp B, AOp A, int TM, int COMP, int WV = 4>
qlin_status launch_tile(const GemmArgs& g, hipStream_t st) {
  // Weight prefetch depth: two stages, except at 256-row tiles with int8 or
  // per-group requantized weights, where register room leaves one.
  // Group-wise W4A4 keeps one (its group constants and fp32 sums take the
  // room), and so do eight-wave tiles, where it measured faster (two waves
  // per SIMD cover the weights' latency), and the W4A4 tiles that run two
  // workgroups per CU (101 against 101-107 us with two stages).
  constexpr int BD = (((B == BOp::W8 || B == BOp::W4Group) && TM == 8) || A == AOp::U4G || WV == 8 ||
                      (A == AOp::U4 && TM == 4)) ? 1 : 2;
  const int64_t tiles = ((g.M + 32 * TM - 1) / (32 * TM)) * ((g.N + kBN - 1) / kBN);
  QLIN_REQUIRE(tiles <= 0x7fffffffLL, QLIN_ERR_SHAPE, "M=%lld too large", (long long)g.M);
  gemm_tile<B, A, TM, BD, COMP, WV><<<dim3(static_cast<unsigned>(tiles)), 64 * WV, 0, st>>>(g);
  QLIN_LAUNCH_CHECK("gemm_tile");
  return QLIN_OK;
}

template <BOp B, AOp A>
qlin_status launch(const GemmArgs& g, bool comp, hipStream_t st) {
  if constexpr (A == AOp::U4G) {
    // Group-wise W4A4: 64-row tiles at every M, two workgroups per CU (the
    // int32 and fp32 accumulators both live in registers).  With an acc
    // buffer, the variant that also writes every group's int32 sums.
    if (g.acc != nullptr) return launch_tile<B, A, 2, 4>(g, st);
    return launch_tile<B, A, 2, 0>(g, st);
  } else {
    // Up to 128 tokens the K-split skinny kernels (one 64-k unit per wave in
    // flight at 128 rows) beat 128-row tiles, of which there would be fewer
    // than one per CU.
    if (!comp && g.M <= 128) {
      // int8 activations from 33 tokens: staged through LDS (measured at
      // 4096 x 11008: M = 64 per channel 16.8 -> 13.3 us, M = 128 26.4 ->
      // 18.7 us), except where the direct form measured faster: the
      // requantizing per-group weights at every such M, and int8 weights at
      // 128 rows up to 96 tokens.
      const int64_t dgrid = g.N / 64;
      if constexpr (A == AOp::I8 && B == BOp::W4Group) {
        // 33-64 tokens: two 64-k units in flight per wave (at 4096 x 11008,
        // M = 48 / 64: 18.2 / 18.7 us against 20.4 / 20.8 through LDS; the
        // vector requantization, not the activation loads, sets the pace).
        if (g.M > 32 && g.M <= 64) {
          launch_skinny<B, A, 2, 2, 8, 2>(g, st);
          QLIN_LAUNCH_CHECK("gemm_skinny");
          return QLIN_OK;
        }
      }
      if constexpr (A == AOp::I8) {
        if (g.M > 32 && g.M <= 64) {
          gemm_skinny_lds<B, 2, 2><<<dim3(static_cast<unsigned>(dgrid)), 512, 0, st>>>(g);
          QLIN_LAUNCH_CHECK("gemm_skinny_lds");
          return QLIN_OK;
        }
        if (g.M > 64 && (B == BOp::W4Shift || (B == BOp::W8 && g.M > 96))) {
          gemm_skinny_lds<B, 4, 1><<<dim3(static_cast<unsigned>(dgrid)), 512, 0, st>>>(g);
          QLIN_LAUNCH_CHECK("gemm_skinny_lds");
          return QLIN_OK;
        }
      }
      if (g.M <= 32)
        launch_skinny<B, A, 1, 2, 8, 4>(g, st);
      else if (g.M <= 64)
        launch_skinny<B, A, 2, 2, 8, 4>(g, st);
      else
        launch_skinny<B, A, 4, 2, 8, 1>(g, st);
      QLIN_LAUNCH_CHECK("gemm_skinny");
      return QLIN_OK;
    }
    if (comp) {
      if constexpr (B == BOp::W8 && A == AOp::I8) {
        if (g.ldO <= kXOLdsLd) return launch_tile<B, A, 4, 5, 8>(g, st);
        if (g.ldO <= kXOMaxLd) return launch_tile<B, A, 4, 2>(g, st);
        return launch_tile<B, A, 4, 1>(g, st);
      }
    }
    // 256-row tiles when they still give every CU a tile: per weight byte
    // streamed (and unpacked) they do twice the matrix-core work.  W4A4
    // instead runs 128-row tiles two workgroups per CU at every M, so that
    // each SIMD holds two waves whose unpacking and waits overlap the other's
    // matrix-core work (2048 x 4096 x 14336: 112 -> 101 us).
    const int64_t tiles_n = (g.N + kBN - 1) / kBN;
    if constexpr (B != BOp::W4U)
      if (((g.M + 255) / 256) * tiles_n >= 256) return launch_tile<B, A, 8, 0>(g, st);
    // 128-row int8 tiles: eight waves (2048 x 4096 x 4096: 41.8 -> 37.2 us
    // in one comparison).
    if constexpr (B == BOp::W8 && A == AOp::I8)
      return launch_tile<B, A, 4, 0, 8>(g, st);
    else
      return launch_tile<B, A, 4, 0>(g, st);
  }
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

qlin_status launch_gemm_bwd(const int8_t* gq, const float* gs, const void* w8t, const float* r, const float* s,
                            const int32_t* O, int32_t nO, const float* cb, int64_t M, int64_t N, int64_t K,
                            uint16_t* dx, int32_t* acc, hipStream_t st) {
  // The product's reduction runs over N (the forward's output channels) and
  // its columns are the forward's K input channels.
  GemmArgs g = base_args(M, K, N, dx, acc);
  g.a = gq;
  g.sa = gs;
  g.b = static_cast<const uint8_t*>(w8t);
  g.sw_f = r;
  g.s = s;
  g.O = O;
  g.nO = nO;
  g.cb = cb;
  g.ldO = static_cast<int>(outlier_ld(nO));
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  if (((g.M + 255) / 256) * tiles_n >= 256) return launch_tile<BOp::W8, AOp::I8, 8, 3>(g, st);
  return launch_tile<BOp::W8, AOp::I8, 4, 3>(g, st);
}

}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_gemm_w8a8(const int8_t* qa, const float* sa, const void* w8,
                                      const uint16_t* sw, int64_t M, int64_t N, int64_t K,
                                      const uint16_t* xO, int32_t nO, const void* WO, uint16_t* y,
                                      int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  QLIN_DIMS(M, K);
  QLIN_DIMS(K, N);
  QLIN_DIMS(M, N);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(qa);
  QLIN_PTR(sa);
  QLIN_PTR(w8);
  QLIN_PTR(sw);
  QLIN_PTR(y);
  QLIN_OPT_PTR(acc);
  if (nO > 0) {
    QLIN_PTR(xO);
    QLIN_PTR(WO);
  } else {
    QLIN_REQUIRE(xO == nullptr && WO == nullptr, QLIN_ERR_INVALID_ARG, "xO and WO must be NULL when nO == 0");
  }
  GemmArgs g = base_args(M, N, K, y, acc);
  g.a = qa;
  g.sa = sa;
  g.b = static_cast<const uint8_t*>(w8);
  g.sw_h = sw;
  g.xO = xO;
  g.WOp = static_cast<const uint8_t*>(WO);
  g.ldO = static_cast<int>(outlier_ld(nO));
  return launch<BOp::W8, AOp::I8>(g, nO > 0, as_stream(stream));
}

extern "C" qlin_status qlin_gemm_w4a8(const int8_t* qa, const float* sa, const void* w4,
                                      const uint16_t* sw, const uint16_t* ratio, int32_t group,
                                      int64_t M, int64_t N, int64_t K, uint16_t* y, int32_t* acc,
                                      void* work, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  QLIN_DIMS(M, K);
  QLIN_DIMS(K, N);
  QLIN_DIMS(M, N);
  QLIN_REQUIRE(group == 0 || group == 128, QLIN_ERR_UNSUPPORTED, "group=%d: only 0 and 128 are provided", group);
  QLIN_OPT_PTR(work);
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
  hipStream_t st = as_stream(stream);
  if (group == 128 && work != nullptr && M > kRequantMinRows) {
    const int64_t chunks = K * N / 32;
    requant_w4_group_kernel<<<dim3(static_cast<unsigned>((chunks + 255) / 256)), 256, 0, st>>>(
        static_cast<const uint8_t*>(w4), ratio, K, N, static_cast<uint8_t*>(work));
    QLIN_LAUNCH_CHECK("requant_w4_group_kernel");
    g.b = static_cast<const uint8_t*>(work);
    g.ratio = nullptr;
    return launch<BOp::W8, AOp::I8>(g, false, st);
  }
  if (group == 128) return launch<BOp::W4Group, AOp::I8>(g, false, st);
  return launch<BOp::W4Shift, AOp::I8>(g, false, st);
}

extern "C" size_t qlin_gemm_w4a8_work_bytes(int64_t M, int64_t N, int64_t K, int32_t group) {
  if (group != 128 || M <= qlin::kRequantMinRows || K <= 0 || K % 128 || N <= 0 || N % 64 ||
      !qlin::dims_ok(M, K) || !qlin::dims_ok(K, N) || !qlin::dims_ok(M, N))
    return 0;
  return static_cast<size_t>(K * N);
}

extern "C" qlin_status qlin_gemm_w4a4(const uint8_t* qa4, const float* sa, const int32_t* za,
                                      const int32_t* rowsum, const void* w4, const float* sw,
                                      const int32_t* zw, const int32_t* colsum, int64_t M, int64_t N,
                                      int64_t K, uint16_t* y, int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  QLIN_DIMS(M, K);
  QLIN_DIMS(K, N);
  QLIN_DIMS(M, N);
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

extern "C" qlin_status qlin_gemm_w4a4_group(const uint8_t* qa4, const float* sa, const int32_t* za,
                                            const int32_t* rowsum, const void* w4, const float* sw,
                                            const int32_t* zw, const int32_t* colsum_g, int64_t M, int64_t N,
                                            int64_t K, uint16_t* y, int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_K_N(K, N);
  QLIN_DIMS(M, K);
  QLIN_DIMS(K, N);
  QLIN_DIMS(M, N);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(qa4);
  QLIN_PTR(sa);
  QLIN_PTR(za);
  QLIN_PTR(rowsum);
  QLIN_PTR(w4);
  QLIN_PTR(sw);
  QLIN_PTR(zw);
  QLIN_PTR(colsum_g);
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
  g.colsum = colsum_g;
  return launch<BOp::W4U, AOp::U4G>(g, false, as_stream(stream));
}
