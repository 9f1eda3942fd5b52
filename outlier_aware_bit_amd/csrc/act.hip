// Activation-side kernels of libqlin (gfx950):
//   qlin_quant_act              per-token symmetric int8 (optionally of X * r)
//   qlin_hadamard_offset        OffQ block Hadamard (all-ones first row) + per-token
//                               asymmetric int4 with the offset in the zero point
//   qlin_hadamard_offset_group  the same transform with a step and zero point per
//                               128-channel group
//
// All are HBM-bound streaming kernels: one wavefront per token, 16-byte
// loads, reductions as wavefront or quad exchanges (no LDS barrier), and
// packed stores.
#include <type_traits>

#include "common.hpp"
#include "internal.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

constexpr int kQuantThreads = 256;  // four wavefronts, two per token

__device__ __forceinline__ void unpack8_f16(v4i raw, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = static_cast<uint32_t>(raw[i]);
    v[2 * i] = h2f(static_cast<uint16_t>(w & 0xffffu));
    v[2 * i + 1] = h2f(static_cast<uint16_t>(w >> 16));
  }
}

__device__ __forceinline__ void load8_f16(const uint16_t* p, float (&v)[8]) {
  unpack8_f16(*reinterpret_cast<const v4i*>(p), v);
}

// r for the 8 channels of chunk c; r is fp32, or fp16 (RT = uint16_t,
// widened exactly to fp32).
template <bool HAS_R, typename RT>
__device__ __forceinline__ void load_r8(const RT* r, int c, float (&rr)[8]) {
  if constexpr (HAS_R) {
    if constexpr (std::is_same_v<RT, float>) {
      const float4 r0 = *reinterpret_cast<const float4*>(r + c * 8);
      const float4 r1 = *reinterpret_cast<const float4*>(r + c * 8 + 4);
      rr[0] = r0.x; rr[1] = r0.y; rr[2] = r0.z; rr[3] = r0.w;
      rr[4] = r1.x; rr[5] = r1.y; rr[6] = r1.z; rr[7] = r1.w;
    } else {
      load8_f16(r + c * 8, rr);
    }
  }
}

// v *= r for the 8 channels of chunk c.
template <bool HAS_R, typename RT>
__device__ __forceinline__ void scale_chunk(const RT* r, int c, float (&v)[8]) {
  if constexpr (HAS_R) {
    float rr[8];
    load_r8<HAS_R>(r, c, rr);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = mul_rn(v[i], rr[i]);
  }
}

template <typename RT>
__device__ __forceinline__ float load_r(const RT* r, int i) {
  if constexpr (std::is_same_v<RT, float>)
    return r[i];
  else
    return h2f(r[i]);
}

__device__ __forceinline__ int sym_code(float v, float inv) {
  float t = rint_f(mul_rn(v, inv));
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return static_cast<int>(t);
}

template <bool HAS_R>
__device__ __forceinline__ uint2 sym_codes8(const float (&v)[8], float inv) {
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    lo |= (static_cast<uint32_t>(sym_code(v[j], inv)) & 0xffu) << (8 * j);
    hi |= (static_cast<uint32_t>(sym_code(v[j + 4], inv)) & 0xffu) << (8 * j);
  }
  return make_uint2(lo, hi);
}

// Per-token symmetric int8: a = max|v|, inv = 127/a, q = clamp(rint(v*inv)).
// WPT wavefronts per token: wave h of a token takes the 64-chunk blocks h,
// h + WPT, ... of the row (chunks of 8 values), the first CH of them held in
// registers as raw fp16 between the absmax and the coding pass (with four
// waves per token, CH = 2 up to K = 4096, 4 up to 8192, 6 up to 12288;
// longer rows re-read the tail from cache: at 4096 x 11008 that re-read
// took 25.1 against 22.9 us with CH = 6).  The waves' maxima meet in LDS across one workgroup
// barrier.  (Four waves per token, one token per workgroup, against two:
// 8.1 -> 7.8 us at 2048 x 4096 with r and xO, 26.3 -> 25.2 at 4096 x 11008.)
//
// Outlier columns (row stride ldO, zero padded): the code of x[m, O[j]], and
// the compensation operand fp16(code * (s[O[j]] - 1)).  With OL (ldO <= 256
// and 2K bytes of LDS per token), O, r[O] and s[O] are fetched before the
// row is needed, and the row is staged in LDS (each wave its own blocks; the
// barrier makes the whole row visible), so that the outlier values are read
// from there; otherwise they are re-read from memory.  Each wave takes every
// WPT-th block of 64 outlier slots.
//
// MF (the momentum step folded in; HAS_R, OL, K <= 512 * WPT * CH): r[O[j]] and
// s[O[j]] are not read but formed from the momentum step's row-block maxima
// (mf.part), which each lane folds for its own slots; the first workgroup
// writes them to mf.s and mf.r.  The maxima kernel leaves a NaN in r at
// each outlier channel (mom_slot_marker), so x * r there is NaN, which the
// maximum (fmaxf) passes over; each lane adds |x[O[j]] * r'| of its own
// slots, gathering x[O[j]] from the row.  The codes of a token go to an LDS
// row first; after a barrier the slots' codes overwrite the outlier
// channels' there, and after another the row is written out.  (A lane that
// reads r[O[j]] after the first workgroup has written the new r gets a
// number instead of the NaN: the maximum is then the same, and the code is
// overwritten all the same.)
constexpr int kOutlierLdMax = 256;
// Tokens per workgroup with WPT wavefronts per token.
constexpr int quant_tokens(int wpt) { return kQuantThreads / 64 / wpt; }
constexpr int kQuantWpt = 4;  // wavefronts per token in the launches below
constexpr int kQuantTokens = quant_tokens(kQuantWpt);
// Register chunks per lane that hold rows of up to 4096 / 8192 channels.
constexpr int kQuantCh4k = 4096 / (512 * kQuantWpt), kQuantCh8k = 8192 / (512 * kQuantWpt);
constexpr int kQuantCh12k = 12288 / (512 * kQuantWpt);

template <bool HAS_R, bool OL, int CH, typename RT = float, bool MF = false, int WPT = 2>
__global__ __launch_bounds__(kQuantThreads) void quant_act_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const RT* __restrict__ r, int8_t* __restrict__ q,
    float* __restrict__ scale, const int32_t* __restrict__ O, int nO, int ldO,
    const float* __restrict__ s, int8_t* __restrict__ qO, uint16_t* __restrict__ xO, MomFold mf) {
  static_assert(!MF || (HAS_R && OL && std::is_same_v<RT, float>), "the momentum fold needs r and the LDS row");
  extern __shared__ __attribute__((aligned(16))) uint8_t qlds[];
  __shared__ float red[kQuantThreads / 64];
  constexpr int kTok = quant_tokens(WPT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = wave % WPT, tok = wave / WPT;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kTok + tok;
  // A token past M still takes part in the workgroup barrier (on row M - 1's
  // data) and stores nothing.
  const bool valid = m < M;
  const uint16_t* xr = x + (valid ? m : M - 1) * K;
  const int nchunks = static_cast<int>(K / 8);
  auto chunk = [&](int i) { return 64 * (WPT * i + half) + lane; };  // this lane's i-th chunk

  // Outlier slots of this lane (j = lane + 64 (WPT i + half)): their channel
  // indices are loaded first, so that the loads of r[O[j]] and s[O[j]] below
  // wait only for them and not for the row issued after them (a wait for a
  // load also waits for every load issued before it).  Unconditional, from
  // a clamped index (a guarded load is a branch that waits for it).
  constexpr int kSl = kOutlierLdMax / (64 * WPT);
  [[maybe_unused]] int oj[kSl];
  if constexpr (OL) {
#pragma unroll
    for (int i = 0; i < kSl; ++i) {
      const int j = lane + 64 * (WPT * i + half);
      const int o = O[j < nO ? j : nO - 1];
      oj[i] = (j < nO && o >= 0 && o < K) ? o : -1;
    }
  }
  // MF: the slots' row-block maxima, w_max and old s, indexed by slot alone
  // and issued ahead of the row.
  [[maybe_unused]] float fpart[MF ? kSl : 1][kMomFoldBlocks], fw[MF ? kSl : 1], fs[MF ? kSl : 1];
  if constexpr (MF) {
#pragma unroll
    for (int i = 0; i < kSl; ++i) {
      const int j = lane + 64 * (WPT * i + half), jc = j < nO ? j : nO - 1;
#pragma unroll
      for (int b = 0; b < kMomFoldBlocks; ++b) fpart[i][b] = mf.part[b * nO + jc];
      fw[i] = mf.wmax[jc];
      fs[i] = mf.part[kMomFoldBlocks * nO + jc];
    }
  }
  // The row: chunks clamped to the row, so that every load is in range and
  // unconditional.
  v4i raw[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = chunk(i);
    raw[i] = *reinterpret_cast<const v4i*>(xr + (c < nchunks ? c : nchunks - 1) * 8);
  }
  // The factors r of the same chunks, also clamped and unconditional (a load
  // under "c < nchunks" is a branch that waits for it).
  [[maybe_unused]] float rch[HAS_R ? CH : 1][8];
  if constexpr (HAS_R) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      load_r8<HAS_R>(r, c < nchunks ? c : nchunks - 1, rch[i]);
    }
  }
  // (Every row and factor load is issued before the wait for the indices.)
  __builtin_amdgcn_sched_barrier(0);
  // r and s of the lane's outlier slots, in flight with the row.  s may be
  // NULL without xO: the load then reads O[0] instead and is not used.
  [[maybe_unused]] float rj[kSl], sm1j[kSl];
  [[maybe_unused]] uint16_t* const rowl = reinterpret_cast<uint16_t*>(qlds + tok * 2 * K);
  [[maybe_unused]] uint16_t xg[MF ? kSl : 1];
  if constexpr (MF) {
    // The slots' values x[O[j]] (their lines are on the way with the row),
    // then the momentum step of the lane's slots.
#pragma unroll
    for (int i = 0; i < kSl; ++i) xg[i] = xr[oj[i] >= 0 ? oj[i] : 0];
#pragma unroll
    for (int i = 0; i < kSl; ++i) {
      float c = fpart[i][0];
#pragma unroll
      for (int b = 1; b < kMomFoldBlocks; ++b) c = fmaxf(c, fpart[i][b]);
      float sn, rn;
      momentum_step(c, fw[i], mf.gamma, fs[i], sn, rn);
      rj[i] = rn;
      sm1j[i] = (oj[i] >= 0) ? sub_rn(sn, 1.0f) : 0.0f;
      if (blockIdx.x == 0 && tok == 0 && oj[i] >= 0) {
        mf.s[oj[i]] = sn;
        mf.r[oj[i]] = rn;
      }
    }
  }
  if constexpr (OL && !MF) {
    const bool wx = xO != nullptr;
    [[maybe_unused]] const float* const sp = wx ? s : reinterpret_cast<const float*>(O);
    if constexpr (!MF) {
#pragma unroll
      for (int i = 0; i < kSl; ++i) {
        const int o = oj[i] >= 0 ? oj[i] : 0;
        rj[i] = HAS_R ? load_r(r, o) : 1.0f;
        const float sv = sp[wx ? o : 0];
        sm1j[i] = (wx && oj[i] >= 0) ? sub_rn(sv, 1.0f) : 0.0f;
      }
    }
    // This wave's blocks of the raw row go to the token's LDS row.
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      if (c < nchunks) *reinterpret_cast<v4i*>(rowl + c * 8) = raw[i];
    }
    for (int i = CH; chunk(i) - lane < nchunks; ++i) {
      const int c = chunk(i);
      if (c < nchunks) *reinterpret_cast<v4i*>(rowl + c * 8) = *reinterpret_cast<const v4i*>(xr + c * 8);
    }
  }

  // v = x * r (HAS_R: held in registers between the two passes), absmax.
  [[maybe_unused]] float vr[HAS_R ? CH : 1][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    // Branch-free: a chunk past the row (a clamped repeat) is scaled too and
    // left out of the maximum by the select.
    const bool in = chunk(i) < nchunks;
    float v[8];
    unpack8_f16(raw[i], v);
    if constexpr (HAS_R) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = mul_rn(v[j], rch[i][j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, in ? fabsf(v[j]) : 0.0f);
    if constexpr (HAS_R) {
#pragma unroll
      for (int j = 0; j < 8; ++j) vr[i][j] = v[j];
    }
  }
  for (int i = CH; chunk(i) - lane < nchunks; ++i) {
    const int c = chunk(i);
    if (c < nchunks) {
      float v[8];
      load8_f16(xr + c * 8, v);
      scale_chunk<HAS_R>(r, c, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
  }
  if constexpr (MF) {
    // The outlier channels, left out above (NaN), with the new r.
#pragma unroll
    for (int i = 0; i < kSl; ++i) amax = fmaxf(amax, oj[i] >= 0 ? fabsf(mul_rn(h2f(xg[i]), rj[i])) : 0.0f);
  }
  amax = wave_max(amax);
  if (lane == 0) red[wave] = amax;
  __syncthreads();  // both halves' maxima, and (OL) the whole staged row
  float a = red[WPT * tok];
#pragma unroll
  for (int w = 1; w < WPT; ++w) a = fmaxf(a, red[WPT * tok + w]);
  if constexpr (MF) {
    // Every wave stays for the barriers below; a token past M stores nothing.
    const float inv = (a == 0.0f) ? 0.0f : div_rn(127.0f, a);
    if (valid && lane == 0 && half == 0) scale[m] = (a == 0.0f) ? 0.0f : div_rn(a, 127.0f);
    int8_t* const qrow = reinterpret_cast<int8_t*>(qlds) + tok * K;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = chunk(i);
      if (c < nchunks) *reinterpret_cast<uint2*>(qrow + c * 8) = sym_codes8<true>(vr[i], inv);
    }
    lds_barrier();
    int code[kSl];
#pragma unroll
    for (int i = 0; i < kSl; ++i) {
      code[i] = (oj[i] >= 0) ? sym_code(mul_rn(h2f(xg[i]), rj[i]), inv) : 0;
      if (oj[i] >= 0) qrow[oj[i]] = static_cast<int8_t>(code[i]);
    }
    lds_barrier();
    if (!valid) return;
    for (int c = lane + 64 * half; c < static_cast<int>(K / 16); c += 64 * WPT)
      *reinterpret_cast<v4i*>(q + m * K + 16 * c) = *reinterpret_cast<const v4i*>(qrow + 16 * c);
#pragma unroll
    for (int i = 0; i < kSl; ++i) {
      const int j = lane + 64 * (WPT * i + half);
      if (j < ldO) xO[m * ldO + j] = f2h_mul(static_cast<float>(code[i]), sm1j[i]);
    }
    return;
  }
  if (!valid) return;
  const float inv = (a == 0.0f) ? 0.0f : div_rn(127.0f, a);
  if (lane == 0 && half == 0) scale[m] = (a == 0.0f) ? 0.0f : div_rn(a, 127.0f);

  int8_t* qr = q + m * K;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = chunk(i);
    if (c < nchunks) {
      float v[8];
      if constexpr (HAS_R) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = vr[i][j];
      } else {
        unpack8_f16(raw[i], v);
      }
      *reinterpret_cast<uint2*>(qr + c * 8) = sym_codes8<HAS_R>(v, inv);
    }
  }
  for (int i = CH; chunk(i) - lane < nchunks; ++i) {
    const int c = chunk(i);
    if (c < nchunks) {
      float v[8];
      load8_f16(xr + c * 8, v);
      scale_chunk<HAS_R>(r, c, v);
      *reinterpret_cast<uint2*>(qr + c * 8) = sym_codes8<HAS_R>(v, inv);
    }
  }
  if (ldO == 0) return;

  if constexpr (OL) {
#pragma unroll
    for (int i = 0; i < kSl; ++i) {
      const int j = lane + 64 * (WPT * i + half);
      if (j < ldO) {
        int code = 0;
        if (oj[i] >= 0) {
          float vv = h2f(rowl[oj[i]]);
          if constexpr (HAS_R) vv = mul_rn(vv, rj[i]);
          code = sym_code(vv, inv);
        }
        if (qO != nullptr) qO[m * ldO + j] = static_cast<int8_t>(code);
        if (xO != nullptr) xO[m * ldO + j] = f2h_mul(static_cast<float>(code), sm1j[i]);
      }
    }
  } else {
    for (int j = lane + 64 * half; j < ldO; j += 64 * WPT) {
      const int o = j < nO ? O[j] : -1;
      int code = 0;
      float sm1 = 0.0f;
      if (o >= 0 && o < K) {
        float vv = h2f(xr[o]);
        if constexpr (HAS_R) vv = mul_rn(vv, load_r(r, o));
        code = sym_code(vv, inv);
        if (xO != nullptr) sm1 = sub_rn(s[o], 1.0f);
      }
      if (qO != nullptr) qO[m * ldO + j] = static_cast<int8_t>(code);
      if (xO != nullptr) xO[m * ldO + j] = f2h_mul(static_cast<float>(code), sm1);
    }
  }
}

// ---------------------------------------------------------------------------
// OffQ: t = (x*d) H_128 per group, exact (float64 butterflies; inputs are fp16
// so every partial sum has at most 47 significant bits), rounded once to fp32;
// then per-token asymmetric int4.
//
// Work split: a 128-channel group is held by 4 consecutive lanes, 32 channels
// each.  Butterflies of span 1..16 stay in the lane; spans 32 and 64 pair the
// lanes of a quad.
// ---------------------------------------------------------------------------
constexpr int kHadRegChunks = 2;  // 32-channel chunks held in registers per lane

// Value of lane ^ 1 (MASK == 1) or lane ^ 2 (MASK == 2) within each quad, by
// DPP quad permutes of the two halves (no LDS round trip).
template <int MASK>
__device__ __forceinline__ double quad_xor_f64(double v) {
  constexpr int ctrl = (MASK == 1) ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  // Every lane of a quad permute has a source, so no "old" value is needed
  // (mov_dpp, all rows and banks enabled).
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b & 0xffffffffu), ctrl, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), ctrl, 0xF, 0xF, true);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}

// Transforms the 32-channel chunk c (group c/4, quarter c%4, with c%4 == lane%4).
__device__ __forceinline__ void hadamard_chunk(const uint16_t* xr, const int8_t* signs, int c,
                                               float (&t)[32]) {
  double u[32];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    v4i raw = *reinterpret_cast<const v4i*>(xr + c * 32 + p * 8);
    const uint2 sraw = *reinterpret_cast<const uint2*>(signs + c * 32 + p * 8);
    // x * d on the fp16 bits: the sign bit (bit 7) of d's bytes 2i and 2i+1
    // is moved to bits 15 and 31 of the mask of fp16 pair i (a byte permute
    // with zero bytes, then an AND) and XORed in.  Exact, as is the widening.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t sw = (i < 2) ? sraw.x : sraw.y;
      const uint32_t sel = (i & 1) ? 0x030c020cu : 0x010c000cu;
      const uint32_t mask = __builtin_amdgcn_perm(0u, sw, sel) & 0x80008000u;
      raw[i] = static_cast<int>(static_cast<uint32_t>(raw[i]) ^ mask);
    }
    float f[8];
    unpack8_f16(raw, f);
#pragma unroll
    for (int j = 0; j < 8; ++j) u[p * 8 + j] = static_cast<double>(f[j]);
  }
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      if ((e & h) == 0) {
        const double a = u[e], b = u[e + h];
        u[e] = a + b;
        u[e + h] = a - b;
      }
    }
  }
  // Spans 32 and 64 pair the lanes of a quad: the lower lane of a pair keeps
  // u + other, the upper one other - u.  Both are fma(u, +-1, other): the
  // product is exact, so the one rounding is that of the add or subtract.
  const int quarter = c & 3;
  {  // span 32: lanes xor 1
    const double sg = (quarter & 1) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) u[e] = __builtin_fma(u[e], sg, quad_xor_f64<1>(u[e]));
  }
  {  // span 64: lanes xor 2
    const double sg = (quarter & 2) ? -1.0 : 1.0;
#pragma unroll
    for (int e = 0; e < 32; ++e) u[e] = __builtin_fma(u[e], sg, quad_xor_f64<2>(u[e]));
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) t[e] = static_cast<float>(u[e]);
}

__device__ __forceinline__ int asym_code(float t, float inv, int z) {
  int c = static_cast<int>(rint_f(mul_rn(t, inv))) + z;
  return c < 0 ? 0 : (c > 15 ? 15 : c);
}

__device__ __forceinline__ uint4 pack_codes(const float (&t)[32], float inv, int z, int& sum) {
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const int code = asym_code(t[e], inv, z);
    sum += code;
    w[e >> 3] |= static_cast<uint32_t>(code) << (4 * (e & 7));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// One wavefront per token (four tokens per workgroup): lane l holds the
// 32-channel chunks c = l + 64 i, so the four chunks of a 128-channel group
// sit in the four lanes of a quad at the same register index, and the
// per-token min, max and code sum are wavefront reductions (no LDS, no
// barrier).  Rows longer than 64 * kHadRegChunks chunks recompute the
// transform of the tail for the coding pass.
constexpr int kHadWaves = 4;

__global__ __launch_bounds__(64 * kHadWaves) void hadamard_offset_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int8_t* __restrict__ signs,
    uint8_t* __restrict__ q4, float* __restrict__ scale, int32_t* __restrict__ zero,
    int32_t* __restrict__ rowsum, float* __restrict__ tout) {
  const int lane = threadIdx.x & 63;
  const int64_t m = static_cast<int64_t>(blockIdx.x) * kHadWaves + (threadIdx.x >> 6);
  if (m >= M) return;  // uniform per wave
  const uint16_t* xr = x + m * K;
  const int nchunks = static_cast<int>(K / 32);  // a multiple of 4: whole quads

  float t[kHadRegChunks][32];
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kHadRegChunks; ++i) {
    const int c = lane + 64 * i;
    if (64 * i < nchunks) {  // uniform: quads are whole
      const int cc = c < nchunks ? c : (c & 3);
      hadamard_chunk(xr, signs, cc, t[i]);
      if (c < nchunks) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          mn = fminf(mn, t[i][e]);
          mx = fmaxf(mx, t[i][e]);
        }
        if (tout != nullptr) {
          float* dst = tout + m * K + static_cast<int64_t>(c) * 32;
#pragma unroll
          for (int e = 0; e < 32; e += 4)
            *reinterpret_cast<float4*>(dst + e) = make_float4(t[i][e], t[i][e + 1], t[i][e + 2], t[i][e + 3]);
        }
      }
    }
  }
  for (int base = 64 * kHadRegChunks; base < nchunks; base += 64) {
    const int c = base + lane;
    const int cc = c < nchunks ? c : (c & 3);
    float tt[32];
    hadamard_chunk(xr, signs, cc, tt);
    if (c < nchunks) {
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        mn = fminf(mn, tt[e]);
        mx = fmaxf(mx, tt[e]);
      }
      if (tout != nullptr) {
        float* dst = tout + m * K + static_cast<int64_t>(c) * 32;
#pragma unroll
        for (int e = 0; e < 32; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(tt[e], tt[e + 1], tt[e + 2], tt[e + 3]);
      }
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const float rng = sub_rn(mx, mn);
  const float inv = (rng == 0.0f) ? 1.0f : div_rn(15.0f, rng);
  const float step = (rng == 0.0f) ? 1.0f : div_rn(rng, 15.0f);
  const int z = static_cast<int>(rint_f(mul_rn(-mn, inv)));

  int sum = 0;
  uint8_t* qr = q4 + m * (K / 2);
#pragma unroll
  for (int i = 0; i < kHadRegChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < nchunks) *reinterpret_cast<uint4*>(qr + static_cast<int64_t>(c) * 16) = pack_codes(t[i], inv, z, sum);
  }
  for (int base = 64 * kHadRegChunks; base < nchunks; base += 64) {
    const int c = base + lane;
    const int cc = c < nchunks ? c : (c & 3);
    float tt[32];
    hadamard_chunk(xr, signs, cc, tt);
    if (c < nchunks) *reinterpret_cast<uint4*>(qr + static_cast<int64_t>(c) * 16) = pack_codes(tt, inv, z, sum);
  }
  sum = wave_sum(sum);
  if (lane == 0) {
    scale[m] = step;
    zero[m] = z;
    rowsum[m] = sum;
  }
}

// Group-wise offsets (OffQ, methodology, grouped implementation): every
// 128-channel group of a token has its own step, zero point and code sum.
// The four chunks of a group sit in the four lanes of a quad, so the group's
// min, max and code sum are two quad exchanges each, and one pass over the
// row suffices: each group is coded as soon as it is transformed.
template <int MASK>
__device__ __forceinline__ int quad_xor_i32(int v) {
  constexpr int ctrl = (MASK == 1) ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, true);
}

__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, __builtin_bit_cast(float, quad_xor_i32<1>(__builtin_bit_cast(int, v))));
  return fminf(v, __builtin_bit_cast(float, quad_xor_i32<2>(__builtin_bit_cast(int, v))));
}

__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, quad_xor_i32<1>(__builtin_bit_cast(int, v))));
  return fmaxf(v, __builtin_bit_cast(float, quad_xor_i32<2>(__builtin_bit_cast(int, v))));
}

__device__ __forceinline__ int quad_sum(int v) {
  v += quad_xor_i32<1>(v);
  return v + quad_xor_i32<2>(v);
}

__global__ __launch_bounds__(64 * kHadWaves) void hadamard_offset_group_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int8_t* __restrict__ signs,
    uint8_t* __restrict__ q4, float* __restrict__ scale, int32_t* __restrict__ zero,
    int32_t* __restrict__ rowsum, float* __restrict__ tout) {
  const int lane = threadIdx.x & 63;
  // Two waves per token: wave half h takes the 64-chunk blocks h, h + 2, ...
  // (a group's four chunks stay in one quad of one wave).
  const int64_t wg = static_cast<int64_t>(blockIdx.x) * kHadWaves + (threadIdx.x >> 6);
  const int64_t m = wg >> 1;
  const int half = static_cast<int>(wg & 1);
  if (m >= M) return;  // uniform per wave
  const uint16_t* xr = x + m * K;
  const int nchunks = static_cast<int>(K / 32);  // a multiple of 4: whole quads
  const int64_t G = K / 128;
  uint8_t* qr = q4 + m * (K / 2);
  for (int base = 64 * half; base < nchunks; base += 128) {  // uniform
    const int c = base + lane;
    // A lane past the row transforms an in-range chunk of the same quarter,
    // so that its quad takes part in the exchanges, and stores nothing.
    const int cc = c < nchunks ? c : (c & 3);
    float t[32];
    hadamard_chunk(xr, signs, cc, t);
    float mn = t[0], mx = t[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
      mn = fminf(mn, t[e]);
      mx = fmaxf(mx, t[e]);
    }
    mn = quad_min(mn);
    mx = quad_max(mx);
    const float rng = sub_rn(mx, mn);
    const float inv = (rng == 0.0f) ? 1.0f : div_rn(15.0f, rng);
    const float step = (rng == 0.0f) ? 1.0f : div_rn(rng, 15.0f);
    const int z = static_cast<int>(rint_f(mul_rn(-mn, inv)));
    int sum = 0;
    const uint4 codes = pack_codes(t, inv, z, sum);
    sum = quad_sum(sum);
    if (c < nchunks) {
      *reinterpret_cast<uint4*>(qr + static_cast<int64_t>(c) * 16) = codes;
      if (tout != nullptr) {
        float* dst = tout + m * K + static_cast<int64_t>(c) * 32;
#pragma unroll
        for (int e = 0; e < 32; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(t[e], t[e + 1], t[e + 2], t[e + 3]);
      }
      if ((c & 3) == 0) {
        const int64_t gi = m * G + (c >> 2);
        scale[gi] = step;
        zero[gi] = z;
        rowsum[gi] = sum;
      }
    }
  }
}

}  // namespace

qlin_status launch_quant_grad(const uint16_t* dy, int64_t M, int64_t N, const uint16_t* sw, int8_t* gq, float* gs,
                              hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((M + kQuantTokens - 1) / kQuantTokens));
  if (N <= 4096)
    quant_act_kernel<true, false, kQuantCh4k, uint16_t, false, kQuantWpt><<<grid, kQuantThreads, 0, st>>>(
        dy, M, N, sw, gq, gs, nullptr, 0, 0, nullptr, nullptr, nullptr, MomFold{});
  else
    quant_act_kernel<true, false, kQuantCh8k, uint16_t, false, kQuantWpt><<<grid, kQuantThreads, 0, st>>>(
        dy, M, N, sw, gq, gs, nullptr, 0, 0, nullptr, nullptr, nullptr, MomFold{});
  QLIN_LAUNCH_CHECK("quant_act_kernel (gradient)");
  return QLIN_OK;
}

qlin_status launch_quant_momentum(const uint16_t* x, int64_t M, int64_t K, const float* r, int8_t* q, float* scale,
                                  const int32_t* O, int32_t nO, uint16_t* xO, const MomFold& mf, hipStream_t st) {
  const int ldO = static_cast<int>(outlier_ld(nO));
  const dim3 grid(static_cast<unsigned>((M + kQuantTokens - 1) / kQuantTokens));
  // The two tokens' rows of codes.
  const size_t lds = static_cast<size_t>(kQuantTokens) * static_cast<size_t>(K);
  if (K <= 4096)
    quant_act_kernel<true, true, kQuantCh4k, float, true, kQuantWpt><<<grid, kQuantThreads, lds, st>>>(
        x, M, K, r, q, scale, O, nO, ldO, nullptr, nullptr, xO, mf);
  else
    quant_act_kernel<true, true, kQuantCh8k, float, true, kQuantWpt><<<grid, kQuantThreads, lds, st>>>(
        x, M, K, r, q, scale, O, nO, ldO, nullptr, nullptr, xO, mf);
  QLIN_LAUNCH_CHECK("quant_act_kernel (momentum folded)");
  return QLIN_OK;
}

}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_quant_act(const uint16_t* x, int64_t M, int64_t K, const float* r,
                                      int8_t* q, float* scale, const int32_t* O, int32_t nO,
                                      const float* s, int8_t* qO, uint16_t* xO, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(x);
  QLIN_PTR(q);
  QLIN_PTR(scale);
  QLIN_OPT_PTR(r);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_REQUIRE(qO != nullptr || xO != nullptr, QLIN_ERR_INVALID_ARG, "nO > 0 needs qO or xO");
    QLIN_OPT_PTR(qO);
    QLIN_OPT_PTR(xO);
    if (xO != nullptr) QLIN_PTR(s);
  } else {
    QLIN_REQUIRE(O == nullptr && qO == nullptr && xO == nullptr, QLIN_ERR_INVALID_ARG,
                 "O, qO and xO must be NULL when nO == 0");
  }
  const int ldO = static_cast<int>(outlier_ld(nO));
  QLIN_REQUIRE(M / kQuantTokens < 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  const dim3 grid(static_cast<unsigned>((M + kQuantTokens - 1) / kQuantTokens));
  // Outlier columns through LDS when they fit (2K bytes per token).
  const size_t ol_lds = static_cast<size_t>(kQuantTokens) * 2 * static_cast<size_t>(K);
  const bool ol = nO > 0 && ldO <= kOutlierLdMax && ol_lds <= 160 * 1024;
  hipStream_t st = as_stream(stream);
  auto go = [&](auto has_r, auto ol_c, auto ch) {
    constexpr bool HR = decltype(has_r)::value, OLc = decltype(ol_c)::value;
    constexpr int CH = decltype(ch)::value;
    quant_act_kernel<HR, OLc, CH, float, false, kQuantWpt><<<grid, kQuantThreads, OLc ? ol_lds : 0, st>>>(
        x, M, K, r, q, scale, O, nO, ldO, s, qO, xO, MomFold{});
  };
  auto go_ch = [&](auto has_r, auto ol_c) {
    if (K <= 4096)
      go(has_r, ol_c, std::integral_constant<int, kQuantCh4k>{});
    else if (K <= 8192)
      go(has_r, ol_c, std::integral_constant<int, kQuantCh8k>{});
    else
      go(has_r, ol_c, std::integral_constant<int, kQuantCh12k>{});
  };
  auto go_ol = [&](auto has_r) {
    if (ol)
      go_ch(has_r, std::true_type{});
    else
      go_ch(has_r, std::false_type{});
  };
  if (r != nullptr)
    go_ol(std::true_type{});
  else
    go_ol(std::false_type{});
  QLIN_LAUNCH_CHECK("quant_act_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_hadamard_offset(const uint16_t* x, int64_t M, int64_t K,
                                            const int8_t* signs, int32_t block, uint8_t* q4,
                                            float* scale, int32_t* zero, int32_t* rowsum,
                                            float* t, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(block == 128, QLIN_ERR_UNSUPPORTED, "block=%d: only 128 is provided", block);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(x);
  QLIN_PTR(signs);
  QLIN_PTR(q4);
  QLIN_PTR(scale);
  QLIN_PTR(zero);
  QLIN_PTR(rowsum);
  QLIN_OPT_PTR(t);
  QLIN_REQUIRE(M / kHadWaves < 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  hadamard_offset_kernel<<<dim3(static_cast<unsigned>((M + kHadWaves - 1) / kHadWaves)), 64 * kHadWaves, 0,
                           as_stream(stream)>>>(x, M, K, signs, q4, scale, zero, rowsum, t);
  QLIN_LAUNCH_CHECK("hadamard_offset_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_hadamard_offset_group(const uint16_t* x, int64_t M, int64_t K,
                                                  const int8_t* signs, int32_t block, uint8_t* q4,
                                                  float* scale, int32_t* zero, int32_t* rowsum,
                                                  float* t, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(block == 128, QLIN_ERR_UNSUPPORTED, "block=%d: only 128 is provided", block);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(x);
  QLIN_PTR(signs);
  QLIN_PTR(q4);
  QLIN_PTR(scale);
  QLIN_PTR(zero);
  QLIN_PTR(rowsum);
  QLIN_OPT_PTR(t);
  QLIN_REQUIRE(2 * M / kHadWaves < 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  hadamard_offset_group_kernel<<<dim3(static_cast<unsigned>((2 * M + kHadWaves - 1) / kHadWaves)), 64 * kHadWaves, 0,
                                 as_stream(stream)>>>(x, M, K, signs, q4, scale, zero, rowsum, t);
  QLIN_LAUNCH_CHECK("hadamard_offset_group_kernel");
  return QLIN_OK;
}
