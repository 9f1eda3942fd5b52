// Quaff's sparse compensation term for one wave's output fragments, on fp16
// matrix cores (v_mfma_f32_32x32x16_f16).
//
// Quaff paper notes, "key design" (decoupled WAQ): Y = X^(sW) splits into the
// static int8 product X^W and X^_{:,O}(s_O - 1)W_O, where (s - 1) vanishes off
// the outlier set O.  The activation side arrives precomputed by the
// quantization kernel as xO[m, j] = fp16(q[m, O[j]] * (s[O[j]] - 1)) with a
// row stride ldO (a multiple of 16, zero padded), so each A fragment is one
// 16-byte load; W_O arrives packed in fragment order (layout.hpp).  The
// accumulation is fp32, onto fragments that already hold acc * sw; the
// caller multiplies by the token step sa[m] afterwards.
#pragma once

#include <utility>

#include "common.hpp"

namespace qlin {

// f[tm][nt]: fragments of rows m0 + 32 tm + [0, 32) and 32-column tiles
// nt32 + nt, transposed like the integer accumulators (W_O is the first
// operand): lane l holds row (l & 31), register v column
// 8*(v>>2) + 4*(l>>5) + (v&3).  Rows at or past M read row M - 1 (their
// results are discarded).
template <int TM, int NT>
__device__ __forceinline__ void comp_accumulate(v16f (&f)[TM][NT], const uint16_t* __restrict__ xO,
                                                int ldO, const uint8_t* __restrict__ WOp, int64_t M,
                                                int64_t N, int64_t m0, int64_t nt32) {
  // Operands of D = 4 k steps are in flight while the matrix cores work on
  // the oldest one; a step's registers are refilled right after its MFMAs.
  constexpr int D = 4;
  const int lane = threadIdx.x & 63;
  const int64_t tiles32 = N / 32;
  const uint16_t* arow[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    int64_t m = m0 + 32 * tm + (lane & 31);
    m = m < M ? m : M - 1;
    arow[tm] = xO + m * ldO + 8 * (lane >> 5);
  }
  const uint8_t* bcol = WOp + (nt32 << 10) + lane * 16;
  auto load = [&](int js, v8h (&ap)[TM], v8h (&bp)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) ap[tm] = *reinterpret_cast<const v8h*>(arow[tm] + 16 * js);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      bp[nt] = *reinterpret_cast<const v8h*>(bcol + ((static_cast<int64_t>(js) * tiles32 + nt) << 10));
  };
  auto mma = [&](const v8h (&ap)[TM], const v8h (&bp)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        f[tm][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bp[nt], ap[tm], f[tm][nt], 0, 0, 0);
  };
  const int nj = ldO / 16;
  const int nfull = nj / D * D;
  v8h ap[D][TM], bp[D][NT];
  if (nfull > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(d, ap[d], bp[d]);
      __builtin_amdgcn_sched_barrier(0);  // issue the slots in order: slot 0 arrives first
    }
    for (int j0 = 0; j0 < nfull; j0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        mma(ap[d], bp[d]);
        const int nxt = j0 + D + d;
        load(nxt < nfull ? nxt : nfull - 1, ap[d], bp[d]);  // past the end: a harmless reload
      }
      // Keep that order: each step's MFMAs, then the refill of its registers.
#pragma unroll
      for (int d = 0; d < D; ++d) {
        __builtin_amdgcn_sched_group_barrier(0x008, TM * NT, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, TM + NT, 0);
      }
    }
  }
  for (int js = nfull; js < nj; ++js) {
    load(js, ap[0], bp[0]);
    mma(ap[0], bp[0]);
  }
}

// As comp_accumulate, with the activation side already staged in LDS: rows
// m0 + [0, 32*TM) of xO at a pitch of `pitch` bytes (xlds), nj k steps of 16.
// The steps run in blocks of D; the W_O fragments of block b + 1 are loaded
// into the other register set before block b's matrix-core work, so each
// load has a whole block of cover.  Steps past nj (padding up to an even
// number of blocks) use zero activation fragments: adding 0 * w_O leaves an
// fp32 sum unchanged.
template <int TM, int NT>
__device__ __forceinline__ void comp_accumulate_lds(v16f (&f)[TM][NT], const uint8_t* xlds, int pitch, int nj,
                                                    const uint8_t* __restrict__ WOp, int64_t N, int64_t nt32) {
  constexpr int D = 4;
  const int lane = threadIdx.x & 63;
  const int64_t tiles32 = N / 32;
  const uint8_t* arow = xlds + (lane & 31) * pitch + 16 * (lane >> 5);
  const uint8_t* bcol = WOp + (nt32 << 10) + lane * 16;
  auto load_block = [&](int blk, v8h (&bp)[D][NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      int js = blk * D + d;
      js = js < nj ? js : nj - 1;  // padding steps: a harmless reload
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bp[d][nt] = *reinterpret_cast<const v8h*>(bcol + ((static_cast<int64_t>(js) * tiles32 + nt) << 10));
    }
  };
  auto mma_block = [&](int blk, const v8h (&bp)[D][NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int js = blk * D + d;
      const bool real = js < nj;
      const int jr = real ? js : nj - 1;
      v8h ap[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const v8h a = *reinterpret_cast<const v8h*>(arow + tm * 32 * pitch + 32 * jr);
        ap[tm] = real ? a : v8h{};
      }
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          f[tm][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bp[d][nt], ap[tm], f[tm][nt], 0, 0, 0);
    }
  };
  const int nb = (nj + D - 1) / D;
  v8h b0[D][NT], b1[D][NT];
  load_block(0, b0);
  for (int blk = 0; blk < nb; blk += 2) {
    load_block(blk + 1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma_block(blk, b0);
    __builtin_amdgcn_sched_barrier(0);
    load_block(blk + 2, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma_block(blk + 1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
}
// As comp_accumulate_lds, with the W_O fragments staged in LDS too: step js,
// column tile nt at wlds + (NT js + nt) * 1 KB + 16 lane (one lane tile each).
// The fragments of step js + 1 are read before the products of step js.
template <int TM, int NT>
__device__ __forceinline__ void comp_accumulate_lds2(v16f (&f)[TM][NT], const uint8_t* xlds, int pitch, int nj,
                                                     const uint8_t* wlds) {
  const int lane = threadIdx.x & 63;
  const uint8_t* arow = xlds + (lane & 31) * pitch + 16 * (lane >> 5);
  const uint8_t* bcol = wlds + lane * 16;
  auto read = [&](int js, v8h (&ap)[TM], v8h (&bp)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) ap[tm] = *reinterpret_cast<const v8h*>(arow + tm * 32 * pitch + 32 * js);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bp[nt] = *reinterpret_cast<const v8h*>(bcol + (NT * js + nt) * 1024);
  };
  auto mma = [&](const v8h (&ap)[TM], const v8h (&bp)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        f[tm][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bp[nt], ap[tm], f[tm][nt], 0, 0, 0);
  };
  if (nj <= 0) return;
  v8h a0[TM], b0[NT], a1[TM], b1[NT];
  read(0, a0, b0);
  int js = 0;
  for (; js + 2 <= nj; js += 2) {
    read(js + 1, a1, b1);
    mma(a0, b0);
    if (js + 2 < nj) read(js + 2, a0, b0);
    mma(a1, b1);
  }
  if (js < nj) mma(a0, b0);
}

}  // namespace qlin
