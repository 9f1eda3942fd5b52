// Quaff's sparse compensation term for one wave's output fragments, on fp16
// matrix cores (v_mfma_f32_32x32x16_f16).
//
// Quaff paper notes, "key design" (decoupled WAQ): Y = X^(sW) splits into the
// static int8 product X^W and X^_{:,O}(s_O - 1)W_O, where (s - 1) vanishes off
// the outlier set O.  The activation side arrives precomputed by the
// quantization kernel as xO[m, j] = fp16(q[m, O[j]] * (s[O[j]] - 1)) with a
// row stride ldO (a multiple of 16, zero padded), so each A fragment is one
// 16-byte load; W_O arrives packed in fragment order (layout.hpp).  The
// accumulation is fp32, added onto fragments that already hold acc * sw; the
// caller multiplies by the token step sa[m] afterwards.
#pragma once

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
  const int lane = threadIdx.x & 63;
  const int64_t tiles32 = N / 32;
  const uint16_t* arow[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    int64_t m = m0 + 32 * tm + (lane & 31);
    m = m < M ? m : M - 1;
    arow[tm] = xO + m * ldO + 8 * (lane >> 5);
  }
  for (int js = 0; js < ldO / 16; ++js) {
    v8h ap[TM], bp[NT];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) ap[tm] = *reinterpret_cast<const v8h*>(arow[tm] + 16 * js);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      bp[nt] = *reinterpret_cast<const v8h*>(WOp + ((static_cast<int64_t>(js) * tiles32 + nt32 + nt) << 10) + lane * 16);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        f[tm][nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bp[nt], ap[tm], f[tm][nt], 0, 0, 0);
  }
}

}  // namespace qlin
