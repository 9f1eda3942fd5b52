// Quaff's sparse compensation term for one output tile, on fp16 matrix cores.
//
// Quaff paper notes, "key design" (decoupled WAQ): Y = X^(sW) splits into the
// static int8 product X^W and X^_{:,O}(s_O - 1)W_O, where (s - 1) vanishes off
// the outlier set O.  With X^_{m,o} = qO[m,o] * sa[m], the tile accumulates
//     acc[m,n] += sum_j fp16(qO[m,j] * (s[O[j]] - 1)) * WO[j,n]
// (fp32 accumulation); the caller multiplies by sa[m] afterwards.
//
// Operands are staged through LDS in chunks of 32 outlier channels (the K of
// v_mfma_f32_16x16x32_f16): A' as [BM][32] and W_O transposed as [BN][32],
// rows padded to 80 bytes so the 16-byte fragment reads of 8 consecutive rows
// fall on distinct banks.
#pragma once

#include "common.hpp"

namespace qlin {

constexpr int kCompChunk = 32;
constexpr int kCompRowHalfs = 40;  // 32 values + 8 padding (80 bytes)

template <int BM, int BN>
constexpr int comp_lds_bytes() {
  return (BM + BN) * kCompRowHalfs * 2 + kCompChunk * 4;
}

// acc[tm][tn]: 16x16 fp32 fragments of this wave (lane l -> column l & 15,
// rows 4 * (l >> 4) + i).  The wave owns rows wrow0 + [0, 16*TM) and columns
// wcol0 + [0, 16*TN) of the BM x BN tile at (m0, n0).
template <int BM, int BN, int NTHREADS, int TM, int TN>
__device__ __forceinline__ void comp_accumulate(v4f (&acc)[TM][TN], const int8_t* __restrict__ qO,
                                                const int32_t* __restrict__ O, int nO,
                                                const float* __restrict__ s,
                                                const uint16_t* __restrict__ WO, int64_t M,
                                                int64_t N, int64_t K, int64_t m0, int64_t n0,
                                                int wrow0, int wcol0, uint8_t* lds) {
  _Float16* lA = reinterpret_cast<_Float16*>(lds);
  _Float16* lB = lA + BM * kCompRowHalfs;
  float* lS = reinterpret_cast<float*>(lB + BN * kCompRowHalfs);
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  for (int j0 = 0; j0 < nO; j0 += kCompChunk) {
    __syncthreads();
    if (tid < kCompChunk) {
      const int j = j0 + tid;
      float v = 0.0f;
      if (j < nO) {
        const int o = O[j];
        if (o >= 0 && o < K) v = sub_rn(s[o], 1.0f);
      }
      lS[tid] = v;
    }
    __syncthreads();
    // A' = fp16(qO * (s - 1)), rows beyond M and channels beyond nO are 0.
    for (int idx = tid; idx < BM * kCompChunk; idx += NTHREADS) {
      const int mm = idx / kCompChunk, jj = idx % kCompChunk;
      const int64_t m = m0 + mm;
      const int j = j0 + jj;
      float v = 0.0f;
      if (m < M && j < nO) v = mul_rn(static_cast<float>(qO[m * nO + j]), lS[jj]);
      lA[mm * kCompRowHalfs + jj] = static_cast<_Float16>(v);
    }
    // W_O rows j0..j0+31, columns n0..n0+BN-1, stored transposed [n][j].
    for (int idx = tid; idx < kCompChunk * (BN / 8); idx += NTHREADS) {
      const int jj = idx / (BN / 8), nc = idx % (BN / 8);
      const int j = j0 + jj;
      const int64_t n = n0 + nc * 8;
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (j < nO && n < N) raw = *reinterpret_cast<const uint4*>(WO + static_cast<int64_t>(j) * N + n);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint16_t b = static_cast<uint16_t>((w[i >> 1] >> (16 * (i & 1))) & 0xffffu);
        lB[(nc * 8 + i) * kCompRowHalfs + jj] = __builtin_bit_cast(_Float16, b);
      }
    }
    __syncthreads();
    v8h af[TM], bf[TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      af[tm] = *reinterpret_cast<const v8h*>(lA + (wrow0 + tm * 16 + (lane & 15)) * kCompRowHalfs + 8 * (lane >> 4));
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
      bf[tn] = *reinterpret_cast<const v8h*>(lB + (wcol0 + tn * 16 + (lane & 15)) * kCompRowHalfs + 8 * (lane >> 4));
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
  }
}

}  // namespace qlin
