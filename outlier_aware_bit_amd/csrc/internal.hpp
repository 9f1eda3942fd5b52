// Launchers shared between the source files of libqlin (not exported).  The
// caller validates every argument; these only launch.
#pragma once

#include "common.hpp"

namespace qlin {

// Per-token symmetric int8 of G = dy * sw (sw fp16 [N], widened to fp32):
// gq int8 [M x N], gs fp32 [M].
qlin_status launch_quant_grad(const uint16_t* dy, int64_t M, int64_t N, const uint16_t* sw, int8_t* gq, float* gs,
                              hipStream_t st);

// dx[m, k] = fp16(r[k] * (gs[m] * acc[m, k] + [k = O[j]] (s[k] - 1) * cb[m * ldO + j])),
// acc = gq [M x N] times the transposed weights (QLIN_LAYOUT_W8T of [K x N]).
qlin_status launch_gemm_bwd(const int8_t* gq, const float* gs, const void* w8t, const float* r, const float* s,
                            const int32_t* O, int32_t nO, const float* cb, int64_t M, int64_t N, int64_t K,
                            uint16_t* dx, int32_t* acc, hipStream_t st);

// Momentum update folded into the quantizer (qlin_quaff_momentum_quant): the
// column maxima of the outlier channels are taken over kMomFoldBlocks row
// blocks by momentum_block_kernel, and every quantizer workgroup folds them.
constexpr int kMomFoldBlocks = 4;
struct MomFold {
  // [(kMomFoldBlocks + 1) x nO]: row block b's max |x[:, O[j]]| at b * nO + j,
  // then s[O[j]] as it was before the step.
  const float* part;
  const float* wmax;  // [nO]: max_n |W[O[j], n]|
  float gamma;
  float* s;  // s and r at the outlier channels, written by the first workgroup
  float* r;
};

// Between the two launches r[O[j]] holds a NaN whose low bits are j (j < 256):
// the quantizer finds its outlier channels in the r it reads for the row.
constexpr uint32_t kMomSlotTag = 0x7ff00000u, kMomSlotMask = 0xffu;
__device__ __forceinline__ float mom_slot_marker(int j) {
  return __builtin_bit_cast(float, kMomSlotTag | static_cast<uint32_t>(j));
}

// qlin_quant_act with r and xO (nO in [1, 256], K <= 8192), where r[O[j]],
// s[O[j]] are those of the momentum step folded from mf.part rather than
// read from r and s; r must already hold 1 / s at every other channel.
qlin_status launch_quant_momentum(const uint16_t* x, int64_t M, int64_t K, const float* r, int8_t* q, float* scale,
                                  const int32_t* O, int32_t nO, uint16_t* xO, const MomFold& mf, hipStream_t st);

}  // namespace qlin
