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

}  // namespace qlin
