// Packed weight layouts read by the GEMM kernels (private to libqlin).
//
// All layouts are built from 1 KB "lane tiles": 64 lanes x 16 bytes, which is
// exactly what one wavefront loads with one 16-byte load per lane.  Lane l
// covers output column n = 16*nt + (l & 15) and the 16-wide k slice
// g = l >> 4 of a 64-wide k step, which is the operand layout of
// v_mfma_i32_16x16x64_i8 (16 k values per lane; the k order inside the slice
// only has to agree between the two operands).
//
//   W8  : [K/64][N/16][64 lanes][16 bytes]   byte j = code(k = 64*s + 16*g + j)
//   W4S : [K/128][N/16][64 lanes][16 bytes]  bytes 0..7: k step 2s, 8..15: k step 2s+1;
//         within 8 bytes (two 32-bit words) byte b of word i holds
//         code(16*g + 8*i + b) in the low nibble and code(16*g + 8*i + 4 + b)
//         in the high nibble, so (w << 4) & 0xF0F0F0F0 and w & 0xF0F0F0F0 give
//         the shifted int8 values 16*q4 for k = 8i+0..3 and 8i+4..7 in order.
//   W4U : same tiling as W4S with the natural packing: byte b of the 8 holds
//         code(16*g + 2b) | code(16*g + 2b + 1) << 4, i.e. the packing of the
//         int4 activations, so both operands unpack to the same k order.
#pragma once

#include <stdint.h>

namespace qlin {

constexpr int kLaneTileBytes = 1024;

inline int64_t packed_bytes_w8(int64_t K, int64_t N) { return K * N; }
inline int64_t packed_bytes_w4(int64_t K, int64_t N) { return K * N / 2; }

}  // namespace qlin
