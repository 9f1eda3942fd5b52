// Packed weight layouts read by the GEMM kernels (private to libqlin).
//
// Every layout is a grid of 1 KB "lane tiles": 64 lanes x 16 bytes, what one
// wavefront loads with a single 16-byte load per lane.  Lane l of a tile
// serves output column 32*nt + (l & 31) and the k half (l >> 5) of a k step,
// which is the B-operand layout of v_mfma_i32_32x32x32_i8 (16 int8 per lane)
// and of v_mfma_f32_32x32x16_f16 (8 fp16 per lane).  The order of k inside a
// lane only has to agree between the A and B operands.
//
//   W8  tile (s, nt), s < K/32:   byte j of lane l = code(k = 32 s + 16 (l>>5) + j)
//   W4S tile (p, nt), p < K/64:   bytes 0..7: k step 2p, bytes 8..15: k step 2p+1
//        (k = 64 p + 32 h + 16 (l>>5) + j for half h); within each 8 bytes,
//        byte b of word i holds code(8 i + b) in the low nibble and
//        code(8 i + 4 + b) in the high nibble, so (w << 4) & 0xF0F0F0F0 and
//        w & 0xF0F0F0F0 are the int8 values 16*q4 for j = 8i+0..3 and 8i+4..7.
//   W4U same tiling as W4S with the natural packing (byte b of each 8 holds
//        code(2b) | code(2b+1) << 4), the packing of the int4 activations, so
//        both operands unpack to the same k order.
//   WO  tile (s, nt), s < ldO/16: fp16 value i of lane l = WO[16 s + 8 (l>>5) + i][n]
//        (rows beyond nO are zero).
// W8, W4S, W4U: the tiles of a 32-column strip are contiguous along K, tile
// (s, nt) starting at byte (nt * KT + s) * 1024 with KT = K/32 (W8) or K/64
// (W4): a kernel that owns a strip streams one contiguous range of memory.
// WO: tile (s, nt) starts at byte ((s * (N/32)) + nt) * 1024.
#pragma once

#include <stdint.h>

namespace qlin {

constexpr int kLaneTileBytes = 1024;

inline int64_t outlier_ld(int64_t nO) { return (nO + 15) / 16 * 16; }

}  // namespace qlin
