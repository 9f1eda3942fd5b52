// Quaff kernels of libqlin (gfx950):
//   qlin_momentum_update    targeted momentum scaling on the fixed outlier set O
//   qlin_weight_row_absmax  max_n |W_O[o, n]| for beta
//   qlin_outlier_comp       the sparse compensation term added to Y
//
// Source: "Quaff: Quantized Parameter-Efficient Fine-Tuning under Outlier
// Spatial Stability Hypothesis" (paper notes), "key design".
#include <mutex>

#include "common.hpp"
#include "comp.hpp"
#include "internal.hpp"
#include "layout.hpp"

namespace qlin {
namespace {

constexpr int kMomThreads = 256;

// Momentum update, one workgroup per 64-channel strip of X (one 128-byte
// line per token row).  The outliers of a strip share its lines, so reading
// the whole strip once per row fetches every line of X that holds an outlier
// exactly once, with no reduction across workgroups.  The rows of strips
// without an outlier are read too (about 3 of 64 strips at 205 outliers in
// 4096 channels), so that no load waits for the outlier bookkeeping.
// (Splitting a strip's rows over several
// workgroups needs either a second launch to fold their maxima or
// device-scope fences, which write back and invalidate the per-XCD L2
// caches; both cost more than the extra workgroups save at 2048 tokens.)
//   c_k   = max_m |x[m, k]| for the 64 channels k of the strip
//   o in O in the strip:  beta = max(1, sqrt(c_o / wmax)) (1 if wmax == 0),
//                         s_o = gamma*s_o + (1-gamma)*beta, r_o = 1/s_o
//   other channels:       r_k = 1/s_k
constexpr int kStripThreads = 1024;
constexpr int kStripLoads = 16;                             // 16-byte loads in flight per thread
constexpr int kStripRows = kStripThreads / 8 * kStripLoads;  // rows per pass (8 lanes per row)

__global__ __launch_bounds__(kStripThreads) void momentum_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int32_t* __restrict__ O, int nO,
    const float* __restrict__ wmax, float gamma, float* __restrict__ s, float* __restrict__ r) {
  __shared__ float red[kStripThreads / 64][64];
  __shared__ int owner[64];  // 1 + index into O of the outlier at this channel, or 0
  const int64_t strip = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Issue order: the first outlier index of this thread and s of its channel
  // (threads below 64), then the strip's rows, so that the outlier
  // bookkeeping below waits only for the former while the rows are in
  // flight (a wait for a load also waits for every load issued before it).
  // Every load is unconditional, from a clamped, in-range address: a load
  // under a condition compiles to a branch, and after the join the compiler
  // can only count the loads of the shortest path.  Without outliers or rows
  // (x may then be NULL) the row loads read 16 bytes of s instead and are
  // not folded in.
  const bool rx = M > 0 && nO > 0;  // uniform
  const int32_t* const Op = (nO > 0) ? O : reinterpret_cast<const int32_t*>(s);
  const int o_raw = Op[(tid < nO) ? tid : 0];
  const float s_k = s[strip * 64 + lane];
  const uint16_t* const col = (rx ? x : reinterpret_cast<const uint16_t*>(s)) + strip * 64 + (tid & 7) * 8;
  const int64_t ldx = rx ? K : 0;
  const int64_t row0 = tid >> 3;
  auto load_rows = [&](int64_t mb, v4i (&v)[kStripLoads]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kStripLoads; ++i) {
      // Rows past M repeat row M - 1: the maximum is unchanged.
      int64_t m = mb + row0 + static_cast<int64_t>(kStripThreads / 8) * i;
      m = m < M ? m : M - 1;
      v[i] = *reinterpret_cast<const v4i*>(col + m * ldx);
    }
  };
  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // channels 8*(tid&7) + [0, 8)
  auto fold_rows = [&](const v4i (&v)[kStripLoads]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kStripLoads; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = static_cast<uint32_t>(v[i][w]);
        cm[2 * w] = fmaxf(cm[2 * w], fabsf(h2f(static_cast<uint16_t>(u & 0xffffu))));
        cm[2 * w + 1] = fmaxf(cm[2 * w + 1], fabsf(h2f(static_cast<uint16_t>(u >> 16))));
      }
  };
  v4i v[kStripLoads];
  load_rows(0, v);
  if (tid < 64) owner[tid] = 0;
  __syncthreads();
  const int o0 = (tid < nO) ? o_raw : -1;
  if (o0 >= 0 && o0 < K && o0 / 64 == strip) owner[o0 % 64] = tid + 1;
  for (int j = tid + kStripThreads; j < nO; j += kStripThreads) {
    const int o = O[j];
    if (o >= 0 && o < K && o / 64 == strip) owner[o % 64] = j + 1;
  }
  __syncthreads();
  // The outlier's weight-row maximum, also in flight with the rows.
  const int own = (tid < 64) ? owner[tid] : 0;
  const float* const wp = (nO > 0) ? wmax : s;
  const float wm_raw = wp[(own != 0) ? own - 1 : 0];
  const float wm = (own != 0) ? wm_raw : 0.0f;
  if (rx) {
    fold_rows(v);
    for (int64_t mb = kStripRows; mb < M; mb += kStripRows) {
      load_rows(mb, v);
      __builtin_amdgcn_sched_barrier(0);  // all of a pass's loads before any use
      fold_rows(v);
    }
  }
  // Lanes with equal (lane & 7) hold the same channels: combine over lane bits 3..5.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v = cm[c];
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    cm[c] = v;
  }
  if (lane < 8) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[wave][lane * 8 + c] = cm[c];
  }
  __syncthreads();
  if (tid < 64) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < kStripThreads / 64; ++w) c = fmaxf(c, red[w][tid]);
    const int64_t k = strip * 64 + tid;
    if (own != 0) {
      float sn, rn;
      momentum_step(c, wm, gamma, s_k, sn, rn);
      s[k] = sn;
      r[k] = rn;
    } else {
      r[k] = div_rn(1.0f, s_k);
    }
  }
}

// Momentum update in two launches over a workspace, for when the batch is
// long enough that one workgroup per strip leaves most CUs idle.
// momentum_partial_kernel: workgroup (strip, rb) takes the 64 channels of a
// strip over the rows [rb * rows, (rb + 1) * rows) and writes the maxima of
// the strip's outlier channels to part[rb * nO + j]; the row-block 0
// workgroups also write r = 1/s for the strip's other channels.
// momentum_fold_kernel: per outlier j, c = max over the row blocks, then the
// update of s[O[j]] and r[O[j]] (same arithmetic as momentum_kernel).
constexpr int kPartThreads = 256;                       // 8 lanes per row, 32 rows per pass
constexpr int kPartLoads = 4;                           // rows in flight per thread
constexpr int kPartRows = kPartThreads / 8 * kPartLoads;  // 128 rows per pass
constexpr int kMaxRowBlocks = 16;

__global__ __launch_bounds__(kPartThreads) void momentum_partial_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int32_t* __restrict__ O, int nO,
    const float* __restrict__ s, float* __restrict__ r, int64_t rows, float* __restrict__ part) {
  __shared__ float red[kPartThreads / 64][64];
  __shared__ int owner[64];  // 1 + index into O of the outlier at this channel, or 0
  const int64_t strip = blockIdx.x, rb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 64) owner[tid] = 0;
  __syncthreads();
  for (int j = tid; j < nO; j += kPartThreads) {
    const int o = O[j];
    if (o >= 0 && o < K && o / 64 == strip) owner[o % 64] = j + 1;
  }
  __syncthreads();
  if (rb == 0 && tid < 64 && owner[tid] == 0) r[strip * 64 + tid] = div_rn(1.0f, s[strip * 64 + tid]);
  if (!__syncthreads_or(tid < 64 && owner[tid] != 0)) return;

  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // channels 8*(tid&7) + [0, 8)
  const int64_t m_lo = rb * rows, m_hi = (m_lo + rows < M) ? m_lo + rows : M;
  const uint16_t* col = x + strip * 64 + (tid & 7) * 8;
  for (int64_t mb = m_lo + (tid >> 3); mb < m_hi; mb += kPartRows) {
    v4i v[kPartLoads];
#pragma unroll
    for (int i = 0; i < kPartLoads; ++i) {
      // Rows past the block read its last row (always in range): no branch
      // per load, and a repeated row leaves the maximum unchanged.
      int64_t m = mb + static_cast<int64_t>(kPartThreads / 8) * i;
      m = m < m_hi ? m : m_hi - 1;
      v[i] = *reinterpret_cast<const v4i*>(col + m * K);
    }
#pragma unroll
    for (int i = 0; i < kPartLoads; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = static_cast<uint32_t>(v[i][w]);
        cm[2 * w] = fmaxf(cm[2 * w], fabsf(h2f(static_cast<uint16_t>(u & 0xffffu))));
        cm[2 * w + 1] = fmaxf(cm[2 * w + 1], fabsf(h2f(static_cast<uint16_t>(u >> 16))));
      }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v = cm[c];
    v = fmaxf(v, __shfl_xor(v, 8));
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    cm[c] = v;
  }
  if (lane < 8) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[wave][lane * 8 + c] = cm[c];
  }
  __syncthreads();
  if (tid < 64 && owner[tid] != 0) {
    float c = 0.0f;
#pragma unroll
    for (int w = 0; w < kPartThreads / 64; ++w) c = fmaxf(c, red[w][tid]);
    part[rb * nO + owner[tid] - 1] = c;
  }
}

__global__ __launch_bounds__(kMomThreads) void momentum_fold_kernel(
    const float* __restrict__ part, int rblocks, int64_t K, const int32_t* __restrict__ O, int nO,
    const float* __restrict__ wmax, float gamma, float* __restrict__ s, float* __restrict__ r) {
  const int j = blockIdx.x * kMomThreads + threadIdx.x;
  if (j >= nO) return;
  const int o = O[j];
  if (o < 0 || o >= K) return;
  float c = 0.0f;
  for (int b = 0; b < rblocks; ++b) c = fmaxf(c, part[static_cast<int64_t>(b) * nO + j]);
  float sn, rn;
  momentum_step(c, wmax[j], gamma, s[o], sn, rn);
  s[o] = sn;
  r[o] = rn;
}

// Momentum maxima for the quantizer's fold: workgroup (strip, b) takes the 64
// channels of a strip over the rows of block b of kMomFoldBlocks, 16 rows in
// flight per thread (one pass of 512 rows), and writes the maxima of the
// strip's outlier channels to part[b * nO + j]; block 0 also copies s[O[j]]
// to part[kMomFoldBlocks * nO + j] (the quantizer reads the old s there
// while its first workgroup writes the new one), writes r = 1 / s for the
// strip's other channels and the marker of slot j at r[O[j]] (nO <= 256).  As in momentum_kernel, every load is issued
// before the outlier bookkeeping, from clamped in-range addresses.
constexpr int kBlkThreads = 256;  // 8 lanes per row, 32 rows per load
constexpr int kBlkLoads = 16;
constexpr int kBlkRows = kBlkThreads / 8 * kBlkLoads;

__global__ __launch_bounds__(kBlkThreads) void momentum_block_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const int32_t* __restrict__ O, int nO,
    const float* __restrict__ s, float* __restrict__ r, int64_t rows, float* __restrict__ part) {
  __shared__ float red[kBlkThreads / 64][64];
  __shared__ int owner[64];  // 1 + index into O of the outlier at this channel, or 0
  const int64_t strip = blockIdx.x, rb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int o_raw = O[(tid < nO) ? tid : 0];
  const float s_k = s[strip * 64 + lane];
  const uint16_t* const col = x + strip * 64 + (tid & 7) * 8;
  // Rows past the block (or the batch) repeat its last row, or row 0 for a
  // block past the batch: in range, and the maximum over all blocks is
  // unchanged.
  const int64_t m_lo = rb * rows, m_hi = (m_lo + rows < M) ? m_lo + rows : M;
  const int64_t last = (m_hi > m_lo) ? m_hi - 1 : 0;
  v4i v[kBlkLoads];
  auto load_rows = [&](int64_t mb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kBlkLoads; ++i) {
      int64_t m = mb + (tid >> 3) + static_cast<int64_t>(kBlkThreads / 8) * i;
      m = m < m_hi ? m : last;
      v[i] = *reinterpret_cast<const v4i*>(col + m * K);
    }
  };
  float cm[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};  // channels 8*(tid&7) + [0, 8)
  auto fold_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kBlkLoads; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t u = static_cast<uint32_t>(v[i][w]);
        cm[2 * w] = fmaxf(cm[2 * w], fabsf(h2f(static_cast<uint16_t>(u & 0xffffu))));
        cm[2 * w + 1] = fmaxf(cm[2 * w + 1], fabsf(h2f(static_cast<uint16_t>(u >> 16))));
      }
  };
  load_rows(m_lo);
  if (tid < 64) owner[tid] = 0;
  __syncthreads();
  const int o0 = (tid < nO) ? o_raw : -1;
  if (o0 >= 0 && o0 < K && o0 / 64 == strip) owner[o0 % 64] = tid + 1;
  for (int j = tid + kBlkThreads; j < nO; j += kBlkThreads) {
    const int o = O[j];
    if (o >= 0 && o < K && o / 64 == strip) owner[o % 64] = j + 1;
  }
  __syncthreads();
  fold_rows();
  for (int64_t mb = m_lo + kBlkRows; mb < m_hi; mb += kBlkRows) {
    load_rows(mb);
    __builtin_amdgcn_sched_barrier(0);  // all of a pass's loads before any use
    fold_rows();
  }
  // Lanes with equal (lane & 7) hold the same channels: combine over lane bits 3..5.
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float t = cm[c];
    t = fmaxf(t, __shfl_xor(t, 8));
    t = fmaxf(t, __shfl_xor(t, 16));
    t = fmaxf(t, __shfl_xor(t, 32));
    cm[c] = t;
  }
  if (lane < 8) {
#pragma unroll
    for (int c = 0; c < 8; ++c) red[wave][lane * 8 + c] = cm[c];
  }
  __syncthreads();
  if (tid < 64) {
    const int own = owner[tid];
    if (own != 0) {
      float c = 0.0f;
#pragma unroll
      for (int w = 0; w < kBlkThreads / 64; ++w) c = fmaxf(c, red[w][tid]);
      part[rb * nO + own - 1] = c;
      if (rb == 0) {
        part[static_cast<int64_t>(kMomFoldBlocks) * nO + own - 1] = s_k;
        r[strip * 64 + tid] = mom_slot_marker(own - 1);
      }
    } else if (rb == 0) {
      r[strip * 64 + tid] = div_rn(1.0f, s_k);
    }
  }
}

// The two-launch form is used from kWorkMinRows tokens: below, one workgroup
// per strip reads its strip at the rate of one CU in about the time of the
// second launch (measured at 4096 x 4096: 11.7 us for either form; at 8192,
// 22.4 against 18.9 us; at 32768, 75.7 against 48.8 us).
constexpr int64_t kWorkMinRows = 4096;

// Row blocks of the two-launch update: 128 rows per block at least, at most
// kMaxRowBlocks blocks.
int64_t momentum_row_blocks(int64_t M) {
  int64_t rb = (M + kPartRows - 1) / kPartRows;
  rb = rb < 1 ? 1 : rb;
  return rb < kMaxRowBlocks ? rb : kMaxRowBlocks;
}

__global__ __launch_bounds__(kMomThreads) void row_absmax_kernel(const uint16_t* __restrict__ w,
                                                                 int64_t N, float* __restrict__ out) {
  __shared__ float red[kMomThreads / 64];
  const int64_t i = blockIdx.x;
  const uint16_t* row = w + i * N;
  float a = 0.0f;
  for (int64_t c = threadIdx.x; c < N / 8; c += kMomThreads) {
    const uint4 raw = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint32_t v[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a = fmaxf(a, fabsf(h2f(static_cast<uint16_t>(v[q] & 0xffffu))));
      a = fmaxf(a, fabsf(h2f(static_cast<uint16_t>(v[q] >> 16))));
    }
  }
  a = block_max<kMomThreads / 64>(a, red);
  if (threadIdx.x == 0) out[i] = a;
}

// Standalone compensation: y = fp16(y + sa * sum_j xO[m,j] * WO[j,n]) on
// 64 x 256 tiles, four waves of 64 x 64 (both operands arrive in fragment
// order), two workgroups per CU, so that one's products overlap the other's
// read-modify-write of y (128-row tiles, one per CU: 13.1 us at 2048 x 208
// x 4096; 64 rows: 12.1; 32 rows: 12.6).  The read-modify-write of y goes through the wave's own LDS rows,
// 32 x 64 at a time: whole 128-byte row pieces are read and written (eight
// lanes per row), and each lane works on its fragment's runs of four
// adjacent columns in between.
constexpr int kCompTM = 2, kCompThreads = 256;
constexpr int kCompPitch = 144;  // bytes per staged row: 128 + 16 spreads rows over the banks

__global__ __launch_bounds__(kCompThreads, 2) void outlier_comp_kernel(
    const uint16_t* __restrict__ xO, int ldO, const float* __restrict__ sa,
    const uint8_t* __restrict__ WOp, int64_t M, int64_t N, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t ylds[kCompThreads / 64][32 * kCompPitch];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * 32 * kCompTM;
  const int64_t wcol0 = static_cast<int64_t>(blockIdx.x) * 256 + 64 * wave;
  if (wcol0 >= N) return;
  v16f f[kCompTM][2];
#pragma unroll
  for (int a = 0; a < kCompTM; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) f[a][b] = v16f{};
  comp_accumulate<kCompTM, 2>(f, xO, ldO, WOp, M, N, m0, wcol0 / 32);
  uint8_t* const yl = ylds[wave];
  const int r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int tm = 0; tm < kCompTM; ++tm) {
    // Rows past M: the clamped row is read and nothing is written back.
    v4i blk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 3) + 8 * i, chunk = lane & 7;
      int64_t mr = m0 + 32 * tm + row;
      mr = mr < M ? mr : M - 1;
      blk[i] = *reinterpret_cast<const v4i*>(y + mr * N + wcol0 + 8 * chunk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 3) + 8 * i, chunk = lane & 7;
      *reinterpret_cast<v4i*>(yl + row * kCompPitch + chunk * 16) = blk[i];
    }
    // One wave's LDS operations complete in order: a compiler fence suffices.
    asm volatile("" ::: "memory");
    int64_t mc = m0 + 32 * tm + r;
    mc = mc < M ? mc : M - 1;
    const float sam = sa[mc];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint2* p = reinterpret_cast<uint2*>(yl + r * kCompPitch + (32 * nt + 8 * q + 4 * h) * 2);
        const uint2 old = *p;
        const uint16_t in[4] = {static_cast<uint16_t>(old.x & 0xffffu), static_cast<uint16_t>(old.x >> 16),
                                static_cast<uint16_t>(old.y & 0xffffu), static_cast<uint16_t>(old.y >> 16)};
        uint16_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = f2h(h2f(in[j]) + sam * f[tm][nt][4 * q + j]);
        *p = make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (lane >> 3) + 8 * i, chunk = lane & 7;
      const int64_t mr = m0 + 32 * tm + row;
      const v4i d = *reinterpret_cast<const v4i*>(yl + row * kCompPitch + chunk * 16);
      if (mr < M) *reinterpret_cast<v4i*>(y + mr * N + wcol0 + 8 * chunk) = d;
    }
    asm volatile("" ::: "memory");
  }
}

// STE backward, compensation part: cb[m, j] = sum_n dy[m, n] * w_o[j, n] in
// fp32 (fp16 products on the matrix cores) for j < nO, zero for
// nO <= j < ldO.  A small product (N long, ldO narrow) bound by moving the
// operands from L2 into the compute units: a workgroup takes 32 rows and
// kGradCB column blocks of 32, its kGradWaves waves take the 64-wide blocks
// of n in turn (wave w: blocks w, w + kGradWaves, ...).  A wave moves each
// block through its own LDS region: coalesced 16-byte loads (eight lanes per
// 128-byte row piece, kGradD blocks in flight), then reads in the fragment
// order of v_mfma_f32_32x32x16_f16 (lane: row l & 31, 8 consecutive n from
// 8 (l >> 5) on).  Each row's eight 16-byte chunks sit permuted by the xor
// with grad_swz(row), so that 16 lanes reading one chunk of 16 consecutive
// rows touch all 64 banks once (8 lanes of an aligned half: 32 distinct
// banks).  The waves' sums meet in LDS in a fixed pairing order (w and
// w + 4, then w and w + 2, then 0 and 1): the result does not depend on
// timing.
constexpr int kGradCB = 2, kGradWaves = 8, kGradThreads = 64 * kGradWaves, kGradD = 2;
constexpr int kGradBW = 64;                      // n per block
constexpr int kGradCPR = kGradBW / 8;            // 16-byte chunks per row
constexpr int kGradRPL = 64 / kGradCPR;          // rows per load
constexpr int kGradRows = 32 * (1 + kGradCB);    // staged rows per block: dy, then w_o
constexpr int kGradLoads = kGradRows / kGradRPL;

__device__ __forceinline__ int grad_swz(int row) { return ((row >> 1) & 3) | (((row ^ (row >> 3)) & 1) << 2); }
__device__ __forceinline__ int grad_slot(int row, int chunk) { return kGradCPR * row + (chunk ^ grad_swz(row)); }

// One wave's sweep over its blocks k = 0 .. cnt - 1 (block wave + kGradWaves k
// of n) with the first NB column blocks live.  The loop body stores block k
// from registers into LDS, refills those registers with block k + kGradD and
// multiplies block k; the steady-state loop has no branch, so that the
// compiler's load counting waits only for the block being stored.
template <int NB>
__device__ __forceinline__ void grad_sweep(const uint16_t* const* src, const int* dst, v4i* lds, int wave,
                                           int cnt, int nblk, int lane, v16f* acc) {
  constexpr int L = (32 / kGradRPL) * (1 + NB);  // loads per block: dy rows, then the live w_o rows
  v4i reg[kGradD][L];
  auto issue = [&](int k, v4i* r) {
    int blk = wave + kGradWaves * k;
    blk = blk < nblk ? blk : nblk - 1;  // the first kGradD loads of a short sweep
    const int64_t off = kGradBW * static_cast<int64_t>(blk);
#pragma unroll
    for (int t = 0; t < L; ++t) r[t] = *reinterpret_cast<const v4i*>(src[t] + off);
  };
  const int rrow = lane & 31, rchunk = lane >> 5;
  auto step = [&](v4i* r, bool refill, int next) {
#pragma unroll
    for (int t = 0; t < L; ++t) lds[dst[t]] = r[t];
    if (refill) issue(next, r);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int st = 0; st < kGradBW / 16; ++st) {
      const v8h a = __builtin_bit_cast(v8h, lds[grad_slot(rrow, 2 * st + rchunk)]);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const v8h bv = __builtin_bit_cast(v8h, lds[grad_slot(32 + 32 * b + rrow, 2 * st + rchunk)]);
        acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bv, acc[b], 0, 0, 0);
      }
    }
    // The next block's stores to this region come after these reads.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Unconditional, so that the loop's load counting starts from one state.
#pragma unroll
  for (int d = 0; d < kGradD; ++d) issue(d, reg[d]);
  int k0 = 0;
  for (; k0 + 2 * kGradD <= cnt; k0 += kGradD) {
#pragma unroll
    for (int d = 0; d < kGradD; ++d) step(reg[d], true, k0 + d + kGradD);
  }
  // Fewer than 2 kGradD blocks remain.
#pragma unroll
  for (int d = 0; d < kGradD; ++d) {
    if (k0 + d < cnt) {
      if (k0 + d + kGradD < cnt) step(reg[d], true, k0 + d + kGradD);
      else step(reg[d], false, 0);
    }
  }
#pragma unroll
  for (int d = 0; d < kGradD; ++d)
    if (k0 + kGradD + d < cnt) step(reg[d], false, 0);
}

__global__ __launch_bounds__(kGradThreads) void outlier_grad_kernel(const uint16_t* __restrict__ dy,
                                                                   const uint16_t* __restrict__ w_o, int64_t M,
                                                                   int64_t N, int nO, int ldO,
                                                                   float* __restrict__ cb) {
  static_assert(kGradCB == 2, "the sweep is instantiated for one or two live column blocks");
  __shared__ v4i stage[kGradWaves][kGradCPR * kGradRows];
  __shared__ float red[kGradWaves / 2][kGradCB][16][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 32;
  const int jb0 = blockIdx.y * kGradCB;
  // Load t brings rows kGradRPL t .. kGradRPL (t + 1) - 1 of the block: lane l
  // takes row kGradRPL t + l / kGradCPR, chunk l % kGradCPR.  Rows past M
  // repeat row M - 1, columns past nO repeat row nO - 1 (their sums are
  // dropped at the store); a column block wholly past nO is neither loaded
  // nor multiplied.
  const uint16_t* src[kGradLoads];
  int dst[kGradLoads];
#pragma unroll
  for (int t = 0; t < kGradLoads; ++t) {
    const int row = kGradRPL * t + lane / kGradCPR, chunk = lane % kGradCPR;
    if (row < 32) {
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      src[t] = dy + m * N + 8 * chunk;
    } else {
      int j = 32 * jb0 + row - 32;
      j = j < nO ? j : nO - 1;
      src[t] = w_o + static_cast<int64_t>(j) * N + 8 * chunk;
    }
    dst[t] = grad_slot(row, chunk);
  }
  const int nblk = static_cast<int>(N / kGradBW);
  const int cnt = nblk > wave ? (nblk - wave + kGradWaves - 1) / kGradWaves : 0;
  v16f acc[kGradCB];
#pragma unroll
  for (int b = 0; b < kGradCB; ++b) acc[b] = v16f{};
  if (32 * (jb0 + 1) < nO) grad_sweep<2>(src, dst, stage[wave], wave, cnt, nblk, lane, acc);
  else grad_sweep<1>(src, dst, stage[wave], wave, cnt, nblk, lane, acc);
  // Pairwise reduction over the waves in a fixed order.
#pragma unroll
  for (int span = kGradWaves / 2; span >= 1; span /= 2) {
    if (wave >= span && wave < 2 * span) {
#pragma unroll
      for (int b = 0; b < kGradCB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wave - span][b][v][lane] = acc[b][v];
    }
    __syncthreads();
    if (wave < span) {
#pragma unroll
      for (int b = 0; b < kGradCB; ++b)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][v] += red[wave][b][v][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // Lane l holds column (l & 31) and rows frag_row(v, l) of each block.
#pragma unroll
  for (int b = 0; b < kGradCB; ++b) {
    const int j = 32 * (jb0 + b) + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t row = m0 + frag_row(v, lane);
      if (j < ldO && row < M) cb[row * ldO + j] = j < nO ? acc[b][v] : 0.0f;
    }
  }
}

// Partial maxima of the allocation-free momentum update: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code reaches
// it only through the address hipGetSymbolAddress gives for each device.
constexpr int kScratchOutliers = 8192;
constexpr int64_t kScratchFloats = static_cast<int64_t>(kMaxRowBlocks) * kScratchOutliers;
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
float* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The device address of `scratch` on the device of `st` (looked up once per
// device, with that device current).
qlin_status scratch_on(hipStream_t st, float** out) {
  int dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return fail(QLIN_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(QLIN_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev, kMaxDevices - 1);
  std::call_once(g_scratch_once[dev], [dev]() {
    int cur = -1;
    hipError_t err = hipGetDevice(&cur);
    if (err == hipSuccess && cur != dev) err = hipSetDevice(dev);
    void* p = nullptr;
    if (err == hipSuccess) err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (err == hipSuccess) err = back;
    }
    g_scratch_err[dev] = err;
    g_scratch[dev] = static_cast<float*>(p);
  });
  if (g_scratch_err[dev] != hipSuccess)
    return fail(QLIN_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch[dev];
  return QLIN_OK;
}

qlin_status launch_momentum(const uint16_t* x, int64_t M, int64_t K, const int32_t* O, int32_t nO,
                            const float* wmax_O, float gamma, float* s, float* r, float* work, hipStream_t st) {
  if (work == nullptr || M < kWorkMinRows) {
    momentum_kernel<<<dim3(static_cast<unsigned>(K / 64)), kStripThreads, 0, st>>>(x, M, K, O, nO, wmax_O, gamma,
                                                                                   s, r);
    QLIN_LAUNCH_CHECK("momentum_kernel");
    return QLIN_OK;
  }
  const int64_t rb = momentum_row_blocks(M), rows = (M + rb - 1) / rb;
  momentum_partial_kernel<<<dim3(static_cast<unsigned>(K / 64), static_cast<unsigned>(rb)), kPartThreads, 0, st>>>(
      x, M, K, O, nO, s, r, rows, work);
  QLIN_LAUNCH_CHECK("momentum_partial_kernel");
  if (nO > 0) {
    momentum_fold_kernel<<<dim3(static_cast<unsigned>((nO + kMomThreads - 1) / kMomThreads)), kMomThreads, 0, st>>>(
        work, static_cast<int>(rb), K, O, nO, wmax_O, gamma, s, r);
    QLIN_LAUNCH_CHECK("momentum_fold_kernel");
  }
  return QLIN_OK;
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" size_t qlin_momentum_work_bytes(int64_t M, int32_t nO) {
  if (M < 0 || nO < 0) return 0;
  return static_cast<size_t>(momentum_row_blocks(M)) * static_cast<size_t>(nO) * sizeof(float);
}

extern "C" qlin_status qlin_momentum_update(const uint16_t* x, int64_t M, int64_t K,
                                            const int32_t* O, int32_t nO, const float* wmax_O,
                                            float gamma, float* s, float* r, float* work, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  QLIN_REQUIRE(gamma >= 0.0f && gamma <= 1.0f, QLIN_ERR_INVALID_ARG, "gamma=%g must be in [0, 1]", (double)gamma);
  QLIN_PTR(s);
  QLIN_PTR(r);
  QLIN_OPT_PTR(work);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_PTR(wmax_O);
    if (M > 0) QLIN_PTR(x);
  }
  QLIN_REQUIRE(K / 64 <= 0x7fffffffLL, QLIN_ERR_SHAPE, "K too large");
  return launch_momentum(x, M, K, O, nO, wmax_O, gamma, s, r, work, as_stream(stream));
}

extern "C" size_t qlin_quaff_momentum_quant_work_bytes(int64_t M, int32_t nO) {
  if (M < 0 || nO < 0) return 0;
  const size_t fused = static_cast<size_t>(kMomFoldBlocks + 1) * static_cast<size_t>(nO) * sizeof(float);
  const size_t two = qlin_momentum_work_bytes(M, nO);
  return fused > two ? fused : two;
}

extern "C" qlin_status qlin_quaff_momentum_quant(const uint16_t* x, int64_t M, int64_t K, const int32_t* O,
                                                 int32_t nO, const float* wmax_O, float gamma, float* s, float* r,
                                                 float* work, int8_t* q, float* scale, uint16_t* xO,
                                                 void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  QLIN_REQUIRE(gamma >= 0.0f && gamma <= 1.0f, QLIN_ERR_INVALID_ARG, "gamma=%g must be in [0, 1]", (double)gamma);
  QLIN_PTR(s);
  QLIN_PTR(r);
  QLIN_OPT_PTR(work);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_PTR(wmax_O);
    if (M > 0) QLIN_PTR(xO);
  } else {
    QLIN_REQUIRE(O == nullptr && xO == nullptr, QLIN_ERR_INVALID_ARG, "O and xO must be NULL when nO == 0");
  }
  if (M > 0) {
    QLIN_PTR(x);
    QLIN_PTR(q);
    QLIN_PTR(scale);
  }
  QLIN_REQUIRE(K / 64 <= 0x7fffffffLL && M / 2 < 0x7fffffffLL, QLIN_ERR_SHAPE, "M or K too large");
  // The folded form needs a workspace, the outlier slots of the quantizer's
  // LDS path and rows that fit its registers; otherwise the two calls it
  // stands for, which give the same result.
  const bool fold = work != nullptr && M > 0 && nO > 0 && outlier_ld(nO) <= 256 && K <= 8192;
  if (!fold) {
    const qlin_status st = qlin_momentum_update(x, M, K, O, nO, wmax_O, gamma, s, r, work, stream);
    if (st != QLIN_OK) return st;
    return qlin_quant_act(x, M, K, r, q, scale, O, nO, s, nullptr, xO, stream);
  }
  hipStream_t st = as_stream(stream);
  const int64_t rows = (M + kMomFoldBlocks - 1) / kMomFoldBlocks;
  momentum_block_kernel<<<dim3(static_cast<unsigned>(K / 64), kMomFoldBlocks), kBlkThreads, 0, st>>>(
      x, M, K, O, nO, s, r, rows, work);
  QLIN_LAUNCH_CHECK("momentum_block_kernel");
  return launch_quant_momentum(x, M, K, r, q, scale, O, nO, xO, MomFold{work, wmax_O, gamma, s, r}, st);
}

extern "C" qlin_status qlin_momentum_update_noalloc(const uint16_t* x, int64_t M, int64_t K, const int32_t* O,
                                                    int32_t nO, const float* wmax_O, float gamma, float* s,
                                                    float* r, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  QLIN_REQUIRE(nO <= kScratchOutliers, QLIN_ERR_SHAPE,
               "nO=%d: the static scratch holds partial maxima for at most %d outlier channels", nO,
               kScratchOutliers);
  QLIN_REQUIRE(gamma >= 0.0f && gamma <= 1.0f, QLIN_ERR_INVALID_ARG, "gamma=%g must be in [0, 1]", (double)gamma);
  QLIN_PTR(s);
  QLIN_PTR(r);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_PTR(wmax_O);
    if (M > 0) QLIN_PTR(x);
  }
  QLIN_REQUIRE(K / 64 <= 0x7fffffffLL, QLIN_ERR_SHAPE, "K too large");
  float* work = nullptr;
  const qlin_status st = scratch_on(as_stream(stream), &work);
  if (st != QLIN_OK) return st;
  return launch_momentum(x, M, K, O, nO, wmax_O, gamma, s, r, work, as_stream(stream));
}

extern "C" qlin_status qlin_weight_row_absmax(const uint16_t* w_rows, int64_t R, int64_t N,
                                              float* out, void* stream) {
  QLIN_REQUIRE(R >= 0, QLIN_ERR_INVALID_ARG, "R=%lld is negative", (long long)R);
  QLIN_REQUIRE(N > 0 && N % 64 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 64", (long long)N);
  QLIN_DIMS(R, N);
  if (R == 0) return QLIN_OK;
  QLIN_PTR(w_rows);
  QLIN_PTR(out);
  QLIN_REQUIRE(R <= 0x7fffffffLL, QLIN_ERR_SHAPE, "R too large");
  row_absmax_kernel<<<dim3(static_cast<unsigned>(R)), kMomThreads, 0, as_stream(stream)>>>(w_rows, N, out);
  QLIN_LAUNCH_CHECK("row_absmax_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_outlier_comp(const uint16_t* xO, const float* sa, int32_t nO,
                                         const void* WO, int64_t M, int64_t N, uint16_t* y,
                                         void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(N > 0 && N % 64 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 64", (long long)N);
  QLIN_DIMS(M, N);
  QLIN_REQUIRE(nO >= 0, QLIN_ERR_INVALID_ARG, "nO=%d is negative", nO);
  if (M == 0 || nO == 0) return QLIN_OK;
  QLIN_PTR(xO);
  QLIN_PTR(sa);
  QLIN_PTR(WO);
  QLIN_PTR(y);
  const int64_t gy = (M + 32 * kCompTM - 1) / (32 * kCompTM);
  QLIN_REQUIRE(gy <= 65535, QLIN_ERR_SHAPE, "M too large");
  const dim3 grid(static_cast<unsigned>((N + 255) / 256), static_cast<unsigned>(gy));
  outlier_comp_kernel<<<grid, kCompThreads, 0, as_stream(stream)>>>(
      xO, static_cast<int>(outlier_ld(nO)), sa, static_cast<const uint8_t*>(WO), M, N, y);
  QLIN_LAUNCH_CHECK("outlier_comp_kernel");
  return QLIN_OK;
}

extern "C" qlin_status qlin_quaff_backward(const uint16_t* dy, int64_t M, int64_t N, int64_t K,
                                           const uint16_t* sw, const void* w8t, const float* s, const float* r,
                                           const int32_t* O, int32_t nO, const uint16_t* w_o, int8_t* gq,
                                           float* gs, float* cb, uint16_t* dx, int32_t* acc, void* stream) {
  QLIN_REQUIRE(M >= 0, QLIN_ERR_INVALID_ARG, "M=%lld is negative", (long long)M);
  QLIN_REQUIRE(K > 0 && K % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)K);
  QLIN_DIMS(M, K);
  QLIN_REQUIRE(N > 0 && N % 128 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 128", (long long)N);
  QLIN_DIMS(M, N);
  QLIN_DIMS(K, N);
  QLIN_REQUIRE(nO >= 0 && nO <= K, QLIN_ERR_SHAPE, "nO=%d must be in [0, K]", nO);
  if (M == 0) return QLIN_OK;
  QLIN_PTR(dy);
  QLIN_PTR(sw);
  QLIN_PTR(w8t);
  QLIN_PTR(s);
  QLIN_PTR(r);
  QLIN_PTR(gq);
  QLIN_PTR(gs);
  QLIN_PTR(dx);
  QLIN_OPT_PTR(acc);
  if (nO > 0) {
    QLIN_PTR(O);
    QLIN_PTR(w_o);
    QLIN_PTR(cb);
  } else {
    QLIN_REQUIRE(O == nullptr && w_o == nullptr && cb == nullptr, QLIN_ERR_INVALID_ARG,
                 "O, w_o and cb must be NULL when nO == 0");
  }
  const int64_t gx = (M + 31) / 32;
  QLIN_REQUIRE(gx <= 0x7fffffffLL, QLIN_ERR_SHAPE, "M too large");
  hipStream_t st = as_stream(stream);
  qlin_status rc = launch_quant_grad(dy, M, N, sw, gq, gs, st);
  if (rc != QLIN_OK) return rc;
  if (nO > 0) {
    const int ldO = static_cast<int>(outlier_ld(nO));
    const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>((ldO + 32 * kGradCB - 1) / (32 * kGradCB)));
    outlier_grad_kernel<<<grid, kGradThreads, 0, st>>>(dy, w_o, M, N, nO, ldO, cb);
    QLIN_LAUNCH_CHECK("outlier_grad_kernel");
  }
  return launch_gemm_bwd(gq, gs, w8t, r, s, O, nO, cb, M, N, K, dx, acc, st);
}
