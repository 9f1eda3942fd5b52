// Shared host and device helpers of libqlin (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlin.h"

namespace qlin {

// ---------------------------------------------------------------- host side
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
qlin_status fail(qlin_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Maps the last HIP launch error to QLIN_ERR_HIP.
qlin_status launch_status(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validation helpers: return a status from the enclosing entry point.
#define QLIN_REQUIRE(cond, code, ...)                 \
  do {                                                \
    if (!(cond)) return ::qlin::fail((code), __VA_ARGS__); \
  } while (0)

#define QLIN_PTR(p)                                                                  \
  do {                                                                               \
    QLIN_REQUIRE((p) != nullptr, QLIN_ERR_INVALID_ARG, "%s: null pointer", #p);      \
    QLIN_REQUIRE(::qlin::aligned16(p), QLIN_ERR_ALIGN, "%s: not 16-byte aligned", #p); \
  } while (0)

#define QLIN_OPT_PTR(p)                                                              \
  do {                                                                               \
    QLIN_REQUIRE((p) == nullptr || ::qlin::aligned16(p), QLIN_ERR_ALIGN,             \
                 "%s: not 16-byte aligned", #p);                                     \
  } while (0)

#define QLIN_K_N(K, N)                                                                       \
  do {                                                                                       \
    QLIN_REQUIRE((K) > 0 && (K) % 128 == 0, QLIN_ERR_SHAPE, "K=%lld must be a positive multiple of 128", (long long)(K)); \
    QLIN_REQUIRE((N) > 0 && (N) % 64 == 0, QLIN_ERR_SHAPE, "N=%lld must be a positive multiple of 64", (long long)(N));   \
  } while (0)

// Size limits of every entry point: each dimension below 2^31 and each
// matrix operand at most 2^40 elements (far beyond device memory), so that no
// size, byte count, grid or index computed on the host or in a kernel
// overflows 64 bits.
constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr int64_t kMaxElems = int64_t(1) << 40;
inline bool dims_ok(int64_t a, int64_t b) {
  return a >= 0 && b >= 0 && a < kMaxDim && b < kMaxDim && a * b <= kMaxElems;
}

#define QLIN_DIMS(a, b)                                                                                  \
  QLIN_REQUIRE(::qlin::dims_ok((a), (b)), QLIN_ERR_SHAPE,                                                \
               "%s x %s = %lld x %lld: each dimension must be below 2^31 and their product at most 2^40", \
               #a, #b, (long long)(a), (long long)(b))

#define QLIN_LAUNCH_CHECK(what)                  \
  do {                                           \
    qlin_status st_ = ::qlin::launch_status(what); \
    if (st_ != QLIN_OK) return st_;              \
  } while (0)

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- device side
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Row of register v of a 32 x 32 matrix-core accumulator fragment in lane l
// (the column is l & 31).
__device__ __forceinline__ int frag_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ __forceinline__ float h2f(uint16_t b) {
  return static_cast<float>(__builtin_bit_cast(_Float16, b));
}
__device__ __forceinline__ uint16_t f2h(float f) {  // round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// fp16 of the fp32 product a * b: rounded to fp32, then to fp16, as written.
// Left alone, the compiler turns the product and the conversion into one
// mixed-precision fma with a +0 addend, whatever the contraction setting,
// which (at least) turns a -0 product into +0; the empty asm keeps the
// product in a register of its own.
__device__ __forceinline__ uint16_t f2h_mul(float a, float b) {
  float p = __fmul_rn(a, b);
  asm volatile("" : "+v"(p));
  return f2h(p);
}

// IEEE single-precision operations with one rounding each (never contracted).
__device__ __forceinline__ float mul_rn(float a, float b) { return __fmul_rn(a, b); }
__device__ __forceinline__ float add_rn(float a, float b) { return __fadd_rn(a, b); }
__device__ __forceinline__ float sub_rn(float a, float b) { return __fsub_rn(a, b); }
__device__ __forceinline__ float div_rn(float a, float b) { return a / b; }
// HIP's __fsqrt_rn maps to the approximate native square root unless OCML's
// rounded operations are enabled; the sqrtf builtin is lowered to the
// correctly rounded sequence (v_sqrt_f32 plus residual checks of both
// neighbours), and '/' to the IEEE division sequence.
__device__ __forceinline__ float sqrt_rn(float a) { return __builtin_sqrtf(a); }
__device__ __forceinline__ float rint_f(float a) { return __builtin_rintf(a); }

// Quaff targeted momentum scaling for one outlier channel ("Quaff" paper
// notes, key design): c = max_m |x[m, o]|, wm = max_n |W[o, n]|,
// beta = max(1, sqrt(c / wm)) (1 when wm == 0), s' = gamma s + (1 - gamma) beta
// and r' = 1 / s', one rounding per operation.
__device__ __forceinline__ void momentum_step(float c, float wm, float gamma, float s, float& sn, float& rn) {
  float beta = 1.0f;
  if (wm != 0.0f) beta = fmaxf(1.0f, sqrt_rn(div_rn(c, wm)));
  const float g1 = sub_rn(1.0f, gamma);
  sn = add_rn(mul_rn(gamma, s), mul_rn(g1, beta));
  rn = div_rn(1.0f, sn);
}

// Workgroup barrier for LDS only: waits for this wave's LDS traffic, then for
// every wave of the group.  Outstanding global loads are not waited for
// (__syncthreads() waits for every memory operation of the wave first).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wavefront (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide reductions over `nwaves` waves through a small LDS array.
template <int NWAVES>
__device__ __forceinline__ float block_max(float v, float* lds) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) r = fmaxf(r, lds[i]);
  return r;
}
template <int NWAVES>
__device__ __forceinline__ float block_min(float v, float* lds) {
  v = wave_min(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < NWAVES; ++i) r = fminf(r, lds[i]);
  return r;
}
template <int NWAVES>
__device__ __forceinline__ int block_sum(int v, int* lds) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) lds[w] = v;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) r += lds[i];
  return r;
}

}  // namespace qlin
