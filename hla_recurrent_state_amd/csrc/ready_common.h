// Device helpers shared by the gfx950 kernels of the state reader: bf16
// widening and round-to-nearest-even narrowing, 16-byte vector unpacking,
// wave reductions, the MLP activations and the MFMA operand types.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ready_internal.h"

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// D += A * B on one 16 x 16 output block with K = 32 (bf16 in, fp32 out).
// Lane l holds A[l % 16][8 (l / 16) .. + 7], B[8 (l / 16) .. + 7][l % 16] and
// D[4 (l / 16) .. + 3][l % 16].
__device__ __forceinline__ f32x4 mfma16x16x32(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even; NaN stays a NaN.  The conversion is
// gfx950's v_cvt_pk_bf16_f32 (what a __bf16 conversion compiles to), which
// agrees with rounding the fp32 bit pattern to nearest even on every one of
// the 2^32 inputs (checked exhaustively on the GPU; NaN inputs give NaN) and
// converts two values per instruction, with no branch.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two values, the first in the low half
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VW = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float ld(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static __forceinline__ void st(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
  __device__ static __forceinline__ void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int VW = 8;
  __device__ static __forceinline__ float ld(const void* p, int64_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
  __device__ static __forceinline__ void st(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = f32_to_bf16_rne(v); }
  __device__ static __forceinline__ void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xffff0000u);
    o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xffff0000u);
  }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ float activation(float x, int act) {
  if (act == READY_ACT_SILU) return x / (1.0f + expf(-x));
  if (act == READY_ACT_GELU_TANH) {
    const float c = 0.7978845608028654f;  // sqrt(2 / pi)
    return 0.5f * x * (1.0f + tanhf(c * (x + 0.044715f * x * x * x)));
  }
  return fmaxf(x, 0.0f);
}


// Pack 8 fp32 values into 8 bf16 (round to nearest even), element 0 in the
// low half of the first word.
__device__ __forceinline__ u32x4 pack_bf16x8(const float* x) {
  u32x4 v;
  v.x = f32x2_to_bf16x2_rne(x[0], x[1]);
  v.y = f32x2_to_bf16x2_rne(x[2], x[3]);
  v.z = f32x2_to_bf16x2_rne(x[4], x[5]);
  v.w = f32x2_to_bf16x2_rne(x[6], x[7]);
  return v;
}

// Sum of squares of the 8 bf16 values of a 16-byte chunk.
__device__ __forceinline__ float sumsq_bf16x8(const u32x4& v) {
  float x[8];
  Elem<uint16_t>::unpack(v, x);
  float s = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) s += x[e] * x[e];
  return s;
}

// The hardware hands workgroup i to XCD i % 8, and each XCD has its own L2.
// With a grid of 8 * per blocks, this gives each XCD the contiguous work
// items [xcd * per, xcd * per + per), so items that share operands (numbered
// next to each other by the caller) meet in one L2.  Returns -1 for the
// padding blocks past `total`.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks, int total) {
  const int per = nblocks >> 3;
  const int q = (bid & 7) * per + (bid >> 3);
  return q < total ? q : -1;
}

// Launch on `s`; with stage events the start and stop of the kernel itself
// are recorded by the dispatch.
#define READY_LAUNCH(kern, grid, block, lds, s, ev, ...)                                         \
  do {                                                                                           \
    if ((ev).start || (ev).stop)                                                                 \
      hipExtLaunchKernelGGL(kern, grid, block, lds, s, (ev).start, (ev).stop, 0u, __VA_ARGS__); \
    else                                                                                         \
      hipLaunchKernelGGL(kern, grid, block, lds, s, __VA_ARGS__);                                \
  } while (0)
