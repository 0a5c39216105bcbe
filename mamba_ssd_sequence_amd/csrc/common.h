// Shared device helpers for the gfx950 (CDNA4) kernels of the SSD / 2Mamba
// sequence mixer: vector types, bf16 conversion, MFMA wrappers and the
// wave-level reductions.
//
// MFMA fragment conventions used throughout (wave64, 16x16 output tiles):
//   lane l, column n = l % 16, lane group g = l / 16 (0..3)
//   D/C (16x16 fp32, 4 values): D[4g + r][n], r = 0..3
//   bf16 16x16x32: A holds A[m = n][k in group g: 8 values]
//                  B holds B[k in group g: 8 values][n]
//   f32  16x16x4 : A holds A[m = n][k = g], B holds B[k = g][n]
// Only the pairing of k between A and B matters for a product, so the kernels
// choose the k order per lane group to match whatever layout the operand
// already has in registers (see the "permuted k" notes in each kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int BLK = 64;  // tokens per block in every forward kernel

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (compiles to v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ __bf16 f32_to_bf16(float x) { return (__bf16)x; }

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// x if c else 0, per component (a select of the whole struct would be
// lowered through memory)
__device__ __forceinline__ uint4 keep_if(bool c, const uint4& x) {
  return make_uint4(c ? x.x : 0u, c ? x.y : 0u, c ? x.z : 0u, c ? x.w : 0u);
}

// 2^x on the hardware exponential (v_exp_f32, about 1 ulp; results below the
// smallest normal flush to 0, which only ever happens for decays that are 0
// to fp32 accuracy anyway); with x = y log2(e) it gives e^y.
constexpr float LOG2E = 1.4426950408889634f;
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// softplus(x) = max(x, 0) + log1p(exp(-|x|)), written from its definition.
__device__ __forceinline__ float softplus_f(float x) {
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

// Sum across the four lane groups (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float sum_over_groups(float x) {
  x += __shfl_xor(x, 16, WAVE);
  x += __shfl_xor(x, 32, WAVE);
  return x;
}

// Loads of the q/k/v element type as fp32.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float ld(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
};

}  // namespace ssd
