// ssd_decode_step: one recurrent token step of the order-p mixer, in place.
//
// 2Mamba2Furious, Algorithm 6 (2Mamba inference): with phi(x) = x (order 1)
// or vec(x x^T) (order 2, D = d_h^2),
//     H_up   <- alpha H_up   + phi(k) (v dt)^T        [D x d_h]
//     H_down <- alpha H_down + phi(k)                 [D]
//     y       = phi(q)^T H_up / phi(q)^T H_down       (states after the update)
// with the Mamba-2 discretisation of Algorithm 3: dt = softplus(dt_P +
// dt_bias), alpha = exp(A dt), A = -exp(A_log).
//
// The step is pure streaming: every state element is read once and written
// once (order 2, d_h 64: 1 MiB + 16 KiB per sequence and head), so the
// kernel is HBM-bound.  One workgroup per (sequence, head) -- 1024 threads for
// the large order-2 states, 256 for the small ones; each thread owns one
// 16-byte column group of the state rows it visits, keeps several row loads
// in flight (non-temporal: the state has no reuse within a step), fuses the
// update with the output contraction, and the partial outputs are reduced
// across lanes and waves at the end.  (A sweep of rows in flight x workgroup
// size on the 256 x 32-head, d_h 64 order-2 step favoured 4 rows x 1024
// threads: 71.5% of the HBM peak against 67.6% for 8 rows x 256 threads.)
#include "common.h"
#include "launch.h"

namespace ssd {

template <typename St, int DH, int ORDER, int NTH>
__global__ __launch_bounds__(NTH) void k_decode(const St* __restrict__ q, const St* __restrict__ k,
                                                const St* __restrict__ v,
                                                const float* __restrict__ dt_proj,
                                                const float* __restrict__ dt_bias,
                                                const float* __restrict__ A_log, int64_t H,
                                                float* __restrict__ state,
                                                float* __restrict__ norm, float* __restrict__ y) {
  constexpr int D = ORDER == 1 ? DH : DH * DH;
  constexpr int CG = DH / 4;         // 16-byte column groups per state row
  constexpr int RPP = NTH / CG;      // rows per pass of the workgroup
  constexpr int UMAX = NTH >= 1024 ? 4 : 8;
  constexpr int U = (D / RPP) < UMAX ? (D / RPP) : UMAX;  // rows in flight per thread
  constexpr int NWV = NTH / WAVE;
  static_assert(U >= 1, "workgroup too large for the state");
  static_assert(D % (RPP * U) == 0, "row loop must tile the state");
  __shared__ float qs[DH], ks[DH], vs[DH];
  __shared__ f32x4 red4[NWV][WAVE];
  __shared__ float redd[NWV];

  const int64_t sh = blockIdx.x;
  const int64_t h = sh % H;
  const int tid = threadIdx.x;
  const float dtv = softplus_f(dt_proj[sh] + dt_bias[h]);
  const float alpha = expf(-expf(A_log[h]) * dtv);
  if (tid < DH) {
    qs[tid] = Elem<St>::ld(q, sh * DH + tid);
    ks[tid] = Elem<St>::ld(k, sh * DH + tid);
    vs[tid] = Elem<St>::ld(v, sh * DH + tid) * dtv;
  }
  __syncthreads();

  const int cg = tid % CG, r0 = tid / CG;
  const f32x4 vd = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
  f32x4 acc = zero4();
  float* Sp = state + sh * (int64_t)D * DH + 4 * cg;
  for (int rb = r0; rb < D; rb += RPP * U) {
    f32x4 s[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + (int64_t)(rb + u * RPP) * DH));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rw = rb + u * RPP;
      float fk, fq;
      if (ORDER == 1) {
        fk = ks[rw];
        fq = qs[rw];
      } else {
        const int a = rw / DH, b = rw - (rw / DH) * DH;
        fk = ks[a] * ks[b];
        fq = qs[a] * qs[b];
      }
      const f32x4 ns = alpha * s[u] + fk * vd;
      __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(Sp + (int64_t)rw * DH));
      acc += fq * ns;
    }
  }
  float dacc = 0.f;
  float* zp = norm + sh * (int64_t)D;
  for (int e = tid; e < D; e += NTH) {
    float fk, fq;
    if (ORDER == 1) {
      fk = ks[e];
      fq = qs[e];
    } else {
      const int a = e / DH, b = e - (e / DH) * DH;
      fk = ks[a] * ks[b];
      fq = qs[a] * qs[b];
    }
    const float nz = alpha * zp[e] + fk;
    zp[e] = nz;
    dacc += fq * nz;
  }
  // reduce acc over threads sharing a column group: within the wave first
  const int lane = tid & (WAVE - 1), wave = tid / WAVE;
#pragma unroll
  for (int off = CG; off < WAVE; off <<= 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], off, WAVE);
  }
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) dacc += __shfl_xor(dacc, off, WAVE);
  red4[wave][lane] = acc;
  if (lane == 0) redd[wave] = dacc;
  __syncthreads();
  if (tid < CG) {
    f32x4 t = red4[0][tid];
    float den = redd[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
      t += red4[w][tid];
      den += redd[w];
    }
    f32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = t[r] / den;
    *reinterpret_cast<f32x4*>(y + sh * DH + 4 * tid) = o;
  }
}

hipError_t launch_decode(bool bf16, int64_t DH, int order, const void* q, const void* k,
                         const void* v, const float* dt_proj, const float* dt_bias,
                         const float* A_log, int64_t S, int64_t H, float* state, float* norm_state,
                         float* y, hipStream_t stream) {
  const dim3 grid((unsigned)(S * H));
  // order-2 states stream with 1024-thread workgroups, order-1 with 256
#define SSD_LAUNCH_DEC(ST, DHV, ORD)                                                             \
  hipLaunchKernelGGL((k_decode<ST, DHV, ORD, ORD == 2 ? 1024 : 256>), grid,                    \
                     dim3(ORD == 2 ? 1024 : 256), 0, stream, static_cast<const ST*>(q),         \
                     static_cast<const ST*>(k), static_cast<const ST*>(v), dt_proj, dt_bias,   \
                     A_log, H, state, norm_state, y)
  if (bf16) {
    if (DH == 64) {
      if (order == 2) SSD_LAUNCH_DEC(uint16_t, 64, 2);
      else SSD_LAUNCH_DEC(uint16_t, 64, 1);
    } else {
      if (order == 2) SSD_LAUNCH_DEC(uint16_t, 32, 2);
      else SSD_LAUNCH_DEC(uint16_t, 32, 1);
    }
  } else {
    if (DH == 64) {
      if (order == 2) SSD_LAUNCH_DEC(float, 64, 2);
      else SSD_LAUNCH_DEC(float, 64, 1);
    } else {
      if (order == 2) SSD_LAUNCH_DEC(float, 32, 2);
      else SSD_LAUNCH_DEC(float, 32, 1);
    }
  }
#undef SSD_LAUNCH_DEC
  return hipGetLastError();
}

}  // namespace ssd
