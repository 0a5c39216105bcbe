// Internal launchers and workspace layout of the backward pass (bwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "launch.h"

namespace ssd {

// Backward workspace (float offsets), blocks of 64 tokens, E = D d_h + D with
// D = d_h^order:
//   tb   [BH, nblk]          block decay totals (order 1)
//   sst  [BH, nblk, E]       forward increments, then (in place) the state
//                            entering each block, S_c and z_c (recomputed)
//   gst  [BH, nblk, E]       R_c, r_c, then (in place) the gradient of the
//                            state leaving each block, G_{c+1} and g_{c+1}
//   dnum [BH, nblk, 64, d_h] dy / den;  dden [BH, nblk, 64]
//   btot [BH, nblk]          order 2: each block's total of the per-token
//                            terms of the decay gradient
struct BwdLayout {
  size_t tb, sst, gst, dnum, dden, btot, total_floats;
};

inline BwdLayout bwd_layout(int64_t BH, int64_t N, int64_t DH, int order) {
  const size_t nbk = (size_t)(BH * n_blocks(N));
  const size_t D = order == 1 ? (size_t)DH : (size_t)(DH * DH);
  const size_t E = D * (size_t)DH + D;
  auto up = [](size_t x) { return (x + 63) & ~(size_t)63; };
  BwdLayout L;
  size_t off = 0;
  L.tb = off;   off = up(off + nbk);
  L.sst = off;  off = up(off + nbk * E);
  L.gst = off;  off = up(off + nbk * E);
  L.dnum = off; off = up(off + nbk * 64 * (size_t)DH);
  L.dden = off; off = up(off + nbk * 64);
  L.btot = off; off = up(off + (order == 2 ? nbk : 0));
  L.total_floats = off;
  return L;
}

// Backward of the order-1 or order-2 mixer (order 2: bf16 inputs, d_h 64):
// gradients with respect to q, k, v, dt (through the value operand v dt) and
// the per-token log-decay a.  dt may be NULL (v is the value operand; ddt is
// then NULL too).
hipError_t launch_backward(int order, bool bf16, int64_t DH, const void* q, const void* k,
                           const void* v, const float* dt, const float* a_cs, const float* y,
                           const float* den, const float* dy, int64_t BH, int64_t N, int64_t chunk,
                           float* dq, float* dk, float* dv, float* ddt, float* da, float* ws,
                           hipStream_t stream);
hipError_t launch_backward_o1(bool bf16, int64_t DH, const void* q, const void* k, const void* v,
                              const float* dt, const float* a_cs, const float* y, const float* den,
                              const float* dy, int64_t BH, int64_t N, int64_t chunk, float* dq,
                              float* dk, float* dv, float* ddt, float* da, float* ws,
                              hipStream_t stream);

// Chain rule through Algorithm 3's discretisation (per-head sums in d_dt_bias
// and d_A_log); ddt may be NULL (no value-operand gradient).
hipError_t launch_prep_backward(const float* dt_proj, const float* dt_bias, const float* A_log,
                                const float* da, const float* ddt, int64_t B, int64_t H, int64_t N,
                                float* d_dt_proj, float* d_dt_bias, float* d_A_log,
                                hipStream_t stream);

// Chain rule through the A-mask: d_A_proj from da; d_dt_proj from ddt when
// dt_proj is given.
hipError_t launch_prep_amask_backward(const float* A_proj, const float* dt_proj, const float* da,
                                      const float* ddt, int64_t B, int64_t H, int64_t N,
                                      float* d_A_proj, float* d_dt_proj, hipStream_t stream);

}  // namespace ssd
