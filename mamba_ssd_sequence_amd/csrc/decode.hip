// ssd_decode_step / ssd_decode_step_amask: one recurrent token step of the
// order-p mixer, in place; ssd_state_pack / ssd_state_unpack: the two layouts
// of the order-2 state.
//
// 2Mamba2Furious, Algorithm 6 (2Mamba inference): with phi(x) = x (order 1)
// or vec(x x^T) (order 2, D = d_h^2),
//     H_up   <- alpha H_up   + phi(k) v_op^T          [D x d_h]
//     H_down <- alpha H_down + phi(k)                 [D]
//     y       = phi(q)^T H_up / phi(q)^T H_down       (states after the update)
// with either the Mamba-2 discretisation of Algorithm 3 (dt = softplus(dt_P +
// dt_bias), alpha = exp(A dt), A = -exp(A_log), v_op = v dt) or the A-mask
// Algorithm 6 prints (alpha = exp(-softplus(h W_A)); v_op = v softplus(dt_P)
// as in Algorithm 4, or plain v).
//
// Packed order-2 layout: k (x) k is symmetric in its two indices, so state
// rows (a, b) and (b, a) are equal; the packed layout stores the rows a <= b
// only (D' = d_h (d_h + 1) / 2, row-major over the upper triangle: row
// a d_h - a (a - 1) / 2 + b - a) and the query side counts the off-diagonal
// rows twice.  Same state, about half the bytes.
//
// The step is pure streaming: every state element is read once and written
// once (order 2, d_h 64: 1 MiB + 16 KiB per sequence and head, 520 KiB
// packed), so the kernel is HBM-bound.  One workgroup per (sequence, head);
// the per-row features phi(k)_r and (weighted) phi(q)_r are tabulated in LDS
// first; each thread owns one 16-byte column group of the state rows it
// visits, keeps several row loads in flight (non-temporal: the state has no
// reuse within a step), fuses the update with the output contraction, and the
// partial outputs are reduced across lanes and waves at the end.  Workgroup
// size and rows in flight per layout: see launch_decode.  (Issuing the first
// row loads before the set-up, to hide it, was measured slower.)
#include "common.h"
#include "launch.h"

namespace ssd {

// number of state rows of one (sequence, head)
template <int DH, int ORDER, bool PACKED>
struct Rows {
  static constexpr int value = ORDER == 1 ? DH : (PACKED ? DH * (DH + 1) / 2 : DH * DH);
};

__device__ __forceinline__ int packed_row(int a, int b, int dh) {
  return a * dh - a * (a - 1) / 2 + (b - a);
}

template <typename St, int DH, int ORDER, int NTH, int UR, bool PACKED>
__global__ __launch_bounds__(NTH) void k_decode(const St* __restrict__ q, const St* __restrict__ k,
                                                const St* __restrict__ v,
                                                const float* __restrict__ dt_proj,
                                                const float* __restrict__ dt_bias,
                                                const float* __restrict__ A_log,
                                                const float* __restrict__ A_proj, int64_t H,
                                                float* __restrict__ state,
                                                float* __restrict__ norm, float* __restrict__ y,
                                                DecodeConv conv) {
  constexpr int R = Rows<DH, ORDER, PACKED>::value;
  constexpr int CG = DH / 4;         // 16-byte column groups per state row
  constexpr int RPP = NTH / CG;      // rows per pass of the workgroup
  constexpr int U = (R / RPP) < UR ? (R / RPP) : UR;  // rows in flight per thread
  constexpr int STEP = RPP * U;
  constexpr int RMAIN = (R / STEP) * STEP;  // rows of the unrolled loop (>= STEP); the rest one by one
  constexpr int NWV = NTH / WAVE;
  constexpr int RT = ORDER == 2 ? R : 1;
  static_assert(U >= 1, "workgroup too large for the state");
  __shared__ float qs[DH], ks[DH], vs[DH];
  __shared__ float fkT[RT], fqT[RT];  // order 2: phi(k)_r, weight_r phi(q)_r
  __shared__ f32x4 red4[NWV][WAVE];
  __shared__ float redd[NWV];

  const int64_t sh = blockIdx.x;
  const int64_t h = sh % H;
  const int tid = threadIdx.x;
  float dtv, alpha;
  if (A_proj) {  // the A-mask: alpha = exp(-softplus(A_P)); dt without bias, or none
    dtv = dt_proj ? softplus_f(dt_proj[sh]) : 1.f;
    alpha = expf(-softplus_f(A_proj[sh]));
  } else {
    dtv = softplus_f(dt_proj[sh] + dt_bias[h]);
    alpha = expf(-expf(A_log[h]) * dtv);
  }
  const int tq = tid < DH ? tid : 0;
  float lq = Elem<St>::ld(q, sh * DH + tq), lk = Elem<St>::ld(k, sh * DH + tq),
        lv = Elem<St>::ld(v, sh * DH + tq);
  if (conv.w && tid < DH) {
    // Algorithm 6's window-2 convolution of channel (., h, tid) of q, k, v:
    // the previous raw token from the conv state, then this step's raw token
    // stored in its place (each workgroup owns its (sequence, head) slice;
    // the read precedes the write in this thread)
    St* cst = static_cast<St*>(conv.state);
    const int64_t s = sh / H;
    float x[3] = {lq, lk, lv};
    const St raw[3] = {q[sh * DH + tid], k[sh * DH + tid], v[sh * DH + tid]};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int64_t ci = ((s * 3 + i) * H + h) * DH + tid;
      const int64_t wi = ((int64_t)i * H + h) * DH + tid;
      const float prev = Elem<St>::ld(cst, ci);
      float c = conv.w[2 * wi] * prev + conv.w[2 * wi + 1] * x[i];
      if (conv.b) c += conv.b[wi];
      if (conv.act) c = c / (1.f + expf(-c));
      x[i] = c;
      cst[ci] = raw[i];
    }
    lq = x[0];
    lk = x[1];
    lv = x[2];
  }
  if (tid < DH) {
    qs[tid] = lq;
    ks[tid] = lk;
    vs[tid] = lv * dtv;
  }
  __syncthreads();
  if constexpr (ORDER == 2) {
    for (int e = tid; e < DH * DH; e += NTH) {
      const int a = e / DH, b = e - (e / DH) * DH;
      if (!PACKED) {
        fkT[e] = ks[a] * ks[b];
        fqT[e] = qs[a] * qs[b];
      } else if (a <= b) {
        const int p = packed_row(a, b, DH);
        fkT[p] = ks[a] * ks[b];
        fqT[p] = (a == b ? 1.f : 2.f) * (qs[a] * qs[b]);
      }
    }
    __syncthreads();
  }
  const float* fk = ORDER == 2 ? fkT : ks;
  const float* fq = ORDER == 2 ? fqT : qs;

  const int cg = tid % CG, r0 = tid / CG;
  float* Sp = state + sh * (int64_t)R * DH + 4 * cg;
  const f32x4 vd = {vs[4 * cg], vs[4 * cg + 1], vs[4 * cg + 2], vs[4 * cg + 3]};
  f32x4 acc = zero4();
  for (int rb = r0; rb < RMAIN; rb += STEP) {
    f32x4 s[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + (int64_t)(rb + u * RPP) * DH));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rw = rb + u * RPP;
      const f32x4 ns = alpha * s[u] + fk[rw] * vd;
      __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(Sp + (int64_t)rw * DH));
      acc += fq[rw] * ns;
    }
  }
  if constexpr (RMAIN < R) {  // the last rows when the passes do not tile the state
    for (int rw = RMAIN + r0; rw < R; rw += RPP) {
      const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sp + (int64_t)rw * DH));
      const f32x4 ns = alpha * t + fk[rw] * vd;
      __builtin_nontemporal_store(ns, reinterpret_cast<f32x4*>(Sp + (int64_t)rw * DH));
      acc += fq[rw] * ns;
    }
  }
  float dacc = 0.f;
  float* zp = norm + sh * (int64_t)R;
  for (int e = tid; e < R; e += NTH) {
    const float nz = alpha * zp[e] + fk[e];
    zp[e] = nz;
    dacc += fq[e] * nz;
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

hipError_t launch_decode(bool bf16, int64_t DH, int order, bool packed, const void* q,
                         const void* k, const void* v, const float* dt_proj, const float* dt_bias,
                         const float* A_log, const float* A_proj, int64_t S, int64_t H,
                         float* state, float* norm_state, float* y, hipStream_t stream,
                         DecodeConv conv) {
  const dim3 grid((unsigned)(S * H));
  // workgroup size x rows in flight per thread: order 2 full 1024 x 4 (71.7%
  // of the HBM peak on the 256 x 32-head step), packed 512 x 8 (68.5%, against
  // 66.9% at 1024 x 4), order 1 256 x 8
#define DEC_NTH(ORD, PK) (ORD == 1 ? 256 : (PK ? 512 : 1024))
#define DEC_ROWS(ORD, PK) (ORD == 1 ? 8 : (PK ? 8 : 4))
#define SSD_LAUNCH_DEC(ST, DHV, ORD, PK)                                                         \
  hipLaunchKernelGGL((k_decode<ST, DHV, ORD, DEC_NTH(ORD, PK), DEC_ROWS(ORD, PK), PK>), grid,   \
                     dim3(DEC_NTH(ORD, PK)), 0, stream, static_cast<const ST*>(q),               \
                     static_cast<const ST*>(k), static_cast<const ST*>(v), dt_proj, dt_bias,   \
                     A_log, A_proj, H, state, norm_state, y, conv)
#define SSD_DEC_ORDERS(ST, DHV)                      \
  if (order == 1) SSD_LAUNCH_DEC(ST, DHV, 1, false); \
  else if (packed) SSD_LAUNCH_DEC(ST, DHV, 2, true); \
  else SSD_LAUNCH_DEC(ST, DHV, 2, false);
  if (bf16) {
    if (DH == 64) {
      SSD_DEC_ORDERS(uint16_t, 64)
    } else {
      SSD_DEC_ORDERS(uint16_t, 32)
    }
  } else {
    if (DH == 64) {
      SSD_DEC_ORDERS(float, 64)
    } else {
      SSD_DEC_ORDERS(float, 32)
    }
  }
#undef SSD_DEC_ORDERS
#undef SSD_LAUNCH_DEC
#undef DEC_ROWS
#undef DEC_NTH
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// layout conversion of the order-2 states; workgroup (bh, a) covers the rows
// with first index a
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void k_state_pack(const float* __restrict__ S,
                                                    const float* __restrict__ z,
                                                    float* __restrict__ Sp,
                                                    float* __restrict__ zp) {
  constexpr int CG = DH / 4, RP = DH * (DH + 1) / 2;
  const int64_t bh = blockIdx.x / DH;
  const int a = blockIdx.x - (int)(bh * DH);
  const float* Sb = S + bh * (int64_t)DH * DH * DH;
  float* Spb = Sp + bh * (int64_t)RP * DH;
  // packed row (a, b), b >= a: the mean of full rows (a, b) and (b, a)
  for (int i = threadIdx.x; i < (DH - a) * CG; i += 256) {
    const int b = a + i / CG, c = 4 * (i % CG);
    const f32x4 x = *reinterpret_cast<const f32x4*>(Sb + (a * DH + b) * DH + c);
    const f32x4 t = *reinterpret_cast<const f32x4*>(Sb + (b * DH + a) * DH + c);
    *reinterpret_cast<f32x4*>(Spb + packed_row(a, b, DH) * DH + c) = 0.5f * (x + t);
  }
  const int b = a + threadIdx.x;
  if (b < DH) {
    const float* zb = z + bh * DH * DH;
    zp[bh * RP + packed_row(a, b, DH)] = 0.5f * (zb[a * DH + b] + zb[b * DH + a]);
  }
}

template <int DH>
__global__ __launch_bounds__(256) void k_state_unpack(const float* __restrict__ Sp,
                                                      const float* __restrict__ zp,
                                                      float* __restrict__ S,
                                                      float* __restrict__ z) {
  constexpr int CG = DH / 4, RP = DH * (DH + 1) / 2;
  const int64_t bh = blockIdx.x / DH;
  const int a = blockIdx.x - (int)(bh * DH);
  const float* Spb = Sp + bh * (int64_t)RP * DH;
  float* Sb = S + bh * (int64_t)DH * DH * DH;
  for (int i = threadIdx.x; i < DH * CG; i += 256) {
    const int b = i / CG, c = 4 * (i % CG);
    const int p = a <= b ? packed_row(a, b, DH) : packed_row(b, a, DH);
    *reinterpret_cast<f32x4*>(Sb + (a * DH + b) * DH + c) =
        *reinterpret_cast<const f32x4*>(Spb + p * DH + c);
  }
  const int b = threadIdx.x;
  if (b < DH) {
    const int p = a <= b ? packed_row(a, b, DH) : packed_row(b, a, DH);
    z[bh * DH * DH + a * DH + b] = zp[bh * RP + p];
  }
}

hipError_t launch_state_layout(bool to_packed, int64_t DH, int64_t BH, const float* src_S,
                               const float* src_z, float* dst_S, float* dst_z,
                               hipStream_t stream) {
  const dim3 grid((unsigned)(BH * DH)), blk(256);
  if (to_packed) {
    if (DH == 64) hipLaunchKernelGGL(k_state_pack<64>, grid, blk, 0, stream, src_S, src_z, dst_S, dst_z);
    else hipLaunchKernelGGL(k_state_pack<32>, grid, blk, 0, stream, src_S, src_z, dst_S, dst_z);
  } else {
    if (DH == 64) hipLaunchKernelGGL(k_state_unpack<64>, grid, blk, 0, stream, src_S, src_z, dst_S, dst_z);
    else hipLaunchKernelGGL(k_state_unpack<32>, grid, blk, 0, stream, src_S, src_z, dst_S, dst_z);
  }
  return hipGetLastError();
}

}  // namespace ssd
