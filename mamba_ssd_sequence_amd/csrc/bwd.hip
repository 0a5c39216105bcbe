// Backward pass of the order-1 chunked mixer (ssd_backward) and of the
// discretisations (ssd_prep_backward, ssd_prep_amask_backward).
//
// The pages train these models but print no gradients; what is computed here
// is the chain rule applied to the same definitions as the forward pass
// (2Mamba2Furious, Algorithm 1's masked product and row-sum normaliser with
// Algorithm 4's decay mask, Algorithm 3's discretisation).  Per 64-token
// block c of a head, with block-relative cumsums cs_i, e_i = e^{cs_i}, the
// block total T, w_j = e^{T - cs_j} and the state S_c, z_c entering the block:
//
//   y_i = num_i / den_i,  num_i = sum_{j<=i} W_ij vop_j + e_i S_c^T q_i,
//   den_i = sum_{j<=i} W_ij + e_i q_i . z_c,  W_ij = (q_i . k_j) e^{cs_i - cs_j},
//   S_{c+1} = e^T S_c + sum_j w_j k_j vop_j^T,  z_{c+1} = e^T z_c + sum_j w_j k_j.
//
// Given dy: dnum_i = dy_i / den_i, dden_i = -dy_i . y_i / den_i.  The
// gradient reaching the state entering block c from the block's own outputs
// is R_c = sum_i e_i q_i dnum_i^T (and r_c = sum_i e_i dden_i q_i); the total
// gradient of S_c is G_c = R_c + e^{T_c} G_{c+1}, a scan over the blocks in
// reverse.  Block c then needs S_c and G_{c+1}:
//   intra:  dW_ij = dnum_i . vop_j + dden_i (j <= i), C_ij = dW_ij e^{cs_i - cs_j},
//           dq_i += sum_j C_ij k_j, dk_j += sum_i C_ij q_i,
//           dvop_j += sum_i W_ij dnum_i, dcs_i += sum_j dW_ij W_ij,
//           dcs_j -= sum_i dW_ij W_ij;
//   inter:  dq_i += e_i (S_c dnum_i + dden_i z_c), dcs_i += q_i . that;
//   state:  t_j = G_{c+1} vop_j + g_{c+1}, dk_j += w_j t_j,
//           dvop_j += w_j G_{c+1}^T k_j, dcs_j -= w_j k_j . t_j,
//           dT = sum_j w_j k_j . t_j + e^T (<G_{c+1}, S_c> + <g_{c+1}, z_c>),
//           added to dcs of the block's last token (T is its cumsum);
//   da_t = sum_{i >= t in the block} dcs_i (cs is the cumsum of a from the
//   block start); dv = dvop dt, ddt = sum_c dvop_c v_c.
//
// Everything is computed in fp32 (the inputs are exact in fp32).  Kernels:
//   k_bwd_outer  (x2)  per block, sum_i wgt_i x_i y_i^T and sum_i wgt_i zw_i x_i:
//                      the block's state increment (forward states, recomputed)
//                      and R_c, r_c; the latter also writes dnum and dden
//   k_state_pass       forward scan of the increments -> S_c (shared with the forward)
//   k_bwd_rev_pass     reverse scan of R_c -> G_{c+1}
//   k_bwd_rows         pair products (W, C, the two sums of dW W), dq, and the row
//                      parts of dcs
//   k_bwd_cols         dk, dvop -> dv, ddt, the column and state parts of dcs, da
#include "common.h"
#include "launch.h"
#include "bwd.h"

namespace ssd {

namespace {

constexpr int PF = BLK + 1;  // fp32 LDS row pitch (odd: strided reads spread over the banks)

struct BlockGeo {
  int64_t bh, blk, t0, row;  // row: token index of (bh, 0)
  int nvalid;
  float base;  // cumsum before the block (0 at a chunk start)
};

__device__ __forceinline__ BlockGeo block_geo(int64_t nblk, int64_t N, int64_t chunk,
                                              const float* a_cs) {
  BlockGeo b;
  b.bh = blockIdx.x / nblk;
  b.blk = blockIdx.x - b.bh * nblk;
  b.t0 = b.blk * BLK;
  b.row = b.bh * N;
  b.nvalid = (int)((N - b.t0) < BLK ? (N - b.t0) : BLK);
  b.base = (b.t0 % chunk == 0) ? 0.f : a_cs[b.row + b.t0 - 1];
  return b;
}

// Row r (token t0 + r) of a [.., N, DH] array: QC values from column c0, as
// fp32; zero for rows past the block's end.
template <typename St, int QC>
__device__ __forceinline__ void load_row(const St* p, const BlockGeo& g, int r, int c0, float* out) {
  const bool ok = r < g.nvalid;
  const int64_t off = (g.row + g.t0 + (ok ? r : 0)) * (int64_t)(4 * QC) + c0;
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    const float x = Elem<St>::ld(p, off + u);
    out[u] = ok ? x : 0.f;
  }
}

// sum over the 4 consecutive lanes of a row (lanes 4r .. 4r + 3)
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 1, WAVE);
  x += __shfl_xor(x, 2, WAVE);
  return x;
}

}  // namespace

// ---------------------------------------------------------------------------
// k_bwd_outer: per block, out[b][c] = sum_i wgt_i x_ib y_ic and
// out[DH*DH + b] = sum_i wgt_i zw_i x_ib, the state-slot layout.
// MODE 0 (forward increment): x = k, y = v dt, wgt_j = e^{T - cs_j}, zw = 1;
// also writes the block total T.  MODE 1 (R_c, r_c): x = q, y = dnum,
// wgt_i = e^{cs_i}, zw = dden; also writes dnum and dden.
// Thread t: row r = t / 4 (staging) / state row b = t / 4 (products), and a
// quarter of the columns.
// ---------------------------------------------------------------------------
template <typename St, int DH, int MODE>
__global__ __launch_bounds__(256) void k_bwd_outer(const St* __restrict__ xs, const St* __restrict__ vs,
                                                   const float* __restrict__ dt,
                                                   const float* __restrict__ y,
                                                   const float* __restrict__ den,
                                                   const float* __restrict__ dy,
                                                   const float* __restrict__ a_cs, int64_t N,
                                                   int64_t chunk, int64_t nblk,
                                                   float* __restrict__ tb,
                                                   float* __restrict__ out,
                                                   float* __restrict__ dnum_out,
                                                   float* __restrict__ dden_out) {
  constexpr int QC = DH / 4;
  constexpr int E = DH * DH + DH;
  __shared__ float X[BLK * PF], Y[BLK * PF], wz[BLK];
  const BlockGeo g = block_geo(nblk, N, chunk, a_cs);
  const int tid = threadIdx.x, r = tid >> 2, c0 = (tid & 3) * QC;
  const int64_t slot = g.bh * nblk + g.blk;
  const bool ok = r < g.nvalid;
  const float cs = ok ? a_cs[g.row + g.t0 + r] - g.base : 0.f;
  const float T = a_cs[g.row + g.t0 + g.nvalid - 1] - g.base;

  float xr[QC], yr[QC];
  load_row<St, QC>(xs, g, r, c0, xr);
  float wgt, zw;
  if constexpr (MODE == 0) {
    load_row<St, QC>(vs, g, r, c0, yr);
    const float d = ok ? (dt ? dt[g.row + g.t0 + r] : 1.f) : 0.f;
#pragma unroll
    for (int u = 0; u < QC; ++u) yr[u] *= d;
    wgt = ok ? expf(T - cs) : 0.f;
    zw = 1.f;
    if (tid == 0) tb[slot] = T;
  } else {
    // dnum = dy / den, dden = -dy . y / den for this row
    const int64_t ro = g.row + g.t0 + (ok ? r : 0);
    const float dn = den[ro];
    float yy[QC], dd[QC], dot = 0.f;
#pragma unroll
    for (int u = 0; u < QC; ++u) {
      yy[u] = y[ro * DH + c0 + u];
      dd[u] = dy[ro * DH + c0 + u];
      dot += yy[u] * dd[u];
    }
    dot = sum4(dot);
    const float rd = 1.f / dn;
#pragma unroll
    for (int u = 0; u < QC; ++u) yr[u] = ok ? dd[u] * rd : 0.f;
    zw = ok ? -dot * rd : 0.f;
    wgt = ok ? expf(cs) : 0.f;
    float* dno = dnum_out + slot * (BLK * DH) + r * DH + c0;
#pragma unroll
    for (int u = 0; u < QC; ++u) dno[u] = yr[u];
    if ((tid & 3) == 0) dden_out[slot * BLK + r] = zw;
  }
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    X[r * PF + c0 + u] = wgt * xr[u];
    Y[r * PF + c0 + u] = yr[u];
  }
  if ((tid & 3) == 0) wz[r] = zw;
  __syncthreads();

  // state row b = tid / 4 (DH rows), columns c0 ..
  const int b = tid >> 2;
  if (b < DH) {
    float acc[QC], az = 0.f;
#pragma unroll
    for (int u = 0; u < QC; ++u) acc[u] = 0.f;
#pragma unroll 4
    for (int i = 0; i < BLK; ++i) {
      const float xb = X[i * PF + b];
#pragma unroll
      for (int u = 0; u < QC; ++u) acc[u] += xb * Y[i * PF + c0 + u];
      az += xb * wz[i];
    }
    float* o = out + slot * (int64_t)E;
#pragma unroll
    for (int u = 0; u < QC; ++u) o[b * DH + c0 + u] = acc[u];
    if ((tid & 3) == 0) o[DH * DH + b] = az;
  }
}

// ---------------------------------------------------------------------------
// k_bwd_rev_pass: in place, slot c <- sum over c' > c of the increments of
// c', decayed: acc = 0; for c = last .. 0: (slot c, acc) <- (acc, e^{T_c} acc
// + slot c).  One state entry per thread, all blocks of the head.
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void k_bwd_rev_pass(int64_t nblk, int eblocks,
                                                      const float* __restrict__ tb,
                                                      float* __restrict__ state) {
  constexpr int E = DH * DH + DH;
  const int64_t bh = blockIdx.x / eblocks;
  const int e = (int)(blockIdx.x - bh * eblocks) * 256 + threadIdx.x;
  if (e >= E) return;
  float* p = state + bh * nblk * E + e;
  const float* t = tb + bh * nblk;
  float acc = 0.f;
  constexpr int U = 16;
  int64_t c = nblk;  // slots [c, nblk) are done
  for (; c >= U; c -= U) {
    float d[U], T[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      d[u] = p[(c - 1 - u) * E];
      T[u] = t[c - 1 - u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[(c - 1 - u) * E] = acc;
      acc = expf(T[u]) * acc + d[u];
    }
  }
  for (; c > 0; --c) {
    const float d = p[(c - 1) * E];
    const float T = t[c - 1];
    p[(c - 1) * E] = acc;
    acc = expf(T) * acc + d;
  }
}

// ---------------------------------------------------------------------------
// k_bwd_rows: the pair products of a block and everything indexed by the
// query row: W and C (to the workspace, for k_bwd_cols), the row and column
// sums of dW W, dq (intra + inter), and the row part of dcs.
// Pair tile of thread t: rows 4 (t / 16) .., columns 4 (t % 16) ..; row
// mapping of the contractions: row t / 4, a quarter of the columns.
// ---------------------------------------------------------------------------
template <typename St, int DH>
__global__ __launch_bounds__(256) void k_bwd_rows(const St* __restrict__ q, const St* __restrict__ k,
                                                  const St* __restrict__ v,
                                                  const float* __restrict__ dt,
                                                  const float* __restrict__ a_cs, int64_t N,
                                                  int64_t chunk, int64_t nblk,
                                                  const float* __restrict__ sst,
                                                  const float* __restrict__ dnw,
                                                  const float* __restrict__ ddw,
                                                  float* __restrict__ ww, float* __restrict__ cw,
                                                  float* __restrict__ rowp,
                                                  float* __restrict__ colp,
                                                  float* __restrict__ dq) {
  constexpr int QC = DH / 4;
  constexpr int E = DH * DH + DH;
  __shared__ float A[BLK * PF], Bm[BLK * PF];
  __shared__ float csl[BLK], ddl[BLK], rowl[BLK], zl[DH], colw[4][BLK];
  const BlockGeo g = block_geo(nblk, N, chunk, a_cs);
  const int tid = threadIdx.x, r = tid >> 2, c0 = (tid & 3) * QC;
  const int64_t slot = g.bh * nblk + g.blk;
  const float* st = sst + slot * (int64_t)E;

  // phase 1: s = Q K^T on the pair tile
  float qr[QC], kr[QC];
  load_row<St, QC>(q, g, r, c0, qr);
  load_row<St, QC>(k, g, r, c0, kr);
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    A[r * PF + c0 + u] = qr[u];
    Bm[r * PF + c0 + u] = kr[u];
  }
  if (tid < BLK) {
    const bool ok = tid < g.nvalid;
    csl[tid] = ok ? a_cs[g.row + g.t0 + tid] - g.base : 0.f;
    ddl[tid] = ddw[slot * BLK + tid];
  }
  if (tid < DH) zl[tid] = st[DH * DH + tid];
  __syncthreads();
  const int ti = tid >> 4, tj = tid & 15;
  float s[4][4], a[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int u = 0; u < 4; ++u) s[x][u] = a[x][u] = 0.f;
#pragma unroll 4
  for (int b = 0; b < DH; ++b) {
    float qa[4], kb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      qa[x] = A[(4 * ti + x) * PF + b];
      kb[x] = Bm[(4 * tj + x) * PF + b];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int u = 0; u < 4; ++u) s[x][u] += qa[x] * kb[u];
  }
  __syncthreads();

  // phase 2: dnum . vop on the pair tile
  float dn[QC], vr[QC];
  {
    const float* dp = dnw + slot * (BLK * DH) + r * DH + c0;
#pragma unroll
    for (int u = 0; u < QC; ++u) dn[u] = dp[u];
    load_row<St, QC>(v, g, r, c0, vr);
    const float d = r < g.nvalid ? (dt ? dt[g.row + g.t0 + r] : 1.f) : 0.f;
#pragma unroll
    for (int u = 0; u < QC; ++u) {
      A[r * PF + c0 + u] = dn[u];
      Bm[r * PF + c0 + u] = vr[u] * d;
    }
  }
  __syncthreads();
#pragma unroll 4
  for (int c = 0; c < DH; ++c) {
    float da_[4], vb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      da_[x] = A[(4 * ti + x) * PF + c];
      vb[x] = Bm[(4 * tj + x) * PF + c];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int u = 0; u < 4; ++u) a[x][u] += da_[x] * vb[u];
  }

  // pair quantities: W, C = dW D, P = dW W (zero outside j <= i < nvalid)
  float rowP[4] = {0.f, 0.f, 0.f, 0.f}, colP[4] = {0.f, 0.f, 0.f, 0.f};
  float Cq[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = 4 * ti + x;
    f32x4 Wv, Cv;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = 4 * tj + u;
      const bool ok = j <= i && i < g.nvalid;
      const float D = ok ? expf(csl[i] - csl[j]) : 0.f;
      const float W = s[x][u] * D;
      const float dW = ok ? a[x][u] + ddl[i] : 0.f;
      const float C = dW * D;
      const float P = dW * W;
      Wv[u] = W;
      Cv[u] = C;
      Cq[x][u] = C;
      rowP[x] += P;
      colP[u] += P;
    }
    *reinterpret_cast<f32x4*>(&ww[slot * (BLK * BLK) + i * BLK + 4 * tj]) = Wv;
    *reinterpret_cast<f32x4*>(&cw[slot * (BLK * BLK) + i * BLK + 4 * tj]) = Cv;
  }
  // row sums over the 16 lanes of a tile row (lanes 16 ti .. 16 ti + 15)
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    float p = rowP[x];
    p += __shfl_xor(p, 1, WAVE);
    p += __shfl_xor(p, 2, WAVE);
    p += __shfl_xor(p, 4, WAVE);
    p += __shfl_xor(p, 8, WAVE);
    rowP[x] = p;
  }
  // column sums: over the 4 tile rows of a wave (lanes xor 16, 32), then waves
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float p = colP[u];
    p += __shfl_xor(p, 16, WAVE);
    p += __shfl_xor(p, 32, WAVE);
    colP[u] = p;
  }
  __syncthreads();  // phase-2 operands no longer needed
  if (tj == 0) {
#pragma unroll
    for (int x = 0; x < 4; ++x) rowl[4 * ti + x] = rowP[x];
  }
  if ((tid & 63) < 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) colw[tid >> 6][4 * tj + u] = colP[u];
  }
  // phase 3: dq_intra = C K
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int u = 0; u < 4; ++u) A[(4 * ti + x) * PF + 4 * tj + u] = Cq[x][u];
#pragma unroll
  for (int u = 0; u < QC; ++u) Bm[r * PF + c0 + u] = kr[u];
  __syncthreads();
  if (tid < BLK)
    colp[slot * BLK + tid] = (colw[0][tid] + colw[1][tid]) + (colw[2][tid] + colw[3][tid]);
  float dqi[QC];
#pragma unroll
  for (int u = 0; u < QC; ++u) dqi[u] = 0.f;
#pragma unroll 4
  for (int j = 0; j < BLK; ++j) {
    const float cij = A[r * PF + j];
#pragma unroll
    for (int u = 0; u < QC; ++u) dqi[u] += cij * Bm[j * PF + c0 + u];
  }
  __syncthreads();

  // phase 4: inter part, u_ib = sum_c S_c[b][c] dnum_ic for this row's b
  // range; dq_inter = e_i (u_i + dden_i z_c)
  for (int e = tid; e < DH * DH; e += 256) Bm[(e / DH) * PF + (e % DH)] = st[e];
#pragma unroll
  for (int u = 0; u < QC; ++u) A[r * PF + c0 + u] = dn[u];
  __syncthreads();
  const float ei = r < g.nvalid ? expf(csl[r]) : 0.f;
  float acc[QC];
#pragma unroll
  for (int u = 0; u < QC; ++u) acc[u] = 0.f;
#pragma unroll 4
  for (int c = 0; c < DH; ++c) {
    const float dnc = A[r * PF + c];
#pragma unroll
    for (int u = 0; u < QC; ++u) acc[u] += Bm[(c0 + u) * PF + c] * dnc;
  }
  float dcs_inter = 0.f;
  float dqo[QC];
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    const float inter = ei * (acc[u] + ddl[r] * zl[c0 + u]);
    dcs_inter += qr[u] * inter;
    dqo[u] = dqi[u] + inter;
  }
  dcs_inter = sum4(dcs_inter);
  if (r < g.nvalid) {
    float* o = dq + (g.row + g.t0 + r) * DH + c0;
#pragma unroll
    for (int u = 0; u < QC; ++u) o[u] = dqo[u];
    if ((tid & 3) == 0) rowp[slot * BLK + r] = rowl[r] + dcs_inter;
  }
}

// ---------------------------------------------------------------------------
// k_bwd_cols: everything indexed by the key row j: dk (intra + state), dvop
// (intra + state) -> dv and ddt, dcs (row part from k_bwd_rows, column part,
// state part, dT at the last token) -> da.  Thread t: row j = t / 4, a
// quarter of the columns.
// ---------------------------------------------------------------------------
template <typename St, int DH>
__global__ __launch_bounds__(256) void k_bwd_cols(const St* __restrict__ q, const St* __restrict__ k,
                                                  const St* __restrict__ v,
                                                  const float* __restrict__ dt,
                                                  const float* __restrict__ a_cs, int64_t N,
                                                  int64_t chunk, int64_t nblk,
                                                  const float* __restrict__ sst,
                                                  const float* __restrict__ gst,
                                                  const float* __restrict__ dnw,
                                                  const float* __restrict__ ww,
                                                  const float* __restrict__ cw,
                                                  const float* __restrict__ rowp,
                                                  const float* __restrict__ colp,
                                                  float* __restrict__ dk, float* __restrict__ dv,
                                                  float* __restrict__ ddt,
                                                  float* __restrict__ da) {
  constexpr int QC = DH / 4;
  constexpr int E = DH * DH + DH;
  __shared__ float A[BLK * PF], Bm[BLK * PF], Cm[BLK * PF];
  __shared__ float gl[DH], dcl[BLK], red[4];
  const BlockGeo g = block_geo(nblk, N, chunk, a_cs);
  const int tid = threadIdx.x, j = tid >> 2, c0 = (tid & 3) * QC;
  const int64_t slot = g.bh * nblk + g.blk;
  const float* st = sst + slot * (int64_t)E;
  const float* gs = gst + slot * (int64_t)E;
  const bool ok = j < g.nvalid;
  const float cs = ok ? a_cs[g.row + g.t0 + j] - g.base : 0.f;
  const float T = a_cs[g.row + g.t0 + g.nvalid - 1] - g.base;
  const float wj = ok ? expf(T - cs) : 0.f;
  const float dtj = ok ? (dt ? dt[g.row + g.t0 + j] : 1.f) : 0.f;

  // phase 1: dk_intra[j] = sum_i C[i][j] q_i
  float qr[QC], kr[QC], vr[QC];
  load_row<St, QC>(q, g, j, c0, qr);
  load_row<St, QC>(k, g, j, c0, kr);
  load_row<St, QC>(v, g, j, c0, vr);
  const float* cb = cw + slot * (BLK * BLK);
  for (int e = tid; e < BLK * BLK; e += 256) A[(e / BLK) * PF + (e % BLK)] = cb[e];
#pragma unroll
  for (int u = 0; u < QC; ++u) Bm[j * PF + c0 + u] = qr[u];
  __syncthreads();
  float dkj[QC];
#pragma unroll
  for (int u = 0; u < QC; ++u) dkj[u] = 0.f;
#pragma unroll 4
  for (int i = 0; i < BLK; ++i) {
    const float cij = A[i * PF + j];
#pragma unroll
    for (int u = 0; u < QC; ++u) dkj[u] += cij * Bm[i * PF + c0 + u];
  }
  __syncthreads();

  // phase 2: dvop_intra[j] = sum_i W[i][j] dnum_i
  const float* wb = ww + slot * (BLK * BLK);
  for (int e = tid; e < BLK * BLK; e += 256) A[(e / BLK) * PF + (e % BLK)] = wb[e];
  {
    const float* dp = dnw + slot * (BLK * DH) + j * DH + c0;
#pragma unroll
    for (int u = 0; u < QC; ++u) Bm[j * PF + c0 + u] = dp[u];
  }
  __syncthreads();
  float dvj[QC];
#pragma unroll
  for (int u = 0; u < QC; ++u) dvj[u] = 0.f;
#pragma unroll 4
  for (int i = 0; i < BLK; ++i) {
    const float wij = A[i * PF + j];
#pragma unroll
    for (int u = 0; u < QC; ++u) dvj[u] += wij * Bm[i * PF + c0 + u];
  }
  __syncthreads();

  // phase 3: the state terms with G = G_{c+1}: t_j = G vop_j + g,
  // dk_j += w_j t_j, dvop_j += w_j G^T k_j, k_j . t_j
  for (int e = tid; e < DH * DH; e += 256) A[(e / DH) * PF + (e % DH)] = gs[e];
  if (tid < DH) gl[tid] = gs[DH * DH + tid];
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    Bm[j * PF + c0 + u] = vr[u] * dtj;  // vop
    Cm[j * PF + c0 + u] = kr[u];
  }
  __syncthreads();
  float tj[QC], gk[QC];
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    tj[u] = gl[c0 + u];
    gk[u] = 0.f;
  }
#pragma unroll 4
  for (int c = 0; c < DH; ++c) {
    const float vc = Bm[j * PF + c];  // t_b = g_b + sum_c G[b][c] vop_jc, b in this quarter
#pragma unroll
    for (int u = 0; u < QC; ++u) tj[u] += A[(c0 + u) * PF + c] * vc;
  }
#pragma unroll 4
  for (int b = 0; b < DH; ++b) {
    const float kb = Cm[j * PF + b];  // (G^T k_j)_c, c in this quarter
#pragma unroll
    for (int u = 0; u < QC; ++u) gk[u] += A[b * PF + c0 + u] * kb;
  }
  float kt = 0.f;
#pragma unroll
  for (int u = 0; u < QC; ++u) {
    dkj[u] += wj * tj[u];
    kt += kr[u] * tj[u];
    dvj[u] += wj * gk[u];
  }
  kt = sum4(kt);
  // <G, S_c> + <g, z_c> over the block's state slots
  float gsd = 0.f;
  for (int e = tid; e < E; e += 256) gsd += gs[e] * st[e];
  for (int off = 1; off < WAVE; off <<= 1) gsd += __shfl_xor(gsd, off, WAVE);
  // sum_j w_j k_j . t_j over the block (one lane per row)
  float wkt = ((tid & 3) == 0) ? wj * kt : 0.f;
  for (int off = 1; off < WAVE; off <<= 1) wkt += __shfl_xor(wkt, off, WAVE);
  if ((tid & 63) == 0) red[tid >> 6] = wkt + expf(T) * gsd;
  __syncthreads();
  const float dT = (red[0] + red[1]) + (red[2] + red[3]);

  // outputs of row j
  float ddtj = 0.f;
#pragma unroll
  for (int u = 0; u < QC; ++u) ddtj += dvj[u] * vr[u];
  ddtj = sum4(ddtj);
  if (ok) {
    const int64_t o = (g.row + g.t0 + j) * DH + c0;
#pragma unroll
    for (int u = 0; u < QC; ++u) {
      dk[o + u] = dkj[u];
      dv[o + u] = dvj[u] * dtj;
    }
  }
  if ((tid & 3) == 0) {
    float dcs = 0.f;
    if (ok) {
      dcs = rowp[slot * BLK + j] - colp[slot * BLK + j] - wj * kt;
      if (j == g.nvalid - 1) dcs += dT;
      if (ddt) ddt[g.row + g.t0 + j] = ddtj;
    }
    dcl[j] = dcs;
  }
  __syncthreads();
  // da_t = sum_{s >= t} dcs_s within the block: a reverse scan by wave 0
  if (tid < BLK) {
    float x = dcl[BLK - 1 - tid];  // lane l holds dcs of token 63 - l
    for (int off = 1; off < WAVE; off <<= 1) {
      const float y = __shfl_up(x, off, WAVE);
      if (tid >= off) x += y;
    }
    const int t = BLK - 1 - tid;
    if (t < g.nvalid) da[g.row + g.t0 + t] = x;
  }
}

// ---------------------------------------------------------------------------
// ssd_prep_backward / ssd_prep_amask_backward: elementwise chain rule, and the
// per-head sums (one workgroup per head, fixed order: deterministic).
// MODE 0 (Algorithm 3): x = dt_P + dt_bias, dt = softplus(x), a = A dt,
//   A = -exp(A_log): g_dt = ddt + da A, d_dt_P = g_dt sigmoid(x),
//   d_dt_bias[h] = sum d_dt_P, d_A_log[h] = A sum da dt.
// MODE 1 (A-mask): a = -softplus(A_P): d_A_P = -da sigmoid(A_P); dt =
//   softplus(dt_P) (if given): d_dt_P = ddt sigmoid(dt_P).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + expf(-x)); }

template <int MODE>
__global__ __launch_bounds__(256) void k_prep_bwd(const float* __restrict__ p0,
                                                  const float* __restrict__ p1,
                                                  const float* __restrict__ A_log,
                                                  const float* __restrict__ da,
                                                  const float* __restrict__ ddt, int64_t B,
                                                  int64_t H, int64_t N, float* __restrict__ o0,
                                                  float* __restrict__ o1,
                                                  float* __restrict__ o2) {
  // one workgroup per head h, looping over the batch and the tokens
  const int64_t h = blockIdx.x;
  __shared__ float red[2][4];
  float sb = 0.f, sa = 0.f;
  float A = 0.f, bias = 0.f;
  if (MODE == 0) {
    A = -expf(A_log[h]);
    bias = p1[h];
  }
  for (int64_t b = 0; b < B; ++b) {
    const int64_t base = (b * H + h) * N;
    for (int64_t n = threadIdx.x; n < N; n += 256) {
      const int64_t i = base + n;
      if (MODE == 0) {
        const float x = p0[i] + bias;
        const float dtv = softplus_f(x);
        const float gdt = (ddt ? ddt[i] : 0.f) + da[i] * A;
        const float d = gdt * sigmoid_f(x);
        o0[i] = d;
        sb += d;
        sa += da[i] * dtv;
      } else {
        o0[i] = -da[i] * sigmoid_f(p0[i]);
        if (p1) o1[i] = ddt[i] * sigmoid_f(p1[i]);
      }
    }
  }
  if (MODE == 0) {
    for (int off = 1; off < WAVE; off <<= 1) {
      sb += __shfl_xor(sb, off, WAVE);
      sa += __shfl_xor(sa, off, WAVE);
    }
    if ((threadIdx.x & 63) == 0) {
      red[0][threadIdx.x >> 6] = sb;
      red[1][threadIdx.x >> 6] = sa;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      o1[h] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
      o2[h] = A * ((red[1][0] + red[1][1]) + (red[1][2] + red[1][3]));
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename St, int DH>
static hipError_t bwd_o1_typed(const void* q, const void* k, const void* v, const float* dt,
                               const float* a_cs, const float* y, const float* den,
                               const float* dy, int64_t BH, int64_t N, int64_t chunk,
                               float* dq, float* dk, float* dv, float* ddt, float* da,
                               const BwdLayout& L, float* ws, hipStream_t stream) {
  const int64_t nb = n_blocks(N);
  const dim3 grid((unsigned)(BH * nb)), blk(256);
  const St* qs = static_cast<const St*>(q);
  const St* ks = static_cast<const St*>(k);
  const St* vs = static_cast<const St*>(v);
  float* tb = ws + L.tb;
  float* sst = ws + L.sst;
  float* gst = ws + L.gst;
  float* dnw = ws + L.dnum;
  float* ddw = ws + L.dden;
  float* wwp = ws + L.w;
  float* cwp = ws + L.c;
  float* rowp = ws + L.rowp;
  float* colp = ws + L.colp;
  constexpr int E = DH * DH + DH;
  const int eblocks = (E + 255) / 256;
  // forward states S_c (recomputed in fp32) and the gradients R_c
  hipLaunchKernelGGL((k_bwd_outer<St, DH, 0>), grid, blk, 0, stream, ks, vs, dt, nullptr, nullptr,
                     nullptr, a_cs, N, chunk, nb, tb, sst, nullptr, nullptr);
  hipLaunchKernelGGL((k_bwd_outer<St, DH, 1>), grid, blk, 0, stream, qs, nullptr, nullptr, y, den,
                     dy, a_cs, N, chunk, nb, nullptr, gst, dnw, ddw);
  hipError_t e = launch_state_pass(DH, BH, N, tb, sst, nullptr, nullptr, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwd_rev_pass<DH>, dim3((unsigned)(BH * eblocks)), blk, 0, stream, nb, eblocks,
                     tb, gst);
  hipLaunchKernelGGL((k_bwd_rows<St, DH>), grid, blk, 0, stream, qs, ks, vs, dt, a_cs, N, chunk, nb,
                     sst, dnw, ddw, wwp, cwp, rowp, colp, dq);
  hipLaunchKernelGGL((k_bwd_cols<St, DH>), grid, blk, 0, stream, qs, ks, vs, dt, a_cs, N, chunk, nb,
                     sst, gst, dnw, wwp, cwp, rowp, colp, dk, dv, ddt, da);
  return hipGetLastError();
}

hipError_t launch_backward_o1(bool bf16, int64_t DH, const void* q, const void* k, const void* v,
                              const float* dt, const float* a_cs, const float* y, const float* den,
                              const float* dy, int64_t BH, int64_t N, int64_t chunk, float* dq,
                              float* dk, float* dv, float* ddt, float* da, float* ws,
                              hipStream_t stream) {
  const BwdLayout L = bwd_layout(BH, N, DH);
  if (bf16) {
    if (DH == 64)
      return bwd_o1_typed<uint16_t, 64>(q, k, v, dt, a_cs, y, den, dy, BH, N, chunk, dq, dk, dv, ddt, da, L, ws, stream);
    return bwd_o1_typed<uint16_t, 32>(q, k, v, dt, a_cs, y, den, dy, BH, N, chunk, dq, dk, dv, ddt, da, L, ws, stream);
  }
  if (DH == 64)
    return bwd_o1_typed<float, 64>(q, k, v, dt, a_cs, y, den, dy, BH, N, chunk, dq, dk, dv, ddt, da, L, ws, stream);
  return bwd_o1_typed<float, 32>(q, k, v, dt, a_cs, y, den, dy, BH, N, chunk, dq, dk, dv, ddt, da, L, ws, stream);
}

hipError_t launch_prep_backward(const float* dt_proj, const float* dt_bias, const float* A_log,
                                const float* da, const float* ddt, int64_t B, int64_t H, int64_t N,
                                float* d_dt_proj, float* d_dt_bias, float* d_A_log,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_prep_bwd<0>, dim3((unsigned)H), dim3(256), 0, stream, dt_proj, dt_bias, A_log, da,
                     ddt, B, H, N, d_dt_proj, d_dt_bias, d_A_log);
  return hipGetLastError();
}

hipError_t launch_prep_amask_backward(const float* A_proj, const float* dt_proj, const float* da,
                                      const float* ddt, int64_t B, int64_t H, int64_t N,
                                      float* d_A_proj, float* d_dt_proj, hipStream_t stream) {
  hipLaunchKernelGGL(k_prep_bwd<1>, dim3((unsigned)H), dim3(256), 0, stream, A_proj, dt_proj, nullptr, da,
                     ddt, B, H, N, d_A_proj, d_dt_proj, nullptr);
  return hipGetLastError();
}

}  // namespace ssd
