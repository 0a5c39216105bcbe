// Order-2 (2Mamba) inter-block numerator: an on-chip scan of the d_h^2 x d_h
// state over 64-token blocks.
//
// 2Mamba2Furious, Algorithm 6: with order-2 features phi(x) = vec(x x^T) the
// numerator state H_up is D x d_h (D = d_h^2 = 4096 at d_h = 64, 1 MiB fp32
// per head).  Over one block of tokens j with decay weights
// w_j = exp(A^CS_last - A^CS_j) it evolves as
//     S <- exp(T_blk) S + sum_j w_j phi(k_j) (v dt)_j^T,
// and the inter-block contribution to the numerator of token i is
//     exp(A^CS_i - A^CS_start) phi(q_i)^T S_in.
// Writing the state row index as (a, b), both contractions factor per a:
//     update : S_a += K^T (u_a * Vdt),        u_ja = w_j k_ja
//     output : Y   += qe_a * (Q S_a),         qe_ia = q_ia exp(A^CS_i - A^CS_start)
// so phi(q), phi(k) are never formed: only the per-row scalings u and qe are.
//
// Decomposition.  The 1 MiB state never leaves the chip: each workgroup owns
// an a-slice (8*AW values of a) x a 16-column value slice, held as MFMA
// accumulators across the whole sequence, and walks the blocks in order.
// 8 waves per workgroup; wave w owns AW values of a (AW x 64 x 16 fp32 = AW*16
// VGPRs per lane).  Per block a wave runs 16*AW v_mfma_f32_16x16x32_bf16 for
// the output and 16*AW for the update; the A operand of the output product is
// the state itself (its accumulator layout, read as a permuted-k operand after
// a bf16 conversion), and the A operand of the update is K^T, loaded once per
// block.  The a-slice partial sums of the output go to the workspace; the
// output kernel adds the P_a partials of a row.
//
// Grid: B*H x P_a x 4 workgroups (P_a = 64 / (8*AW)), 512 threads each.
#include "common.h"
#include "launch.h"

namespace ssd {

namespace {
constexpr int DH = 64;
constexpr int NW = 8;     // waves per workgroup
constexpr int CW = 16;    // value columns per workgroup
constexpr int PQ = DH + 8;  // bf16 row pitch (elements)
constexpr int PF = BLK + 4; // fp32 row pitch
}  // namespace

template <int AW>
__global__ __launch_bounds__(512) void k_o2_state(const uint16_t* __restrict__ q,
                                                  const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v,
                                                  const float* __restrict__ dt,
                                                  const float* __restrict__ a_cs, int64_t BH,
                                                  int64_t N, int64_t chunk,
                                                  float* __restrict__ part,
                                                  float* __restrict__ final_state) {
  constexpr int SL = NW * AW;       // a values per workgroup
  constexpr int PA = DH / SL;       // a-slices per head
  __shared__ __attribute__((aligned(16))) __bf16 Qs[BLK * PQ];   // [i][b]
  __shared__ __attribute__((aligned(16))) __bf16 KTs[DH * PQ];   // [b][j]
  __shared__ __attribute__((aligned(16))) float VT[CW * PF];     // [c][j] value operand slice
  __shared__ __attribute__((aligned(16))) float us[SL * PF];     // [a][j] = w_j k_ja
  __shared__ __attribute__((aligned(16))) float qes[SL * PF];    // [a][i] = q_ia e^{cs_i}
  __shared__ __attribute__((aligned(16))) float red[NW * 16 * WAVE];
  __shared__ float csl[BLK];
  __shared__ float wv[BLK];

  const int tid = threadIdx.x;
  const int wave = tid / WAVE, lane = tid & (WAVE - 1), n = lane & 15, g = lane >> 4;
  const int pc = blockIdx.x & 3;
  const int pa = (blockIdx.x >> 2) % PA;
  const int64_t bh = (blockIdx.x >> 2) / PA;
  const int a0 = pa * SL;   // first a of this workgroup
  const int c0 = pc * CW;   // first value column of this workgroup
  const int64_t row = bh * N;
  const int64_t nblk = n_blocks(N);

  // state S[a][b][c] for this wave's AW rows a: accumulators, b-tile bt
  f32x4 S[AW][4];
#pragma unroll
  for (int ai = 0; ai < AW; ++ai)
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) S[ai][bt] = zero4();

  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t t0 = blk * BLK;
    const int nvalid = (int)((N - t0) < BLK ? (N - t0) : BLK);
    const float base = (t0 % chunk == 0) ? 0.f : a_cs[row + t0 - 1];
    const float cs_last = a_cs[row + t0 + nvalid - 1];
    const float eT = expf(cs_last - base);

    // ---- stage the block ------------------------------------------------
    {
      // Q rows (16 B per thread) and K transposed
      const int j = tid >> 3, seg = tid & 7;
      uint4 qv = make_uint4(0, 0, 0, 0), kv = make_uint4(0, 0, 0, 0);
      if (j < nvalid) {
        qv = *reinterpret_cast<const uint4*>(q + (row + t0 + j) * DH + seg * 8);
        kv = *reinterpret_cast<const uint4*>(k + (row + t0 + j) * DH + seg * 8);
      }
      *reinterpret_cast<uint4*>(&Qs[j * PQ + seg * 8]) = qv;
      const uint16_t* kh = reinterpret_cast<const uint16_t*>(&kv);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const uint16_t bits = kh[s];
        KTs[(seg * 8 + s) * PQ + j] = __builtin_bit_cast(__bf16, bits);
      }
    }
    if (tid < BLK) {
      float c = 0.f, w = 0.f;
      if (tid < nvalid) {
        const float acs = a_cs[row + t0 + tid];
        c = acs - base;
        w = expf(cs_last - acs);
      }
      csl[tid] = c;
      wv[tid] = w;
    }
    for (int e = tid; e < BLK * CW; e += NW * WAVE) {
      const int j = e / CW, c = e - (e / CW) * CW;
      float val = 0.f;
      if (j < nvalid) {
        val = bf16_to_f32(v[(row + t0 + j) * DH + c0 + c]);
        if (dt) val *= dt[row + t0 + j];
      }
      VT[c * PF + j] = val;
    }
    __syncthreads();
    for (int e = tid; e < SL * BLK; e += NW * WAVE) {
      const int a = e / BLK, j = e - (e / BLK) * BLK;
      us[a * PF + j] = wv[j] * (float)KTs[(a0 + a) * PQ + j];
      qes[a * PF + j] = (float)Qs[j * PQ + a0 + a] * expf(csl[j]);
    }
    __syncthreads();

    // ---- per-wave work --------------------------------------------------
    bf16x8 KTf[4][2];  // A operand of the update: K^T[b][j], contiguous k = j
#pragma unroll
    for (int bt = 0; bt < 4; ++bt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        KTf[bt][kb] = *reinterpret_cast<const bf16x8*>(&KTs[(bt * 16 + n) * PQ + kb * 32 + 8 * g]);
    bf16x8 Qf[4][2];   // B operand of the output: Q^T[b][i], permuted k = b
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const __bf16* p = &Qs[(it * 16 + n) * PQ + kb * 32 + 4 * g];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Qf[it][kb][r] = lo[r];
          Qf[it][kb][4 + r] = hi[r];
        }
      }
    float vd[2][8];    // value operand for the update's B, k = j contiguous
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 8; ++s) vd[kb][s] = VT[n * PF + kb * 32 + 8 * g + s];

    f32x4 Y[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) Y[it] = zero4();

#pragma unroll
    for (int ai = 0; ai < AW; ++ai) {
      const int al = wave * AW + ai;  // a within the workgroup slice
      // output with the entering state: T^T[c][i] = sum_b S[b][c] Q[i][b]
      bf16x8 SA[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          SA[kb][r] = (__bf16)S[ai][2 * kb][r];
          SA[kb][4 + r] = (__bf16)S[ai][2 * kb + 1][r];
        }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        f32x4 T = mfma_bf16(SA[0], Qf[it][0], zero4());
        T = mfma_bf16(SA[1], Qf[it][1], T);
        const float qe = qes[al * PF + it * 16 + n];
        Y[it] += qe * T;
      }
      // update: S = e^T S + K^T (u_a * Vdt)
      bf16x8 Bu[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 8; ++s) Bu[kb][s] = (__bf16)(us[al * PF + kb * 32 + 8 * g + s] * vd[kb][s]);
#pragma unroll
      for (int bt = 0; bt < 4; ++bt) {
        f32x4 acc = eT * S[ai][bt];
        acc = mfma_bf16(KTf[bt][0], Bu[0], acc);
        acc = mfma_bf16(KTf[bt][1], Bu[1], acc);
        S[ai][bt] = acc;
      }
    }

    // ---- reduce the output over the workgroup's waves -------------------
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * 16 + it * 4 + r) * WAVE + lane] = Y[it][r];
    __syncthreads();
    for (int o = tid; o < 16 * WAVE; o += NW * WAVE) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w * 16 * WAVE + o];
      const int reg = o / WAVE, ln = o - (o / WAVE) * WAVE;
      const int it = reg >> 2, r = reg & 3;
      const int i = it * 16 + (ln & 15), c = 4 * (ln >> 4) + r;
      if (i < nvalid) part[(((int64_t)pa * BH + bh) * N + t0 + i) * DH + c0 + c] = s;
    }
    __syncthreads();
  }

  if (final_state) {
#pragma unroll
    for (int ai = 0; ai < AW; ++ai) {
      const int a = a0 + wave * AW + ai;
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b = bt * 16 + 4 * g + r;
          final_state[((bh * DH + a) * DH + b) * DH + c0 + n] = S[ai][bt][r];
        }
    }
  }
}

hipError_t launch_o2_state(const void* q, const void* k, const void* v, const float* dt,
                           const float* a_cs, int64_t BH, int64_t N, int64_t chunk, float* part,
                           float* final_state, hipStream_t stream) {
  const int AW = o2_aw(BH);
  const int PA = o2_pa(BH);
  const dim3 grid((unsigned)(BH * PA * 4)), blk(NW * WAVE);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (AW == 4)
    hipLaunchKernelGGL(k_o2_state<4>, grid, blk, 0, stream, qq, kk, vv, dt, a_cs, BH, N, chunk, part, final_state);
  else if (AW == 2)
    hipLaunchKernelGGL(k_o2_state<2>, grid, blk, 0, stream, qq, kk, vv, dt, a_cs, BH, N, chunk, part, final_state);
  else
    hipLaunchKernelGGL(k_o2_state<1>, grid, blk, 0, stream, qq, kk, vv, dt, a_cs, BH, N, chunk, part, final_state);
  return hipGetLastError();
}

}  // namespace ssd
