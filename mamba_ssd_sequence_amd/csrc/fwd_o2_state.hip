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
//     update : S_a += K^T diag(k_:a) X,          X_jc = w_j (v dt)_jc
//     output : Y   += diag(qe_:a) (Q S_a),       qe_ia = q_ia exp(A^CS_i - A^CS_start)
// so phi(q), phi(k) are never formed, only the per-row scalings.
//
// Decomposition.  The 1 MiB state never leaves the chip: each workgroup owns
// an a-slice (8*AW values of a) x a 16-column value slice, held as MFMA
// accumulators (fp32) across the whole sequence, and walks the blocks in
// order.  Wave w owns AW values of a (AW x 64 x 16 fp32 = 16*AW VGPRs/lane).
// The A operand of the output product is the state itself (its accumulator
// layout read as a permuted-k operand), the A operand of the update is K^T.
// The workgroup's partial output (its a-slice) is reduced over its waves in
// LDS and written to the workspace; the output kernel adds the P_a partials.
//
// Precision.  Both products run on v_mfma_f32_16x16x32_f16 (same rate as
// bf16) with exact power-of-two scales chosen per block: q*2^tau < 2^13 and
// k*2^kap in (-1, 1) (bf16 inputs convert to fp16 exactly), the state operand
// S*2^sig where sig follows a running upper bound M >= max|S|
// (M <- e^T M + sum_j w_j max|k_j|^2 max|v_j dt_j|, kept below 2^13 after
// scaling), and the update operand (k_ja 2^kap) * X_jc with
// X_jc = w_j (v dt)_jc 2^(sig - 2 kap) < 2^15, formed by packed fp16 multiplies.
// fp16's 11-bit significand matters here: the factored sum over (a, b) can
// cancel when q is nearly orthogonal to the block's keys, and a bf16 rounding
// of the state is amplified there beyond the bf16 tolerance.  Every thread
// reads the block's scalars itself and takes the same scale decisions, so no
// barrier is needed for them.
//
// Pipeline, one barrier per block n: reduce block n-1's partial outputs
// (LDS) into the workspace; decide the scales of block n+1 and copy its
// record (prefetched into registers one iteration earlier) into the other LDS
// slot; issue the loads of block n+2; run block n's MFMA work and write its
// partial output to LDS.  Half of the waves do the MFMA work first and the
// other half last, so every SIMD keeps its matrix core busy while the other
// wave does the bookkeeping.  The per-block operands arrive pre-converted from
// the block-prep kernel, so staging is plain copies.
//
// Grid: B*H x P_a x 4 workgroups (P_a = 64 / (8*AW)), 512 threads each; when
// B*H is a multiple of 8 the workgroups of one head share an XCD (and its L2).
#include "common.h"
#include "launch.h"

namespace ssd {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int DH = 64;
constexpr int CW = 16;      // value columns per workgroup
constexpr int PH = DH + 8;  // fp16 row pitch (elements): 144 B
constexpr int EXP_CLAMP = 64;

__device__ __forceinline__ f32x4 mfma_f16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// exponent e with x < 2^e (x > 0 finite); 0 otherwise
__device__ __forceinline__ int exp_ceil(float x) {
  if (!(x > 0.f) || !isfinite(x)) return 0;
  int e;
  frexpf(x, &e);
  return e;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ float max8_abs_bf16(const uint4& u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xffff0000u)));
  }
  return m;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) x += __shfl_xor(x, off, WAVE);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, WAVE));
  return x;
}
}  // namespace

template <int AW>
__global__ __launch_bounds__(512) void k_o2_state(const uint8_t* __restrict__ rec, int64_t BH,
                                                  int64_t N, int xcd_map,
                                                  float* __restrict__ part,
                                                  float* __restrict__ final_state) {
  constexpr int NW = 8;               // waves per workgroup
  constexpr int NT = NW * WAVE;       // threads
  constexpr int SL = NW * AW;         // a values per workgroup
  constexpr int PA = DH / SL;         // a-slices per head
  static_assert(BLK * DH / 8 == NT && CW * DH / 2 == NT, "thread mapping");

  // staging (by block parity) and partial-output buffers; e^{cs} rows rotate
  // over three slots because the drain of block n-1 may still read them while
  // block n+1 is staged
  __shared__ __attribute__((aligned(16))) _Float16 Qh[2][BLK * PH];  // [i][perm b] q 2^tau
  __shared__ __attribute__((aligned(16))) _Float16 KTh[2][DH * PH];  // [b][j] k 2^kap
  __shared__ __attribute__((aligned(16))) _Float16 Xh[2][CW * PH];   // [c][j] X 2^xi
  __shared__ __attribute__((aligned(16))) float red[2][NW][BLK * CW];  // [i][c] per wave
  __shared__ float st_ecs[3][BLK];

  const int tid = threadIdx.x;
  const int wave = tid / WAVE, lane = tid & (WAVE - 1), n = lane & 15, g = lane >> 4;
  int pc, pa;
  int64_t bh;
  if (xcd_map) {
    // workgroups are dispatched round-robin over the 8 XCDs: give all the
    // workgroups of one head the same id mod 8, so they share one L2
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int p = s % (PA * 4);
    bh = (int64_t)(s / (PA * 4)) * 8 + xcd;
    pa = p >> 2;
    pc = p & 3;
  } else {
    pc = blockIdx.x & 3;
    pa = (blockIdx.x >> 2) % PA;
    bh = (blockIdx.x >> 2) / PA;
  }
  const int a0 = pa * SL;
  const int c0 = pc * CW;
  const int64_t nblk = n_blocks(N);
  const uint8_t* rec_h = rec + bh * nblk * (int64_t)REC_BYTES;

  // copy roles: q / k^T row r8 and 16-byte segment sg; one 32-bit word of
  // the workgroup's 16 X^T rows
  const int r8 = tid >> 3, sg = tid & 7;
  const int xr = tid >> 5, xw = tid & 31;
  // column of q_:a in the permuted q layout, for this wave's a values
  int qpos[AW];
#pragma unroll
  for (int ai = 0; ai < AW; ++ai) {
    const int a = a0 + wave * AW + ai, bl = a & 31;
    qpos[ai] = (a & ~31) + (bl < 16 ? 8 * (bl >> 2) + (bl & 3) : 8 * ((bl - 16) >> 2) + 4 + (bl & 3));
  }

  // ---- registers of the prefetched block -------------------------------------
  uint4 pq, pk;
  uint32_t px, pe = 0;
  float pdelta, peT;
  int ptau, pkap, pxi;
  auto prefetch = [&](int64_t blk) {
    const uint8_t* R = rec_h + blk * (int64_t)REC_BYTES;
    pq = *reinterpret_cast<const uint4*>(R + REC_QH + (r8 * DH + sg * 8) * 2);
    pk = *reinterpret_cast<const uint4*>(R + REC_KT + (r8 * DH + sg * 8) * 2);
    px = *reinterpret_cast<const uint32_t*>(R + REC_XT + ((c0 + xr) * DH + 2 * xw) * 2);
    if (tid < BLK) pe = *reinterpret_cast<const uint32_t*>(R + REC_ECS + 4 * tid);
    const float* sc = reinterpret_cast<const float*>(R + REC_SC);  // uniform address
    pdelta = sc[1];
    ptau = __float_as_int(sc[2]);
    pkap = __float_as_int(sc[3]);
    pxi = __float_as_int(sc[4]);
    peT = sc[5];
  };

  // scale state, identical in every thread
  float M = 0.f;     // upper bound of max |S| (true units) after the last decided block
  int sig_dec = 0;   // sigma of the last decided block: S is held as S * 2^sigma
  struct Blk {
    int sig, shift, tau, kap, xi;
    float eT;
  };
  Blk nx{}, cur{}, prv{};

  // decide the scales of the prefetched block blk and copy it into its slots
  auto stage = [&](int64_t blk) {
    const int sl = (int)(blk & 1);
    nx.tau = ptau;
    nx.kap = pkap;
    nx.xi = pxi;
    nx.eT = peT;
    // every update operand X 2^(sig - 2 kap) < 4 delta 2^sig <= 4 M 2^sig <= 2^15
    const float m_after = peT * M + pdelta;
    const float mh = fmaxf(M, m_after);
    int sig = sig_dec;
    if (mh > 0.f && isfinite(mh)) {
      const int target = clampi(13 - exp_ceil(mh), -EXP_CLAMP, EXP_CLAMP);
      if (sig > target || sig < target - 12) sig = target;
    }
    nx.shift = sig - sig_dec;
    nx.sig = sig;
    sig_dec = sig;
    M = m_after;
    *reinterpret_cast<uint4*>(&Qh[sl][r8 * PH + sg * 8]) = pq;
    *reinterpret_cast<uint4*>(&KTh[sl][r8 * PH + sg * 8]) = pk;
    *reinterpret_cast<uint32_t*>(&Xh[sl][xr * PH + 2 * xw]) = px;
    if (tid < BLK) st_ecs[blk % 3][tid] = __uint_as_float(pe);
  };

  // partial output of block blk (its scales in p) -> workspace, scaled to
  // true units: e^{cs_i} 2^-(sig + 2 tau)
  auto drain = [&](int64_t blk, const Blk& p) {
    if (tid < BLK * CW / 4) {
      const int64_t t0 = blk * BLK;
      const int nv = (int)((N - t0) < BLK ? (N - t0) : BLK);
      const int i = tid >> 2, c4 = (tid & 3) * 4;
      const float* rd = &red[blk & 1][0][i * CW + c4];
      f32x4 s = *reinterpret_cast<const f32x4*>(rd);
#pragma unroll
      for (int w = 1; w < NW; ++w) s += *reinterpret_cast<const f32x4*>(rd + w * BLK * CW);
      const float f = st_ecs[blk % 3][i] * ldexpf(ldexpf(1.f, -p.sig), -2 * p.tau);
      if (i < nv) *reinterpret_cast<f32x4*>(&part[(((int64_t)pa * BH + bh) * N + t0 + i) * DH + c0 + c4]) = s * f;
    }
  };

  f32x4 S[AW][4];
#pragma unroll
  for (int ai = 0; ai < AW; ++ai)
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) S[ai][bt] = zero4();

  // MFMA work of block blk: output with the entering state, then the update
  auto compute = [&](int64_t blk) {
    const int sl = (int)(blk & 1);
    if (cur.shift != 0) {
      const float f = ldexpf(1.f, cur.shift);
#pragma unroll
      for (int ai = 0; ai < AW; ++ai)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) S[ai][bt] *= f;
    }
    if constexpr (AW >= 4) {
      // four a values per wave: output pass then update pass, so that the
      // Q and K^T operand fragments are never live together (register file)
      // T^T[c][i] = sum_b S[b][c] Q[i][b];  Y[i][c] += q_ia T^T[c][i]
      {
        const _Float16* Q = Qh[sl];
        f16x8 Qf[4][2];  // B operand: Q^T[b][i], permuted k = b (pre-ordered)
  #pragma unroll
        for (int it = 0; it < 4; ++it)
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            Qf[it][kb] = *reinterpret_cast<const f16x8*>(&Q[(it * 16 + n) * PH + kb * 32 + 8 * g]);
        f32x4 Y[4];
  #pragma unroll
        for (int it = 0; it < 4; ++it) Y[it] = zero4();
  #pragma unroll
        for (int ai = 0; ai < AW; ++ai) {
          f16x8 SA[2];
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
            for (int r = 0; r < 4; ++r) {
              SA[kb][r] = (_Float16)S[ai][2 * kb][r];
              SA[kb][4 + r] = (_Float16)S[ai][2 * kb + 1][r];
            }
  #pragma unroll
          for (int it = 0; it < 4; ++it) {
            f32x4 T = mfma_f16(SA[0], Qf[it][0], zero4());
            T = mfma_f16(SA[1], Qf[it][1], T);
            Y[it] += (float)Q[(it * 16 + n) * PH + qpos[ai]] * T;
          }
        }
        float* rd = red[sl][wave];
  #pragma unroll
        for (int it = 0; it < 4; ++it) *reinterpret_cast<f32x4*>(&rd[(it * 16 + n) * CW + 4 * g]) = Y[it];
      }
      // S = e^T S + K^T ((k_:a 2^kap) * X 2^(sig - 2 kap))
      {
        const _Float16* KT = KTh[sl];
        f16x8 Kf[4][2];  // A operand: K^T[b][j], k = j contiguous
  #pragma unroll
        for (int bt = 0; bt < 4; ++bt)
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            Kf[bt][kb] = *reinterpret_cast<const f16x8*>(&KT[(bt * 16 + n) * PH + kb * 32 + 8 * g]);
        // X 2^xi -> X 2^(sig - 2 kap): exact power-of-two factors (d <= 2 since
        // max X 2^xi >= 2^13; below 2^-48 the terms are negligible and dropped)
        const int d = cur.sig - 2 * cur.kap - cur.xi;
        f16x8 xh[2];
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) xh[kb] = *reinterpret_cast<const f16x8*>(&Xh[sl][n * PH + kb * 32 + 8 * g]);
        if (d < -48) {
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) xh[kb] = xh[kb] * (_Float16)0.f;
        } else if (d >= -14) {
          if (d != 0) {
            const _Float16 f = (_Float16)ldexpf(1.f, d);
  #pragma unroll
            for (int kb = 0; kb < 2; ++kb) xh[kb] = xh[kb] * f;
          }
        } else {
          const int d1 = d / 2, d2 = d - d1;
          const _Float16 f1 = (_Float16)ldexpf(1.f, d1), f2 = (_Float16)ldexpf(1.f, d2);
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) xh[kb] = (xh[kb] * f1) * f2;
        }
  #pragma unroll
        for (int ai = 0; ai < AW; ++ai) {
          const int a = a0 + wave * AW + ai;  // the K^T row of k_:a
          f16x8 Bu[2];
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            Bu[kb] = *reinterpret_cast<const f16x8*>(&KT[a * PH + kb * 32 + 8 * g]) * xh[kb];
  #pragma unroll
          for (int bt = 0; bt < 4; ++bt) {
            f32x4 acc = cur.eT * S[ai][bt];
            acc = mfma_f16(Kf[bt][0], Bu[0], acc);
            acc = mfma_f16(Kf[bt][1], Bu[1], acc);
            S[ai][bt] = acc;
          }
        }
      }
    } else {
      // per a: output with the entering state, T^T[c][i] = sum_b S[b][c] Q[i][b],
      // Y[i][c] += q_ia T^T[c][i]; then the update
      // S = e^T S + K^T ((k_:a 2^kap) * X 2^(sig - 2 kap)).  The two chains of
      // each a are independent, so their MFMA and VALU work interleave.
      const _Float16* Q = Qh[sl];
      const _Float16* KT = KTh[sl];
      f16x8 Qf[4][2];  // output B operand: Q^T[b][i], permuted k = b (pre-ordered)
  #pragma unroll
      for (int it = 0; it < 4; ++it)
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          Qf[it][kb] = *reinterpret_cast<const f16x8*>(&Q[(it * 16 + n) * PH + kb * 32 + 8 * g]);
      f16x8 Kf[4][2];  // update A operand: K^T[b][j], k = j contiguous
  #pragma unroll
      for (int bt = 0; bt < 4; ++bt)
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          Kf[bt][kb] = *reinterpret_cast<const f16x8*>(&KT[(bt * 16 + n) * PH + kb * 32 + 8 * g]);
      // X 2^xi -> X 2^(sig - 2 kap): exact power-of-two factors (d <= 2 since
      // max X 2^xi >= 2^13; below 2^-48 the terms are negligible and dropped)
      const int d = cur.sig - 2 * cur.kap - cur.xi;
      f16x8 xh[2];
  #pragma unroll
      for (int kb = 0; kb < 2; ++kb) xh[kb] = *reinterpret_cast<const f16x8*>(&Xh[sl][n * PH + kb * 32 + 8 * g]);
      if (d < -48) {
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) xh[kb] = xh[kb] * (_Float16)0.f;
      } else if (d >= -14) {
        if (d != 0) {
          const _Float16 f = (_Float16)ldexpf(1.f, d);
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb) xh[kb] = xh[kb] * f;
        }
      } else {
        const int d1 = d / 2, d2 = d - d1;
        const _Float16 f1 = (_Float16)ldexpf(1.f, d1), f2 = (_Float16)ldexpf(1.f, d2);
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) xh[kb] = (xh[kb] * f1) * f2;
      }
      f32x4 Y[4];
  #pragma unroll
      for (int it = 0; it < 4; ++it) Y[it] = zero4();
  #pragma unroll
      for (int ai = 0; ai < AW; ++ai) {
        f16x8 SA[2];
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            SA[kb][r] = (_Float16)S[ai][2 * kb][r];
            SA[kb][4 + r] = (_Float16)S[ai][2 * kb + 1][r];
          }
        const int a = a0 + wave * AW + ai;  // the K^T row of k_:a
        f16x8 Bu[2];
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          Bu[kb] = *reinterpret_cast<const f16x8*>(&KT[a * PH + kb * 32 + 8 * g]) * xh[kb];
  #pragma unroll
        for (int it = 0; it < 4; ++it) {
          f32x4 T = mfma_f16(SA[0], Qf[it][0], zero4());
          T = mfma_f16(SA[1], Qf[it][1], T);
          const int bt = it;
          f32x4 acc = cur.eT * S[ai][bt];
          acc = mfma_f16(Kf[bt][0], Bu[0], acc);
          acc = mfma_f16(Kf[bt][1], Bu[1], acc);
          S[ai][bt] = acc;
          Y[it] += (float)Q[(it * 16 + n) * PH + qpos[ai]] * T;
        }
      }
      float* rd = red[sl][wave];
  #pragma unroll
      for (int it = 0; it < 4; ++it) *reinterpret_cast<f32x4*>(&rd[(it * 16 + n) * CW + 4 * g]) = Y[it];
    }
  };

  // prologue: stage block 0, prefetch block 1
  prefetch(0);
  stage(0);
  cur = nx;
  if (nblk > 1) prefetch(1);
  __syncthreads();

  // Per block: the first four waves run the MFMA work first, the other four
  // drain/stage first, so each SIMD (waves w and w+4) overlaps the matrix
  // work of one wave with the bookkeeping of the other.
  for (int64_t blk = 0; blk < nblk; ++blk) {
    const bool more = blk + 1 < nblk;
    if (wave < NW / 2) {
      compute(blk);
      if (blk > 0) drain(blk - 1, prv);
      if (more) stage(blk + 1);
    } else {
      if (blk > 0) drain(blk - 1, prv);
      if (more) stage(blk + 1);
      compute(blk);
    }
    if (blk + 2 < nblk) prefetch(blk + 2);
    prv = cur;
    cur = nx;
    __syncthreads();
  }
  drain(nblk - 1, prv);

  if (final_state) {
    const float f = ldexpf(1.f, -sig_dec);
#pragma unroll
    for (int ai = 0; ai < AW; ++ai) {
      const int a = a0 + wave * AW + ai;
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int b = bt * 16 + 4 * g + r;
          final_state[((bh * DH + a) * DH + b) * DH + c0 + n] = S[ai][bt][r] * f;
        }
    }
  }
}

hipError_t launch_o2_state(const void* rec, int64_t BH, int64_t N, float* part,
                           float* final_state, hipStream_t stream) {
  const int AW = o2_aw(BH);
  const int PA = o2_pa(BH);
  const int xcd_map = (BH % 8) == 0;
  const dim3 grid((unsigned)(BH * PA * 4)), blk(8 * WAVE);
  const uint8_t* r = static_cast<const uint8_t*>(rec);
  if (AW == 4)
    hipLaunchKernelGGL((k_o2_state<4>), grid, blk, 0, stream, r, BH, N, xcd_map, part, final_state);
  else if (AW == 2)
    hipLaunchKernelGGL((k_o2_state<2>), grid, blk, 0, stream, r, BH, N, xcd_map, part, final_state);
  else
    hipLaunchKernelGGL((k_o2_state<1>), grid, blk, 0, stream, r, BH, N, xcd_map, part, final_state);
  return hipGetLastError();
}

}  // namespace ssd
