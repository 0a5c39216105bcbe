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
// an a-slice (NW*AW values of a) x a 16-column value slice, held as MFMA
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
// of the state is amplified there beyond the bf16 tolerance.  Every wave takes
// the same scale decisions from the same LDS data, so no extra barrier is
// needed.
//
// Pipeline, per block n (two barriers):
//   A: issue the global loads of block n+1 into registers; MFMA work of
//      block n from LDS; block n+1 statistics from the loaded registers;
//      the wave's partial output -> LDS.
//   B: reduce the partial outputs -> workspace; scales of block n+1; convert
//      and stage block n+1 into LDS.
//
// Grid: B*H x P_a x 4 workgroups (P_a = 64 / (NW*AW)), NW*64 threads each.
#include "common.h"
#include "launch.h"

namespace ssd {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int DH = 64;
constexpr int CW = 16;      // value columns per workgroup
constexpr int PH = DH + 8;  // fp16 row pitch (elements): 144 B
constexpr int PF = BLK + 4; // fp32 row pitch (elements)
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

template <int NW, int AW>
__global__ __launch_bounds__(NW * 64) void k_o2_state(const uint16_t* __restrict__ q,
                                                      const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v,
                                                      const float* __restrict__ dt,
                                                      const float* __restrict__ a_cs, int64_t BH,
                                                      int64_t N, int64_t chunk,
                                                      float* __restrict__ part,
                                                      float* __restrict__ final_state) {
  constexpr int NT = NW * WAVE;       // threads
  constexpr int SL = NW * AW;         // a values per workgroup
  constexpr int PA = DH / SL;         // a-slices per head
  constexpr int QKV = BLK * DH / 8;   // 16-byte q (or k) segments per block
  constexpr int QPT = QKV / NT;       // per thread
  constexpr int VPT = BLK * CW / NT;  // v elements per thread
  static_assert(QKV % NT == 0 && (BLK * CW) % NT == 0 && VPT >= 1, "thread mapping");
  static_assert(DH % SL == 0, "slice");

  __shared__ __attribute__((aligned(16))) _Float16 Qh[BLK * PH];  // [i][b] q 2^tau
  __shared__ __attribute__((aligned(16))) _Float16 KTh[DH * PH];  // [b][j] k 2^kap
  __shared__ __attribute__((aligned(16))) float VT[CW * PF];      // [c][j] v dt
  __shared__ __attribute__((aligned(16))) _Float16 Ka[SL * PH];   // [a][j] k_ja 2^kap
  __shared__ __attribute__((aligned(16))) float Qa[SL * PF];      // [a][i] q_ia e^{cs_i}
  __shared__ __attribute__((aligned(16))) float red[NW * 16 * WAVE];
  __shared__ float wv[BLK];        // w_j of the staged block
  __shared__ float st_csl[BLK];    // block-local cumsum of the next block
  __shared__ float st_dt[BLK];     // dt of the next block (1 without dt)
  __shared__ float st_vmax[BLK];   // max_{c in slice} |v_jc|
  __shared__ float st_qw[NW], st_kw[NW];

  const int tid = threadIdx.x;
  const int wave = tid / WAVE, lane = tid & (WAVE - 1), n = lane & 15, g = lane >> 4;
  const int pc = blockIdx.x & 3;
  const int pa = (blockIdx.x >> 2) % PA;
  const int64_t bh = (blockIdx.x >> 2) / PA;
  const int a0 = pa * SL;
  const int c0 = pc * CW;
  const int64_t row = bh * N;
  const int64_t nblk = n_blocks(N);

  // ---- registers holding the prefetched next block --------------------------
  uint4 pq[QPT], pk[QPT];
  uint32_t pv[(VPT + 1) / 2];
  float pcs = 0.f, pdt = 1.f, pbase = 0.f;

  auto prefetch = [&](int64_t blk) {
    const int64_t t0 = blk * BLK;
    const int nv = (int)((N - t0) < BLK ? (N - t0) : BLK);
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int s = tid + u * NT, j = s >> 3, seg = s & 7;
      pq[u] = make_uint4(0, 0, 0, 0);
      pk[u] = make_uint4(0, 0, 0, 0);
      if (j < nv) {
        pq[u] = *reinterpret_cast<const uint4*>(q + (row + t0 + j) * DH + seg * 8);
        pk[u] = *reinterpret_cast<const uint4*>(k + (row + t0 + j) * DH + seg * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; u += 2) {
      // two consecutive columns of one row per 32-bit load
      const int e = (tid + (u / 2) * NT) * 2, j = e / CW, c = e - (e / CW) * CW;
      pv[u / 2] = 0;
      if (j < nv) pv[u / 2] = *reinterpret_cast<const uint32_t*>(v + (row + t0 + j) * DH + c0 + c);
    }
    if (tid < BLK) {
      pcs = 0.f;
      pdt = 1.f;
      if (tid < nv) {
        pcs = a_cs[row + t0 + tid];
        if (dt) pdt = dt[row + t0 + tid];
      }
    }
    if (tid == 0) pbase = (t0 % chunk == 0) ? 0.f : a_cs[row + t0 - 1];
  };

  // statistics of the prefetched block -> LDS (waits for the loads)
  auto stats = [&](int64_t blk) {
    const int64_t t0 = blk * BLK;
    const int nv = (int)((N - t0) < BLK ? (N - t0) : BLK);
    float qm = 0.f, km = 0.f;
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const float qr = max8_abs_bf16(pq[u]);
      const float kr = max8_abs_bf16(pk[u]);
      qm = fmaxf(qm, qr);
      km = fmaxf(km, kr);
    }
    qm = wave_max(qm);
    km = wave_max(km);
    if (lane == 0) {
      st_qw[wave] = qm;
      st_kw[wave] = km;
    }
#pragma unroll
    for (int u = 0; u < VPT; u += 2) {
      const int e = (tid + (u / 2) * NT) * 2, j = e / CW;
      float vm = fmaxf(fabsf(bf16_lo(pv[u / 2])), fabsf(bf16_hi(pv[u / 2])));
      // CW/2 = 8 consecutive threads hold one row's slice
      vm = fmaxf(vm, __shfl_xor(vm, 1, WAVE));
      vm = fmaxf(vm, __shfl_xor(vm, 2, WAVE));
      vm = fmaxf(vm, __shfl_xor(vm, 4, WAVE));
      if ((e & (CW - 1)) == 0) st_vmax[j] = vm;
    }
    if (tid < BLK) {
      const float base = __shfl(pbase, 0, WAVE);  // thread 0 is in wave 0, as are tid < 64
      st_csl[tid] = tid < nv ? pcs - base : 0.f;
      st_dt[tid] = pdt;
    }
  };

  // scale state, identical in every wave
  int sig = 0;      // S is held as S * 2^sig
  int shift = 0;    // pending rescale of the held state (applied before use)
  int tau = 0, kap = 0;
  float eT = 1.f;
  float M = 0.f;    // upper bound of max |S| (true units)

  // every wave: decide the scales of the staged block; then every thread
  // converts its prefetched registers into the LDS staging buffers
  auto prepare = [&](int64_t blk) {
    const int64_t t0 = blk * BLK;
    const int nv = (int)((N - t0) < BLK ? (N - t0) : BLK);
    const float T = st_csl[nv - 1];
    eT = expf(T);
    float qmax = 0.f, kmax = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      qmax = fmaxf(qmax, st_qw[w]);
      kmax = fmaxf(kmax, st_kw[w]);
    }
    tau = clampi(13 - exp_ceil(qmax), -EXP_CLAMP, EXP_CLAMP);
    kap = clampi(-exp_ceil(kmax), -EXP_CLAMP, EXP_CLAMP);
    // bound of this block's contribution, one token per lane.  It uses the
    // block-wide max|k| (not each token's own): then also every update operand
    // X_j 2^(sig - 2 kap) < 4 w_j max|v_j dt_j| max|k|^2 2^sig <= 4 M 2^sig <= 2^15
    // stays inside fp16's range.
    const float wj = lane < nv ? expf(T - st_csl[lane]) : 0.f;
    const float delta = wave_sum(wj * st_vmax[lane] * fabsf(st_dt[lane])) * (kmax * kmax);
    const float m_after = eT * M + delta;
    const float mh = fmaxf(M, m_after);
    if (mh > 0.f && isfinite(mh)) {
      const int target = clampi(13 - exp_ceil(mh), -EXP_CLAMP, EXP_CLAMP);
      if (sig > target || sig < target - 12) {
        shift += target - sig;
        sig = target;
      }
    }
    M = m_after;

    const float sq = ldexpf(1.f, tau), sk = ldexpf(1.f, kap);
#pragma unroll
    for (int u = 0; u < QPT; ++u) {
      const int s = tid + u * NT, j = s >> 3, seg = s & 7;
      const uint32_t qw[4] = {pq[u].x, pq[u].y, pq[u].z, pq[u].w};
      const uint32_t kw[4] = {pk[u].x, pk[u].y, pk[u].z, pk[u].w};
      f16x8 qh;
      float kf[8], qf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[2 * i] = bf16_lo(qw[i]);
        qf[2 * i + 1] = bf16_hi(qw[i]);
        kf[2 * i] = bf16_lo(kw[i]);
        kf[2 * i + 1] = bf16_hi(kw[i]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qh[i] = (_Float16)(qf[i] * sq);
        KTh[(seg * 8 + i) * PH + j] = (_Float16)(kf[i] * sk);
      }
      *reinterpret_cast<f16x8*>(&Qh[j * PH + seg * 8]) = qh;
      const float ecs = expf(st_csl[j]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int al = seg * 8 + i - a0;
        if (al >= 0 && al < SL) {
          Ka[al * PH + j] = (_Float16)(kf[i] * sk);
          Qa[al * PF + j] = qf[i] * ecs;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < VPT; u += 2) {
      const int e = (tid + (u / 2) * NT) * 2, j = e / CW, c = e - (e / CW) * CW;
      const float d = st_dt[j];
      VT[c * PF + j] = bf16_lo(pv[u / 2]) * d;
      VT[(c + 1) * PF + j] = bf16_hi(pv[u / 2]) * d;
    }
    if (tid < BLK) wv[tid] = tid < nv ? expf(T - st_csl[tid]) : 0.f;
  };

  f32x4 S[AW][4];
#pragma unroll
  for (int ai = 0; ai < AW; ++ai)
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) S[ai][bt] = zero4();

  // prologue
  prefetch(0);
  stats(0);
  __syncthreads();
  prepare(0);
  __syncthreads();

  for (int64_t blk = 0; blk < nblk; ++blk) {
    const int64_t t0 = blk * BLK;
    const int nv = (int)((N - t0) < BLK ? (N - t0) : BLK);
    const bool more = blk + 1 < nblk;
    if (more) prefetch(blk + 1);

    // ---- phase A: MFMA work of block blk ------------------------------------
    if (shift != 0) {
      const float f = ldexpf(1.f, shift);
#pragma unroll
      for (int ai = 0; ai < AW; ++ai)
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) S[ai][bt] *= f;
      shift = 0;
    }
    // output pass over this wave's a values, with the entering state:
    // T^T[c][i] = sum_b S[b][c] Q[i][b];  Y[i][c] += qe_ia T^T[c][i]
    {
      f16x8 Qf[4][2];  // B operand: Q^T[b][i], permuted k = b
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const _Float16* p = &Qh[(it * 16 + n) * PH + kb * 32 + 4 * g];
          const f16x4 lo = *reinterpret_cast<const f16x4*>(p);
          const f16x4 hi = *reinterpret_cast<const f16x4*>(p + 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            Qf[it][kb][r] = lo[r];
            Qf[it][kb][4 + r] = hi[r];
          }
        }
      f32x4 Y[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) Y[it] = zero4();
#pragma unroll
      for (int ai = 0; ai < AW; ++ai) {
        const int al = wave * AW + ai;
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
          Y[it] += Qa[al * PF + it * 16 + n] * T;
        }
      }
      const float ys = ldexpf(1.f, -sig) * ldexpf(1.f, -tau);
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(wave * 16 + it * 4 + r) * WAVE + lane] = Y[it][r] * ys;
    }

    // update pass: S = e^T S + K^T ((k_:a 2^kap) * X)
    {
      f16x8 Kf[4][2];  // A operand: K^T[b][j], k = j contiguous
#pragma unroll
      for (int bt = 0; bt < 4; ++bt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          Kf[bt][kb] = *reinterpret_cast<const f16x8*>(&KTh[(bt * 16 + n) * PH + kb * 32 + 8 * g]);
      const float sx = ldexpf(1.f, sig) * ldexpf(ldexpf(1.f, -kap), -kap);
      f16x8 xh[2];  // X_jc 2^(sig - 2 kap) for this lane's column c = n
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int j = kb * 32 + 8 * g + s;
          xh[kb][s] = (_Float16)(VT[n * PF + j] * wv[j] * sx);
        }
#pragma unroll
      for (int ai = 0; ai < AW; ++ai) {
        const int al = wave * AW + ai;
        f16x8 Bu[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          Bu[kb] = *reinterpret_cast<const f16x8*>(&Ka[al * PH + kb * 32 + 8 * g]) * xh[kb];
#pragma unroll
        for (int bt = 0; bt < 4; ++bt) {
          f32x4 acc = eT * S[ai][bt];
          acc = mfma_f16(Kf[bt][0], Bu[0], acc);
          acc = mfma_f16(Kf[bt][1], Bu[1], acc);
          S[ai][bt] = acc;
        }
      }
    }

    if (more) stats(blk + 1);
    __syncthreads();

    // ---- phase B: partial output of block blk; stage block blk+1 -----------
    for (int o = tid; o < 16 * WAVE; o += NT) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w * 16 * WAVE + o];
      const int reg = o / WAVE, ln = o - (o / WAVE) * WAVE;
      const int it = reg >> 2, r = reg & 3;
      const int i = it * 16 + (ln & 15), c = 4 * (ln >> 4) + r;
      if (i < nv) part[(((int64_t)pa * BH + bh) * N + t0 + i) * DH + c0 + c] = s;
    }
    if (more) prepare(blk + 1);
    __syncthreads();
  }

  if (final_state) {
    const float f = ldexpf(1.f, -sig);
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

hipError_t launch_o2_state(const void* q, const void* k, const void* v, const float* dt,
                           const float* a_cs, int64_t BH, int64_t N, int64_t chunk, float* part,
                           float* final_state, hipStream_t stream) {
  constexpr int NW = 8;
  const int AW = o2_aw(BH);
  const int PA = o2_pa(BH);
  const dim3 grid((unsigned)(BH * PA * 4)), blk(NW * WAVE);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  if (AW == 4)
    hipLaunchKernelGGL((k_o2_state<NW, 4>), grid, blk, 0, stream, qq, kk, vv, dt, a_cs, BH, N, chunk, part, final_state);
  else if (AW == 2)
    hipLaunchKernelGGL((k_o2_state<NW, 2>), grid, blk, 0, stream, qq, kk, vv, dt, a_cs, BH, N, chunk, part, final_state);
  else
    hipLaunchKernelGGL((k_o2_state<NW, 1>), grid, blk, 0, stream, qq, kk, vv, dt, a_cs, BH, N, chunk, part, final_state);
  return hipGetLastError();
}

}  // namespace ssd
