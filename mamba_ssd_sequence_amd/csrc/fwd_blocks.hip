// Block-parallel pieces of the chunked forward (both orders), 64-token blocks.
//
//   k_chunk_state : per block, the state contribution sum_j w_j k_j val_j^T
//                   and sum_j w_j k_j, w_j = exp(A^CS_last - A^CS_j)
//                   (Algorithm 6's update summed over one block; MFMA).
//   k_state_pass  : exclusive scan over blocks, S <- exp(T_blk) S + dS, in
//                   place, so each block slot ends up holding the state that
//                   enters it (elementwise, one thread per state entry).
//   k_output      : the masked product within the block (Algorithms 1, 4, 5:
//                   w_ij = (q_i.k_j)^p exp(A^CS_i - A^CS_j), j <= i), plus the
//                   inter-block part exp(A^CS_i - A^CS_start) phi(q_i)^T S_in,
//                   then y = num / den (Algorithm 1's row-sum normaliser).
//
// The decays are exponentials of non-positive differences of chunk-local
// cumsums only (mask first, then exp).
//
// MFMA use: bf16 inputs run v_mfma_f32_16x16x32_bf16 (bf16 operands, fp32
// accumulate); fp32 inputs run v_mfma_f32_16x16x4_f32 so that fp32 mode stays
// fp32 throughout.  Each wave of the output kernel owns one 16-row tile of
// queries; the score tile is produced transposed (K Q^T) so its accumulator
// layout is directly the B operand of the (scores * mask) x V product.
#include "common.h"
#include "launch.h"

namespace ssd {

template <bool BF> struct Cfg;
template <> struct Cfg<true> {
  using C = __bf16;        // operand type staged in LDS
  using St = uint16_t;     // storage type of q/k/v in HBM
  using F = bf16x8;        // MFMA operand fragment
  static constexpr int KS = 32;   // k per MFMA
  static constexpr int PAD = 8;   // LDS row padding (elements)
  static __device__ __forceinline__ F ld(const C* M, int P, int row, int ks, int g) {
    return *reinterpret_cast<const bf16x8*>(&M[row * P + ks * 32 + 8 * g]);
  }
  static __device__ __forceinline__ f32x4 mma(const F& a, const F& b, const f32x4& c) {
    return mfma_bf16(a, b, c);
  }
};
template <> struct Cfg<false> {
  using C = float;
  using St = float;
  using F = float;
  static constexpr int KS = 4;
  static constexpr int PAD = 4;
  static __device__ __forceinline__ F ld(const C* M, int P, int row, int ks, int g) {
    return M[row * P + ks * 4 + g];
  }
  static __device__ __forceinline__ f32x4 mma(const F& a, const F& b, const f32x4& c) {
    return mfma_f32(a, b, c);
  }
};

// ---------------------------------------------------------------------------
// k_chunk_state
// ---------------------------------------------------------------------------
template <bool BF, int DH>  // (fp32 inputs; BF is false)
__global__ __launch_bounds__(256) void k_chunk_state_f32(const void* __restrict__ kp,
                                                     const void* __restrict__ vp,
                                                     const float* __restrict__ dt,
                                                     const float* __restrict__ a_cs, int64_t N,
                                                     int64_t chunk, int64_t nblk,
                                                     float* __restrict__ tb,
                                                     float* __restrict__ state) {
  using G = Cfg<BF>;
  using C = typename G::C;
  using St = typename G::St;
  constexpr int P = BLK + G::PAD;
  __shared__ __attribute__((aligned(16))) C wKT[DH * P];  // [b][j] = w_j k_jb (bf16: high part)
  __shared__ __attribute__((aligned(16))) C wKL[BF ? DH * P : 1];  // bf16: w_j k_jb - high part
  __shared__ __attribute__((aligned(16))) C VT[DH * P];   // [c][j] = val_jc
  __shared__ float wv[BLK];
  __shared__ float dtv[BLK];

  const St* k = static_cast<const St*>(kp);
  const St* v = static_cast<const St*>(vp);
  const int64_t bh = blockIdx.x / nblk, blk = blockIdx.x - bh * nblk;
  const int64_t t0 = blk * BLK;
  const int nvalid = (int)((N - t0) < BLK ? (N - t0) : BLK);
  const int64_t row = bh * N;
  const int tid = threadIdx.x;

  const float base = (t0 % chunk == 0) ? 0.f : a_cs[row + t0 - 1];
  const float cs_last = a_cs[row + t0 + nvalid - 1];
  if (tid < BLK) {
    float w = 0.f, d = 0.f;
    if (tid < nvalid) {
      w = expf(cs_last - a_cs[row + t0 + tid]);
      d = dt ? dt[row + t0 + tid] : 1.f;
    }
    wv[tid] = w;
    dtv[tid] = d;
  }
  if (tid == 0) tb[bh * nblk + blk] = cs_last - base;
  __syncthreads();

  for (int e = tid; e < BLK * DH; e += 256) {
    const int j = e / DH, d = e - (e / DH) * DH;
    float kv = 0.f, vv = 0.f;
    if (j < nvalid) {
      kv = Elem<St>::ld(k, (row + t0 + j) * DH + d);
      vv = Elem<St>::ld(v, (row + t0 + j) * DH + d);
    }
    const float wk = wv[j] * kv;
    const C hi = (C)wk;
    wKT[d * P + j] = hi;
    if constexpr (BF) wKL[d * P + j] = (C)(wk - (float)hi);
    VT[d * P + j] = (C)(vv * dtv[j]);
  }
  __syncthreads();

  const int wave = tid / WAVE, lane = tid & (WAVE - 1), n = lane & 15, g = lane >> 4;
  constexpr int NT = DH / 16;
  float* out = state + (bh * nblk + blk) * (int64_t)(DH * DH + DH);
  // bf16 operands: w*k is split into high + low bf16 parts (two products), so
  // the state keeps ~16 significant bits of each weighted key; the value
  // operand is used as rounded once.
  for (int tile = wave; tile < NT * NT; tile += 4) {
    const int ct = tile / NT, bt = tile - (tile / NT) * NT;
    f32x4 acc = zero4();
#pragma unroll
    for (int ks = 0; ks < BLK / G::KS; ++ks) {
      const auto a = G::ld(VT, P, ct * 16 + n, ks, g);
      acc = G::mma(a, G::ld(wKT, P, bt * 16 + n, ks, g), acc);
      if constexpr (BF) acc = G::mma(a, G::ld(wKL, P, bt * 16 + n, ks, g), acc);
    }
    // acc[r] = dS^T[c = 16ct + 4g + r][b = 16bt + n]  ->  dS[b][c]
    *reinterpret_cast<f32x4*>(&out[(bt * 16 + n) * DH + ct * 16 + 4 * g]) = acc;
  }
  if (tid < DH) {
    float s = 0.f;
    for (int j = 0; j < BLK; ++j) {
      s += (float)wKT[tid * P + j];
      if constexpr (BF) s += (float)wKL[tid * P + j];
    }
    out[DH * DH + tid] = s;
  }
}

// bf16 inputs: one memory round trip (q is not needed; k and v segments of
// two consecutive tokens per thread are loaded before anything else), k^T and
// (v dt)^T staged in LDS with transposing 4-byte stores (a token pair per
// store), and the weighted-key operand (w k)^T formed in registers: wave w
// takes the column tile b in [16 w, 16 w + 16) of every row tile c, so its
// operand fragments are those of one b-tile, split into high + low bf16
// parts; z = sum_j w_j k_j comes from the same fp32 products.
template <int DH>
__global__ __launch_bounds__(256) void k_chunk_state_bf16(const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const float* __restrict__ dt,
                                                          const float* __restrict__ a_cs,
                                                          int64_t N, int64_t chunk, int64_t nblk,
                                                          float* __restrict__ tb,
                                                          float* __restrict__ state) {
  constexpr int P = BLK + 8;         // LDS row pitch (bf16 elements)
  constexpr int SEG = DH / 8;        // 16-byte segments per row
  static_assert(BLK * SEG / 2 == 256 || BLK * SEG / 2 == 128, "segment mapping");
  constexpr int NT = DH / 16;
  static_assert(NT <= 4, "one b-tile per wave");
  __shared__ __attribute__((aligned(16))) __bf16 KT[DH * P];  // [b][j] k_jb
  __shared__ __attribute__((aligned(16))) __bf16 VT[DH * P];  // [c][j] v_jc dt_j
  __shared__ float wv[BLK];

  const int64_t bh = blockIdx.x / nblk, blk = blockIdx.x - bh * nblk;
  const int64_t t0 = blk * BLK;
  const int nvalid = (int)((N - t0) < BLK ? (N - t0) : BLK);
  const int64_t row = bh * N;
  const int tid = threadIdx.x;

  // reads, all issued up front; rows past a ragged block's end read the
  // last valid row (zeroed below: no load under a lane-divergent branch)
  const bool act = tid < BLK * SEG / 2;  // thread -> (token pair, segment)
  const int pr = (tid / SEG) % (BLK / 2), sg = tid % SEG, j0 = 2 * pr;
  const int r0 = min(j0, nvalid - 1), r1 = min(j0 + 1, nvalid - 1);
  const uint4 k0 = *reinterpret_cast<const uint4*>(k + (row + t0 + r0) * DH + sg * 8);
  const uint4 k1 = *reinterpret_cast<const uint4*>(k + (row + t0 + r1) * DH + sg * 8);
  const uint4 v0 = *reinterpret_cast<const uint4*>(v + (row + t0 + r0) * DH + sg * 8);
  const uint4 v1 = *reinterpret_cast<const uint4*>(v + (row + t0 + r1) * DH + sg * 8);
  const float d0 = dt ? dt[row + t0 + r0] : 1.f, d1 = dt ? dt[row + t0 + r1] : 1.f;
  const int ja = min(tid & (BLK - 1), nvalid - 1);
  const float acs = a_cs[row + t0 + ja];
  const float base = (t0 % chunk == 0) ? 0.f : a_cs[row + t0 - 1];
  const float cs_last = a_cs[row + t0 + nvalid - 1];

  if (tid < BLK) wv[tid] = tid < nvalid ? expf(cs_last - acs) : 0.f;
  if (tid == 0) tb[bh * nblk + blk] = cs_last - base;
  if (act) {
    const bool ok0 = j0 < nvalid, ok1 = j0 + 1 < nvalid;
    const uint4 ka = keep_if(ok0, k0), kb = keep_if(ok1, k1);
    const uint4 va = keep_if(ok0, v0), vb = keep_if(ok1, v1);
    const uint32_t kw0[4] = {ka.x, ka.y, ka.z, ka.w}, kw1[4] = {kb.x, kb.y, kb.z, kb.w};
    const uint32_t vw0[4] = {va.x, va.y, va.z, va.w}, vw1[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int d = sg * 8 + 2 * u + hh;
        const uint32_t kb0 = hh ? (kw0[u] >> 16) : (kw0[u] & 0xffffu);
        const uint32_t kb1 = hh ? (kw1[u] >> 16) : (kw1[u] & 0xffffu);
        *reinterpret_cast<uint32_t*>(&KT[d * P + j0]) = kb0 | (kb1 << 16);
        const float a0 = __uint_as_float(hh ? (vw0[u] & 0xffff0000u) : (vw0[u] << 16)) * d0;
        const float a1 = __uint_as_float(hh ? (vw1[u] & 0xffff0000u) : (vw1[u] << 16)) * d1;
        const __bf16 pv[2] = {(__bf16)a0, (__bf16)a1};
        *reinterpret_cast<uint32_t*>(&VT[d * P + j0]) = __builtin_bit_cast(uint32_t, pv);
      }
  }
  __syncthreads();

  const int wave = tid / WAVE, lane = tid & (WAVE - 1), n = lane & 15, g = lane >> 4;
  float* out = state + (bh * nblk + blk) * (int64_t)(DH * DH + DH);
  if (wave < NT) {
    const int bt = wave;
    // B operand (w k)^T[b = 16 bt + n][j = 32 ks + 8 g ..]: high + low parts;
    // z_b from the fp32 products
    bf16x8 bhi[BLK / 32], blo[BLK / 32];
    float zp = 0.f;
#pragma unroll
    for (int ks = 0; ks < BLK / 32; ++ks) {
      const bf16x8 kr = *reinterpret_cast<const bf16x8*>(&KT[(bt * 16 + n) * P + ks * 32 + 8 * g]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wk = (float)kr[e] * wv[ks * 32 + 8 * g + e];
        const __bf16 h = (__bf16)wk;
        bhi[ks][e] = h;
        blo[ks][e] = (__bf16)(wk - (float)h);
        zp += wk;
      }
    }
    zp = sum_over_groups(zp);
    if (g == 0) out[DH * DH + bt * 16 + n] = zp;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < BLK / 32; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&VT[(ct * 16 + n) * P + ks * 32 + 8 * g]);
        acc = mfma_bf16(a, bhi[ks], acc);
        acc = mfma_bf16(a, blo[ks], acc);
      }
      // acc[r] = dS^T[c = 16 ct + 4 g + r][b = 16 bt + n] -> dS[b][c]
      *reinterpret_cast<f32x4*>(&out[(bt * 16 + n) * DH + ct * 16 + 4 * g]) = acc;
    }
  }
}

hipError_t launch_chunk_state(bool bf16, int64_t DH, const void* k, const void* v, const float* dt,
                              const float* a_cs, int64_t BH, int64_t N, int64_t chunk, float* tb,
                              float* state, hipStream_t stream) {
  const int64_t nb = n_blocks(N);
  const dim3 grid((unsigned)(BH * nb)), blk(256);
  const uint16_t* kb = static_cast<const uint16_t*>(k);
  const uint16_t* vb = static_cast<const uint16_t*>(v);
  if (bf16 && DH == 64)
    hipLaunchKernelGGL((k_chunk_state_bf16<64>), grid, blk, 0, stream, kb, vb, dt, a_cs, N, chunk, nb, tb, state);
  else if (bf16 && DH == 32)
    hipLaunchKernelGGL((k_chunk_state_bf16<32>), grid, blk, 0, stream, kb, vb, dt, a_cs, N, chunk, nb, tb, state);
  else if (!bf16 && DH == 64)
    hipLaunchKernelGGL((k_chunk_state_f32<false, 64>), grid, blk, 0, stream, k, v, dt, a_cs, N, chunk, nb, tb, state);
  else
    hipLaunchKernelGGL((k_chunk_state_f32<false, 32>), grid, blk, 0, stream, k, v, dt, a_cs, N, chunk, nb, tb, state);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k_state_pass
// ---------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(256) void k_state_pass(int64_t nblk, int eblocks,
                                                    const float* __restrict__ tb,
                                                    float* __restrict__ state,
                                                    float* __restrict__ fS,
                                                    float* __restrict__ fz,
                                                    const float* __restrict__ iS,
                                                    const float* __restrict__ iz) {
  constexpr int E = DH * DH + DH;
  const int64_t bh = blockIdx.x / eblocks;
  const int e = (int)(blockIdx.x - bh * eblocks) * 256 + threadIdx.x;
  if (e >= E) return;
  float* p = state + bh * nblk * E + e;
  const float* t = tb + bh * nblk;
  // the state before the first block: zero, or the caller's initial state
  // (same entry order as the final state: S row-major, then z)
  float s = 0.f;
  if (iS) s = e < DH * DH ? iS[bh * DH * DH + e] : iz[bh * DH + (e - DH * DH)];
  int64_t b = 0;
  // 32 blocks' loads in flight per thread: the scan is latency-bound
  // otherwise (one state entry per thread, a strided walk over the blocks)
  constexpr int U = 32;
  for (; b + U <= nblk; b += U) {
    float d[U], T[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      d[u] = p[(b + u) * E];
      T[u] = t[b + u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[(b + u) * E] = s;
      s = expf(T[u]) * s + d[u];
    }
  }
  for (; b < nblk; ++b) {
    const float d = p[b * E];
    const float T = t[b];
    p[b * E] = s;
    s = expf(T) * s + d;
  }
  if (e < DH * DH) {
    if (fS) fS[bh * DH * DH + e] = s;
  } else {
    if (fz) fz[bh * DH + (e - DH * DH)] = s;
  }
}

hipError_t launch_state_pass(int64_t DH, int64_t BH, int64_t N, const float* tb, float* state,
                             float* final_S, float* final_z, const float* init_S,
                             const float* init_z, hipStream_t stream) {
  const int64_t nb = n_blocks(N);
  const int E = (int)(DH * DH + DH);
  const int eblocks = (E + 255) / 256;
  const dim3 grid((unsigned)(BH * eblocks)), blk(256);
  if (DH == 64)
    hipLaunchKernelGGL(k_state_pass<64>, grid, blk, 0, stream, nb, eblocks, tb, state, final_S, final_z,
                       init_S, init_z);
  else
    hipLaunchKernelGGL(k_state_pass<32>, grid, blk, 0, stream, nb, eblocks, tb, state, final_S, final_z,
                       init_S, init_z);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// k_output
// ---------------------------------------------------------------------------
// (registers capped for five waves per SIMD where the LDS allows five
// workgroups per CU: order 2 (29 KB) and order 1 with bf16 inputs (28 KB);
// the fp32 variants are bound by LDS)
template <bool BF, int DH, int ORDER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BF ? 5 : 1, 8))) void k_output(const void* __restrict__ qp,
                                                const void* __restrict__ kp,
                                                const void* __restrict__ vp,
                                                const float* __restrict__ dt,
                                                const float* __restrict__ a_cs, int64_t BH,
                                                int64_t N, int64_t chunk, int64_t nblk,
                                                const float* __restrict__ state,
                                                const float* __restrict__ part,
                                                float* __restrict__ y, float* __restrict__ den) {
  using G = Cfg<BF>;
  using C = typename G::C;
  using St = typename G::St;
  constexpr int PQ = DH + G::PAD;   // pitch of rows indexed by feature
  constexpr int PJ = BLK + G::PAD;  // pitch of rows indexed by token
  constexpr int NT = DH / 16;
  // Order 1 with bf16 inputs (SPLIT): the entering state, in high and low
  // bf16 parts, is staged first in the space that k and v take afterwards
  // (the inter-block product runs in between), which keeps the workgroup at
  // 28 KB of LDS; fp32 inputs stage it in an array of its own; order 2 reads
  // its rows into registers.
  constexpr bool SPLIT = ORDER == 1 && BF;
  static_assert(!SPLIT || 2 * DH * PQ <= BLK * PQ + DH * PJ, "state fits the k / v space");
  __shared__ __attribute__((aligned(16))) C Qs[BLK * PQ];   // [i][d]
  __shared__ __attribute__((aligned(16))) C KV[BLK * PQ + DH * PJ];
  __shared__ __attribute__((aligned(16))) C SinX[ORDER == 1 && !SPLIT ? DH * PQ : 1];
  C* const Ks = KV;               // [j][d]
  C* const VT = KV + BLK * PQ;    // [c][j]  value operand, transposed
  C* const SinT = SPLIT ? KV : SinX;  // [c][b] the entering state, transposed (bf16: high part)
  C* const SinL = KV + DH * PQ;   // [c][b] SPLIT: low part
  __shared__ float dred[ORDER == 2 ? 4 * BLK : 1];  // order 2: per-wave parts of q^T Z q
  __shared__ float zin[DH];
  __shared__ float csl[BLK];
  __shared__ float dtv[BLK];

  const St* q = static_cast<const St*>(qp);
  const St* k = static_cast<const St*>(kp);
  const St* v = static_cast<const St*>(vp);
  int64_t bh, blk;
  if constexpr (ORDER == 2 && BF) {
    // the two blocks of a step (2m, 2m + 1) go to workgroups 8 apart, i.e. to
    // the same XCD (workgroups are dispatched round-robin over the 8 XCDs),
    // so that the second block's read of the first block's k and v (its
    // direct term) finds them in that XCD's L2
    const int64_t np = (nblk + 1) / 2, xcd = blockIdx.x & 7, s8 = blockIdx.x >> 3;
    const int64_t P = 8 * (s8 >> 1) + xcd;  // (head, step) pair index
    if (P >= BH * np) return;
    bh = P / np;
    blk = 2 * (P - bh * np) + (s8 & 1);
    if (blk >= nblk) return;  // the empty second block of a last step
  } else {
    bh = blockIdx.x / nblk;
    blk = blockIdx.x - bh * nblk;
  }
  const int64_t t0 = blk * BLK;
  const int nvalid = (int)((N - t0) < BLK ? (N - t0) : BLK);
  const int64_t row = bh * N;
  const int tid = threadIdx.x;

  // Every global read of the block is issued here, before the first barrier,
  // so that a block costs one memory round trip: the block's cumsum and dt,
  // q / k / v (bf16), the entering state, and at order 2 the inter-block
  // partials of this thread's query row and the partner block (below).
  // Decays are exp2 of differences of cumsums kept in log2 units (cs log2 e).
  const float base = (t0 % chunk == 0) ? 0.f : a_cs[row + t0 - 1];
  float c_own = 0.f, d_own = 0.f;
  if (tid < nvalid) {  // tid < BLK
    c_own = (a_cs[row + t0 + tid] - base) * LOG2E;
    d_own = dt ? dt[row + t0 + tid] : 1.f;
  }
  const int it = tid / WAVE, lane = tid & (WAVE - 1), n = lane & 15, g = lane >> 4;
  const int il = it * 16 + n;  // this lane's query row within the block

  // bf16: q and k rows as 16-byte segments (segment e % SEG of row e / SEG
  // for e = tid, tid + 256), v as the same segment of the token pair
  // 2 (tid / SEG), + 1, with the two tokens' dt
  constexpr int SEG = DH / 8;
  constexpr int NQ = BF ? BLK * SEG / 256 : 1;
  static_assert(!BF || ((NQ == 1 || NQ == 2) && (BLK / 2) * SEG <= 256), "segment mapping");
  uint4 gq0 = make_uint4(0, 0, 0, 0), gk0 = gq0, gq1 = gq0, gk1 = gq0, gv0 = gq0, gv1 = gq0;
  float gd0 = 0.f, gd1 = 0.f;
  if constexpr (BF) {
    const uint16_t* qb = static_cast<const uint16_t*>(qp) + (row + t0) * DH;
    const uint16_t* kb = static_cast<const uint16_t*>(kp) + (row + t0) * DH;
    const uint16_t* vb = static_cast<const uint16_t*>(vp) + (row + t0) * DH;
    {
      const int j = tid / SEG, sg = tid % SEG;
      if (j < nvalid) {
        gq0 = *reinterpret_cast<const uint4*>(qb + j * DH + sg * 8);
        gk0 = *reinterpret_cast<const uint4*>(kb + j * DH + sg * 8);
      }
    }
    if constexpr (NQ == 2) {
      const int j = (tid + 256) / SEG, sg = tid % SEG;
      if (j < nvalid) {
        gq1 = *reinterpret_cast<const uint4*>(qb + j * DH + sg * 8);
        gk1 = *reinterpret_cast<const uint4*>(kb + j * DH + sg * 8);
      }
    }
    if (tid < (BLK / 2) * SEG) {
      const int j0 = 2 * (tid / SEG), sg = tid % SEG;
      if (j0 < nvalid) {
        gv0 = *reinterpret_cast<const uint4*>(vb + j0 * DH + sg * 8);
        gd0 = dt ? dt[row + t0 + j0] : 1.f;
      }
      if (j0 + 1 < nvalid) {
        gv1 = *reinterpret_cast<const uint4*>(vb + (j0 + 1) * DH + sg * 8);
        gd1 = dt ? dt[row + t0 + j0 + 1] : 1.f;
      }
    }
  }
  // entering state: order 1, DH * DH floats as float4 (element 4 e4 .. of
  // the block slot for e4 = tid + 256 u) and the d_h normaliser entries;
  // order 2, the normaliser state Z (symmetric, upper 16 x 16 tiles stored):
  // wave it takes the rows b of tile it, lane (n, g) the 8 entries c = 32 ks
  // + 8 g .. of row 16 it + n, from tile ct = c / 16 when ct >= it (the A
  // operand of (Z' Q^T) with Z' the upper tiles of Z, off-diagonal ones
  // doubled: q^T Z' q = q^T Z q); lanes whose tile lies below the diagonal
  // read the diagonal tile and use 0
  // (order 2: the normaliser state entering the block's two-block step, which
  // the state scan leaves in the slot of the step's first block; the second
  // block adds the first block's share from its direct term below)
  const int64_t zslot = (ORDER == 2 && BF) ? (blk & ~(int64_t)1) : blk;
  const float* st = state + (bh * nblk + zslot) * (int64_t)(DH * DH + DH);
  constexpr int NS4 = DH * DH / 4 / 256;
  static_assert(NS4 * 256 * 4 == DH * DH && (ORDER == 1 || NS4 == 4), "state mapping");
  f32x4 gs[NS4];
  if constexpr (ORDER == 2) {
#pragma unroll
    for (int u = 0; u < NS4; ++u) {
      const int ct = 2 * (u >> 1) + (g >> 1), col = 8 * (g & 1) + 4 * (u & 1);
      gs[u] = *reinterpret_cast<const f32x4*>(&st[256 * z_tile(it, ct < it ? it : ct) + 16 * n + col]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < NS4; ++u) gs[u] = *reinterpret_cast<const f32x4*>(&st[4 * (tid + 256 * u)]);
  }
  float gzin = 0.f;
  if (ORDER == 1 && tid < DH) gzin = st[DH * DH + tid];
  // order 2: the inter-block numerator partials of row il (columns 16 ct +
  // 4 g ..)
  f32x4 gp[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) gp[ct] = zero4();
  if constexpr (ORDER == 2) {
    // (rows past a ragged block's end read a padding row; results unused)
    const float* pp = part + (bh * o2_part_rows(N) + t0 + il) * 64;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) gp[ct] = *reinterpret_cast<const f32x4*>(pp + ct * 16 + 4 * g);
  }

  // Order 2: the numerator scan advances over steps of two blocks and gives
  // the second block of a step only the state entering the step, so the first
  // block's tokens reach it here as a direct (unmasked) term.  Its k and v
  // rows are loaded now and staged after the block's own products.
  constexpr bool PAIRS = ORDER == 2 && BF;
  const bool partner = PAIRS && (blk & 1);
  float den_p = 0.f;  // the first block's share of the normaliser (second blocks)
  uint4 pka = make_uint4(0, 0, 0, 0), pkb = pka, pva = pka, pvb = pka;  // (registers, not an array)
  float pcs = 0.f, pdt = 0.f, pT = 0.f;
  if (PAIRS && partner) {
    const int64_t tp = t0 - BLK;  // the first block of the step (always full)
    const float base_p = (tp % chunk == 0) ? 0.f : a_cs[row + tp - 1];
    pT = (a_cs[row + tp + BLK - 1] - base_p) * LOG2E;
    if (tid < BLK) {
      pcs = (a_cs[row + tp + tid] - base_p) * LOG2E;
      pdt = dt ? dt[row + tp + tid] : 1.f;
    }
    // k: the 16-byte segment tid % 8 of rows tid / 8 and 32 + tid / 8; v: the
    // same segment of the token pair 2 (tid / 8), 2 (tid / 8) + 1
    const uint16_t* kb = static_cast<const uint16_t*>(kp) + (row + tp) * DH;
    const uint16_t* vb = static_cast<const uint16_t*>(vp) + (row + tp) * DH;
    pka = *reinterpret_cast<const uint4*>(kb + (tid >> 3) * DH + (tid & 7) * 8);
    pkb = *reinterpret_cast<const uint4*>(kb + (32 + (tid >> 3)) * DH + (tid & 7) * 8);
    pva = *reinterpret_cast<const uint4*>(vb + (2 * (tid >> 3)) * DH + (tid & 7) * 8);
    pvb = *reinterpret_cast<const uint4*>(vb + (2 * (tid >> 3) + 1) * DH + (tid & 7) * 8);
  }

  // ---- staging into LDS ---------------------------------------------------
  if (tid < BLK) {
    csl[tid] = c_own;
    dtv[tid] = d_own;
  }
  // bf16: k rows and the value operand v dt, transposed (each LDS store
  // carries a token pair)
  auto stage_kv = [&]() {
   if constexpr (BF) {
    {
      const int j = tid / SEG, sg = tid % SEG;
      *reinterpret_cast<uint4*>(&Ks[j * PQ + sg * 8]) = gk0;
    }
    if constexpr (NQ == 2) {
      const int j = (tid + 256) / SEG, sg = tid % SEG;
      *reinterpret_cast<uint4*>(&Ks[j * PQ + sg * 8]) = gk1;
    }
    if (tid < (BLK / 2) * SEG) {
      const int j0 = 2 * (tid / SEG), sg = tid % SEG;
      const uint32_t w0[4] = {gv0.x, gv0.y, gv0.z, gv0.w}, w1[4] = {gv1.x, gv1.y, gv1.z, gv1.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float a0 = __uint_as_float(hh ? (w0[u] & 0xffff0000u) : (w0[u] << 16)) * gd0;
          const float a1 = __uint_as_float(hh ? (w1[u] & 0xffff0000u) : (w1[u] << 16)) * gd1;
          C pr[2] = {(C)a0, (C)a1};
          *reinterpret_cast<uint32_t*>(&VT[(sg * 8 + 2 * u + hh) * PJ + j0]) = __builtin_bit_cast(uint32_t, pr);
        }
      }
    }
   }
  };
  if constexpr (BF) {
    {
      const int j = tid / SEG, sg = tid % SEG;
      *reinterpret_cast<uint4*>(&Qs[j * PQ + sg * 8]) = gq0;
    }
    if constexpr (NQ == 2) {
      const int j = (tid + 256) / SEG, sg = tid % SEG;
      *reinterpret_cast<uint4*>(&Qs[j * PQ + sg * 8]) = gq1;
    }
    if constexpr (!SPLIT) stage_kv();
  }
  if constexpr (ORDER == 1) {
#pragma unroll
    for (int u = 0; u < NS4; ++u) {
      const int e = 4 * (tid + 256 * u), b = e / DH, c4 = e % DH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x = gs[u][r];
        const C hi = (C)x;
        SinT[(c4 + r) * PQ + b] = hi;
        if constexpr (BF) SinL[(c4 + r) * PQ + b] = (C)(x - (float)hi);
      }
    }
  }
  if (ORDER == 1 && tid < DH) zin[tid] = gzin;
  if constexpr (!BF) {
    // fp32 inputs: element-wise staging, v scaled by dt from LDS
    __syncthreads();
    for (int e = tid; e < BLK * DH; e += 256) {
      const int j = e / DH, d = e - (e / DH) * DH;
      float qv = 0.f, kv = 0.f, vv = 0.f;
      if (j < nvalid) {
        const int64_t off = (row + t0 + j) * DH + d;
        qv = Elem<St>::ld(q, off);
        kv = Elem<St>::ld(k, off);
        vv = Elem<St>::ld(v, off);
      }
      Qs[j * PQ + d] = (C)qv;
      Ks[j * PQ + d] = (C)kv;
      VT[d * PJ + j] = (C)(vv * dtv[j]);
    }
  }
  __syncthreads();
  const float cs_i = csl[il];

  // order 1: the inter-block product D[c][i] = sum_b S_in[b][c] Q[i][b], with
  // the state in high + low bf16 parts (the factored sum over b can cancel
  // when q is nearly orthogonal to the keys, so a single bf16 rounding of the
  // state would be amplified), and the normaliser part q . z
  f32x4 inter[NT];
  float den_x = 0.f;
  auto inter_product = [&]() {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DH / G::KS; ++ks) {
        const auto b = G::ld(Qs, PQ, il, ks, g);
        acc = G::mma(G::ld(SinT, PQ, ct * 16 + n, ks, g), b, acc);
        if constexpr (BF) acc = G::mma(G::ld(SinL, PQ, ct * 16 + n, ks, g), b, acc);
      }
      inter[ct] = acc;
    }
    for (int b = g * (DH / 4); b < (g + 1) * (DH / 4); ++b) den_x += (float)Qs[il * PQ + b] * zin[b];
    den_x = sum_over_groups(den_x);
  };
  if constexpr (SPLIT) {
    inter_product();
    __syncthreads();  // the state's space is free: stage k and v there
    stage_kv();
    __syncthreads();
  }

  if constexpr (ORDER == 2) {
    // q^T Z q for all 64 rows over this wave's 16 rows b of Z': (Z' Q^T)[b][i]
    // on MFMA with Z' in high + low bf16 parts (the factored sum can cancel
    // when q is nearly orthogonal to the keys), then sum_b q_ib (Z' Q^T)[b][i]
    bf16x8 zhi[2], zlo[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ct = 2 * ks + (g >> 1);
      const float wz = ct < it ? 0.f : (ct > it ? 2.f : 1.f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = gs[2 * ks + (e >> 2)][e & 3] * wz;
        const __bf16 h = (__bf16)x;
        zhi[ks][e] = h;
        zlo[ks][e] = (__bf16)(x - (float)h);
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (2 * ks + 1 < it) continue;  // both tiles of this k-range lie below the diagonal
        const bf16x8 b = G::ld(Qs, PQ, t * 16 + n, ks, g);
        acc = mfma_bf16(zhi[ks], b, acc);
        acc = mfma_bf16(zlo[ks], b, acc);
      }
      // acc[r] = (Z' Q^T)[b = 16 it + 4 g + r][i = 16 t + n]
      const bf16x4 qc = *reinterpret_cast<const bf16x4*>(&Qs[(t * 16 + n) * PQ + it * 16 + 4 * g]);
      float p = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) p += (float)qc[r] * acc[r];
      p = sum_over_groups(p);
      if (g == 0) dred[it * BLK + t * 16 + n] = p;
    }
  }

  // scores, transposed: W[jt][r] = w(i = il, j = 16 jt + 4g + r)
  f32x4 W[4];
  float den_l = 0.f;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    W[jt] = zero4();
    if (jt <= it) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DH / G::KS; ++ks)
        acc = G::mma(G::ld(Ks, PQ, jt * 16 + n, ks, g), G::ld(Qs, PQ, il, ks, g), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = jt * 16 + 4 * g + r;
        float s = acc[r];
        if (ORDER == 2) s = s * s;
        const float w = (j <= il && j < nvalid) ? s * exp2_fast(cs_i - csl[j]) : 0.f;
        W[jt][r] = w;
        den_l += w;
      }
    }
  }

  // num^T[c][i] = sum_j VT[c][j] W[i][j]
  f32x4 num[NT];
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) num[ct] = zero4();
  if constexpr (BF) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (2 * kb <= it) {
        bf16x8 bw;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bw[r] = (__bf16)W[2 * kb][r];
          bw[4 + r] = (__bf16)W[2 * kb + 1][r];
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const C* base_p = &VT[(ct * 16 + n) * PJ + kb * 32 + 4 * g];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(base_p);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(base_p + 16);
          bf16x8 a;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            a[r] = lo[r];
            a[4 + r] = hi[r];
          }
          num[ct] = mfma_bf16(a, bw, num[ct]);
        }
      }
    }
  } else {
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      if (jt <= it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int ct = 0; ct < NT; ++ct)
            num[ct] = mfma_f32(VT[(ct * 16 + n) * PJ + jt * 16 + 4 * g + r], W[jt][r], num[ct]);
        }
      }
    }
  }
  den_l = sum_over_groups(den_l);

  if constexpr (PAIRS) {
   if (partner) {
    // direct term of the step's first block: num^T[c][i] += sum_j
    // (v dt)_jc (q_i . k_j)^2 e^{cs_i + T' - cs'_j}, with every j before i.
    // Ks, VT and dtv are restaged with the partner block once every wave is
    // done with them.
    __syncthreads();
    *reinterpret_cast<uint4*>(&Ks[(tid >> 3) * PQ + (tid & 7) * 8]) = pka;
    *reinterpret_cast<uint4*>(&Ks[(32 + (tid >> 3)) * PQ + (tid & 7) * 8]) = pkb;
    if (tid < BLK) {
      csl[tid] = pcs;  // the block's own values stay in cs_i (registers)
      dtv[tid] = pdt;
    }
    __syncthreads();
    {
      const int j0 = 2 * (tid >> 3), sg = tid & 7;
      const uint32_t w0[4] = {pva.x, pva.y, pva.z, pva.w};
      const uint32_t w1[4] = {pvb.x, pvb.y, pvb.z, pvb.w};
      const float d0 = dtv[j0], d1 = dtv[j0 + 1];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float a0 = __uint_as_float(hh ? (w0[u] & 0xffff0000u) : (w0[u] << 16)) * d0;
          const float a1 = __uint_as_float(hh ? (w1[u] & 0xffff0000u) : (w1[u] << 16)) * d1;
          C pr[2] = {(C)a0, (C)a1};
          *reinterpret_cast<uint32_t*>(&VT[(sg * 8 + 2 * u + hh) * PJ + j0]) = __builtin_bit_cast(uint32_t, pr);
        }
      }
    }
    __syncthreads();
    f32x4 Wp[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < DH / G::KS; ++ks)
        acc = G::mma(G::ld(Ks, PQ, jt * 16 + n, ks, g), G::ld(Qs, PQ, il, ks, g), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = jt * 16 + 4 * g + r;
        Wp[jt][r] = acc[r] * acc[r] * exp2_fast(cs_i + pT - csl[j]);
        den_p += Wp[jt][r];
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        bf16x8 bw;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bw[r] = (__bf16)Wp[2 * kb][r];
          bw[4 + r] = (__bf16)Wp[2 * kb + 1][r];
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          const C* base_p = &VT[(ct * 16 + n) * PJ + kb * 32 + 4 * g];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(base_p);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(base_p + 16);
          bf16x8 a;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            a[r] = lo[r];
            a[4 + r] = hi[r];
          }
          num[ct] = mfma_bf16(a, bw, num[ct]);
        }
      }
    }
   }
  }

  // inter-block part, decayed from the block start.  Order 1: the product
  // above.  Order 2: the numerators come from the state scan; q^T Z q from
  // the per-wave parts.
  const float eci = exp2_fast(cs_i);
  if constexpr (ORDER == 1) {
    if constexpr (!SPLIT) inter_product();
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) num[ct] += eci * inter[ct];
  } else {
    __syncthreads();  // every wave's part of q^T Z q is in dred
    den_x = (dred[il] + dred[BLK + il]) + (dred[2 * BLK + il] + dred[3 * BLK + il]);
    // the second block of a step: Z entered the step one block earlier
    // (decay e^{T'} more), and the first block's keys add their terms
    if (partner) den_x *= exp2_fast(pT);
    den_l += sum_over_groups(den_p);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) num[ct] += gp[ct];
  }
  const float dtot = den_l + eci * den_x;

  if (il < nvalid) {
    float* yp = y + (row + t0 + il) * DH;
    const float rd = 1.f / dtot;
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = num[ct][r] * rd;
      *reinterpret_cast<f32x4*>(yp + ct * 16 + 4 * g) = o;
    }
    if (den && g == 0) den[row + t0 + il] = dtot;
  }
}

hipError_t launch_output(bool bf16, int64_t DH, int order, const void* q, const void* k,
                         const void* v, const float* dt, const float* a_cs, int64_t BH, int64_t N,
                         int64_t chunk, const float* state, const float* part, float* y,
                         float* den, hipStream_t stream) {
  const int64_t nb = n_blocks(N);
  // order 2: workgroups in groups of 16 (8 step pairs) over the XCDs, see k_output
  const int64_t g2 = 16 * ((BH * ((nb + 1) / 2) + 7) / 8);
  const dim3 grid((unsigned)(order == 2 ? g2 : BH * nb)), blk(256);
#define SSD_LAUNCH_OUT(BFV, DHV, ORD)                                                           \
  hipLaunchKernelGGL((k_output<BFV, DHV, ORD>), grid, blk, 0, stream, q, k, v, dt, a_cs, BH, N, \
                     chunk, nb, state, part, y, den)
  if (order == 2) {
    SSD_LAUNCH_OUT(true, 64, 2);
  } else if (bf16) {
    if (DH == 64) SSD_LAUNCH_OUT(true, 64, 1);
    else SSD_LAUNCH_OUT(true, 32, 1);
  } else {
    if (DH == 64) SSD_LAUNCH_OUT(false, 64, 1);
    else SSD_LAUNCH_OUT(false, 32, 1);
  }
#undef SSD_LAUNCH_OUT
  return hipGetLastError();
}

}  // namespace ssd
