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
// an a-slice (SL values of a) x an 8-column value slice, held as MFMA
// accumulators (fp32) across the whole sequence, and walks the blocks in
// order.  Each of its 8 waves owns AW values of a (in quads) on the 8
// columns; one 32x32 accumulator tile covers 32 values of b x (4 values of
// a x 8 columns), so the state of a quad is two tiles (32 VGPRs/lane).  With
// >= 32 heads a workgroup holds all 64 values of a (no partial outputs to
// combine), with fewer heads half of them.  On gfx950 the 32x32x16 MFMA (32
// cycles) absorbs the per-element VALU work of this scan (decay, fp16
// conversion, row scalings) with little loss, and its operand fragments
// (32 rows x 16 bytes at a 144-byte pitch) read LDS without bank conflicts.
// The A operand of the output product is the state itself (its accumulator
// layout read as a permuted-k operand), the A operand of the update is K^T.
// The workgroup's output (over its a-slice) is reduced over its waves in LDS
// and written to the workspace; the output kernel adds the P_a a-slices.
//
// Precision.  Both products run on v_mfma_f32_32x32x16_f16 (same rate as
// bf16) with exact power-of-two scales: q*2^tau < 2^13 and k*2^kap in (-1, 1)
// per block (bf16 inputs convert to fp16 exactly), the state held as
// S*2^sig with sig from the scale scan (a running upper bound M >= max|S|,
// M <- e^T M + sum_j w_j max|k_j|^2 max|v_j dt_j|, keeps S*2^sig below 2^13),
// and the update operand (k_ja 2^kap) * X_jc with X_jc = w_j (v dt)_jc
// 2^(sig - 2 kap) < 2^15, formed by packed fp16 multiplies.  fp16's 11-bit
// significand matters here: the factored sum over (a, b) can cancel when q is
// nearly orthogonal to the block's keys, and a bf16 rounding of the state is
// amplified there beyond the bf16 tolerance.  A change of sig between blocks
// is folded into the decay factor, e^T 2^(sig_n - sig_{n-1}), so rescaling
// costs nothing; all per-block scalars come precomputed in the record.
//
// Pipeline, one barrier per block n: reduce block n-1's partial outputs
// (LDS) into the workspace; copy block n+1's record (prefetched into
// registers one iteration earlier) into the other LDS slot; issue the loads
// of block n+2 at once, so they have a whole block to arrive; run block n's
// MFMA work and write its partial output to LDS.
// Half of the waves do the MFMA work first and the other half last, so every
// SIMD keeps its matrix core busy while the other wave does the bookkeeping.
// Within the MFMA work the VALU operations are placed by hand between the
// MFMAs (a wave issues in order, so VALU work that waits on a chain's result
// would otherwise leave the matrix core idle).
// The per-block operands arrive pre-converted from the block-prep kernel, so
// staging is plain copies.
//
// Grid: B*H x P_a x 8 workgroups (P_a = 64 / (8*AW)), 512 threads each; when
// B*H is a multiple of 8 the workgroups of one head share an XCD (and its L2).
#include "common.h"
#include "launch.h"

namespace ssd {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

namespace {
constexpr int DH = 64;
constexpr int CW = 8;       // value columns per workgroup
constexpr int NCS = 64 / CW;  // column slices per head
constexpr int PH = DH + 8;  // fp16 row pitch (elements): 144 B

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}




}  // namespace

template <int NW, int AW>
__global__ __launch_bounds__(NW * 64) void k_o2_state(const uint8_t* __restrict__ rec, int64_t BH,
                                                      int64_t N, int xcd_map,
                                                      float* __restrict__ part,
                                                      float* __restrict__ final_state) {
  constexpr int NT = NW * WAVE;       // threads
  constexpr int NAG = NW;             // a groups (one per wave)
  constexpr int SL = NAG * AW;        // a values per workgroup
  constexpr int PA = DH / SL;         // a-slices per head
  constexpr int NQD = AW / 4;         // a quads per wave
  constexpr int NI = BLK * DH / 8 / NT;   // 16-byte q / k^T segments per thread
  constexpr int NXW = CW * DH / 2;        // 32-bit X^T words per block
  constexpr int NX = (NXW + NT - 1) / NT; // ... per thread
  constexpr bool STAGGER = NW == 8;   // two waves per SIMD
  static_assert(AW % 4 == 0 && NI >= 1 && NX >= 1, "thread mapping");
  static_assert(NQD == 1 || NQD == 2, "one or two a-quads per wave");

  // staging (by block parity) and partial-output buffers; e^{cs} rows rotate
  // over three slots because the drain of block n-1 may still read them while
  // block n+1 is staged
  __shared__ __attribute__((aligned(16))) _Float16 Qh[2][BLK * PH];  // [i][perm b] q 2^tau
  __shared__ __attribute__((aligned(16))) _Float16 KTh[2][DH * PH];  // [b][j] k 2^kap
  __shared__ __attribute__((aligned(16))) _Float16 Xh[2][CW * PH];   // [c][j] X 2^(sig - 2 kap)
  __shared__ f32x4 red[2][NW][2 * WAVE];  // per wave, in accumulator order
  __shared__ float st_ecs[3][BLK];

  const int tid = threadIdx.x;
  // the wave index, provably uniform across the wave (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int lane = tid & (WAVE - 1), n32 = lane & 31, h = lane >> 5;
  int pc, pa;
  int64_t bh;
  if (xcd_map) {
    // workgroups are dispatched round-robin over the 8 XCDs: give all the
    // workgroups of one head the same id mod 8, so they share one L2
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    const int p = s % (PA * NCS);
    bh = (int64_t)(s / (PA * NCS)) * 8 + xcd;
    pa = p / NCS;
    pc = p % NCS;
  } else {
    pc = blockIdx.x % NCS;
    pa = (blockIdx.x / NCS) % PA;
    bh = (blockIdx.x / NCS) / PA;
  }
  const int a0 = pa * SL;
  const int c0 = pc * CW;
  // this wave: a values a0 + ag AW .. + AW - 1 (in quads), value columns
  // c0 .. c0 + 7; lane n32 of a 32x32 tile column holds a quad member n32 / 8
  // and column n32 % 8
  const int ag = wave;
  const int aw0 = a0 + ag * AW;
  // slot of q_{:, a} for the first a of each quad in the record's q row (its
  // 4-column subgroups are stored in the order 0, 2, 1, 3 of each 16-group)
  int qpos[NQD];
#pragma unroll
  for (int qd = 0; qd < NQD; ++qd) {
    const int a = aw0 + 4 * qd, G = (a >> 2) & 3;
    qpos[qd] = (a & ~15) + 4 * (G == 1 ? 2 : (G == 2 ? 1 : G));
  }
  const int64_t nblk = n_blocks(N);
  const int64_t Np = nblk * BLK;  // partial rows per head (padded)
  const uint8_t* rec_h = rec + bh * nblk * (int64_t)REC_BYTES;

  // ---- registers of the prefetched block -------------------------------------
  uint4 pq[NI], pk[NI];
  uint32_t px[NX];
  uint32_t pe;
  struct Blk {
    int sig_in, tau;  // scale exponents of the entering state and of q
    float eTs;        // decay and rescale factor of the state
    uint32_t xf;      // two fp16 factors for X
    int sig_out;      // scale exponent of the state after the block
  };
  Blk nx{}, cur{}, prv{};
  auto prefetch = [&](int64_t blk) {
    const uint8_t* R = rec_h + blk * (int64_t)REC_BYTES;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int idx = tid + u * NT, r = idx >> 3, sg = idx & 7;
      pq[u] = *reinterpret_cast<const uint4*>(R + REC_QH + (r * DH + sg * 8) * 2);
      pk[u] = *reinterpret_cast<const uint4*>(R + REC_KT + (r * DH + sg * 8) * 2);
    }
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int idx = (tid + u * NT) % NXW, xr = idx >> 5, xw = idx & 31;
      px[u] = *reinterpret_cast<const uint32_t*>(R + REC_XT + ((c0 + xr) * DH + 2 * xw) * 2);
    }
    pe = *reinterpret_cast<const uint32_t*>(R + REC_ECS + 4 * (tid & (BLK - 1)));
    const int* sc = reinterpret_cast<const int*>(R + REC_SC);  // uniform address
    nx.sig_in = sc[SC_SIG_IN];
    nx.tau = sc[SC_TAU];
    nx.eTs = __int_as_float(sc[SC_ETS]);
    nx.xf = (uint32_t)sc[SC_XF];
    nx.sig_out = sc[SC_SIG_OUT];
  };

  // copy the prefetched block blk into its LDS slot, X scaled to the state's
  // scale (a block beyond the last one is copied into the slot no block
  // reads any more)
  auto stage = [&](int64_t blk) {
    const int sl = (int)(blk & 1);
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int idx = tid + u * NT, r = idx >> 3, sg = idx & 7;
      *reinterpret_cast<uint4*>(&Qh[sl][r * PH + sg * 8]) = pq[u];
      *reinterpret_cast<uint4*>(&KTh[sl][r * PH + sg * 8]) = pk[u];
    }
    const f16x2 xf = __builtin_bit_cast(f16x2, nx.xf);
#pragma unroll
    for (int u = 0; u < NX; ++u) {
      const int idx = tid + u * NT, xr = idx >> 5, xw = idx & 31;
      if (NT * NX == NXW || idx < NXW) {
        const f16x2 x = (__builtin_bit_cast(f16x2, px[u]) * xf[0]) * xf[1];
        *reinterpret_cast<f16x2*>(&Xh[sl][xr * PH + 2 * xw]) = x;
      }
    }
    st_ecs[blk % 3][tid & (BLK - 1)] = __uint_as_float(pe);
  };

  // partial output of block blk (its scales in p) -> workspace, scaled to
  // true units: e^{cs_i} 2^-(sig_in + 2 tau)
  auto drain = [&](int64_t blk, const Blk& p) {
    // two columns per thread, so that the first NT/2 threads share the work
    constexpr int ND = BLK * CW / 2;
    if (NT == ND || tid < ND) {
      const int64_t t0 = blk * BLK;
      const int i = tid / (CW / 2), c2 = (tid % (CW / 2)) * 2;
      // element (i, c2..c2+1) sits in components c2%4.. of accumulator slot
      // i/32 of lane i%32 + 32 (c2/4) of every wave
      const int idx = (i >> 5) * WAVE + (i & 31) + 32 * (c2 >> 2);
      const float* rb = reinterpret_cast<const float*>(&red[blk & 1][0][idx]) + (c2 & 3);
      constexpr int WS = 2 * WAVE * 4;  // floats per wave
      float s0 = rb[0], s1 = rb[1];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        s0 += rb[w * WS];
        s1 += rb[w * WS + 1];
      }
      const float f = st_ecs[blk % 3][i] * ldexpf(ldexpf(1.f, -p.sig_in), -2 * p.tau);
      float2 o;
      o.x = s0 * f;
      o.y = s1 * f;
      *reinterpret_cast<float2*>(&part[(((int64_t)pa * BH + bh) * Np + t0 + i) * DH + c0 + c2]) = o;
    }
  };

  // state: quad qd, b-tile bt (32 rows) -> 32 x 32 accumulator over
  // (b) x (a = aw0 + 4 qd + n32/8, c = c0 + n32%8); lane (n32, h)
  // holds the rows b = 32 bt + 8 q + 4 h + s in register 4 q + s
  f32x16 S[NQD][2];
#pragma unroll
  for (int p = 0; p < NQD; ++p)
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) S[p][bt] = f32x16{};
  // fp16 copy of quad 0's state, made at the end of the previous block's
  // update so that the first output chain can start at once
  f16x8 SA0[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) SA0[kk] = f16x8{};

  // MFMA work of block blk.  Output: T^T[(a, c)][i] = sum_b S[b][(a, c)]
  // Q[i][b] over 16-row k-steps kk (b in 16 kk + {4h..4h+3, 8+4h..8+4h+3} on
  // lane half h, matching the record's q column order), then
  // Y[i][c] += sum_a q_ia T^T[(a, c)][i].  Update: S = eTs S + K^T ((k_:a
  // 2^kap) * X 2^(sig - 2 kap)) over 16-token k-steps (tokens 16 kk + 8 h ..
  // +7 on lane half h).
  //
  // A wave issues in order, so the VALU work (fp16 conversion of the state,
  // decay, row scalings, update operands) is interleaved by hand with the
  // MFMA chains: slot m holds one MFMA and the VALU work that is ready by
  // then (results of a chain are used two or more slots after its last
  // MFMA, LDS operands are read two to four slots ahead).  Scheduling
  // barriers keep the compiler from regrouping the slots.
  auto compute = [&](int64_t blk) {
    const int sl = (int)(blk & 1);
    const _Float16* Q = Qh[sl];
    const _Float16* KT = KTh[sl];
    const _Float16* XT = Xh[sl];
    const float eT = cur.eTs;

    f16x8 SA1[4];          // fp16 copy of quad 1's state
    f16x8 Qf[2][4];        // B operand of the output: Q^T[b][i], i = 32 it + n32
    f16x4 qv[NQD][2];      // q values of the quad's a's for token 32 it + n32
    f32x16 T[NQD][2];      // output chains (quad, it)
    f32x4 Y[2] = {zero4(), zero4()};
    f16x8 xh[4];           // X^T[c][j], c = n32 % 8
    f16x8 Kr[NQD][4];      // K^T row of k_:a for the quad's a = aw0 + 4 qd + n32/8
    f16x8 Bu[NQD][4];      // update B operand
    f16x8 Kf[2][4];        // update A operand: K^T[b][j], b = 32 bt + n32

    auto SB = [] { __builtin_amdgcn_sched_barrier(0); };
    auto rdQ = [&](int it) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        Qf[it][kk] = *reinterpret_cast<const f16x8*>(&Q[(it * 32 + n32) * PH + kk * 16 + 8 * h]);
    };
    auto rdK = [&](int bt) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        Kf[bt][kk] = *reinterpret_cast<const f16x8*>(&KT[(bt * 32 + n32) * PH + kk * 16 + 8 * h]);
    };
    auto rdX = [&] {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        xh[kk] = *reinterpret_cast<const f16x8*>(&XT[(n32 & 7) * PH + kk * 16 + 8 * h]);
    };
    auto rdKr = [&](int q) {
      const int a = aw0 + 4 * q + (n32 >> 3);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        Kr[q][kk] = *reinterpret_cast<const f16x8*>(&KT[a * PH + kk * 16 + 8 * h]);
    };
    auto rdqv = [&] {
#pragma unroll
      for (int q = 0; q < NQD; ++q)
#pragma unroll
        for (int it = 0; it < 2; ++it)
          qv[q][it] = *reinterpret_cast<const f16x4*>(&Q[(it * 32 + n32) * PH + qpos[q]]);
    };
    // MFMAs
    auto out = [&](int q, int it, int kk, const f16x8* SA) {
      T[q][it] = mfma32(SA[kk], Qf[it][kk], kk == 0 ? f32x16{} : T[q][it]);
    };
    auto upd = [&](int q, int bt, int kk) { S[q][bt] = mfma32(Kf[bt][kk], Bu[q][kk], S[q][bt]); };
    // VALU units (four instructions each)
    // (the empty asm consumes the result in place, so that the conversion is
    // not moved to the loop's end where its value is carried)
    auto cvt = [&](f16x8* SA, int q, int kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) SA[kk][e] = (_Float16)S[q][kk >> 1][8 * (kk & 1) + e];
      asm volatile("" ::"v"(SA[kk]));
    };
    auto mul = [&](int q, int bt, int g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[q][bt][4 * g + e] *= eT;
    };
    // rows 8 m + 4 h + s of T: quad member m, column 4 h + s
    auto fy = [&](int q, int it, int m) {
      const float qa = (float)qv[q][it][m];
#pragma unroll
      for (int s = 0; s < 4; ++s) Y[it][s] = fmaf(qa, T[q][it][4 * m + s], Y[it][s]);
    };
    auto bu = [&](int q, int kk) { Bu[q][kk] = Kr[q][kk] * xh[kk]; };
    auto wr = [&] {
#pragma unroll
      for (int it = 0; it < 2; ++it) red[sl][wave][it * WAVE + lane] = Y[it];
    };

    if constexpr (NQD == 2) {
      // chains: C(q, it) = out over kk, U(q, bt) = upd over kk, in the order
      // C00 C10 C01 C11 U00 U01 U10 U11
      rdQ(0); rdqv(); cvt(SA1, 1, 0); cvt(SA1, 1, 1); SB();
      out(0, 0, 0, SA0); cvt(SA1, 1, 2); rdQ(1); SB();
      out(0, 0, 1, SA0); cvt(SA1, 1, 3); mul(0, 0, 0); SB();
      out(0, 0, 2, SA0); mul(0, 0, 1); SB();
      out(0, 0, 3, SA0); mul(0, 0, 2); mul(0, 0, 3); SB();
      out(1, 0, 0, SA1); mul(0, 1, 0); SB();
      out(1, 0, 1, SA1); mul(0, 1, 1); mul(0, 1, 2); SB();
      out(1, 0, 2, SA1); mul(0, 1, 3); rdX(); SB();
      out(1, 0, 3, SA1); fy(0, 0, 0); fy(0, 0, 1); SB();
      out(0, 1, 0, SA0); fy(0, 0, 2); rdKr(0); SB();
      out(0, 1, 1, SA0); fy(0, 0, 3); SB();
      out(0, 1, 2, SA0); fy(1, 0, 0); fy(1, 0, 1); SB();
      out(0, 1, 3, SA0); fy(1, 0, 2); SB();
      out(1, 1, 0, SA1); fy(1, 0, 3); bu(0, 0); SB();
      out(1, 1, 1, SA1); bu(0, 1); rdK(0); SB();
      out(1, 1, 2, SA1); bu(0, 2); bu(0, 3); SB();
      out(1, 1, 3, SA1); fy(0, 1, 0); SB();
      upd(0, 0, 0); fy(0, 1, 1); fy(0, 1, 2); rdK(1); SB();
      upd(0, 0, 1); fy(0, 1, 3); rdKr(1); SB();
      upd(0, 0, 2); mul(1, 0, 0); mul(1, 0, 1); SB();
      upd(0, 0, 3); mul(1, 0, 2); SB();
      upd(0, 1, 0); mul(1, 0, 3); bu(1, 0); SB();
      upd(0, 1, 1); bu(1, 1); SB();
      upd(0, 1, 2); bu(1, 2); bu(1, 3); SB();
      upd(0, 1, 3); fy(1, 1, 0); SB();
      upd(1, 0, 0); fy(1, 1, 1); fy(1, 1, 2); SB();
      upd(1, 0, 1); fy(1, 1, 3); SB();
      upd(1, 0, 2); mul(1, 1, 0); mul(1, 1, 1); SB();
      upd(1, 0, 3); mul(1, 1, 2); mul(1, 1, 3); SB();
      upd(1, 1, 0); cvt(SA0, 0, 0); cvt(SA0, 0, 1); SB();
      upd(1, 1, 1); cvt(SA0, 0, 2); SB();
      upd(1, 1, 2); cvt(SA0, 0, 3); wr(); SB();
      upd(1, 1, 3); SB();
    } else {
      // chains C00 C01 U00 U01
      rdQ(0); rdqv(); SB();
      out(0, 0, 0, SA0); mul(0, 0, 0); rdQ(1); SB();
      out(0, 0, 1, SA0); mul(0, 0, 1); mul(0, 0, 2); SB();
      out(0, 0, 2, SA0); mul(0, 0, 3); rdX(); rdKr(0); SB();
      out(0, 0, 3, SA0); mul(0, 1, 0); mul(0, 1, 1); SB();
      out(0, 1, 0, SA0); mul(0, 1, 2); rdK(0); SB();
      out(0, 1, 1, SA0); mul(0, 1, 3); bu(0, 0); SB();
      out(0, 1, 2, SA0); bu(0, 1); bu(0, 2); rdK(1); SB();
      out(0, 1, 3, SA0); bu(0, 3); fy(0, 0, 0); SB();
      upd(0, 0, 0); fy(0, 0, 1); fy(0, 0, 2); SB();
      upd(0, 0, 1); fy(0, 0, 3); SB();
      upd(0, 0, 2); fy(0, 1, 0); fy(0, 1, 1); SB();
      upd(0, 0, 3); fy(0, 1, 2); SB();
      upd(0, 1, 0); fy(0, 1, 3); SB();
      upd(0, 1, 1); SB();
      upd(0, 1, 2); cvt(SA0, 0, 0); cvt(SA0, 0, 1); wr(); SB();
      upd(0, 1, 3); SB();
      cvt(SA0, 0, 2); cvt(SA0, 0, 3); SB();
    }
  };

  // prologue: stage block 0, prefetch block 1
  prefetch(0);
  stage(0);
  cur = nx;
  prefetch(nblk > 1 ? 1 : 0);
  __syncthreads();

  // Per block n: MFMA work of n, drain of n-1, staging of n+1, loads of n+2,
  // one barrier.  With two waves per SIMD the first four waves run the MFMA
  // work first and the other four the bookkeeping first; each group has a
  // loop of its own (every wave passes the same barriers), so the loads of a
  // block have a single destination and are waited for only where the staging
  // consumes them.  The loads for block n+2 are issued right after the
  // registers are free, a whole block ahead of their use.
  if (!STAGGER || wave < NW / 2) {
    for (int64_t blk = 0; blk < nblk; ++blk) {
      const Blk nxt = nx;  // scales of block blk + 1 (prefetched)
      compute(blk);
      if (blk > 0) drain(blk - 1, prv);
      stage(blk + 1);
      prefetch(blk + 2 < nblk ? blk + 2 : nblk - 1);
      prv = cur;
      cur = nxt;
      __syncthreads();
    }
  } else {
    for (int64_t blk = 0; blk < nblk; ++blk) {
      const Blk nxt = nx;
      if (blk > 0) drain(blk - 1, prv);
      stage(blk + 1);
      prefetch(blk + 2 < nblk ? blk + 2 : nblk - 1);
      compute(blk);
      prv = cur;
      cur = nxt;
      __syncthreads();
    }
  }
  drain(nblk - 1, prv);

  if (final_state) {
    const float f = ldexpf(1.f, -prv.sig_out);
    const int c = c0 + (n32 & 7);
#pragma unroll
    for (int qd = 0; qd < NQD; ++qd) {
      const int a = aw0 + 4 * qd + (n32 >> 3);
#pragma unroll
      for (int bt = 0; bt < 2; ++bt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = bt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          final_state[((bh * DH + a) * DH + b) * DH + c] = S[qd][bt][r] * f;
        }
    }
  }
}

hipError_t launch_o2_state(const void* rec, int64_t BH, int64_t N, float* part,
                           float* final_state, hipStream_t stream) {
  const int AW = o2_aw(BH);
  const int PA = o2_pa(BH);
  const int xcd_map = (BH % 8) == 0;
  const uint8_t* r = static_cast<const uint8_t*>(rec);
  const dim3 grid((unsigned)(BH * PA * NCS));
  if (AW == 8)
    hipLaunchKernelGGL((k_o2_state<8, 8>), grid, dim3(8 * WAVE), 0, stream, r, BH, N, xcd_map, part, final_state);
  else
    hipLaunchKernelGGL((k_o2_state<8, 4>), grid, dim3(8 * WAVE), 0, stream, r, BH, N, xcd_map, part, final_state);
  return hipGetLastError();
}

}  // namespace ssd
