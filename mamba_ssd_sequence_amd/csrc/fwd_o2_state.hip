// Order-2 (2Mamba) inter-block numerator: an on-chip scan of the d_h^2 x d_h
// state over steps of two 64-token blocks.
//
// 2Mamba2Furious, Algorithm 6: with order-2 features phi(x) = vec(x x^T) the
// numerator state H_up is D x d_h (D = d_h^2 = 4096 at d_h = 64, 1 MiB fp32
// per head).  Over a step of tokens j (two blocks, 2m and 2m+1) with decay
// weights w_j = exp(A^CS_end - A^CS_j) it evolves as
//     S <- exp(T_2m + T_2m+1) S + sum_j w_j phi(k_j) (v dt)_j^T,
// and the contribution of the state entering the step to the numerator of
// a token i of the step is
//     exp(A^CS_i - A^CS_start) phi(q_i)^T S_in.
// Writing the state row index as (a, b), both contractions factor per a:
//     update : S_a += K^T diag(k_:a) X,          X_jc = w_j (v dt)_jc
//     output : Y   += diag(qe_:a) (Q S_a),       qe_ia = q_ia exp(A^CS_i - A^CS_start)
// so phi(q), phi(k) are never formed, only the per-row scalings.  The second
// block of a step misses the first block's tokens in this product; the
// output kernel adds them as a direct term.  Steps of two blocks halve the
// per-element work on the state (decay, fp16 conversion) per token.
//
// Decomposition.  The 1 MiB state never leaves the chip: each workgroup owns
// an a-slice (SL values of a) x an 8-column value slice, held as MFMA
// accumulators (fp32) across the whole sequence, and walks the steps in
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
// amplified there beyond the bf16 tolerance.  A change of sig between steps
// is folded into the decay factor, e^T 2^(sig_m - sig_{m-1}), so rescaling
// costs nothing; all scalars come precomputed in the block records.
//
// Pipeline, one barrier per step m: reduce step m-1's partial outputs (LDS)
// into the workspace; copy step m+1's two records (prefetched into
// registers one iteration earlier) into the other LDS slot; issue the loads
// of step m+2 at once, so they have a whole step to arrive; run step m's
// MFMA work and write its partial outputs to LDS.
// Half of the waves do the MFMA work first and the other half last, so every
// SIMD keeps its matrix core busy while the other wave does the bookkeeping.
// Within the MFMA work the VALU operations are placed by hand between the
// MFMAs (a wave issues in order, so VALU work that waits on a chain's result
// would otherwise leave the matrix core idle): slot m holds one MFMA and
// the VALU work that is ready by then (a chain's result is used three or
// more slots after its last MFMA, LDS operands are read ahead), the output
// and update chains of the two blocks alternate, and scheduling barriers
// keep the compiler from regrouping the slots.  The per-block operands
// arrive pre-converted from the block-prep kernel, so staging is plain
// copies.
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
  constexpr int NI = BLK * DH / 8 / NT;   // 16-byte q / k^T segments per thread and block
  constexpr int NXW = CW * DH / 2;        // 32-bit X^T words per block
  static_assert(NT == 512 && NI == 1 && 2 * NXW == NT, "thread mapping: 8 waves");
  static_assert(NQD == 1 || NQD == 2, "one or two a-quads per wave");

  // staging (by step parity, then block within the step) and partial-output
  // buffers; e^{cs} rows rotate over three slots because the drain of step
  // m-1 may still read them while step m+1 is staged
  __shared__ __attribute__((aligned(16))) _Float16 Qh[2][2][BLK * PH];  // [i][perm b] q 2^tau
  __shared__ __attribute__((aligned(16))) _Float16 KTh[2][2][DH * PH];  // [b][j] k 2^kap
  __shared__ __attribute__((aligned(16))) _Float16 Xh[2][2][CW * PH];   // [c][j] X 2^(sig - 2 kap)
  __shared__ f32x4 red[2][NW][4 * WAVE];  // per wave, in accumulator order (4 token tiles)
  __shared__ float st_ecs[3][2][BLK];

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
  const int nblk = (int)n_blocks(N);
  const int nstep = (nblk + 1) / 2;
  const int64_t Np = o2_part_rows(N);  // partial rows per head (whole steps)
  const uint8_t* rec_h = rec + bh * nblk * (int64_t)REC_BYTES;

  // ---- registers of the prefetched step ---------------------------------------
  // thread tid copies the 16-byte q / k^T segment tid of each block, the X^T
  // word tid % 256 of block tid / 256 and the e^{cs} entry tid % 64 of block
  // (tid / 64) % 2
  // (named registers rather than arrays, which the compiler would place in
  // memory)
  uint4 pq0, pq1, pk0, pk1;
  uint32_t px;
  uint32_t pe;
  struct Stp {
    int sig_in;       // scale exponent of the state entering the step
    int sig_out;      // ... after the step
    float eTs;        // decay and rescale factor of the state over the step
    int tau0, tau1;   // q scale exponents of the two blocks
    uint32_t xf0, xf1;  // two fp16 factors for X of each block (0 for an empty block)
    float epre0, epre1;  // decay from the start of the step to the start of each block
  };
  Stp nx{}, cur{}, prv{};
  auto prefetch = [&](int st) {
    const int b0 = 2 * st, b1 = 2 * st + 1 < nblk ? 2 * st + 1 : nblk - 1;
    const uint8_t* R0 = rec_h + b0 * (int64_t)REC_BYTES;
    const uint8_t* R1 = rec_h + b1 * (int64_t)REC_BYTES;
    {
      const int r = tid >> 3, sg = tid & 7;
      pq0 = *reinterpret_cast<const uint4*>(R0 + REC_QH + (r * DH + sg * 8) * 2);
      pk0 = *reinterpret_cast<const uint4*>(R0 + REC_KT + (r * DH + sg * 8) * 2);
      pq1 = *reinterpret_cast<const uint4*>(R1 + REC_QH + (r * DH + sg * 8) * 2);
      pk1 = *reinterpret_cast<const uint4*>(R1 + REC_KT + (r * DH + sg * 8) * 2);
    }
    const int* sc0 = reinterpret_cast<const int*>(R0 + REC_SC);  // uniform addresses
    const int* sc1 = reinterpret_cast<const int*>(R1 + REC_SC);
    nx.sig_in = sc0[SC_SIG_IN];
    nx.sig_out = sc0[SC_SIG_OUT];
    nx.eTs = __int_as_float(sc0[SC_ETS]);
    nx.tau0 = sc0[SC_TAU];
    nx.tau1 = sc1[SC_TAU];
    nx.xf0 = (uint32_t)sc0[SC_XF];
    nx.xf1 = 2 * st + 1 < nblk ? (uint32_t)sc1[SC_XF] : 0u;  // an empty second block
    nx.epre0 = __int_as_float(sc0[SC_EPRE]);
    nx.epre1 = __int_as_float(sc1[SC_EPRE]);
    {
      const int hb = tid >> 8, idx = tid & (NXW - 1), xr = idx >> 5, xw = idx & 31;
      const int b = 2 * st + hb < nblk ? 2 * st + hb : nblk - 1;
      px = *reinterpret_cast<const uint32_t*>(rec_h + b * (int64_t)REC_BYTES + REC_XT +
                                              ((c0 + xr) * DH + 2 * xw) * 2);
    }
    {
      const int hb = (tid >> 6) & 1;
      const int b = 2 * st + hb < nblk ? 2 * st + hb : nblk - 1;
      pe = *reinterpret_cast<const uint32_t*>(rec_h + b * (int64_t)REC_BYTES + REC_ECS + 4 * (tid & (BLK - 1)));
    }
  };

  // copy the prefetched step st into its LDS slot, X scaled to the state's
  // scale (a step beyond the last one is copied into the slot no step reads
  // any more)
  auto stage = [&](int st) {
    const int sl = st & 1;
    {
      const int r = tid >> 3, sg = tid & 7;
      *reinterpret_cast<uint4*>(&Qh[sl][0][r * PH + sg * 8]) = pq0;
      *reinterpret_cast<uint4*>(&KTh[sl][0][r * PH + sg * 8]) = pk0;
      *reinterpret_cast<uint4*>(&Qh[sl][1][r * PH + sg * 8]) = pq1;
      *reinterpret_cast<uint4*>(&KTh[sl][1][r * PH + sg * 8]) = pk1;
    }
    {
      const int hb = tid >> 8, idx = tid & (NXW - 1), xr = idx >> 5, xw = idx & 31;
      const f16x2 xf = __builtin_bit_cast(f16x2, hb ? nx.xf1 : nx.xf0);
      const f16x2 x = (__builtin_bit_cast(f16x2, px) * xf[0]) * xf[1];
      *reinterpret_cast<f16x2*>(&Xh[sl][hb][xr * PH + 2 * xw]) = x;
    }
    if (tid < 2 * BLK) st_ecs[st % 3][tid >> 6][tid & (BLK - 1)] = __uint_as_float(pe);
  };

  // partial outputs of step st (its scales in p) -> workspace, scaled to
  // true units: e^{cs_i} epre 2^-(sig_in + 2 tau).  Thread tid handles block
  // tid / 256, token (tid / 4) % 64 and columns 2 (tid % 4) .. + 1, which sit
  // in components c2 % 4 .. of accumulator slot (token tile) of lane
  // i % 32 + 32 (c2 / 4) of every wave.
  auto drain = [&](int st, const Stp& p) {
    const int hb = tid >> 8, i = (tid >> 2) & (BLK - 1), c2 = (tid & 3) * 2;
    const int t = 2 * hb + (i >> 5);
    const int idx = t * WAVE + (i & 31) + 32 * (c2 >> 2);
    const float* rb = reinterpret_cast<const float*>(&red[st & 1][0][idx]) + (c2 & 3);
    constexpr int WS = 4 * WAVE * 4;  // floats per wave
    float s0 = rb[0], s1 = rb[1];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      s0 += rb[w * WS];
      s1 += rb[w * WS + 1];
    }
    const float f = st_ecs[st % 3][hb][i] * (hb ? p.epre1 : p.epre0) *
                    ldexpf(ldexpf(1.f, -p.sig_in), -2 * (hb ? p.tau1 : p.tau0));
    float2 o;
    o.x = s0 * f;
    o.y = s1 * f;
    const int64_t row = (int64_t)(2 * st + hb) * BLK + i;
    *reinterpret_cast<float2*>(&part[(((int64_t)pa * BH + bh) * Np + row) * DH + c0 + c2]) = o;
  };

  // state: quad qd, b-tile bt (32 rows) -> 32 x 32 accumulator over
  // (b) x (a = aw0 + 4 qd + n32/8, c = c0 + n32%8); lane (n32, h)
  // holds the rows b = 32 bt + 8 q + 4 h + s in register 4 q + s
  f32x16 S[NQD][2];
#pragma unroll
  for (int p = 0; p < NQD; ++p)
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) S[p][bt] = f32x16{};
  // fp16 copy of quad 0's state, made at the end of the previous step's
  // update so that the first output chain can start at once
  f16x8 SA0[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) SA0[kk] = f16x8{};

  // MFMA work of step st.  Output over token tiles t (32 tokens: block t / 2,
  // rows 32 (t % 2) ..): T^T[(a, c)][i] = sum_b S[b][(a, c)] Q[i][b] over
  // 16-row k-steps kk (b in 16 kk + {4h..4h+3, 8+4h..8+4h+3} on lane half h,
  // matching the record's q column order), then Y[i][c] += sum_a q_ia
  // T^T[(a, c)][i].  Update: S = eTs S + sum over both blocks hb of K^T
  // ((k_:a 2^kap) * X 2^(sig - 2 kap)) over 16-token k-steps (tokens 16 kk +
  // 8 h .. +7 on lane half h).
  auto compute = [&](int st) {
    const int sl = st & 1;
    const float eT = cur.eTs;

    f16x8 SA1[4];          // fp16 copy of quad 1's state
    f16x8 Qf[4][4];        // B operand of the output: Q^T[b][i] of token tile t
    f16x4 qv[NQD][4];      // q values of the quad's a's for the lane's token of tile t
    f32x16 T[NQD][4];      // output chains (quad, token tile)
    f32x4 Y[4] = {zero4(), zero4(), zero4(), zero4()};
    f16x8 xh[2][4];        // X^T[c][j] of block hb, c = n32 % 8
    f16x8 Kr[NQD][2][4];   // K^T row of k_:a of block hb for a = aw0 + 4 qd + n32/8
    f16x8 Bu[NQD][2][4];   // update B operand
    f16x8 Kf[2][2][4];     // update A operand: K^T[b][j] of block hb, b = 32 bt + n32

    auto SB = [] { __builtin_amdgcn_sched_barrier(0); };
    auto rdQ = [&](int t) {
      const _Float16* Q = Qh[sl][t >> 1];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        Qf[t][kk] = *reinterpret_cast<const f16x8*>(&Q[((t & 1) * 32 + n32) * PH + kk * 16 + 8 * h]);
    };
    auto rdqv = [&](int t) {
      const _Float16* Q = Qh[sl][t >> 1];
#pragma unroll
      for (int q = 0; q < NQD; ++q)
        qv[q][t] = *reinterpret_cast<const f16x4*>(&Q[((t & 1) * 32 + n32) * PH + qpos[q]]);
    };
    auto rdK = [&](int bt, int hb) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        Kf[hb][bt][kk] = *reinterpret_cast<const f16x8*>(&KTh[sl][hb][(bt * 32 + n32) * PH + kk * 16 + 8 * h]);
    };
    auto rdX = [&](int hb) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        xh[hb][kk] = *reinterpret_cast<const f16x8*>(&Xh[sl][hb][(n32 & 7) * PH + kk * 16 + 8 * h]);
    };
    auto rdKr = [&](int q, int hb) {
      const int a = aw0 + 4 * q + (n32 >> 3);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        Kr[q][hb][kk] = *reinterpret_cast<const f16x8*>(&KTh[sl][hb][a * PH + kk * 16 + 8 * h]);
    };
    // MFMAs
    auto out = [&](int q, int t, int kk, const f16x8* SA) {
      T[q][t] = mfma32(SA[kk], Qf[t][kk], kk == 0 ? f32x16{} : T[q][t]);
    };
    auto upd = [&](int q, int bt, int hb, int kk) {
      S[q][bt] = mfma32(Kf[hb][bt][kk], Bu[q][hb][kk], S[q][bt]);
    };
    // VALU units (four instructions each); the empty asm consumes a
    // conversion's result in place, so that it is not moved to the loop's
    // end where its value is carried
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
    auto fy = [&](int q, int t, int m) {
      const float qa = (float)qv[q][t][m];
#pragma unroll
      for (int s = 0; s < 4; ++s) Y[t][s] = fmaf(qa, T[q][t][4 * m + s], Y[t][s]);
    };
    auto bu = [&](int q, int hb, int kk) { Bu[q][hb][kk] = Kr[q][hb][kk] * xh[hb][kk]; };
    auto wr = [&] {
#pragma unroll
      for (int t = 0; t < 4; ++t) red[sl][wave][t * WAVE + lane] = Y[t];
    };

    if constexpr (NQD == 2) {
      rdQ(0); rdqv(0); cvt(SA1, 1, 0); cvt(SA1, 1, 1); SB();
      out(0, 0, 0, SA0); cvt(SA1, 1, 2); SB();
      out(0, 0, 1, SA0); cvt(SA1, 1, 3); mul(0, 0, 0); SB();
      out(0, 0, 2, SA0); mul(0, 0, 1); SB();
      out(0, 0, 3, SA0); mul(0, 0, 2); mul(0, 0, 3); rdQ(1); SB();
      out(1, 0, 0, SA1); mul(0, 1, 0); SB();
      out(1, 0, 1, SA1); mul(0, 1, 1); mul(0, 1, 2); rdqv(1); SB();
      out(1, 0, 2, SA1); fy(0, 0, 0); SB();
      out(1, 0, 3, SA1); fy(0, 0, 1); fy(0, 0, 2); SB();
      out(0, 1, 0, SA0); fy(0, 0, 3); SB();
      out(0, 1, 1, SA0); mul(0, 1, 3); mul(1, 0, 0); SB();
      out(0, 1, 2, SA0); fy(1, 0, 0); SB();
      out(0, 1, 3, SA0); fy(1, 0, 1); fy(1, 0, 2); rdQ(2); SB();
      out(1, 1, 0, SA1); fy(1, 0, 3); SB();
      out(1, 1, 1, SA1); mul(1, 0, 1); mul(1, 0, 2); rdqv(2); SB();
      out(1, 1, 2, SA1); fy(0, 1, 0); SB();
      out(1, 1, 3, SA1); fy(0, 1, 1); fy(0, 1, 2); SB();
      out(0, 2, 0, SA0); fy(0, 1, 3); SB();
      out(0, 2, 1, SA0); mul(1, 0, 3); mul(1, 1, 0); SB();
      out(0, 2, 2, SA0); fy(1, 1, 0); SB();
      out(0, 2, 3, SA0); fy(1, 1, 1); fy(1, 1, 2); rdQ(3); SB();
      out(1, 2, 0, SA1); fy(1, 1, 3); SB();
      out(1, 2, 1, SA1); mul(1, 1, 1); mul(1, 1, 2); rdqv(3); SB();
      out(1, 2, 2, SA1); fy(0, 2, 0); SB();
      out(1, 2, 3, SA1); fy(0, 2, 1); fy(0, 2, 2); SB();
      out(0, 3, 0, SA0); fy(0, 2, 3); rdX(0); rdKr(0, 0); SB();
      out(0, 3, 1, SA0); mul(1, 1, 3); SB();
      out(0, 3, 2, SA0); fy(1, 2, 0); SB();
      out(0, 3, 3, SA0); fy(1, 2, 1); fy(1, 2, 2); SB();
      out(1, 3, 0, SA1); fy(1, 2, 3); rdK(0, 0); SB();
      out(1, 3, 1, SA1); bu(0, 0, 0); bu(0, 0, 1); SB();
      out(1, 3, 2, SA1); bu(0, 0, 2); SB();
      out(1, 3, 3, SA1); bu(0, 0, 3); fy(0, 3, 0); SB();
      upd(0, 0, 0, 0); fy(0, 3, 1); rdKr(1, 0); rdK(1, 0); SB();
      upd(0, 0, 0, 1); fy(0, 3, 2); SB();
      upd(0, 0, 0, 2); fy(0, 3, 3); SB();
      upd(0, 0, 0, 3); fy(1, 3, 0); SB();
      upd(0, 1, 0, 0); fy(1, 3, 1); SB();
      upd(0, 1, 0, 1); fy(1, 3, 2); fy(1, 3, 3); SB();
      upd(0, 1, 0, 2); bu(1, 0, 0); bu(1, 0, 1); wr(); SB();
      upd(0, 1, 0, 3); bu(1, 0, 2); bu(1, 0, 3); SB();
      upd(1, 0, 0, 0); rdX(1); rdKr(0, 1); SB();
      upd(1, 0, 0, 1); SB();
      upd(1, 0, 0, 2); rdK(0, 1); SB();
      upd(1, 0, 0, 3); bu(0, 1, 0); SB();
      upd(1, 1, 0, 0); bu(0, 1, 1); SB();
      upd(1, 1, 0, 1); bu(0, 1, 2); SB();
      upd(1, 1, 0, 2); bu(0, 1, 3); rdK(1, 1); SB();
      upd(1, 1, 0, 3); SB();
      upd(0, 0, 1, 0); rdKr(1, 1); SB();
      upd(0, 0, 1, 1); SB();
      upd(0, 0, 1, 2); SB();
      upd(0, 0, 1, 3); bu(1, 1, 0); SB();
      upd(0, 1, 1, 0); bu(1, 1, 1); SB();
      upd(0, 1, 1, 1); bu(1, 1, 2); SB();
      upd(0, 1, 1, 2); bu(1, 1, 3); SB();
      upd(0, 1, 1, 3); cvt(SA0, 0, 0); SB();
      upd(1, 0, 1, 0); cvt(SA0, 0, 1); SB();
      upd(1, 0, 1, 1); SB();
      upd(1, 0, 1, 2); cvt(SA0, 0, 2); SB();
      upd(1, 0, 1, 3); cvt(SA0, 0, 3); SB();
      upd(1, 1, 1, 0); SB();
      upd(1, 1, 1, 1); SB();
      upd(1, 1, 1, 2); SB();
      upd(1, 1, 1, 3); SB();
    } else {
      rdQ(0); rdqv(0); SB();
      out(0, 0, 0, SA0); mul(0, 0, 0); rdQ(1); SB();
      out(0, 0, 1, SA0); mul(0, 0, 1); rdqv(1); SB();
      out(0, 0, 2, SA0); mul(0, 0, 2); SB();
      out(0, 0, 3, SA0); mul(0, 0, 3); rdQ(2); SB();
      out(0, 1, 0, SA0); mul(0, 1, 0); SB();
      out(0, 1, 1, SA0); mul(0, 1, 1); rdqv(2); SB();
      out(0, 1, 2, SA0); fy(0, 0, 0); SB();
      out(0, 1, 3, SA0); fy(0, 0, 1); rdQ(3); SB();
      out(0, 2, 0, SA0); fy(0, 0, 2); rdX(0); rdKr(0, 0); SB();
      out(0, 2, 1, SA0); fy(0, 0, 3); rdqv(3); SB();
      out(0, 2, 2, SA0); fy(0, 1, 0); SB();
      out(0, 2, 3, SA0); bu(0, 0, 0); SB();
      out(0, 3, 0, SA0); bu(0, 0, 1); rdK(0, 0); SB();
      out(0, 3, 1, SA0); bu(0, 0, 2); SB();
      out(0, 3, 2, SA0); bu(0, 0, 3); SB();
      out(0, 3, 3, SA0); fy(0, 1, 1); SB();
      upd(0, 0, 0, 0); fy(0, 1, 2); rdX(1); rdKr(0, 1); rdK(1, 0); SB();
      upd(0, 0, 0, 1); fy(0, 1, 3); SB();
      upd(0, 0, 0, 2); mul(0, 1, 2); rdK(0, 1); SB();
      upd(0, 0, 0, 3); mul(0, 1, 3); SB();
      upd(0, 1, 0, 0); fy(0, 2, 0); fy(0, 2, 1); SB();
      upd(0, 1, 0, 1); fy(0, 2, 2); fy(0, 2, 3); SB();
      upd(0, 1, 0, 2); bu(0, 1, 0); bu(0, 1, 1); rdK(1, 1); SB();
      upd(0, 1, 0, 3); bu(0, 1, 2); bu(0, 1, 3); SB();
      upd(0, 0, 1, 0); fy(0, 3, 0); fy(0, 3, 1); SB();
      upd(0, 0, 1, 1); fy(0, 3, 2); fy(0, 3, 3); SB();
      upd(0, 0, 1, 2); wr(); SB();
      upd(0, 0, 1, 3); SB();
      upd(0, 1, 1, 0); SB();
      upd(0, 1, 1, 1); SB();
      upd(0, 1, 1, 2); cvt(SA0, 0, 0); SB();
      upd(0, 1, 1, 3); cvt(SA0, 0, 1); SB();
      cvt(SA0, 0, 2); cvt(SA0, 0, 3); SB();
    }
  };

  // prologue: stage step 0, prefetch step 1
  prefetch(0);
  stage(0);
  cur = nx;
  prefetch(nstep > 1 ? 1 : 0);
  __syncthreads();

  // Per step m: MFMA work of m, drain of m-1, staging of m+1, loads of m+2,
  // one barrier.  With two waves per SIMD the first four waves run the MFMA
  // work first and the other four the bookkeeping first; each group has a
  // loop of its own (every wave passes the same barriers), so the loads of a
  // step have a single destination and are waited for only where the staging
  // consumes them.  The loads for step m+2 are issued right after the
  // registers are free, a whole step ahead of their use.
  if (wave < NW / 2) {
    for (int st = 0; st < nstep; ++st) {
      const Stp nxt = nx;  // scales of step st + 1 (prefetched)
      compute(st);
      if (st > 0) drain(st - 1, prv);
      stage(st + 1);
      prefetch(st + 2 < nstep ? st + 2 : nstep - 1);
      prv = cur;
      cur = nxt;
      __syncthreads();
    }
  } else {
    for (int st = 0; st < nstep; ++st) {
      const Stp nxt = nx;
      if (st > 0) drain(st - 1, prv);
      stage(st + 1);
      prefetch(st + 2 < nstep ? st + 2 : nstep - 1);
      compute(st);
      prv = cur;
      cur = nxt;
      __syncthreads();
    }
  }
  drain(nstep - 1, prv);

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
