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
// For one value column c, write the state as the d_h x d_h matrix
// S_c[b][a] (row index (a, b) of H_up); both contractions are then plain
// matrix products with a per-row or per-column scaling:
//     update : S_c[b][a] += sum_j k_jb (k_ja X_jc),   X_jc = w_j (v dt)_jc
//     output : Y[i][c]   += sum_a q_ia sum_b S_c[b][a] q_ib   (times e^{A^CS_i - A^CS_start})
// so phi(q), phi(k) are never formed.  The second block of a step misses the
// first block's tokens in this product; the output kernel adds them as a
// direct term.  Steps of two blocks halve the per-element work on the state
// (decay, fp16 conversion) per token.
//
// Decomposition.  The 1 MiB state never leaves the chip: each wave holds
// S_c for one value column c as 32 x 32 MFMA accumulator tiles (fp32; rows
// b, columns a) across the whole sequence.  With >= 32 heads (NAT = 2
// a-tiles, eight columns per workgroup) a wave holds three of the four
// tiles: S_c is symmetric in (a, b) (k (x) k is), so the tile (a-tile 0,
// b-tile 1) is the transpose of (a-tile 1, b-tile 0); it is neither updated
// nor held, and its share of the output, equal to that of its transpose, is
// taken as twice the latter's (in exact high + low fp16 parts, so that the
// pair's one rounding is not doubled), which saves a quarter of the update
// MFMAs and of the decay.  With fewer heads a wave holds the two tiles of one
// a-half (NAT = 1, two waves per column, four columns per workgroup, so that
// the grid still covers the chip; the compute-first waves hold a-tile 0, the
// others a-tile 1).  In this layout the
// update's per-column factor k_ja comes from the same K^T operand fragment
// the product itself uses (a and b index the same keys), and the output's
// per-row factor q_ia from the Q operand fragment, so besides q, k^T and X
// nothing is read from LDS; the a-contraction of the output finishes within
// the wave (plus one cross-half shuffle), so a workgroup's output needs no
// reduction over waves or workgroups.  On gfx950 the 32x32x16 MFMA (32
// cycles) absorbs the per-element VALU work (decay, fp16 conversion, row
// scalings, update operands), and its operand fragments (32 rows x 16 bytes
// at a 144-byte pitch) read LDS without bank conflicts.  The A operand of
// the output product is the state itself (its accumulator layout read as a
// permuted-k operand), the A operand of the update is K^T.
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
// Pipeline, one barrier per step m: write step m-1's outputs (LDS) to the
// workspace (compute-first waves only); copy step m+1's two records
// (prefetched into registers one iteration earlier) into the other LDS slot;
// issue the loads of step m+2 at once, so they have a whole step to arrive;
// run step m's MFMA work and write its outputs to LDS.  Half of the waves do
// the MFMA work first and the other half last, so every SIMD keeps its
// matrix core busy while the other wave does the bookkeeping.  Within the MFMA work the VALU operations
// are placed by hand between the MFMAs (a wave issues in order, so VALU work
// that waits on a chain's result would otherwise leave the matrix core
// idle): slot m holds one MFMA and the VALU work that is ready by then (a
// chain's result is used three or more slots after its last MFMA, LDS
// operands are read ahead, about one 16-byte read per slot), and scheduling
// barriers keep the compiler from regrouping the slots; gen_o2_schedule.py
// places the work and writes the two marked slot blocks below.  The
// per-block operands arrive pre-converted from the block-prep kernel, so
// staging is plain copies.
//
// Grid: B*H x (64 / columns per workgroup) workgroups, 512 threads each; when
// B*H is a multiple of 8 the workgroups of one head share an XCD (and its L2).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace ssd {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {
constexpr int DH = 64;
constexpr int PH = DH + 8;  // fp16 row pitch (elements): 144 B
constexpr int RP = 9;       // output row pitch (floats)

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
}  // namespace

template <int NAT, bool INIT>
__global__ __launch_bounds__(512) void k_o2_state(const uint8_t* __restrict__ rec, int64_t BH,
                                                  int64_t N, int xcd_map,
                                                  float* __restrict__ part,
                                                  float* __restrict__ final_state,
                                                  float* __restrict__ zst,
                                                  float* __restrict__ final_norm,
                                                  const float* __restrict__ S0,
                                                  const float* __restrict__ Z0) {
  constexpr int NW = 8, NT = NW * WAVE;  // waves, threads
  constexpr int CWG = NW * NAT / 2;      // value columns per workgroup
  constexpr int NCS = DH / CWG;          // column slices per head
  constexpr int NXW = CWG * DH / 2;      // 32-bit X^T words per block
  static_assert(NAT == 1 || NAT == 2, "one or two a-tiles per wave");
  constexpr int ZPW = Z_FLOATS / NCS;       // stored normaliser entries per workgroup
  constexpr int ZE = ZPW >= 320 ? 2 : 1;    // ... per scanning thread
  constexpr int ZTH = ZPW / ZE;             // scanning threads (compute-first ones)
  static_assert(BLK * DH / 8 == NT && 2 * NXW <= NT, "thread mapping");
  static_assert(ZPW * NCS == Z_FLOATS && ZTH * ZE == ZPW && ZTH <= NT / 2, "normaliser mapping");

  // staging (by step parity, then block within the step), outputs, and the
  // e^{cs} rows (over three slots, because the write-out of step m-1 may
  // still read them while step m+1 is staged)
  __shared__ __attribute__((aligned(16))) _Float16 Qh[2][2][BLK * PH];  // [i][perm b] q 2^tau
  __shared__ __attribute__((aligned(16))) _Float16 KTh[2][2][DH * PH];  // [b][j] k 2^kap
  __shared__ __attribute__((aligned(16))) _Float16 Xh[2][2][CWG * PH];  // [c][j] X 2^(sig - 2 kap)
  __shared__ float yo[2][2][BLK * RP];                                  // [i][wave] outputs
  __shared__ float st_ecs[3][2][BLK];
  __shared__ float zrun[NT / 2][ZE];  // running normaliser state (compute-first threads)

  const int tid = threadIdx.x;
  // the wave index, provably uniform across the wave (scalar branches)
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const int lane = tid & (WAVE - 1), n32 = lane & 31, h = lane >> 5;
  int pc;
  int64_t bh;
  if (xcd_map) {
    // workgroups are dispatched round-robin over the 8 XCDs: give all the
    // workgroups of one head the same id mod 8, so they share one L2
    const int xcd = blockIdx.x & 7, s = blockIdx.x >> 3;
    bh = (int64_t)(s / NCS) * 8 + xcd;
    pc = s % NCS;
  } else {
    pc = blockIdx.x % NCS;
    bh = blockIdx.x / NCS;
  }
  const int c0 = pc * CWG;
  // this wave: value column c0 + cl, a-tiles 0 and 1 (NAT = 2), or a-tile
  // wave / 4 (NAT = 1: the compute-first waves hold a-tile 0, the others
  // a-tile 1); its outputs go to slot yi of an output row
  const int cl = NAT == 2 ? wave : wave & 3;
  const int yi = NAT == 2 ? wave : 2 * (wave & 3) + (wave >> 2);
  const int nblk = (int)n_blocks(N);
  const int nstep = (nblk + 1) / 2;
  const int64_t Np = o2_part_rows(N);  // output rows per head (whole steps)
  const uint8_t* rec_h = rec + bh * nblk * (int64_t)REC_BYTES;

  // ---- registers of the prefetched step ---------------------------------------
  // thread tid copies the 16-byte q / k^T segment tid of each block, the X^T
  // word tid % (2 NXW) (block, column, pair of tokens) and the e^{cs} entry
  // tid % 64 of block (tid / 64) % 2 (named registers rather than arrays,
  // which the compiler would place in memory)
  uint4 pq0, pq1, pk0, pk1;
  uint32_t px, pe;
  struct Stp {
    int sig_in;          // scale exponent of the state entering the step
    int sig_out;         // ... after the step
    float eTs;           // decay and rescale factor of the state over the step
    int tau0, tau1;      // q scale exponents of the two blocks
    uint32_t xf0, xf1;   // two fp16 factors for X of each block (0 for an empty block)
    float epre0, epre1;  // decay from the start of the step to the start of each block
  };
  Stp nx{}, cur{}, prv{};
  const int xi2 = tid % (2 * NXW), xhb = xi2 / NXW, xidx = xi2 % NXW, xr = xidx >> 5, xw = xidx & 31;
  auto prefetch = [&](int st) {
    const int b0 = 2 * st, b1 = 2 * st + 1 < nblk ? 2 * st + 1 : nblk - 1;
    // addresses as one uniform base and unsigned 32-bit per-thread offsets
    // (the second block's record is d1 bytes after the first's)
    const uint8_t* R0 = rec_h + b0 * (int64_t)REC_BYTES;
    const uint8_t* R1 = rec_h + b1 * (int64_t)REC_BYTES;
    const uint32_t d1 = (uint32_t)(b1 - b0) * REC_BYTES;
    {
      const uint32_t o = ((tid >> 3) * DH + (tid & 7) * 8) * 2;
      pq0 = *reinterpret_cast<const uint4*>(R0 + (REC_QH + o));
      pk0 = *reinterpret_cast<const uint4*>(R0 + (REC_KT + o));
      pq1 = *reinterpret_cast<const uint4*>(R0 + (d1 + REC_QH + o));
      pk1 = *reinterpret_cast<const uint4*>(R0 + (d1 + REC_KT + o));
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
    px = *reinterpret_cast<const uint32_t*>(R0 + ((xhb ? d1 : 0u) + REC_XT + (uint32_t)((c0 + xr) * DH + 2 * xw) * 2));
    pe = *reinterpret_cast<const uint32_t*>(R0 + ((((tid >> 6) & 1) ? d1 : 0u) + REC_ECS + 4u * (tid & (BLK - 1))));
  };

  // copy the prefetched step st into its LDS slot, X scaled to the state's
  // scale (a step beyond the last one is copied into the slot no step reads
  // any more; threads that hold the same X word write it to the same place)
  auto stage = [&](int st) {
    const int sl = st & 1;
    {
      const int r = tid >> 3, sg = tid & 7;
      *reinterpret_cast<uint4*>(&Qh[sl][0][r * PH + sg * 8]) = pq0;
      *reinterpret_cast<uint4*>(&KTh[sl][0][r * PH + sg * 8]) = pk0;
      *reinterpret_cast<uint4*>(&Qh[sl][1][r * PH + sg * 8]) = pq1;
      *reinterpret_cast<uint4*>(&KTh[sl][1][r * PH + sg * 8]) = pk1;
    }
    const f16x2 xf = __builtin_bit_cast(f16x2, xhb ? nx.xf1 : nx.xf0);
    const f16x2 x = (__builtin_bit_cast(f16x2, px) * xf[0]) * xf[1];
    *reinterpret_cast<f16x2*>(&Xh[sl][xhb][xr * PH + 2 * xw]) = x;
    if (tid < 2 * BLK) st_ecs[st % 3][tid >> 6][tid & (BLK - 1)] = __uint_as_float(pe);
  };

  // outputs of step st (its scales in p) -> workspace, scaled to true units:
  // e^{cs_i} epre 2^-(sig_in + 2 tau).  Only the compute-first waves write
  // outputs (their bookkeeping is off the critical path); thread tid < 256
  // handles, for both blocks, token tid / 4 and, with eight columns per
  // workgroup, the columns 2 (tid % 4) .. + 1; with four, column tid % 4 (the
  // sum of its two a-half waves).
  auto drain = [&](int st, const Stp& p) {
    const int i = (tid >> 2) & (BLK - 1), q4 = tid & 3;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float* yr = &yo[st & 1][hb][i * RP];
      // the power of two is applied last (one ldexp of the product), so that
      // no intermediate factor leaves the fp32 range
      const float f = st_ecs[st % 3][hb][i] * (hb ? p.epre1 : p.epre0);
      const int sh = -p.sig_in - 2 * (hb ? p.tau1 : p.tau0);
      float* dst = part + (bh * Np + (int64_t)(2 * st) * BLK) * DH + c0 + (uint32_t)((hb * BLK + i) * DH);
      if constexpr (NAT == 2) {
        float2 o;
        o.x = ldexpf(yr[2 * q4] * f, sh);
        o.y = ldexpf(yr[2 * q4 + 1] * f, sh);
        *reinterpret_cast<float2*>(dst + 2 * q4) = o;
      } else {
        dst[q4] = ldexpf((yr[2 * q4] + yr[2 * q4 + 1]) * f, sh);
      }
    }
  };

  // normaliser state Z = sum_j w_j k_j k_j^T (2Mamba2Furious, Algorithm 6:
  // the denominator q_i^T Z q_i), scanned over the blocks in place: the slot
  // of block b holds Z_blk(b) (from the block-prep kernel), Z_in(b + 1) =
  // e^{T_b} Z_in(b) + Z_blk(b), and the slot of the first block of each
  // two-block step receives Z entering the step (the output kernel adds the
  // first block's share to the second block's rows directly).  Only the upper
  // 16 x 16 tiles of the symmetric Z are stored (Z_FLOATS floats).  Each
  // workgroup scans its 1 / NCS share of them, ZE per thread on the first ZTH
  // compute-first threads, in the slack of those threads' bookkeeping: the
  // loads are issued after their MFMA work and consumed before the barrier,
  // so no register is held across the MFMA work; the running sums stay in
  // LDS.  The other threads read a valid entry too (a load under a
  // lane-divergent branch would be waited for at the branch's end) and do
  // not store.
  constexpr int64_t ZS = DH * DH + DH;  // floats per block slot
  const bool zact = tid < ZTH;
  const int zi = (zact ? tid : ZTH - 1) * ZE;  // this thread's first entry in the share
  float* const zb = zst + bh * nblk * ZS + pc * ZPW;  // (uniform; zi is added per thread)
  auto zp = [&](int b) { return zb + b * ZS + (uint32_t)zi; };
  float2 zd0{}, zd1{};
  float zT0 = 0.f, zT1 = 0.f;
  auto zload = [&](int st) {
    const int b0 = 2 * st, b1 = 2 * st + 1;
    zT0 = __int_as_float(reinterpret_cast<const int*>(rec_h + b0 * (int64_t)REC_BYTES + REC_SC)[SC_ET]);
    if constexpr (ZE == 2) zd0 = *reinterpret_cast<const float2*>(zp(b0));
    else zd0.x = *zp(b0);
    if (b1 < nblk) {
      zT1 = __int_as_float(reinterpret_cast<const int*>(rec_h + b1 * (int64_t)REC_BYTES + REC_SC)[SC_ET]);
      if constexpr (ZE == 2) zd1 = *reinterpret_cast<const float2*>(zp(b1));
      else zd1.x = *zp(b1);
    }
  };
  auto zscan = [&](int st) {
    const int b0 = 2 * st, b1 = 2 * st + 1;
    float2 s{}, s1{}, s2{};
    s.x = zrun[tid][0];
    if constexpr (ZE == 2) s.y = zrun[tid][1];
    s1.x = zT0 * s.x + zd0.x;
    s1.y = zT0 * s.y + zd0.y;
    s2 = s1;
    if (b1 < nblk) {
      s2.x = zT1 * s1.x + zd1.x;
      s2.y = zT1 * s1.y + zd1.y;
    }
    if (zact) {  // (Z entering the step, in its first block's slot)
      if constexpr (ZE == 2) *reinterpret_cast<float2*>(zp(b0)) = s;
      else *zp(b0) = s.x;
    }
    zrun[tid][0] = s2.x;
    if constexpr (ZE == 2) zrun[tid][1] = s2.y;
  };

  // state: a-tile at (32 values of a), b-tile bt -> 32 x 32 accumulator over
  // (b) x (a = 32 at + n32), value column c0 + cl; lane (n32, h) holds the
  // rows b = 32 bt + 8 q + 4 h + s in register 4 q + s
  f32x16 S[NAT][2];
  constexpr int A1 = NAT - 1;  // the second a-tile (used with NAT = 2 only)
#pragma unroll
  for (int p = 0; p < NAT; ++p)
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) S[p][bt] = f32x16{};
  // fp16 copy of the first a-tile's state, made at the end of the previous
  // step's update so that the first output chain can start at once
  f16x8 SA0[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) SA0[kk] = f16x8{};

  // MFMA work of step st; AT is the a-tile of the wave's first tile.  Output
  // over token tiles t (32 tokens: block t / 2, rows 32 (t % 2) ..):
  // T^T[a][i] = sum_b S_c[b][a] Q[i][b] over 16-row k-steps kk (b in 16 kk +
  // {4h..4h+3, 8+4h..8+4h+3} on lane half h, matching the record's q column
  // order), then Y[i] += sum_a q_ia T^T[a][i].  Update: S_c = eTs S_c + sum
  // over both blocks hb of K^T ((k_:a 2^kap) * X_:c 2^(sig - 2 kap)) over
  // 16-token k-steps (tokens 16 kk + 8 h .. +7 on lane half h).
  auto compute = [&](int st, auto ATc) {
    constexpr int AT = decltype(ATc)::value;
    const int sl = st & 1;
    const float eT = cur.eTs;

    f16x8 SA1[4];         // fp16 copy of the second a-tile's state
    f16x8 Qf[4][4];       // B operand of the output: Q^T[b][i] of token tile t
    f32x16 T[NAT][4];     // output chains (a-tile, token tile)
    f32x4 Y[4] = {zero4(), zero4(), zero4(), zero4()};  // four independent partial sums per tile
    f16x8 xh[2][4];       // X^T[c][j] of block hb (the same on every lane of a half)
    f16x8 Bu[NAT][2][4];  // update B operand
    f16x8 Kf[2][2][4];    // K^T[b][j] of block hb, b = 32 bt + n32

    auto SB = [] { __builtin_amdgcn_sched_barrier(0); };
    auto rdQ = [&](int t, int kk) {
      Qf[t][kk] = *reinterpret_cast<const f16x8*>(&Qh[sl][t >> 1][((t & 1) * 32 + n32) * PH + kk * 16 + 8 * h]);
    };
    auto rdK = [&](int bt, int hb, int kk) {
      Kf[hb][bt][kk] = *reinterpret_cast<const f16x8*>(&KTh[sl][hb][(bt * 32 + n32) * PH + kk * 16 + 8 * h]);
    };
    auto rdX = [&](int hb, int kk) {
      xh[hb][kk] = *reinterpret_cast<const f16x8*>(&Xh[sl][hb][cl * PH + kk * 16 + 8 * h]);
    };
    // MFMAs (at: the wave's tile index, AT + at the a-tile)
    auto out = [&](int at, int t, int kk) {
      const f16x8* SA = at == 0 ? SA0 : SA1;
      T[at][t] = mfma32(SA[kk], Qf[t][kk], kk == 0 ? f32x16{} : T[at][t]);
    };
    auto upd = [&](int at, int bt, int hb, int kk) {
      S[at][bt] = mfma32(Kf[hb][bt][kk], Bu[at][hb][kk], S[at][bt]);
    };
    // VALU units (four instructions each); the empty asm consumes a
    // conversion's result in place, so that it is not moved to the loop's
    // end where its value is carried
    auto cvt = [&](f16x8* SA, int at, int kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) SA[kk][e] = (_Float16)S[at][kk >> 1][8 * (kk & 1) + e];
      asm volatile("" ::"v"(SA[kk]));
    };
    auto mul = [&](int at, int bt, int g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) S[at][bt][4 * g + e] *= eT;
    };
    // two a-tiles per wave: the state is symmetric in (a, b), so the tile of
    // a-tile 0 and b-tile 1 is the transpose of S[1][0] and is not held; its
    // share of the output, sum_{a in 0, b in 1} q_a q_b S[b][a], equals that
    // of S[1][0], so the second a-tile's chain takes twice S[1][0] (over
    // kk = 0, 1) in high and low fp16 parts (the one fp16 copy then carries
    // no rounding that the missing tile would have averaged out), then
    // S[1][1] (kk = 2, 3); the first a-tile's chain takes S[0][0] alone
    f16x8 SH[2], SL[2];
    auto cvh = [&](int kk, int p) {
      const float x0 = S[A1][0][8 * kk + 2 * p], x1 = S[A1][0][8 * kk + 2 * p + 1];
      f16x2 hh = __builtin_convertvector((f32x2){x0, x1}, f16x2);
      hh = hh + hh;  // = fp16(2 x), exact: |2 S 2^sig| < 2^14
      // the low part of 2 x: 2 x - hh is exact in fp32, formed by one mixed
      // fp32 / fp16 fma per value (no conversion of hh back to fp32)
      const f32x2 r = {fmaf(x0, 2.f, -(float)hh[0]), fmaf(x1, 2.f, -(float)hh[1])};
      const f16x2 ll = __builtin_convertvector(r, f16x2);
      SH[kk][2 * p] = hh[0];
      SH[kk][2 * p + 1] = hh[1];
      SL[kk][2 * p] = ll[0];
      SL[kk][2 * p + 1] = ll[1];
    };
    auto outp = [&](int t, int j) {
      const f16x8& A = j < 2 ? SH[j] : j < 4 ? SL[j - 2] : SA1[j - 2];
      const int kk = j < 4 ? (j & 1) : j - 2;
      T[A1][t] = mfma32(A, Qf[t][kk], j == 0 ? f32x16{} : T[A1][t]);
    };
    // rows 8 m + 4 h + s of T: a = 32 (AT + at) + 8 m + 4 h + s, whose q value
    // is element 4 (m % 2) + s of the lane's Q fragment 2 (AT + at) + m / 2
    auto fy = [&](int at, int t, int m) {
      const f16x8& qf = Qf[t][2 * (AT + at) + (m >> 1)];
#pragma unroll
      for (int s = 0; s < 4; ++s) Y[t][s] = fmaf((float)qf[4 * (m & 1) + s], T[at][t][4 * m + s], Y[t][s]);
    };
    // k_ja for a = 32 (AT + at) + n32 is the lane's K^T fragment of b-tile AT + at
    auto bu = [&](int at, int hb, int kk) { Bu[at][hb][kk] = Kf[hb][AT + at][kk] * xh[hb][kk]; };
    // each token's sum over the a's of the wave (the two lane halves hold
    // different a's), written by both halves to the same place
    auto wr = [&] {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float y = (Y[t][0] + Y[t][1]) + (Y[t][2] + Y[t][3]);
        // y + (y of lane ^ 32) without an LDS round trip: swapping the
        // halves of two copies gives the lower and the upper half's value
        // on every lane
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
        y = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        yo[sl][t >> 1][((t & 1) * 32 + n32) * RP + yi] = y;
      }
    };

    if constexpr (NAT == 2) {
      // -- generated schedule, 2 a-tiles per wave --
      rdQ(0, 0); rdQ(0, 1); rdQ(0, 2); rdQ(0, 3); rdQ(1, 0); rdQ(1, 1); cvh(0, 0); cvh(0, 1); SB();
      out(0, 0, 0); cvh(0, 2); SB();
      out(0, 0, 1); cvh(0, 3); cvh(1, 0); SB();
      out(0, 1, 0); cvh(1, 1); SB();
      out(0, 1, 1); cvh(1, 2); cvh(1, 3); SB();
      outp(0, 0); cvt(SA1, 1, 2); SB();
      outp(0, 1); cvt(SA1, 1, 3); fy(0, 0, 0); rdQ(1, 2); SB();
      outp(0, 2); fy(0, 0, 1); rdQ(1, 3); SB();
      outp(0, 3); fy(0, 0, 2); fy(0, 0, 3); rdQ(2, 0); SB();
      outp(0, 4); fy(0, 1, 0); rdQ(2, 1); SB();
      outp(0, 5); fy(0, 1, 1); fy(0, 1, 2); rdQ(3, 0); SB();
      outp(1, 0); fy(0, 1, 3); rdQ(3, 1); SB();
      outp(1, 1); mul(0, 0, 0); mul(0, 0, 1); SB();
      outp(1, 2); fy(1, 0, 0); SB();
      outp(1, 3); fy(1, 0, 1); fy(1, 0, 2); SB();
      outp(1, 4); fy(1, 0, 3); SB();
      outp(1, 5); mul(0, 0, 2); mul(0, 0, 3); rdQ(2, 2); SB();
      out(0, 2, 0); mul(1, 0, 0); rdQ(2, 3); SB();
      out(0, 2, 1); mul(1, 0, 1); mul(1, 0, 2); SB();
      out(0, 3, 0); fy(1, 1, 0); SB();
      out(0, 3, 1); fy(1, 1, 1); fy(1, 1, 2); SB();
      outp(2, 0); fy(1, 1, 3); rdK(0, 0, 0); SB();
      outp(2, 1); fy(0, 2, 0); fy(0, 2, 1); rdQ(3, 2); SB();
      outp(2, 2); fy(0, 2, 2); rdQ(3, 3); SB();
      outp(2, 3); fy(0, 2, 3); fy(0, 3, 0); rdK(1, 0, 0); SB();
      outp(2, 4); fy(0, 3, 1); rdX(0, 0); SB();
      outp(2, 5); fy(0, 3, 2); fy(0, 3, 3); rdK(0, 0, 1); SB();
      outp(3, 0); mul(1, 0, 3); rdK(1, 0, 1); SB();
      outp(3, 1); bu(0, 0, 0); bu(1, 0, 0); rdX(0, 1); SB();
      outp(3, 2); fy(1, 2, 0); rdK(0, 0, 2); SB();
      outp(3, 3); fy(1, 2, 1); rdK(1, 0, 2); SB();
      outp(3, 4); bu(0, 0, 1); rdX(0, 2); rdK(0, 0, 3); SB();
      outp(3, 5); fy(1, 2, 2); rdK(1, 0, 3); rdX(0, 3); SB();
      upd(0, 0, 0, 0); fy(1, 2, 3); rdK(0, 1, 0); SB();
      upd(0, 0, 0, 1); bu(0, 0, 2); rdK(1, 1, 0); SB();
      upd(0, 0, 0, 2); bu(0, 0, 3); rdX(1, 0); SB();
      upd(0, 0, 0, 3); bu(1, 0, 1); rdK(0, 1, 1); SB();
      upd(1, 0, 0, 0); bu(1, 0, 2); rdK(1, 1, 1); SB();
      upd(1, 0, 0, 1); bu(1, 0, 3); rdX(1, 1); SB();
      upd(1, 0, 0, 2); mul(1, 1, 0); mul(1, 1, 1); rdK(0, 1, 2); SB();
      upd(1, 0, 0, 3); mul(1, 1, 2); mul(1, 1, 3); rdK(1, 1, 2); SB();
      upd(1, 1, 0, 0); fy(1, 3, 0); fy(1, 3, 1); rdX(1, 2); SB();
      upd(1, 1, 0, 1); fy(1, 3, 2); fy(1, 3, 3); rdK(0, 1, 3); SB();
      upd(1, 1, 0, 2); bu(0, 1, 0); rdK(1, 1, 3); wr(); SB();
      upd(1, 1, 0, 3); bu(0, 1, 1); rdX(1, 3); SB();
      upd(0, 0, 1, 0); bu(0, 1, 2); SB();
      upd(0, 0, 1, 1); bu(1, 1, 0); SB();
      upd(0, 0, 1, 2); bu(0, 1, 3); SB();
      upd(0, 0, 1, 3); bu(1, 1, 1); SB();
      upd(1, 0, 1, 0); bu(1, 1, 2); SB();
      upd(1, 0, 1, 1); bu(1, 1, 3); SB();
      upd(1, 0, 1, 2); cvt(SA0, 0, 0); SB();
      upd(1, 0, 1, 3); cvt(SA0, 0, 1); SB();
      upd(1, 1, 1, 0); SB();
      upd(1, 1, 1, 1); SB();
      upd(1, 1, 1, 2); SB();
      upd(1, 1, 1, 3); SB();
      // -- end of generated schedule --
    } else {
      // -- generated schedule, 1 a-tile per wave --
      rdQ(0, 0); rdQ(0, 1); rdQ(0, 2); rdQ(0, 3); rdQ(1, 0); rdQ(1, 1); rdQ(1, 2); rdQ(1, 3); SB();
      out(0, 0, 0); mul(0, 0, 0); rdK(0, 0, 0); SB();
      out(0, 0, 1); mul(0, 0, 1); rdK(1, 0, 0); SB();
      out(0, 0, 2); mul(0, 0, 2); rdX(0, 0); SB();
      out(0, 0, 3); mul(0, 0, 3); rdK(0, 0, 1); SB();
      out(0, 1, 0); mul(0, 1, 0); rdK(1, 0, 1); rdX(0, 1); SB();
      out(0, 1, 1); bu(0, 0, 0); rdK(0, 0, 2); rdK(1, 0, 2); SB();
      out(0, 1, 2); mul(0, 1, 1); rdX(0, 2); rdK(0, 0, 3); SB();
      out(0, 1, 3); bu(0, 0, 1); rdK(1, 0, 3); rdX(0, 3); SB();
      upd(0, 0, 0, 0); mul(0, 1, 2); rdQ(2, 0); SB();
      upd(0, 0, 0, 1); bu(0, 0, 2); rdQ(2, 1); SB();
      upd(0, 0, 0, 2); bu(0, 0, 3); rdQ(2, 2); SB();
      upd(0, 0, 0, 3); mul(0, 1, 3); rdQ(2, 3); SB();
      upd(0, 1, 0, 0); fy(0, 0, 0); fy(0, 0, 1); rdQ(3, 0); SB();
      upd(0, 1, 0, 1); fy(0, 0, 2); fy(0, 0, 3); rdQ(3, 1); SB();
      upd(0, 1, 0, 2); fy(0, 1, 0); rdQ(3, 2); SB();
      upd(0, 1, 0, 3); fy(0, 1, 1); rdQ(3, 3); SB();
      out(0, 2, 0); fy(0, 1, 2); rdK(0, 1, 0); SB();
      out(0, 2, 1); fy(0, 1, 3); rdK(1, 1, 0); SB();
      out(0, 2, 2); rdX(1, 0); SB();
      out(0, 2, 3); rdK(0, 1, 1); SB();
      out(0, 3, 0); rdK(1, 1, 1); rdX(1, 1); SB();
      out(0, 3, 1); bu(0, 1, 0); rdK(0, 1, 2); rdK(1, 1, 2); SB();
      out(0, 3, 2); fy(0, 2, 0); rdX(1, 2); rdK(0, 1, 3); SB();
      out(0, 3, 3); bu(0, 1, 1); rdK(1, 1, 3); rdX(1, 3); SB();
      upd(0, 0, 1, 0); fy(0, 2, 1); SB();
      upd(0, 0, 1, 1); bu(0, 1, 2); SB();
      upd(0, 0, 1, 2); bu(0, 1, 3); SB();
      upd(0, 0, 1, 3); fy(0, 2, 2); SB();
      upd(0, 1, 1, 0); fy(0, 2, 3); SB();
      upd(0, 1, 1, 1); fy(0, 3, 0); fy(0, 3, 1); SB();
      upd(0, 1, 1, 2); fy(0, 3, 2); fy(0, 3, 3); SB();
      upd(0, 1, 1, 3); cvt(SA0, 0, 0); wr(); SB();
      cvt(SA0, 0, 1); cvt(SA0, 0, 2); cvt(SA0, 0, 3); SB();
      // -- end of generated schedule --
    }
  };

  // prologue: the initial states (if any), stage step 0, prefetch step 1
  prefetch(0);
  cur = nx;
  stage(0);
  prefetch(nstep > 1 ? 1 : 0);
  if (wave < NW / 2) {
    // running normaliser sums: zero, or the initial state's stored entries
#pragma unroll
    for (int e = 0; e < ZE; ++e) {
      float z = 0.f;
      if (Z0) {
        const int E = pc * ZPW + zi + e, t = E >> 8, w = E & 255;
        const int bt = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3, ct = bt + t - z_tile(bt, bt);
        z = Z0[bh * DH * DH + (16 * bt + (w >> 4)) * DH + 16 * ct + (w & 15)];
      }
      zrun[tid][e] = z;
    }
    zload(0);
    zscan(0);
  }
  __syncthreads();

  // initial numerator state, S0[a][b][c] (row (a, b) of H_up, the layout of
  // final_state), taken at the top of the first step: the workgroup's
  // columns c0 .. c0 + CWG - 1 pass through LDS (q's second staging slot,
  // not written before the first step's staging) in passes of AP values of
  // a; each lane then takes its accumulator entries, scaled to the first
  // step's 2^sig_in, and forms the fp16 copy of its first a-tile.  (Loaded
  // before the loop instead, the accumulators' longer live range makes the
  // register allocator spill inside the loop.)
  auto load_initial_state = [&] {
    // AS: floats per value of a, padded so that the lanes of a pass (eight
    // consecutive a) read distinct LDS banks
    constexpr int AP = 8, V4 = CWG / 4, AS = DH * CWG + 4;
    static_assert(AP * AS * sizeof(float) <= sizeof(Qh[1]), "initial-state staging fits");
    float* buf = reinterpret_cast<float*>(&Qh[1][0][0]);
    const float* s0h = S0 + bh * (int64_t)DH * DH * DH;
    const float sc = ldexpf(1.f, cur.sig_in);
#pragma unroll 1
    for (int pass = 0; pass < DH / AP; ++pass) {
      for (int e = tid; e < AP * DH * V4; e += NT) {
        const int row = e / V4, part = e % V4;  // row = (a - AP pass) * 64 + b
        const int64_t a = AP * pass + row / DH, b = row % DH;
        *reinterpret_cast<f32x4*>(&buf[(row / DH) * AS + (row % DH) * CWG + 4 * part]) =
            *reinterpret_cast<const f32x4*>(&s0h[(a * DH + b) * DH + c0 + 4 * part]);
      }
      __syncthreads();
#pragma unroll
      for (int at = 0; at < NAT; ++at) {
        const int a = 32 * (NAT == 2 ? at : (wave >> 2)) + n32;
        if (a / AP == pass) {
#pragma unroll
          for (int bt = 0; bt < 2; ++bt) {
            // (the state is symmetric in (a, b): with two a-tiles per wave the
            // rows (a, b), a >= 32 > b, stand for their mirrors (b, a) too)
            if (NAT == 2 && at == 0 && bt == 1) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int b = bt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
              S[at][bt][r] = buf[(a - AP * pass) * AS + b * CWG + cl] * sc;
            }
          }
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int kk = 0; kk < (NAT == 2 ? 2 : 4); ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) SA0[kk][e] = (_Float16)S[0][kk >> 1][8 * (kk & 1) + e];
  };

  // Per step m: MFMA work of m, write-out of m-1 (compute-first waves),
  // staging of m+1, loads of m+2, one barrier.  With two waves per SIMD the first four waves run the
  // MFMA work first and the other four the bookkeeping first; each group has
  // a loop of its own (every wave passes the same barriers), so the loads of
  // a step have a single destination and are waited for only where the
  // staging consumes them.  The loads for step m+2 are issued right after
  // the registers are free, a whole step ahead of their use.
  if (wave < NW / 2) {
    // the prologue's loads are complete before the loop: a load still in
    // flight at the loop's entry would make the compiler wait for every
    // outstanding load at the top of each step (also for the loads of step
    // st + 2, issued a step ahead)
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    for (int st = 0; st < nstep; ++st) {
      const Stp nxt = nx;  // scales of step st + 1 (prefetched)
      if constexpr (INIT)
        if (st == 0) load_initial_state();
      compute(st, std::integral_constant<int, 0>{});
      const bool zs = st + 1 < nstep;
      if (zs) zload(st + 1);
      if (st > 0) drain(st - 1, prv);
      stage(st + 1);
      prefetch(st + 2 < nstep ? st + 2 : nstep - 1);
      if (zs) zscan(st + 1);
      prv = cur;
      cur = nxt;
      __syncthreads();
    }
  } else {
    for (int st = 0; st < nstep; ++st) {
      const Stp nxt = nx;
      if constexpr (INIT)
        if (st == 0) load_initial_state();
      stage(st + 1);
      prefetch(st + 2 < nstep ? st + 2 : nstep - 1);
      compute(st, std::integral_constant<int, NAT == 2 ? 0 : 1>{});
      prv = cur;
      cur = nxt;
      __syncthreads();
    }
  }
  if (wave < NW / 2) {
    drain(nstep - 1, prv);
    if (final_norm && zact) {
      // the full d_h x d_h Z: an entry of an off-diagonal tile also goes to
      // its mirror position
      float* fz = final_norm + bh * DH * DH;
#pragma unroll
      for (int e = 0; e < ZE; ++e) {
        const int E = pc * ZPW + zi + e, t = E >> 8, w = E & 255;
        const int bt = t < 4 ? 0 : t < 7 ? 1 : t < 9 ? 2 : 3, ct = bt + t - z_tile(bt, bt);
        const int b = 16 * bt + (w >> 4), c = 16 * ct + (w & 15);
        const float z = zrun[tid][e];
        fz[b * DH + c] = z;
        if (bt != ct) fz[c * DH + b] = z;
      }
    }
  }

  if (final_state) {
    const float f = ldexpf(1.f, -prv.sig_out);
    const int c = c0 + cl;
#pragma unroll
    for (int at = 0; at < NAT; ++at) {
      const int a = 32 * (NAT == 2 ? at : (wave >> 2)) + n32;
#pragma unroll
      for (int bt = 0; bt < 2; ++bt) {
        if (NAT == 2 && at == 0 && bt == 1) continue;  // written as the mirror of S[1][0]
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = bt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const float x = S[at][bt][r] * f;
          final_state[((bh * DH + a) * DH + b) * DH + c] = x;
          if (NAT == 2 && at == 1 && bt == 0) final_state[((bh * DH + b) * DH + a) * DH + c] = x;
        }
      }
    }
  }
}

hipError_t launch_o2_state(const void* rec, int64_t BH, int64_t N, float* part,
                           float* final_state, float* zstate, float* final_norm, const float* S0,
                           const float* Z0, hipStream_t stream) {
  const int xcd_map = (BH % 8) == 0;
  const uint8_t* r = static_cast<const uint8_t*>(rec);
#define SSD_LAUNCH_O2(NATV, INITV, WGS)                                                       \
  hipLaunchKernelGGL((k_o2_state<NATV, INITV>), dim3((unsigned)(BH * (WGS))), dim3(512), 0,  \
                     stream, r, BH, N, xcd_map, part, final_state, zstate, final_norm, S0, Z0)
  if (o2_nat(BH) == 2) {
    if (S0) SSD_LAUNCH_O2(2, true, 8);
    else SSD_LAUNCH_O2(2, false, 8);
  } else {
    if (S0) SSD_LAUNCH_O2(1, true, 16);
    else SSD_LAUNCH_O2(1, false, 16);
  }
#undef SSD_LAUNCH_O2
  return hipGetLastError();
}

}  // namespace ssd
