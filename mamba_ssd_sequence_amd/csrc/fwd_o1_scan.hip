// Order-1 forward (Mamba-2S: Algorithms 1, 3, 4; the state of Algorithm 6)
// with bf16 inputs, as one sequential scan over the 64-token blocks per
// (head, segment of the sequence).  The d_h x d_h state never leaves the
// chip: each block is read once (q, k, v, dt, a_cs), its outputs are the
// masked product within the block plus the decayed inter-block term
// e^{cs_i} q_i^T S, normalised by the row sum plus e^{cs_i} q_i . z, and the
// state then advances to the end of the block,
// S <- e^T S + sum_j w_j k_j (v dt)_j^T, z <- e^T z + sum_j w_j k_j with
// w_j = e^{T - cs_j} (cs block-relative, T the block total; every exponent
// is a non-positive difference of chunk-local cumsums).
//
// Segments: the sequence is cut into nseg segments of whole blocks so that
// the heads times segments cover the CUs twice.  An aggregate pass
// (k_o1_segagg) writes the state contribution and total log-decay of each
// segment but the last, a prefix pass (k_o1_segprefix) turns them in place
// into the state entering each following segment (the initial state carried
// through S <- 2^{T_s'} S + A_s' for s' < s), and the scan of segment s
// starts from that one slot.  With at most O1_FOLD_SEGS segments there is no
// prefix pass: the scan sums the earlier segments' contributions itself.
//
// Per block, wave w owns query rows 16 w .. 16 w + 15 and (for the update)
// state rows b = 16 w .. 16 w + 15 (d_h 32: waves 0, 1), every value column.
// Products on v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
//   scores   s^T[j][i] = K Q^T (its accumulator layout is the B operand of the
//            next product after a permutation of k shared by both operands)
//   numer.   num^T[c][i] = sum_j v_jc (w_ij dt_j), w_ij = s_ij 2^{cs_i - cs_j}
//            (j <= i), w dt rounded to bf16 once (v is exact in bf16)
//   inter    inter^T[c][i] = sum_b S^T[c][b] q_ib, the state in high + low
//            bf16 parts (a single rounding would be amplified where q is
//            nearly orthogonal to the keys)
//   update   S[b][c] += sum_j (k_jb dw_j) v_jc, dw_j = w_j dt_j, the fp32
//            operand in high + low bf16 parts
// The score exponentials, the rounding of w dt and the split of k dw are
// done once per block and serve every value column.
// Each wave's query rows stay in registers (the only operand it alone uses).
// LDS: two sets of block operands (the next block is staged while this one
// is computed; its global loads, and the next query rows, are issued one
// block ahead) and one copy of the state operand, written between two
// barriers; 76 KB at d_h 64, so that two workgroups share a CU.  Index
// arithmetic is 32-bit within a head (N d_h < 2^31, checked by the caller).
#include "common.h"
#include "launch.h"

namespace ssd {

// up to this many segments per head the scan sums the earlier segments'
// contributions itself (no prefix pass)
constexpr int O1_FOLD_SEGS = 8;

namespace {

template <int DH>
struct alignas(16) O1Set {
  static constexpr int PQ = DH + 8;   // pitch (elements) of rows indexed by feature
  static constexpr int PJ = BLK + 8;  // pitch of rows indexed by token
  __bf16 K[BLK * PQ];   // [j][d]
  __bf16 KT[DH * PJ];   // [d][j]
  __bf16 VT[DH * PJ];   // [c][j]
  float cs[BLK];        // block-relative cumsum, log2 units
  float dt[BLK];        // dt (1 without dt), 0 past the block's end
  float w[BLK];         // 2^{T - cs_j}, 0 past the block's end
  float dw[BLK];        // w_j dt_j
  float T;              // block total, log2 units
};

template <int DH>
struct alignas(16) O1State {
  static constexpr int PS = DH + 8;
  __bf16 hi[DH * PS];  // [c][b]
  __bf16 lo[DH * PS];
  float z[DH];
};

// Global reads of one block held in registers until staged.  Block operands
// past a ragged block's end are copies of its last valid row (finite); every
// product that could see them carries a zero weight there.
struct O1Regs {
  uint4 k0, k1, v0, v1;
  float cs, dt;  // a_cs and dt of token tid % 64 (clamped to the block)
};

}  // namespace

template <int DH>
__global__ __launch_bounds__(256) void k_o1_scan(const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ k,
                                                 const uint16_t* __restrict__ v,
                                                 const float* __restrict__ dt,
                                                 const float* __restrict__ a_cs, int BH, int N,
                                                 int chunk_blocks, int nseg, int nbs,
                                                 const float* __restrict__ S0,
                                                 const float* __restrict__ z0,
                                                 float* __restrict__ agg, float* __restrict__ y,
                                                 float* __restrict__ den, float* __restrict__ Sf,
                                                 float* __restrict__ zf, float* __restrict__ sink) {
  constexpr int NCT = DH / 16;          // 16-column tiles of the values
  constexpr int SEG = DH / 8;           // 16-byte segments per row
  constexpr int NKP = (BLK / 2) * SEG;  // threads staging k and v as token pairs
  constexpr int NSW = DH / 16;          // waves that hold state rows
  constexpr int AGGF = DH * DH + DH + 1;  // floats per aggregate
  using Set = O1Set<DH>;
  using Stt = O1State<DH>;
  constexpr int PQ = Set::PQ, PJ = Set::PJ, PS = Stt::PS;
  constexpr int NKS = DH / 32;          // 32-wide steps over d
  static_assert(NKP <= 256, "load mapping");
  __shared__ __attribute__((aligned(16))) Set sets[2];
  __shared__ __attribute__((aligned(16))) Stt sts[1];

  const int p = blockIdx.x;
  if (p >= BH * nseg) return;
  const int bh = p / nseg, seg = p - bh * nseg;
  const int nblk = (N + BLK - 1) / BLK;
  const int b0 = seg * nbs, b1 = b0 + nbs < nblk ? b0 + nbs : nblk;
  // per-head bases; offsets within a head are 32-bit
  const uint16_t* qh = q + (int64_t)bh * N * DH;
  const uint16_t* kh = k + (int64_t)bh * N * DH;
  const uint16_t* vh = v + (int64_t)bh * N * DH;
  const float* csh = a_cs + (int64_t)bh * N;
  const float* dth = (dt ? dt : a_cs) + (int64_t)bh * N;

  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int il = 16 * wv + n;  // query row of this lane
  const bool sw = wv < NSW;    // this wave holds state rows 16 wv .. 16 wv + 15
  const int bs = 16 * wv + n;  // its z entry

  // ---- global loads of block b into registers ----------------------------
  // Every thread issues the same loads for every block, at rows clamped to
  // the block's valid rows, so the loop body's memory operations are
  // straight-line and the compiler's wait before staging counts only the
  // loads it needs.
  const int tk = tid % NKP, jp = 2 * (tk / SEG), sgp = tk % SEG;  // token pair, segment
  auto load_block = [&](int b, O1Regs& R) {
    const int t0 = b * BLK;
    const int last = (N - t0 < BLK ? N - t0 : BLK) - 1;
    const int ja = t0 + (jp < last ? jp : last), jb = t0 + (jp + 1 < last ? jp + 1 : last);
    R.k0 = *reinterpret_cast<const uint4*>(kh + ja * DH + sgp * 8);
    R.k1 = *reinterpret_cast<const uint4*>(kh + jb * DH + sgp * 8);
    R.v0 = *reinterpret_cast<const uint4*>(vh + ja * DH + sgp * 8);
    R.v1 = *reinterpret_cast<const uint4*>(vh + jb * DH + sgp * 8);
    const int tl = lane < last ? lane : last;
    R.cs = csh[t0 + tl];
    R.dt = dth[t0 + tl];
  };

  // ---- staging of block b from registers into a buffer set ---------------
  // a_cs is chunk-local and a block never straddles a chunk: the cumsum
  // before block b is 0 at a chunk start, else the last a_cs of block b - 1
  // (full, same chunk), carried in prev_raw (wave 0)
  float prev_raw = 0.f;
  auto stage_block = [&](int b, const O1Regs& R, Set& S) {
    const int nv = N - b * BLK < BLK ? N - b * BLK : BLK;
    if (tid < NKP) {
      *reinterpret_cast<uint4*>(&S.K[jp * PQ + sgp * 8]) = R.k0;
      *reinterpret_cast<uint4*>(&S.K[(jp + 1) * PQ + sgp * 8]) = R.k1;
      // transposed: the token pair (jp, jp + 1) of one feature / column per store
      const uint32_t a[4] = {R.k0.x, R.k0.y, R.k0.z, R.k0.w};
      const uint32_t c[4] = {R.k1.x, R.k1.y, R.k1.z, R.k1.w};
      const uint32_t e[4] = {R.v0.x, R.v0.y, R.v0.z, R.v0.w};
      const uint32_t f[4] = {R.v1.x, R.v1.y, R.v1.z, R.v1.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int d = sgp * 8 + 2 * u;
        *reinterpret_cast<uint32_t*>(&S.KT[d * PJ + jp]) = (a[u] & 0xffffu) | (c[u] << 16);
        *reinterpret_cast<uint32_t*>(&S.KT[(d + 1) * PJ + jp]) = (a[u] >> 16) | (c[u] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&S.VT[d * PJ + jp]) = (e[u] & 0xffffu) | (f[u] << 16);
        *reinterpret_cast<uint32_t*>(&S.VT[(d + 1) * PJ + jp]) = (e[u] >> 16) | (f[u] & 0xffff0000u);
      }
    }
    if (tid < BLK) {  // wave 0
      // the block's last a_cs sits in lane nv - 1
      const float lastv = __shfl(R.cs, nv - 1, WAVE);
      const float base = (b % chunk_blocks == 0) ? 0.f : prev_raw;
      prev_raw = lastv;
      const float T = (lastv - base) * LOG2E;
      const bool ok = tid < nv;
      const float cs = ok ? (R.cs - base) * LOG2E : T;
      const float w = ok ? exp2_fast(T - cs) : 0.f;
      const float d = ok ? (dt ? R.dt : 1.f) : 0.f;
      S.cs[tid] = cs;
      S.dt[tid] = d;
      S.w[tid] = w;
      S.dw[tid] = w * d;
      if (tid == 0) S.T = T;
    }
  };

  // ---- the state entering the segment -------------------------------------
  // lane (n, g) of a state wave: st[ct][r] = S[b = 16 wv + 4 g + r][c = 16 ct + n],
  // zs = z[bs]
  f32x4 st[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) st[ct] = zero4();
  float zs = 0.f;
  const int sb = 16 * wv + 4 * g;  // first state row of this lane
  // this lane's query fragments q[il][32 ks + 8 g .. + 7] (the B operand of
  // the scores and of the inter product), one block ahead
  auto load_q = [&](int b, bf16x8 (&qf)[NKS]) {
    const int t0 = b * BLK;
    const int last = (N - t0 < BLK ? N - t0 : BLK) - 1;
    const int r = t0 + (il < last ? il : last);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qh + r * DH + 32 * ks + 8 * g);
  };
  // the state as the inter product's operand: S^T[c][b] in high and low parts
  auto write_state = [&](Stt& S) {
    if (sw) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        bf16x4 h4, l4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 h = (__bf16)st[ct][r];
          h4[r] = h;
          l4[r] = (__bf16)(st[ct][r] - (float)h);
        }
        *reinterpret_cast<bf16x4*>(&S.hi[(16 * ct + n) * PS + sb]) = h4;
        *reinterpret_cast<bf16x4*>(&S.lo[(16 * ct + n) * PS + sb]) = l4;
      }
      if (g == 0) S.z[bs] = zs;
    }
  };
  if (b0 % chunk_blocks != 0) prev_raw = csh[b0 * BLK - 1];
  O1Regs R;
  bf16x8 qc[NKS], qn[NKS];
  load_q(b0, qn);
  load_block(b0, R);
  // the state entering the segment, read while the first block's loads are
  // in flight: the initial state for the first segment, else the prefix
  // that k_o1_segprefix left in the previous segment's aggregate slot
  if (sw && nseg <= O1_FOLD_SEGS && seg > 0) {
    // few segments: k_o1_segagg left each earlier segment's own contribution
    // A_s (from a zero state) and log2 decay total T_s, and the entering
    // state is summed here, latest segment first,
    //   E = sum_{l < seg} 2^{d_l} A_{seg-1-l} + 2^{d_seg} S0,
    //   d_l = sum_{l' < l} T_{seg-1-l'};
    // every slot's loads are issued at once (indices past the first segment
    // clamped to it, with a zero weight)
    const float* base = agg + (int64_t)bh * (nseg - 1) * AGGF;
    float d = 0.f;
#pragma unroll
    for (int l = 0; l < O1_FOLD_SEGS - 1; ++l) {
      const int sl = seg - 1 - l >= 0 ? seg - 1 - l : 0;
      const float* sp = base + (int64_t)sl * AGGF;
      const float sc = l < seg ? exp2_fast(d) : 0.f;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ct][r] += sc * sp[(sb + r) * DH + 16 * ct + n];
      zs += sc * sp[DH * DH + bs];
      if (l < seg) d += sp[DH * DH + DH];
    }
    if (S0) {
      const float sc = exp2_fast(d);
      const float* sp = S0 + (int64_t)bh * DH * DH;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ct][r] += sc * sp[(sb + r) * DH + 16 * ct + n];
      zs += sc * z0[(int64_t)bh * DH + bs];
    }
  } else if (sw) {
    const float* sp = nullptr;
    const float* zp0 = nullptr;
    if (seg > 0) {
      sp = agg + ((int64_t)bh * (nseg - 1) + seg - 1) * AGGF;
      zp0 = sp + DH * DH;
    } else if (S0) {
      sp = S0 + (int64_t)bh * DH * DH;
      zp0 = z0 + (int64_t)bh * DH;
    }
    if (sp) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ct][r] = sp[(sb + r) * DH + 16 * ct + n];
      zs = zp0[bs];
    }
  }
  write_state(sts[0]);
  stage_block(b0, R, sets[0]);
  load_block(b0 + 1 < b1 ? b0 + 1 : b1 - 1, R);
  // stores to the sink, as the loop body issues after its loads: the
  // compiler's count of memory operations in flight at the loop head then
  // agrees on both ways in
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) *reinterpret_cast<f32x4*>(sink + 4 * g) = st[ct];
  sink[16] = zs;
  __syncthreads();

  for (int b = b0; b < b1; ++b) {
    const int cur = (b - b0) & 1;
    Set& S = sets[cur];
    if (b + 1 < b1) stage_block(b + 1, R, sets[cur ^ 1]);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qc[ks] = qn[ks];
    load_q(b + 1 < b1 ? b + 1 : b1 - 1, qn);
    load_block(b + 2 < b1 ? b + 2 : b1 - 1, R);  // (a repeat of the last block at the end)
    const int t0 = b * BLK;
    const int nv = N - t0 < BLK ? N - t0 : BLK;

    {
      const Stt& SI = sts[0];
      const float cs_i = S.cs[il];
      // scores s(i = il, j = 16 jt + 4 g + r) for the key tiles jt <= wv,
      // masked and decayed; Wd = w dt
      f32x4 Wd[4];
      float den_l = 0.f;
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        Wd[jt] = zero4();
        if (jt <= wv) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            acc = mfma_bf16(*reinterpret_cast<const bf16x8*>(&S.K[(16 * jt + n) * PQ + 32 * ks + 8 * g]),
                            qc[ks], acc);
          const f32x4 csj = *reinterpret_cast<const f32x4*>(&S.cs[16 * jt + 4 * g]);
          const f32x4 dtj = *reinterpret_cast<const f32x4*>(&S.dt[16 * jt + 4 * g]);
          if (jt < wv && nv == BLK) {
            // a key tile wholly before the wave's rows of a full block: no mask
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float w = acc[r] * exp2_fast(cs_i - csj[r]);
              den_l += w;
              Wd[jt][r] = w * dtj[r];
            }
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int j = 16 * jt + 4 * g + r;
              const float w = (j <= il && j < nv) ? acc[r] * exp2_fast(cs_i - csj[r]) : 0.f;
              den_l += w;
              Wd[jt][r] = w * dtj[r];
            }
          }
        }
      }
      // num^T[c][i] = sum_j v_jc Wd(i, j); k order within a 32-wide step:
      // lane group g takes tokens 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3
      bf16x8 bw[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          bw[kb][r] = (__bf16)Wd[2 * kb][r];
          bw[kb][4 + r] = (__bf16)Wd[2 * kb + 1][r];
        }
      f32x4 num[NCT], inter[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        num[ct] = zero4();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (2 * kb <= wv) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(&S.VT[(16 * ct + n) * PJ + 32 * kb + 4 * g]);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(&S.VT[(16 * ct + n) * PJ + 32 * kb + 16 + 4 * g]);
            bf16x8 av;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              av[r] = lo[r];
              av[4 + r] = hi[r];
            }
            num[ct] = mfma_bf16(av, bw[kb], num[ct]);
          }
        }
        // inter^T[c][i] = sum_b S^T[c][b] q_ib, high + low parts
        inter[ct] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          inter[ct] = mfma_bf16(*reinterpret_cast<const bf16x8*>(&SI.hi[(16 * ct + n) * PS + 32 * ks + 8 * g]),
                                qc[ks], inter[ct]);
          inter[ct] = mfma_bf16(*reinterpret_cast<const bf16x8*>(&SI.lo[(16 * ct + n) * PS + 32 * ks + 8 * g]),
                                qc[ks], inter[ct]);
        }
      }
      // q . z over this lane's fragments (d = 32 ks + 8 g ..), then over the groups
      float den_x = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f32x4 za = *reinterpret_cast<const f32x4*>(&SI.z[32 * ks + 8 * g]);
        const f32x4 zb = *reinterpret_cast<const f32x4*>(&SI.z[32 * ks + 8 * g + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) den_x += (float)qc[ks][e] * za[e] + (float)qc[ks][4 + e] * zb[e];
      }
      den_x = sum_over_groups(den_x);
      den_l = sum_over_groups(den_l);
      const float ei = exp2_fast(cs_i);
      const float dtot = den_l + ei * den_x;
      // rows past a ragged block's end (and den when not asked for) go to
      // the sink, so that the stores too are unconditional; every lane group
      // writes the same den value
      const float rd = 1.f / dtot;
      float* yr = y + (int64_t)bh * N * DH + (t0 + il) * DH;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = (num[ct][r] + ei * inter[ct][r]) * rd;
        *reinterpret_cast<f32x4*>(il < nv ? yr + 16 * ct + 4 * g : sink + 4 * g) = o;
      }
      *(den && il < nv ? den + (int64_t)bh * N + t0 + il : sink + 16) = dtot;
    }

    // state update to the end of the block: S[b][c] = e^T S[b][c] +
    // sum_j (k_jb dw_j) v_jc, the operand k dw split once for every column tile
    const float T = S.T;
    if (sw) {
      const float eT = exp2_fast(T);
      // (z_b = sum_j w_j k_jb is summed over the same 16 tokens of this lane)
      bf16x8 ah[2], al[2];
      float zp = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 kt = *reinterpret_cast<const bf16x8*>(&S.KT[bs * PJ + 32 * ks + 8 * g]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&S.dw[32 * ks + 8 * g]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&S.dw[32 * ks + 8 * g + 4]);
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(&S.w[32 * ks + 8 * g]);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(&S.w[32 * ks + 8 * g + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kv = (float)kt[e];
          const float x = kv * (e < 4 ? d0[e] : d1[e - 4]);
          zp += kv * (e < 4 ? w0[e] : w1[e - 4]);
          const __bf16 h = (__bf16)x;
          ah[ks][e] = h;
          al[ks][e] = (__bf16)(x - (float)h);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        st[ct] *= eT;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&S.VT[(16 * ct + n) * PJ + 32 * ks + 8 * g]);
          st[ct] = mfma_bf16(ah[ks], bv, st[ct]);
          st[ct] = mfma_bf16(al[ks], bv, st[ct]);
        }
      }
      zs = eT * zs + sum_over_groups(zp);
    }
    if (b + 1 < b1) {
      __syncthreads();  // every wave is done with the state entering block b
      write_state(sts[0]);
    }
    __syncthreads();
  }

  {
    if (Sf && seg == nseg - 1 && sw) {
      float* sf = Sf + (int64_t)bh * DH * DH;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) sf[(sb + r) * DH + 16 * ct + n] = st[ct][r];
      if (g == 0) zf[(int64_t)bh * DH + bs] = zs;
    }
  }
}

// Segment aggregates (the scan forms each segment's entering state from them)
// with the four waves of a
// workgroup on four contiguous quarters of the segment at once: each wave
// runs its quarter's blocks with no barrier, A_w <- 2^T A_w + C_blk with
// C_blk = sum_j (k_j dw_j) (v_j)^T and z_w likewise, in its own LDS buffers;
// then A = sum_w 2^{T after quarter w} A_w, and the same for z.  The products
// are those of the scan's update (16x16x32 bf16, the operand k dw in high +
// low parts); z_b = sum_j w_j k_jb is summed alongside the split.
// (LDS admits two workgroups per CU at d_h 64, four at d_h 32; the
// waves-per-EU bound keeps the registers within what that many waves per SIMD
// allow)
template <int DH>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(128 / DH))) void k_o1_segagg(const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v,
                                                   const float* __restrict__ dt,
                                                   const float* __restrict__ a_cs, int BH, int N,
                                                   int chunk_blocks, int nseg, int nbs,
                                                   float* __restrict__ agg) {
  constexpr int NT = DH / 16;            // 16-wide tiles of the state rows and columns
  constexpr int SEG = DH / 8;            // 16-byte segments per row
  constexpr int NIT = (BLK / 2) * SEG / WAVE;  // (token pair, segment) items per lane
  constexpr int PJ = BLK + 8;
  constexpr int AGGF = DH * DH + DH + 1;
  struct alignas(16) WaveBuf {
    __bf16 KT[DH * PJ];  // [d][j]
    __bf16 VT[DH * PJ];  // [c][j]
    float w[BLK];        // 2^{T - cs_j}, 0 past the block's end
    float dw[BLK];       // w_j dt_j
  };
  static_assert(sizeof(WaveBuf) >= (DH * DH + DH) * sizeof(float), "partials fit a wave's buffer");
  __shared__ __attribute__((aligned(16))) WaveBuf wb[4];
  __shared__ float wT[4];

  const int p = blockIdx.x;
  if (p >= BH * (nseg - 1)) return;
  const int bh = p / (nseg - 1), seg = p - bh * (nseg - 1);
  const int nblk = (N + BLK - 1) / BLK;
  const int b0 = seg * nbs, b1 = b0 + nbs < nblk ? b0 + nbs : nblk;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int qr = (b1 - b0 + 3) / 4;  // blocks per quarter
  const int bw0 = b0 + wv * qr < b1 ? b0 + wv * qr : b1;
  const int bw1 = bw0 + qr < b1 ? bw0 + qr : b1;
  const uint16_t* kh = k + (int64_t)bh * N * DH;
  const uint16_t* vh = v + (int64_t)bh * N * DH;
  const float* csh = a_cs + (int64_t)bh * N;
  const float* dth = (dt ? dt : a_cs) + (int64_t)bh * N;
  WaveBuf& B = wb[wv];

  // acc[bt][ct][r] = A_w[b = 16 bt + 4 g + r][c = 16 ct + n]; zacc[bt]: z_w[16 bt + n]
  f32x4 acc[NT][NT];
#pragma unroll
  for (int bt = 0; bt < NT; ++bt)
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) acc[bt][ct] = zero4();
  float zacc[NT];
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) zacc[bt] = 0.f;
  float Tw = 0.f;

  uint4 rk0[NIT], rk1[NIT], rv0[NIT], rv1[NIT];
  float rcs = 0.f, rdt = 0.f;
  auto load = [&](int b) {
    const int t0 = b * BLK;
    const int last = (N - t0 < BLK ? N - t0 : BLK) - 1;
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const int it = lane + WAVE * u, jp = 2 * (it / SEG), sg = it % SEG;
      const int ja = t0 + (jp < last ? jp : last), jb = t0 + (jp + 1 < last ? jp + 1 : last);
      rk0[u] = *reinterpret_cast<const uint4*>(kh + ja * DH + sg * 8);
      rk1[u] = *reinterpret_cast<const uint4*>(kh + jb * DH + sg * 8);
      rv0[u] = *reinterpret_cast<const uint4*>(vh + ja * DH + sg * 8);
      rv1[u] = *reinterpret_cast<const uint4*>(vh + jb * DH + sg * 8);
    }
    const int tl = t0 + (lane < last ? lane : last);
    rcs = csh[tl];
    rdt = dth[tl];
  };
  float prev_raw = 0.f;
  if (bw0 < bw1 && bw0 % chunk_blocks != 0) prev_raw = csh[bw0 * BLK - 1];
  for (int b = bw0; b < bw1; ++b) {
    const int nv = N - b * BLK < BLK ? N - b * BLK : BLK;
    load(b);
    // stage this block (transposed token pairs)
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const int it = lane + WAVE * u, jp = 2 * (it / SEG), sg = it % SEG;
      const uint32_t a[4] = {rk0[u].x, rk0[u].y, rk0[u].z, rk0[u].w};
      const uint32_t c[4] = {rk1[u].x, rk1[u].y, rk1[u].z, rk1[u].w};
      const uint32_t e[4] = {rv0[u].x, rv0[u].y, rv0[u].z, rv0[u].w};
      const uint32_t f[4] = {rv1[u].x, rv1[u].y, rv1[u].z, rv1[u].w};
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int d = sg * 8 + 2 * uu;
        *reinterpret_cast<uint32_t*>(&B.KT[d * PJ + jp]) = (a[uu] & 0xffffu) | (c[uu] << 16);
        *reinterpret_cast<uint32_t*>(&B.KT[(d + 1) * PJ + jp]) = (a[uu] >> 16) | (c[uu] & 0xffff0000u);
        *reinterpret_cast<uint32_t*>(&B.VT[d * PJ + jp]) = (e[uu] & 0xffffu) | (f[uu] << 16);
        *reinterpret_cast<uint32_t*>(&B.VT[(d + 1) * PJ + jp]) = (e[uu] >> 16) | (f[uu] & 0xffff0000u);
      }
    }
    const float lastv = __shfl(rcs, nv - 1, WAVE);
    const float base = (b % chunk_blocks == 0) ? 0.f : prev_raw;
    prev_raw = lastv;
    const float T = (lastv - base) * LOG2E;
    {
      const bool ok = lane < nv;
      const float cs = ok ? (rcs - base) * LOG2E : T;
      const float w = ok ? exp2_fast(T - cs) : 0.f;
      B.w[lane] = w;
      B.dw[lane] = w * (ok ? (dt ? rdt : 1.f) : 0.f);
    }
    __builtin_amdgcn_wave_barrier();  // (the wave's own LDS writes precede its reads)

    const float eT = exp2_fast(T);
    Tw += T;
    if (b != bw0) {  // (the accumulators are still zero at the wave's first block)
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) acc[bt][ct] *= eT;
      }
    }
    float zp[NT];
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) zp[bt] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(&B.dw[32 * ks + 8 * g]);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(&B.dw[32 * ks + 8 * g + 4]);
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(&B.w[32 * ks + 8 * g]);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(&B.w[32 * ks + 8 * g + 4]);
      bf16x8 bv[NT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
        bv[ct] = *reinterpret_cast<const bf16x8*>(&B.VT[(16 * ct + n) * PJ + 32 * ks + 8 * g]);
#pragma unroll
      for (int bt = 0; bt < NT; ++bt) {
        const bf16x8 kt = *reinterpret_cast<const bf16x8*>(&B.KT[(16 * bt + n) * PJ + 32 * ks + 8 * g]);
        bf16x8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float kv = (float)kt[e];
          const float x = kv * (e < 4 ? d0[e] : d1[e - 4]);
          zp[bt] += kv * (e < 4 ? w0[e] : w1[e - 4]);
          const __bf16 h = (__bf16)x;
          ah[e] = h;
          al[e] = (__bf16)(x - (float)h);
        }
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) {
          acc[bt][ct] = mfma_bf16(ah, bv[ct], acc[bt][ct]);
          acc[bt][ct] = mfma_bf16(al, bv[ct], acc[bt][ct]);
        }
      }
    }
#pragma unroll
    for (int bt = 0; bt < NT; ++bt) zacc[bt] = eT * zacc[bt] + sum_over_groups(zp[bt]);
    __builtin_amdgcn_wave_barrier();  // (reads of this block before the next staging)
  }

  // combine the quarters: A = sum_w 2^{T_{w+1} + .. + T_3} A_w
  if (lane == 0) wT[wv] = Tw;
  __syncthreads();
  float after = 0.f;
  for (int w2 = wv + 1; w2 < 4; ++w2) after += wT[w2];
  const float f = exp2_fast(after);
  float* part = reinterpret_cast<float*>(&B);  // [b][c] then z[b]
#pragma unroll
  for (int bt = 0; bt < NT; ++bt) {
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[(16 * bt + 4 * g + r) * DH + 16 * ct + n] = f * acc[bt][ct][r];
    if (g == 0) part[DH * DH + 16 * bt + n] = f * zacc[bt];
  }
  __syncthreads();
  float* a = agg + ((int64_t)bh * (nseg - 1) + seg) * AGGF;
  for (int e = tid; e < DH * DH + DH; e += 256) {
    float x = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) x += reinterpret_cast<const float*>(&wb[w2])[e];
    a[e] = x;
  }
  if (tid == 0) a[DH * DH + DH] = (wT[0] + wT[1]) + (wT[2] + wT[3]);
}

// Prefix of the segment aggregates, in place: slot s (segment s's state
// contribution A_s, z contribution and log2 decay total T_s, from
// k_o1_segagg) becomes the state entering segment s + 1,
//   P_{s+1} = 2^{T_s} P_s + A_s,  P_0 = the initial state (or 0),
// for the d_h^2 state and d_h z entries (T_s is left as it is).  One thread
// per entry of a head's slot, its slots read eight at a time so that their
// loads are in flight together; the chain itself is the scan's former
// per-workgroup composition, done once per head instead of once per segment.
template <int DH>
__global__ __launch_bounds__(256) void k_o1_segprefix(int BH, int nseg, const float* __restrict__ S0,
                                                      const float* __restrict__ z0,
                                                      float* __restrict__ agg) {
  constexpr int NE = DH * DH + DH;  // state and z entries of a slot
  constexpr int AGGF = NE + 1;
  constexpr int PER = (NE + 255) / 256;  // workgroups per head
  const int bh = blockIdx.x / PER;
  const int e = (blockIdx.x - bh * PER) * 256 + threadIdx.x;
  if (bh >= BH || e >= NE) return;
  float* a = agg + (int64_t)bh * (nseg - 1) * AGGF;
  float p = 0.f;
  if (S0) p = e < DH * DH ? S0[(int64_t)bh * DH * DH + e] : z0[(int64_t)bh * DH + (e - DH * DH)];
  for (int s0 = 0; s0 < nseg - 1; s0 += 8) {
    float x[8], t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u < nseg - 1 ? s0 + u : nseg - 2;
      x[u] = a[(int64_t)s * AGGF + e];
      t[u] = a[(int64_t)s * AGGF + NE];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < nseg - 1) {
        p = exp2_fast(t[u]) * p + x[u];
        a[(int64_t)(s0 + u) * AGGF + e] = p;
      }
    }
  }
}

// Segments: enough workgroups for two per CU where the sequence allows,
// each segment at least 4 blocks.
void o1_scan_segments(int64_t BH, int64_t DH, int64_t N, int* nseg, int* nbs) {
  (void)DH;
  const int64_t nblk = (N + BLK - 1) / BLK;
  int64_t s = (512 + BH - 1) / BH;
  const int64_t smax = nblk / 4 > 1 ? nblk / 4 : 1;
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  const int64_t per = (nblk + s - 1) / s;
  *nbs = (int)per;
  *nseg = (int)((nblk + per - 1) / per);
}

size_t o1_scan_agg_floats(int64_t BH, int64_t DH, int64_t N) {
  int ns, nb;
  o1_scan_segments(BH, DH, N, &ns, &nb);
  return (size_t)(BH * (ns - 1)) * (size_t)(DH * DH + DH + 1);
}

bool o1_scan_supported(int64_t BH, int64_t DH, int64_t N) {
  return (DH == 32 || DH == 64) && N * DH < ((int64_t)1 << 31) &&
         BH * ((N + BLK - 1) / BLK) < ((int64_t)1 << 31);
}

hipError_t launch_o1_scan(bool agg_pass, int64_t DH, const void* q, const void* k, const void* v,
                          const float* dt, const float* a_cs, int64_t BH, int64_t N, int64_t chunk,
                          const float* S0, const float* z0, float* agg, float* y, float* den,
                          float* Sf, float* zf, float* sink, hipStream_t stream) {
  int nseg, nbs;
  o1_scan_segments(BH, DH, N, &nseg, &nbs);
  if (agg_pass && nseg == 1) return hipSuccess;  // a single segment needs no aggregates
  const int64_t P = BH * (agg_pass ? nseg - 1 : nseg);
  const dim3 grid((unsigned)P), blk(256);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  const int cb = (int)(chunk / BLK);
#define SSD_O1_SCAN(DHV)                                                                    \
  hipLaunchKernelGGL((k_o1_scan<DHV>), grid, blk, 0, stream, qq, kk, vv, dt, a_cs, (int)BH, \
                     (int)N, cb, nseg, nbs, S0, z0, agg, y, den, Sf, zf, sink)
  if (agg_pass) {
    const int64_t ne = DH * DH + DH;
    const dim3 gp((unsigned)(BH * ((ne + 255) / 256)));
    if (DH == 64) {
      hipLaunchKernelGGL((k_o1_segagg<64>), grid, blk, 0, stream, kk, vv, dt, a_cs, (int)BH, (int)N, cb,
                         nseg, nbs, agg);
      if (nseg > O1_FOLD_SEGS)
        hipLaunchKernelGGL((k_o1_segprefix<64>), gp, blk, 0, stream, (int)BH, nseg, S0, z0, agg);
    } else {
      hipLaunchKernelGGL((k_o1_segagg<32>), grid, blk, 0, stream, kk, vv, dt, a_cs, (int)BH, (int)N, cb,
                         nseg, nbs, agg);
      if (nseg > O1_FOLD_SEGS)
        hipLaunchKernelGGL((k_o1_segprefix<32>), gp, blk, 0, stream, (int)BH, nseg, S0, z0, agg);
    }
  } else {
    if (DH == 64) SSD_O1_SCAN(64);
    else SSD_O1_SCAN(32);
  }
#undef SSD_O1_SCAN
  return hipGetLastError();
}

}  // namespace ssd
