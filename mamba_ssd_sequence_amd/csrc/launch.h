// Internal (non-exported) launchers and workspace layout of libssd.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ssd {

// Forward work is organised in blocks of 64 tokens.
__host__ __device__ inline int64_t n_blocks(int64_t N) { return (N + 63) / 64; }

// Order-2 state kernel (8 waves per workgroup): a-tiles of 32 values of a
// per wave, 2 (one value column per wave, 8 columns per workgroup) with
// >= 32 heads, else 1 (two waves per column, 4 columns per workgroup), so that
// the grid still covers the chip.  A workgroup holds all 64 values of a, so
// its outputs are complete inter-block numerators (no partial sums).
inline int o2_nat(int64_t BH) { return BH >= 32 ? 2 : 1; }

// The order-2 numerator state scan advances over steps of two blocks
// (2m, 2m+1); a last step without partner gets an empty second block.
// Partial-output rows per head are padded to whole steps.
__host__ __device__ inline int64_t o2_part_rows(int64_t N) { return (n_blocks(N) + 1) / 2 * 2 * 64; }

// Order-2 per-block operand record (bytes), written by the block-prep kernel
// and read by the state scan:
//   QH  [64 i][64]   fp16 q_ib 2^tau; within each 16-column group the 4-column
//                    subgroups are stored in the order 0, 2, 1, 3 (the order in
//                    which the permuted-k 32x32 MFMA operand reads them)
//   KT  [64 b][64 j] fp16 k_jb 2^kap (transposed)
//   XT  [64 c][64 j] fp16 X_jc 2^xi, X_jc = w_j dt_j v_jc, w_j = e^{T - cs_j}
//                    for the second block of a step; the first block weights
//                    its tokens to the end of the step, w_j = e^{T + T' - cs_j}
//                    with T' the decay total of the second block
//   ECS [64]         fp32 e^{cs_i} (decay from the block start to token i)
//   SC  [12 words]   written by the block-prep kernel: fp32 T, fp32 delta
//                    (bound of any |entry| of the block's share of the step's
//                    state increment), int32 tau, kap, xi, fp32 e^T; then by
//                    the scale scan, for the step the block belongs to: int32
//                    sig_in (scale exponent of the state entering the step),
//                    fp32 eTs (e^{T_2m + T_2m+1} 2^(sig_out - sig_in), the
//                    factor that decays and rescales the state), two fp16
//                    factors taking X 2^xi to X 2^(sig_out - 2 kap), int32
//                    sig_out, fp32 epre (decay from the start of the step to
//                    the start of the block: 1 or e^{T_2m})
constexpr int REC_QH = 0, REC_KT = 8192, REC_XT = 16384, REC_ECS = 24576, REC_SC = 24832;
constexpr int SC_T = 0, SC_DELTA = 1, SC_TAU = 2, SC_KAP = 3, SC_XI = 4, SC_ET = 5, SC_SIG_IN = 6,
              SC_ETS = 7, SC_XF = 8, SC_SIG_OUT = 9, SC_EPRE = 10;
constexpr int REC_BYTES = 24880;

// Order-2 normaliser state Z (d_h = 64, symmetric) in a block's state slot:
// only its upper 16 x 16 tiles (bt <= ct, 10 of 16) are stored, tile (bt, ct)
// row-major at float offset 256 z_tile(bt, ct), so that Z[b][c] for
// b in tile bt <= ct and c in tile ct sits at 256 z_tile(bt, ct) + 16 (b % 16)
// + c % 16.
constexpr int Z_TILES = 10, Z_FLOATS = 256 * Z_TILES;

// An order-2 initial numerator state S0 is reduced to this many partial
// maxima of |S0| per head (the scale scan's starting bound).
constexpr int O2_INIT_PARTS = 64;
__host__ __device__ constexpr int z_tile(int bt, int ct) { return bt * 4 - bt * (bt - 1) / 2 + (ct - bt); }

// Workspace layout (float offsets), in this order:
//   tb     [BH, nblk]                 block decay totals
//   state  [BH, nblk, DH*DH + DH]     per-block state contributions, then
//                                     (in place) the state entering each block
//                                     (order 1: S and z; order 2: the upper
//                                     tiles of Z, Z_FLOATS floats, rest unused)
//   part   [BH, rows, 64]             order 2 only: inter-block numerators
//                                     (rows = o2_part_rows(N), padded to
//                                     whole steps)
//   rec    [BH, nblk] x REC_BYTES     order 2 only: operand records
//   initmax [BH, O2_INIT_PARTS]       order 2 only: partial maxima of |S0|
struct WsLayout {
  size_t tb, state, part, rec, initmax, total_floats;
};

inline WsLayout ws_layout(int64_t B, int64_t H, int64_t N, int64_t DH, int order) {
  const int64_t BH = B * H, nb = n_blocks(N);
  WsLayout L;
  L.tb = 0;
  size_t off = (size_t)(BH * nb);
  off = (off + 63) & ~(size_t)63;
  L.state = off;
  off += (size_t)(BH * nb) * (size_t)(DH * DH + DH);
  off = (off + 63) & ~(size_t)63;
  L.part = off;
  if (order == 2) off += (size_t)BH * (size_t)o2_part_rows(N) * 64;
  off = (off + 63) & ~(size_t)63;
  L.rec = off;
  if (order == 2) off += (size_t)(BH * nb) * (REC_BYTES / 4);
  off = (off + 63) & ~(size_t)63;
  L.initmax = off;
  if (order == 2) off += (size_t)BH * O2_INIT_PARTS;
  L.total_floats = off;
  return L;
}

hipError_t launch_prep(const float* dt_proj, const float* dt_bias, const float* A_log, int64_t B,
                       int64_t H, int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                       hipStream_t stream);

// dst[0 .. n) = src (or 0 if src is NULL); n >= 1.
hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream);

// Algorithms 4 / 5 A-mask: a = -softplus(A_proj), dt = softplus(dt_proj) (no
// bias) if dt_proj is not NULL (dt is then written), chunk-local cumsum.
hipError_t launch_prep_amask(const float* A_proj, const float* dt_proj, int64_t B, int64_t H,
                             int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                             hipStream_t stream);

// Per-block state contributions: state[bh,blk] = sum_j w_j k_j val_j^T and
// sum_j w_j k_j with w_j = exp(A^CS_last - A^CS_j); val = v*dt (dt != NULL) or v.
hipError_t launch_chunk_state(bool bf16, int64_t DH, const void* k, const void* v, const float* dt,
                              const float* a_cs, int64_t BH, int64_t N, int64_t chunk, float* tb,
                              float* state, hipStream_t stream);

// In-place exclusive scan over blocks: state[bh,blk] <- state entering blk,
// starting from (init_S, init_z) when given (else zero).
hipError_t launch_state_pass(int64_t DH, int64_t BH, int64_t N, const float* tb, float* state,
                             float* final_S, float* final_z, const float* init_S,
                             const float* init_z, hipStream_t stream);

// Intra-block masked product + inter-block part + normalisation -> y, den.
hipError_t launch_output(bool bf16, int64_t DH, int order, const void* q, const void* k,
                         const void* v, const float* dt, const float* a_cs, int64_t BH, int64_t N,
                         int64_t chunk, const float* state, const float* part, float* y,
                         float* den, hipStream_t stream);

// Order 1 with bf16 inputs: the sequential scan per (head, segment).
// agg_pass: the segment aggregates and, in place, their prefixes from S0, z0
// (or zero): the state entering each segment but the first (nothing when the
// sequence is one segment); otherwise the outputs, each segment starting from
// its prefix (the first from S0, z0 or zero), and the final states when Sf is
// given.  sink: 32 floats of scratch that take the stores of rows past a
// ragged end.
void o1_scan_segments(int64_t BH, int64_t DH, int64_t N, int* nseg, int* nbs);
size_t o1_scan_agg_floats(int64_t BH, int64_t DH, int64_t N);
bool o1_scan_supported(int64_t BH, int64_t DH, int64_t N);  // d_h 32/64, N d_h < 2^31
hipError_t launch_o1_scan(bool agg_pass, int64_t DH, const void* q, const void* k, const void* v,
                          const float* dt, const float* a_cs, int64_t BH, int64_t N, int64_t chunk,
                          const float* S0, const float* z0, float* agg, float* y, float* den,
                          float* Sf, float* zf, float* sink, hipStream_t stream);

// Order 2, per block (parallel): the normaliser state contribution
// sum_j w_j k_j k_j^T (as launch_chunk_state with k as the value) and the
// operand record of the numerator scan.
hipError_t launch_o2_blockprep(const void* q, const void* k, const void* v, const float* dt,
                               const float* a_cs, int64_t BH, int64_t N, int64_t chunk, float* tb,
                               float* state, void* rec, hipStream_t stream);

// Order-2 initial state: O2_INIT_PARTS partial maxima of |S0| per head.
hipError_t launch_o2_initmax(const float* S0, int64_t BH, float* initmax, hipStream_t stream);

// Order-2 scale scan: per head, the running bound of the numerator state and
// the per-block scale exponents of the state scan (record words SC_SIG_IN ..);
// the bound starts at max |S0| (from initmax, if not NULL) or 0.
hipError_t launch_o2_scale_scan(void* rec, int64_t BH, int64_t N, const float* initmax,
                                hipStream_t stream);

// Order-2 inter-block numerator: on-chip state scan over the block records.
// The same kernel scans the normaliser state in place over the per-block
// slots of `zstate` (Z_blk -> Z entering the block, as launch_state_pass) and
// writes the final Z to final_norm (if not NULL).
// The scans start from (S0, Z0) when given (the initial numerator and
// normaliser states, the layouts of final_state and final_norm), else zero.
hipError_t launch_o2_state(const void* rec, int64_t BH, int64_t N, float* part,
                           float* final_state, float* zstate, float* final_norm, const float* S0,
                           const float* Z0, hipStream_t stream);

// The window-2 short convolution of Algorithm 6 on the decode path: per
// channel x^c = w[.., 0] x_prev + w[.., 1] x (+ b), optional SiLU; the conv
// state holds the previous step's raw q, k, v and receives this step's.
struct DecodeConv {
  const float* w;  // [3, H, d_h, 2] (q, k, v channels) or NULL: no convolution
  const float* b;  // [3, H, d_h] or NULL
  void* state;     // [S, 3, H, d_h], the q/k/v element type, in/out
  int act;         // 0: none (Algorithm 6), 1: SiLU (Algorithm 3's sigma)
};

// One decode step.  A_proj == NULL: the Mamba-2 discretisation (dt_proj,
// dt_bias, A_log); else the A-mask (A_proj, optional dt_proj).  packed: the
// order-2 states in the packed layout (rows a <= b).  conv.w == NULL: q, k, v
// are used as given.
hipError_t launch_decode(bool bf16, int64_t DH, int order, bool packed, const void* q,
                         const void* k, const void* v, const float* dt_proj, const float* dt_bias,
                         const float* A_log, const float* A_proj, int64_t S, int64_t H,
                         float* state, float* norm_state, float* y, hipStream_t stream,
                         DecodeConv conv = DecodeConv{nullptr, nullptr, nullptr, 0});

// Order-2 state layout conversion over BH (sequence, head) pairs: full ->
// packed (the symmetric part) when to_packed, else packed -> full.
hipError_t launch_state_layout(bool to_packed, int64_t DH, int64_t BH, const float* src_S,
                               const float* src_z, float* dst_S, float* dst_z,
                               hipStream_t stream);

}  // namespace ssd
