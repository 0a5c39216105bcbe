// ssd_prep / ssd_prep_amask: discretisation and chunk-local cumulative
// log-decay.
//
// 2Mamba2Furious, Algorithm 3 (Mamba-2 forward pass): A = -exp(A_log),
// dt = softplus(dt_P + dt_bias), A^CS = cumsum(A * dt).  Algorithms 4 and 5
// (the A-mask of Mamba-2S / 2Mamba): a per-token A = -softplus(A_P) and
// A^CS = cumsum(A), with dt = softplus(dt_P) (no bias) for the value operand
// or no dt at all.  The cumsum is inclusive and restarts at every chunk
// boundary; chunk totals are written separately, so no decay is ever computed
// from a large global sum.
//
// Two forms.  When N is a multiple of 4 (every row 16-byte aligned; all the
// workloads here), k_prep4: each lane owns 4 consecutive tokens (16-byte
// loads and stores), chunk/4 lanes cover a chunk, the chunk's cumsum is a
// scan of the lane totals within that segment of lanes, and softplus uses a
// log1p written for its range (softplus_v).  Otherwise k_prep: one wave per
// chunk, each lane 1 or 2 tokens, a wave-wide scan of the lane totals
// (Hillis-Steele over __shfl_up).  HBM traffic per token and head: 4 B in,
// 8 B out.
#include "common.h"
#include "launch.h"

namespace ssd {

// MODE 0: Algorithm 3; 1: A-mask with dt; 2: A-mask without dt
template <int TPL, int MODE>  // tokens per lane: chunk / 64
__global__ __launch_bounds__(256) void k_prep(const float* __restrict__ dt_proj,
                                              const float* __restrict__ dt_bias,
                                              const float* __restrict__ A_log,
                                              const float* __restrict__ A_proj, int64_t H, int64_t N,
                                              int64_t n_chunks, int64_t total_chunks,
                                              float* __restrict__ dt_out, float* __restrict__ a_cs,
                                              float* __restrict__ a_chunk) {
  constexpr int CHUNK = TPL * WAVE;
  const int lane = threadIdx.x & (WAVE - 1);
  const int64_t gchunk = (int64_t)blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x / WAVE);
  if (gchunk >= total_chunks) return;
  const int64_t bh = gchunk / n_chunks;
  const int64_t c = gchunk - bh * n_chunks;
  const int64_t h = bh % H;
  const float A = MODE == 0 ? -expf(A_log[h]) : 0.f;
  const float bias = MODE == 0 ? dt_bias[h] : 0.f;
  const int64_t t0 = c * CHUNK + (int64_t)lane * TPL;
  const int64_t row = bh * N;

  float dts[TPL], run[TPL];
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < TPL; ++s) {
    const int64_t t = t0 + s;
    float d = 0.f, a = 0.f;
    if (t < N) {
      if constexpr (MODE == 0) {
        d = softplus_f(dt_proj[row + t] + bias);
        a = A * d;
      } else {
        a = -softplus_f(A_proj[row + t]);
        if constexpr (MODE == 1) d = softplus_f(dt_proj[row + t]);
      }
    }
    dts[s] = d;
    acc += a;
    run[s] = acc;
  }
  // inclusive scan of the lane totals across the wave
  float incl = acc;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const float o = __shfl_up(incl, off, WAVE);
    if (lane >= off) incl += o;
  }
  const float offset = incl - acc;
#pragma unroll
  for (int s = 0; s < TPL; ++s) {
    const int64_t t = t0 + s;
    if (t < N) {
      if constexpr (MODE != 2) dt_out[row + t] = dts[s];
      a_cs[row + t] = offset + run[s];
    }
  }
  if (lane == WAVE - 1) a_chunk[bh * n_chunks + c] = incl;
}

// softplus(x) = max(x, 0) + log1p(e) with e = e^{-|x|} in (0, 1], log1p
// written for that range: the series e (1 - e/2 + e^2/3 - e^3/4 + e^4/5)
// below e = 2^-6 (truncation below 2^-30 of the result), else log(u) with
// u = 1 + e rounded and the rounding's first-order correction
// ((u - 1) - e) / u, log(u) = log2(u) ln 2 on the hardware logarithm.
__device__ __forceinline__ float softplus_v(float x) {
  const float e = expf(-fabsf(x));
  float l;
  if (e < 0.015625f) {
    l = e * fmaf(e, fmaf(e, fmaf(e, fmaf(e, 0.2f, -0.25f), 1.f / 3.f), -0.5f), 1.f);
  } else {
    const float u = 1.f + e;
    l = __builtin_amdgcn_logf(u) * 0.69314718055994531f - ((u - 1.f) - e) / u;
  }
  return fmaxf(x, 0.f) + l;
}

// Vector form (N a multiple of 4, so that every row starts 16-byte aligned):
// each lane owns 4 consecutive tokens (one 16-byte load, two 16-byte stores),
// SEG = chunk / 4 lanes cover one chunk, a wave covers 64 / SEG chunks, and
// the chunk's inclusive cumsum is a scan of the lane totals within each SEG-
// lane segment (__shfl_up over segments of SEG lanes).  A ragged last chunk
// of a row masks whole 4-token groups (N % 4 == 0).
template <int SEG, int MODE>
__global__ __launch_bounds__(256) void k_prep4(const float* __restrict__ dt_proj,
                                               const float* __restrict__ dt_bias,
                                               const float* __restrict__ A_log,
                                               const float* __restrict__ A_proj, uint32_t H,
                                               uint32_t N, uint32_t n_chunks,
                                               uint32_t total_chunks,
                                               float* __restrict__ dt_out,
                                               float* __restrict__ a_cs,
                                               float* __restrict__ a_chunk) {
  constexpr int CHUNK = 4 * SEG, CPW = WAVE / SEG;
  const int lane = threadIdx.x & (WAVE - 1), sub = lane % SEG;
  const uint32_t g = (blockIdx.x * (blockDim.x / WAVE) + threadIdx.x / WAVE) * CPW + lane / SEG;
  const bool live_chunk = g < total_chunks;
  const uint32_t gc = live_chunk ? g : total_chunks - 1;
  const uint32_t bh = gc / n_chunks, c = gc - bh * n_chunks, h = bh % H;
  const uint32_t t = c * CHUNK + 4 * sub;  // first token of this lane in its row
  const bool live = live_chunk && t < N;
  const int64_t off = (int64_t)bh * N + t;
  f32x4 x = zero4();
  if (live) x = *reinterpret_cast<const f32x4*>((MODE == 0 ? dt_proj : A_proj) + off);
  f32x4 xd = zero4();
  if (MODE == 1 && live) xd = *reinterpret_cast<const f32x4*>(dt_proj + off);
  const float A = MODE == 0 ? -expf(A_log[h]) : 0.f;
  const float bias = MODE == 0 ? dt_bias[h] : 0.f;
  f32x4 d = zero4(), run;
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float a;
    if constexpr (MODE == 0) {
      d[s] = softplus_v(x[s] + bias);
      a = A * d[s];
    } else {
      a = -softplus_v(x[s]);
      if constexpr (MODE == 1) d[s] = softplus_v(xd[s]);
    }
    acc += live ? a : 0.f;
    run[s] = acc;
  }
  // inclusive scan of the lane totals within the chunk's segment of lanes
  float incl = acc;
#pragma unroll
  for (int o = 1; o < SEG; o <<= 1) {
    const float p = __shfl_up(incl, o, SEG);
    if (sub >= o) incl += p;
  }
  const float base = incl - acc;
  if (live) {
    if constexpr (MODE != 2) *reinterpret_cast<f32x4*>(dt_out + off) = d;
    f32x4 cs;
#pragma unroll
    for (int s = 0; s < 4; ++s) cs[s] = base + run[s];
    *reinterpret_cast<f32x4*>(a_cs + off) = cs;
  }
  // the chunk total: the inclusive sum at the segment's last lane (lanes past
  // a ragged chunk's end add 0)
  if (live_chunk && sub == SEG - 1) a_chunk[(int64_t)bh * n_chunks + c] = incl;
}

template <int MODE>
static hipError_t launch_prep_mode(const float* dt_proj, const float* dt_bias, const float* A_log,
                                   const float* A_proj, int64_t B, int64_t H, int64_t N,
                                   int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                                   hipStream_t stream) {
  const int64_t n_chunks = (N + chunk - 1) / chunk;
  const int64_t total = B * H * n_chunks;
  const int waves_per_block = 4;
  if (N % 4 == 0 && total < ((int64_t)1 << 31) && B * H * N < ((int64_t)1 << 32)) {
    const int cpw = (int)(WAVE / (chunk / 4));  // chunks per wave
    const int64_t grid4 = (total + waves_per_block * cpw - 1) / (waves_per_block * cpw);
    if (chunk == 64)
      hipLaunchKernelGGL((k_prep4<16, MODE>), dim3((unsigned)grid4), dim3(256), 0, stream, dt_proj,
                         dt_bias, A_log, A_proj, (uint32_t)H, (uint32_t)N, (uint32_t)n_chunks,
                         (uint32_t)total, dt, a_cs, a_chunk);
    else
      hipLaunchKernelGGL((k_prep4<32, MODE>), dim3((unsigned)grid4), dim3(256), 0, stream, dt_proj,
                         dt_bias, A_log, A_proj, (uint32_t)H, (uint32_t)N, (uint32_t)n_chunks,
                         (uint32_t)total, dt, a_cs, a_chunk);
    return hipGetLastError();
  }
  const int64_t grid = (total + waves_per_block - 1) / waves_per_block;
  if (chunk == 64)
    hipLaunchKernelGGL((k_prep<1, MODE>), dim3((unsigned)grid), dim3(256), 0, stream, dt_proj, dt_bias,
                       A_log, A_proj, H, N, n_chunks, total, dt, a_cs, a_chunk);
  else
    hipLaunchKernelGGL((k_prep<2, MODE>), dim3((unsigned)grid), dim3(256), 0, stream, dt_proj, dt_bias,
                       A_log, A_proj, H, N, n_chunks, total, dt, a_cs, a_chunk);
  return hipGetLastError();
}

hipError_t launch_prep(const float* dt_proj, const float* dt_bias, const float* A_log, int64_t B,
                       int64_t H, int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                       hipStream_t stream) {
  return launch_prep_mode<0>(dt_proj, dt_bias, A_log, nullptr, B, H, N, chunk, dt, a_cs, a_chunk,
                             stream);
}

hipError_t launch_prep_amask(const float* A_proj, const float* dt_proj, int64_t B, int64_t H,
                             int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                             hipStream_t stream) {
  if (dt_proj)
    return launch_prep_mode<1>(dt_proj, nullptr, nullptr, A_proj, B, H, N, chunk, dt, a_cs, a_chunk,
                               stream);
  return launch_prep_mode<2>(nullptr, nullptr, nullptr, A_proj, B, H, N, chunk, nullptr, a_cs,
                             a_chunk, stream);
}

// dst[0 .. n) = src[0 .. n), or 0 where src is NULL (the final states of an
// empty segment)
__global__ __launch_bounds__(256) void k_copy_or_zero(float* __restrict__ dst,
                                                      const float* __restrict__ src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_copy_or_zero(float* dst, const float* src, int64_t n, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(k_copy_or_zero, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     stream, dst, src, n);
  return hipGetLastError();
}

}  // namespace ssd
