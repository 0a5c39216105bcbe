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
// One wave per chunk.  Each lane owns chunk/64 consecutive tokens (1 or 2):
// it forms dt and a = A*dt for them, a running sum over its own tokens, then
// a wave-wide inclusive scan of the lane totals (Hillis-Steele over
// __shfl_up) supplies each lane's offset.  HBM traffic per token and head:
// 4 B in, 8 B out.
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

template <int MODE>
static hipError_t launch_prep_mode(const float* dt_proj, const float* dt_bias, const float* A_log,
                                   const float* A_proj, int64_t B, int64_t H, int64_t N,
                                   int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                                   hipStream_t stream) {
  const int64_t n_chunks = (N + chunk - 1) / chunk;
  const int64_t total = B * H * n_chunks;
  const int waves_per_block = 4;
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
