// C ABI of libssd.so: argument validation (before any HIP call) and dispatch
// to the gfx950 kernels.  See include/ssd.h for the contract of every call.
#include "ssd.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "bwd.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = {0};
thread_local hipEvent_t* g_events = nullptr;
thread_local int g_n_events = 0;
thread_local int g_timed = 0;

// Records the next timing event (if a registration is active) on `stream`.
struct Timer {
  hipEvent_t* ev;
  int n, i = 0;
  hipStream_t stream;
  Timer(hipStream_t s) : ev(g_events), n(g_n_events), stream(s) {
    g_events = nullptr;
    g_n_events = 0;
    g_timed = 0;
    mark();
  }
  void mark() {
    if (ev && i < n) {
      (void)hipEventRecord(ev[i], stream);
      g_timed = i;
      ++i;
    }
  }
};

ssd_status fail(ssd_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_err() { g_err[0] = 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// product of positive sizes with overflow detection (limit 2^62)
// a * b for sizes >= 0 (0 allowed: an empty input), false on a negative size
// or an overflow past 2^62
bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a && b > ((int64_t)1 << 62) / a) return false;
  *out = a * b;
  return true;
}

struct Range {
  const char* name;
  const void* p;
  size_t bytes;
};

bool overlap(const Range& a, const Range& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

ssd_status check_alias(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j]))
        return fail(SSD_ERR_ALIAS, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j]))
        return fail(SSD_ERR_ALIAS, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }
  return SSD_OK;
}

ssd_status check_aligned(const Range* rs, int n) {
  for (int i = 0; i < n; ++i)
    if (rs[i].p && !aligned16(rs[i].p))
      return fail(SSD_ERR_ALIGN, "%s is not 16-byte aligned", rs[i].name);
  return SSD_OK;
}

ssd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SSD_OK;
  return fail(SSD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shared validation of the forward arguments; fills element counts.
ssd_status validate_forward_sizes(int64_t B, int64_t H, int64_t N, int64_t d_h, int order,
                                  int64_t chunk, int dtype, int64_t* BH, int64_t* BHN,
                                  int64_t* BHNd) {
  if (!mul_ok(B, H, BH) || !mul_ok(*BH, N, BHN) || !mul_ok(*BHN, d_h, BHNd))
    return fail(SSD_ERR_SHAPE, "B, H, N must be >= 0, d_h >= 1, and their product must not overflow");
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (order != 1 && order != 2) return fail(SSD_ERR_UNSUPPORTED, "order %d (1 or 2)", order);
  if (chunk != 64 && chunk != 128) return fail(SSD_ERR_UNSUPPORTED, "chunk %lld (64 or 128)", (long long)chunk);
  if (order == 1 && d_h != 32 && d_h != 64)
    return fail(SSD_ERR_UNSUPPORTED, "d_h %lld at order 1 (32 or 64)", (long long)d_h);
  if (order == 2 && d_h != 64) return fail(SSD_ERR_UNSUPPORTED, "d_h %lld at order 2 (64)", (long long)d_h);
  if (order == 2 && dtype != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "order 2 requires bf16 inputs");
  if (*BH * ((N + 63) / 64) > (int64_t)0x7fffffff) return fail(SSD_ERR_SHAPE, "grid too large");
  return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char* ssd_status_str(int s) {
  switch (s) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL: return "SSD_ERR_NULL";
    case SSD_ERR_SHAPE: return "SSD_ERR_SHAPE";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN";
    case SSD_ERR_ALIAS: return "SSD_ERR_ALIAS";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
    default: return "SSD_ERR_UNKNOWN";
  }
}

const char* ssd_last_error(void) { return g_err; }

ssd_status ssd_prep(const float* dt_proj, const float* dt_bias, const float* A_log, int64_t B,
                    int64_t H, int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                    hipStream_t stream) {
  try {
    clear_err();
    int64_t BH, BHN;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &BHN))
      return fail(SSD_ERR_SHAPE, "ssd_prep: B, H, N must be >= 0 and must not overflow");
    if (chunk != 64 && chunk != 128)
      return fail(SSD_ERR_UNSUPPORTED, "ssd_prep: chunk %lld (64 or 128)", (long long)chunk);
    if (BHN == 0) return SSD_OK;  // empty input: nothing to compute
    if (!dt_proj || !dt_bias || !A_log || !dt || !a_cs || !a_chunk)
      return fail(SSD_ERR_NULL, "ssd_prep: a required pointer is NULL");
    const int64_t nc = (N + chunk - 1) / chunk;
    if ((BH * nc + 3) / 4 > (int64_t)0x7fffffff) return fail(SSD_ERR_SHAPE, "ssd_prep: grid too large");
    const Range ins[] = {{"dt_proj", dt_proj, (size_t)BHN * 4},
                         {"dt_bias", dt_bias, (size_t)H * 4},
                         {"A_log", A_log, (size_t)H * 4}};
    const Range outs[] = {{"dt", dt, (size_t)BHN * 4},
                          {"a_cs", a_cs, (size_t)BHN * 4},
                          {"a_chunk", a_chunk, (size_t)(BH * nc) * 4}};
    ssd_status s;
    if ((s = check_aligned(ins, 3)) != SSD_OK || (s = check_aligned(outs, 3)) != SSD_OK) return s;
    if ((s = check_alias(outs, 3, ins, 3)) != SSD_OK) return s;
    return hip_status(ssd::launch_prep(dt_proj, dt_bias, A_log, B, H, N, chunk, dt, a_cs, a_chunk, stream),
                      "ssd_prep launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_prep: unexpected exception");
  }
}

ssd_status ssd_prep_amask(const float* A_proj, const float* dt_proj, int64_t B, int64_t H,
                          int64_t N, int64_t chunk, float* dt, float* a_cs, float* a_chunk,
                          hipStream_t stream) {
  try {
    clear_err();
    int64_t BH, BHN;
    if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, &BHN))
      return fail(SSD_ERR_SHAPE, "ssd_prep_amask: B, H, N must be >= 0 and must not overflow");
    if (chunk != 64 && chunk != 128)
      return fail(SSD_ERR_UNSUPPORTED, "ssd_prep_amask: chunk %lld (64 or 128)", (long long)chunk);
    if (BHN == 0) return SSD_OK;  // empty input: nothing to compute
    if (!A_proj || !a_cs || !a_chunk)
      return fail(SSD_ERR_NULL, "ssd_prep_amask: a required pointer is NULL");
    if ((dt_proj == nullptr) != (dt == nullptr))
      return fail(SSD_ERR_NULL, "ssd_prep_amask: dt_proj and dt must both be given or both be NULL");
    const int64_t nc = (N + chunk - 1) / chunk;
    if ((BH * nc + 3) / 4 > (int64_t)0x7fffffff)
      return fail(SSD_ERR_SHAPE, "ssd_prep_amask: grid too large");
    const Range ins[] = {{"A_proj", A_proj, (size_t)BHN * 4}, {"dt_proj", dt_proj, (size_t)BHN * 4}};
    const Range outs[] = {{"dt", dt, (size_t)BHN * 4},
                          {"a_cs", a_cs, (size_t)BHN * 4},
                          {"a_chunk", a_chunk, (size_t)(BH * nc) * 4}};
    ssd_status s;
    if ((s = check_aligned(ins, 2)) != SSD_OK || (s = check_aligned(outs, 3)) != SSD_OK) return s;
    if ((s = check_alias(outs, 3, ins, 2)) != SSD_OK) return s;
    return hip_status(ssd::launch_prep_amask(A_proj, dt_proj, B, H, N, chunk, dt, a_cs, a_chunk, stream),
                      "ssd_prep_amask launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_prep_amask: unexpected exception");
  }
}

size_t ssd_forward_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d_h, int order,
                                  int64_t chunk, int dtype) {
  int64_t BH, BHN, BHNd;
  if (validate_forward_sizes(B, H, N, d_h, order, chunk, dtype, &BH, &BHN, &BHNd) != SSD_OK) return 0;
  if (BHN == 0) return 0;  // an empty input needs no workspace
  return ssd::ws_layout(B, H, N, d_h, order).total_floats * sizeof(float);
}

}  // extern "C"

namespace {

// Scratch memory of ssd_forward_noalloc: a file-scope device array (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, taken once per device on that device's first call.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

ssd_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "ssd_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(SSD_ERR_HIP, "ssd_forward_noalloc: device %d beyond the %d supported", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "ssd_forward_noalloc: hipGetSymbolAddress(scratch)");
    if (!p) return fail(SSD_ERR_HIP, "ssd_forward_noalloc: hipGetSymbolAddress returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SSD_OK;
}

// ssd_forward and ssd_forward_noalloc: every argument check, then (noalloc)
// the device's scratch array in place of the caller's workspace, then the
// launches.
ssd_status forward_core(const char* fn, bool noalloc, const void* q, const void* k, const void* v,
                        const float* dt, const float* a_cs, const float* initial_state,
                        const float* initial_norm, int64_t B, int64_t H, int64_t N, int64_t d_h,
                        int order, int64_t chunk, int dtype, float* y, float* den,
                        float* final_state, float* final_norm, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  int64_t BH, BHN, BHNd;
  ssd_status s = validate_forward_sizes(B, H, N, d_h, order, chunk, dtype, &BH, &BHN, &BHNd);
  if (s != SSD_OK) return s;
  if (BH == 0) return SSD_OK;  // no heads: nothing to compute
  if ((final_state == nullptr) != (final_norm == nullptr))
    return fail(SSD_ERR_NULL, "%s: final_state and final_norm must be given together", fn);
  if ((initial_state == nullptr) != (initial_norm == nullptr))
    return fail(SSD_ERR_NULL, "%s: initial_state and initial_norm must be given together", fn);
  const size_t es = dtype == SSD_BF16 ? 2 : 4;
  const int64_t D = order == 1 ? d_h : d_h * d_h;
  if (BHN == 0) {
    // an empty segment (N = 0): the final states are the initial ones (or zero)
    if (!final_state) return SSD_OK;
    const Range ins0[] = {{"initial_state", initial_state, (size_t)(BH * D * d_h) * 4},
                          {"initial_norm", initial_norm, (size_t)(BH * D) * 4}};
    const Range outs0[] = {{"final_state", final_state, (size_t)(BH * D * d_h) * 4},
                           {"final_norm", final_norm, (size_t)(BH * D) * 4}};
    if ((s = check_aligned(ins0, 2)) != SSD_OK || (s = check_aligned(outs0, 2)) != SSD_OK) return s;
    if ((s = check_alias(outs0, 2, ins0, 2)) != SSD_OK) return s;
    hipError_t e = ssd::launch_copy_or_zero(final_state, initial_state, BH * D * d_h, stream);
    if (e == hipSuccess) e = ssd::launch_copy_or_zero(final_norm, initial_norm, BH * D, stream);
    return hip_status(e, "final-state copy launch");
  }
  if (!q || !k || !v || !a_cs || !y) return fail(SSD_ERR_NULL, "%s: a required pointer is NULL", fn);
  const size_t need = ssd::ws_layout(B, H, N, d_h, order).total_floats * sizeof(float);
  if (noalloc) {
    if (need > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
      return fail(SSD_ERR_WORKSPACE,
                  "%s: these sizes need %zu bytes of scratch, more than the %zu bytes this entry point "
                  "holds per device; call ssd_forward with a workspace instead",
                  fn, need, (size_t)SSD_NOALLOC_SCRATCH_BYTES);
  } else if (workspace_bytes < need || (need && !workspace)) {
    return fail(SSD_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  }
  const Range ins[] = {{"q", q, (size_t)BHNd * es},  {"k", k, (size_t)BHNd * es},
                       {"v", v, (size_t)BHNd * es},  {"dt", dt, (size_t)BHN * 4},
                       {"a_cs", a_cs, (size_t)BHN * 4},
                       {"initial_state", initial_state, (size_t)(BH * D * d_h) * 4},
                       {"initial_norm", initial_norm, (size_t)(BH * D) * 4}};
  const Range outs[] = {{"y", y, (size_t)BHNd * 4},
                        {"den", den, (size_t)BHN * 4},
                        {"final_state", final_state, (size_t)(BH * D * d_h) * 4},
                        {"final_norm", final_norm, (size_t)(BH * D) * 4},
                        {"workspace", noalloc ? nullptr : workspace, need}};
  if ((s = check_aligned(ins, 7)) != SSD_OK || (s = check_aligned(outs, 5)) != SSD_OK) return s;
  if ((s = check_alias(outs, 5, ins, 7)) != SSD_OK) return s;
  // every check done: only now the first HIP call
  if (noalloc && (s = scratch_of_current_device(&workspace)) != SSD_OK) return s;

  const bool bf = dtype == SSD_BF16;
  Timer tm(stream);
  const ssd::WsLayout L = ssd::ws_layout(B, H, N, d_h, order);
  float* ws = static_cast<float*>(workspace);
  float* tb = ws + L.tb;
  float* st = ws + L.state;
  hipError_t e;
  if (order == 1 && bf && ssd::o1_scan_supported(BH, d_h, N)) {
    // bf16 inputs: the sequential scan per (head, segment); the segment
    // aggregates and their prefixes (when the sequence is cut into segments)
    // go to the state region of the workspace
    float* agg = st;
    const size_t na = (ssd::o1_scan_agg_floats(BH, d_h, N) + 63) & ~(size_t)63;
    float* sink = st + na;
    if (na + 64 > L.part - L.state)
      return fail(SSD_ERR_WORKSPACE, "%s: internal: segment aggregates exceed the workspace", fn);
    if ((e = ssd::launch_o1_scan(true, d_h, q, k, v, dt, a_cs, BH, N, chunk, initial_state, initial_norm,
                                 agg, nullptr, nullptr, nullptr, nullptr, sink, stream)) != hipSuccess)
      return hip_status(e, "o1_scan aggregate launch");
    tm.mark();
    e = ssd::launch_o1_scan(false, d_h, q, k, v, dt, a_cs, BH, N, chunk, initial_state, initial_norm,
                            agg, y, den, final_state, final_norm, sink, stream);
    tm.mark();
    return hip_status(e, "o1_scan launch");
  }
  if (order == 1) {
    if ((e = ssd::launch_chunk_state(bf, d_h, k, v, dt, a_cs, BH, N, chunk, tb, st, stream)) != hipSuccess)
      return hip_status(e, "chunk_state launch");
    tm.mark();
    if ((e = ssd::launch_state_pass(d_h, BH, N, tb, st, final_state, final_norm, initial_state,
                                    initial_norm, stream)) != hipSuccess)
      return hip_status(e, "state_pass launch");
    tm.mark();
    e = ssd::launch_output(bf, d_h, 1, q, k, v, dt, a_cs, BH, N, chunk, st, nullptr, y, den, stream);
    tm.mark();
    return hip_status(e, "output launch");
  }
  // order 2: per-block preparation (normaliser contributions Z_blk and the
  // numerator operand records), the scale scan, the on-chip numerator scan
  // (which also scans Z), and the output kernel.
  float* part = ws + L.part;
  void* rec = ws + L.rec;
  if ((e = ssd::launch_o2_blockprep(q, k, v, dt, a_cs, BH, N, chunk, tb, st, rec, stream)) != hipSuccess)
    return hip_status(e, "o2_blockprep launch");
  tm.mark();
  float* initmax = nullptr;
  if (initial_state) {
    initmax = ws + L.initmax;
    if ((e = ssd::launch_o2_initmax(initial_state, BH, initmax, stream)) != hipSuccess)
      return hip_status(e, "o2_initmax launch");
  }
  if ((e = ssd::launch_o2_scale_scan(rec, BH, N, initmax, stream)) != hipSuccess)
    return hip_status(e, "o2_scale_scan launch");
  tm.mark();
  if ((e = ssd::launch_o2_state(rec, BH, N, part, final_state, st, final_norm, initial_state,
                                initial_norm, stream)) != hipSuccess)
    return hip_status(e, "o2_state launch");
  tm.mark();
  e = ssd::launch_output(true, 64, 2, q, k, v, dt, a_cs, BH, N, chunk, st, part, y, den, stream);
  tm.mark();
  return hip_status(e, "output launch");
}

}  // namespace

extern "C" {

ssd_status ssd_forward(const void* q, const void* k, const void* v, const float* dt,
                       const float* a_cs, const float* initial_state, const float* initial_norm,
                       int64_t B, int64_t H, int64_t N, int64_t d_h, int order,
                       int64_t chunk, int dtype, float* y, float* den, float* final_state,
                       float* final_norm, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  try {
    clear_err();
    return forward_core("ssd_forward", false, q, k, v, dt, a_cs, initial_state, initial_norm, B, H, N,
                        d_h, order, chunk, dtype, y, den, final_state, final_norm, workspace,
                        workspace_bytes, stream);
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_forward: unexpected exception");
  }
}

ssd_status ssd_forward_noalloc(const void* q, const void* k, const void* v, const float* dt,
                               const float* a_cs, const float* initial_state,
                               const float* initial_norm, int64_t B, int64_t H, int64_t N,
                               int64_t d_h, int order, int64_t chunk, int dtype, float* y,
                               float* den, float* final_state, float* final_norm,
                               hipStream_t stream) {
  try {
    clear_err();
    return forward_core("ssd_forward_noalloc", true, q, k, v, dt, a_cs, initial_state, initial_norm, B,
                        H, N, d_h, order, chunk, dtype, y, den, final_state, final_norm, nullptr, 0,
                        stream);
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_forward_noalloc: unexpected exception");
  }
}

ssd_status ssd_set_timing_events(hipEvent_t* events, int n) {
  clear_err();
  if (events && n < 5) return fail(SSD_ERR_SHAPE, "ssd_set_timing_events: n must be >= 5");
  g_events = events;
  g_n_events = events ? n : 0;
  return SSD_OK;
}

int ssd_timing_count(void) { return g_timed; }

// Shared by both decode entry points: sizes, parameters, pointers, alignment
// and overlap; `params` are the per-token / per-head decay inputs.
static ssd_status decode_common(const char* fn, const void* q, const void* k, const void* v,
                         const Range* params, int n_params, int64_t S, int64_t H, int64_t d_h,
                         int order, int dtype, int layout, float* state, float* norm_state,
                         float* y, bool* empty) {
  int64_t SH, SHd;
  *empty = false;
  if (!mul_ok(S, H, &SH) || !mul_ok(SH, d_h, &SHd))
    return fail(SSD_ERR_SHAPE, "%s: S, H must be >= 0 and must not overflow", fn);
  if (dtype != SSD_F32 && dtype != SSD_BF16) return fail(SSD_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (order != 1 && order != 2) return fail(SSD_ERR_UNSUPPORTED, "order %d (1 or 2)", order);
  if (d_h != 32 && d_h != 64) return fail(SSD_ERR_UNSUPPORTED, "d_h %lld (32 or 64)", (long long)d_h);
  if (layout != SSD_STATE_FULL && layout != SSD_STATE_PACKED)
    return fail(SSD_ERR_UNSUPPORTED, "%s: layout %d", fn, layout);
  if (layout == SSD_STATE_PACKED && order != 2)
    return fail(SSD_ERR_UNSUPPORTED, "%s: the packed layout is for order 2", fn);
  if (SH == 0) {  // no sequences or heads: nothing to compute
    *empty = true;
    return SSD_OK;
  }
  if (!q || !k || !v || !state || !norm_state || !y)
    return fail(SSD_ERR_NULL, "%s: a required pointer is NULL", fn);
  if (SH > (int64_t)0x7fffffff) return fail(SSD_ERR_SHAPE, "%s: grid too large", fn);
  const int64_t D = order == 1 ? d_h : (layout == SSD_STATE_PACKED ? d_h * (d_h + 1) / 2 : d_h * d_h);
  int64_t nstate;
  if (!mul_ok(SH, D * d_h, &nstate)) return fail(SSD_ERR_SHAPE, "%s: state too large", fn);
  const size_t es = dtype == SSD_BF16 ? 2 : 4;
  constexpr int MAX_PARAMS = 8;
  if (n_params > MAX_PARAMS) return fail(SSD_ERR_HIP, "%s: internal: too many parameter ranges", fn);
  Range ins[3 + MAX_PARAMS] = {{"q", q, (size_t)SHd * es}, {"k", k, (size_t)SHd * es},
                               {"v", v, (size_t)SHd * es}};
  for (int i = 0; i < n_params; ++i) ins[3 + i] = params[i];
  const Range outs[] = {{"state", state, (size_t)nstate * 4},
                        {"norm_state", norm_state, (size_t)(SH * D) * 4},
                        {"y", y, (size_t)SHd * 4}};
  ssd_status s;
  if ((s = check_aligned(ins, 3 + n_params)) != SSD_OK || (s = check_aligned(outs, 3)) != SSD_OK)
    return s;
  return check_alias(outs, 3, ins, 3 + n_params);
}

ssd_status ssd_decode_step(const void* q, const void* k, const void* v, const float* dt_proj,
                           const float* dt_bias, const float* A_log, int64_t S, int64_t H,
                           int64_t d_h, int order, int dtype, int layout, float* state,
                           float* norm_state, float* y, hipStream_t stream) {
  try {
    clear_err();
    int64_t SH = 0;
    (void)mul_ok(S, H, &SH);
    const Range params[] = {{"dt_proj", dt_proj, (size_t)SH * 4},
                            {"dt_bias", dt_bias, (size_t)(H > 0 ? H : 0) * 4},
                            {"A_log", A_log, (size_t)(H > 0 ? H : 0) * 4}};
    bool empty;
    ssd_status s = decode_common("ssd_decode_step", q, k, v, params, 3, S, H, d_h, order, dtype,
                                 layout, state, norm_state, y, &empty);
    if (s != SSD_OK || empty) return s;
    if (!dt_proj || !dt_bias || !A_log)
      return fail(SSD_ERR_NULL, "ssd_decode_step: a required pointer is NULL");
    return hip_status(ssd::launch_decode(dtype == SSD_BF16, d_h, order, layout == SSD_STATE_PACKED, q, k,
                                         v, dt_proj, dt_bias, A_log, nullptr, S, H, state, norm_state,
                                         y, stream),
                      "decode launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_decode_step: unexpected exception");
  }
}

ssd_status ssd_decode_step_amask(const void* q, const void* k, const void* v, const float* A_proj,
                                 const float* dt_proj, int64_t S, int64_t H, int64_t d_h,
                                 int order, int dtype, int layout, float* state,
                                 float* norm_state, float* y, hipStream_t stream) {
  try {
    clear_err();
    int64_t SH = 0;
    (void)mul_ok(S, H, &SH);
    const Range params[] = {{"A_proj", A_proj, (size_t)SH * 4}, {"dt_proj", dt_proj, (size_t)SH * 4}};
    bool empty;
    ssd_status s = decode_common("ssd_decode_step_amask", q, k, v, params, 2, S, H, d_h, order, dtype,
                                 layout, state, norm_state, y, &empty);
    if (s != SSD_OK || empty) return s;
    if (!A_proj) return fail(SSD_ERR_NULL, "ssd_decode_step_amask: A_proj is NULL");
    return hip_status(ssd::launch_decode(dtype == SSD_BF16, d_h, order, layout == SSD_STATE_PACKED, q, k,
                                         v, dt_proj, nullptr, nullptr, A_proj, S, H, state,
                                         norm_state, y, stream),
                      "decode launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_decode_step_amask: unexpected exception");
  }
}

ssd_status ssd_decode_step_conv(const void* q, const void* k, const void* v, const float* conv_w,
                                const float* conv_b, int conv_act, void* conv_state,
                                const float* A_proj, const float* dt_proj, const float* dt_bias,
                                const float* A_log, int64_t S, int64_t H, int64_t d_h, int order,
                                int dtype, int layout, float* state, float* norm_state, float* y,
                                hipStream_t stream) {
  try {
    clear_err();
    const char* fn = "ssd_decode_step_conv";
    int64_t SH = 0, SHd = 0;
    (void)mul_ok(S, H, &SH);
    (void)mul_ok(SH, d_h, &SHd);
    const int64_t Hd = (H > 0 ? H : 0) * (d_h > 0 ? d_h : 0);
    const size_t es = dtype == SSD_BF16 ? 2 : 4;
    const Range params[] = {{"A_proj", A_proj, (size_t)SH * 4},
                            {"dt_proj", dt_proj, (size_t)SH * 4},
                            {"dt_bias", dt_bias, (size_t)(H > 0 ? H : 0) * 4},
                            {"A_log", A_log, (size_t)(H > 0 ? H : 0) * 4},
                            {"conv_w", conv_w, (size_t)(3 * Hd * 2) * 4},
                            {"conv_b", conv_b, (size_t)(3 * Hd) * 4}};
    bool empty;
    ssd_status s = decode_common(fn, q, k, v, params, 6, S, H, d_h, order, dtype, layout, state,
                                 norm_state, y, &empty);
    if (s != SSD_OK || empty) return s;
    if (conv_act != 0 && conv_act != 1) return fail(SSD_ERR_UNSUPPORTED, "%s: conv_act %d (0 or 1)", fn, conv_act);
    if (!conv_w || !conv_state) return fail(SSD_ERR_NULL, "%s: conv_w and conv_state are required", fn);
    if (A_proj) {
      if (dt_bias || A_log)
        return fail(SSD_ERR_UNSUPPORTED, "%s: with A_proj (the A-mask) dt_bias and A_log must be NULL", fn);
    } else if (!dt_proj || !dt_bias || !A_log) {
      return fail(SSD_ERR_NULL, "%s: without A_proj, dt_proj, dt_bias and A_log are required", fn);
    }
    // the conv state is read and written in place: it must not overlap any
    // other argument
    const Range cs{"conv_state", conv_state, (size_t)(3 * SHd) * es};
    if (!aligned16(conv_state)) return fail(SSD_ERR_ALIGN, "%s: conv_state is not 16-byte aligned", fn);
    const Range others[] = {{"q", q, (size_t)SHd * es}, {"k", k, (size_t)SHd * es},
                            {"v", v, (size_t)SHd * es}, params[0], params[1], params[2], params[3],
                            params[4], params[5]};
    if ((s = check_alias(&cs, 1, others, 9)) != SSD_OK) return s;
    int64_t D = order == 1 ? d_h : (layout == SSD_STATE_PACKED ? d_h * (d_h + 1) / 2 : d_h * d_h);
    const Range outs[] = {{"state", state, (size_t)(SH * D * d_h) * 4},
                          {"norm_state", norm_state, (size_t)(SH * D) * 4}, {"y", y, (size_t)SHd * 4}};
    if ((s = check_alias(outs, 3, &cs, 1)) != SSD_OK) return s;
    return hip_status(ssd::launch_decode(dtype == SSD_BF16, d_h, order, layout == SSD_STATE_PACKED, q, k, v,
                                         dt_proj, dt_bias, A_log, A_proj, S, H, state, norm_state, y, stream,
                                         ssd::DecodeConv{conv_w, conv_b, conv_state, conv_act}),
                      "decode launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_decode_step_conv: unexpected exception");
  }
}

// ssd_state_pack / ssd_state_unpack
static ssd_status state_layout(const char* fn, bool to_packed, const float* src_S, const float* src_z,
                               int64_t BH, int64_t d_h, float* dst_S, float* dst_z,
                               hipStream_t stream) {
  clear_err();
  if (BH < 0) return fail(SSD_ERR_SHAPE, "%s: BH must be >= 0", fn);
  if (d_h != 32 && d_h != 64) return fail(SSD_ERR_UNSUPPORTED, "d_h %lld (32 or 64)", (long long)d_h);
  if (BH == 0) return SSD_OK;
  if (!src_S || !src_z || !dst_S || !dst_z) return fail(SSD_ERR_NULL, "%s: a required pointer is NULL", fn);
  const int64_t Df = d_h * d_h, Dp = d_h * (d_h + 1) / 2;
  int64_t nf, np_;
  if (!mul_ok(BH, Df * d_h, &nf) || !mul_ok(BH, Dp * d_h, &np_) || BH * d_h > (int64_t)0x7fffffff)
    return fail(SSD_ERR_SHAPE, "%s: state too large", fn);
  const int64_t ns = to_packed ? nf : np_, nd = to_packed ? np_ : nf;
  const int64_t zs = (to_packed ? Df : Dp) * BH, zd = (to_packed ? Dp : Df) * BH;
  const Range ins[] = {{"source state", src_S, (size_t)ns * 4}, {"source norm", src_z, (size_t)zs * 4}};
  const Range outs[] = {{"state", dst_S, (size_t)nd * 4}, {"norm", dst_z, (size_t)zd * 4}};
  ssd_status s;
  if ((s = check_aligned(ins, 2)) != SSD_OK || (s = check_aligned(outs, 2)) != SSD_OK) return s;
  if ((s = check_alias(outs, 2, ins, 2)) != SSD_OK) return s;
  return hip_status(ssd::launch_state_layout(to_packed, d_h, BH, src_S, src_z, dst_S, dst_z, stream),
                    "state layout launch");
}

ssd_status ssd_state_pack(const float* state, const float* norm_state, int64_t BH, int64_t d_h,
                          float* state_p, float* norm_p, hipStream_t stream) {
  try {
    return state_layout("ssd_state_pack", true, state, norm_state, BH, d_h, state_p, norm_p, stream);
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_state_pack: unexpected exception");
  }
}

ssd_status ssd_state_unpack(const float* state_p, const float* norm_p, int64_t BH, int64_t d_h,
                            float* state, float* norm_state, hipStream_t stream) {
  try {
    return state_layout("ssd_state_unpack", false, state_p, norm_p, BH, d_h, state, norm_state, stream);
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_state_unpack: unexpected exception");
  }
}

size_t ssd_backward_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d_h, int order,
                                   int64_t chunk, int dtype) {
  int64_t BH, BHN, BHNd;
  if (validate_forward_sizes(B, H, N, d_h, order, chunk, dtype, &BH, &BHN, &BHNd) != SSD_OK) return 0;
  if (BHN == 0) return 0;
  return ssd::bwd_layout(BH, N, d_h, order).total_floats * sizeof(float);
}

ssd_status ssd_backward(const void* q, const void* k, const void* v, const float* dt,
                        const float* a_cs, const float* y, const float* den, const float* dy,
                        int64_t B, int64_t H, int64_t N, int64_t d_h, int order, int64_t chunk,
                        int dtype, float* dq, float* dk, float* dv, float* ddt, float* da,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    clear_err();
    int64_t BH, BHN, BHNd;
    ssd_status s = validate_forward_sizes(B, H, N, d_h, order, chunk, dtype, &BH, &BHN, &BHNd);
    if (s != SSD_OK) return s;
    if (BHN == 0) return SSD_OK;  // nothing to differentiate
    if (!q || !k || !v || !a_cs || !y || !den || !dy || !dq || !dk || !dv || !da)
      return fail(SSD_ERR_NULL, "ssd_backward: a required pointer is NULL");
    if ((dt == nullptr) != (ddt == nullptr))
      return fail(SSD_ERR_NULL, "ssd_backward: dt and ddt must be given together");
    const size_t need = ssd::bwd_layout(BH, N, d_h, order).total_floats * sizeof(float);
    if (workspace_bytes < need || !workspace)
      return fail(SSD_ERR_WORKSPACE, "ssd_backward: workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : (size_t)0);
    const size_t es = dtype == SSD_BF16 ? 2 : 4;
    const Range ins[] = {{"q", q, (size_t)BHNd * es},  {"k", k, (size_t)BHNd * es},
                         {"v", v, (size_t)BHNd * es},  {"dt", dt, (size_t)BHN * 4},
                         {"a_cs", a_cs, (size_t)BHN * 4}, {"y", y, (size_t)BHNd * 4},
                         {"den", den, (size_t)BHN * 4}, {"dy", dy, (size_t)BHNd * 4}};
    const Range outs[] = {{"dq", dq, (size_t)BHNd * 4}, {"dk", dk, (size_t)BHNd * 4},
                          {"dv", dv, (size_t)BHNd * 4}, {"ddt", ddt, (size_t)BHN * 4},
                          {"da", da, (size_t)BHN * 4},  {"workspace", workspace, need}};
    if ((s = check_aligned(ins, 8)) != SSD_OK || (s = check_aligned(outs, 6)) != SSD_OK) return s;
    if ((s = check_alias(outs, 6, ins, 8)) != SSD_OK) return s;
    return hip_status(ssd::launch_backward(order, dtype == SSD_BF16, d_h, q, k, v, dt, a_cs, y, den, dy, BH,
                                           N, chunk, dq, dk, dv, ddt, da, static_cast<float*>(workspace),
                                           stream),
                      "backward launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_backward: unexpected exception");
  }
}

// shared size validation of the two discretisation backward calls
static ssd_status prep_bwd_sizes(const char* fn, int64_t B, int64_t H, int64_t N, int64_t* BHN) {
  int64_t BH;
  if (!mul_ok(B, H, &BH) || !mul_ok(BH, N, BHN))
    return fail(SSD_ERR_SHAPE, "%s: B, H, N must be >= 0 and must not overflow", fn);
  if (H > (int64_t)0x7fffffff) return fail(SSD_ERR_SHAPE, "%s: H too large", fn);
  return SSD_OK;
}

ssd_status ssd_prep_backward(const float* dt_proj, const float* dt_bias, const float* A_log,
                             const float* da, const float* ddt, int64_t B, int64_t H, int64_t N,
                             float* d_dt_proj, float* d_dt_bias, float* d_A_log, hipStream_t stream) {
  try {
    clear_err();
    int64_t BHN;
    ssd_status s = prep_bwd_sizes("ssd_prep_backward", B, H, N, &BHN);
    if (s != SSD_OK) return s;
    if (H == 0) return SSD_OK;
    if (!dt_bias || !A_log || !d_dt_bias || !d_A_log || (BHN && (!dt_proj || !da || !d_dt_proj)))
      return fail(SSD_ERR_NULL, "ssd_prep_backward: a required pointer is NULL");
    const Range ins[] = {{"dt_proj", dt_proj, (size_t)BHN * 4}, {"dt_bias", dt_bias, (size_t)H * 4},
                         {"A_log", A_log, (size_t)H * 4},       {"da", da, (size_t)BHN * 4},
                         {"ddt", ddt, (size_t)BHN * 4}};
    const Range outs[] = {{"d_dt_proj", d_dt_proj, (size_t)BHN * 4},
                          {"d_dt_bias", d_dt_bias, (size_t)H * 4},
                          {"d_A_log", d_A_log, (size_t)H * 4}};
    if ((s = check_aligned(ins, 5)) != SSD_OK || (s = check_aligned(outs, 3)) != SSD_OK) return s;
    if ((s = check_alias(outs, 3, ins, 5)) != SSD_OK) return s;
    return hip_status(ssd::launch_prep_backward(dt_proj, dt_bias, A_log, da, ddt, B, H, N, d_dt_proj,
                                                d_dt_bias, d_A_log, stream),
                      "prep backward launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_prep_backward: unexpected exception");
  }
}

ssd_status ssd_prep_amask_backward(const float* A_proj, const float* dt_proj, const float* da,
                                   const float* ddt, int64_t B, int64_t H, int64_t N,
                                   float* d_A_proj, float* d_dt_proj, hipStream_t stream) {
  try {
    clear_err();
    int64_t BHN;
    ssd_status s = prep_bwd_sizes("ssd_prep_amask_backward", B, H, N, &BHN);
    if (s != SSD_OK) return s;
    if (BHN == 0) return SSD_OK;
    if (!A_proj || !da || !d_A_proj)
      return fail(SSD_ERR_NULL, "ssd_prep_amask_backward: a required pointer is NULL");
    if ((dt_proj == nullptr) != (ddt == nullptr) || (dt_proj == nullptr) != (d_dt_proj == nullptr))
      return fail(SSD_ERR_NULL, "ssd_prep_amask_backward: dt_proj, ddt and d_dt_proj go together");
    const Range ins[] = {{"A_proj", A_proj, (size_t)BHN * 4}, {"dt_proj", dt_proj, (size_t)BHN * 4},
                         {"da", da, (size_t)BHN * 4},         {"ddt", ddt, (size_t)BHN * 4}};
    const Range outs[] = {{"d_A_proj", d_A_proj, (size_t)BHN * 4},
                          {"d_dt_proj", d_dt_proj, (size_t)BHN * 4}};
    if ((s = check_aligned(ins, 4)) != SSD_OK || (s = check_aligned(outs, 2)) != SSD_OK) return s;
    if ((s = check_alias(outs, 2, ins, 4)) != SSD_OK) return s;
    return hip_status(ssd::launch_prep_amask_backward(A_proj, dt_proj, da, ddt, B, H, N, d_A_proj,
                                                      d_dt_proj, stream),
                      "prep amask backward launch");
  } catch (...) {
    return fail(SSD_ERR_HIP, "ssd_prep_amask_backward: unexpected exception");
  }
}

}  // extern "C"
