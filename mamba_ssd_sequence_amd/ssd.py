"""Thin Python binding of libssd.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/ssd.h.  PyTorch supplies device memory and
the current HIP stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.

    dt, a_cs, a_chunk = prep(dt_proj, dt_bias, A_log, chunk)
    y = forward(q, k, v, dt, a_cs, order=2, chunk=64)
    y = decode_step(q, k, v, dt_proj, dt_bias, A_log, state, norm_state, order=2)
    y = decode_step_amask(q, k, v, A_proj, dt_proj, state, norm_state, order=2)
    y = decode_step_conv(q, k, v, conv_w, conv_b, conv_state, state, norm_state, order=2, A_proj=A_proj)
    state_p, norm_p = state_pack(state, norm_state)
    dq, dk, dv, ddt, da = backward(q, k, v, dt, a_cs, y, den, dy, order=2, chunk=64)
    d_dt_proj, d_dt_bias, d_A_log = prep_backward(dt_proj, dt_bias, A_log, da, ddt)
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libssd.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "ssd.h")

SSD_OK = 0
SSD_F32 = 0
SSD_BF16 = 1
SSD_STATE_FULL = 0
SSD_STATE_PACKED = 1
SSD_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/ssd.h
STATUS = ["SSD_OK", "SSD_ERR_NULL", "SSD_ERR_SHAPE", "SSD_ERR_UNSUPPORTED", "SSD_ERR_ALIGN",
          "SSD_ERR_ALIAS", "SSD_ERR_WORKSPACE", "SSD_ERR_HIP"]

_lib = None


class SSDError(RuntimeError):
    def __init__(self, status: int, msg: str):
        name = STATUS[status] if 0 <= status < len(STATUS) else str(status)
        super().__init__(f"{name}: {msg}")
        self.status = status


def _declare(lib):
    i64, vp, fp, i32, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.ssd_abi_version.restype = ctypes.c_int
    lib.ssd_abi_version.argtypes = []
    lib.ssd_status_str.restype = ctypes.c_char_p
    lib.ssd_status_str.argtypes = [ctypes.c_int]
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_last_error.argtypes = []
    lib.ssd_prep.restype = ctypes.c_int
    lib.ssd_prep.argtypes = [fp, fp, fp, i64, i64, i64, i64, fp, fp, fp, vp]
    lib.ssd_prep_amask.restype = ctypes.c_int
    lib.ssd_prep_amask.argtypes = [fp, fp, i64, i64, i64, i64, fp, fp, fp, vp]
    lib.ssd_forward_workspace_size.restype = sz
    lib.ssd_forward_workspace_size.argtypes = [i64, i64, i64, i64, i32, i64, i32]
    lib.ssd_forward.restype = ctypes.c_int
    lib.ssd_forward.argtypes = [vp, vp, vp, fp, fp, fp, fp, i64, i64, i64, i64, i32, i64, i32,
                                fp, fp, fp, fp, vp, sz, vp]
    lib.ssd_forward_noalloc.restype = ctypes.c_int
    lib.ssd_forward_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, fp, i64, i64, i64, i64, i32, i64, i32,
                                        fp, fp, fp, fp, vp]
    lib.ssd_set_timing_events.restype = ctypes.c_int
    lib.ssd_set_timing_events.argtypes = [vp, ctypes.c_int]
    lib.ssd_timing_count.restype = ctypes.c_int
    lib.ssd_timing_count.argtypes = []
    lib.ssd_decode_step.restype = ctypes.c_int
    lib.ssd_decode_step.argtypes = [vp, vp, vp, fp, fp, fp, i64, i64, i64, i32, i32, i32, fp, fp, fp, vp]
    lib.ssd_decode_step_amask.restype = ctypes.c_int
    lib.ssd_decode_step_amask.argtypes = [vp, vp, vp, fp, fp, i64, i64, i64, i32, i32, i32, fp, fp, fp, vp]
    lib.ssd_decode_step_conv.restype = ctypes.c_int
    lib.ssd_decode_step_conv.argtypes = [vp, vp, vp, fp, fp, i32, vp, fp, fp, fp, fp, i64, i64, i64, i32,
                                         i32, i32, fp, fp, fp, vp]
    lib.ssd_state_pack.restype = ctypes.c_int
    lib.ssd_state_pack.argtypes = [fp, fp, i64, i64, fp, fp, vp]
    lib.ssd_state_unpack.restype = ctypes.c_int
    lib.ssd_state_unpack.argtypes = [fp, fp, i64, i64, fp, fp, vp]
    lib.ssd_backward_workspace_size.restype = sz
    lib.ssd_backward_workspace_size.argtypes = [i64, i64, i64, i64, i32, i64, i32]
    lib.ssd_backward.restype = ctypes.c_int
    lib.ssd_backward.argtypes = [vp, vp, vp, fp, fp, fp, fp, fp, i64, i64, i64, i64, i32, i64, i32,
                                 fp, fp, fp, fp, fp, vp, sz, vp]
    lib.ssd_prep_backward.restype = ctypes.c_int
    lib.ssd_prep_backward.argtypes = [fp, fp, fp, fp, fp, i64, i64, i64, fp, fp, fp, vp]
    lib.ssd_prep_amask_backward.restype = ctypes.c_int
    lib.ssd_prep_amask_backward.argtypes = [fp, fp, fp, fp, i64, i64, i64, fp, fp, vp]
    return lib


def lib():
    """Load libssd.so (built in-tree by ``python -m mamba_ssd_sequence_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mamba_ssd_sequence_amd.build` (no fallback path exists)")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/ssd.h."""
    with open(HEADER) as f:
        txt = f.read()
    return sorted(set(re.findall(r"^\s*(?:ssd_status|size_t|int|const char\*)\s+(ssd_\w+)\s*\(", txt, re.M)))


def _check(status: int):
    if status != SSD_OK:
        raise SSDError(status, lib().ssd_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _qkv_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise ValueError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def prep(dt_proj, dt_bias, A_log, chunk: int, out=None):
    """ssd_prep: returns (dt [B,H,N], a_cs [B,H,N], a_chunk [B,H,ceil(N/chunk)])."""
    torch = _torch()
    f32 = torch.float32
    _require(dt_proj, "dt_proj", f32)
    dev = dt_proj.device
    _require(dt_bias, "dt_bias", f32, dev)
    _require(A_log, "A_log", f32, dev)
    B, H, N = dt_proj.shape
    if dt_bias.shape != (H,) or A_log.shape != (H,):
        raise ValueError("dt_bias and A_log must have shape [H]")
    nc = -(-N // chunk)
    if out is None:
        out = (torch.empty_like(dt_proj), torch.empty_like(dt_proj),
               torch.empty((B, H, nc), dtype=f32, device=dev))
    dt, a_cs, a_chunk = out
    _check(lib().ssd_prep(_ptr(dt_proj), _ptr(dt_bias), _ptr(A_log), B, H, N, chunk,
                          _ptr(dt), _ptr(a_cs), _ptr(a_chunk), _stream(dev)))
    return dt, a_cs, a_chunk


def prep_amask(A_proj, dt_proj, chunk: int, out=None):
    """ssd_prep_amask (the A-mask of Algorithms 4 and 5): returns (dt or None,
    a_cs, a_chunk); dt_proj None means no dt (plain value operand)."""
    torch = _torch()
    f32 = torch.float32
    _require(A_proj, "A_proj", f32)
    dev = A_proj.device
    if dt_proj is not None:
        _require(dt_proj, "dt_proj", f32, dev)
        if dt_proj.shape != A_proj.shape:
            raise ValueError("dt_proj must have the shape of A_proj")
    B, H, N = A_proj.shape
    nc = -(-N // chunk)
    if out is None:
        out = (torch.empty_like(A_proj) if dt_proj is not None else None, torch.empty_like(A_proj),
               torch.empty((B, H, nc), dtype=f32, device=dev))
    dt, a_cs, a_chunk = out
    _check(lib().ssd_prep_amask(_ptr(A_proj), _ptr(dt_proj), B, H, N, chunk, _ptr(dt), _ptr(a_cs),
                                _ptr(a_chunk), _stream(dev)))
    return dt, a_cs, a_chunk


def workspace_size(B, H, N, d_h, order, chunk, dtype) -> int:
    return int(lib().ssd_forward_workspace_size(B, H, N, d_h, order, chunk, dtype))


def forward(q, k, v, dt, a_cs, order: int, chunk: int, *, y=None, den=None,
            final_state=None, final_norm=None, workspace=None, initial_state=None,
            initial_norm=None):
    """ssd_forward: y [B,H,N,d_h] fp32 (den and final states optional outputs;
    initial states optional inputs).  workspace: a uint8 device tensor, None
    (one is allocated), or "noalloc" for ssd_forward_noalloc (the library's
    per-device scratch; sizes up to SSD_NOALLOC_SCRATCH_BYTES of workspace)."""
    torch = _torch()
    _require(q, "q")
    dev = q.device
    dtype = _qkv_dtype(q)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, q.dtype, dev)
        if t.shape != q.shape:
            raise ValueError(f"{name} shape {tuple(t.shape)} != q shape {tuple(q.shape)}")
    B, H, N, d_h = q.shape
    if dt is not None:
        _require(dt, "dt", torch.float32, dev)
    _require(a_cs, "a_cs", torch.float32, dev)
    if y is None:
        y = torch.empty((B, H, N, d_h), dtype=torch.float32, device=dev)
    for name, t in (("y", y), ("den", den), ("final_state", final_state), ("final_norm", final_norm),
                    ("initial_state", initial_state), ("initial_norm", initial_norm)):
        if t is not None:
            _require(t, name, torch.float32, dev)
    if workspace == "noalloc":
        # ssd_forward_noalloc: the library's own per-device scratch, no workspace
        _check(lib().ssd_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a_cs), _ptr(initial_state),
                                         _ptr(initial_norm), B, H, N, d_h, order, chunk, dtype, _ptr(y),
                                         _ptr(den), _ptr(final_state), _ptr(final_norm), _stream(dev)))
        return y
    need = workspace_size(B, H, N, d_h, order, chunk, dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().ssd_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(dt), _ptr(a_cs), _ptr(initial_state),
                             _ptr(initial_norm), B, H, N, d_h, order,
                             chunk, dtype, _ptr(y), _ptr(den), _ptr(final_state), _ptr(final_norm),
                             _ptr(workspace), wbytes, _stream(dev)))
    return y


class KernelTimer:
    """Per-kernel HIP-event timing of one ssd_forward call (events recorded by
    the library on its own stream, between its kernel launches)."""

    N_EVENTS = 8

    def __init__(self):
        torch = _torch()
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(self.N_EVENTS)]
        for e in self.events:  # materialise the underlying hipEvent_t
            e.record()
        self._arr = (ctypes.c_void_p * self.N_EVENTS)(*[e.cuda_event for e in self.events])
        self.count = 0

    def arm(self):
        _check(lib().ssd_set_timing_events(self._arr, self.N_EVENTS))

    def collect(self):
        """After ssd_forward: remember how many kernels were bracketed."""
        self.count = lib().ssd_timing_count()

    def durations_ms(self):
        """Per-kernel durations (call after synchronising)."""
        return [self.events[i].elapsed_time(self.events[i + 1]) for i in range(self.count)]


def _decode_common(q, k, v, params, state, norm_state, order, y, packed):
    torch = _torch()
    _require(q, "q")
    dev = q.device
    dtype = _qkv_dtype(q)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, q.dtype, dev)
    S, H, d_h = q.shape
    for name, t in params + (("state", state), ("norm_state", norm_state)):
        if t is not None:
            _require(t, name, torch.float32, dev)
    if y is None:
        y = torch.empty((S, H, d_h), dtype=torch.float32, device=dev)
    layout = SSD_STATE_PACKED if packed else SSD_STATE_FULL
    return dev, dtype, S, H, d_h, layout, y


def decode_step(q, k, v, dt_proj, dt_bias, A_log, state, norm_state, order: int, *, y=None,
                packed=False):
    """ssd_decode_step: updates state/norm_state in place, returns y [S,H,d_h] fp32.
    packed: the order-2 states are in the packed layout (rows a <= b)."""
    dev, dtype, S, H, d_h, layout, y = _decode_common(
        q, k, v, (("dt_proj", dt_proj), ("dt_bias", dt_bias), ("A_log", A_log)), state, norm_state,
        order, y, packed)
    _check(lib().ssd_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(dt_proj), _ptr(dt_bias), _ptr(A_log),
                                 S, H, d_h, order, dtype, layout, _ptr(state), _ptr(norm_state), _ptr(y),
                                 _stream(dev)))
    return y


def decode_step_amask(q, k, v, A_proj, dt_proj, state, norm_state, order: int, *, y=None,
                      packed=False):
    """ssd_decode_step_amask (Algorithm 6 as printed): decay exp(-softplus(A_P));
    value operand v softplus(dt_P), or plain v when dt_proj is None."""
    dev, dtype, S, H, d_h, layout, y = _decode_common(
        q, k, v, (("A_proj", A_proj), ("dt_proj", dt_proj)), state, norm_state, order, y, packed)
    _check(lib().ssd_decode_step_amask(_ptr(q), _ptr(k), _ptr(v), _ptr(A_proj),
                                       _ptr(dt_proj) if dt_proj is not None else None,
                                       S, H, d_h, order, dtype, layout, _ptr(state), _ptr(norm_state),
                                       _ptr(y), _stream(dev)))
    return y


def decode_step_conv(q, k, v, conv_w, conv_b, conv_state, state, norm_state, order: int, *,
                     A_proj=None, dt_proj=None, dt_bias=None, A_log=None, act=False, y=None,
                     packed=False):
    """ssd_decode_step_conv: Algorithm 6's window-2 convolution of the raw q, k,
    v [S,H,d_h] (conv_w [3,H,d_h,2], conv_b [3,H,d_h] or None, SiLU if act)
    with the previous raw token held in conv_state [S,3,H,d_h] (updated in
    place), then the decode step: the A-mask with A_proj (optional dt_proj),
    else the Mamba-2 discretisation (dt_proj, dt_bias, A_log)."""
    dev, dtype, S, H, d_h, layout, y = _decode_common(
        q, k, v, (("A_proj", A_proj), ("dt_proj", dt_proj), ("dt_bias", dt_bias), ("A_log", A_log),
                  ("conv_w", conv_w), ("conv_b", conv_b)), state, norm_state, order, y, packed)
    _require(conv_state, "conv_state", q.dtype, dev)
    if tuple(conv_state.shape) != (S, 3, H, d_h) or tuple(conv_w.shape) != (3, H, d_h, 2):
        raise ValueError(f"conv_state {tuple(conv_state.shape)} / conv_w {tuple(conv_w.shape)} do not match "
                         f"[{S},3,{H},{d_h}] / [3,{H},{d_h},2]")
    if conv_b is not None and tuple(conv_b.shape) != (3, H, d_h):
        raise ValueError(f"conv_b {tuple(conv_b.shape)} does not match [3,{H},{d_h}]")
    _check(lib().ssd_decode_step_conv(_ptr(q), _ptr(k), _ptr(v), _ptr(conv_w), _ptr(conv_b), 1 if act else 0,
                                      _ptr(conv_state), _ptr(A_proj), _ptr(dt_proj), _ptr(dt_bias),
                                      _ptr(A_log), S, H, d_h, order, dtype, layout, _ptr(state),
                                      _ptr(norm_state), _ptr(y), _stream(dev)))
    return y


def _state_layout(fn, src_S, src_z, to_packed, out):
    torch = _torch()
    _require(src_S, "state", torch.float32)
    dev = src_S.device
    _require(src_z, "norm", torch.float32, dev)
    lead = src_S.shape[:-2]
    d_h = src_S.shape[-1]
    BH = 1
    for n in lead:
        BH *= n
    src_rows = d_h * d_h if to_packed else d_h * (d_h + 1) // 2
    if src_S.shape[-2] != src_rows or tuple(src_z.shape) != tuple(lead) + (src_rows,):
        raise ValueError(f"state shape {tuple(src_S.shape)} / norm shape {tuple(src_z.shape)} "
                         f"do not match {src_rows} rows of width {d_h}")
    rows = d_h * (d_h + 1) // 2 if to_packed else d_h * d_h
    if out is None:
        out = (torch.empty(lead + (rows, d_h), dtype=torch.float32, device=dev),
               torch.empty(lead + (rows,), dtype=torch.float32, device=dev))
    _check(fn(_ptr(src_S), _ptr(src_z), BH, d_h, _ptr(out[0]), _ptr(out[1]), _stream(dev)))
    return out


def state_pack(state, norm_state, out=None):
    """ssd_state_pack: full order-2 states [..., d_h^2, d_h], [..., d_h^2] ->
    packed [..., d_h(d_h+1)/2, d_h], [..., d_h(d_h+1)/2]."""
    return _state_layout(lib().ssd_state_pack, state, norm_state, True, out)


def state_unpack(state_p, norm_p, out=None):
    """ssd_state_unpack: packed order-2 states -> the full layout."""
    return _state_layout(lib().ssd_state_unpack, state_p, norm_p, False, out)


def backward(q, k, v, dt, a_cs, y, den, dy, order: int, chunk: int, *, workspace=None):
    """ssd_backward: returns dq, dk, dv, ddt (None when dt is None), da."""
    torch = _torch()
    _require(q, "q")
    dev = q.device
    dtype = _qkv_dtype(q)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, q.dtype, dev)
    B, H, N, d_h = q.shape
    for name, t in (("a_cs", a_cs), ("y", y), ("den", den), ("dy", dy)) + ((("dt", dt),) if dt is not None else ()):
        _require(t, name, torch.float32, dev)
    dq, dk, dv = (torch.empty((B, H, N, d_h), dtype=torch.float32, device=dev) for _ in range(3))
    da = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ddt = torch.empty((B, H, N), dtype=torch.float32, device=dev) if dt is not None else None
    need = lib().ssd_backward_workspace_size(B, H, N, d_h, order, chunk, dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wptr = _ptr(workspace) if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    opt = lambda t: _ptr(t) if t is not None else None
    _check(lib().ssd_backward(_ptr(q), _ptr(k), _ptr(v), opt(dt), _ptr(a_cs), _ptr(y), _ptr(den), _ptr(dy),
                              B, H, N, d_h, order, chunk, dtype, _ptr(dq), _ptr(dk), _ptr(dv), opt(ddt),
                              _ptr(da), wptr, wbytes, _stream(dev)))
    return dq, dk, dv, ddt, da


def prep_backward(dt_proj, dt_bias, A_log, da, ddt=None):
    """ssd_prep_backward: returns d_dt_proj [B,H,N], d_dt_bias [H], d_A_log [H]."""
    torch = _torch()
    _require(dt_proj, "dt_proj", torch.float32)
    dev = dt_proj.device
    for name, t in (("dt_bias", dt_bias), ("A_log", A_log), ("da", da)) + ((("ddt", ddt),) if ddt is not None else ()):
        _require(t, name, torch.float32, dev)
    B, H, N = dt_proj.shape
    d_dt_proj = torch.empty_like(dt_proj)
    d_bias = torch.empty((H,), dtype=torch.float32, device=dev)
    d_alog = torch.empty((H,), dtype=torch.float32, device=dev)
    _check(lib().ssd_prep_backward(_ptr(dt_proj), _ptr(dt_bias), _ptr(A_log), _ptr(da),
                                   _ptr(ddt) if ddt is not None else None, B, H, N, _ptr(d_dt_proj),
                                   _ptr(d_bias), _ptr(d_alog), _stream(dev)))
    return d_dt_proj, d_bias, d_alog


def prep_amask_backward(A_proj, dt_proj, da, ddt=None):
    """ssd_prep_amask_backward: returns d_A_proj and d_dt_proj (None without dt_proj)."""
    torch = _torch()
    _require(A_proj, "A_proj", torch.float32)
    dev = A_proj.device
    _require(da, "da", torch.float32, dev)
    if (dt_proj is None) != (ddt is None):
        raise ValueError("dt_proj and ddt go together")
    if dt_proj is not None:
        _require(dt_proj, "dt_proj", torch.float32, dev)
        _require(ddt, "ddt", torch.float32, dev)
    B, H, N = A_proj.shape
    d_A = torch.empty_like(A_proj)
    d_dt = torch.empty_like(A_proj) if dt_proj is not None else None
    opt = lambda t: _ptr(t) if t is not None else None
    _check(lib().ssd_prep_amask_backward(_ptr(A_proj), opt(dt_proj), _ptr(da), opt(ddt), B, H, N,
                                         _ptr(d_A), opt(d_dt), _stream(dev)))
    return d_A, d_dt
