"""The C ABI on the CPU: the library loads, exports every function include/ssd.h
declares, and rejects bad arguments before any HIP call (fake, never
dereferenced addresses are passed; no call here reaches a kernel launch)."""
import ctypes

import pytest

from mamba_ssd_sequence_amd import ssd

A = [0x100000 * (i + 1) for i in range(24)]  # distinct, 16-byte aligned fake addresses


@pytest.fixture(scope="module")
def lib():
    return ssd.lib()


def test_exports_every_header_function(lib):
    names = ssd.header_functions()
    assert set(names) >= {"ssd_prep", "ssd_prep_amask", "ssd_forward", "ssd_forward_workspace_size",
                          "ssd_forward_noalloc", "ssd_decode_step", "ssd_decode_step_amask",
                          "ssd_decode_step_conv",
                          "ssd_state_pack",
                          "ssd_state_unpack", "ssd_backward", "ssd_backward_workspace_size",
                          "ssd_prep_backward", "ssd_prep_amask_backward",
                          "ssd_abi_version", "ssd_status_str", "ssd_last_error"}
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.ssd_abi_version() == 6
    for i, name in enumerate(ssd.STATUS):
        assert lib.ssd_status_str(i).decode() == name
    assert lib.ssd_status_str(99).decode() == "SSD_ERR_UNKNOWN"


def prep(lib, *, ptrs=None, B=1, H=2, N=100, chunk=64):
    p = list(A[:6]) if ptrs is None else ptrs
    return lib.ssd_prep(p[0], p[1], p[2], B, H, N, chunk, p[3], p[4], p[5], None)


def test_prep_errors(lib):
    assert prep(lib, ptrs=[A[0], None, A[2], A[3], A[4], A[5]]) == 1
    assert "NULL" in lib.ssd_last_error().decode()
    assert prep(lib, B=-1) == 2
    assert prep(lib, N=-5) == 2
    assert prep(lib, B=1 << 40, H=1 << 40) == 2
    assert prep(lib, chunk=32) == 3
    assert prep(lib, ptrs=[A[0] + 4] + A[1:6]) == 4
    assert prep(lib, ptrs=A[:3] + [A[0]] + A[4:6]) == 5  # dt output aliases dt_proj
    assert prep(lib, ptrs=A[:3] + [A[3], A[3] + 16, A[5]]) == 5  # outputs overlap each other


def prep_amask(lib, *, ptrs=None, B=1, H=2, N=100, chunk=64):
    p = [A[0], A[1], A[3], A[4], A[5]] if ptrs is None else ptrs
    return lib.ssd_prep_amask(p[0], p[1], B, H, N, chunk, p[2], p[3], p[4], None)


def test_prep_amask_errors(lib):
    assert prep_amask(lib, ptrs=[None, A[1], A[3], A[4], A[5]]) == 1
    assert prep_amask(lib, ptrs=[A[0], None, A[3], A[4], A[5]]) == 1  # dt without dt_proj
    assert "both" in lib.ssd_last_error().decode()
    assert prep_amask(lib, ptrs=[A[0], A[1], None, A[4], A[5]]) == 1  # dt_proj without dt
    assert prep_amask(lib, B=-1) == 2
    assert prep_amask(lib, N=-1) == 2
    assert prep_amask(lib, chunk=256) == 3
    assert prep_amask(lib, ptrs=[A[0] + 8, A[1], A[3], A[4], A[5]]) == 4
    assert prep_amask(lib, ptrs=[A[0], A[1], A[3], A[0], A[5]]) == 5  # a_cs aliases A_proj
    assert prep_amask(lib, ptrs=[A[0], None, None, A[4], A[4] + 16]) == 5  # outputs overlap


def fwd(lib, *, B=1, H=2, N=100, d_h=64, order=1, chunk=64, dtype=1, ws=None, wbytes=None,
        q=A[0], dt=A[3], y=A[10], den=None, fs=None, fn=None, s0=None, z0=None):
    need = lib.ssd_forward_workspace_size(B, H, N, d_h, order, chunk, dtype)
    ws = A[20] if ws is None else ws
    wbytes = need if wbytes is None else wbytes
    return lib.ssd_forward(q, A[1], A[2], dt, A[4], s0, z0, B, H, N, d_h, order, chunk, dtype,
                           y, den, fs, fn, ws, wbytes, None)


def test_forward_errors(lib):
    assert fwd(lib, q=None) == 1
    assert fwd(lib, y=None) == 1
    assert fwd(lib, fs=A[11], fn=None) == 1
    assert fwd(lib, N=-1) == 2
    assert fwd(lib, d_h=48) == 3
    assert fwd(lib, order=3) == 3
    assert fwd(lib, chunk=256) == 3
    assert fwd(lib, dtype=7) == 3
    assert fwd(lib, order=2, d_h=32) == 3
    assert fwd(lib, order=2, dtype=0) == 3
    assert fwd(lib, q=A[0] + 2) == 4
    assert fwd(lib, y=A[1]) == 5  # y aliases k
    assert "output y overlaps input k" in lib.ssd_last_error().decode()
    assert fwd(lib, den=A[10] + 16) == 5  # den overlaps y
    assert fwd(lib, s0=A[12], z0=None) == 1  # initial_state without initial_norm
    assert "initial_state" in lib.ssd_last_error().decode()
    assert fwd(lib, s0=A[12] + 4, z0=A[13]) == 4
    assert fwd(lib, s0=A[12], z0=A[13], fs=A[12], fn=A[14]) == 5  # final_state aliases initial_state
    assert fwd(lib, wbytes=16) == 6
    assert fwd(lib, ws=0) == 6


def fwd_noalloc(lib, *, B=1, H=2, N=100, d_h=64, order=1, q=A[0], y=A[10]):
    return lib.ssd_forward_noalloc(q, A[1], A[2], A[3], A[4], None, None, B, H, N, d_h, order, 64, 1,
                                   y, None, None, None, None)


def test_forward_noalloc_errors(lib):
    # sizes whose workspace exceeds the library's per-device scratch are
    # rejected before any HIP call (every call here is invalid)
    assert lib.ssd_forward_workspace_size(2, 16, 4096, 64, 2, 64, 1) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    assert fwd_noalloc(lib, B=2, H=16, N=4096, order=2) == 6
    msg = lib.ssd_last_error().decode()
    assert "scratch" in msg and str(ssd.SSD_NOALLOC_SCRATCH_BYTES) in msg
    assert fwd_noalloc(lib, q=None) == 1
    assert fwd_noalloc(lib, d_h=48) == 3
    assert fwd_noalloc(lib, y=A[1]) == 5  # y aliases k
    assert fwd_noalloc(lib, B=0) == 0     # empty: nothing to do


def test_workspace_size(lib):
    # order 1: block totals + per-block states; order 2 adds the a-slice partials
    B, H, N, d = 2, 3, 200, 64
    nb = -(-N // 64)
    w1 = lib.ssd_forward_workspace_size(B, H, N, d, 1, 64, 1)
    assert w1 >= 4 * (B * H * nb + B * H * nb * (d * d + d))
    w2 = lib.ssd_forward_workspace_size(B, H, N, d, 2, 64, 1)
    assert w2 > w1 + 4 * B * H * N * 64
    assert lib.ssd_forward_workspace_size(B, H, N, 48, 1, 64, 1) == 0
    assert lib.ssd_forward_workspace_size(-1, H, N, d, 1, 64, 1) == 0
    assert lib.ssd_forward_workspace_size(B, H, 0, d, 2, 64, 1) == 0  # empty: no workspace


def dec(lib, *, S=1, H=1, d_h=64, order=2, dtype=1, layout=0, q=A[0], state=A[6], norm=A[7], y=A[8]):
    return lib.ssd_decode_step(q, A[1], A[2], A[3], A[4], A[5], S, H, d_h, order, dtype, layout,
                               state, norm, y, None)


def dec_amask(lib, *, S=1, H=1, d_h=64, order=2, layout=0, A_proj=A[3], dt_proj=A[4], norm=A[7]):
    return lib.ssd_decode_step_amask(A[0], A[1], A[2], A_proj, dt_proj, S, H, d_h, order, 1, layout,
                                     A[6], norm, A[8], None)


def test_decode_errors(lib):
    assert dec(lib, q=None) == 1
    assert dec(lib, state=None) == 1
    assert dec(lib, S=-1) == 2
    assert dec(lib, d_h=16) == 3
    assert dec(lib, order=0) == 3
    assert dec(lib, dtype=2) == 3
    assert dec(lib, y=A[8] + 8) == 4
    assert dec(lib, y=A[0]) == 5
    assert "y" in lib.ssd_last_error().decode() and "q" in lib.ssd_last_error().decode()
    assert dec(lib, norm=A[6] + 64) == 5  # norm_state inside state
    assert dec(lib, layout=2) == 3
    assert dec(lib, layout=1, order=1) == 3  # packing is for order 2


def test_decode_amask_errors(lib):
    assert dec_amask(lib, A_proj=None) == 1
    assert dec_amask(lib, A_proj=A[3] + 4) == 4
    assert dec_amask(lib, dt_proj=A[6]) == 5       # dt_proj inside the state output
    assert dec_amask(lib, norm=A[3]) == 5          # an output over A_proj
    assert dec_amask(lib, layout=1, order=1) == 3
    assert dec_amask(lib, d_h=48) == 3
    assert dec_amask(lib, S=-2) == 2


def dec_conv(lib, *, S=1, H=1, d_h=64, order=2, layout=0, conv_w=A[9], conv_b=A[10], act=0, cst=A[11],
             A_proj=A[3], dt_proj=A[4], dt_bias=None, A_log=None, norm=A[7]):
    return lib.ssd_decode_step_conv(A[0], A[1], A[2], conv_w, conv_b, act, cst, A_proj, dt_proj, dt_bias,
                                    A_log, S, H, d_h, order, 1, layout, A[6], norm, A[8], None)


def test_decode_conv_errors(lib):
    # every call here is rejected before any HIP call (none is valid)
    assert dec_conv(lib, conv_w=None) == 1
    assert dec_conv(lib, cst=None) == 1
    assert dec_conv(lib, act=2) == 3
    assert dec_conv(lib, dt_bias=A[12]) == 3                  # A-mask with Mamba-2 parameters
    assert dec_conv(lib, A_proj=None, dt_bias=None) == 1      # Mamba-2 without its parameters
    assert dec_conv(lib, cst=A[11] + 8) == 4
    assert dec_conv(lib, conv_w=A[9] + 4) == 4
    assert dec_conv(lib, cst=A[0]) == 5                        # conv state over q
    assert "conv_state" in lib.ssd_last_error().decode()
    assert dec_conv(lib, cst=A[6]) == 5                        # conv state inside the state output
    assert dec_conv(lib, cst=A[9] + 128) == 5                  # conv state over the weights
    assert dec_conv(lib, norm=A[9]) == 5                       # an output over the weights
    assert dec_conv(lib, d_h=48) == 3
    assert dec_conv(lib, S=-1) == 2
    assert dec_conv(lib, S=0, conv_w=None) == 0                # empty: nothing to do


def test_state_layout_errors(lib):
    for fn in (lib.ssd_state_pack, lib.ssd_state_unpack):
        assert fn(None, A[1], 2, 64, A[2], A[3], None) == 1
        assert fn(A[0], A[1], 2, 48, A[2], A[3], None) == 3
        assert fn(A[0], A[1], -1, 64, A[2], A[3], None) == 2
        assert fn(A[0], A[1], 2, 64, A[2] + 4, A[3], None) == 4
        assert fn(A[0], A[1], 2, 64, A[0], A[3], None) == 5  # destination over the source
        assert fn(None, None, 0, 64, None, None, None) == 0   # empty


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 64)
    with pytest.raises(ValueError):
        ssd.prep(x, torch.zeros(2), torch.zeros(2), 64)


def test_empty_inputs_are_valid_no_ops(lib):
    """Sizes of 0 are an empty input: OK with no work, NULL allowed for the
    zero-byte arrays (no call here reaches a kernel launch)."""
    assert lib.ssd_prep(None, None, None, 0, 2, 100, 64, None, None, None, None) == 0
    assert lib.ssd_prep(None, None, None, 1, 2, 0, 64, None, None, None, None) == 0
    assert lib.ssd_prep(None, None, None, 1, 2, 0, 48, None, None, None, None) == 3  # still validated
    assert lib.ssd_prep_amask(None, None, 1, 0, 10, 128, None, None, None, None) == 0
    for order in (1, 2):
        assert lib.ssd_forward(None, None, None, None, None, None, None, 1, 2, 0, 64, order, 64, 1,
                               None, None, None, None, None, 0, None) == 0
        assert lib.ssd_forward(None, None, None, None, None, None, None, 0, 2, 10, 64, order, 64, 1,
                               None, None, None, None, None, 0, None) == 0
    assert lib.ssd_forward(None, None, None, None, None, None, None, 1, 2, 0, 48, 1, 64, 1,
                           None, None, None, None, None, 0, None) == 3
    assert lib.ssd_decode_step(None, None, None, None, None, None, 0, 4, 64, 2, 1, 0,
                               None, None, None, None) == 0
    assert lib.ssd_decode_step_amask(None, None, None, None, None, 3, 0, 64, 2, 1, 1,
                                     None, None, None, None) == 0


def bwd(lib, *, order=1, d_h=64, dt=A[3], ddt=A[12], dq=A[9], ws=A[15], wsb=1 << 40, N=100):
    return lib.ssd_backward(A[0], A[1], A[2], dt, A[4], A[5], A[6], A[7], 1, 2, N, d_h, order, 64, 1,
                            dq, A[10], A[11], ddt, A[13], ws, wsb, None)


def test_backward_errors(lib):
    assert bwd(lib, order=2, d_h=32) == 3               # order 2: d_h 64 only
    assert bwd(lib, order=3) == 3
    assert bwd(lib, d_h=48) == 3
    assert bwd(lib, dq=None) == 1
    assert bwd(lib, ddt=None) == 1                      # dt given without ddt
    assert bwd(lib, dt=None) == 1                       # ddt given without dt
    assert bwd(lib, ws=None, wsb=0) == 6
    assert bwd(lib, wsb=16) == 6
    assert bwd(lib, dq=A[9] + 4) == 4
    assert bwd(lib, dq=A[0]) == 5                       # dq over q
    assert bwd(lib, N=0) == 0                           # empty: nothing to do
    need = lib.ssd_backward_workspace_size(1, 2, 100, 64, 1, 64, 1)
    assert need >= 4 * 2 * 2 * (64 * 64 + 64)
    assert lib.ssd_backward_workspace_size(1, 2, 100, 64, 2, 64, 1) >= 4 * 2 * 2 * (64 ** 3 + 64 ** 2)
    assert lib.ssd_backward_workspace_size(1, 2, 100, 64, 2, 64, 0) == 0  # order 2 needs bf16


def test_prep_backward_errors(lib):
    assert lib.ssd_prep_backward(A[0], None, A[2], A[3], A[4], 1, 2, 10, A[5], A[6], A[7], None) == 1
    assert lib.ssd_prep_backward(A[0], A[1], A[2], A[3], A[4], -1, 2, 10, A[5], A[6], A[7], None) == 2
    assert lib.ssd_prep_backward(A[0], A[1], A[2], A[3], A[4], 1, 2, 10, A[0], A[6], A[7], None) == 5
    assert lib.ssd_prep_amask_backward(A[0], A[1], A[2], None, 1, 2, 10, A[5], A[6], None) == 1
    assert lib.ssd_prep_amask_backward(None, None, A[2], None, 1, 2, 10, A[5], None, None) == 1
    assert lib.ssd_prep_amask_backward(A[0], None, A[2], None, 1, 2, 10, A[2], None, None) == 5
    assert lib.ssd_prep_amask_backward(None, None, None, None, 1, 2, 0, None, None, None) == 0
