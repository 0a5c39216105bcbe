"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Every test runs the library on seeded inputs and compares element by element
with the oracle on the same stored values, using the row-scaled metric of
tests/parity.py (tol 1e-4 for fp32 inputs, 2e-2 for bf16 inputs).  Small
cases check every row; the full-size workloads are run in the launch
configuration the benchmark times and checked on sampled rows (first and last
block, block boundaries +-1, random rows), which the oracle evaluates one by
one.
"""
import dataclasses

import numpy as np
import pytest

from mamba_ssd_sequence_amd import inputs as I
from oracle import ssd_oracle as O
from parity import TOL, row_error, sample_rows, to_dev_f32, to_dev_qkv, worst

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_sequence_amd import ssd
    ssd.lib()


# the workloads, plus order 1 with bf16 inputs at d_h 32 (two 16-column
# slices per head in the order-1 scan)
TEST_CONFIGS = {**I.ALL_CONFIGS,
                "o1_bf16_d32": dataclasses.replace(I.CONFIGS["o1_bf16_2k"], name="o1_bf16_d32", d_h=32)}


def ssd_mod():
    from mamba_ssd_sequence_amd import ssd
    return ssd


def say(*a):
    print(*a, flush=True)


def run_forward(inp, order, chunk, *, with_dt=True, want_den=False, want_final=False):
    ssd = ssd_mod()
    c = inp.cfg
    q, k, v = (to_dev_qkv(x, c.dtype) for x in (inp.q, inp.k, inp.v))
    dtp, bias, alog = to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log)
    dt, a_cs, a_chunk = ssd.prep(dtp, bias, alog, chunk)
    B, H, N, d = q.shape
    D = d ** order
    den = torch.empty((B, H, N), device="cuda") if want_den else None
    fs = torch.empty((B, H, D, d), device="cuda") if want_final else None
    fn = torch.empty((B, H, D), device="cuda") if want_final else None
    y = ssd.forward(q, k, v, dt if with_dt else None, a_cs, order, chunk, den=den,
                    final_state=fs, final_norm=fn)
    torch.cuda.synchronize()
    out = {"y": y.cpu().numpy(), "dt": dt.cpu().numpy(), "a_cs": a_cs.cpu().numpy(),
           "a_chunk": a_chunk.cpu().numpy()}
    if want_den:
        out["den"] = den.cpu().numpy()
    if want_final:
        out["fs"] = fs.cpu().numpy()
        out["fn"] = fn.cpu().numpy()
    return out


def oracle_forward(inp, order, rows=None, with_dt=True):
    q, k, v = inp.qkv_f64()
    if with_dt:
        return O.forward_ref(q, k, v, inp.dt_proj, inp.dt_bias, inp.A_log, order, rows=rows)
    _, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    return O.forward_quadratic(q, k, v, a, order, rows=rows)


# ---------------------------------------------------------------------------
# prep
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(I.CONFIGS))
def test_prep_full_size(name):
    cfg = I.CONFIGS[name]
    say("prep", name)
    inp = I.make_forward_inputs(cfg)
    ssd = ssd_mod()
    dt, a_cs, a_chunk = ssd.prep(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias),
                                 to_dev_f32(inp.A_log), cfg.chunk)
    torch.cuda.synchronize()
    dt_r, cs_r, tot_r = O.prep_ref(inp.dt_proj, inp.dt_bias, inp.A_log, cfg.chunk)
    np.testing.assert_allclose(dt.cpu().numpy(), dt_r, rtol=2e-6, atol=0)
    # a <= 0, so |chunk-local cumsum| is the running sum of |a|; an fp32 scan of
    # at most 128 terms is accurate to a small multiple of eps times that sum
    err = np.abs(a_cs.cpu().numpy() - cs_r)
    bound = 1e-5 * np.abs(cs_r) + 1e-6
    assert np.all(err <= bound), float((err / bound).max())
    np.testing.assert_allclose(a_chunk.cpu().numpy(), tot_r, rtol=2e-6, atol=1e-6)


# ---------------------------------------------------------------------------
# forward: small shapes, every row, ragged tails
# ---------------------------------------------------------------------------

SMALL = [
    # (config to draw from, order, d_h override via config, N, chunk)
    ("o1_f32_small", 1, 1, 2, 1, 64), ("o1_f32_small", 1, 1, 2, 63, 64), ("o1_f32_small", 1, 1, 2, 65, 128),
    ("o1_f32_small", 1, 2, 1, 200, 64), ("o1_f32_small", 1, 1, 1, 300, 128),
    ("o1_bf16_2k", 1, 1, 2, 1, 64), ("o1_bf16_2k", 1, 1, 2, 129, 64), ("o1_bf16_2k", 1, 2, 2, 333, 128),
    # order 1, bf16: d_h 32; sequences cut into 2 and 3 segments (a ragged last
    # block, chunk 64 and 128)
    ("o1_bf16_d32", 1, 1, 2, 129, 64), ("o1_bf16_d32", 1, 2, 1, 1100, 128), ("o1_bf16_2k", 1, 1, 3, 1500, 64),
    ("o2_bf16_4k", 2, 1, 1, 1, 64), ("o2_bf16_4k", 2, 1, 2, 64, 64), ("o2_bf16_4k", 2, 1, 2, 65, 64),
    ("o2_bf16_4k", 2, 2, 1, 257, 128), ("o2_bf16_4k", 2, 1, 3, 700, 64),
    # 32 heads: the state scan's one-wave-per-column layout and head-to-XCD
    # mapping (5 blocks: the last step has an empty second block; 3 blocks of a
    # chunk of 128)
    ("o2_bf16_4k", 2, 2, 16, 300, 64), ("o2_bf16_4k", 2, 4, 8, 130, 128),
]


@pytest.mark.parametrize("name,order,B,H,N,chunk", SMALL)
def test_forward_small(name, order, B, H, N, chunk):
    say("forward small", name, order, B, H, N, chunk)
    cfg = TEST_CONFIGS[name]
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=N + 7 * H)
    got = run_forward(inp, order, chunk, want_den=True)
    ref = oracle_forward(inp, order)
    err = row_error(got["y"], ref["y"], ref["scale"])
    say("  err", err)
    assert err <= TOL[cfg.dtype]
    den_err = np.abs(got["den"] - ref["den"]) / (ref["kappa"] * np.abs(ref["den"]))
    assert float(den_err.max()) <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["o1_bf16_2k", "o2_bf16_4k"])
def test_forward_plain_value_operand(name):
    """dt = NULL: v itself is the value operand (Algorithm 5 as printed)."""
    cfg = I.CONFIGS[name]
    inp = I.make_forward_inputs(cfg, B=1, H=2, N=190, seed=3)
    got = run_forward(inp, cfg.order, 64, with_dt=False)
    ref = oracle_forward(inp, cfg.order, with_dt=False)
    assert row_error(got["y"], ref["y"], ref["scale"]) <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["o1_f32_small", "o1_bf16_2k", "o2_bf16_4k"])
def test_chunk_size_invariance(name):
    cfg = I.CONFIGS[name]
    inp = I.make_forward_inputs(cfg, B=1, H=2, N=640, seed=5)
    a = run_forward(inp, cfg.order, 64)
    b = run_forward(inp, cfg.order, 128)
    ref = oracle_forward(inp, cfg.order)
    assert row_error(a["y"], ref["y"], ref["scale"]) <= TOL[cfg.dtype]
    assert row_error(b["y"], ref["y"], ref["scale"]) <= TOL[cfg.dtype]


# (B, H, N): at order 2, 2 heads use the two-wave-per-column state layout and
# 32 heads the one-wave layout; N = 300 ends on a step with one block
@pytest.mark.parametrize("name,B,H,N", [("o1_f32_small", 1, 2, 200), ("o1_bf16_2k", 1, 2, 200),
                                        ("o1_bf16_2k", 1, 2, 1500), ("o1_bf16_d32", 2, 1, 1300),
                                        ("o2_bf16_4k", 1, 2, 200), ("o2_bf16_4k", 2, 16, 300)])
def test_final_state_matches_recurrence(name, B, H, N):
    cfg = TEST_CONFIGS[name]
    say("final state", name, B, H, N)
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=11)
    got = run_forward(inp, cfg.order, cfg.chunk, want_final=True)
    q, k, v = inp.qkv_f64()
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    _, _, S, z = O.forward_recurrent(q, k, v * dt[..., None], a, cfg.order)
    tol = TOL[cfg.dtype]
    assert np.abs(got["fs"] - S).max() <= tol * np.abs(S).max()
    assert np.abs(got["fn"] - z).max() <= tol * np.abs(z).max()


def _forward_arrays(cfg, q, k, v, dtp, bias, alog, order, chunk, S0=None, z0=None):
    """GPU forward over given (sliced) stored inputs; returns y, final S and z."""
    ssd = ssd_mod()
    qd, kd, vd = (to_dev_qkv(np.ascontiguousarray(x), cfg.dtype) for x in (q, k, v))
    dt, a_cs, _ = ssd.prep(to_dev_f32(dtp), to_dev_f32(bias), to_dev_f32(alog), chunk)
    B, H, N, d = qd.shape
    D = d ** order
    fs = torch.empty((B, H, D, d), device="cuda")
    fn = torch.empty((B, H, D), device="cuda")
    y = ssd.forward(qd, kd, vd, dt, a_cs, order, chunk, final_state=fs, final_norm=fn,
                    initial_state=None if S0 is None else to_dev_f32(S0),
                    initial_norm=None if z0 is None else to_dev_f32(z0))
    torch.cuda.synchronize()
    return y.cpu().numpy(), fs.cpu().numpy(), fn.cpu().numpy()


# (config, B, H, N, chunk, split point): at order 2, 2 heads use the
# two-wave-per-column state layout and 32 heads the one-wave layout; the
# initial state enters in the first step of the suffix (a single step of
# 70 tokens, or 14 steps); order 1 with bf16 inputs: suffixes of 8 segments
# (the scan sums the earlier segments and the initial state itself) and of
# 10 segments (the prefix pass carries the initial state)
@pytest.mark.parametrize("name,B,H,N,chunk,n1", [
    ("o1_f32_small", 1, 2, 200, 64, 100), ("o1_bf16_2k", 1, 2, 300, 128, 191),
    ("o1_bf16_2k", 1, 2, 3000, 128, 1000), ("o1_bf16_2k", 1, 2, 4000, 64, 1500),
    ("o1_bf16_d32", 1, 1, 2300, 64, 700),
    ("o2_bf16_4k", 1, 2, 300, 64, 128), ("o2_bf16_4k", 1, 2, 250, 128, 77),
    ("o2_bf16_4k", 2, 16, 300, 64, 150), ("o2_bf16_4k", 2, 16, 400, 64, 330),
    ("o2_bf16_4k", 1, 2, 2000, 64, 300)])
def test_initial_state_continues_the_sequence(name, B, H, N, chunk, n1):
    """ssd_forward from the states a prefix leaves (Algorithm 6 hand-off) gives
    the full sequence's outputs for the suffix and its final states (order 1
    with bf16 inputs: prefix and suffix are cut into segments)."""
    cfg = TEST_CONFIGS[name]
    say("initial state", name, B, H, N, chunk, n1)
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=5 + n1)
    order = cfg.order
    pre = lambda x: x[:, :, :n1]
    suf = lambda x: x[:, :, n1:]
    _, S1, z1 = _forward_arrays(cfg, pre(inp.q), pre(inp.k), pre(inp.v), pre(inp.dt_proj),
                                inp.dt_bias, inp.A_log, order, chunk)
    y2, S2, z2 = _forward_arrays(cfg, suf(inp.q), suf(inp.k), suf(inp.v), suf(inp.dt_proj),
                                 inp.dt_bias, inp.A_log, order, chunk, S0=S1, z0=z1)
    ref = oracle_forward(inp, order)
    err = row_error(y2, ref["y"][:, :, n1:], ref["scale"][:, :, n1:])
    say("  err", err)
    assert err <= TOL[cfg.dtype]
    qf, kf, vf = inp.qkv_f64()
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    _, _, S, z = O.forward_recurrent(qf, kf, vf * dt[..., None], a, order)
    tol = TOL[cfg.dtype]
    assert np.abs(S2 - S).max() <= tol * np.abs(S).max()
    assert np.abs(z2 - z).max() <= tol * np.abs(z).max()


def test_deterministic():
    cfg = I.CONFIGS["o2_bf16_4k"]
    inp = I.make_forward_inputs(cfg, B=1, H=2, N=300, seed=2)
    a = run_forward(inp, 2, 64)["y"]
    b = run_forward(inp, 2, 64)["y"]
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name,order", [("o1_bf16_2k", 1), ("o2_bf16_4k", 2)])
def test_graph_capture_replays_match_eager(name, order):
    """ssd_prep + ssd_forward captured in a HIP graph (no memset nodes: the
    library launches kernels only) and replayed several times, with other
    eager work and synchronisations between the replays: every replay
    reproduces the eager result bit for bit."""
    ssd = ssd_mod()
    cfg = I.CONFIGS[name]
    say("graph capture", name)
    inp = I.make_forward_inputs(cfg, B=1, H=4, N=333, seed=12)
    other = I.make_forward_inputs(cfg, B=1, H=4, N=333, seed=13)
    dev = [to_dev_qkv(x, cfg.dtype) for x in (inp.q, inp.k, inp.v)] + \
          [to_dev_f32(x) for x in (inp.dt_proj, inp.dt_bias, inp.A_log)]
    odev = [to_dev_qkv(x, cfg.dtype) for x in (other.q, other.k, other.v)] + \
           [to_dev_f32(x) for x in (other.dt_proj, other.dt_bias, other.A_log)]
    B, H, N, d = dev[0].shape
    ws = torch.empty(ssd.workspace_size(B, H, N, d, order, cfg.chunk, 1 if cfg.dtype == I.BF16 else 0),
                     dtype=torch.uint8, device="cuda")
    dt, a_cs, a_chunk = (torch.empty((B, H, n), device="cuda") for n in (N, N, -(-N // cfg.chunk)))
    y = torch.empty((B, H, N, d), device="cuda")

    def step(t, out):
        ssd.prep(t[3], t[4], t[5], cfg.chunk, out=(dt, a_cs, a_chunk))
        ssd.forward(t[0], t[1], t[2], dt, a_cs, order, cfg.chunk, y=out, workspace=ws)

    step(dev, y)
    torch.cuda.synchronize()
    want = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(dev, y)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(dev, y)
    y_other = torch.empty_like(y)
    for rep in range(3):
        y.zero_()
        step(odev, y_other)  # eager work on other inputs in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), rep


# ---------------------------------------------------------------------------
# forward: the full-size workloads, sampled rows
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["o1_f32_small", "o1_bf16_2k", "o2_bf16_4k", "o1_bf16_4k", "o1_bf16_d32"])
def test_forward_full_size_all_rows(name):
    """The workloads up to N = 4096 at full size, in the benchmark's launch,
    against the oracle on every row of every head (and order 1 at d_h 32 at
    the 2K shape)."""
    cfg = TEST_CONFIGS[name]
    say("forward full, all rows", name)
    inp = I.make_forward_inputs(cfg)
    got = run_forward(inp, cfg.order, cfg.chunk, want_den=True)
    ref = oracle_forward(inp, cfg.order)
    err = row_error(got["y"], ref["y"], ref["scale"])
    say("  ", name, worst(got["y"], ref["y"], ref["scale"]))
    assert err <= TOL[cfg.dtype]
    den_err = np.abs(got["den"] - ref["den"]) / (ref["kappa"] * np.abs(ref["den"]))
    say("   normaliser: max err", float(den_err.max()))
    assert float(den_err.max()) <= TOL[cfg.dtype]


@pytest.mark.parametrize("name", ["o2_bf16_64k", "o1_bf16_64k"])
def test_forward_full_size_64k(name):
    """The 64K workloads at full size (512 chunks of 128), in the benchmark's
    launch.  Two heads densely: the first and last chunk, every 64-token
    block boundary +-1 over all 65536 tokens, 1024 random rows, and the
    final states against the oracle's unrolled recurrence; every other head
    on its first and last chunk and 256 random rows."""
    cfg = I.ALL_CONFIGS[name]
    say("forward full 64K", name)
    inp = I.make_forward_inputs(cfg)
    got = run_forward(inp, cfg.order, cfg.chunk, want_den=True, want_final=True)
    q, k, v = inp.qkv_f64()
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    vop = v * dt[..., None]
    rng = np.random.default_rng(99)
    dense_heads = (3, 12)
    tol = TOL[cfg.dtype]
    for h in range(cfg.H):
        dense = h in dense_heads
        rows = sample_rows(cfg.N, 1024 if dense else 256, rng, block=cfg.chunk, boundaries=dense)
        if dense:
            # block boundaries of the 64-token blocks too (the kernels' unit)
            rows = np.union1d(rows, sample_rows(cfg.N, 0, rng, block=64))
        sl = (slice(0, 1), slice(h, h + 1))
        ref = O.forward_quadratic(q[sl], k[sl], vop[sl], a[sl], cfg.order, rows=rows)
        y = got["y"][sl][:, :, rows]
        err = row_error(y, ref["y"], ref["scale"])
        say(f"   head {h}: {len(rows)} rows, {worst(y, ref['y'], ref['scale'], rows)}")
        assert err <= tol, h
        den_err = np.abs(got["den"][sl][:, :, rows] - ref["den"]) / (ref["kappa"] * np.abs(ref["den"]))
        assert float(den_err.max()) <= tol, h
        if dense:
            S, z = O.final_state_closed_form(k[sl], vop[sl], a[sl], cfg.order)
            fs_err = np.abs(got["fs"][sl] - S).max() / np.abs(S).max()
            fn_err = np.abs(got["fn"][sl] - z).max() / np.abs(z).max()
            say(f"   head {h}: final state err {fs_err:.3e}, final norm err {fn_err:.3e}")
            assert fs_err <= tol and fn_err <= tol, h
    assert np.all(np.isfinite(got["y"]))


@pytest.mark.parametrize("name", ["o2_bf16_64k", "o1_bf16_64k"])
def test_forward_offsets_past_2e31_elements(name):
    """Tensors of more than 2^31 elements: 17 distinct heads of the 64K
    workload, tiled 32 times over H = 544 (q, k, v, y: 2.28e9 elements each;
    heads 512 and up start past element 2^31 of y, and the order-2 workspace
    spans 32 GB).  Every copy of a head must reproduce its source head (the
    copy at the lowest offset) bit for bit in y, den and the final states,
    which an index that wrapped at 32 bits anywhere would break; two source
    heads are checked against the oracle on sampled rows (at 544 heads the
    order-2 state scan runs its one-wave-per-column layout on 64K tokens)."""
    ssd = ssd_mod()
    cfg = I.ALL_CONFIGS[name]
    HS, REP = 17, 32
    H = HS * REP
    say("offsets past 2^31", name, "H", H)
    src = I.make_forward_inputs(cfg, H=HS)
    assert H * cfg.N * cfg.d_h > 2 ** 31
    q, k, v = (to_dev_qkv(x, cfg.dtype).repeat(1, REP, 1, 1) for x in (src.q, src.k, src.v))
    dtp = to_dev_f32(src.dt_proj).repeat(1, REP, 1)
    bias, alog = to_dev_f32(src.dt_bias).repeat(REP), to_dev_f32(src.A_log).repeat(REP)
    dt, a_cs, _ = ssd.prep(dtp, bias, alog, cfg.chunk)
    D = cfg.d_h ** cfg.order
    den = torch.empty((1, H, cfg.N), device="cuda")
    fs = torch.empty((1, H, D, cfg.d_h), device="cuda")
    fn = torch.empty((1, H, D), device="cuda")
    say("   forward")
    y = ssd.forward(q, k, v, dt, a_cs, cfg.order, cfg.chunk, den=den, final_state=fs, final_norm=fn)
    torch.cuda.synchronize()
    del q, k, v, dtp, dt, a_cs
    say("   copies against their sources")
    for t, nm in ((y, "y"), (den, "den"), (fs, "final_state"), (fn, "final_norm")):
        base = t[:, :HS]
        for r in range(1, REP):
            assert torch.equal(t[:, r * HS:(r + 1) * HS], base), (nm, r)
    assert bool(torch.isfinite(y[:, :HS]).all())
    qs, ks, vs = src.qkv_f64()
    dts, a = O.discretise(src.dt_proj, src.dt_bias, src.A_log)
    vop = vs * dts[..., None]
    rng = np.random.default_rng(7)
    for h in (2, 13):
        rows = sample_rows(cfg.N, 256, rng, block=cfg.chunk, boundaries=False)
        sl = (slice(0, 1), slice(h, h + 1))
        ref = O.forward_quadratic(qs[sl], ks[sl], vop[sl], a[sl], cfg.order, rows=rows)
        got = y[:, h:h + 1, rows].cpu().numpy()
        err = row_error(got, ref["y"], ref["scale"])
        say(f"   head {h} (and its copies up to head {h + (REP - 1) * HS}): {len(rows)} rows, "
            f"{worst(got, ref['y'], ref['scale'], rows)}")
        assert err <= TOL[cfg.dtype], h
    del y, den, fs, fn
    torch.cuda.empty_cache()


# (B, H, decay per token): H = 3 runs the order-2 state scan's
# two-wave-per-column layout and B*H = 32 the one-wave layout; at 0.1 per
# token the 640 tail tokens decay the state by e^-64 (its scale exponent
# passes 64)
@pytest.mark.parametrize("B,H,decay", [(1, 3, 0.05), (2, 16, 0.05), (1, 3, 0.1)])
def test_zero_tail(B, H, decay):
    """A padded tail: from token 384 on, head h has zero keys (h % 3 == 0),
    zero values (h % 3 == 1) or both (h % 3 == 2).  Such blocks add nothing
    to the states (Algorithm 6), which keep decaying; the tail's outputs are
    the decayed earlier tokens' weighted mean (Algorithm 5's weights).  The
    outputs and final states match the oracle, and are finite."""
    cfg = I.CONFIGS["o2_bf16_4k"]
    say("zero tail", B, H, decay)
    N, t0 = 1024, 384
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=41)
    inp.A_log[:] = 0.0                                   # A = -1
    inp.dt_proj[:] = 0.0
    inp.dt_bias[:] = np.log(np.expm1(decay))             # dt = decay, a = -decay
    for h in range(H):
        if h % 3 in (0, 2):
            inp.k[:, h, t0:] = 0
        if h % 3 in (1, 2):
            inp.v[:, h, t0:] = 0
    got = run_forward(inp, 2, cfg.chunk, want_den=True, want_final=True)
    assert np.all(np.isfinite(got["y"])) and np.all(np.isfinite(got["fs"]))
    ref = oracle_forward(inp, 2)
    err = row_error(got["y"], ref["y"], ref["scale"])
    say("  ", worst(got["y"], ref["y"], ref["scale"]))
    assert err <= TOL[cfg.dtype]
    q, k, v = inp.qkv_f64()
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    S, z = O.final_state_closed_form(k, v * dt[..., None], a, 2)
    for b in range(B):
        for h in range(H):
            fs_err = np.abs(got["fs"][b, h] - S[b, h]).max() / np.abs(S[b, h]).max()
            fn_err = np.abs(got["fn"][b, h] - z[b, h]).max() / np.abs(z[b, h]).max()
            assert fs_err <= TOL[cfg.dtype] and fn_err <= TOL[cfg.dtype], (b, h, fs_err, fn_err)


# ---------------------------------------------------------------------------
# the A-mask of Algorithms 4 and 5 (ssd_prep_amask + the same forward)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", list(I.CONFIGS))
@pytest.mark.parametrize("with_dt", [True, False])
def test_prep_amask_full_size(name, with_dt):
    cfg = I.CONFIGS[name]
    say("prep amask", name, with_dt)
    inp = I.make_forward_inputs(cfg)
    ssd = ssd_mod()
    dtp = inp.dt_proj if with_dt else None
    dt, a_cs, a_chunk = ssd.prep_amask(to_dev_f32(inp.A_proj), to_dev_f32(dtp) if with_dt else None,
                                       cfg.chunk)
    torch.cuda.synchronize()
    dt_r, cs_r, tot_r = O.prep_amask_ref(inp.A_proj, dtp, cfg.chunk)
    if with_dt:
        np.testing.assert_allclose(dt.cpu().numpy(), dt_r, rtol=2e-6, atol=0)
    else:
        assert dt is None
    err = np.abs(a_cs.cpu().numpy() - cs_r)  # a < 0: as in test_prep_full_size
    bound = 1e-5 * np.abs(cs_r) + 1e-6
    assert np.all(err <= bound), float((err / bound).max())
    np.testing.assert_allclose(a_chunk.cpu().numpy(), tot_r, rtol=2e-6, atol=1e-6)


def run_forward_amask(inp, order, chunk, with_dt):
    ssd = ssd_mod()
    q, k, v = (to_dev_qkv(x, inp.cfg.dtype) for x in (inp.q, inp.k, inp.v))
    dt, a_cs, _ = ssd.prep_amask(to_dev_f32(inp.A_proj), to_dev_f32(inp.dt_proj) if with_dt else None,
                                 chunk)
    B, H, N, d = q.shape
    den = torch.empty((B, H, N), device="cuda")
    y = ssd.forward(q, k, v, dt, a_cs, order, chunk, den=den)
    torch.cuda.synchronize()
    return y.cpu().numpy(), den.cpu().numpy()


# (config, order, B, H, N, chunk, value operand V*dt (Algorithm 4) or plain V (Algorithm 5))
AMASK = [
    ("o1_f32_small", 1, 1, 2, 200, 64, True), ("o1_bf16_2k", 1, 2, 2, 333, 128, True),
    ("o1_bf16_2k", 1, 1, 2, 130, 64, False),
    # order 1, bf16: sequences cut into segments (the A-mask's decays through the segment pass)
    ("o1_bf16_2k", 1, 1, 2, 1500, 64, True), ("o1_bf16_d32", 1, 1, 1, 1100, 128, False),
    ("o2_bf16_4k", 2, 1, 2, 257, 64, False), ("o2_bf16_4k", 2, 2, 16, 300, 64, False),
    ("o2_bf16_4k", 2, 1, 3, 200, 128, True),
]


@pytest.mark.parametrize("name,order,B,H,N,chunk,with_dt", AMASK)
def test_forward_amask_small(name, order, B, H, N, chunk, with_dt):
    say("forward amask", name, order, B, H, N, chunk, with_dt)
    cfg = TEST_CONFIGS[name]
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=3 * N + H)
    y, den = run_forward_amask(inp, order, chunk, with_dt)
    q, k, v = inp.qkv_f64()
    ref = O.forward_amask_ref(q, k, v, inp.A_proj, inp.dt_proj if with_dt else None, order)
    err = row_error(y, ref["y"], ref["scale"])
    say("  err", err)
    assert err <= TOL[cfg.dtype]
    den_err = np.abs(den - ref["den"]) / (ref["kappa"] * np.abs(ref["den"]))
    assert float(den_err.max()) <= TOL[cfg.dtype]


def test_forward_amask_full_size_2mamba():
    # Algorithm 5 at the order-2 4K workload: plain V, sampled rows
    cfg = I.CONFIGS["o2_bf16_4k"]
    say("forward amask full o2_bf16_4k")
    inp = I.make_forward_inputs(cfg)
    y, _ = run_forward_amask(inp, 2, cfg.chunk, False)
    rows = sample_rows(cfg.N, 48, np.random.default_rng(5))
    q, k, v = inp.qkv_f64()
    ref = O.forward_amask_ref(q, k, v, inp.A_proj, None, 2, rows=rows)
    err = row_error(y[:, :, rows], ref["y"], ref["scale"])
    say("  err", err)
    assert err <= TOL[cfg.dtype]


# ---------------------------------------------------------------------------
# decode: the step evaluates Algorithm 6's state form (phi(q)^T S / phi(q)^T z),
# so its outputs are measured with the state form's error scale
# (scale_state: sums over the feature products q_a.. k_a..)
# ---------------------------------------------------------------------------

def run_decode_steps(dec, order, steps, S=None, check_heads=None):
    """Run `steps` decode steps on the GPU from a zero state; returns per-step
    y (all, or only check_heads rows) and the final state/norm of check_heads."""
    ssd = ssd_mod()
    c = dec.cfg
    S = c.S if S is None else S
    D = c.d_h ** order
    state = torch.zeros((S, c.H, D, c.d_h), device="cuda")
    norm = torch.zeros((S, c.H, D), device="cuda")
    bias, alog = to_dev_f32(dec.dt_bias), to_dev_f32(dec.A_log)
    ys, ins = [], []
    for (q, k, v, dtp) in dec.steps(steps, S=S):
        y = ssd.decode_step(to_dev_qkv(q, c.dtype), to_dev_qkv(k, c.dtype), to_dev_qkv(v, c.dtype),
                            to_dev_f32(dtp), bias, alog, state, norm, order)
        if check_heads is None:
            ys.append(y.cpu().numpy())
            ins.append((q, k, v, dtp))
        else:
            s_idx, h_idx = check_heads
            ys.append(y[s_idx, h_idx].cpu().numpy())
            ins.append(tuple(x[s_idx, h_idx] for x in (q, k, v, dtp)))
    torch.cuda.synchronize()
    if check_heads is None:
        return ys, ins, state.cpu().numpy(), norm.cpu().numpy()
    s_idx, h_idx = check_heads
    return ys, ins, state[s_idx, h_idx].cpu().numpy(), norm[s_idx, h_idx].cpu().numpy()


def decode_reference(ins, dtype, A_log, dt_bias, order, h_idx=None):
    """The oracle over the decode steps (recurrence), plus the quadratic-form
    diagnostics for the row-scaled metric."""
    up = I.bf16_bits_to_f64 if dtype == I.BF16 else (lambda x: x.astype(np.float64))
    qs = np.stack([up(x[0]) for x in ins], axis=-2)  # [S,H,T,d] or [M,T,d]
    ks = np.stack([up(x[1]) for x in ins], axis=-2)
    vs = np.stack([up(x[2]) for x in ins], axis=-2)
    dtp = np.stack([x[3] for x in ins], axis=-1).astype(np.float64)
    if h_idx is not None:  # [M,T,...] rows of (s,h) pairs: treat as B=1, H=M with per-row params
        qs, ks, vs, dtp = qs[None], ks[None], vs[None], dtp[None]
        A_log, dt_bias = A_log[h_idx], dt_bias[h_idx]
    return O.forward_ref(qs, ks, vs, dtp, dt_bias, A_log, order)


@pytest.mark.parametrize("order,d_h,dtype", [(1, 32, I.F32), (1, 64, I.BF16), (2, 32, I.BF16),
                                             (2, 64, I.BF16), (2, 64, I.F32)])
def test_decode_small(order, d_h, dtype):
    say("decode small", order, d_h, dtype)
    cfg = I.DecodeConfig("t", S=3, H=2, d_h=d_h, order=order, steps=17, dtype=dtype, seed=order * 10 + d_h)
    dec = I.make_decode_inputs(cfg)
    ys, ins, st, nz = run_decode_steps(dec, order, cfg.steps)
    ref = decode_reference(ins, dtype, dec.A_log.astype(np.float64), dec.dt_bias.astype(np.float64), order)
    y = np.stack(ys, axis=2)  # [S,H,T,d]
    assert row_error(y, ref["y"], ref["scale_state"]) <= TOL[dtype]
    # final state against the token recurrence
    up = I.bf16_bits_to_f64 if dtype == I.BF16 else (lambda x: x.astype(np.float64))
    Sx = np.zeros((cfg.S, cfg.H, d_h ** order, d_h))
    zx = np.zeros((cfg.S, cfg.H, d_h ** order))
    for (q, k, v, dtp) in ins:
        _, Sx, zx, _ = O.decode_step_ref(Sx, zx, up(q), up(k), up(v), dtp, dec.dt_bias, dec.A_log, order)
    assert np.abs(st - Sx).max() <= 1e-5 * np.abs(Sx).max()
    assert np.abs(nz - zx).max() <= 1e-5 * np.abs(zx).max()


def decode_pairs(cfg, rng, n=128):
    """n distinct (sequence, head) pairs of the decode workload."""
    flat = rng.choice(cfg.S * cfg.H, size=n, replace=False)
    return flat // cfg.H, flat % cfg.H


def decode_final_state_ref(ins, dec, h_idx, dtype, order, amask=False, with_dt=True):
    """The states of the checked (sequence, head) pairs after the decode steps,
    from the oracle's unrolled recurrence (rows of pairs as B = 1, H = M)."""
    up = I.bf16_bits_to_f64 if dtype == I.BF16 else (lambda x: x.astype(np.float64))
    ks = np.stack([up(x[1]) for x in ins], axis=-2)[None]  # [1,M,T,d]
    vs = np.stack([up(x[2]) for x in ins], axis=-2)[None]
    dtp = np.stack([x[3] for x in ins], axis=-1).astype(np.float64)[None]
    if amask:
        A_P = np.stack([x[4] for x in ins], axis=-1).astype(np.float64)[None]
        dt, a = O.discretise_amask(A_P, dtp if with_dt else None)
    else:
        dt, a = O.discretise(dtp, dec.dt_bias.astype(np.float64)[h_idx], dec.A_log.astype(np.float64)[h_idx])
    vop = vs if dt is None else vs * dt[..., None]
    S, z = O.final_state_closed_form(ks, vop, a, order)
    return S[0], z[0]


def test_decode_full_size_sampled():
    """The order-2 decode workload (256 x 32 heads, 128 steps) run at full size;
    128 (sequence, head) pairs are checked at every step, and their states
    after the last step against the oracle's."""
    cfg = I.DECODE_CONFIGS["o2_decode"]
    say("decode full")
    dec = I.make_decode_inputs(cfg)
    s_idx, h_idx = decode_pairs(cfg, np.random.default_rng(5))
    ys, ins, st, nz = run_decode_steps(dec, cfg.order, cfg.steps, check_heads=(s_idx, h_idx))
    ref = decode_reference(ins, cfg.dtype, dec.A_log.astype(np.float64), dec.dt_bias.astype(np.float64),
                           cfg.order, h_idx=h_idx)
    y = np.stack(ys, axis=1)[None]  # [1,M,T,d]
    err = row_error(y, ref["y"], ref["scale_state"])
    say("  ", worst(y, ref["y"], ref["scale_state"]))
    assert err <= TOL[cfg.dtype]
    S, z = decode_final_state_ref(ins, dec, h_idx, cfg.dtype, cfg.order)
    fs_err = np.abs(st - S).max() / np.abs(S).max()
    fn_err = np.abs(nz - z).max() / np.abs(z).max()
    say(f"   final state err {fs_err:.3e}, final norm err {fn_err:.3e}")
    assert fs_err <= 1e-5 and fn_err <= 1e-5


@pytest.mark.parametrize("packed", [False, True])
def test_decode_offsets_past_2e31_elements(packed):
    """Order-2 decode states of more than 2^31 elements: 16 distinct
    sequences of 32 heads tiled 32 times (S = 512; 2.1e9 state entries in the
    packed layout, 4.3e9 in the full one, so every sequence from 256 on
    starts past element 2^31 of the full state).  Over 4 steps every copy
    must reproduce its source sequence bit for bit in y and both states, and
    one source sequence (all heads) is checked against the oracle."""
    ssd = ssd_mod()
    SS, REP, T = 16, 32, 4
    cfg = I.DecodeConfig("big", S=SS, H=32, d_h=64, order=2, steps=T, dtype=I.BF16, seed=5)
    say("decode offsets past 2^31, packed" if packed else "decode offsets past 2^31, full layout")
    dec = I.make_decode_inputs(cfg)
    D = cfg.d_h * (cfg.d_h + 1) // 2 if packed else cfg.d_h ** 2
    S = SS * REP
    assert S * cfg.H * D * cfg.d_h > 2 ** 31
    state = torch.zeros((S, cfg.H, D, cfg.d_h), device="cuda")
    norm = torch.zeros((S, cfg.H, D), device="cuda")
    bias, alog = to_dev_f32(dec.dt_bias), to_dev_f32(dec.A_log)
    ys, ins = [], []
    for (q, k, v, dtp) in dec.steps(T):
        y = ssd.decode_step(*(to_dev_qkv(x, cfg.dtype).repeat(REP, 1, 1) for x in (q, k, v)),
                            to_dev_f32(dtp).repeat(REP, 1), bias, alog, state, norm, 2, packed=packed)
        for r in range(1, REP):
            assert torch.equal(y[r * SS:(r + 1) * SS], y[:SS]), ("y", r)
        ys.append(y[:SS].cpu().numpy())
        ins.append((q, k, v, dtp))
    torch.cuda.synchronize()
    for t, nm in ((state, "state"), (norm, "norm")):
        for r in range(1, REP):
            assert torch.equal(t[r * SS:(r + 1) * SS], t[:SS]), (nm, r)
    del state, norm
    torch.cuda.empty_cache()
    s0 = 5
    ref = decode_reference([tuple(x[s0:s0 + 1] for x in st) for st in ins], cfg.dtype,
                           dec.A_log.astype(np.float64), dec.dt_bias.astype(np.float64), 2)
    y = np.stack([x[s0:s0 + 1] for x in ys], axis=2)  # [1,H,T,d]
    err = row_error(y, ref["y"], ref["scale_state"])
    say(f"   sequence {s0} (and its copies up to {s0 + (REP - 1) * SS}), all heads: max err {err:.3e}")
    assert err <= TOL[cfg.dtype]


def test_prefill_then_decode():
    """Forward over N tokens hands its final states to decode; continuing for T
    tokens equals the oracle over N + T tokens."""
    ssd = ssd_mod()
    cfg = I.CONFIGS["o2_bf16_4k"]
    N, T = 130, 6
    inp = I.make_forward_inputs(cfg, B=2, H=2, N=N + T, seed=21)
    pre = I.ForwardInputs(I.CONFIGS["o2_bf16_4k"], inp.q[:, :, :N], inp.k[:, :, :N], inp.v[:, :, :N],
                          inp.dt_proj[:, :, :N], inp.A_log, inp.dt_bias)
    got = run_forward(pre, 2, 64, want_final=True)
    state = torch.from_numpy(got["fs"]).cuda()
    norm = torch.from_numpy(got["fn"]).cuda()
    B, H = 2, 2
    bias, alog = to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log)
    ys = []
    for t in range(N, N + T):
        q, k, v = (to_dev_qkv(np.ascontiguousarray(x[:, :, t]), cfg.dtype) for x in (inp.q, inp.k, inp.v))
        y = ssd.decode_step(q, k, v, to_dev_f32(inp.dt_proj[:, :, t]), bias, alog, state, norm, 2)
        ys.append(y.cpu().numpy())
    ref = oracle_forward(inp, 2, rows=np.arange(N, N + T))
    y = np.stack(ys, axis=2)
    assert row_error(y, ref["y"], ref["scale_state"]) <= TOL[cfg.dtype]


# ---------------------------------------------------------------------------
# decode: the A-mask as Algorithm 6 prints it, and the packed order-2 layout
# ---------------------------------------------------------------------------

def run_decode_variant(dec, order, steps, *, amask, with_dt=True, packed=False, check_heads=None):
    """Decode `steps` steps from a zero state with the A-mask and/or the packed
    layout; returns per-step y, the step inputs, and the final states (all
    heads, or check_heads only)."""
    ssd = ssd_mod()
    c = dec.cfg
    d = c.d_h
    D = d if order == 1 else (d * (d + 1) // 2 if packed else d * d)
    state = torch.zeros((c.S, c.H, D, d), device="cuda")
    norm = torch.zeros((c.S, c.H, D), device="cuda")
    bias, alog = to_dev_f32(dec.dt_bias), to_dev_f32(dec.A_log)
    ys, ins = [], []
    for (q, k, v, dtp, A_P) in dec.steps(steps, with_A=True):
        qd, kd, vd = (to_dev_qkv(x, c.dtype) for x in (q, k, v))
        if amask:
            y = ssd.decode_step_amask(qd, kd, vd, to_dev_f32(A_P), to_dev_f32(dtp) if with_dt else None,
                                      state, norm, order, packed=packed)
        else:
            y = ssd.decode_step(qd, kd, vd, to_dev_f32(dtp), bias, alog, state, norm, order, packed=packed)
        if check_heads is None:
            ys.append(y.cpu().numpy())
            ins.append((q, k, v, dtp, A_P))
        else:
            s_idx, h_idx = check_heads
            ys.append(y[s_idx, h_idx].cpu().numpy())
            ins.append(tuple(x[s_idx, h_idx] for x in (q, k, v, dtp, A_P)))
    torch.cuda.synchronize()
    if check_heads is None:
        return ys, ins, state.cpu().numpy(), norm.cpu().numpy()
    s_idx, h_idx = check_heads
    return ys, ins, state[s_idx, h_idx].cpu().numpy(), norm[s_idx, h_idx].cpu().numpy()


def decode_variant_reference(ins, dtype, dec, order, *, amask, with_dt, h_idx=None, states=True):
    """The oracle for run_decode_variant: the quadratic form over the steps
    (outputs and their error scale) and (if `states`) the recurrence's final
    full states."""
    up = I.bf16_bits_to_f64 if dtype == I.BF16 else (lambda x: x.astype(np.float64))
    A_log, dt_bias = dec.A_log.astype(np.float64), dec.dt_bias.astype(np.float64)
    if h_idx is not None:
        A_log, dt_bias = A_log[h_idx], dt_bias[h_idx]
    S = z = None
    for (q, k, v, dtp, A_P) in (ins if states else ()):
        q, k, v = up(q), up(k), up(v)
        if S is None:
            D = q.shape[-1] ** order
            S = np.zeros(q.shape[:-1] + (D, q.shape[-1]))
            z = np.zeros(q.shape[:-1] + (D,))
        if amask:
            _, S, z, _ = O.decode_step_amask_ref(S, z, q, k, v, A_P, dtp if with_dt else None, order)
        elif h_idx is None:
            _, S, z, _ = O.decode_step_ref(S, z, q, k, v, dtp, dt_bias, A_log, order)
        else:  # per-row head parameters: rows of (s, h) pairs as S = 1, H = M
            _, S1, z1, _ = O.decode_step_ref(S[None], z[None], q[None], k[None], v[None], dtp[None],
                                             dt_bias, A_log, order)
            S, z = S1[0], z1[0]
    stack = lambda j: np.stack([up(x[j]) if j < 3 else x[j].astype(np.float64) for x in ins], axis=-2 if j < 3 else -1)
    qs, ks, vs, dtp, A_P = (stack(j) for j in range(5))
    if h_idx is not None:
        qs, ks, vs, dtp, A_P = (x[None] for x in (qs, ks, vs, dtp, A_P))
    if amask:
        ref = O.forward_amask_ref(qs, ks, vs, A_P, dtp if with_dt else None, order)
    else:
        ref = O.forward_ref(qs, ks, vs, dtp, dt_bias, A_log, order)
    return ref, S, z


# (order, d_h, dtype, A-mask, value operand v*dt, packed layout)
DECODE_VARIANTS = [
    (2, 64, I.BF16, False, True, True), (2, 32, I.BF16, False, True, True), (2, 64, I.F32, False, True, True),
    (2, 64, I.BF16, True, False, False), (2, 64, I.BF16, True, True, True), (2, 32, I.F32, True, False, True),
    (1, 64, I.BF16, True, True, False), (1, 32, I.F32, True, False, False),
]


@pytest.mark.parametrize("order,d_h,dtype,amask,with_dt,packed", DECODE_VARIANTS)
def test_decode_variants_small(order, d_h, dtype, amask, with_dt, packed):
    say("decode variant", order, d_h, dtype, "amask" if amask else "mamba2", with_dt, "packed" if packed else "full")
    cfg = I.DecodeConfig("t", S=3, H=2, d_h=d_h, order=order, steps=17, dtype=dtype, seed=70 + d_h + order)
    dec = I.make_decode_inputs(cfg)
    ys, ins, st, nz = run_decode_variant(dec, order, cfg.steps, amask=amask, with_dt=with_dt, packed=packed)
    ref, Sx, zx = decode_variant_reference(ins, dtype, dec, order, amask=amask, with_dt=with_dt)
    y = np.stack(ys, axis=2)  # [S,H,T,d]
    err = row_error(y, ref["y"], ref["scale_state"])
    say("  err", err)
    assert err <= TOL[dtype]
    if packed:
        Sx, zx = O.pack_state(Sx, zx, d_h)
    assert st.shape == Sx.shape and nz.shape == zx.shape
    assert np.abs(st - Sx).max() <= 1e-5 * np.abs(Sx).max()
    assert np.abs(nz - zx).max() <= 1e-5 * np.abs(zx).max()


def test_decode_packed_full_size_sampled():
    """The order-2 decode workload (256 x 32 heads, 128 steps) in the packed
    layout; 128 (sequence, head) pairs are checked at every step and at the end."""
    cfg = I.DECODE_CONFIGS["o2_decode"]
    say("decode packed full")
    dec = I.make_decode_inputs(cfg)
    s_idx, h_idx = decode_pairs(cfg, np.random.default_rng(6))
    ys, ins, st, nz = run_decode_variant(dec, 2, cfg.steps, amask=False, packed=True,
                                         check_heads=(s_idx, h_idx))
    ref = decode_variant_reference(ins, cfg.dtype, dec, 2, amask=False, with_dt=True, h_idx=h_idx,
                                   states=False)[0]
    y = np.stack(ys, axis=1)[None]  # [1,M,T,d]
    err = row_error(y, ref["y"], ref["scale_state"])
    say("  ", worst(y, ref["y"], ref["scale_state"]))
    assert err <= TOL[cfg.dtype]
    S, z = decode_final_state_ref(ins, dec, h_idx, cfg.dtype, 2)
    Sp, zp = O.pack_state(S, z, cfg.d_h)
    assert np.abs(st - Sp).max() <= 1e-5 * np.abs(Sp).max()
    assert np.abs(nz - zp).max() <= 1e-5 * np.abs(zp).max()


@pytest.mark.parametrize("d_h", [32, 64])
def test_state_pack_unpack(d_h):
    """Packing keeps the rows a <= b (bit-exact for symmetric states), unpacking
    restores the full layout; an asymmetric state packs to its symmetric part."""
    ssd = ssd_mod()
    say("state pack/unpack", d_h)
    rng = np.random.default_rng(60 + d_h)
    X = rng.standard_normal((2, 3, d_h, d_h, d_h)).astype(np.float32)
    sym = (X + X.transpose(0, 1, 3, 2, 4)) * np.float32(0.5)  # rows (a,b) and (b,a) identical
    S = np.ascontiguousarray(sym.reshape(2, 3, d_h * d_h, d_h))
    zm = rng.standard_normal((2, 3, d_h, d_h)).astype(np.float32)
    z = np.ascontiguousarray(((zm + zm.transpose(0, 1, 3, 2)) * np.float32(0.5)).reshape(2, 3, d_h * d_h))
    Sp, zp = ssd.state_pack(to_dev_f32(S), to_dev_f32(z))
    want_S, want_z = O.pack_state(S, z, d_h)
    np.testing.assert_array_equal(Sp.cpu().numpy(), want_S)
    np.testing.assert_array_equal(zp.cpu().numpy(), want_z)
    S2, z2 = ssd.state_unpack(Sp, zp)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(S2.cpu().numpy(), S)
    np.testing.assert_array_equal(z2.cpu().numpy(), z)
    # asymmetric: the mean of the two rows, within one rounding of the fp32 sum
    A = np.ascontiguousarray(X.reshape(2, 3, d_h * d_h, d_h))
    Az = np.ascontiguousarray(zm.reshape(2, 3, d_h * d_h))
    Ap, Azp = ssd.state_pack(to_dev_f32(A), to_dev_f32(Az))
    want_A, want_Az = O.pack_state(A, Az, d_h)
    assert np.all(np.abs(Ap.cpu().numpy() - want_A) <= 2.0 ** -24 * np.abs(want_A))
    assert np.all(np.abs(Azp.cpu().numpy() - want_Az) <= 2.0 ** -24 * np.abs(want_Az))


def test_prefill_then_decode_amask_packed():
    """2Mamba inference as Algorithm 6 prints it: an A-mask prefill (plain V)
    hands its final states, packed, to the A-mask decode step; continuing for T
    tokens equals the oracle over N + T tokens."""
    ssd = ssd_mod()
    cfg = I.CONFIGS["o2_bf16_4k"]
    N, T = 130, 6
    inp = I.make_forward_inputs(cfg, B=2, H=2, N=N + T, seed=23)
    say("prefill amask -> packed decode")
    q, k, v = (to_dev_qkv(np.ascontiguousarray(x[:, :, :N]), cfg.dtype) for x in (inp.q, inp.k, inp.v))
    _, a_cs, _ = ssd.prep_amask(to_dev_f32(np.ascontiguousarray(inp.A_proj[:, :, :N])), None, 64)
    D = 64 * 64
    fs = torch.empty((2, 2, D, 64), device="cuda")
    fn = torch.empty((2, 2, D), device="cuda")
    ssd.forward(q, k, v, None, a_cs, 2, 64, final_state=fs, final_norm=fn)
    state, norm = ssd.state_pack(fs, fn)
    ys = []
    for t in range(N, N + T):
        qt, kt, vt = (to_dev_qkv(np.ascontiguousarray(x[:, :, t]), cfg.dtype) for x in (inp.q, inp.k, inp.v))
        y = ssd.decode_step_amask(qt, kt, vt, to_dev_f32(np.ascontiguousarray(inp.A_proj[:, :, t])), None,
                                  state, norm, 2, packed=True)
        ys.append(y.cpu().numpy())
    qf, kf, vf = inp.qkv_f64()
    ref = O.forward_amask_ref(qf, kf, vf, inp.A_proj, None, 2, rows=np.arange(N, N + T))
    y = np.stack(ys, axis=2)
    err = row_error(y, ref["y"], ref["scale_state"])
    say("  err", err)
    assert err <= TOL[cfg.dtype]


# ---------------------------------------------------------------------------
# decode with Algorithm 6's window-2 convolution
# ---------------------------------------------------------------------------

# (order, d_h, dtype, A-mask decay (else Mamba-2), conv bias, SiLU, packed layout)
DECODE_CONV = [(2, 64, I.BF16, True, True, False, False), (2, 64, I.BF16, True, False, False, True),
               (2, 32, I.F32, False, True, True, False), (1, 64, I.BF16, True, True, True, False),
               (1, 32, I.F32, False, False, False, False)]


@pytest.mark.parametrize("order,d_h,dtype,amask,bias,act,packed", DECODE_CONV)
def test_decode_conv_small(order, d_h, dtype, amask, bias, act, packed):
    """T decode steps with the window-2 convolution from zero states and a
    zero conv state: each step's y against the oracle (the masked quadratic
    form over the convolved sequence, row-scaled metric), the final states
    against the oracle's steps, and the conv state, which must hold the last
    raw token bit for bit."""
    ssd = ssd_mod()
    say("decode conv", order, d_h, dtype, "amask" if amask else "mamba2", bias, act, packed)
    cfg = I.DecodeConfig("t", S=3, H=2, d_h=d_h, order=order, steps=13, dtype=dtype, seed=90 + d_h + order)
    dec = I.make_decode_inputs(cfg)
    rng = np.random.default_rng(91 + order)
    w = np.stack([rng.uniform(-0.5, 0.5, (3, cfg.H, d_h)), rng.uniform(0.5, 1.5, (3, cfg.H, d_h))],
                 axis=-1).astype(np.float32)
    b = rng.normal(0.0, 0.1, (3, cfg.H, d_h)).astype(np.float32) if bias else None
    D = d_h if order == 1 else (d_h * (d_h + 1) // 2 if packed else d_h * d_h)
    state = torch.zeros((cfg.S, cfg.H, D, d_h), device="cuda")
    norm = torch.zeros((cfg.S, cfg.H, D), device="cuda")
    tdt = torch.bfloat16 if dtype == I.BF16 else torch.float32
    cst = torch.zeros((cfg.S, 3, cfg.H, d_h), dtype=tdt, device="cuda")
    wd, bd = to_dev_f32(w), (to_dev_f32(b) if bias else None)
    bias_d, alog_d = to_dev_f32(dec.dt_bias), to_dev_f32(dec.A_log)
    up = I.bf16_bits_to_f64 if dtype == I.BF16 else (lambda x: x.astype(np.float64))
    Sx = np.zeros((cfg.S, cfg.H, d_h ** order, d_h))
    zx = np.zeros((cfg.S, cfg.H, d_h ** order))
    cx = np.zeros((cfg.S, 3, cfg.H, d_h))
    ys, conv = [], [[], [], []]
    act_s = "silu" if act else None
    for (q, k, v, dtp, A_P) in dec.steps(cfg.steps, with_A=True):
        qd, kd, vd = (to_dev_qkv(x, dtype) for x in (q, k, v))
        if amask:
            y = ssd.decode_step_conv(qd, kd, vd, wd, bd, cst, state, norm, order, A_proj=to_dev_f32(A_P),
                                     dt_proj=to_dev_f32(dtp), act=act, packed=packed)
            kw = dict(A_proj=A_P, dt_proj=dtp)
        else:
            y = ssd.decode_step_conv(qd, kd, vd, wd, bd, cst, state, norm, order, dt_proj=to_dev_f32(dtp),
                                     dt_bias=bias_d, A_log=alog_d, act=act, packed=packed)
            kw = dict(dt_proj=dtp, dt_bias=dec.dt_bias, A_log=dec.A_log)
        ys.append(y.cpu().numpy())
        for i, x in enumerate((q, k, v)):
            conv[i].append(O.conv_window2(up(x), cx[:, i], w[i], None if b is None else b[i], act_s))
        _, Sx, zx, cx, _ = O.decode_step_conv_ref(Sx, zx, cx, up(q), up(k), up(v), w, b, act_s, order, **kw)
    torch.cuda.synchronize()
    y = np.stack(ys, axis=2)  # [S,H,T,d]
    qc, kc, vc = (np.stack(c, axis=2) for c in conv)
    A_Ps = np.stack([s_[4] for s_ in dec.steps(cfg.steps, with_A=True)], axis=-1).astype(np.float64)
    dtps = np.stack([s_[3] for s_ in dec.steps(cfg.steps, with_A=True)], axis=-1).astype(np.float64)
    if amask:
        ref = O.forward_amask_ref(qc, kc, vc, A_Ps, dtps, order)
    else:
        ref = O.forward_ref(qc, kc, vc, dtps, dec.dt_bias, dec.A_log, order)
    err = row_error(y, ref["y"], ref["scale_state"])
    say("  ", worst(y, ref["y"], ref["scale_state"]))
    assert err <= TOL[dtype]
    st, nz = state.cpu().numpy(), norm.cpu().numpy()
    if packed:
        Sx, zx = O.pack_state(Sx, zx, d_h)
    assert np.abs(st - Sx).max() <= 1e-5 * np.abs(Sx).max()
    assert np.abs(nz - zx).max() <= 1e-5 * np.abs(zx).max()
    last = [x for x in dec.steps(cfg.steps, with_A=True)][-1]
    want = np.stack([np.ascontiguousarray(x) for x in last[:3]], axis=1)  # [S,3,H,d] stored values
    got_cs = cst.cpu()
    got_cs = (got_cs.view(torch.int16).numpy().view(np.uint16) if dtype == I.BF16 else got_cs.numpy())
    assert np.array_equal(got_cs, want.astype(got_cs.dtype) if dtype != I.BF16 else want)


# ---------------------------------------------------------------------------
# empty inputs and the method's degenerate cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", [1, 2])
def test_empty_segment(order):
    """N = 0: nothing to compute; the final states are the initial ones (or 0)."""
    say("empty segment", order)
    ssd = ssd_mod()
    B, H, d = 2, 3, 64
    D = d ** order
    q = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    dtp = torch.empty((B, H, 0), device="cuda")
    dt, a_cs, a_chunk = ssd.prep(dtp, torch.zeros(H, device="cuda"), torch.zeros(H, device="cuda"), 64)
    assert dt.shape == (B, H, 0) and a_chunk.shape == (B, H, 0)
    fs = torch.full((B, H, D, d), 7.0, device="cuda")
    fn = torch.full((B, H, D), 7.0, device="cuda")
    y = ssd.forward(q, q.clone(), q.clone(), dt, a_cs, order, 64, final_state=fs, final_norm=fn)
    torch.cuda.synchronize()
    assert y.shape == (B, H, 0, d)
    assert float(fs.abs().max()) == 0.0 and float(fn.abs().max()) == 0.0
    s0 = torch.randn((B, H, D, d), device="cuda")
    z0 = torch.rand((B, H, D), device="cuda")
    ssd.forward(q, q.clone(), q.clone(), dt, a_cs, order, 64, final_state=fs, final_norm=fn,
                initial_state=s0, initial_norm=z0)
    torch.cuda.synchronize()
    assert torch.equal(fs, s0) and torch.equal(fn, z0)


@pytest.mark.parametrize("name", ["o1_bf16_2k", "o2_bf16_4k"])
def test_no_decay_is_causal_linear_attention(name):
    """A -> 0 (A_log = -40): the decay mask is all ones and the mixer is plain
    causal (order-p) linear attention (Algorithm 1 with the causal mask)."""
    cfg = I.CONFIGS[name]
    say("no decay", name)
    inp = I.make_forward_inputs(cfg, B=1, H=4, N=260, seed=31)
    inp.A_log[:] = -40.0
    got = run_forward(inp, cfg.order, cfg.chunk)
    q, k, v = inp.qkv_f64()
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    assert np.abs(a).max() < 1e-15
    ref = O.forward_quadratic(q, k, v * dt[..., None], np.zeros_like(a), cfg.order)
    err = row_error(got["y"], ref["y"], ref["scale"])
    say("  err", err)
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("name,order,N", [("o2_bf16_4k", 2, 200), ("o1_bf16_2k", 1, 1500)])
def test_full_decay_keeps_only_the_token_itself(name, order, N):
    """A dt -> -inf: every earlier token is masked out and y_i = (v dt)_i (the
    diagonal score cancels; order 2: it is positive).  Checked element by
    element against the oracle (whose error scale is then 2 |(v dt)_ic|: a
    relative error per element).  Order 1 at N = 1500 runs through six
    segments: every state and segment aggregate decays to zero."""
    cfg = TEST_CONFIGS[name]
    say("full decay", name, order, N)
    inp = I.make_forward_inputs(cfg, B=1, H=2, N=N, seed=32)
    inp.A_log[:] = 6.0       # A = -403
    inp.dt_bias[:] = 5.0     # dt ~ 5: a ~ -2000 per token
    got = run_forward(inp, order, 64)
    q, k, v = inp.qkv_f64()
    dt, _ = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    ref = oracle_forward(inp, order)
    np.testing.assert_allclose(ref["y"], v * dt[..., None], rtol=1e-12, atol=0)
    err = row_error(got["y"], ref["y"], ref["scale"])
    say("  ", worst(got["y"], ref["y"], ref["scale"]))
    assert err <= TOL[cfg.dtype]


@pytest.mark.parametrize("name,order,N", [("o2_bf16_4k", 2, 333), ("o1_bf16_2k", 1, 1500)])
def test_constant_value_gives_the_value(name, order, N):
    """A constant plain V (dt = NULL): every output row is that V (a
    combination of equal rows whose weights sum to one; Algorithm 5's are
    >= 0).  Checked element by element (the oracle's error scale is 2 |V_c|
    there at order 2; at order 1 it also carries the normaliser's condition)."""
    cfg = TEST_CONFIGS[name]
    say("constant value", name, order, N)
    inp = I.make_forward_inputs(cfg, B=1, H=2, N=N, seed=33)
    row = inp.v[0, 0, 0].copy()
    inp.v[:] = row
    got = run_forward(inp, order, 64, with_dt=False)
    ref = oracle_forward(inp, order, with_dt=False)
    expect = np.broadcast_to(I.bf16_bits_to_f64(row), ref["y"].shape)
    np.testing.assert_allclose(ref["y"], expect, rtol=1e-12, atol=0)
    err = row_error(got["y"], ref["y"], ref["scale"])
    say("  ", worst(got["y"], ref["y"], ref["scale"]))
    assert err <= TOL[cfg.dtype]


# ---------------------------------------------------------------------------
# backward (order 1): the GPU gradients against the oracle's, with the
# oracle's y and den as the saved forward outputs (so that only the backward
# is measured)
# ---------------------------------------------------------------------------

def run_backward(q, k, v, dt, a_cs, y, den, dy, chunk, order=1):
    ssd = ssd_mod()
    out = ssd.backward(q, k, v, dt, a_cs, y, den, dy, order, chunk)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in out]


def backward_case(cfg, B, H, N, seed, positive, with_dt, chunk, order=1):
    """Inputs of the workload's generator (positive: |x| + 0.05 for q and k,
    normalisers bounded away from 0), the oracle's forward and backward, and
    the GPU backward on the same values."""
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=seed)
    qf, kf, vf = inp.qkv_f64()
    if positive:
        qf, kf = np.abs(qf) + 0.05, np.abs(kf) + 0.05
        store = lambda x: I._store(x, cfg.dtype)
        qs, ks = store(qf), store(kf)
        up = I.bf16_bits_to_f64 if cfg.dtype == I.BF16 else (lambda x: x.astype(np.float64))
        qf, kf = up(qs), up(ks)
    else:
        qs, ks = inp.q, inp.k
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    vop = vf * dt[..., None] if with_dt else vf
    ref_f = O.forward_quadratic(qf, kf, vop, a, order)
    dy = np.random.default_rng(seed + 1).standard_normal(vf.shape)
    dy = dy.astype(np.float32).astype(np.float64)
    ref = O.backward_quadratic(qf, kf, vop, a, order, dy)
    ssd = ssd_mod()
    dt_d, a_cs, _ = ssd.prep(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log), chunk)
    got = run_backward(to_dev_qkv(qs, cfg.dtype), to_dev_qkv(ks, cfg.dtype), to_dev_qkv(inp.v, cfg.dtype),
                       dt_d if with_dt else None, a_cs, to_dev_f32(ref_f["y"]), to_dev_f32(ref_f["den"]),
                       to_dev_f32(dy), chunk, order)
    dq, dk, dv, ddt, da = got
    # the oracle's gradients of v and dt through the value operand v dt
    if with_dt:
        ref_dv = ref["dvop"] * dt[..., None]
        ref_ddt = (ref["dvop"] * vf).sum(axis=-1)
    else:
        ref_dv, ref_ddt = ref["dvop"], None
    return {"dq": (dq, ref["dq"]), "dk": (dk, ref["dk"]), "dv": (dv, ref_dv), "da": (da, ref["da"]),
            "ddt": (ddt, ref_ddt)}, (qf, kf, vop, a, dy)


def rel_to_max(got, ref):
    return float(np.abs(got - ref).max() / np.abs(ref).max())


# (config, order, B, H, N, chunk, value operand v*dt)
BWD = [
    ("o1_f32_small", 1, 1, 2, 1, 64, True), ("o1_f32_small", 1, 1, 2, 63, 64, True),
    ("o1_f32_small", 1, 2, 1, 200, 128, True), ("o1_f32_small", 1, 1, 2, 130, 64, False),
    ("o1_bf16_2k", 1, 1, 2, 64, 64, True), ("o1_bf16_2k", 1, 2, 2, 333, 128, True),
    ("o1_bf16_2k", 1, 1, 3, 700, 64, False),
    ("o2_bf16_4k", 2, 1, 2, 1, 64, True), ("o2_bf16_4k", 2, 1, 2, 65, 64, True),
    ("o2_bf16_4k", 2, 2, 1, 200, 128, False), ("o2_bf16_4k", 2, 1, 3, 333, 64, True),
]


@pytest.mark.parametrize("name,order,B,H,N,chunk,with_dt", BWD)
def test_backward_small(name, order, B, H, N, chunk, with_dt):
    """Well-conditioned inputs (positive features): every gradient within
    1e-4 of the largest reference element of its tensor (fp32 arithmetic,
    products on split-bf16 operands: at most 3 2^-16 of each term)."""
    cfg = I.CONFIGS[name]
    say("backward", name, order, B, H, N, chunk, with_dt)
    res, _ = backward_case(cfg, B, H, N, seed=5 * N + H, positive=True, with_dt=with_dt, chunk=chunk,
                           order=order)
    dv_max = float(np.abs(res["dv"][1]).max())
    for n, (g, r) in res.items():
        if r is None:
            assert g is None
            continue
        # a gradient that is exactly 0 (N = 1: y_0 is the value operand) is
        # measured against the value gradient's size
        denom = float(np.abs(r).max())
        if denom <= 1e-8 * dv_max:
            denom = dv_max
        err = float(np.abs(g - r).max()) / denom
        say("  ", n, err)
        assert err <= 1e-4, n


@pytest.mark.parametrize("name,N", [("o1_f32_small", 256), ("o1_bf16_2k", 320), ("o2_bf16_4k", 200)])
def test_backward_workload_inputs(name, N):
    """The workload's own inputs (signed features, some normalisers near 0):
    every element within 1e-4 of its first-order error scale (the oracle's
    backward_error_scale), and the tensors' norm-wise errors small."""
    cfg = I.CONFIGS[name]
    say("backward workload inputs", name, N)
    res, (qf, kf, vop, a, dy) = backward_case(cfg, 1, 2, N, seed=17, positive=False, with_dt=True,
                                              chunk=cfg.chunk, order=cfg.order)
    sc = O.backward_error_scale(qf, kf, vop, a, cfg.order, dy)
    for n in ("dq", "dk", "da"):
        g, r = res[n]
        err = float((np.abs(g - r) / sc[n]).max())
        nrm = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        say("  ", n, err, nrm)
        assert err <= 1e-4 and nrm <= 1e-3, n
    assert all(np.all(np.isfinite(res[n][0])) for n in res if res[n][0] is not None)


def test_backward_full_size_sampled_heads():
    """The order-1 2K workload (4 x 16 heads, N 2048) through the backward at
    full size, in the launch the library uses; two heads checked against the
    oracle (positive features)."""
    cfg = I.CONFIGS["o1_bf16_2k"]
    say("backward full size")
    inp = I.make_forward_inputs(cfg)
    store = lambda x: I._store(x, cfg.dtype)
    qf, kf = (I.bf16_bits_to_f64(store(np.abs(I.bf16_bits_to_f64(x)) + 0.05)) for x in (inp.q, inp.k))
    qs, ks = store(qf), store(kf)
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    vop = I.bf16_bits_to_f64(inp.v) * dt[..., None]
    heads = [(0, 3), (3, 14)]
    dy = np.random.default_rng(8).standard_normal(vop.shape).astype(np.float32)
    # y and den for every head (the kernels read all of them): the GPU forward
    # on the same inputs; the checked heads' y and den are the oracle's
    ssd = ssd_mod()
    dt_d, a_cs, _ = ssd.prep(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log), cfg.chunk)
    q_d, k_d, v_d = to_dev_qkv(qs, cfg.dtype), to_dev_qkv(ks, cfg.dtype), to_dev_qkv(inp.v, cfg.dtype)
    den_d = torch.empty(inp.dt_proj.shape, device="cuda")
    y_d = ssd.forward(q_d, k_d, v_d, dt_d, a_cs, 1, cfg.chunk, den=den_d)
    refs = {}
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rf = O.forward_quadratic(qf[sl], kf[sl], vop[sl], a[sl], 1)
        y_d[b, h] = torch.from_numpy(rf["y"][0, 0].astype(np.float32)).cuda()
        den_d[b, h] = torch.from_numpy(rf["den"][0, 0].astype(np.float32)).cuda()
        refs[(b, h)] = O.backward_quadratic(qf[sl], kf[sl], vop[sl], a[sl], 1, dy[sl].astype(np.float64))
    dq, dk, dv, ddt, da = run_backward(q_d, k_d, v_d, dt_d, a_cs, y_d, den_d, to_dev_f32(dy), cfg.chunk)
    for (b, h), ref in refs.items():
        for n, g in (("dq", dq), ("dk", dk), ("da", da)):
            err = rel_to_max(g[b, h], ref[n][0, 0])
            say("  head", b, h, n, err)
            assert err <= 1e-4, (b, h, n)
        err = rel_to_max(dv[b, h], ref["dvop"][0, 0] * dt[b, h][:, None])
        assert err <= 1e-4, (b, h, "dv")


def test_backward_order2_full_size_sampled_heads():
    """The order-2 4K workload (2 x 16 heads, N 4096) through the backward at
    full size; two heads checked against the oracle (positive features)."""
    cfg = I.CONFIGS["o2_bf16_4k"]
    say("backward order 2 full size")
    inp = I.make_forward_inputs(cfg)
    store = lambda x: I._store(x, cfg.dtype)
    qf, kf = (I.bf16_bits_to_f64(store(np.abs(I.bf16_bits_to_f64(x)) + 0.05)) for x in (inp.q, inp.k))
    qs, ks = store(qf), store(kf)
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    vop = I.bf16_bits_to_f64(inp.v) * dt[..., None]
    heads = [(0, 5), (1, 12)]
    dy = np.random.default_rng(9).standard_normal(vop.shape).astype(np.float32)
    ssd = ssd_mod()
    dt_d, a_cs, _ = ssd.prep(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log), cfg.chunk)
    q_d, k_d, v_d = to_dev_qkv(qs, cfg.dtype), to_dev_qkv(ks, cfg.dtype), to_dev_qkv(inp.v, cfg.dtype)
    den_d = torch.empty(inp.dt_proj.shape, device="cuda")
    y_d = ssd.forward(q_d, k_d, v_d, dt_d, a_cs, 2, cfg.chunk, den=den_d)
    refs = {}
    for (b, h) in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rf = O.forward_quadratic(qf[sl], kf[sl], vop[sl], a[sl], 2)
        y_d[b, h] = torch.from_numpy(rf["y"][0, 0].astype(np.float32)).cuda()
        den_d[b, h] = torch.from_numpy(rf["den"][0, 0].astype(np.float32)).cuda()
        refs[(b, h)] = O.backward_quadratic(qf[sl], kf[sl], vop[sl], a[sl], 2, dy[sl].astype(np.float64))
    dq, dk, dv, ddt, da = run_backward(q_d, k_d, v_d, dt_d, a_cs, y_d, den_d, to_dev_f32(dy), cfg.chunk, 2)
    for (b, h), ref in refs.items():
        for n, g in (("dq", dq), ("dk", dk), ("da", da)):
            err = rel_to_max(g[b, h], ref[n][0, 0])
            say("  head", b, h, n, err)
            assert err <= 1e-4, (b, h, n)
        err = rel_to_max(dv[b, h], ref["dvop"][0, 0] * dt[b, h][:, None])
        assert err <= 1e-4, (b, h, "dv")


def test_backward_order2_long_sequence_decay_gradient():
    """Order 2 beyond 256 blocks (N 17100: 268 blocks, the last one ragged),
    where the decay gradient's suffix over later blocks runs in two chunks:
    da against -(1/2) sum_{s >= t} k_s . dk_s formed in fp64 from the same
    run's k and dk (an identity of the definition, pinned on the oracle by
    test_backward_decay_gradient_from_key_gradients; it holds at any size),
    and every gradient finite.  The tolerance is relative to the same sum of
    the terms' magnitudes."""
    cfg = I.CONFIGS["o2_bf16_4k"]
    N = 17100
    say("backward order 2 long sequence", N)
    inp = I.make_forward_inputs(cfg, B=1, H=1, N=N, seed=41)
    ssd = ssd_mod()
    dt_d, a_cs, _ = ssd.prep(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log), cfg.chunk)
    q_d, k_d, v_d = (to_dev_qkv(x, cfg.dtype) for x in (inp.q, inp.k, inp.v))
    den_d = torch.empty(inp.dt_proj.shape, device="cuda")
    y_d = ssd.forward(q_d, k_d, v_d, dt_d, a_cs, 2, cfg.chunk, den=den_d)
    dy = np.random.default_rng(42).standard_normal(y_d.shape).astype(np.float32)
    dq, dk, dv, ddt, da = run_backward(q_d, k_d, v_d, dt_d, a_cs, y_d, den_d, to_dev_f32(dy), cfg.chunk, 2)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv), ("ddt", ddt), ("da", da)):
        assert np.isfinite(g).all(), name
    kf = I.bf16_bits_to_f64(inp.k)
    term = -0.5 * (kf * dk.astype(np.float64)).sum(axis=-1)  # [1, 1, N]
    ref = np.cumsum(term[..., ::-1], axis=-1)[..., ::-1]
    mag = np.cumsum(np.abs(term)[..., ::-1], axis=-1)[..., ::-1]
    err = float((np.abs(da - ref) / (mag + 1e-30)).max())
    say("  da against the key-gradient identity", err)
    assert err <= 1e-5


@pytest.mark.parametrize("amask", [False, True])
def test_prep_backward(amask):
    """The discretisation's chain rule against the oracle's."""
    ssd = ssd_mod()
    cfg = I.CONFIGS["o1_bf16_2k"]
    inp = I.make_forward_inputs(cfg, B=2, H=3, N=200, seed=31)
    rng = np.random.default_rng(32)
    da = rng.standard_normal(inp.dt_proj.shape).astype(np.float32)
    ddt = rng.standard_normal(inp.dt_proj.shape).astype(np.float32)
    if not amask:
        g = ssd.prep_backward(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log),
                              to_dev_f32(da), to_dev_f32(ddt))
        ref = O.prep_backward_ref(inp.dt_proj, inp.dt_bias, inp.A_log, da, ddt)
        for x, r in zip(g, ref):
            np.testing.assert_allclose(x.cpu().numpy(), r, rtol=1e-4, atol=1e-5 * np.abs(r).max())
    else:
        dA, ddtp = ssd.prep_amask_backward(to_dev_f32(inp.A_proj), to_dev_f32(inp.dt_proj), to_dev_f32(da),
                                           to_dev_f32(ddt))
        rA, rdt = O.prep_amask_backward_ref(inp.A_proj, inp.dt_proj, da, ddt)
        np.testing.assert_allclose(dA.cpu().numpy(), rA, rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(ddtp.cpu().numpy(), rdt, rtol=1e-5, atol=1e-7)
