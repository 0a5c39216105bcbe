"""ssd_forward_noalloc (the forward for callers that cannot allocate: its
scratch is the library's per-device array) against ssd_forward with a
caller workspace: two calls in a row, the second with a smaller input, both
orders; the outputs must be identical (same kernels on the same inputs)."""
import numpy as np
import pytest

from mamba_ssd_sequence_amd import inputs as I
from parity import to_dev_f32, to_dev_qkv

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(cfg, B, H, N, seed, workspace, with_den):
    from mamba_ssd_sequence_amd import ssd
    inp = I.make_forward_inputs(cfg, B=B, H=H, N=N, seed=seed)
    q, k, v = (to_dev_qkv(x, cfg.dtype) for x in (inp.q, inp.k, inp.v))
    dt, a_cs, _ = ssd.prep(to_dev_f32(inp.dt_proj), to_dev_f32(inp.dt_bias), to_dev_f32(inp.A_log), cfg.chunk)
    D = 64 ** cfg.order
    den = torch.empty((B, H, N), device="cuda") if with_den else None
    fs = torch.empty((B, H, D, 64), device="cuda")
    fn = torch.empty((B, H, D), device="cuda")
    y = ssd.forward(q, k, v, dt, a_cs, cfg.order, cfg.chunk, den=den, final_state=fs, final_norm=fn,
                    workspace=workspace)
    return y, den, fs, fn


@pytest.mark.parametrize("name", ["o2_bf16_4k", "o1_bf16_2k"])
def test_forward_noalloc_matches_forward(name):
    cfg = I.CONFIGS[name]
    # two calls in a row, the second with a smaller input (the scratch still
    # holds the first call's contents when the second runs), then the same
    # two through ssd_forward with caller workspaces
    shapes = ((1, 8, 1000, 71), (1, 2, 130, 72))
    got = []
    for (B, H, N, seed) in shapes:
        print("noalloc", name, B, H, N, flush=True)
        got.append(_run(cfg, B, H, N, seed, "noalloc", True))
    torch.cuda.synchronize()
    for (B, H, N, seed), g in zip(shapes, got):
        want = _run(cfg, B, H, N, seed, None, True)
        torch.cuda.synchronize()
        for a, b in zip(g, want):
            assert torch.equal(a, b), (name, B, H, N)
        assert bool(torch.isfinite(g[0]).all())
