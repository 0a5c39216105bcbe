"""Seeded synthetic inputs for the SSD / 2Mamba sequence mixer.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds none of the mixer's arithmetic: it only draws random numbers and stores
them in the exact bit patterns the device receives.  Both the HIP path and the
CPU oracle consume the *same* stored values (the oracle upcasts them to fp64).

Stand-ins (2Mamba2Furious, Algorithm 2 "Mamba-2 Setup" and Algorithm 3
"Mamba-2 Forward Pass"):

* Q, K, V stand for the post-convolution, post-SiLU activations; they are drawn
  as silu(N(0,1)), optionally scaled by 1/sqrt(d_h).
* dt_P stands for the per-token projection h.W_dt; it is drawn as N(0,1).
* A_log is drawn as log(U[1,16]) per head and dt_bias as the inverse softplus
  of dt_init = exp(U[log 1e-3, log 1e-1]), both per head, following the
  initialisation of Algorithm 2.  The inverse softplus is written as
  y + log(-expm1(-y)), the numerically safe form of Algorithm 2's
  dt_init + log(1 - exp(-dt_init)).

* A_P stands for the per-token projection h.W_A of the A-mask of Mamba-2S /
  2Mamba (Algorithms 4 and 5, A = -softplus(h.W_A)); the pages give no
  distribution for it, and it is drawn as N(-3, 1), so that a typical token
  decays by e^{-softplus(-3)} ~ 0.95 (per-token decays from ~0.7 to ~0.999
  within two standard deviations).

Draw order (fixed, numpy PCG64 ``default_rng(seed)``): Q, K, V (each
[B,H,N,d_h]), dt_P [B,H,N], A_log [H], the dt_init exponent [H], then A_P
[B,H,N].
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) in fp64 (the generator's stand-in for the SiLU'd conv)."""
    return x / (1.0 + np.exp(-x))


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bfloat16 (round-to-nearest-even), return uint16 bits.

    The rounding is done once, directly from the fp64 value: the significand is
    scaled to 8 bits and rounded with numpy's half-to-even ``rint``.  Values in
    the bf16 subnormal range are rounded on the fixed 2^-133 grid.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2**e, |m| in [0.5, 1)
    # bf16 keeps 8 significant bits: m*2^8 in [128, 256)
    # subnormal bf16: exponent floor at -125 (m*2^e with e <= -125)
    e_eff = np.maximum(e, -125)
    scaled = np.ldexp(m, 8 + (e - e_eff))
    r = np.rint(scaled)
    y = np.ldexp(r, e_eff - 8)  # exactly representable in fp32
    y32 = y.astype(np.float32)
    return (y32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: sizes, precision and generator options."""

    name: str
    B: int
    H: int
    N: int
    d_h: int
    chunk: int
    order: int
    dtype: str  # "f32" or "bf16" for q, k, v
    qkv_scale: float = 1.0  # multiply silu(...) draws by this (1/sqrt(d_h) when scaled)
    seed: int = 0

    @property
    def D(self) -> int:
        return self.d_h ** self.order

    @property
    def n_chunks(self) -> int:
        return -(-self.N // self.chunk)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    S: int
    H: int
    d_h: int
    order: int
    steps: int
    dtype: str = BF16
    seed: int = 0

    @property
    def D(self) -> int:
        return self.d_h ** self.order


# The five workloads.  Forward: order-1 fp32 (small), order-1 bf16, order-2 bf16
# at 4K, order-2 bf16 at 64K; and the order-2 recurrent decode step.
CONFIGS = {
    "o1_f32_small": Config("o1_f32_small", B=1, H=2, N=256, d_h=32, chunk=64, order=1, dtype=F32),
    "o1_bf16_2k": Config("o1_bf16_2k", B=4, H=16, N=2048, d_h=64, chunk=64, order=1, dtype=BF16),
    "o2_bf16_4k": Config("o2_bf16_4k", B=2, H=16, N=4096, d_h=64, chunk=64, order=2, dtype=BF16,
                         qkv_scale=1.0 / math.sqrt(64)),
    "o2_bf16_64k": Config("o2_bf16_64k", B=1, H=16, N=65536, d_h=64, chunk=128, order=2, dtype=BF16,
                          qkv_scale=1.0 / math.sqrt(64)),
}
# Order 1 at the order-2 shapes (the metric names both orders at 4K and 64K):
# supplementary, measured and parity-tested next to the five workloads.
SUPPLEMENTARY = {
    "o1_bf16_4k": Config("o1_bf16_4k", B=2, H=16, N=4096, d_h=64, chunk=64, order=1, dtype=BF16,
                         qkv_scale=1.0 / math.sqrt(64)),
    "o1_bf16_64k": Config("o1_bf16_64k", B=1, H=16, N=65536, d_h=64, chunk=128, order=1, dtype=BF16,
                          qkv_scale=1.0 / math.sqrt(64)),
}
ALL_CONFIGS = {**CONFIGS, **SUPPLEMENTARY}

DECODE_CONFIGS = {
    "o2_decode": DecodeConfig("o2_decode", S=256, H=32, d_h=64, order=2, steps=128),
}


@dataclasses.dataclass
class ForwardInputs:
    """Stored inputs.  q/k/v are fp32 arrays (fp32 mode) or uint16 bf16 bits."""

    cfg: Config
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dt_proj: np.ndarray  # [B,H,N] fp32
    A_log: np.ndarray  # [H] fp32
    dt_bias: np.ndarray  # [H] fp32
    A_proj: np.ndarray = None  # [B,H,N] fp32 (A-mask projection A_P)

    def qkv_f64(self):
        """The stored q, k, v values, exactly, as fp64 (for the oracle)."""
        if self.cfg.dtype == BF16:
            return tuple(bf16_bits_to_f64(x) for x in (self.q, self.k, self.v))
        return tuple(x.astype(np.float64) for x in (self.q, self.k, self.v))


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return bf16_bits_rne(x64)
    return x64.astype(np.float32)


def draw_head_params(rng: np.random.Generator, H: int):
    """A_log = log(U[1,16]); dt_bias = softplus^-1(exp(U[log 1e-3, log 1e-1]))."""
    A_log = np.log(rng.uniform(1.0, 16.0, size=H))
    dt_init = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=H))
    dt_bias = dt_init + np.log(-np.expm1(-dt_init))
    return A_log.astype(np.float32), dt_bias.astype(np.float32)


def make_forward_inputs(cfg: Config, *, B=None, H=None, N=None, seed=None) -> ForwardInputs:
    """Draw the inputs of a forward workload (sizes may be overridden for tests)."""
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    N = cfg.N if N is None else N
    seed = cfg.seed if seed is None else seed
    cfg = dataclasses.replace(cfg, B=B, H=H, N=N, seed=seed)
    rng = np.random.default_rng(seed)
    shape = (B, H, N, cfg.d_h)
    arrs = []
    for _ in range(3):
        x = silu(rng.standard_normal(shape))
        if cfg.qkv_scale != 1.0:
            x = x * cfg.qkv_scale
        arrs.append(_store(x, cfg.dtype))
    dt_proj = rng.standard_normal((B, H, N)).astype(np.float32)
    A_log, dt_bias = draw_head_params(rng, H)
    A_proj = (rng.standard_normal((B, H, N)) - 3.0).astype(np.float32)
    return ForwardInputs(cfg, arrs[0], arrs[1], arrs[2], dt_proj, A_log, dt_bias, A_proj)


@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    A_log: np.ndarray  # [H] fp32
    dt_bias: np.ndarray  # [H] fp32
    _rng_state: dict

    def steps(self, n_steps=None, S=None, with_A=False):
        """Yield (q, k, v, dt_proj) per step, step-major, sequences [0:S); with
        with_A also the A-mask projection A_P [S,H] ~ N(-3, 1), drawn after
        dt_proj (the other draws are unchanged)."""
        rng = np.random.default_rng()
        rng.bit_generator.state = self._rng_state
        c = self.cfg
        n_steps = c.steps if n_steps is None else n_steps
        for _ in range(n_steps):
            shape = (c.S, c.H, c.d_h)
            qkv = [_store(silu(rng.standard_normal(shape)), c.dtype) for _ in range(3)]
            dt_proj = rng.standard_normal((c.S, c.H)).astype(np.float32)
            out = qkv + [dt_proj]
            if with_A:
                out.append((rng.standard_normal((c.S, c.H)) - 3.0).astype(np.float32))
            if S is not None:
                out = [x[:S] for x in out]
            yield tuple(out)


def make_decode_inputs(cfg: DecodeConfig, *, S=None, H=None, steps=None, seed=None) -> DecodeInputs:
    """Head parameters are drawn first, then per step q, k, v [S,H,d_h] and dt_P [S,H]."""
    cfg = dataclasses.replace(cfg, S=cfg.S if S is None else S, H=cfg.H if H is None else H,
                              steps=cfg.steps if steps is None else steps,
                              seed=cfg.seed if seed is None else seed)
    rng = np.random.default_rng(cfg.seed)
    A_log, dt_bias = draw_head_params(rng, cfg.H)
    return DecodeInputs(cfg, A_log, dt_bias, rng.bit_generator.state)
