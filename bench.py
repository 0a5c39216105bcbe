"""Throughput of the SSD / 2Mamba sequence mixer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-extra]
                    [--no-cpu-baseline] [--settle SECONDS]

A step is one pass of the whole hot path over one batch of synthetic inputs
already resident in HBM: ssd_prep (softplus, A*dt, chunk-local cumsum) followed
by ssd_forward (every kernel of the chunked forward).  The default workload is
the order-2 (2Mamba) forward at N = 4096 (B 2, H 16, d_h 64, bf16 inputs, fp32
accumulation).  One JSON line is printed on stdout; progress goes to stderr.

roofline: the dominant kernel of the step, timed with HIP events that the
library records on its own stream around each of its kernels over K further
steps run after the timed ones (events between kernels add launch gaps, so
the timed steps record none), against MI355X's published dense bf16 MFMA peak (2.5 PFLOP/s) or HBM
bandwidth (8 TB/s).  Algorithmic work per launch (see the design notes):
  order-2 numerator state scan: 4 * D * d_h flops per token and head
      (2 D d_h for phi(q)^T S, 2 D d_h for the phi(k) (v dt)^T update),
  order-1 scan kernel (bf16): q, k, v, dt, a_cs read and y written per token and
      head (3 d_h s_in + 8 + 4 d_h bytes); the whole order-1 step is also
      reported against its algorithmic bytes (3 d_h s_in + 4 + 4 d_h: q, k, v
      and dt_P read, y written),
  decode step: 2 * 4 * (D * d_h + D) bytes per sequence and head (D = d_h^2 rows,
      or d_h (d_h + 1) / 2 in the packed layout),
  backward step: 10 D d_h flops per token and head for the state parts (the
      states and state gradients rebuilt, and the three products with them:
      dq from S, dk and dv from the state gradient) plus 5 * 2 * 64^2 * d_h
      per 64-token block for the block-local products, against the bf16 peak
      (the backward's products run on bf16 matrix cores),
  prep sweep: 12 bytes per token and head (dt_P read, dt and a_cs written).
step_mfma_frac (order 2): the whole step against the chunked form's count,
  n_c [L(L+1)/2 (4 d_h + 2) + 2 (2 L D d_h + 2 L D) + 2 (D d_h + D)] per head.
cpu_baseline: the fp64 oracle (tests' reference implementation, untuned) on a
bounded sample of the same workload, on this machine's host cores.
device_ceilings: what the vendor library reaches on the same GPU (torch's fp16
GEMM at 8192^3 and at 4096^3, whose 1.374e11 flops equal the 4K state scan's
algorithmic count, and a 1 GiB copy), measured outside the timed steps, as
context for the roofline fractions.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mamba_ssd_sequence_amd import inputs as I  # noqa: E402

METRIC = "SSD fwd tokens/sec at N=4K and 64K (order 1/2); % bf16 MFMA peak"
CSRC = os.path.join(ROOT, "mamba_ssd_sequence_amd", "csrc")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
# sources each profiled kernel is built from: a traffic figure measured on one
# version of a kernel is reported only while these files are unchanged
KERNEL_SOURCES = {
    "k_o2_state": ["fwd_o2_state.hip", "launch.h", "common.h"],
    "k_o2_blockprep": ["fwd_o2_prep.hip", "launch.h", "common.h"],
    "k_o2_scale_scan": ["fwd_o2_prep.hip", "launch.h", "common.h"],
    "k_output": ["fwd_blocks.hip", "launch.h", "common.h"],
    "k_o1_scan": ["fwd_o1_scan.hip", "launch.h", "common.h"],
    "k_o1_segagg": ["fwd_o1_scan.hip", "launch.h", "common.h"],
    "k_o1_segprefix": ["fwd_o1_scan.hip", "launch.h", "common.h"],
    "k_decode": ["decode.hip", "launch.h", "common.h"],
    "k_prep": ["prep.hip", "launch.h", "common.h"],
}


def kernel_source_sha(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (calibrated against a plain copy), or None if absent or if the
    kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f).get(f"{kernel}@{workload}")
    except (OSError, ValueError):
        return None
    if not t or t.get("source_sha256") != kernel_source_sha(kernel):
        return None
    return t["traffic_bytes"]
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# order 1 with bf16 inputs: the segment aggregates (none when the sequence is
# one segment) and the scan itself
KERNELS_O1 = ["segment_aggregates", "o1_scan"]
KERNELS_O2 = ["block_prep", "scale_and_norm_scans", "o2_state_scan", "output"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# seconds of GPU load run before each workload's warm-up steps (--settle)
SETTLE_S = 0.25


def settle_clocks(dev):
    """Keep the GPU busy with fp16 GEMMs (torch, hipBLASLt) for SETTLE_S
    seconds, right before a workload's warm-up steps.  Drawing a workload's
    inputs on the host leaves the GPU idle for up to seconds, and an idle GPU
    drops to low clocks: without this the warm-up and the first few dozen
    timed steps would run while the clocks ramp back up (the 4K order-2 step
    takes ~0.20 ms over its first 25 steps and ~0.18 ms once settled), so
    the figure would describe a cold start rather than a running job."""
    import torch
    if SETTLE_S <= 0:
        return
    a = torch.randn(4096, 4096, dtype=torch.float16, device=dev)
    b = torch.randn(4096, 4096, dtype=torch.float16, device=dev)
    t = time.time()
    while time.time() - t < SETTLE_S:
        for _ in range(8):
            c = a @ b
        torch.cuda.synchronize()
    del a, b, c


def to_dev(x, dtype, dev):
    import torch
    if dtype == I.BF16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------

def bench_forward(cfg: I.Config, steps: int, warmup: int, dev, amask: bool = False):
    """amask: the step is ssd_prep_amask (Algorithm 5's A-mask, plain V) and
    ssd_forward with no dt, instead of ssd_prep (Algorithm 3) and V*dt."""
    import torch
    from mamba_ssd_sequence_amd import ssd

    t = time.time()
    inp = I.make_forward_inputs(cfg)
    log(f"[bench] {cfg.name}: inputs drawn in {time.time() - t:.1f}s")
    q, k, v = (to_dev(x, cfg.dtype, dev) for x in (inp.q, inp.k, inp.v))
    dtp, bias, alog = (to_dev(x, I.F32, dev) for x in (inp.dt_proj, inp.dt_bias, inp.A_log))
    B, H, N, d = q.shape
    nc = -(-N // cfg.chunk)
    dt = torch.empty((B, H, N), device=dev)
    a_cs = torch.empty((B, H, N), device=dev)
    a_chunk = torch.empty((B, H, nc), device=dev)
    y = torch.empty((B, H, N, d), device=dev)
    ws = torch.empty(ssd.workspace_size(B, H, N, d, cfg.order, cfg.chunk,
                                        ssd.SSD_BF16 if cfg.dtype == I.BF16 else ssd.SSD_F32),
                     dtype=torch.uint8, device=dev)

    A_proj = to_dev(inp.A_proj, I.F32, dev)

    def step(timer=None):
        if amask:
            ssd.prep_amask(A_proj, None, cfg.chunk, out=(None, a_cs, a_chunk))
        else:
            ssd.prep(dtp, bias, alog, cfg.chunk, out=(dt, a_cs, a_chunk))
        if timer is not None:
            timer.arm()
        ssd.forward(q, k, v, None if amask else dt, a_cs, cfg.order, cfg.chunk, y=y, workspace=ws)
        if timer is not None:
            timer.collect()

    settle_clocks(dev)
    for _ in range(warmup):
        step()
    # the timed steps (nothing recorded between the kernels) ...
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # ... then as many steps again with the library's per-kernel events, for
    # the kernel breakdown (events between kernels add launch gaps, so these
    # steps are not the timed ones)
    timers = [ssd.KernelTimer() for _ in range(steps)]
    for i in range(steps):
        step(timers[i])
    torch.cuda.synchronize()
    names = KERNELS_O2 if cfg.order == 2 else KERNELS_O1
    per = np.array([tm.durations_ms() for tm in timers])  # [steps, kernels]
    kern_ms = dict(zip(names, per.mean(axis=0).tolist()))
    assert bool(torch.isfinite(y).all())
    tokens = B * N
    res = {"workload": cfg.name + ("_amask" if amask else ""), "ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3),
           "kernels_ms": kern_ms, "B": B, "H": H, "N": N, "d_h": d, "order": cfg.order,
           "chunk": cfg.chunk, "dtype": cfg.dtype}
    if cfg.order == 2:
        D = d * d
        flops = 4.0 * D * d * B * H * N
        t_ms = kern_ms["o2_state_scan"]
        ach = flops / (t_ms * 1e-3) / 1e12
        res["roofline"] = {"kernel": "k_o2_state", "bound": "mfma", "achieved": ach,
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / PEAK_BF16_TFLOPS,
                           "traffic": measured_traffic("k_o2_state", cfg.name),
                           "alg_flops_per_launch": flops, "avg_launch_ms": t_ms}
        # whole-step MFMA fraction of the method's chunked work: every flop of
        # the chunked form per head, n_c [L(L+1)/2 (4 d_h + 2) + 2 (2 L D d_h +
        # 2 L D) + 2 (D d_h + D)] with L the chunk, D = d_h^2
        L = cfg.chunk
        n_c = -(-N // L)
        F = B * H * n_c * (L * (L + 1) / 2 * (4 * d + 2) + 2 * (2 * L * D * d + 2 * L * D)
                           + 2 * (D * d + D))
        res["step_alg_flops"] = F
        res["step_mfma_frac"] = F / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
        # measured HBM bytes per launch of every kernel of the step (rocprofv3
        # counters in profiles/traffic.json; null where the sources changed)
        res["kernel_traffic_bytes"] = {k: measured_traffic(k, cfg.name) for k in
                                       ("k_prep", "k_o2_blockprep", "k_o2_scale_scan", "k_o2_state", "k_output")}
        res["step_alg_bytes"] = B * H * N * (3 * d * 2 + 4 + 4 * d)
    else:
        es = 2 if cfg.dtype == I.BF16 else 4
        # the scan kernel: q, k, v, dt and a_cs read, y written (the segment
        # aggregates it also reads are the implementation's, not the method's)
        by = B * H * N * (3 * d * es + 8 + 4 * d)
        t_ms = kern_ms["o1_scan"]
        ach = by / (t_ms * 1e-3) / 1e9
        res["roofline"] = {"kernel": "k_o1_scan", "bound": "hbm", "achieved": ach,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                           "traffic": measured_traffic("k_o1_scan", cfg.name),
                           "alg_bytes_per_launch": by, "avg_launch_ms": t_ms}
        # the whole step (prep + forward) against the method's bytes: q, k, v
        # and dt_P read, y written
        step_by = B * H * N * (3 * d * es + 4 + 4 * d)
        res["step_alg_bytes"] = step_by
        res["step_hbm_frac"] = step_by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS
    return res, inp


def bench_backward(cfg: I.Config, steps: int, warmup: int, dev):
    """A training step's mixer gradients: ssd_backward + ssd_prep_backward on
    the workload's inputs, with the forward's y and den (computed once,
    outside the timed steps) as the saved activations and a random dy."""
    import torch
    from mamba_ssd_sequence_amd import ssd

    inp = I.make_forward_inputs(cfg)
    q, k, v = (to_dev(x, cfg.dtype, dev) for x in (inp.q, inp.k, inp.v))
    dtp, bias, alog = (to_dev(x, I.F32, dev) for x in (inp.dt_proj, inp.dt_bias, inp.A_log))
    B, H, N, d = q.shape
    dt, a_cs, _ = ssd.prep(dtp, bias, alog, cfg.chunk)
    den = torch.empty((B, H, N), device=dev)
    y = ssd.forward(q, k, v, dt, a_cs, cfg.order, cfg.chunk, den=den)
    dy = torch.randn((B, H, N, d), generator=torch.Generator(device=dev).manual_seed(0), device=dev)
    ws = torch.empty(ssd.lib().ssd_backward_workspace_size(B, H, N, d, cfg.order, cfg.chunk,
                                                           ssd.SSD_BF16 if cfg.dtype == I.BF16 else ssd.SSD_F32),
                     dtype=torch.uint8, device=dev)

    def step():
        _, _, _, ddt, da = ssd.backward(q, k, v, dt, a_cs, y, den, dy, cfg.order, cfg.chunk, workspace=ws)
        ssd.prep_backward(dtp, bias, alog, da, ddt)

    settle_clocks(dev)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # algorithmic flops: per token and head 10 D d_h for the state parts (the
    # states S and state gradients G rebuilt, 2 D d_h each; dq from S dnum,
    # dk and dv from G, 2 D d_h each), per 64-token block and head five
    # 64 x 64 x d_h products (scores, dnum vop^T, the scores' gradient times
    # K and times Q, W^T dnum)
    D = d ** cfg.order
    nb = -(-N // 64)
    flops = B * H * (N * 10.0 * D * d + nb * 5 * 2.0 * 64 * 64 * d)
    ach = flops / (ms * 1e-3) / 1e12
    # algorithmic bytes (context): q, k, v read, dt, a_cs, den read, y and dy
    # read (fp32), dq, dk, dv written (fp32), ddt, da and the prep gradients
    es = 2 if cfg.dtype == I.BF16 else 4
    by = B * H * N * (3 * d * es + 2 * 4 * d + 3 * 4 * d + 4 * 4 + 2 * 4)
    return {"workload": cfg.name + "_backward", "ms_per_step": ms, "tokens_per_s": B * N / (ms * 1e-3),
            "B": B, "H": H, "N": N, "d_h": d, "order": cfg.order, "chunk": cfg.chunk,
            "roofline": {"kernel": "step", "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS, "traffic": None,
                         "alg_flops_per_launch": flops, "avg_launch_ms": ms},
            "alg_bytes": by, "hbm_frac_of_alg_bytes": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def bench_prep_sweep(steps: int, warmup: int, dev, B=4, H=32, N=1 << 21, chunk=64):
    """ssd_prep alone on B * H * N = 2^28 tokens x heads (dt_P from torch's
    seeded generator on the device), against the HBM peak: 4 bytes read and
    8 written per token and head."""
    import torch
    from mamba_ssd_sequence_amd import ssd
    g = torch.Generator(device=dev).manual_seed(0)
    dtp = torch.randn((B, H, N), generator=g, device=dev)
    bias = torch.full((H,), -3.0, device=dev)
    alog = torch.zeros((H,), device=dev)
    nc = -(-N // chunk)
    out = (torch.empty((B, H, N), device=dev), torch.empty((B, H, N), device=dev),
           torch.empty((B, H, nc), device=dev))
    settle_clocks(dev)
    for _ in range(warmup):
        ssd.prep(dtp, bias, alog, chunk, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        ssd.prep(dtp, bias, alog, chunk, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    by = B * H * N * 12 + B * H * nc * 4
    ach = by / (ms * 1e-3) / 1e9
    del dtp, out
    return {"workload": "prep_sweep_2^28", "ms_per_step": ms, "tokens_per_s": B * N / (ms * 1e-3),
            "B": B, "H": H, "N": N, "chunk": chunk,
            "roofline": {"kernel": "k_prep", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                         "traffic": measured_traffic("k_prep", "prep_sweep_2^28"),
                         "alg_bytes_per_launch": by, "avg_launch_ms": ms}}


def cpu_baseline_forward(cfg: I.Config, inp, budget_s=12.0):
    """Oracle throughput on a bounded sample: whole heads (quadratic form) when
    they fit the budget, else uniformly sampled rows of one head, extrapolated."""
    from oracle import ssd_oracle as O
    q, k, v = inp.qkv_f64()
    dt, a = O.discretise(inp.dt_proj, inp.dt_bias, inp.A_log)
    vdt = v * dt[..., None]
    B, H, N, _ = q.shape
    if N <= 8192:
        t0 = time.time()
        heads = 0
        while heads < B * H and (heads == 0 or time.time() - t0 < budget_s):
            b, h = divmod(heads, H)
            O.forward_quadratic(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], vdt[b:b + 1, h:h + 1],
                                a[b:b + 1, h:h + 1], cfg.order)
            heads += 1
        el = time.time() - t0
        t_head = el / heads
        sample = f"quadratic-form oracle over {heads} whole head(s) of {B * H}, N={N}"
    else:
        rng = np.random.default_rng(0)
        t0 = time.time()
        done = 0
        while done == 0 or time.time() - t0 < budget_s:
            rows = np.sort(rng.integers(0, N, 64))
            O.forward_quadratic(q[:1, :1], k[:1, :1], vdt[:1, :1], a[:1, :1], cfg.order, rows=rows)
            done += len(rows)
        el = time.time() - t0
        t_head = el / done * N
        sample = (f"quadratic-form oracle on {done} uniformly sampled rows of 1 head (N={N}), "
                  f"extrapolated to all rows and {B * H} heads")
    tokens_per_s = N / (H * t_head)  # B*N tokens need B*H head evaluations
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": sample, "wall_s": el}


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def bench_decode(cfg: I.DecodeConfig, steps: int, warmup: int, dev, packed=False):
    """Decode steps; packed: the order-2 states in the packed layout (rows
    a <= b, D' = d_h (d_h + 1) / 2), whose algorithmic bytes are counted with D'."""
    import torch
    from mamba_ssd_sequence_amd import ssd

    t = time.time()
    dec = I.make_decode_inputs(cfg, steps=steps + warmup)
    toks = [tuple(to_dev(x, cfg.dtype, dev) for x in s[:3]) + (to_dev(s[3], I.F32, dev),)
            for s in dec.steps()]
    log(f"[bench] {cfg.name}: inputs drawn in {time.time() - t:.1f}s")
    D = cfg.d_h ** cfg.order if not packed else cfg.d_h * (cfg.d_h + 1) // 2
    state = torch.zeros((cfg.S, cfg.H, D, cfg.d_h), device=dev)
    norm = torch.zeros((cfg.S, cfg.H, D), device=dev)
    y = torch.empty((cfg.S, cfg.H, cfg.d_h), device=dev)
    bias, alog = to_dev(dec.dt_bias, I.F32, dev), to_dev(dec.A_log, I.F32, dev)
    settle_clocks(dev)
    for i in range(warmup):
        q, k, v, dtp = toks[i]
        ssd.decode_step(q, k, v, dtp, bias, alog, state, norm, cfg.order, y=y, packed=packed)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        q, k, v, dtp = toks[warmup + i]
        ev[i].record()
        ssd.decode_step(q, k, v, dtp, bias, alog, state, norm, cfg.order, y=y, packed=packed)
    ev[steps].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    ms = ev[0].elapsed_time(ev[steps]) / steps
    by = 2.0 * 4 * (D * cfg.d_h + D) * cfg.S * cfg.H
    t_ms = float(np.mean(per))
    ach = by / (t_ms * 1e-3) / 1e9
    name = cfg.name + ("_packed" if packed else "")
    return {"workload": name, "ms_per_step": ms, "tokens_per_s": cfg.S / (ms * 1e-3),
            "S": cfg.S, "H": cfg.H, "d_h": cfg.d_h, "order": cfg.order, "steps": steps,
            "state_layout": "packed" if packed else "full", "state_rows": D,
            "roofline": {"kernel": "k_decode", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                         "traffic": measured_traffic("k_decode", name),
                         "alg_bytes_per_launch": by, "avg_launch_ms": t_ms}}, dec


def cpu_baseline_decode(cfg: I.DecodeConfig, dec, budget_s=10.0):
    from oracle import ssd_oracle as O
    D = cfg.d_h ** cfg.order
    M = 8  # (sequence, head) pairs per oracle call
    St = np.zeros((1, M, D, cfg.d_h))
    zt = np.zeros((1, M, D))
    t0 = time.time()
    n = 0
    for (q, k, v, dtp) in dec.steps(n_steps=cfg.steps):
        sl = (slice(0, 1), slice(0, M))
        _, St, zt, _ = O.decode_step_ref(St, zt, I.bf16_bits_to_f64(q[sl]), I.bf16_bits_to_f64(k[sl]),
                                         I.bf16_bits_to_f64(v[sl]), dtp[sl], dec.dt_bias[:M],
                                         dec.A_log[:M], cfg.order)
        n += 1
        if time.time() - t0 > budget_s:
            break
    el = time.time() - t0
    t_head_step = el / (n * M)
    return {"value": 1.0 / (cfg.H * t_head_step), "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"fp64 recurrence oracle, {M} (sequence, head) pairs x {n} steps, "
                      f"extrapolated to {cfg.S} x {cfg.H} per step", "wall_s": el}


def device_ceilings(dev):
    """What the vendor's own library code reaches on this GPU, as context for
    the roofline fractions (not part of the timed step): torch's fp16 GEMM
    (hipBLASLt) on 8192^3 and on 4096^3 (1.374e11 flops: the order-2 state
    scan's algorithmic count on the 4K workload, so the two times compare
    directly), and a 1 GiB device-to-device copy."""
    import torch
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for M, reps in ((8192, 10), (4096, 40)):
        a = torch.randn(M, M, dtype=torch.float16, device=dev)
        b = torch.randn(M, M, dtype=torch.float16, device=dev)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"torch_fp16_gemm_{M}_tflops"] = 2 * M ** 3 / (ms * 1e-3) / 1e12
        out[f"torch_fp16_gemm_{M}_frac_of_2500"] = out[f"torch_fp16_gemm_{M}_tflops"] / 2500.0
        if M == 4096:
            out["torch_fp16_gemm_4096_us"] = ms * 1e3
        del a, b, c
    n = (1 << 30) // 4
    src = torch.ones(n, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    out["torch_copy_1gib_gbs"] = 2 * (1 << 30) / (ms * 1e-3) / 1e9  # bytes read + written
    del src, dst
    torch.cuda.empty_cache()
    return out


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        n = max((d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"), default=1)
        return int(n)
    except Exception:
        return 1


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="o2_bf16_4k",
                    choices=list(I.ALL_CONFIGS) + list(I.DECODE_CONFIGS) + ["o2_decode_packed"]
                    + ["o1_bf16_2k_backward", "o2_bf16_4k_backward", "prep_sweep_2^28"])
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads (64K forward, decode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S, metavar="SECONDS",
                    help="GPU load (fp16 GEMMs) before each workload's warm-up steps, so that "
                         "the clocks have left their idle state (0: none, a cold start)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (reference for HBM counters)")
    a = ap.parse_args()
    SETTLE_S = a.settle
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the mixer's workloads are per-head independent "
              "and this build has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_calibration:
        nbytes = a.copy_calibration << 20
        src = torch.ones(nbytes // 4, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {nbytes} bytes device to device 3 times")
        return
    from mamba_ssd_sequence_amd import ssd
    ssd.lib()

    if a.workload == "prep_sweep_2^28":
        cfg, res, inp = None, bench_prep_sweep(a.steps, a.warmup, dev), None
    elif a.workload.endswith("_backward"):
        cfg = I.ALL_CONFIGS[a.workload[:-len("_backward")]]
        res, inp = bench_backward(cfg, a.steps, a.warmup, dev), None
    elif a.workload in I.ALL_CONFIGS:
        cfg = I.ALL_CONFIGS[a.workload]
        res, inp = bench_forward(cfg, a.steps, a.warmup, dev)
    else:
        packed = a.workload.endswith("_packed")
        cfg = I.DECODE_CONFIGS[a.workload[:-len("_packed")] if packed else a.workload]
        res, inp = bench_decode(cfg, a.steps, a.warmup, dev, packed=packed)
    log(f"[bench] {a.workload}: {res['ms_per_step']:.4f} ms/step, {res['tokens_per_s']:.4g} tokens/s, "
        f"roofline frac {res['roofline']['frac']:.3f}")

    extra = []
    if not a.no_extra:
        for name in ("o2_bf16_64k", "o1_bf16_2k", "o1_bf16_4k", "o1_bf16_64k", "o2_decode",
                     "o2_decode_packed", "o2_bf16_4k_amask", "o1_bf16_2k_backward",
                     "o2_bf16_4k_backward", "prep_sweep_2^28"):
            if name == a.workload:
                continue
            torch.cuda.empty_cache()
            if name == "prep_sweep_2^28":
                r = bench_prep_sweep(max(3, a.steps // 4), 2, dev)
            elif name == "o2_bf16_4k_amask":
                r, _ = bench_forward(I.CONFIGS["o2_bf16_4k"], a.steps, a.warmup, dev, amask=True)
            elif name in I.ALL_CONFIGS:
                r, _ = bench_forward(I.ALL_CONFIGS[name], max(3, a.steps // 4), 2, dev)
            elif name.endswith("_backward"):
                r = bench_backward(I.CONFIGS[name[:-len("_backward")]], max(3, a.steps // 4), 2, dev)
            elif name == "o2_decode_packed":
                c = I.DECODE_CONFIGS["o2_decode"]
                r, _ = bench_decode(c, c.steps, 3, dev, packed=True)
            else:
                c = I.DECODE_CONFIGS[name]
                r, _ = bench_decode(c, c.steps, 3, dev)
            log(f"[bench] extra {name}: {r['ms_per_step']:.4f} ms/step, {r['tokens_per_s']:.4g} tokens/s, "
                f"roofline frac {r['roofline']['frac']:.3f}")
            extra.append(r)

    ceilings = None
    if not a.no_extra:
        ceilings = device_ceilings(dev)
        log(f"[bench] context: torch fp16 GEMM 8192^3 {ceilings['torch_fp16_gemm_8192_tflops']:.0f} TFLOP/s, "
            f"4096^3 {ceilings['torch_fp16_gemm_4096_us']:.1f} us, "
            f"1 GiB copy {ceilings['torch_copy_1gib_gbs']:.0f} GB/s")

    cpu = None
    if not a.no_cpu_baseline and inp is not None:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        if a.workload in I.ALL_CONFIGS:
            cpu = cpu_baseline_forward(cfg, inp)
        else:
            cpu = cpu_baseline_decode(cfg, inp)
        cpu["host_cpus"] = os.cpu_count()
        cpu["affinity_cpus"] = len(os.sched_getaffinity(0))

    config = {k: res[k] for k in ("workload", "B", "H", "N", "d_h", "order", "chunk", "S", "steps")
              if k in res}
    out = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if getattr(cfg, "dtype", I.BF16) == I.BF16 else "f32",
        "data": "synthetic",
        "config": config,
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "kernels_ms": res.get("kernels_ms"),
        "step_mfma_frac": res.get("step_mfma_frac"),
        "step_hbm_frac": res.get("step_hbm_frac"),
        "extra": extra,
        "device_ceilings": ceilings,
        "device": torch.cuda.get_device_name(dev),
        "clock_settle_s": SETTLE_S,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
