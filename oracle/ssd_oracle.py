"""CPU fp64 oracle for the masked linear-attention sequence mixer (Mamba-2 /
Mamba-2S / 2Mamba) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP path and imports nothing from it:
it receives plain numpy arrays (the stored input values, upcast exactly to
fp64) and computes everything in fp64, in the order the definitions state.

Sources (2Mamba2Furious: Linear in Complexity, Competitive in Accuracy,
Mongaras & Larson):

* Algorithm 1 (linear attention): masked product y = (phi(Q) phi(K)^T * M) V,
  normaliser = row sum of the same masked score matrix, output y / normaliser.
* Algorithm 3 (Mamba-2 forward pass): A = -exp(A_log), dt = softplus(dt_P +
  dt_bias), V_dt = V * dt, A^CS = cumsum(A * dt).
* Algorithms 4 and 5, the A-mask of Mamba-2S / 2Mamba: per-token A =
  -softplus(h W_A), A^CS = cumsum(A) with no dt in it; Algorithm 4 keeps
  V_dt = V * dt with dt = softplus(h W_dt) (no bias), Algorithm 5 uses plain V.
* Algorithms 4 and 5 (Mamba-2S, 2Mamba): decay mask A^M_ij = exp(A^CS_i -
  A^CS_j), causal mask M_ij = [i >= j], and for 2Mamba the scores are squared
  and the normaliser is the row sum of the squared, masked scores.
* Algorithm 6 (2Mamba inference, appendix): the recurrent form, with order-2
  features k (x) k and the two states H_up (numerator) and H_down (normaliser)
  decayed by a_t each step; as printed, a_t = exp(-softplus(h W_A)) (the
  A-mask), also provided next to the Mamba-2 discretisation.
* The backward pass (the pages train these models but print no gradients):
  the chain rule applied to the quadratic form and to Algorithm 3's
  discretisation, written out step by step.
* The symmetric-packed order-2 state (not on the pages; derived from the
  symmetry of k (x) k in Algorithm 6): only the rows (a, b) with a <= b are
  stored, and the query contraction counts the off-diagonal rows twice.

Readings where the pages are silent or garbled (each is also listed with its
reasoning in the design notes):

* the cumulative sum is inclusive (torch/numpy cumsum), so M_ii = 1;
* the normaliser is divided exactly: no epsilon, no absolute value;
* the value operand is V * dt for both orders (Algorithm 5 prints plain V; a
  caller reproduces that by passing the value operand directly);
* phi is the identity inside the mixer (SiLU is applied upstream); order 2 uses
  phi(x) = vec(x x^T) flattened row-major, D = d_h**2;
* the missing output line of Algorithm 6 is y_t = phi(q_t)^T H_up_t /
  phi(q_t)^T H_down_t using the states after the update at t;
* the initial state is zero;
* exp is only ever evaluated on masked (j <= i) differences, never on the
  literal A^M over the whole square (which would overflow above the diagonal).

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle.py (two independent forms agreeing to 1e-10, closed forms,
special cases that reduce to textbook routines, invariants, and the hand-worked
fixtures in tests/golden/).
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# Discretisation (Algorithm 3)
# ---------------------------------------------------------------------------

def softplus(x):
    """softplus(x) = log(1 + e^x), evaluated as max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def discretise(dt_proj, dt_bias, A_log):
    """Algorithm 3: dt = softplus(dt_P + dt_bias), A = -exp(A_log), a = A * dt.

    dt_proj: [..., H, N]; dt_bias, A_log: [H].  Returns (dt, a) with the shape
    of dt_proj; a is the per-token log-decay (always <= 0).
    """
    dt_proj = np.asarray(dt_proj, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    dt = softplus(dt_proj + dt_bias[:, None])
    a = A[:, None] * dt
    return dt, a


def discretise_amask(A_proj, dt_proj=None):
    """Algorithms 4 and 5 (Mamba-2S, 2Mamba): the A-mask A = -softplus(h W_A)
    per token, with A^CS = cumsum(A) -- no dt in the decay.

    A_proj: [..., H, N], the projection A_P = h W_A.  Returns (dt, a): a = A
    (always < 0); dt = softplus(dt_P) with no bias (Algorithm 4, value operand
    V * dt), or None when dt_proj is None (Algorithm 5, plain V).
    """
    a = -softplus(A_proj)
    dt = None if dt_proj is None else softplus(dt_proj)
    return dt, a


def _chunked_cumsum(a, chunk):
    """Inclusive cumsum of a restarted at every chunk start, and chunk totals."""
    N = a.shape[-1]
    n_chunks = -(-N // chunk)
    a_cs = np.empty_like(a)
    a_chunk = np.empty(a.shape[:-1] + (n_chunks,), dtype=np.float64)
    for c in range(n_chunks):
        seg = a[..., c * chunk:(c + 1) * chunk]
        cs = np.cumsum(seg, axis=-1)
        a_cs[..., c * chunk:(c + 1) * chunk] = cs
        a_chunk[..., c] = cs[..., -1]
    return a_cs, a_chunk


def prep_amask_ref(A_proj, dt_proj, chunk):
    """What ssd_prep_amask returns, in fp64: (dt or None, a_cs, a_chunk), with
    a = -softplus(A_P) chunked as in prep_ref."""
    dt, a = discretise_amask(A_proj, dt_proj)
    a_cs, a_chunk = _chunked_cumsum(a, chunk)
    return dt, a_cs, a_chunk


def prep_ref(dt_proj, dt_bias, A_log, chunk):
    """What ssd_prep returns, in fp64.

    Returns (dt, a_cs, a_chunk): dt [B,H,N]; a_cs [B,H,N] the inclusive
    cumulative sum of a = A*dt restarted at every chunk start (positions
    c*chunk .. c*chunk+chunk-1); a_chunk [B,H,n_chunks] the total of a over each
    chunk (the last chunk may be partial).  The global A^CS of Algorithm 3 is
    a_cs plus the sum of the earlier chunk totals.
    """
    dt, a = discretise(dt_proj, dt_bias, A_log)
    N = a.shape[-1]
    n_chunks = -(-N // chunk)
    a_cs = np.empty_like(a)
    a_chunk = np.empty(a.shape[:-1] + (n_chunks,), dtype=np.float64)
    for c in range(n_chunks):
        seg = a[..., c * chunk:(c + 1) * chunk]
        cs = np.cumsum(seg, axis=-1)
        a_cs[..., c * chunk:(c + 1) * chunk] = cs
        a_chunk[..., c] = cs[..., -1]
    return dt, a_cs, a_chunk


# ---------------------------------------------------------------------------
# Feature maps
# ---------------------------------------------------------------------------

def features(x, order):
    """phi(x): identity at order 1; vec(x x^T) (row-major, D = d_h^2) at order 2."""
    x = np.asarray(x, dtype=np.float64)
    if order == 1:
        return x
    if order == 2:
        outer = x[..., :, None] * x[..., None, :]
        return outer.reshape(x.shape[:-1] + (x.shape[-1] ** 2,))
    raise ValueError("order must be 1 or 2")


# ---------------------------------------------------------------------------
# Quadratic (masked attention) form -- Algorithms 1, 4, 5
# ---------------------------------------------------------------------------

def _head_quadratic(q, k, vop, a, order, rows):
    """One head.  q, k: [N,d]; vop: [N,dv]; a: [N] log-decays.

    w_ij = (q_i . k_j)^order * exp(A^CS_i - A^CS_j) for j <= i, else 0.
    Returns num [R,dv], den [R], kappa [R], scale [R] for the requested rows.
    """
    cs = np.cumsum(a)  # inclusive A^CS
    if rows is None:
        G = q @ k.T
        Gp = G ** order
        diff = cs[:, None] - cs[None, :]
        causal = np.tril(np.ones(G.shape, dtype=bool))
        # mask first, then exponentiate only the kept (non-positive) differences
        decay = np.exp(np.where(causal, diff, -np.inf))
        W = Gp * decay
        num = W @ vop
        den = W.sum(axis=1)
        absW = np.abs(W)
        abs_sum = absW.sum(axis=1)
        abs_num = absW @ np.abs(vop)
        # the state form's magnitudes: (sum_a |q_ia||k_ja|)^p in place of |q_i . k_j|^p
        Wst = (np.abs(q) @ np.abs(k).T) ** order * decay
        st_sum = Wst.sum(axis=1)
        st_num = Wst @ np.abs(vop)
    else:
        # the same definition for the requested rows only, a batch of rows at
        # a time: row i uses the tokens j <= i (mask first, then exponentiate
        # the kept, non-positive differences)
        rows = np.asarray(rows, dtype=np.int64)
        R = len(rows)
        dv = vop.shape[1]
        num = np.empty((R, dv))
        den = np.empty(R)
        abs_sum = np.empty(R)
        abs_num = np.empty((R, dv))
        st_sum = np.empty(R)
        st_num = np.empty((R, dv))
        avop, aq, ak = np.abs(vop), np.abs(q), np.abs(k)
        for r0 in range(0, R, 128):
            rb = rows[r0:r0 + 128]
            n = int(rb.max()) + 1
            g = q[rb] @ k[:n].T
            keep = np.arange(n)[None, :] <= rb[:, None]
            decay = np.exp(np.where(keep, cs[rb][:, None] - cs[None, :n], -np.inf))
            w = (g ** order) * decay
            num[r0:r0 + len(rb)] = w @ vop[:n]
            den[r0:r0 + len(rb)] = w.sum(axis=1)
            aw = np.abs(w)
            abs_sum[r0:r0 + len(rb)] = aw.sum(axis=1)
            abs_num[r0:r0 + len(rb)] = aw @ avop[:n]
            wst = (aq[rb] @ ak[:n].T) ** order * decay
            st_sum[r0:r0 + len(rb)] = wst.sum(axis=1)
            st_num[r0:r0 + len(rb)] = wst @ avop[:n]
    with np.errstate(divide="ignore", invalid="ignore"):
        kappa = abs_sum / np.abs(den)
        y = num / den[:, None]
        # first-order rounding bound of a quotient of two sums:
        # |d(n/d)| <= (|dn| + |n/d| |dd|) / |d|, |dn| <= eps sum|w||v|, |dd| <= eps sum|w|
        scale = (abs_num + np.abs(y) * abs_sum[:, None]) / np.abs(den)[:, None]
        # the same bound for the state form (Algorithm 6), y = phi(q)^T S /
        # phi(q)^T z with S, z sums over tokens of phi(k) terms: its sums run
        # over the D feature products q_a.. k_a.., so their rounding is
        # bounded by (sum_a |q_ia||k_ja|)^p per token instead of |q_i . k_j|^p
        scale_state = (st_num + np.abs(y) * st_sum[:, None]) / np.abs(den)[:, None]
    return num, den, kappa, scale, scale_state


def forward_quadratic(q, k, vop, a, order, rows=None):
    """Masked quadratic form over [B,H,N,.] arrays (fp64).

    q, k: [B,H,N,d_h]; vop: [B,H,N,d_v] (the value operand, V*dt end to end);
    a: [B,H,N] per-token log-decay.  rows: optional sorted 1-D array of token
    indices to evaluate (one by one, so that long sequences can be sampled).

    Returns dict with y = num/den, num, den, and the diagnostics
    kappa[i] = sum_j |w_ij| / |den_i| (condition of the normaliser) and
    scale[i, c] = (sum_j |w_ij| |vop_jc| + |y_ic| sum_j |w_ij|) / |den_i|,
    the first-order rounding-error bound of y_ic = num_ic / den_i divided by
    the unit roundoff: a floating-point evaluation of y_ic with relative
    accuracy eps in its sums is off by at most about eps * scale[i, c].
    scale_state[i, c]: the same bound for an evaluation through the states of
    Algorithm 6 (y = phi(q)^T S / phi(q)^T z), whose sums run over the
    feature products: (sum_a |q_ia||k_ja|)^order replaces |q_i . k_j|^order.
    It equals scale when no feature product cancels (d_h = 1, or q and k
    with equal signs per component).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vop = np.asarray(vop, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    B, H, N, _ = q.shape
    R = N if rows is None else len(rows)
    dv = vop.shape[-1]
    out = {n: np.empty((B, H, R, dv)) for n in ("num",)}
    out.update({n: np.empty((B, H, R)) for n in ("den", "kappa")})
    out["scale"] = np.empty((B, H, R, dv))
    out["scale_state"] = np.empty((B, H, R, dv))
    for b in range(B):
        for h in range(H):
            num, den, kap, sc, scs = _head_quadratic(q[b, h], k[b, h], vop[b, h], a[b, h], order, rows)
            out["num"][b, h] = num
            out["den"][b, h] = den
            out["kappa"][b, h] = kap
            out["scale"][b, h] = sc
            out["scale_state"][b, h] = scs
    with np.errstate(divide="ignore", invalid="ignore"):
        out["y"] = out["num"] / out["den"][..., None]
    return out


def forward_ref(q, k, v, dt_proj, dt_bias, A_log, order, rows=None):
    """End-to-end forward from stored inputs: Algorithm 3 discretisation, then
    the masked quadratic form with V_dt = V * dt as the value operand."""
    dt, a = discretise(dt_proj, dt_bias, A_log)
    vdt = np.asarray(v, dtype=np.float64) * dt[..., None]
    out = forward_quadratic(q, k, vdt, a, order, rows=rows)
    out["dt"] = dt
    out["a"] = a
    return out


def forward_amask_ref(q, k, v, A_proj, dt_proj, order, rows=None):
    """End-to-end forward with the A-mask of Algorithms 4 and 5: a =
    -softplus(A_P), A^CS = cumsum(a); value operand V * softplus(dt_P)
    (Algorithm 4) or plain V when dt_proj is None (Algorithm 5)."""
    dt, a = discretise_amask(A_proj, dt_proj)
    vop = np.asarray(v, dtype=np.float64)
    if dt is not None:
        vop = vop * dt[..., None]
    out = forward_quadratic(q, k, vop, a, order, rows=rows)
    out["dt"] = dt
    out["a"] = a
    return out


# ---------------------------------------------------------------------------
# Recurrent form -- Algorithm 6 (and the SSM recurrence h_t = A_t h_{t-1} + B_t x_t)
# ---------------------------------------------------------------------------

def recurrent_step(S, z, q, k, vop, a, order):
    """One recurrence step for a batch of heads (leading dims broadcast).

    S: [..., D, d_v] numerator state (H_up); z: [..., D] normaliser state
    (H_down); q, k: [..., d_h]; vop: [..., d_v]; a: [...] log-decay of this step.
    S <- e^a S + phi(k) vop^T ; z <- e^a z + phi(k) ; y = phi(q)^T S / phi(q)^T z.
    Returns (S, z, y, den).
    """
    alpha = np.exp(np.asarray(a, dtype=np.float64))
    fk = features(k, order)
    fq = features(q, order)
    S = alpha[..., None, None] * S + fk[..., :, None] * np.asarray(vop, dtype=np.float64)[..., None, :]
    z = alpha[..., None] * z + fk
    num = np.einsum("...d,...dv->...v", fq, S)
    den = np.einsum("...d,...d->...", fq, z)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = num / den[..., None]
    return S, z, y, den


def forward_recurrent(q, k, vop, a, order, S0=None, z0=None):
    """Token-by-token recurrence over [B,H,N,.] arrays from a zero state.

    Returns (y [B,H,N,d_v], den [B,H,N], S_N [B,H,D,d_v], z_N [B,H,D]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vop = np.asarray(vop, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    B, H, N, d = q.shape
    dv = vop.shape[-1]
    D = d ** order
    S = np.zeros((B, H, D, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    z = np.zeros((B, H, D)) if z0 is None else np.array(z0, dtype=np.float64)
    y = np.empty((B, H, N, dv))
    den = np.empty((B, H, N))
    for t in range(N):
        S, z, y[:, :, t], den[:, :, t] = recurrent_step(S, z, q[:, :, t], k[:, :, t], vop[:, :, t],
                                                        a[:, :, t], order)
    return y, den, S, z


def final_state_closed_form(k, vop, a, order, S0=None, z0=None, block=2048):
    """The states after the last token, from the recurrence unrolled
    (Algorithm 6: each step decays the states by e^{a_t} and adds phi(k_t)
    vop_t^T, phi(k_t)):
        S_N = e^{A^CS_N} S0 + sum_j e^{A^CS_N - A^CS_j} phi(k_j) vop_j^T,
        z_N = e^{A^CS_N} z0 + sum_j e^{A^CS_N - A^CS_j} phi(k_j),
    with A^CS the inclusive cumsum of a (so the decay from token j to the end
    applies a_{j+1} .. a_N).  Over [B,H,N,.] arrays; the sum is taken over
    blocks of tokens (phi(k) of one block at a time).
    Returns (S_N [B,H,D,d_v], z_N [B,H,D])."""
    k = np.asarray(k, dtype=np.float64)
    vop = np.asarray(vop, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    B, H, N, d = k.shape
    D = d ** order
    cs = np.cumsum(a, axis=-1)
    tot = cs[..., -1] if N else np.zeros((B, H))
    S = np.zeros((B, H, D, vop.shape[-1])) if S0 is None else np.exp(tot)[..., None, None] * S0
    z = np.zeros((B, H, D)) if z0 is None else np.exp(tot)[..., None] * z0
    for b in range(B):
        for h in range(H):
            for j0 in range(0, N, block):
                sl = slice(j0, j0 + block)
                w = np.exp(tot[b, h] - cs[b, h, sl])
                fk = features(k[b, h, sl], order) * w[:, None]
                S[b, h] += fk.T @ vop[b, h, sl]
                z[b, h] += fk.sum(axis=0)
    return S, z


def decode_step_ref(state, norm_state, q, k, v, dt_proj, dt_bias, A_log, order):
    """One decode step for S sequences x H heads (what ssd_decode_step computes).

    state [S,H,D,d_h], norm_state [S,H,D]; q, k, v [S,H,d_h]; dt_proj [S,H];
    dt_bias, A_log [H].  dt = softplus(dt_P + dt_bias), a = -exp(A_log) dt,
    value operand v * dt.  Returns (y [S,H,d_h], new_state, new_norm, den).
    """
    dt_proj = np.asarray(dt_proj, dtype=np.float64)
    dt = softplus(dt_proj + np.asarray(dt_bias, dtype=np.float64)[None, :])
    a = -np.exp(np.asarray(A_log, dtype=np.float64))[None, :] * dt
    vop = np.asarray(v, dtype=np.float64) * dt[..., None]
    S, z, y, den = recurrent_step(state, norm_state, q, k, vop, a, order)
    return y, S, z, den


def decode_step_amask_ref(state, norm_state, q, k, v, A_proj, dt_proj, order):
    """One decode step with the A-mask, as Algorithm 6 prints it: the step's
    decay factor is exp(-softplus(h W_A)) per sequence and head, with no dt in
    it; the value operand is v * softplus(dt_P) (Algorithm 4's dt, no bias) or
    plain v when dt_proj is None (Algorithm 6 and Algorithm 5 use v itself).

    state [S,H,D,d_h], norm_state [S,H,D]; q, k, v [S,H,d_h]; A_proj, dt_proj
    [S,H].  Returns (y [S,H,d_h], new_state, new_norm, den).
    """
    dt, a = discretise_amask(A_proj, dt_proj)
    vop = np.asarray(v, dtype=np.float64)
    if dt is not None:
        vop = vop * dt[..., None]
    S, z, y, den = recurrent_step(state, norm_state, q, k, vop, a, order)
    return y, S, z, den


# ---------------------------------------------------------------------------
# The short convolution of Algorithm 6 (window 2), one decode step
#
# Algorithm 6 forms q^c_t, k^c_t, v^c_t = conv_1d(q_t, k_t, v_t, q_{t-1},
# k_{t-1}, v_{t-1}, window_size = 2) before the order-2 features.  The pages
# do not spell conv_1d out; read here as the depthwise causal convolution of
# the q, k, v channels that Algorithms 3-5 apply over the whole sequence
# (d_conv = 3 d_ssm channels, Algorithm 2), restricted to one step: per
# channel, x^c_t = w0 x_{t-1} + w1 x_t (+ a bias), with x_{-1} = 0.
# Algorithm 6 applies no activation after it; Algorithm 3 applies sigma
# (SiLU), offered as an option.
# ---------------------------------------------------------------------------

def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def conv_window2(x, x_prev, w, b=None, act=None):
    """One step of the window-2 depthwise convolution: x^c = w[..., 0] x_prev
    + w[..., 1] x (+ b), then SiLU if act == "silu".  x, x_prev: [..., C];
    w: [C, 2] (broadcast over the leading dims); b: [C] or None."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = w[..., 0] * np.asarray(x_prev, dtype=np.float64) + w[..., 1] * x
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    if act == "silu":
        y = silu(y)
    elif act is not None:
        raise ValueError("act must be None or 'silu'")
    return y


def decode_step_conv_ref(state, norm_state, conv_state, q, k, v, conv_w, conv_b, act, order,
                         A_proj=None, dt_proj=None, dt_bias=None, A_log=None):
    """One decode step of Algorithm 6 with its window-2 convolution.

    conv_state [S,3,H,d_h]: the previous step's raw q, k, v (zero before the
    first token); conv_w [3,H,d_h,2], conv_b [3,H,d_h] or None; q, k, v
    [S,H,d_h] this step's raw projections.  The convolved q^c, k^c, v^c then
    go through the step: with A_proj given, the A-mask as Algorithm 6 prints
    it (decode_step_amask_ref: a_t = exp(-softplus(A_P)), value v^c, or v^c
    softplus(dt_P) with dt_proj); else the Mamba-2 discretisation
    (decode_step_ref with dt_proj, dt_bias, A_log).
    Returns (y, new_state, new_norm, new_conv_state, den); the new conv state
    holds this step's raw q, k, v."""
    cs = np.asarray(conv_state, dtype=np.float64)
    b = [None] * 3 if conv_b is None else [conv_b[i] for i in range(3)]
    qc, kc, vc = (conv_window2(x, cs[:, i], conv_w[i], b[i], act) for i, x in enumerate((q, k, v)))
    if A_proj is not None:
        y, S, z, den = decode_step_amask_ref(state, norm_state, qc, kc, vc, A_proj, dt_proj, order)
    else:
        y, S, z, den = decode_step_ref(state, norm_state, qc, kc, vc, dt_proj, dt_bias, A_log, order)
    new_cs = np.stack([np.asarray(x, dtype=np.float64) for x in (q, k, v)], axis=1)
    return y, S, z, new_cs, den


# ---------------------------------------------------------------------------
# Symmetric packing of the order-2 state (derived from Algorithm 6)
#
# The order-2 feature k (x) k is symmetric in its two indices, so every state
# row (a, b) equals row (b, a).  The packed layout keeps the rows a <= b only,
# D' = d_h (d_h + 1) / 2 of them, in row-major order of the upper triangle; a
# query's contraction phi(q)^T S then counts each off-diagonal row twice.
# This layout is not on the pages; it is the same state, stored once.
# ---------------------------------------------------------------------------

def packed_pairs(d):
    """The pairs (a, b), a <= b, in packed row order: row p(a, b) = a d -
    a (a - 1) / 2 + (b - a)."""
    return [(a, b) for a in range(d) for b in range(a, d)]


def _pair_rows(d):
    pairs = packed_pairs(d)
    upper = np.array([a * d + b for a, b in pairs])   # full row (a, b)
    lower = np.array([b * d + a for a, b in pairs])   # full row (b, a)
    return pairs, upper, lower


def pack_state(state, norm_state, d):
    """Full order-2 states [.., d^2, d_v], [.., d^2] -> packed [.., D', d_v],
    [.., D'].  Each packed row is the mean of the full rows (a, b) and (b, a):
    the symmetric part, which is all that phi(q)^T S and phi(q)^T z read, and
    the rows themselves when the state is symmetric."""
    _, up, lo = _pair_rows(d)
    S = np.asarray(state, dtype=np.float64)
    z = np.asarray(norm_state, dtype=np.float64)
    return (S[..., up, :] + S[..., lo, :]) / 2.0, (z[..., up] + z[..., lo]) / 2.0


def unpack_state(state_p, norm_p, d):
    """Packed [.., D', d_v], [.., D'] -> full [.., d^2, d_v], [.., d^2]: rows
    (a, b) and (b, a) both take packed row p(min, max)."""
    pairs = packed_pairs(d)
    index = np.empty(d * d, dtype=np.int64)
    for p, (a, b) in enumerate(pairs):
        index[a * d + b] = p
        index[b * d + a] = p
    Sp = np.asarray(state_p, dtype=np.float64)
    zp = np.asarray(norm_p, dtype=np.float64)
    return Sp[..., index, :], zp[..., index]


def packed_features(x, weighted):
    """x_a x_b over the packed pairs; with weighted, the off-diagonal pairs
    count twice (the query side of phi(q)^T S over the packed rows)."""
    x = np.asarray(x, dtype=np.float64)
    pairs = packed_pairs(x.shape[-1])
    ia = np.array([a for a, _ in pairs])
    ib = np.array([b for _, b in pairs])
    f = x[..., ia] * x[..., ib]
    if weighted:
        f = f * np.where(ia == ib, 1.0, 2.0)
    return f


def recurrent_step_packed(state_p, norm_p, q, k, vop, a):
    """recurrent_step at order 2 on packed states: S' <- e^a S' + k_a k_b
    vop^T, z' <- e^a z' + k_a k_b over the pairs a <= b; y = sum_p w_p q_a q_b
    S'_p / sum_p w_p q_a q_b z'_p with w_p = 1 on the diagonal, 2 off it.
    Returns (S', z', y, den)."""
    alpha = np.exp(np.asarray(a, dtype=np.float64))
    fk = packed_features(k, False)
    fq = packed_features(q, True)
    Sp = alpha[..., None, None] * state_p + fk[..., :, None] * np.asarray(vop, dtype=np.float64)[..., None, :]
    zp = alpha[..., None] * norm_p + fk
    num = np.einsum("...d,...dv->...v", fq, Sp)
    den = np.einsum("...d,...d->...", fq, zp)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = num / den[..., None]
    return Sp, zp, y, den


def decode_step_packed_ref(state_p, norm_p, q, k, v, dt_proj, dt_bias, A_log):
    """decode_step_ref at order 2 on packed states (same discretisation)."""
    dt_proj = np.asarray(dt_proj, dtype=np.float64)
    dt = softplus(dt_proj + np.asarray(dt_bias, dtype=np.float64)[None, :])
    a = -np.exp(np.asarray(A_log, dtype=np.float64))[None, :] * dt
    vop = np.asarray(v, dtype=np.float64) * dt[..., None]
    Sp, zp, y, den = recurrent_step_packed(state_p, norm_p, q, k, vop, a)
    return y, Sp, zp, den


def decode_step_amask_packed_ref(state_p, norm_p, q, k, v, A_proj, dt_proj):
    """decode_step_amask_ref at order 2 on packed states."""
    dt, a = discretise_amask(A_proj, dt_proj)
    vop = np.asarray(v, dtype=np.float64)
    if dt is not None:
        vop = vop * dt[..., None]
    Sp, zp, y, den = recurrent_step_packed(state_p, norm_p, q, k, vop, a)
    return y, Sp, zp, den


# ---------------------------------------------------------------------------
# Backward pass (gradients of the forward definitions above; the pages train
# these models, but print no backward pass: this is the chain rule applied to
# the quadratic form and the Algorithm 3 discretisation, step by step)
# ---------------------------------------------------------------------------

def _head_backward(q, k, vop, a, order, dy):
    """One head.  Forward: s = q k^T, W = s^p * D with D_ij = exp(cs_i - cs_j)
    (j <= i), cs = cumsum(a); num = W vop, den = W 1, y = num / den.
    Returns dq, dk, dvop, da for the upstream gradient dy."""
    cs = np.cumsum(a)
    s = q @ k.T
    causal = np.tril(np.ones(s.shape, dtype=bool))
    D = np.exp(np.where(causal, cs[:, None] - cs[None, :], -np.inf))
    W = s ** order * D
    num = W @ vop
    den = W.sum(axis=1)
    y = num / den[:, None]
    # y = num / den
    dnum = dy / den[:, None]
    dden = -(dy * y).sum(axis=1) / den
    # num = W vop, den = W 1
    dW = (dnum @ vop.T + dden[:, None]) * causal
    dvop = W.T @ dnum
    # W = s^p D
    ds = dW * D * order * s ** (order - 1)
    dq = ds @ k
    dk = ds.T @ q
    # D_ij = exp(cs_i - cs_j): d/dcs_i = +W_ij, d/dcs_j = -W_ij
    P = dW * W
    dcs = P.sum(axis=1) - P.sum(axis=0)
    # cs = cumsum(a): da_t = sum_{s >= t} dcs_s
    da = np.cumsum(dcs[::-1])[::-1]
    return dq, dk, dvop, da


def _head_backward_scale(q, k, vop, a, order, dy):
    """Per-element first-order rounding bounds of the gradients of one head,
    divided by the unit roundoff: every gradient is a sum of products, and a
    floating-point evaluation with relative accuracy eps in each of its terms
    is off by at most about eps times the sum of the terms' absolute values
    (with dnum and dden taken at their own bounds).
    Returns the scales of dq, dk, dvop, da (the parity metric of the backward
    tests, as the forward's `scale`)."""
    cs = np.cumsum(a)
    s = q @ k.T
    causal = np.tril(np.ones(s.shape, dtype=bool))
    D = np.exp(np.where(causal, cs[:, None] - cs[None, :], -np.inf))
    W = s ** order * D
    num = W @ vop
    den = W.sum(axis=1)
    y = num / den[:, None]
    # dnum = dy / den and dden = -dy . y / den inherit the rounding of the
    # normaliser and of y, amplified by the normaliser's condition kappa =
    # sum|W| / |den| (the forward's error scale of y covers the latter)
    aW = np.abs(W)
    kappa = aW.sum(axis=1) / np.abs(den)
    yscale = (aW @ np.abs(vop) + np.abs(y) * aW.sum(axis=1)[:, None]) / np.abs(den)[:, None]
    amp = (1.0 + kappa)[:, None]
    adn = np.abs(dy) / np.abs(den)[:, None] * amp
    add = (np.abs(dy) * (np.abs(y) + yscale)).sum(axis=1) / np.abs(den) * amp[:, 0]
    adW = (adn @ np.abs(vop).T + add[:, None]) * causal
    ads = adW * D * order * np.abs(s) ** (order - 1)
    aP = adW * aW
    dcs = aP.sum(axis=1) + aP.sum(axis=0)
    return ads @ np.abs(k), ads.T @ np.abs(q), aW.T @ adn, np.cumsum(dcs[::-1])[::-1]


def backward_error_scale(q, k, vop, a, order, dy):
    """backward_quadratic's per-element error scales over [B,H,N,.] arrays:
    dict dq, dk, dvop, da (see _head_backward_scale)."""
    q, k, vop, a, dy = (np.asarray(x, dtype=np.float64) for x in (q, k, vop, a, dy))
    B, H = q.shape[:2]
    out = {"dq": np.empty_like(q), "dk": np.empty_like(k), "dvop": np.empty_like(vop), "da": np.empty_like(a)}
    for b in range(B):
        for h in range(H):
            r = _head_backward_scale(q[b, h], k[b, h], vop[b, h], a[b, h], order, dy[b, h])
            for name, x in zip(("dq", "dk", "dvop", "da"), r):
                out[name][b, h] = x
    return out


def backward_quadratic(q, k, vop, a, order, dy):
    """Gradients of the masked quadratic form (forward_quadratic's y) with
    respect to its operands, over [B,H,N,.] arrays, for upstream gradient dy
    [B,H,N,d_v].  Returns dict dq, dk, dvop, da (da: per-token log-decay)."""
    q, k, vop, a, dy = (np.asarray(x, dtype=np.float64) for x in (q, k, vop, a, dy))
    B, H = q.shape[:2]
    out = {"dq": np.empty_like(q), "dk": np.empty_like(k), "dvop": np.empty_like(vop), "da": np.empty_like(a)}
    for b in range(B):
        for h in range(H):
            r = _head_backward(q[b, h], k[b, h], vop[b, h], a[b, h], order, dy[b, h])
            for name, x in zip(("dq", "dk", "dvop", "da"), r):
                out[name][b, h] = x
    return out


def prep_backward_ref(dt_proj, dt_bias, A_log, da, ddt):
    """Chain rule through Algorithm 3's discretisation: a = A dt with A =
    -exp(A_log), dt = softplus(dt_P + dt_bias).  da: gradient w.r.t. a
    [B,H,N]; ddt: gradient w.r.t. dt from other uses (the value operand
    v * dt), [B,H,N].  Returns d_dt_proj [B,H,N], d_dt_bias [H], d_A_log [H]."""
    dt_proj = np.asarray(dt_proj, dtype=np.float64)
    x = dt_proj + np.asarray(dt_bias, dtype=np.float64)[:, None]
    A = -np.exp(np.asarray(A_log, dtype=np.float64))
    dt = softplus(x)
    da = np.asarray(da, dtype=np.float64)
    g_dt = np.asarray(ddt, dtype=np.float64) + da * A[:, None]
    sig = 1.0 / (1.0 + np.exp(-x))  # softplus' = logistic
    d_dt_proj = g_dt * sig
    d_dt_bias = d_dt_proj.sum(axis=(0, 2))
    d_A_log = (da * dt).sum(axis=(0, 2)) * A  # dA/dA_log = A
    return d_dt_proj, d_dt_bias, d_A_log


def prep_amask_backward_ref(A_proj, dt_proj, da, ddt):
    """Chain rule through the A-mask of Algorithms 4 and 5: a = -softplus(A_P),
    dt = softplus(dt_P).  Returns d_A_proj and d_dt_proj (None without
    dt_proj)."""
    A_proj = np.asarray(A_proj, dtype=np.float64)
    d_A = -np.asarray(da, dtype=np.float64) / (1.0 + np.exp(-A_proj))
    if dt_proj is None:
        return d_A, None
    dt_proj = np.asarray(dt_proj, dtype=np.float64)
    return d_A, np.asarray(ddt, dtype=np.float64) / (1.0 + np.exp(-dt_proj))


def backward_ref(q, k, v, dt_proj, dt_bias, A_log, order, dy):
    """End-to-end gradients of forward_ref's y: dq, dk, dv, and through the
    discretisation d_dt_proj, d_dt_bias, d_A_log; also the intermediate
    gradients da (w.r.t. a = A dt) and ddt_v (w.r.t. dt through V * dt)."""
    dt, a = discretise(dt_proj, dt_bias, A_log)
    v = np.asarray(v, dtype=np.float64)
    vdt = v * dt[..., None]
    g = backward_quadratic(q, k, vdt, a, order, dy)
    dv = g["dvop"] * dt[..., None]
    ddt_v = (g["dvop"] * v).sum(axis=-1)
    d_dt_proj, d_dt_bias, d_A_log = prep_backward_ref(dt_proj, dt_bias, A_log, g["da"], ddt_v)
    return {"dq": g["dq"], "dk": g["dk"], "dv": dv, "da": g["da"], "ddt_v": ddt_v,
            "d_dt_proj": d_dt_proj, "d_dt_bias": d_dt_bias, "d_A_log": d_A_log}
