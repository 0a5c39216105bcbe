"""Pins for the CPU fp64 oracle, against facts other than the oracle itself.

Each test names the passage of 2Mamba2Furious (Mongaras & Larson) it checks.
The pins are chosen so that a plausible slip in the oracle -- a dropped
diagonal term, an exclusive instead of inclusive cumsum, a sign flip in the
decay, q and k swapped, the power applied to the normaliser only, V instead of
V*dt -- fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import ssd_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def frac(s):
    return float(Fraction(s))


def fracs(x):
    if isinstance(x, list):
        return [fracs(e) for e in x]
    return frac(x)


def rand_case(rng, B, H, N, d, dv=None, a_scale=1.0, signed=True):
    dv = d if dv is None else dv
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d))
    if not signed:
        q, k = np.abs(q), np.abs(k)
    v = rng.standard_normal((B, H, N, dv))
    a = -a_scale * rng.uniform(0.0, 1.0, (B, H, N))
    return q, k, v, a


def rel_err(x, y, scale):
    return np.max(np.abs(x - y) / scale)


# ---------------------------------------------------------------------------
# Hand-worked fixtures (tests/golden/hand_worked.json)
# ---------------------------------------------------------------------------

def load_golden():
    with open(GOLDEN) as f:
        return {c["name"]: c for c in json.load(f)["cases"]}


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("name", ["kernel_level_dh1", "order2_state_dh2", "signed_dh1", "signed_dh2_state_scale"])
def test_golden_kernel_level(name, order):
    """Algorithms 1, 4, 5 on exact hand-worked values (inclusive A^CS).  Where
    the fixture gives them, also the parity metric's error scale and the
    normaliser's condition, worked by hand from their definitions: any factor
    other than 1 in either (a scale twice or half as large, a dropped term, a
    missing absolute value on the signed case) fails here."""
    c = load_golden()[name]
    q = np.array(c["q"], float)[None, None]
    k = np.array(c["k"], float)[None, None]
    vop = np.array(c["vop"], float)[None, None]
    a = np.log(np.array(c["exp_a"], float))[None, None]
    exp = c["expected"][str(order)]
    out = O.forward_quadratic(q, k, vop, a, order)
    np.testing.assert_allclose(out["y"][0, 0], fracs(exp["y"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(out["den"][0, 0], fracs(exp["den"]), rtol=1e-14)
    if "scale" in exp:
        np.testing.assert_allclose(out["scale"][0, 0], fracs(exp["scale"]), rtol=1e-14)
        np.testing.assert_allclose(out["kappa"][0, 0], fracs(exp["kappa"]), rtol=1e-14)
        # the sampled-row evaluation gives the same diagnostics
        rows = O.forward_quadratic(q, k, vop, a, order, rows=np.arange(q.shape[2]))
        np.testing.assert_allclose(rows["scale"][0, 0], fracs(exp["scale"]), rtol=1e-14)
        np.testing.assert_allclose(rows["kappa"][0, 0], fracs(exp["kappa"]), rtol=1e-14)
    if "scale_state" in exp:
        for o in (out, O.forward_quadratic(q, k, vop, a, order, rows=np.arange(q.shape[2]))):
            np.testing.assert_allclose(o["scale_state"][0, 0], fracs(exp["scale_state"]), rtol=1e-14)
    if q.shape[-1] == 1 or (np.all(q >= 0) and np.all(k >= 0)):
        # no feature product can cancel: the state form's scale is the scale
        np.testing.assert_allclose(out["scale_state"], out["scale"], rtol=1e-14)
    y, den, S, z = O.forward_recurrent(q, k, vop, a, order)
    np.testing.assert_allclose(y[0, 0], fracs(exp["y"]), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(den[0, 0], fracs(exp["den"]), rtol=1e-14)
    if "S_final" in exp:
        np.testing.assert_allclose(S[0, 0], fracs(exp["S_final"]), rtol=1e-14)
        np.testing.assert_allclose(z[0, 0], fracs(exp["z_final"]), rtol=1e-14)


@pytest.mark.parametrize("order", [1, 2])
def test_golden_end_to_end(order):
    """Algorithm 3 discretisation + mixer: dt = softplus(0) = ln 2, e^{A dt} = 1/2."""
    c = load_golden()["end_to_end_dh1_ln2"]
    q = np.array(c["q"], float)[None, None]
    k = np.array(c["k"], float)[None, None]
    v = np.array(c["v"], float)[None, None]
    dtp = np.array(c["dt_proj"], float)[None, None]
    out = O.forward_ref(q, k, v, dtp, np.array(c["dt_bias"]), np.array(c["A_log"]), order)
    exp = c["expected"][str(order)]
    ln2 = math.log(2.0)
    np.testing.assert_allclose(out["y"][0, 0] / ln2, fracs(exp["y_over_ln2"]), rtol=1e-14)
    np.testing.assert_allclose(out["den"][0, 0], fracs(exp["den"]), rtol=1e-14)
    dt, a_cs, a_chunk = O.prep_ref(dtp, np.array(c["dt_bias"]), np.array(c["A_log"]), c["chunk"])
    ep = c["expected_prep"]
    np.testing.assert_allclose(dt[0, 0] / ln2, fracs(ep["dt_over_ln2"]), rtol=1e-15)
    np.testing.assert_allclose(a_cs[0, 0] / ln2, fracs(ep["a_cs_over_ln2"]), rtol=1e-15)
    np.testing.assert_allclose(a_chunk[0, 0] / ln2, fracs(ep["a_chunk_over_ln2"]), rtol=1e-15)


# ---------------------------------------------------------------------------
# Two independent derivations: quadratic form vs token recurrence (Algorithm 6)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (17, 2), (64, 4), (130, 8)])
def test_quadratic_equals_recurrence(order, N, d):
    rng = np.random.default_rng(1000 * N + 10 * d + order)
    # non-negative features at order 1 keep den away from 0 so y is comparable
    q, k, v, a = rand_case(rng, 2, 2, N, d, a_scale=0.5, signed=(order == 2))
    quad = O.forward_quadratic(q, k, v, a, order)
    y, den, S, z = O.forward_recurrent(q, k, v, a, order)
    assert rel_err(quad["y"], y, quad["scale"]) <= 1e-10
    np.testing.assert_allclose(den, quad["den"], rtol=1e-10, atol=1e-12)
    # final state = sum_j exp(A^CS_N - A^CS_j) phi(k_j) v_j^T
    cs = np.cumsum(a, axis=-1)
    w = np.exp(cs[..., -1:] - cs)
    fk = O.features(k, order)
    S_ref = np.einsum("bhn,bhnd,bhnv->bhdv", w, fk, v)
    np.testing.assert_allclose(S, S_ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(z, np.einsum("bhn,bhnd->bhd", w, fk), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("N,block", [(1, 4), (37, 8), (130, 64), (130, 1000)])
def test_final_state_closed_form_equals_recurrence(order, N, block):
    """The unrolled state (a sum over tokens, taken in blocks) equals the
    token-by-token recurrence of Algorithm 6, from zero and from an initial
    state."""
    rng = np.random.default_rng(40 + N + order)
    q, k, v, a = rand_case(rng, 2, 2, N, 3, dv=4, a_scale=0.7)
    _, _, S, z = O.forward_recurrent(q, k, v, a, order)
    Sc, zc = O.final_state_closed_form(k, v, a, order, block=block)
    np.testing.assert_allclose(Sc, S, rtol=1e-11, atol=1e-12 * np.abs(S).max())
    np.testing.assert_allclose(zc, z, rtol=1e-11, atol=1e-12 * np.abs(z).max())
    S0 = rng.standard_normal(S.shape)
    z0 = rng.standard_normal(z.shape)
    _, _, S, z = O.forward_recurrent(q, k, v, a, order, S0=S0, z0=z0)
    Sc, zc = O.final_state_closed_form(k, v, a, order, S0=S0, z0=z0, block=block)
    np.testing.assert_allclose(Sc, S, rtol=1e-11, atol=1e-12 * np.abs(S).max())
    np.testing.assert_allclose(zc, z, rtol=1e-11, atol=1e-12 * np.abs(z).max())


@pytest.mark.parametrize("order", [1, 2])
def test_sampled_rows_equal_full(order):
    """The sampled-row evaluation (rows taken in batches) equals the full
    quadratic form on those rows: a few rows, and more rows than one batch in
    an unsorted order."""
    rng = np.random.default_rng(7)
    q, k, v, a = rand_case(rng, 1, 2, 300, 4)
    full = O.forward_quadratic(q, k, v, a, order)
    for rows in (np.array([0, 1, 63, 64, 65, 299]), rng.permutation(300)[:200]):
        part = O.forward_quadratic(q, k, v, a, order, rows=rows)
        for key in ("y", "den", "scale", "kappa"):
            np.testing.assert_allclose(part[key], full[key][:, :, rows], rtol=1e-12)


# ---------------------------------------------------------------------------
# Closed forms and special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", [1, 2])
def test_single_token(order):
    """N = 1: the only weight is on the diagonal, so y_0 = value_0 exactly."""
    rng = np.random.default_rng(3)
    q, k, v, a = rand_case(rng, 1, 3, 1, 5)
    out = O.forward_quadratic(q, k, v, a, order)
    np.testing.assert_allclose(out["y"], v, rtol=1e-15)


@pytest.mark.parametrize("order", [1, 2])
def test_two_tokens_closed_form(order):
    """N = 2: y_1 = (g10 e^{a_1} v_0 + g11 v_1) / (g10 e^{a_1} + g11), g_ij = (q_i.k_j)^p."""
    rng = np.random.default_rng(4)
    q, k, v, a = rand_case(rng, 1, 1, 2, 3, signed=False)
    out = O.forward_quadratic(q, k, v, a, order)
    g10 = float(q[0, 0, 1] @ k[0, 0, 0]) ** order
    g11 = float(q[0, 0, 1] @ k[0, 0, 1]) ** order
    e1 = math.exp(a[0, 0, 1])
    y1 = (g10 * e1 * v[0, 0, 0] + g11 * v[0, 0, 1]) / (g10 * e1 + g11)
    np.testing.assert_allclose(out["y"][0, 0, 1], y1, rtol=1e-13)


@pytest.mark.parametrize("order", [1, 2])
def test_full_decay_is_identity(order):
    """A_log = 25 => a ~ -7e10 dt: every off-diagonal decay underflows, mask = I, y = V dt."""
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 40, 4
    q = np.abs(rng.standard_normal((B, H, N, d))) + 0.1
    k = np.abs(rng.standard_normal((B, H, N, d))) + 0.1
    v = rng.standard_normal((B, H, N, d))
    dtp = rng.standard_normal((B, H, N))
    out = O.forward_ref(q, k, v, dtp, np.zeros(H), np.full(H, 25.0), order)
    np.testing.assert_allclose(out["y"], v * out["dt"][..., None], rtol=1e-14)


@pytest.mark.parametrize("order", [1, 2])
def test_no_decay_is_causal_linear_attention(order):
    """A^CS = 0: plain causal linear attention (Algorithm 1 with causal M), computed
    independently with running prefix sums of phi(k) v^T and phi(k) ("Transformers
    are RNNs" style), using numpy's cumsum."""
    rng = np.random.default_rng(6)
    B, H, N, d = 2, 2, 50, 3
    q = np.abs(rng.standard_normal((B, H, N, d)))
    k = np.abs(rng.standard_normal((B, H, N, d)))
    v = rng.standard_normal((B, H, N, d))
    a = np.zeros((B, H, N))
    out = O.forward_quadratic(q, k, v, a, order)
    if order == 1:
        fq, fk = q, k
    else:
        fq = np.stack([q[..., i] * q[..., j] for i in range(d) for j in range(d)], axis=-1)
        fk = np.stack([k[..., i] * k[..., j] for i in range(d) for j in range(d)], axis=-1)
    KV = np.cumsum(fk[..., :, None] * v[..., None, :], axis=2)
    Ks = np.cumsum(fk, axis=2)
    num = np.einsum("bhnd,bhndv->bhnv", fq, KV)
    den = np.einsum("bhnd,bhnd->bhn", fq, Ks)
    np.testing.assert_allclose(out["y"], num / den[..., None], rtol=1e-11)
    # end to end the same holds when dt_P is very negative: dt -> e^{dt_P}, a -> 0
    dtp = np.full((B, H, N), -40.0)
    e2e = O.forward_ref(q, k, v, dtp, np.zeros(H), np.zeros(H), order)
    assert np.all(np.abs(e2e["a"]) < 1e-16)
    np.testing.assert_allclose(e2e["y"], num / den[..., None] * e2e["dt"][..., None], rtol=1e-11)


@pytest.mark.parametrize("order", [1, 2])
def test_constant_value_operand(order):
    """A constant value operand c gives y = c on every row whose normaliser is nonzero."""
    rng = np.random.default_rng(8)
    q, k, _, a = rand_case(rng, 1, 2, 70, 4, signed=False)
    c = np.array([1.5, -2.0, 0.25, 7.0])
    v = np.broadcast_to(c, q.shape)
    out = O.forward_quadratic(q, k, v, a, order)
    np.testing.assert_allclose(out["y"], np.broadcast_to(c, out["y"].shape), rtol=1e-13)


@pytest.mark.parametrize("order", [1, 2])
def test_homogeneity_and_affine_values(order):
    """y(alpha Q, beta K, lam V + mu) = lam y(Q, K, V) + mu."""
    rng = np.random.default_rng(9)
    q, k, v, a = rand_case(rng, 1, 2, 33, 3, signed=False)
    base = O.forward_quadratic(q, k, v, a, order)
    alt = O.forward_quadratic(-2.5 * q, 0.3 * k, 4.0 * v + 1.25, a, order)
    # the factor (alpha beta)^p, of either sign, cancels between numerator and normaliser
    np.testing.assert_allclose(alt["y"], 4.0 * base["y"] + 1.25, rtol=1e-11, atol=1e-11)


def test_order2_is_order1_on_flattened_features():
    """(q.k)^2 = vec(q q^T).vec(k k^T): order 2 equals order 1 on D = d^2 features."""
    rng = np.random.default_rng(10)
    q, k, v, a = rand_case(rng, 1, 2, 45, 3)
    o2 = O.forward_quadratic(q, k, v, a, 2)
    fq = np.einsum("bhni,bhnj->bhnij", q, q).reshape(q.shape[:-1] + (9,))
    fk = np.einsum("bhni,bhnj->bhnij", k, k).reshape(k.shape[:-1] + (9,))
    o1 = O.forward_quadratic(fq, fk, v, a, 1)
    np.testing.assert_allclose(o2["y"], o1["y"], rtol=1e-11)
    np.testing.assert_allclose(o2["den"], o1["den"], rtol=1e-11)


@pytest.mark.parametrize("order", [1, 2])
def test_prefix_consistency(order):
    """Causality: the first n outputs do not depend on later tokens."""
    rng = np.random.default_rng(11)
    q, k, v, a = rand_case(rng, 1, 1, 140, 4, signed=False)
    full = O.forward_quadratic(q, k, v, a, order)
    for n in (1, 63, 64, 65, 127, 128, 129):
        part = O.forward_quadratic(q[:, :, :n], k[:, :, :n], v[:, :, :n], a[:, :, :n], order)
        np.testing.assert_allclose(part["y"], full["y"][:, :, :n], rtol=1e-12)


def test_order2_weights_nonnegative_and_decays_bounded():
    rng = np.random.default_rng(12)
    q, k, v, a = rand_case(rng, 1, 2, 90, 4, a_scale=3.0)
    out = O.forward_quadratic(q, k, v, a, 2)
    assert np.all(out["den"] > 0)
    np.testing.assert_allclose(out["kappa"], 1.0, rtol=1e-12)
    dt, a2 = O.discretise(rng.standard_normal((1, 2, 90)), np.array([-1.0, 2.0]), np.array([0.3, 2.7]))
    cs = np.cumsum(a2, axis=-1)
    diff = cs[..., :, None] - cs[..., None, :]
    kept = np.broadcast_to(np.tril(np.ones((90, 90), bool)), diff.shape)
    assert np.all(diff[kept] <= 0.0)  # masked exponents never positive: no overflow
    dec = np.exp(diff[kept])
    assert np.all(dec >= 0.0) and np.all(dec <= 1.0)
    assert np.all(dt > 0) and np.all(a2 < 0)


# ---------------------------------------------------------------------------
# Discretisation (Algorithms 2, 3)
# ---------------------------------------------------------------------------

def test_softplus_matches_library_logaddexp():
    x = np.concatenate([np.linspace(-50, 50, 2001), [-745.0, -700.0, 700.0, 0.0]])
    np.testing.assert_allclose(O.softplus(x), np.logaddexp(0.0, x), rtol=1e-15, atol=0)


def test_softplus_inverse_of_dt_bias_init():
    """Algorithm 2: dt_bias = dt_init + log(1 - exp(-dt_init)) inverts softplus."""
    dt_init = np.exp(np.linspace(math.log(1e-3), math.log(1e-1), 101))
    dt_bias = dt_init + np.log(-np.expm1(-dt_init))
    np.testing.assert_allclose(O.softplus(dt_bias), dt_init, rtol=1e-13)


def test_prep_chunks_reconstruct_global_cumsum():
    """Chunk-local inclusive cumsums plus the preceding chunk totals give
    cumsum(A*dt) over the whole sequence, for any chunk size (incl. ragged tails)."""
    rng = np.random.default_rng(13)
    B, H, N = 2, 3, 301
    dtp = rng.standard_normal((B, H, N))
    bias = rng.standard_normal(H)
    alog = np.log(rng.uniform(1, 16, H))
    dt, a = O.discretise(dtp, bias, alog)
    ref = np.cumsum(-np.exp(alog)[:, None] * np.logaddexp(0.0, dtp + bias[:, None]), axis=-1)
    for chunk in (1, 7, 64, 128, 301, 512):
        dt2, cs, tot = O.prep_ref(dtp, bias, alog, chunk)
        np.testing.assert_allclose(dt2, np.logaddexp(0.0, dtp + bias[:, None]), rtol=1e-14)
        offs = np.concatenate([np.zeros((B, H, 1)), np.cumsum(tot, axis=-1)[..., :-1]], axis=-1)
        glob = cs + np.repeat(offs, chunk, axis=-1)[..., :N]
        np.testing.assert_allclose(glob, ref, rtol=1e-12)
        assert tot.shape[-1] == -(-N // chunk)


# ---------------------------------------------------------------------------
# Decode step (Algorithm 6) against the forward form
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", [1, 2])
def test_decode_steps_equal_forward(order):
    rng = np.random.default_rng(14)
    S, H, T, d = 3, 2, 20, 3
    A_log = np.log(rng.uniform(1, 16, H))
    bias = rng.standard_normal(H) - 2.0
    qs = rng.standard_normal((T, S, H, d))
    ks = rng.standard_normal((T, S, H, d))
    vs = rng.standard_normal((T, S, H, d))
    dtps = rng.standard_normal((T, S, H))
    D = d ** order
    st = np.zeros((S, H, D, d))
    nz = np.zeros((S, H, D))
    ys = []
    for t in range(T):
        y, st, nz, _ = O.decode_step_ref(st, nz, qs[t], ks[t], vs[t], dtps[t], bias, A_log, order)
        ys.append(y)
    ys = np.stack(ys, axis=2)  # [S,H,T,d]
    tr = lambda x: np.moveaxis(x, 0, 2)  # [T,S,H,...] -> [S,H,T,...]
    fwd = O.forward_ref(tr(qs), tr(ks), tr(vs), np.moveaxis(dtps, 0, 2), bias, A_log, order)
    assert rel_err(ys, fwd["y"], fwd["scale"]) <= 1e-10


@pytest.mark.parametrize("order", [1, 2])
def test_error_scale_bounds_an_fp32_evaluation(order):
    """The oracle's per-element error scale is the first-order rounding bound of
    y = num/den: an fp32 evaluation of the same quadratic form (signed features,
    so order-1 normalisers nearly cancel on some rows) stays within a small
    multiple of fp32's unit roundoff times that scale on every element."""
    rng = np.random.default_rng(15)
    q, k, v, a = rand_case(rng, 1, 2, 160, 8, a_scale=0.3)
    ref = O.forward_quadratic(q, k, v, a, order)
    q32, k32, v32 = (x.astype(np.float32) for x in (q, k, v))
    cs = np.cumsum(a, axis=-1).astype(np.float32)
    y32 = np.empty_like(v32)
    for h in range(2):
        G = (q32[0, h] @ k32[0, h].T) ** order
        D = np.exp(np.where(np.tril(np.ones((160, 160), bool)), cs[0, h][:, None] - cs[0, h][None, :],
                            -np.inf)).astype(np.float32)
        W = (G * D).astype(np.float32)
        y32[0, h] = (W @ v32[0, h]) / W.sum(axis=1, dtype=np.float32)[:, None]
    err = np.abs(y32 - ref["y"]) / ref["scale"]
    assert err.max() <= 1e-5
    if order == 1:
        assert ref["kappa"].max() > 50  # the case really contains ill-conditioned rows


@pytest.mark.parametrize("order", [1, 2])
def test_state_scale_bounds_an_fp32_recurrent_evaluation(order):
    """An fp32 evaluation through Algorithm 6's states (S, z updated token by
    token, y = phi(q)^T S / phi(q)^T z, every operation rounded to fp32)
    stays within a small multiple of fp32's unit roundoff times scale_state on
    every element (scale_state >= scale everywhere; the hand-worked fixture
    signed_dh2_state_scale pins its value)."""
    rng = np.random.default_rng(16)
    q, k, v, a = rand_case(rng, 1, 2, 120, 6, a_scale=0.3)
    ref = O.forward_quadratic(q, k, v, a, order)
    D = 6 ** order
    S = np.zeros((2, D, 6), np.float32)
    z = np.zeros((2, D), np.float32)
    y32 = np.empty((2, 120, 6))
    for t in range(120):
        al = np.exp(a[0, :, t]).astype(np.float32)
        fk = O.features(k[0, :, t], order).astype(np.float32)
        fq = O.features(q[0, :, t], order).astype(np.float32)
        S = (al[:, None, None] * S + fk[:, :, None] * v[0, :, t].astype(np.float32)[:, None, :]).astype(np.float32)
        z = (al[:, None] * z + fk).astype(np.float32)
        num = np.einsum("hr,hrc->hc", fq, S).astype(np.float32)
        den = np.einsum("hr,hr->h", fq, z).astype(np.float32)
        y32[:, t] = num / den[:, None]
    eps = 2.0 ** -24
    assert (np.abs(y32 - ref["y"][0]) / ref["scale_state"][0]).max() <= 64 * eps
    assert np.all(ref["scale_state"] >= ref["scale"] * (1 - 1e-12))


# ---------------------------------------------------------------------------
# A-mask of Algorithms 4 and 5 (Mamba-2S, 2Mamba): A = -softplus(h W_A),
# A^CS = cumsum(A); Algorithm 4's dt = softplus(h W_dt) without bias
# ---------------------------------------------------------------------------

def test_amask_reduces_to_algorithm3_with_unit_A_and_no_bias():
    # Algorithm 3 with A_log = 0 (A = -1) and dt_bias = 0 gives a = -softplus(dt_P)
    # and dt = softplus(dt_P): exactly the A-mask with A_P = dt_P
    rng = np.random.default_rng(41)
    x = rng.standard_normal((2, 3, 200)) * 2.0
    zeros = np.zeros(3)
    for chunk in (64, 128):
        dt3, cs3, tot3 = O.prep_ref(x, zeros, zeros, chunk)
        dt4, cs4, tot4 = O.prep_amask_ref(x, x, chunk)
        np.testing.assert_array_equal(dt4, dt3)
        np.testing.assert_array_equal(cs4, cs3)
        np.testing.assert_array_equal(tot4, tot3)
    dtn, csn, _ = O.prep_amask_ref(x, None, 64)
    assert dtn is None
    np.testing.assert_array_equal(csn, O.prep_ref(x, zeros, zeros, 64)[1])


@pytest.mark.parametrize("order", [1, 2])
def test_amask_two_tokens_hand_worked(order):
    # A_P = 0 for both tokens: a = -log 2, so token 1 reaches token 2 with weight
    # 1/2.  q = (1, 2), k = (3, 1), v = (4, 5), d_h = 1:
    #   order 1: y_2 = (2*3/2*4 + 2*1*5) / (2*3/2 + 2*1) = 22/5
    #   order 2: y_2 = ((2*3)^2/2*4 + (2*1)^2*5) / ((2*3)^2/2 + (2*1)^2) = 46/11
    # and y_1 = v_1 = 4.  With dt_P = 0 (dt = log 2) the value operand is V log 2.
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([3.0, 1.0]).reshape(1, 1, 2, 1)
    v = np.array([4.0, 5.0]).reshape(1, 1, 2, 1)
    A_P = np.zeros((1, 1, 2))
    y2 = float(Fraction(22, 5)) if order == 1 else float(Fraction(46, 11))
    plain = O.forward_amask_ref(q, k, v, A_P, None, order)["y"][0, 0, :, 0]
    np.testing.assert_allclose(plain, [4.0, y2], rtol=1e-14)
    scaled = O.forward_amask_ref(q, k, v, A_P, np.zeros((1, 1, 2)), order)["y"][0, 0, :, 0]
    np.testing.assert_allclose(scaled, [4.0 * math.log(2), y2 * math.log(2)], rtol=1e-14)


def test_amask_decay_negative_and_monotone():
    x = np.linspace(-30.0, 30.0, 601)
    _, a = O.discretise_amask(x)
    assert np.all(a < 0)
    assert np.all(np.diff(a) < 0)
    np.testing.assert_allclose(a[300], -math.log(2), rtol=1e-15)  # A_P = 0
    np.testing.assert_allclose(a[-1], -30.0, rtol=1e-12)           # softplus(x) ~ x for large x


@pytest.mark.parametrize("order", [1, 2])
def test_initial_state_continues_the_sequence(order):
    """Algorithm 6 with a nonzero initial state: the recurrence over a suffix,
    started from the state a prefix leaves, gives the full sequence's outputs
    (from the quadratic form) and its final state."""
    rng = np.random.default_rng(21)
    q, k, v, a = rand_case(rng, 1, 2, 90, 3, signed=False)
    full = O.forward_quadratic(q, k, v, a, order)
    _, _, S_all, z_all = O.forward_recurrent(q, k, v, a, order)
    for n1 in (1, 37, 64, 89):
        _, _, S1, z1 = O.forward_recurrent(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], a[:, :, :n1], order)
        y2, den2, S2, z2 = O.forward_recurrent(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], a[:, :, n1:],
                                               order, S0=S1, z0=z1)
        assert rel_err(y2, full["y"][:, :, n1:], full["scale"][:, :, n1:]) <= 1e-10
        np.testing.assert_allclose(den2, full["den"][:, :, n1:], rtol=1e-10)
        np.testing.assert_allclose(S2, S_all, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(z2, z_all, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# Algorithm 6 with the A-mask as printed: decay exp(-softplus(h W_A)) per step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("with_dt", [False, True])
def test_amask_decode_steps_equal_forward(order, with_dt):
    # the recurrence fed step by step against the A-mask quadratic form
    rng = np.random.default_rng(51)
    S, H, T, d = 2, 3, 19, 3
    qs, ks, vs = (rng.standard_normal((T, S, H, d)) for _ in range(3))
    A_P = rng.standard_normal((T, S, H)) - 1.0
    dt_P = rng.standard_normal((T, S, H)) if with_dt else None
    D = d ** order
    st, nz = np.zeros((S, H, D, d)), np.zeros((S, H, D))
    ys = []
    for t in range(T):
        y, st, nz, _ = O.decode_step_amask_ref(st, nz, qs[t], ks[t], vs[t], A_P[t],
                                               None if dt_P is None else dt_P[t], order)
        ys.append(y)
    ys = np.stack(ys, axis=2)
    tr = lambda x: None if x is None else np.moveaxis(x, 0, 2)
    fwd = O.forward_amask_ref(tr(qs), tr(ks), tr(vs), tr(A_P), tr(dt_P), order)
    assert rel_err(ys, fwd["y"], fwd["scale"]) <= 1e-10


def test_amask_decode_strong_decay_keeps_the_token():
    # A_P = 45: the factor exp(-softplus(45)) ~ 3e-20 wipes the history, so y_t
    # is the step's own value operand (v * softplus(dt_P))
    rng = np.random.default_rng(52)
    S, H, d = 2, 2, 4
    st, nz = np.zeros((S, H, d * d, d)), np.zeros((S, H, d * d))
    for t in range(5):
        q, k, v = (np.abs(rng.standard_normal((S, H, d))) + 0.1 for _ in range(3))
        dtp = rng.standard_normal((S, H))
        y, st, nz, _ = O.decode_step_amask_ref(st, nz, q, k, v, np.full((S, H), 45.0), dtp, 2)
        np.testing.assert_allclose(y, v * O.softplus(dtp)[..., None], rtol=1e-12)


# ---------------------------------------------------------------------------
# Symmetric packing of the order-2 state (derived from Algorithm 6's k (x) k)
# ---------------------------------------------------------------------------

def test_packed_pairs_layout():
    assert O.packed_pairs(3) == [(0, 0), (0, 1), (0, 2), (1, 1), (1, 2), (2, 2)]
    for d in (1, 2, 5, 32, 64):
        pairs = O.packed_pairs(d)
        assert len(pairs) == d * (d + 1) // 2
        for p, (a, b) in enumerate(pairs):
            assert 0 <= a <= b < d
            assert p == a * d - a * (a - 1) // 2 + (b - a)


def test_pack_unpack_roundtrip_and_symmetric_part():
    rng = np.random.default_rng(53)
    d, dv = 4, 3
    X = rng.standard_normal((2, d, d, dv))
    sym = (X + X.transpose(0, 2, 1, 3)) / 2  # rows (a, b) and (b, a) equal
    S = sym.reshape(2, d * d, dv)
    zm = rng.standard_normal((2, d, d))
    z = ((zm + zm.transpose(0, 2, 1)) / 2).reshape(2, d * d)
    Sp, zp = O.pack_state(S, z, d)
    assert Sp.shape == (2, d * (d + 1) // 2, dv) and zp.shape == (2, d * (d + 1) // 2)
    S2, z2 = O.unpack_state(Sp, zp, d)
    np.testing.assert_array_equal(S2, S)
    np.testing.assert_array_equal(z2, z)
    Sp2, zp2 = O.pack_state(S2, z2, d)
    np.testing.assert_array_equal(Sp2, Sp)
    # an asymmetric state packs to its symmetric part: the packed row (a, b)
    # is the mean of the two full rows
    A = X.reshape(2, d * d, dv)
    Ap, _ = O.pack_state(A, z, d)
    for p, (a, b) in enumerate(O.packed_pairs(d)):
        np.testing.assert_allclose(Ap[:, p], (X[:, a, b] + X[:, b, a]) / 2, rtol=1e-15)


def test_weighted_packed_contraction_brute_force():
    # sum over all (a, b) of q_a q_b M_ab, by a plain double loop, equals the
    # packed contraction with weight 2 off the diagonal, for any M (the packed
    # rows hold M's symmetric part)
    rng = np.random.default_rng(54)
    d = 3
    q = rng.standard_normal(d)
    M = rng.standard_normal((d, d))
    brute = 0.0
    for a in range(d):
        for b in range(d):
            brute += q[a] * q[b] * M[a, b]
    _, Mp = O.pack_state(np.zeros((d * d, 1)), M.reshape(d * d), d)
    packed = float(O.packed_features(q, True) @ Mp)
    assert abs(packed - brute) <= 1e-14 * (1 + abs(brute))
    # the unweighted k side is the upper triangle of k k^T
    k = rng.standard_normal(d)
    np.testing.assert_array_equal(O.packed_features(k, False),
                                  [k[a] * k[b] for a, b in O.packed_pairs(d)])


@pytest.mark.parametrize("amask", [False, True])
def test_packed_decode_equals_full_decode(amask):
    # the packed recurrence gives the full recurrence's outputs, and its states
    # are the packed full states, step after step
    rng = np.random.default_rng(55)
    S, H, T, d = 2, 2, 12, 4
    A_log = np.log(rng.uniform(1, 16, H))
    bias = rng.standard_normal(H) - 2.0
    st, nz = np.zeros((S, H, d * d, d)), np.zeros((S, H, d * d))
    sp, zp = O.pack_state(st, nz, d)
    for t in range(T):
        q, k, v = (rng.standard_normal((S, H, d)) for _ in range(3))
        dtp = rng.standard_normal((S, H))
        if amask:
            A_P = rng.standard_normal((S, H))
            y, st, nz, den = O.decode_step_amask_ref(st, nz, q, k, v, A_P, dtp, 2)
            yp, sp, zp, denp = O.decode_step_amask_packed_ref(sp, zp, q, k, v, A_P, dtp)
        else:
            y, st, nz, den = O.decode_step_ref(st, nz, q, k, v, dtp, bias, A_log, 2)
            yp, sp, zp, denp = O.decode_step_packed_ref(sp, zp, q, k, v, dtp, bias, A_log)
        np.testing.assert_allclose(denp, den, rtol=1e-12)
        np.testing.assert_allclose(yp * den[..., None], y * den[..., None], rtol=1e-10, atol=1e-12)
        want_s, want_z = O.pack_state(st, nz, d)
        np.testing.assert_allclose(sp, want_s, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(zp, want_z, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# Backward pass: gradients of the forward definitions, pinned by central
# finite differences, closed forms and invariances of the mathematics
# ---------------------------------------------------------------------------

def _loss(q, k, vop, a, order, dy):
    return float((O.forward_quadratic(q, k, vop, a, order)["y"] * dy).sum())


@pytest.mark.parametrize("order", [1, 2])
def test_backward_matches_finite_differences(order):
    rng = np.random.default_rng(61)
    q, k, v, a = rand_case(rng, 1, 2, 9, 3, signed=False)
    q, k = q + 0.2, k + 0.2  # keep every normaliser well away from zero
    dy = rng.standard_normal(v.shape)
    g = O.backward_quadratic(q, k, v, a, order, dy)
    h = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dvop", v), ("da", a)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"dq": (xp, k, v, a), "dk": (q, xp, v, a), "dvop": (q, k, xp, a), "da": (q, k, v, xp)}
            argm = {"dq": (xm, k, v, a), "dk": (q, xm, v, a), "dvop": (q, k, xm, a), "da": (q, k, v, xm)}
            num[idx] = (_loss(*args[name], order, dy) - _loss(*argm[name], order, dy)) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("order", [1, 2])
def test_backward_end_to_end_matches_finite_differences(order):
    rng = np.random.default_rng(62)
    B, H, N, d = 1, 2, 7, 3
    q = np.abs(rng.standard_normal((B, H, N, d))) + 0.2
    k = np.abs(rng.standard_normal((B, H, N, d))) + 0.2
    v = rng.standard_normal((B, H, N, d))
    dt_proj = rng.standard_normal((B, H, N))
    dt_bias = rng.standard_normal(H) - 1.0
    A_log = np.log(rng.uniform(1, 4, H))
    dy = rng.standard_normal((B, H, N, d))
    g = O.backward_ref(q, k, v, dt_proj, dt_bias, A_log, order, dy)

    def loss(v_, dtp_, bias_, alog_):
        return float((O.forward_ref(q, k, v_, dtp_, bias_, alog_, order)["y"] * dy).sum())

    h = 1e-6
    for name, x, pos in (("dv", v, 0), ("d_dt_proj", dt_proj, 1), ("d_dt_bias", dt_bias, 2),
                         ("d_A_log", A_log, 3)):
        num = np.empty_like(x)
        for idx in np.ndindex(x.shape):
            xs = [v, dt_proj, dt_bias, A_log]
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (loss(*(xp if i == pos else xs[i] for i in range(4)))
                        - loss(*(xm if i == pos else xs[i] for i in range(4)))) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("order", [1, 2])
def test_backward_single_token_closed_form(order):
    # N = 1: y_0 = vop_0 exactly, so dvop = dy and nothing else has a gradient
    rng = np.random.default_rng(63)
    q, k, v, a = rand_case(rng, 1, 1, 1, 4)
    dy = rng.standard_normal(v.shape)
    g = O.backward_quadratic(q, k, v, a, order, dy)
    np.testing.assert_allclose(g["dvop"], dy, rtol=1e-14)
    for name in ("dq", "dk", "da"):
        assert np.abs(g[name]).max() <= 1e-14 * (1 + np.abs(dy).max())


@pytest.mark.parametrize("order", [1, 2])
def test_backward_invariances(order):
    """Consequences of the definition, exact for any input:
    - y_i is homogeneous of degree 0 in q_i, so sum_c q_ic dq_ic = 0 per row;
    - y is homogeneous of degree 0 in k (all rows), so sum k . dk = 0;
    - a_0 shifts every cumsum equally and cancels in every difference: da_0 = 0;
    - a constant added to every value operand row adds it to every y_i, so
      sum_j dvop_j = sum_i dy_i."""
    rng = np.random.default_rng(64)
    q, k, v, a = rand_case(rng, 1, 2, 40, 5, signed=False)
    dy = rng.standard_normal(v.shape)
    g = O.backward_quadratic(q, k, v, a, order, dy)
    scale = np.abs(g["dq"]).max() * np.abs(q).max()
    assert np.abs((q * g["dq"]).sum(axis=-1)).max() <= 1e-10 * scale
    assert abs((k * g["dk"]).sum()) <= 1e-10 * np.abs(k * g["dk"]).sum()
    assert np.abs(g["da"][..., 0]).max() <= 1e-10 * np.abs(g["da"]).max()
    np.testing.assert_allclose(g["dvop"].sum(axis=2), dy.sum(axis=2), rtol=1e-10)


@pytest.mark.parametrize("order", [1, 2])
def test_backward_decay_gradient_from_key_gradients(order):
    """An identity of the definition, derived independently of the pair sums
    the oracle uses for da: with W_ij = (q_i . k_j)^p e^{cs_i - cs_j},
    sum_j dW_ij W_ij = (q_i . dq_i) / p and sum_i dW_ij W_ij = (k_j . dk_j) / p,
    so dcs_t = (q_t . dq_t - k_t . dk_t) / p; the first term vanishes (y_t is
    homogeneous of degree 0 in q_t), hence da_t = -(1/p) sum_{s >= t} k_s . dk_s
    over the whole sequence.  A slip in the oracle's decay gradient (a sign, a
    row/column sum, the direction of the cumsum, the decay factor of the
    pairs) breaks it."""
    rng = np.random.default_rng(67)
    q, k, v, a = rand_case(rng, 2, 2, 70, 5, a_scale=0.6)
    dy = rng.standard_normal(v.shape)
    g = O.backward_quadratic(q, k, v, a, order, dy)
    kdk = (k * g["dk"]).sum(axis=-1)
    da = -np.cumsum(kdk[..., ::-1], axis=-1)[..., ::-1] / order
    np.testing.assert_allclose(g["da"], da, rtol=1e-9, atol=1e-12 * np.abs(g["da"]).max())


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("case", ["one_token", "two_tokens"])
def test_golden_backward_error_scale(case, order):
    """The gradients' error scales (the backward parity metric) against values
    worked by hand from their definition (tests/golden/hand_worked.json): a
    scale off by any factor, a dropped term or a row / column sum swapped
    fails here."""
    c = load_golden()["backward_error_scale_dh1"][case]
    col = lambda x: np.array(x, float)[None, None, :, None]
    q, k, vop, dy = col(c["q"]), col(c["k"]), col(c["vop"]), col(c["dy"])
    a = np.log(np.array(c.get("exp_a", [0.5] * len(c["q"])), float))[None, None]
    sc = O.backward_error_scale(q, k, vop, a, order, dy)
    exp = c["expected"][str(order)]
    for name in ("dq", "dk", "dvop"):
        np.testing.assert_allclose(sc[name][0, 0, :, 0], fracs(exp[name]), rtol=1e-14, err_msg=name)
    np.testing.assert_allclose(sc["da"][0, 0], fracs(exp["da"]), rtol=1e-14)


@pytest.mark.parametrize("order", [1, 2])
def test_backward_error_scale_bounds_an_fp32_evaluation(order):
    """The gradients' error scales bound an fp32 evaluation of the same
    formulas (signed features, so order-1 normalisers nearly cancel on some
    rows): every element stays within a small multiple of fp32's unit
    roundoff times its scale."""
    rng = np.random.default_rng(65)
    q, k, v, a = rand_case(rng, 1, 2, 96, 6, a_scale=0.3)
    dy = rng.standard_normal(v.shape)
    ref = O.backward_quadratic(q, k, v, a, order, dy)
    sc = O.backward_error_scale(q, k, v, a, order, dy)
    f32 = O.backward_quadratic(*(x.astype(np.float32).astype(np.float64) for x in (q, k, v, a)), order,
                               dy.astype(np.float32).astype(np.float64))
    # an evaluation whose every product and sum is rounded to fp32
    lo = {n: np.empty_like(x) for n, x in ref.items()}
    for h in range(2):
        q32, k32, v32, dy32 = (x[0, h].astype(np.float32) for x in (q, k, v, dy))
        cs = np.cumsum(a[0, h]).astype(np.float32)
        s32 = q32 @ k32.T
        causal = np.tril(np.ones(s32.shape, bool))
        D = np.exp(np.where(causal, cs[:, None] - cs[None, :], -np.inf)).astype(np.float32)
        W = (s32 ** order * D).astype(np.float32)
        den = W.sum(axis=1, dtype=np.float32)
        y = (W @ v32) / den[:, None]
        dnum = dy32 / den[:, None]
        dden = -(dy32 * y).sum(axis=1, dtype=np.float32) / den
        dW = ((dnum @ v32.T + dden[:, None]) * causal).astype(np.float32)
        ds = (dW * D * np.float32(order) * s32 ** (order - 1)).astype(np.float32)
        P = dW * W
        dcs = P.sum(axis=1, dtype=np.float32) - P.sum(axis=0, dtype=np.float32)
        lo["dq"][0, h] = ds @ k32
        lo["dk"][0, h] = ds.T @ q32
        lo["dvop"][0, h] = W.T @ dnum
        lo["da"][0, h] = np.cumsum(dcs[::-1], dtype=np.float32)[::-1]
    for n in ("dq", "dk", "dvop", "da"):
        err = np.abs(lo[n] - ref[n]) / sc[n]
        assert err.max() <= 1e-5, (n, err.max())
    del f32


def test_prep_amask_backward_matches_finite_differences():
    rng = np.random.default_rng(66)
    A_P = rng.standard_normal((1, 2, 6)) * 3
    dt_P = rng.standard_normal((1, 2, 6)) * 3
    da = rng.standard_normal(A_P.shape)
    ddt = rng.standard_normal(A_P.shape)
    gA, gdt = O.prep_amask_backward_ref(A_P, dt_P, da, ddt)

    def loss(ap, dp):
        dt, a = O.discretise_amask(ap, dp)
        return float((a * da).sum() + (dt * ddt).sum())

    h = 1e-6
    for g, pos in ((gA, 0), (gdt, 1)):
        num = np.empty_like(g)
        for idx in np.ndindex(g.shape):
            xs = [A_P.copy(), dt_P.copy()]
            xs[pos][idx] += h
            lp = loss(*xs)
            xs[pos][idx] -= 2 * h
            num[idx] = (lp - loss(*xs)) / (2 * h)
        np.testing.assert_allclose(g, num, rtol=1e-7, atol=1e-9)
    assert O.prep_amask_backward_ref(A_P, None, da, None)[1] is None


# ---------------------------------------------------------------------------
# Algorithm 6's window-2 convolution on the decode path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("order", [1, 2])
def test_decode_conv_hand_worked(order):
    c = load_golden()["decode_conv_dh1"]
    w = np.array(c["conv_w"], float).reshape(3, 1, 1, 2)
    b = np.array(c["conv_b"], float).reshape(3, 1, 1)
    S = np.zeros((1, 1, 1, 1))
    z = np.zeros((1, 1, 1))
    cs = np.zeros((1, 3, 1, 1))
    ys = []
    for st in c["steps"]:
        x = [np.full((1, 1, 1), float(st[n])) for n in ("q", "k", "v")]
        y, S, z, cs, _ = O.decode_step_conv_ref(S, z, cs, *x, w, b, None, order,
                                                A_proj=np.full((1, 1), c["A_proj"]))
        ys.append(float(y[0, 0, 0]))
    exp = c["expected"][str(order)]
    np.testing.assert_allclose(ys, fracs(exp["y"]), rtol=1e-14)
    np.testing.assert_allclose(S[0, 0, 0, 0], frac(exp["S_final"]), rtol=1e-14)
    np.testing.assert_allclose(z[0, 0, 0], frac(exp["z_final"]), rtol=1e-14)
    np.testing.assert_array_equal(cs[0, :, 0, 0], c["expected"]["conv_state_final"])


@pytest.mark.parametrize("order", [1, 2])
@pytest.mark.parametrize("amask,act,bias", [(True, None, True), (False, "silu", False), (True, "silu", True)])
def test_decode_conv_steps_equal_sequence_conv_and_forward(order, amask, act, bias):
    """T decode steps with the convolution, from zero, equal the causal
    depthwise convolution of the whole sequence (numpy.convolve per channel,
    zero before the first token; SiLU as x * scipy.special.expit(x)) followed
    by the masked quadratic form on the convolved q, k, v."""
    from scipy.special import expit
    rng = np.random.default_rng(80 + order)
    Sq, H, d, T = 2, 3, 3, 9
    raw = [rng.standard_normal((T, Sq, H, d)) for _ in range(3)]
    w = rng.standard_normal((3, H, d, 2))
    b = rng.standard_normal((3, H, d)) if bias else None
    A_P = rng.standard_normal((T, Sq, H)) - 1.0
    dt_P = rng.standard_normal((T, Sq, H))
    dt_bias = rng.standard_normal(H) - 2.0
    A_log = rng.uniform(0, 1, H)
    D = d ** order
    S, z = np.zeros((Sq, H, D, d)), np.zeros((Sq, H, D))
    cs = np.zeros((Sq, 3, H, d))
    ys = []
    for t in range(T):
        kw = dict(A_proj=A_P[t], dt_proj=dt_P[t]) if amask else dict(dt_proj=dt_P[t], dt_bias=dt_bias, A_log=A_log)
        y, S, z, cs, _ = O.decode_step_conv_ref(S, z, cs, raw[0][t], raw[1][t], raw[2][t], w, b, act, order, **kw)
        ys.append(y)
    ys = np.stack(ys, axis=2)  # [S,H,T,d]
    # the whole sequences convolved channel by channel
    conv = []
    for i in range(3):
        x = np.moveaxis(raw[i], 0, -1)  # [S,H,d,T]
        out = np.empty_like(x)
        for idx in np.ndindex(x.shape[:-1]):
            hh, cc = idx[1], idx[2]
            out[idx] = np.convolve(x[idx], [w[i, hh, cc, 1], w[i, hh, cc, 0]])[:T]
            if b is not None:
                out[idx] += b[i, hh, cc]
        if act == "silu":
            out = out * expit(out)
        conv.append(np.moveaxis(out, -1, 2))  # [S,H,T,d]
    tr = lambda x: np.moveaxis(x, 0, -1)  # [T,S,H] -> [S,H,T]
    if amask:
        fwd = O.forward_amask_ref(*conv, tr(A_P), tr(dt_P), order)
    else:
        fwd = O.forward_ref(*conv, tr(dt_P), dt_bias, A_log, order)
    assert rel_err(ys, fwd["y"], fwd["scale"]) <= 1e-10
    np.testing.assert_array_equal(cs, np.stack([r[-1] for r in raw], axis=1))


def test_decode_conv_identity_is_the_plain_step():
    """Weights (0, 1), no bias, no activation: the convolution passes the raw
    q, k, v through, and the step is exactly the plain decode step."""
    rng = np.random.default_rng(90)
    Sq, H, d = 2, 2, 4
    q, k, v = (rng.standard_normal((Sq, H, d)) for _ in range(3))
    S0, z0 = rng.standard_normal((Sq, H, d * d, d)), rng.uniform(0, 1, (Sq, H, d * d))
    cs = rng.standard_normal((Sq, 3, H, d))
    w = np.zeros((3, H, d, 2))
    w[..., 1] = 1.0
    A_P = rng.standard_normal((Sq, H))
    y, S, z, _, _ = O.decode_step_conv_ref(S0, z0, cs, q, k, v, w, None, None, 2, A_proj=A_P)
    y2, S2, z2, _ = O.decode_step_amask_ref(S0, z0, q, k, v, A_P, None, 2)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(S, S2)
    np.testing.assert_array_equal(z, z2)
