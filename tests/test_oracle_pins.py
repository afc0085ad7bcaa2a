"""Pins for the fp64 oracle: facts fixed by the pages and by the mathematics of the
recurrence, chosen so that a plausible slip in the oracle (a dropped term, a wrong sign,
decay after instead of before the update, read before the write, a transposed state,
a missing q/k normalisation or scale) fails at least one of them.

The recurrence is the one stated on the nnterp Kimi-Linear encyclopedia page (Notes,
per-key-channel decay; section 04 family docstring) and the gated norm the one on the
Kimi-K3 atlas gate-project page (o_norm code, Parameters table).
"""
import json
import os

import numpy as np
import pytest
import scipy.signal
import torch

from gen import inputs as gi
from oracle import cref
from oracle import kda_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _problem(rng, B=1, T=12, H=2, dk=4, dv=3, g_low=-5.0):
    q = _rand(rng, B, T, H, dk)
    k = _rand(rng, B, T, H, dk)
    v = _rand(rng, B, T, H, dv)
    g = rng.uniform(g_low, 0.0, size=(B, T, H, dk))
    beta = 1.0 / (1.0 + np.exp(-_rand(rng, B, T, H)))
    return q, k, v, g, beta


# ----------------------------------------------------------------- hand-worked examples
def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("impl", ["numpy", "chunked", "c"])
def test_hand_example_recurrence(impl):
    ex = _load("hand_example_dk4_dv2.json")
    args = [np.array(ex[n], dtype=np.float64) for n in ("q", "k", "v", "g", "beta")]
    s0 = np.array(ex["initial_state"], dtype=np.float64)
    if impl == "numpy":
        o, s = R.kda_recurrence(*args, initial_state=s0, l2_eps=ex["l2_eps"])
    elif impl == "chunked":
        o, s = R.kda_chunked(*args, initial_state=s0, l2_eps=ex["l2_eps"], chunk=2)
    else:
        q, k, v, g, beta = (a.astype(np.float32) for a in args)
        o, s = cref.recurrence(q, k, v, g, beta, s0.astype(np.float32), l2_eps=ex["l2_eps"])
    # fp32 storage of ln(1/2) in the C path rounds exp(g) by ~3e-8 relative.
    tol = ex["tolerance"] if impl != "c" else 1e-6
    np.testing.assert_allclose(o, np.array(ex["expected_o"]), rtol=0, atol=tol)
    np.testing.assert_allclose(s, np.array(ex["expected_final_state"]), rtol=0, atol=tol)


def test_hand_example_gated_rmsnorm():
    ex = _load("hand_example_gated_rmsnorm.json")
    y = R.gated_rmsnorm(np.array(ex["x"]), np.array(ex["gate"]), np.array(ex["weight"]), ex["eps"])
    np.testing.assert_allclose(y, np.array(ex["expected_y"]), rtol=0, atol=ex["tolerance"])


# ----------------------------------------------------------------- gated norm special cases
def test_gated_rmsnorm_reduces_to_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = _rand(rng, 5, 7, 128)
    w = 1.0 + 0.1 * _rand(rng, 128)
    gate = np.full_like(x, 60.0)        # sigmoid(60) == 1.0 in fp64
    y = R.gated_rmsnorm(x, gate, w, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def test_gated_rmsnorm_invariants():
    rng = np.random.default_rng(2)
    x = _rand(rng, 9, 16)
    w = 1.0 + 0.1 * _rand(rng, 16)
    gate = _rand(rng, 9, 16)
    eps = 1e-3
    y = R.gated_rmsnorm(x, gate, w, eps)
    sig = 1.0 / (1.0 + np.exp(-gate))
    m = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean((y / (w * sig)) ** 2, axis=-1), m / (m + eps), rtol=1e-12)
    assert np.all(R.gated_rmsnorm(np.zeros_like(x), gate, w, eps) == 0.0)
    # scale invariance of the normalisation (eps -> 0)
    np.testing.assert_allclose(R.gated_rmsnorm(7.0 * x, gate, w, 0.0), R.gated_rmsnorm(x, gate, w, 0.0),
                               rtol=1e-12)


# ----------------------------------------------------------------- recurrence closed forms
def test_p1_no_write_no_decay_keeps_state():
    rng = np.random.default_rng(3)
    q, k, v, g, beta = _problem(rng)
    s0 = _rand(rng, 1, 2, 4, 3)
    o, s = R.kda_recurrence(q, k, v, np.zeros_like(g), np.zeros_like(beta), s0)
    np.testing.assert_array_equal(s, s0)
    qn = R.l2_normalize(q) / 2.0
    np.testing.assert_allclose(o, np.einsum("bthi,hij->bthj", qn, s0[0]), rtol=1e-13, atol=1e-14)


def test_p2_pure_decay_closed_form():
    rng = np.random.default_rng(4)
    q, k, v, g, beta = _problem(rng, T=9)
    s0 = _rand(rng, 1, 2, 4, 3)
    o, s, states = R.kda_recurrence(q, k, v, g, np.zeros_like(beta), s0, return_states=True)
    G = np.cumsum(g, axis=1)                                     # [B,T,H,dk]
    expect = np.exp(G)[..., None] * s0[:, None]                  # [B,T,H,dk,dv]
    np.testing.assert_allclose(states, expect, rtol=1e-13, atol=1e-15)
    qn = R.l2_normalize(q) / 2.0
    np.testing.assert_allclose(o, np.einsum("bthi,bthij->bthj", qn, expect), rtol=1e-12, atol=1e-15)


def test_p3_single_token():
    rng = np.random.default_rng(5)
    q, k, v, g, beta = _problem(rng, T=1, H=1, dk=5, dv=4)
    s0 = _rand(rng, 1, 1, 5, 4)
    o, s = R.kda_recurrence(q, k, v, g, beta, s0)
    kh = R.l2_normalize(k[0, 0, 0])
    qh = R.l2_normalize(q[0, 0, 0]) / np.sqrt(5)
    D = np.diag(np.exp(g[0, 0, 0]))
    Sp = D @ s0[0, 0]
    s1 = Sp + beta[0, 0, 0] * np.outer(kh, v[0, 0, 0] - Sp.T @ kh)
    np.testing.assert_allclose(s[0, 0], s1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], s1.T @ qh, rtol=1e-13, atol=1e-14)
    # from a zero state: S1 = beta k v^T, o1 = beta (k.q) v
    o, s = R.kda_recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(s[0, 0], beta[0, 0, 0] * np.outer(kh, v[0, 0, 0]), rtol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], beta[0, 0, 0] * (kh @ qh) * v[0, 0, 0], rtol=1e-13)


def test_p4_disjoint_keys_gated_linear_attention():
    """One-hot keys on distinct channels make the removal term vanish, leaving gated
    linear attention with per-channel decays: a closed form."""
    rng = np.random.default_rng(6)
    T, dk, dv = 6, 8, 3
    chans = rng.permutation(dk)[:T]
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, chans] = rng.uniform(0.5, 2.0, T)     # not unit length: the L2 norm makes it one-hot
    q = _rand(rng, 1, T, 1, dk)
    v = _rand(rng, 1, T, 1, dv)
    g = rng.uniform(-2.0, 0.0, size=(1, T, 1, dk))
    beta = rng.uniform(0.1, 0.9, size=(1, T, 1))
    o, s = R.kda_recurrence(q, k, v, g, beta, l2_eps=0.0)
    kh = R.l2_normalize(k[0, :, 0], 0.0)
    qh = R.l2_normalize(q[0, :, 0], 0.0) / np.sqrt(dk)
    G = np.cumsum(g[0, :, 0], axis=0)
    for t in range(T):
        ref = sum(beta[0, s_, 0] * np.sum(qh[t] * kh[s_] * np.exp(G[t] - G[s_])) * v[0, s_, 0]
                  for s_ in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], ref, rtol=1e-12, atol=1e-14)
    S_ref = sum(beta[0, t, 0] * np.outer(np.exp(G[-1] - G[t]) * kh[t], v[0, t, 0]) for t in range(T))
    np.testing.assert_allclose(s[0, 0], S_ref, rtol=1e-12, atol=1e-14)


def test_p5_delta_rule_write_property_and_overwrite():
    rng = np.random.default_rng(7)
    q, k, v, g, beta = _problem(rng, T=10, H=1, dk=6, dv=5)
    o, s, st = R.kda_recurrence(q, k, v, g, beta, l2_eps=0.0, return_states=True)
    kh = R.l2_normalize(k[0, :, 0], 0.0)
    prev = np.zeros((6, 5))
    for t in range(10):
        Sp = np.exp(g[0, t, 0])[:, None] * prev
        lhs = kh[t] @ st[0, t, 0]
        rhs = (1.0 - beta[0, t, 0]) * (kh[t] @ Sp) + beta[0, t, 0] * v[0, t, 0]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)
        prev = st[0, t, 0]
    # beta = 1, no decay, orthonormal keys: an associative memory where the latest value
    # written under a key replaces the earlier one.
    dk, dv, T = 4, 3, 9
    chans = np.array([0, 1, 2, 1, 3, 0, 2, 2, 1])
    k = np.zeros((1, T, 1, dk))
    k[0, np.arange(T), 0, chans] = 1.0
    v = _rand(rng, 1, T, 1, dv)
    q = k.copy()
    o, s = R.kda_recurrence(q, k, v, np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), l2_eps=0.0)
    for t in range(T):
        np.testing.assert_allclose(o[0, t, 0], v[0, t, 0] / np.sqrt(dk), rtol=1e-13, atol=1e-14)
    for c in range(dk):
        last = max(t for t in range(T) if chans[t] == c)
        np.testing.assert_allclose(s[0, 0, c], v[0, last, 0], rtol=1e-13, atol=1e-14)


def test_p6_linear_in_values_and_initial_state():
    rng = np.random.default_rng(8)
    q, k, v1, g, beta = _problem(rng, T=11)
    v2 = _rand(rng, *v1.shape)
    s1, s2 = _rand(rng, 1, 2, 4, 3), _rand(rng, 1, 2, 4, 3)
    a, b = 0.7, -1.3
    o1, f1 = R.kda_recurrence(q, k, v1, g, beta, s1)
    o2, f2 = R.kda_recurrence(q, k, v2, g, beta, s2)
    o3, f3 = R.kda_recurrence(q, k, a * v1 + b * v2, g, beta, a * s1 + b * s2)
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, rtol=1e-11, atol=1e-12)


def test_p7_scalar_case_is_first_order_filter():
    """dk = dv = 1 with constant g, beta: s_t = (1 - beta) e^g s_{t-1} + beta sign(k_t) v_t,
    a constant-coefficient first-order IIR filter (scipy.signal.lfilter)."""
    rng = np.random.default_rng(9)
    T = 40
    q = _rand(rng, 1, T, 1, 1)
    k = _rand(rng, 1, T, 1, 1)
    v = _rand(rng, 1, T, 1, 1)
    gv, bv = -0.3, 0.4
    g = np.full((1, T, 1, 1), gv)
    beta = np.full((1, T, 1), bv)
    o, s = R.kda_recurrence(q, k, v, g, beta, l2_eps=0.0)
    a = (1.0 - bv) * np.exp(gv)
    x = bv * np.sign(k[0, :, 0, 0]) * v[0, :, 0, 0]
    sref = scipy.signal.lfilter([1.0], [1.0, -a], x)
    np.testing.assert_allclose(o[0, :, 0, 0], np.sign(q[0, :, 0, 0]) * sref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s[0, 0, 0, 0], sref[-1], rtol=1e-12)


@pytest.mark.parametrize("chunk", [1, 2, 4, 16, 64])
@pytest.mark.parametrize("g_low,g_high", [(-5.0, 0.0), (-5.0, -3.0), (-0.05, 0.0)])
def test_p8_chunked_form_equals_recurrence(chunk, g_low, g_high):
    rng = np.random.default_rng(10 + chunk)
    B, T, H, dk, dv = 2, 37, 2, 8, 6
    q, k, v, _, beta = _problem(rng, B=B, T=T, H=H, dk=dk, dv=dv)
    g = rng.uniform(g_low, g_high, size=(B, T, H, dk))
    s0 = _rand(rng, B, H, dk, dv)
    o, s = R.kda_recurrence(q, k, v, g, beta, s0)
    oc, sc = R.kda_chunked(q, k, v, g, beta, s0, chunk=chunk)
    np.testing.assert_allclose(oc, o, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sc, s, rtol=1e-10, atol=1e-12)


def test_p9_split_invariance():
    rng = np.random.default_rng(11)
    q, k, v, g, beta = _problem(rng, T=20)
    s0 = _rand(rng, 1, 2, 4, 3)
    o, s = R.kda_recurrence(q, k, v, g, beta, s0)
    for cut in (1, 7, 19):
        oa, sa = R.kda_recurrence(q[:, :cut], k[:, :cut], v[:, :cut], g[:, :cut], beta[:, :cut], s0)
        ob, sb = R.kda_recurrence(q[:, cut:], k[:, cut:], v[:, cut:], g[:, cut:], beta[:, cut:], sa)
        np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sb, s, rtol=1e-12, atol=1e-14)


def test_p10_varlen_layouts_agree():
    lengths = (9, 4, 13)
    x = gi.varlen_packed(lengths, H=2, d=8)
    args = [x.f64(n) for n in ("q", "k", "v", "g", "beta")]
    o, s = R.kda_recurrence(*args, initial_state=x.initial_state, cu_seqlens=x.cu_seqlens)
    cu = x.cu_seqlens
    for n in range(len(lengths)):
        sl = slice(cu[n], cu[n + 1])
        on, sn = R.kda_recurrence(*[a[:, sl] for a in args], initial_state=x.initial_state[n:n + 1])
        np.testing.assert_allclose(o[:, sl], on, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(s[n:n + 1], sn, rtol=1e-13, atol=1e-15)
    for left in (False, True):
        p = gi.padded_from_packed(x, left=left)
        pa = [p.f64(n) for n in ("q", "k", "v", "g", "beta")]
        op, sp = R.kda_recurrence(*pa, initial_state=p.initial_state, mask=p.mask)
        np.testing.assert_allclose(sp, s, rtol=1e-13, atol=1e-15)
        for n in range(len(lengths)):
            valid = p.mask[n] != 0
            np.testing.assert_allclose(op[n, valid], o[0, cu[n]:cu[n + 1]], rtol=1e-13, atol=1e-15)
            assert np.all(op[n, ~valid] == 0.0)
        # the chunked form handles padding the same way
        oc, sc = R.kda_chunked(*pa, initial_state=p.initial_state, mask=p.mask, chunk=4)
        np.testing.assert_allclose(oc, op, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(sc, sp, rtol=1e-10, atol=1e-12)


def test_p12_state_difference_never_grows():
    """With unit keys, 0 < beta < 1 and g <= 0 the per-token map S -> (I - b k k^T) D S
    is non-expansive, so two runs on the same tokens from different initial states draw
    together.  A wrong sign on the removal term (I + b k k^T) breaks this."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta = _problem(rng, T=30, H=3, dk=6, dv=4, g_low=-0.2)
    sa, sb = _rand(rng, 1, 3, 6, 4), _rand(rng, 1, 3, 6, 4)
    _, _, st_a = R.kda_recurrence(q, k, v, g, beta, sa, return_states=True)
    _, _, st_b = R.kda_recurrence(q, k, v, g, beta, sb, return_states=True)
    d = np.sqrt(np.sum((st_a - st_b) ** 2, axis=(-1, -2)))[0]   # [T, H]
    d0 = np.sqrt(np.sum((sa - sb) ** 2, axis=(-1, -2)))[0]
    d = np.concatenate([d0[None], d], axis=0)
    assert np.all(d[1:] <= d[:-1] * (1 + 1e-12))


def test_q_scale_and_normalisation():
    """Scaling q or k by any positive factor changes nothing (in-kernel L2 norm), and the
    read is scaled by 1/sqrt(dk)."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta = _problem(rng, T=8, dk=16, dv=4)
    o, s = R.kda_recurrence(q, k, v, g, beta, l2_eps=0.0)
    o2, s2 = R.kda_recurrence(3.0 * q, 0.25 * k, v, g, beta, l2_eps=0.0)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(s2, s, rtol=1e-12, atol=1e-14)
    o3, _ = R.kda_recurrence(q, k, v, g, beta, l2_eps=0.0, scale=1.0)
    np.testing.assert_allclose(o3 / 4.0, o, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- numpy oracle vs C oracle
def test_p12_c_oracle_matches_numpy_tiny():
    x = gi.tiny()
    o, s = R.kda_recurrence(x.f64("q"), x.f64("k"), x.f64("v"), x.g, x.beta)
    oc, sc = cref.recurrence(x.q, x.k, x.v, x.g, x.beta, in_dtype="f32")
    assert R.rel_err(oc, o) < 1e-12 and R.rel_err(sc, s) < 1e-12
    assert np.all(np.isfinite(oc)) and np.all(np.isfinite(sc))


def test_p12_c_oracle_matches_numpy_bf16_cut_with_state_mask_and_heads():
    x = gi.prefill(T=256, H=6)
    rng = np.random.default_rng(14)
    s0 = (0.02 * rng.standard_normal((1, 6, 128, 128))).astype(np.float32)
    o, s = R.kda_recurrence(x.f64("q"), x.f64("k"), x.f64("v"), x.g, x.beta, s0)
    oc, sc = cref.recurrence(x.q, x.k, x.v, x.g, x.beta, s0, in_dtype="bf16")
    assert R.rel_err(oc, o) < 1e-12 and R.rel_err(sc, s) < 1e-12
    heads = [5, 1]
    oh, sh = cref.recurrence(x.q, x.k, x.v, x.g, x.beta, s0, in_dtype="bf16", heads=heads)
    np.testing.assert_allclose(oh, oc[:, :, heads], rtol=0, atol=0)
    np.testing.assert_allclose(sh, sc[:, heads], rtol=0, atol=0)
    # varlen and mask forms through the C path
    lengths = (40, 7, 21)
    xv = gi.varlen_packed(lengths, H=2, d=16)
    args = [xv.f64(n) for n in ("q", "k", "v", "g", "beta")]
    o, s = R.kda_recurrence(*args, initial_state=xv.initial_state, cu_seqlens=xv.cu_seqlens)
    oc, sc = cref.recurrence(xv.q, xv.k, xv.v, xv.g, xv.beta, xv.initial_state, in_dtype="bf16",
                             cu_seqlens=xv.cu_seqlens)
    assert R.rel_err(oc, o) < 1e-12 and R.rel_err(sc, s) < 1e-12
    p = gi.padded_from_packed(xv, left=True)
    op, sp = cref.recurrence(p.q, p.k, p.v, p.g, p.beta, p.initial_state, in_dtype="bf16", mask=p.mask)
    assert R.rel_err(sp, s) < 1e-12


# ----------------------------------------------------------------- one decay per head
def test_per_head_decay_closed_form_without_writes():
    """beta = 0 with one decay per (token, head): every entry of head h's state scales by
    exp(sum_t g_t[h]); heads decay independently (a head mix-up or an axis slip fails)."""
    rng = np.random.default_rng(31)
    B, T, H, dk, dv = 1, 9, 3, 4, 5
    q, k, v, _, _ = _problem(rng, B, T, H, dk, dv)
    g = rng.uniform(-2.0, 0.0, size=(B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S = R.kda_recurrence(q, k, v, g, np.zeros((B, T, H)), S0)
    for h in range(H):
        np.testing.assert_allclose(S[0, h], np.exp(g[0, :, h].sum()) * S0[0, h], rtol=1e-13)
    qn = R.l2_normalize(q) / np.sqrt(dk)
    t = 4
    np.testing.assert_allclose(o[0, t, 1], np.exp(g[0, :t + 1, 1].sum()) * (S0[0, 1].T @ qn[0, t, 1]), rtol=1e-12)


def test_per_head_decay_is_the_per_channel_decay_repeated():
    """The gated DeltaNet's scalar decay is KDA's per-channel decay with all key channels
    of a head equal; also through the chunked form and the C oracle."""
    rng = np.random.default_rng(32)
    B, T, H, dk, dv = 2, 21, 2, 8, 6
    q, k, v, _, beta = _problem(rng, B, T, H, dk, dv)
    g = rng.uniform(-5.0, 0.0, size=(B, T, H))
    S0 = 0.1 * rng.standard_normal((B, H, dk, dv))
    gfull = np.repeat(g[..., None], dk, axis=-1)
    o1, s1 = R.kda_recurrence(q, k, v, g, beta, S0)
    o2, s2 = R.kda_recurrence(q, k, v, gfull, beta, S0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    o3, s3 = R.kda_chunked(q, k, v, g, beta, S0, chunk=8)
    np.testing.assert_allclose(o3, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s3, s1, rtol=1e-10, atol=1e-12)
    o4, s4 = cref.recurrence(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                             g.astype(np.float32), beta.astype(np.float32), S0.astype(np.float32))
    o5, s5 = R.kda_recurrence(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
                              g.astype(np.float32), beta.astype(np.float32), S0.astype(np.float32))
    np.testing.assert_allclose(o4, o5, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(s4, s5, rtol=1e-9, atol=1e-11)


def test_per_token_states_are_the_final_states_of_the_prefixes():
    """The state after token t (the per-token states the pages read) is the final state of
    the same recurrence run over tokens 0..t; a padding token repeats the carried state."""
    rng = np.random.default_rng(33)
    B, T, H, dk, dv = 2, 7, 2, 4, 3
    q, k, v, g, beta = _problem(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv))
    m = np.ones((B, T), np.uint8)
    m[1, 3] = 0
    _, fin, states = R.kda_recurrence(q, k, v, g, beta, S0, mask=m, return_states=True)
    for t in range(T):
        _, ft = R.kda_recurrence(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], g[:, :t + 1], beta[:, :t + 1], S0,
                                 mask=m[:, :t + 1])
        np.testing.assert_allclose(states[:, t], ft, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(states[1, 3], states[1, 2])
    np.testing.assert_array_equal(states[:, -1], fin)



# ----------------------------------------------------------------- the parity measure
def test_rel_err_hand_values():
    """rel_err is max|got - ref| / rms(ref): hand-computed cases that tell apart the
    plausible slips (rms of got instead of ref, a mean instead of the max, a signed
    difference)."""
    # max|diff| = 2, rms(ref) = sqrt((1 + 16) / 2) = sqrt(8.5)
    assert R.rel_err([1.0, 2.0], [1.0, 4.0]) == pytest.approx(2.0 / np.sqrt(8.5), rel=1e-15)
    # the arguments are not symmetric: rms of the second one, sqrt((1 + 4) / 2)
    assert R.rel_err([1.0, 4.0], [1.0, 2.0]) == pytest.approx(2.0 / np.sqrt(2.5), rel=1e-15)
    # one error of 3 among 100 entries of a unit reference: the max (3), not the mean (0.03)
    got = np.ones(100)
    got[7] = 4.0
    assert R.rel_err(got, np.ones(100)) == pytest.approx(3.0, rel=1e-15)
    # absolute difference: a sign flip of a unit entry is an error of 2
    assert R.rel_err([-1.0], [1.0]) == pytest.approx(2.0, rel=1e-15)
    # an all-zero reference falls back to the absolute max error
    assert R.rel_err([0.5, -0.25], [0.0, 0.0]) == 0.5
    # shapes are flattened alike: a [2, 2] pair gives the same value as its flattening
    a, b = np.array([[1.0, 2.0], [3.0, 4.0]]), np.array([[1.0, 2.5], [3.0, 3.0]])
    assert R.rel_err(a, b) == pytest.approx(1.0 / np.sqrt((1 + 6.25 + 9 + 9) / 4), rel=1e-15)


def test_c_oracle_norm_flag_and_scale_match_numpy():
    """The C oracle's in-kernel L2 norm switch and query scale on raw (not unit) q and k,
    against the numpy recurrence whose normalisation is pinned above."""
    rng = np.random.default_rng(21)
    B, T, H, d = 1, 24, 3, 16
    q = (rng.standard_normal((B, T, H, d)) * np.array([0.05, 1.0, 40.0])[None, None, :, None]).astype(np.float32)
    k = (rng.standard_normal((B, T, H, d)) * np.array([40.0, 0.05, 1.0])[None, None, :, None]).astype(np.float32)
    v = rng.standard_normal((B, T, H, d)).astype(np.float32)
    g = rng.uniform(-5.0, 0.0, (B, T, H, d)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))).astype(np.float32)
    for use_l2, scale in ((True, None), (True, 0.3), (False, 0.3)):
        qq, kk = (q, k) if use_l2 else (R.l2_normalize(q), R.l2_normalize(k))
        o, s = R.kda_recurrence(qq, kk, v, g, beta, scale=scale, use_qk_l2norm=use_l2)
        oc, sc = cref.recurrence(np.asarray(qq, np.float32), np.asarray(kk, np.float32), v, g, beta,
                                 in_dtype="f32", scale=scale, use_qk_l2norm=use_l2)
        assert R.rel_err(oc, o) < 1e-6 and R.rel_err(sc, s) < 1e-6
    # the norm matters on these inputs: skipping it changes the result by O(1)
    o_norm, _ = R.kda_recurrence(q, k, v, g, beta)
    o_raw, _ = R.kda_recurrence(q, k, v, g, beta, use_qk_l2norm=False)
    assert not np.all(np.isfinite(o_raw)) or R.rel_err(o_raw, o_norm) > 1.0
