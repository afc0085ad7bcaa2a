"""Pins for the short-convolution oracle: facts fixed by the pages' module (a depthwise
Conv1d of width 4 with padding 3, then SiLU) and by the mathematics of a causal FIR
filter, chosen so that a plausible slip (reversed taps, an off-by-one shift, the
activation applied before the filter, padding tokens entering the window, a state that
keeps activations instead of inputs) fails at least one of them.

Kimi-K3 atlas, KDA layer page (kda-init code: ShortConvolution, activation 'silu');
nnterp Kimi-Linear page (module tree: Conv1d groups = channels, kernel 4, padding 3).
"""
import numpy as np
import pytest
import scipy.signal
import torch

from gen import inputs as gi
from oracle import short_conv as C


def test_impulse_response_gives_the_taps_in_correlation_order():
    """A unit impulse at token t0 in channel c produces z_{t0+i} = w[c, W-1-i]: the newest
    input meets the last tap (Conv1d correlation with W-1 zeros of left padding)."""
    rng = np.random.default_rng(1)
    T, D, W = 12, 3, 4
    w = rng.uniform(-1, 1, size=(D, W))
    x = np.zeros((1, T, D))
    x[0, 5, 1] = 1.0
    z, _ = C.short_conv(x, w, activation=None)
    for i in range(W):
        assert z[0, 5 + i, 1] == w[1, W - 1 - i]
    assert np.all(z[0, :5] == 0) and np.all(z[0, 5 + W:] == 0)
    assert np.all(z[0, :, 0] == 0) and np.all(z[0, :, 2] == 0)


def test_matches_torch_conv1d_module_definition():
    """The pages' module: Conv1d(D, D, kernel_size=W, padding=W-1, groups=D, bias=False),
    causal by keeping the first T outputs, then SiLU."""
    rng = np.random.default_rng(2)
    B, T, D, W = 2, 17, 5, 4
    x = rng.standard_normal((B, T, D))
    w = rng.uniform(-0.5, 0.5, size=(D, W))
    conv = torch.nn.Conv1d(D, D, kernel_size=W, padding=W - 1, groups=D, bias=False).double()
    with torch.no_grad():
        conv.weight.copy_(torch.from_numpy(w)[:, None, :])
        ref = torch.nn.functional.silu(conv(torch.from_numpy(x).transpose(1, 2))[..., :T]).transpose(1, 2).numpy()
    y, _ = C.short_conv(x, w)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_linear_part_is_a_causal_fir_filter_with_carried_inputs():
    """Without the activation each channel is the FIR filter b = reversed taps, run over the
    carried inputs followed by the sequence (scipy.signal.lfilter)."""
    rng = np.random.default_rng(3)
    T, D, W = 20, 4, 4
    x = rng.standard_normal((1, T, D))
    w = rng.uniform(-1, 1, size=(D, W))
    st = rng.standard_normal((1, W - 1, D))
    z, fin = C.short_conv(x, w, st, activation=None)
    for c in range(D):
        full = np.concatenate([st[0, :, c], x[0, :, c]])
        ref = scipy.signal.lfilter(w[c, ::-1], [1.0], full)[W - 1:]
        np.testing.assert_allclose(z[0, :, c], ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(fin[0], x[0, T - (W - 1):])


def test_activation_is_silu_after_the_filter():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 9, 6)) * 3
    w = np.zeros((6, 4))
    w[:, 3] = 1.0                                       # identity filter
    y, _ = C.short_conv(x, w)
    ref = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-14)
    assert C.silu(np.array([0.0]))[0] == 0.0


def test_split_invariance_and_one_token_steps():
    """Running [0, T1) then [T1, T) from the carried state equals one run; so does a chain
    of one-token calls (the decode form)."""
    x = gi.conv_inputs("split", B=2, T=23, D=8, seed=5, with_state=True)
    xs, w, st = x.f64("x"), x.weight, x.f64("initial_state")
    y, fin = C.short_conv(xs, w, st)
    y1, s1 = C.short_conv(xs[:, :9], w, st)
    y2, s2 = C.short_conv(xs[:, 9:], w, s1)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(s2, fin)
    s = st
    outs = []
    for t in range(x.T):
        yt, s = C.short_conv(xs[:, t:t + 1], w, s)
        outs.append(yt)
    np.testing.assert_allclose(np.concatenate(outs, 1), y, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(s, fin)


def test_short_sequences_keep_the_older_carried_inputs():
    """Fewer tokens than W-1: the final state is the tail of the carried inputs followed by
    the tokens."""
    x = gi.conv_inputs("short", B=1, T=2, D=4, seed=6, with_state=True)
    _, fin = C.short_conv(x.f64("x"), x.weight, x.f64("initial_state"))
    np.testing.assert_array_equal(fin[0, 0], x.f64("initial_state")[0, 2])
    np.testing.assert_array_equal(fin[0, 1:], x.f64("x")[0])


def test_packed_padded_and_per_sequence_runs_agree():
    lengths = (7, 1, 0, 12, 3)
    cu = gi.varlen_cu_seqlens(lengths)
    x = gi.conv_inputs("vl", B=1, T=int(cu[-1]), D=6, seed=7, with_state=True, cu_seqlens=cu)
    xs, w, st = x.f64("x"), x.weight, x.f64("initial_state")
    y, fin = C.short_conv(xs, w, st, cu_seqlens=cu)
    for n in range(len(lengths)):
        yn, fn = C.short_conv(xs[:, cu[n]:cu[n + 1]], w, st[n:n + 1])
        np.testing.assert_array_equal(y[:, cu[n]:cu[n + 1]], yn)
        np.testing.assert_array_equal(fin[n], fn[0])
    for left in (False, True):
        p = gi.conv_padded_from_packed(x, left=left)
        yp, fp = C.short_conv(p.f64("x"), w, st, mask=p.mask)
        np.testing.assert_array_equal(fp, fin)
        for n in range(len(lengths)):
            ln = lengths[n]
            lo = p.T - ln if left else 0
            np.testing.assert_array_equal(yp[n, lo:lo + ln], y[0, cu[n]:cu[n + 1]])
        assert np.all(yp[p.mask == 0] == 0)


def test_mask_holes_equal_removing_the_tokens():
    x = gi.conv_inputs("holes", B=1, T=15, D=3, seed=8, with_state=True)
    m = np.ones((1, 15), np.uint8)
    m[0, [2, 3, 9, 14]] = 0
    xs, w, st = x.f64("x"), x.weight, x.f64("initial_state")
    y, fin = C.short_conv(xs, w, st, mask=m)
    keep = m[0] == 1
    yc, fc = C.short_conv(xs[:, keep], w, st)
    np.testing.assert_array_equal(y[:, keep], yc)
    np.testing.assert_array_equal(fin, fc)
