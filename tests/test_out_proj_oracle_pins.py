"""Pins for the gated-norm + output-projection oracle: the pages' printed parameter counts
(Kimi-K3 atlas, gate-project page, Parameters table), the orientation of the projection
(a slip between y W and y W^T fails), and agreement with torch's Linear in fp64."""
import numpy as np
import torch

from oracle import kda_ref as R
from oracle import out_proj as P


def test_parameter_counts_printed_on_the_page():
    heads, hd, hidden = 96, 128, 7168
    assert heads * hd * hidden == 88_080_384          # output projection, no bias
    assert hd == 128                                   # gated RMSNorm weight
    assert heads * hd * hidden + hd == 88_080_512      # per-instance total


def test_projection_orientation_with_a_selection_matrix():
    """W[n, j] = 1 where j = perm[n]: out must pick columns of y (out = y W^T)."""
    rng = np.random.default_rng(1)
    rows, heads, hd, N = 3, 4, 8, 20
    o = rng.standard_normal((rows, heads, hd))
    gate = rng.standard_normal((rows, heads, hd))
    w = 1 + 0.1 * rng.standard_normal(hd)
    perm = rng.choice(heads * hd, N, replace=False)
    W = np.zeros((N, heads * hd))
    W[np.arange(N), perm] = 1.0
    y, out = P.gated_norm_proj(o, gate, w, W, 1e-6)
    np.testing.assert_array_equal(out, y[:, perm])
    np.testing.assert_allclose(y.reshape(rows, heads, hd), R.gated_rmsnorm(o, gate, w, 1e-6), rtol=0, atol=0)


def test_matches_torch_linear_without_bias():
    rng = np.random.default_rng(2)
    rows, heads, hd, N = 5, 6, 16, 40
    o = rng.standard_normal((rows, heads, hd))
    gate = rng.standard_normal((rows, heads, hd))
    w = 1 + 0.1 * rng.standard_normal(hd)
    W = rng.standard_normal((N, heads * hd)) / np.sqrt(heads * hd)
    y, out = P.gated_norm_proj(o, gate, w, W, 1e-6)
    lin = torch.nn.Linear(heads * hd, N, bias=False).double()
    with torch.no_grad():
        lin.weight.copy_(torch.from_numpy(W))
        ref = lin(torch.from_numpy(y)).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
