"""fp64 numpy oracle for the layer's exit: the sigmoid-gated RMSNorm of each head's output
followed by the output projection.  TEST INFRASTRUCTURE ONLY.

What is computed, and where the pages fix it
--------------------------------------------
* Kimi-K3 atlas, gate-project page (the decode setting after P = 1,000 positions): the
  head outputs [B, 96 heads, 1, 128] enter as [B, 1, 12288] and leave as [B, 1, 7168];
  the Parameters table gives 128 for the gated RMSNorm and 88,080,384 (= 12,288 x 7,168)
  for the output projection, with no bias.  The model code there applies o_norm(o, g)
  per head, flattens the heads, then o_proj.
* The gated norm itself is kda_ref.gated_rmsnorm (pinned separately).

out[r, n] = sum_j y[r, j] * W[n, j], with y = the gated-normed heads flattened to
heads x head_dim and W the projection in the Linear layout [out_features, in_features].

Parity status: pinned (tests/test_out_proj_oracle_pins.py).
"""
from __future__ import annotations

import numpy as np

from oracle import kda_ref as R


def gated_norm_proj(o, gate, norm_weight, proj_weight, eps: float):
    """o, gate [rows, heads, head_dim]; norm_weight [head_dim]; proj_weight [N, heads*head_dim].
    Returns (y [rows, heads*head_dim], out [rows, N]) in fp64."""
    o = np.asarray(o, dtype=np.float64)
    rows, heads, hd = o.shape
    y = R.gated_rmsnorm(o, np.asarray(gate, dtype=np.float64), np.asarray(norm_weight, dtype=np.float64), eps)
    y = y.reshape(rows, heads * hd)
    out = y @ np.asarray(proj_weight, dtype=np.float64).T
    return y, out


def project(x, proj_weight):
    """out = x W^T (the output projection alone), fp64."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(proj_weight, dtype=np.float64).T

