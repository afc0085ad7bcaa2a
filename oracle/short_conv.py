"""fp64 numpy oracle for the causal short convolution in front of the KDA kernel.
TEST INFRASTRUCTURE ONLY.

What is computed, and where the pages fix it
--------------------------------------------
* Kimi-K3 atlas, KDA layer page (the kda-init code excerpt): the projected queries,
  keys and values each pass a ShortConvolution of kernel_size = short_conv_kernel_size
  (4 in config.json, linear_attn_config) with activation 'silu'.
* nnterp Kimi-Linear page, the printed module tree: the convolution is a Conv1d with
  groups equal to the channel count (one filter per channel), kernel_size 4, padding 3,
  no bias; and the Notes on KDA: the convolution sits between the projections and the
  delta rule, so besides the recurrent state the layer has to keep a few of its most
  recent input tokens between calls.

Per channel c, with W the width and w[c, 0..W-1] its taps, a token t of a sequence gives
    z_t[c] = sum_{j=0}^{W-1} w[c, j] * x_{t-(W-1)+j}[c]          (Conv1d correlation order,
                                                                  left padding W-1: causal)
    y_t[c] = silu(z_t[c]) = z_t[c] / (1 + exp(-z_t[c]))
where x before the first token of a sequence comes from its carried state (the W-1
inputs that preceded it, oldest first) or is zero when no state is given.  The state
after the call holds the last W-1 inputs of each sequence, oldest first.

Readings taken where the pages are silent: the carried state holds
raw inputs, not activations; a padding-mask zero skips the token (output 0, the window
does not advance, so padding never enters the window), matching the recurrence's mask;
cu_seqlens restarts the window per sequence from that sequence's state.

Parity status: pinned (tests/test_conv_oracle_pins.py).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def short_conv(x, weight, initial_state=None, *, cu_seqlens=None, mask=None, activation: Optional[str] = "silu"):
    """x [B, T, D]; weight [D, W]; initial_state [N, W-1, D] or None (zeros).
    Returns (y [B, T, D], final_state [N, W-1, D]), fp64.  With cu_seqlens (B = 1) the
    N sequences are packed along T; otherwise sequence n is batch row n (N = B)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    B, T, D = x.shape
    W = w.shape[1]
    if cu_seqlens is not None:
        cu = [int(c) for c in cu_seqlens]
        segs = [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    else:
        segs = [(b, 0, T) for b in range(B)]
    N = len(segs)
    y = np.zeros((B, T, D))
    final = np.zeros((N, W - 1, D))
    for n, (b, s, e) in enumerate(segs):
        hist = np.zeros((W - 1, D)) if initial_state is None else np.array(initial_state[n], dtype=np.float64)
        for t in range(s, e):
            if mask is not None and mask[b, t] == 0:
                continue                          # padding: output 0, window unchanged
            window = np.concatenate([hist, x[b, t][None, :]], axis=0)   # [W, D], oldest first
            z = np.sum(w.T * window, axis=0)
            y[b, t] = silu(z) if activation == "silu" else z
            hist = window[1:]
        final[n] = hist
    return y, final
