"""fp64 numpy oracle for the Kimi Delta Attention (KDA) core.  TEST INFRASTRUCTURE ONLY.

What is computed, and where the pages fix it
--------------------------------------------
* nnterp Kimi-Linear page, Notes, section on KDA decaying each key channel, and the
  family-module docstring (section 04): KDA is a gated DeltaNet whose log decay g is
  per key channel, [batch, seq, heads, key_dim], float32 and non-positive; the state is
  [batch, heads, key_dim, value_dim]; the state decays channel by channel before each
  delta-rule update; betas [batch, seq, heads] arrive already squashed into (0, 1); the
  kernel itself L2-normalises queries and keys (the values the page tabulates are
  un-normalised), and it also applies the 1/sqrt(key_dim) query scale.
* Same page, section 02 (support() table): state_input is None at the start of a
  prompt; state_output is the state leaving the layer; head outputs are taken before
  the gated norm.
* Kimi-K3 atlas, gate-project page (Parameters table and the o_norm code): the head
  outputs pass a sigmoid-gated RMSNorm over each head of head_dim features, with one
  head_dim-sized weight (128 parameters).

Per head, with S of shape [dk, dv], one token does, in this order:
    S <- diag(exp(g_t)) S                        (decay every key channel)
    S <- S + beta_t k_t (v_t - S^T k_t)^T        (delta rule: remove beta k k^T S, write beta k v^T)
    o_t = S^T q_t                                (read the updated state)
with k_t = k/||k||, q_t = q/||q|| / sqrt(dk).

Readings taken where the pages are silent:
  decay before the update and the read after the write; g is a natural log; the L2
  norm is x / sqrt(sum x^2 + 1e-6); a padding-mask zero leaves the state untouched
  and gives a zero output; cu_seqlens restarts the recurrence per sequence with that
  sequence's initial state; the gated norm normalises first, then multiplies by the
  weight and sigmoid(gate).

Parity status: pinned (tests/test_oracle_pins.py).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

L2_EPS = 1e-6


def l2_normalize(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis (the in-kernel q/k L2 norm)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def per_channel_decay(g, dk: int) -> np.ndarray:
    """g as one log decay per key channel, [B,T,H,dk].  A per-head decay [B,T,H] (the
    gated DeltaNet's: nnterp Kimi-Linear page, Notes, where KDA is that model with the
    decay made per channel) applies the same factor to every key channel of the head."""
    g = np.asarray(g, dtype=np.float64)
    if g.ndim == 3:
        g = np.repeat(g[..., None], dk, axis=-1)
    return g


def _segments(B: int, T: int, cu_seqlens) -> list:
    """(batch row, first token, end token) for every independent sequence."""
    if cu_seqlens is None:
        return [(b, 0, T) for b in range(B)]
    cu = [int(c) for c in cu_seqlens]
    if B != 1:
        raise ValueError("cu_seqlens needs a packed batch of 1")
    return [(0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def kda_recurrence(q, k, v, g, beta, initial_state=None, *, scale: Optional[float] = None,
                   use_qk_l2norm: bool = True, l2_eps: float = L2_EPS, mask=None,
                   cu_seqlens=None, return_states: bool = False):
    """Token-by-token KDA recurrence in fp64.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; g: [B,T,H,dk] (natural-log decays, <= 0), or
    [B,T,H] for one decay per head; beta: [B,T,H]; initial_state: [N,H,dk,dv] or None
    (zeros); mask: [B,T] (0 = padding)
    or None; cu_seqlens: [N+1] with B == 1, or None.
    Returns o [B,T,H,dv] and final_state [N,H,dk,dv]; with return_states also the
    state after every token, [B,T,H,dk,dv] (padding positions keep the carried state).
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    g = per_channel_decay(g, dk)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    if cu_seqlens is not None and mask is not None:
        raise ValueError("give cu_seqlens or mask, not both")
    segs = _segments(B, T, cu_seqlens)
    N = len(segs)
    if initial_state is None:
        final = np.zeros((N, H, dk, dv))
    else:
        final = np.array(initial_state, dtype=np.float64).reshape(N, H, dk, dv).copy()
    o = np.zeros((B, T, H, dv))
    states = np.zeros((B, T, H, dk, dv)) if return_states else None
    for n, (b, t0, t1) in enumerate(segs):
        S = final[n].copy()                                   # [H, dk, dv]
        for t in range(t0, t1):
            if mask is not None and mask[b, t] == 0:
                if return_states:
                    states[b, t] = S
                continue
            kt, qt = k[b, t], q[b, t]                         # [H, dk]
            if use_qk_l2norm:
                kt = l2_normalize(kt, l2_eps)
                qt = l2_normalize(qt, l2_eps)
            qt = qt * scale
            S = S * np.exp(g[b, t])[:, :, None]              # decay each key channel (row of S)
            r = np.einsum("hi,hij->hj", kt, S)               # k^T S
            u = beta[b, t][:, None] * (v[b, t] - r)          # beta (v - k^T S)
            S = S + kt[:, :, None] * u[:, None, :]           # S + k u^T
            o[b, t] = np.einsum("hi,hij->hj", qt, S)         # S^T q
            if return_states:
                states[b, t] = S
        final[n] = S
    if return_states:
        return o, final, states
    return o, final


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def gated_rmsnorm(x, gate, weight, eps: float):
    """y = weight * x / sqrt(mean(x^2) + eps) * sigmoid(gate), over the last axis.

    The gated RMSNorm after the kernel (Kimi-K3 atlas gate-project page: o_norm with a
    sigmoid activation over each head of head_dim features; one [head_dim] weight).
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(weight, np.float64) * (x / np.sqrt(ms + eps)) * sigmoid(gate)


def kda_chunked(q, k, v, g, beta, initial_state=None, *, chunk: int = 64,
                scale: Optional[float] = None, use_qk_l2norm: bool = True,
                l2_eps: float = L2_EPS, mask=None, cu_seqlens=None):
    """The same recurrence evaluated chunk by chunk (fp64), used only to check the chunked
    algebra that a blocked kernel relies on.  The prompt kernel works in 64-token blocks
    and passes only the state between them, never a per-token state (nnterp
    Kimi-Linear page, Notes, "Loading").  Within one chunk, with S0 the incoming state,
    G_r the running sum of g over the chunk up to token r (inclusive), and the
    normalised k_s, q_r:

      A[s,j]   = beta_s sum_c k_sc k_jc exp(G_sc - G_jc)      j < s
      (I + A) U = diag(beta) (V - (k * exp(G)) S0)            (unit lower-triangular solve)
      Bqk[r,s] = sum_c q_rc k_sc exp(G_rc - G_sc)             s <= r
      O        = (q * exp(G)) S0 + Bqk U
      S_next   = diag(exp(G_last)) S0 + (k * exp(G_last - G))^T U

    Every exponent above is <= 0 (G is non-increasing), so fp64 never overflows here.
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    g = per_channel_decay(g, dk)
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    segs = _segments(B, T, cu_seqlens)
    N = len(segs)
    final = (np.zeros((N, H, dk, dv)) if initial_state is None
             else np.array(initial_state, dtype=np.float64).reshape(N, H, dk, dv).copy())
    o = np.zeros((B, T, H, dv))
    for n, (b, t0, t1) in enumerate(segs):
        for h in range(H):
            S = final[n, h].copy()
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                kk, qq = k[b, c0:c1, h], q[b, c0:c1, h]
                gg, bb, vv = g[b, c0:c1, h].copy(), beta[b, c0:c1, h].copy(), v[b, c0:c1, h]
                if mask is not None:
                    keep = mask[b, c0:c1] != 0
                    gg[~keep] = 0.0
                    bb[~keep] = 0.0
                if use_qk_l2norm:
                    kk = l2_normalize(kk, l2_eps)
                    qq = l2_normalize(qq, l2_eps)
                qq = qq * scale
                G = np.cumsum(gg, axis=0)                                  # [L, dk]
                L = c1 - c0
                diff = G[:, None, :] - G[None, :, :]                      # G_r - G_s, [L, L, dk]
                lower_strict = np.tril(np.ones((L, L), bool), -1)
                lower_incl = np.tril(np.ones((L, L), bool), 0)
                dec = np.exp(np.where(lower_incl[:, :, None], diff, -np.inf))
                A = bb[:, None] * np.einsum("sc,jc,sjc->sj", kk, kk, dec) * lower_strict
                Bqk = np.einsum("rc,sc,rsc->rs", qq, kk, dec)
                rhs = bb[:, None] * (vv - (kk * np.exp(G)) @ S)
                U = np.linalg.solve(np.eye(L) + A, rhs)
                out = (qq * np.exp(G)) @ S + Bqk @ U
                if mask is not None:
                    out[mask[b, c0:c1] == 0] = 0.0
                o[b, c0:c1, h] = out
                S = np.exp(G[-1])[:, None] * S + (kk * np.exp(G[-1] - G)).T @ U
            final[n, h] = S
    return o, final


def rel_err(got, ref) -> float:
    """max |got - ref| / rms(ref), the parity measure used throughout."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        return float(np.max(np.abs(got - ref))) if got.size else 0.0
    return float(np.max(np.abs(got - ref)) / rms)
