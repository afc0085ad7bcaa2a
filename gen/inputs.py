"""Seeded synthetic inputs for the KDA mixer core.

This module only draws random numbers and casts dtypes.  It holds none of the
recurrence's arithmetic, so both the HIP path (through its tests and the
benchmark) and the fp64 oracle can take their inputs from here without sharing
any of the method.

The workloads are shaped like the Kimi Delta Attention layer described on the
Kimi-K3 atlas pages (96 heads of head_dim 128, "config.json", linear_attn_config)
and on the nnterp Kimi-Linear page ("support()" value table: queries and keys
[batch, seq, heads, key_dim], values [batch, seq, heads, value_dim], decays
[batch, seq, heads, key_dim] float32 non-positive, betas [batch, seq, heads]).
The pages name no dataset; every tensor here is synthetic.

Draw order inside one generator is fixed: q, k, v, g, beta-logits,
initial_state, gate, norm_weight.  bf16 tensors are returned as uint16 arrays
holding the raw bf16 bits, rounded from fp32 to nearest-even.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------- dtype helpers
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the raw 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bits to fp32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of an input array (fp32, or raw bf16 bits) to fp64."""
    if dtype == BF16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _unit_rows_f32(x: np.ndarray) -> np.ndarray:
    """Scale each last-axis row to unit Euclidean length (the configs draw q, k this way)."""
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def store_as(x: np.ndarray, dtype: str) -> np.ndarray:
    """x as a tensor of `dtype` would hold it: fp32 values, or raw bf16 bits rounded to
    nearest even from the fp32 values."""
    return _cast(np.asarray(x, dtype=np.float32), dtype)


# --------------------------------------------------------------------------- container
@dataclasses.dataclass
class KdaInputs:
    """One seeded problem.  Shapes follow the kernel call (query, key, value, g=, beta=,
    initial_state=) with the padding mask or cu_seqlens and the gated-norm operands."""

    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    in_dtype: str                       # "f32" or "bf16" for q, k, v, gate
    q: np.ndarray                       # [B,T,H,dk]
    k: np.ndarray                       # [B,T,H,dk]
    v: np.ndarray                       # [B,T,H,dv]
    g: np.ndarray                       # [B,T,H,dk] fp32, <= 0 ([B,T,H]: one decay per head)
    beta: np.ndarray                    # [B,T,H] fp32 in (0,1)
    initial_state: Optional[np.ndarray] = None   # [N,H,dk,dv] fp32
    gate: Optional[np.ndarray] = None            # [B,T,H,dv]
    norm_weight: Optional[np.ndarray] = None     # [dv] fp32
    norm_eps: float = 1e-6
    cu_seqlens: Optional[np.ndarray] = None      # [N+1] int32
    mask: Optional[np.ndarray] = None            # [B,T] uint8, 1 = token, 0 = padding
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1 if self.cu_seqlens is not None else self.B

    def f64(self, name: str) -> Optional[np.ndarray]:
        """An input widened exactly to fp64 (None stays None)."""
        x = getattr(self, name)
        if x is None:
            return None
        if name in ("q", "k", "v", "gate"):
            return to_f64(x, self.in_dtype)
        return np.asarray(x, dtype=np.float64)


def _draw(rng: np.random.Generator, shape, kind: str, dtype=np.float32, **kw) -> np.ndarray:
    if kind == "normal":
        return rng.standard_normal(size=shape, dtype=dtype) * np.float32(kw.get("std", 1.0)) + np.float32(kw.get("mean", 0.0))
    if kind == "uniform":
        lo, hi = kw["low"], kw["high"]
        return (rng.random(size=shape, dtype=dtype) * np.float32(hi - lo) + np.float32(lo)).astype(np.float32)
    raise ValueError(kind)


def _sigmoid_f32(x: np.ndarray) -> np.ndarray:
    # beta is a logistic function of a normal draw: the write strengths reach the kernel
    # already squashed into (0, 1) (nnterp Kimi-Linear page, Notes, KDA paragraph).
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def make_inputs(
    name: str,
    *,
    B: int,
    T: int,
    H: int,
    dk: int,
    dv: int,
    chunk: int = 64,
    in_dtype: str = BF16,
    seed: int = 0,
    g_range=(-5.0, 0.0),
    g_ranges_by_head: Optional[Sequence] = None,
    initial_state_std: Optional[float] = None,
    num_seqs: Optional[int] = None,
    norm: bool = False,
    norm_eps: float = 1e-6,
    cu_seqlens: Optional[Sequence[int]] = None,
    mask: Optional[np.ndarray] = None,
    normalize_qk: bool = True,
    qk_scale_by_head: Optional[Sequence[float]] = None,
    decay_per_head: bool = False,
) -> KdaInputs:
    """Draw one problem in the fixed order q, k, v, g, beta-logits, initial_state, gate, w.

    q and k are N(0, 1) rows scaled to unit length (normalize_qk), then multiplied per head
    by qk_scale_by_head (k takes the factors in reverse head order) when given.
    g is uniform in [low, high) per element (log decay, <= 0); with g_ranges_by_head each
    head h gets its own range.  beta = sigmoid(N(0,1)).  initial_state ~ N(0, std) when a
    std is given.  gate ~ N(0,1) and w ~ 1 + N(0, 0.1) when norm is set.
    """
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, T, H, dk), "normal")
    k = _draw(rng, (B, T, H, dk), "normal")
    if normalize_qk:
        q = _unit_rows_f32(q)
        k = _unit_rows_f32(k)
    if qk_scale_by_head is not None:
        # raw (not unit) queries and keys: head h's rows are multiplied by the factor
        # qk_scale_by_head[h % len], so the in-kernel L2 norm has work to do
        f = np.asarray([qk_scale_by_head[h % len(qk_scale_by_head)] for h in range(H)], np.float32)
        q = (q * f[None, None, :, None]).astype(np.float32)
        k = (k * f[::-1][None, None, :, None]).astype(np.float32)
    v = _draw(rng, (B, T, H, dv), "normal")
    if decay_per_head:        # one decay per (token, head): the gated DeltaNet's scalar decay
        g = _draw(rng, (B, T, H), "uniform", low=g_range[0], high=g_range[1])
    elif g_ranges_by_head is None:
        g = _draw(rng, (B, T, H, dk), "uniform", low=g_range[0], high=g_range[1])
    else:
        u = rng.random(size=(B, T, H, dk), dtype=np.float32)
        lo = np.array([r[0] for r in g_ranges_by_head], np.float32)[None, None, :, None]
        hi = np.array([r[1] for r in g_ranges_by_head], np.float32)[None, None, :, None]
        g = (u * (hi - lo) + lo).astype(np.float32)
    np.minimum(g, np.float32(0.0), out=g)
    beta = _sigmoid_f32(_draw(rng, (B, T, H), "normal"))
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32)
    n = num_seqs if num_seqs is not None else (len(cu) - 1 if cu is not None else B)
    init = None
    if initial_state_std is not None:
        init = _draw(rng, (n, H, dk, dv), "normal", std=initial_state_std)
    gate = w = None
    if norm:
        gate = _draw(rng, (B, T, H, dv), "normal")
        w = _draw(rng, (dv,), "normal", std=0.1, mean=1.0)
    return KdaInputs(
        name=name, B=B, T=T, H=H, dk=dk, dv=dv, chunk=chunk, in_dtype=in_dtype,
        q=_cast(q, in_dtype), k=_cast(k, in_dtype), v=_cast(v, in_dtype), g=g, beta=beta,
        initial_state=init, gate=None if gate is None else _cast(gate, in_dtype),
        norm_weight=w, norm_eps=norm_eps, cu_seqlens=cu,
        mask=None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8), seed=seed,
    )


# --------------------------------------------------------------------------- the workloads
VARLEN_LENGTHS = (8192, 6000, 3000, 777)


def tiny(seed: int = 0) -> KdaInputs:
    """B=1, T=64, H=2, dk=dv=16, chunk 16, all fp32, no initial state, gated norm on."""
    return make_inputs("tiny", B=1, T=64, H=2, dk=16, dv=16, chunk=16, in_dtype=F32,
                       seed=seed, norm=True)


def prefill(T: int = 2048, seed: int = 0, *, H: int = 96, d: int = 128, norm: bool = False) -> KdaInputs:
    """Single-prompt prefill at the 96-head, 128-dim layer shape (T=2048 config; T=8192 headline)."""
    return make_inputs(f"prefill_T{T}", B=1, T=T, H=H, dk=d, dv=d, chunk=64, in_dtype=BF16,
                       seed=seed, norm=norm)


def varlen_cu_seqlens(lengths: Sequence[int] = VARLEN_LENGTHS) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def varlen_packed(lengths: Sequence[int] = VARLEN_LENGTHS, seed: int = 0, *, H: int = 96,
                  d: int = 128) -> KdaInputs:
    """Varlen prefill: sequences packed as [1, sum(lengths), H, d] with cu_seqlens, carried
    initial state N(0, 0.02), fused gated norm (eps 1e-6, w ~ 1 + N(0, 0.1))."""
    cu = varlen_cu_seqlens(lengths)
    return make_inputs("varlen_packed", B=1, T=int(cu[-1]), H=H, dk=d, dv=d, chunk=64,
                       in_dtype=BF16, seed=seed, initial_state_std=0.02,
                       num_seqs=len(lengths), norm=True, cu_seqlens=cu)


def padded_from_packed(x: KdaInputs, *, left: bool = False) -> KdaInputs:
    """The same sequences as a packed problem, laid out as [N, max_len, H, d] with a 0/1 mask
    (right padding by default, left padding when asked).  Padding slots hold zeros."""
    cu = x.cu_seqlens
    lengths = np.diff(cu)
    N, L = len(lengths), int(lengths.max())

    def pad(a):
        if a is None:
            return None
        out = np.zeros((N, L) + a.shape[2:], dtype=a.dtype)
        for n in range(N):
            ln = int(lengths[n])
            seg = a[0, cu[n]:cu[n + 1]]
            if left:
                out[n, L - ln:] = seg
            else:
                out[n, :ln] = seg
        return out

    mask = np.zeros((N, L), np.uint8)
    for n in range(N):
        ln = int(lengths[n])
        if left:
            mask[n, L - ln:] = 1
        else:
            mask[n, :ln] = 1
    return dataclasses.replace(
        x, name=x.name.replace("packed", "padded"), B=N, T=L,
        q=pad(x.q), k=pad(x.k), v=pad(x.v), g=pad(x.g), beta=pad(x.beta), gate=pad(x.gate),
        cu_seqlens=None, mask=mask)


def decode_prompt(row: int, P: int = 1000, seed: int = 0, *, H: int = 96, d: int = 128) -> KdaInputs:
    """The P prompt tokens of decode batch row `row` (one generator per row, so a
    64-row state never needs all rows' prompts in host memory at once)."""
    return make_inputs(f"decode_prompt_r{row}", B=1, T=P, H=H, dk=d, dv=d, chunk=64,
                       in_dtype=BF16, seed=(seed, 1, row))


def decode_step(B: int = 64, seed: int = 0, *, H: int = 96, d: int = 128, norm: bool = True) -> KdaInputs:
    """The one new token of each of B decode rows: [B, 1, H, d] bf16 q/k/v, fp32 g, beta.
    The fp32 state [B, H, d, d] is supplied separately (a prompt's final state)."""
    return make_inputs("decode_step", B=B, T=1, H=H, dk=d, dv=d, chunk=64, in_dtype=BF16,
                       seed=(seed, 2), norm=norm)


def long_context(T: int = 65536, seed: int = 0, *, H: int = 96, d: int = 128) -> KdaInputs:
    """Long prefill: g ~ U[-5,-3) on the first half of the heads and U[-0.05,0) on the
    rest, fused gated norm, no initial state."""
    ranges = [(-5.0, -3.0)] * (H // 2) + [(-0.05, 0.0)] * (H - H // 2)
    return make_inputs(f"long_T{T}", B=1, T=T, H=H, dk=d, dv=d, chunk=64, in_dtype=BF16,
                       seed=seed, g_ranges_by_head=ranges, norm=True)


# --------------------------------------------------------------------------- short convolution
@dataclasses.dataclass
class ConvInputs:
    """One seeded problem for the causal short convolution in front of the kernel: x holds
    projected queries, keys or values [B, T, D] (D = heads x head_dim, or the three
    concatenated), one width-W filter per channel, and the carried inputs of each sequence."""

    name: str
    B: int
    T: int
    D: int
    width: int
    in_dtype: str
    x: np.ndarray                                # [B, T, D] (raw bf16 bits or fp32)
    weight: np.ndarray                           # [D, W] fp32
    initial_state: Optional[np.ndarray] = None   # [N, W-1, D] in in_dtype
    cu_seqlens: Optional[np.ndarray] = None
    mask: Optional[np.ndarray] = None
    seed: int = 0

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1 if self.cu_seqlens is not None else self.B

    def f64(self, name: str) -> Optional[np.ndarray]:
        a = getattr(self, name)
        if a is None:
            return None
        if name in ("x", "initial_state"):
            return to_f64(a, self.in_dtype)
        return np.asarray(a, dtype=np.float64)


def conv_inputs(name: str, *, B: int, T: int, D: int, width: int = 4, in_dtype: str = BF16,
                seed: int = 0, with_state: bool = False, num_seqs: Optional[int] = None,
                cu_seqlens: Optional[Sequence[int]] = None, mask: Optional[np.ndarray] = None) -> ConvInputs:
    """Draw in the fixed order x, weight, initial_state.  x ~ N(0,1) (the projections the
    configs feed the kernel); weight ~ U(-1/sqrt(W), 1/sqrt(W)), the default initialisation
    of a depthwise Conv1d of kernel size W (the pages give no trained weights); the
    carried inputs ~ N(0,1) like x."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (B, T, D), "normal")
    bound = 1.0 / np.sqrt(width)
    w = _draw(rng, (D, width), "uniform", low=-bound, high=bound)
    cu = None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32)
    n = num_seqs if num_seqs is not None else (len(cu) - 1 if cu is not None else B)
    init = _draw(rng, (n, width - 1, D), "normal") if with_state else None
    return ConvInputs(name=name, B=B, T=T, D=D, width=width, in_dtype=in_dtype, x=_cast(x, in_dtype),
                      weight=w, initial_state=None if init is None else _cast(init, in_dtype),
                      cu_seqlens=cu, mask=None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8),
                      seed=seed)


@dataclasses.dataclass
class LayerConv:
    """The three short convolutions in front of a KdaInputs problem whose q, k and v are
    the raw projections: taps (wq, wk, wv) fp32 [H*d, W] and, optionally, the carried
    inputs (q, k, v) [N, W-1, H*d] in the problem's input dtype."""

    width: int
    weights: tuple
    initial: Optional[tuple] = None


def layer_conv(x: KdaInputs, *, width: int = 4, seed: int = 0, with_state: bool = False) -> LayerConv:
    """Draw (from a generator of its own, so x's draws stay as they are) wq, wk, wv, then the
    carried inputs of q, k, v.  Taps ~ U(-1/sqrt(W), 1/sqrt(W)) as in conv_inputs; carried
    inputs ~ N(0, 1), like the raw projections."""
    rng = np.random.default_rng((seed, 3))
    bound = 1.0 / np.sqrt(width)
    ws = tuple(_draw(rng, (x.H * d, width), "uniform", low=-bound, high=bound) for d in (x.dk, x.dk, x.dv))
    init = None
    if with_state:
        n = x.num_seqs
        init = tuple(_cast(_draw(rng, (n, width - 1, x.H * d), "normal"), x.in_dtype) for d in (x.dk, x.dk, x.dv))
    return LayerConv(width=width, weights=ws, initial=init)


def conv_padded_from_packed(x: ConvInputs, *, left: bool = False) -> ConvInputs:
    """The packed sequences of x as [N, max_len, D] rows with a 0/1 mask."""
    cu = x.cu_seqlens
    lengths = np.diff(cu)
    N, L = len(lengths), int(lengths.max())
    out = np.zeros((N, L, x.D), dtype=x.x.dtype)
    mask = np.zeros((N, L), np.uint8)
    for n in range(N):
        ln = int(lengths[n])
        lo = L - ln if left else 0
        out[n, lo:lo + ln] = x.x[0, cu[n]:cu[n + 1]]
        mask[n, lo:lo + ln] = 1
    return dataclasses.replace(x, name=x.name + ("_left" if left else "_right"), B=N, T=L, x=out,
                               cu_seqlens=None, mask=mask)


# --------------------------------------------------------------------------- layer exit
@dataclasses.dataclass
class ProjInputs:
    """The layer's exit at decode: head outputs o and output-gate values [rows, heads,
    head_dim] (bf16 bits), the norm weight [head_dim] fp32 and the output projection
    [out_features, heads * head_dim] (bf16 bits; the pages give no trained weights)."""

    name: str
    rows: int
    heads: int
    head_dim: int
    out_features: int
    o: np.ndarray
    gate: np.ndarray
    norm_weight: np.ndarray
    proj_weight: np.ndarray
    eps: float = 1e-6
    seed: int = 0


def proj_inputs(name: str, *, rows: int, heads: int = 96, head_dim: int = 128, out_features: int = 7168,
                seed: int = 0) -> ProjInputs:
    """Draw in the fixed order o, gate, norm weight, projection.  o, gate ~ N(0,1); the norm
    weight ~ 1 + N(0, 0.1) as in the gated-norm configs; the projection ~ U(-1/sqrt(K),
    1/sqrt(K)) with K = heads * head_dim, the default initialisation of a bias-free Linear."""
    rng = np.random.default_rng(seed)
    o = _draw(rng, (rows, heads, head_dim), "normal")
    gate = _draw(rng, (rows, heads, head_dim), "normal")
    w = _draw(rng, (head_dim,), "normal", std=0.1, mean=1.0)
    K = heads * head_dim
    bound = 1.0 / np.sqrt(K)
    W = _draw(rng, (out_features, K), "uniform", low=-bound, high=bound)
    return ProjInputs(name=name, rows=rows, heads=heads, head_dim=head_dim, out_features=out_features,
                      o=_cast(o, BF16), gate=_cast(gate, BF16), norm_weight=w, proj_weight=_cast(W, BF16), seed=seed)

