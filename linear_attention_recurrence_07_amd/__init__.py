"""Kimi Delta Attention (KDA) mixer core for MI355X (gfx950): Python binding.

A thin ctypes layer over libkda.so (see include/kda.h).  It only marshals arguments:
torch tensors supply device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  If libkda.so is missing, importing
works but every call raises; there is no CPU fallback.

    o, final_state = chunk_prefill(q, k, v, g, beta, initial_state=None)
    o, final_state, y = chunk_prefill(..., gate=gate, norm_weight=w)      # fused gated norm
    ws = chunk_prepare(q, k, g, beta); o, final_state = chunk_scan(v, ws)   # the same, in two launches
    o = recurrent_step(q, k, v, g, beta, state)                            # state updated in place
    y = gated_rmsnorm(x, gate, w)
    y, conv_state = short_conv(x, weight, conv_state)                      # causal width-4 conv + SiLU

The call mirrors the kernels on the nnterp Kimi-Linear page (section 04): queries,
keys, values [B, T, H, d], g= per-key-channel log decays [B, T, H, dk] (fp32, <= 0),
beta= write strengths [B, T, H], initial_state= [N, H, dk, dv] or None; it returns the
head outputs and the last state.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = ["chunk_prefill", "chunk_prefill_workspace_size", "chunk_prefill_status", "chunk_prepare", "chunk_scan",
           "recurrent_step",
           "gated_rmsnorm", "short_conv", "gated_norm_proj", "gated_norm_proj_noalloc", "out_proj", "library_path", "load_library", "KdaError", "version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
# kda_status_t (include/kda.h)
(KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE, KDA_ERR_ALIGN, KDA_ERR_CONFLICT, KDA_ERR_WORKSPACE,
 KDA_ERR_UNSUPPORTED, KDA_ERR_HIP, KDA_ERR_TIMEOUT) = range(10)
_STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE", 4: "KDA_ERR_ALIGN",
           5: "KDA_ERR_CONFLICT", 6: "KDA_ERR_WORKSPACE", 7: "KDA_ERR_UNSUPPORTED", 8: "KDA_ERR_HIP",
           9: "KDA_ERR_TIMEOUT"}


class KdaError(RuntimeError):
    """A non-OK status from libkda.so."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


class KdaConvParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("D", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("width", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class KdaConv(ctypes.Structure):
    _fields_ = [("width", ctypes.c_int32), ("activation", ctypes.c_int32),
                ("weight_q", ctypes.c_void_p), ("weight_k", ctypes.c_void_p), ("weight_v", ctypes.c_void_p),
                ("initial_q", ctypes.c_void_p), ("initial_k", ctypes.c_void_p), ("initial_v", ctypes.c_void_p),
                ("final_q", ctypes.c_void_p), ("final_k", ctypes.c_void_p), ("final_v", ctypes.c_void_p)]


class KdaParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("scale", ctypes.c_float),
                ("use_qk_l2norm", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("norm_eps", ctypes.c_float),
                ("decay_per_head", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libkda.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it first "
                           "(python -c 'import __graft_entry__ as e; e.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.kda_chunk_prefill.restype = ctypes.c_int
    lib.kda_chunk_prefill.argtypes = [ctypes.POINTER(KdaParams)] + [P] * 13 + [P, ctypes.c_size_t, P]
    lib.kda_chunk_prefill_conv.restype = ctypes.c_int
    lib.kda_chunk_prefill_conv.argtypes = [ctypes.POINTER(KdaParams), ctypes.POINTER(KdaConv)] + [P] * 13 + \
        [P, ctypes.c_size_t, P]
    lib.kda_recurrent_step_conv.restype = ctypes.c_int
    lib.kda_recurrent_step_conv.argtypes = [ctypes.POINTER(KdaParams), ctypes.POINTER(KdaConv)] + [P] * 12
    lib.kda_chunk_prefill_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_prefill_workspace_size.argtypes = [ctypes.POINTER(KdaParams), i32]
    lib.kda_chunk_prefill_states.restype = ctypes.c_int
    lib.kda_chunk_prefill_states.argtypes = [ctypes.POINTER(KdaParams)] + [P] * 15 + [ctypes.c_size_t, P]
    lib.kda_chunk_prefill_states_workspace_size.restype = ctypes.c_size_t
    lib.kda_chunk_prefill_states_workspace_size.argtypes = [ctypes.POINTER(KdaParams), i32]
    lib.kda_chunk_prefill_status.restype = ctypes.c_int
    lib.kda_chunk_prefill_status.argtypes = [ctypes.POINTER(KdaParams), i32, P, ctypes.c_size_t, P]
    lib.kda_chunk_prepare.restype = ctypes.c_int
    lib.kda_chunk_prepare.argtypes = [ctypes.POINTER(KdaParams)] + [P] * 7 + [ctypes.c_size_t, P]
    lib.kda_chunk_scan.restype = ctypes.c_int
    lib.kda_chunk_scan.argtypes = [ctypes.POINTER(KdaParams)] + [P] * 4 + [ctypes.c_size_t] + [P] * 6
    lib.kda_gated_norm_proj.restype = ctypes.c_int
    lib.kda_gated_norm_proj.argtypes = [P] * 6 + [i64, i32, i32, i32, f32, i32, P, ctypes.c_size_t, P]
    lib.kda_gated_norm_proj_noalloc.restype = ctypes.c_int
    lib.kda_gated_norm_proj_noalloc.argtypes = [P] * 6 + [i64, i32, i32, i32, f32, i32, P]
    lib.kda_out_proj.restype = ctypes.c_int
    lib.kda_out_proj.argtypes = [P, P, P, i64, i32, i32, i32, P, ctypes.c_size_t, P]
    lib.kda_out_proj_workspace_size.restype = ctypes.c_size_t
    lib.kda_out_proj_workspace_size.argtypes = [i64, i32, i32]
    lib.kda_short_conv.restype = ctypes.c_int
    lib.kda_short_conv.argtypes = [ctypes.POINTER(KdaConvParams)] + [P] * 8
    lib.kda_recurrent_step.restype = ctypes.c_int
    lib.kda_recurrent_step.argtypes = [ctypes.POINTER(KdaParams)] + [P] * 12
    lib.kda_recurrent_states.restype = ctypes.c_int
    lib.kda_recurrent_states.argtypes = [ctypes.POINTER(KdaParams)] + [P] * 13
    lib.kda_gated_rmsnorm.restype = ctypes.c_int
    lib.kda_gated_rmsnorm.argtypes = [P, P, P, P, i64, i32, f32, i32, i32, P]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def version() -> str:
    return load_library().kda_version().decode()


def _check(status: int) -> None:
    if status != 0:
        raise KdaError(status, load_library().kda_last_error().decode())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KDA_BF16
    if t == torch.float32:
        return KDA_F32
    raise TypeError(f"unsupported dtype {t}: use bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, device) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _params(B, T, H, dk, dv, *, num_seqs=0, chunk=0, scale=None, use_qk_l2norm=True,
            in_dtype=KDA_BF16, out_dtype=KDA_BF16, norm_eps=1e-6, decay_per_head=False) -> KdaParams:
    return KdaParams(B, T, H, dk, dv, num_seqs, chunk, 0.0 if scale is None else float(scale),
                     1 if use_qk_l2norm else 0, in_dtype, out_dtype, float(norm_eps),
                     1 if decay_per_head else 0)


def _decay_layout(g: torch.Tensor, B: int, T: int, H: int, dk: int) -> bool:
    """True for one decay per head ([B, T, H]: the gated DeltaNet's scalar decay), False
    for one per key channel ([B, T, H, dk]: KDA)."""
    if g.dtype != torch.float32:
        raise TypeError("g must be float32")
    if g.shape == (B, T, H):
        return True
    if g.shape == (B, T, H, dk):
        return False
    raise ValueError("g must be [B,T,H,dk] (per key channel) or [B,T,H] (per head)")


def _check_cu_seqlens(cu: torch.Tensor, T: int) -> None:
    c = cu.tolist()
    if len(c) < 2 or c[0] != 0 or c[-1] > T or any(b < a for a, b in zip(c, c[1:])):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at or before T")


def _shape(t: torch.Tensor, name: str, shape, dtype) -> torch.Tensor:
    """A caller-supplied buffer must have exactly the shape and dtype the kernel writes or
    reads: the library sees only its address, so a smaller buffer would be overrun."""
    shape = tuple(int(x) for x in shape)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _on_device(device, *named) -> None:
    """Device, placement and contiguity checks, after every shape and dtype check."""
    for name, t in named:
        if t is not None:
            _dev(t, name, device)


def _seq_count(cu_seqlens: Optional[torch.Tensor], B: int) -> int:
    if cu_seqlens is None:
        return B
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be a 1-D tensor of N + 1 offsets")
    if cu_seqlens.device.type != "cpu" and cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    return cu_seqlens.numel() - 1


def _seq_device(cu_seqlens: Optional[torch.Tensor], T: int, dev) -> Optional[torch.Tensor]:
    if cu_seqlens is None:
        return None
    if cu_seqlens.device.type == "cpu":
        _check_cu_seqlens(cu_seqlens, T)
        return cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
    return _dev(cu_seqlens, "cu_seqlens", dev)


def _mask_device(attention_mask: Optional[torch.Tensor], B: int, T: int, dev) -> Optional[torch.Tensor]:
    if attention_mask is None:
        return None
    if tuple(attention_mask.shape) != (B, T):
        raise ValueError("attention_mask must be [B, T]")
    return (attention_mask != 0).to(device=dev, dtype=torch.uint8).contiguous()


def chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                  beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None, *,
                  cu_seqlens: Optional[torch.Tensor] = None,
                  attention_mask: Optional[torch.Tensor] = None,
                  gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                  norm_eps: float = 1e-6, scale: Optional[float] = None,
                  use_qk_l2norm_in_kernel: bool = True, chunk: int = 0,
                  output_dtype: Optional[torch.dtype] = None,
                  out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                  y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  head_outputs: bool = True, states: Optional[torch.Tensor] = None, _conv=None):
    """Chunked prefill.  Returns (o, final_state), or (o, final_state, y) with the fused
    sigmoid-gated RMSNorm when gate and norm_weight are given.  With the norm and
    head_outputs=False no o is returned (None): the head outputs pass through y, which is
    then normalised in place.

    states ([B,T,H,dk,dv] float32 on the device), when given, receives the state after
    every token, computed through the chunked form (kda_chunk_prefill_states: bf16
    inputs, dk = dv = 128); it needs head_outputs=True.

    cu_seqlens ([N+1] int32; a CPU tensor is validated then copied to the GPU) packs N
    sequences into B = 1; attention_mask ([B, T], nonzero = token) marks padding.
    out, final_state and y, when given, must be [B,T,H,dv], float32 [N,H,dk,dv] and
    [B,T,H,dv]; o and y share one dtype (out's when out is given, else output_dtype or
    q's).  workspace (a device tensor) is scratch of at least the library's reported
    size; one is allocated per call when it is not given.
    """
    lib = load_library()
    dev = q.device
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B,T,H,dk] and v [B,T,H,dv]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    in_dt = q.dtype
    for name, t in (("k", k), ("v", v)):
        if t.dtype != in_dt:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {in_dt}")
    if k.shape != q.shape or v.shape[:3] != (B, T, H):
        raise ValueError("q, k must be [B,T,H,dk] and v [B,T,H,dv]")
    per_head = _decay_layout(g, B, T, H, dk)
    _shape(beta, "beta", (B, T, H), torch.float32)
    N = _seq_count(cu_seqlens, B)
    if initial_state is not None:
        _shape(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    norm = gate is not None or norm_weight is not None
    if not head_outputs and not norm:
        raise ValueError("head_outputs=False needs the gated norm (gate and norm_weight)")
    if norm and (gate is None or norm_weight is None):
        raise ValueError("the gated norm needs both gate and norm_weight")
    out_dt = out.dtype if (out is not None and head_outputs) else (output_dtype or in_dt)
    _dtype_code(out_dt)
    if out is not None and head_outputs:
        _shape(out, "out", (B, T, H, dv), out_dt)
    if final_state is not None:
        _shape(final_state, "final_state", (N, H, dk, dv), torch.float32)
    if states is not None:
        if not head_outputs or _conv is not None:
            raise ValueError("per-token states need head_outputs=True and no fused convolution")
        _shape(states, "states", (B, T, H, dk, dv), torch.float32)
        _dev(states, "states", dev)
    if norm:
        _shape(gate, "gate", (B, T, H, dv), in_dt)
        _shape(norm_weight, "norm_weight", (dv,), torch.float32)
        if y is not None:
            _shape(y, "y", (B, T, H, dv), out_dt)
    _on_device(dev, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("initial_state", initial_state),
               ("out", out if head_outputs else None), ("final_state", final_state), ("gate", gate),
               ("norm_weight", norm_weight), ("y", y if norm else None))
    cu_dev = _seq_device(cu_seqlens, T, dev)
    mask_dev = _mask_device(attention_mask, B, T, dev)
    o = None
    if head_outputs:
        o = out if out is not None else torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    fs = final_state if final_state is not None else torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if norm:
        y = y if y is not None else torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    else:
        y = None
    p = _params(B, T, H, dk, dv, num_seqs=N if cu_dev is not None else 0, chunk=chunk, scale=scale,
                use_qk_l2norm=use_qk_l2norm_in_kernel, in_dtype=_dtype_code(in_dt),
                out_dtype=_dtype_code(out_dt), norm_eps=norm_eps, decay_per_head=per_head)
    size_fn = lib.kda_chunk_prefill_workspace_size if states is None else lib.kda_chunk_prefill_states_workspace_size
    need = size_fn(ctypes.byref(p), 1 if cu_dev is not None else 0)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None
    else:
        _dev(workspace, "workspace", dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if states is not None:
        _check(lib.kda_chunk_prefill_states(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                            _ptr(initial_state), _ptr(cu_dev), _ptr(mask_dev), _ptr(o), _ptr(fs),
                                            _ptr(gate), _ptr(norm_weight), _ptr(y), _ptr(states), _ptr(workspace),
                                            ws_bytes, _stream(dev)))
    elif _conv is None:
        _check(lib.kda_chunk_prefill(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(initial_state), _ptr(cu_dev), _ptr(mask_dev), _ptr(o), _ptr(fs),
                                     _ptr(gate), _ptr(norm_weight), _ptr(y), _ptr(workspace), ws_bytes,
                                     _stream(dev)))
    else:
        cv = _conv(N, H, dk, in_dt, dev)
        _check(lib.kda_chunk_prefill_conv(ctypes.byref(p), ctypes.byref(cv), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                          _ptr(beta), _ptr(initial_state), _ptr(cu_dev), _ptr(mask_dev), _ptr(o),
                                          _ptr(fs), _ptr(gate), _ptr(norm_weight), _ptr(y), _ptr(workspace),
                                          ws_bytes, _stream(dev)))
    return (o, fs) if y is None else (o, fs, y)


class _ConvSpec:
    """Marshals the fused short convolution's tensors into a KdaConv once the problem's
    sizes are known; keeps the final carried inputs it allocates in `final`."""

    def __init__(self, weights, initial, final, with_final, activation):
        if activation not in ("silu", None):
            raise ValueError("activation must be 'silu' or None")
        if len(weights) != 3:
            raise ValueError("conv_weights must be (weight_q, weight_k, weight_v)")
        self.weights, self.initial, self.final = tuple(weights), initial, final
        self.with_final, self.silu = with_final, activation == "silu"

    def __call__(self, N, H, d, in_dt, dev):
        W = self.weights[0].shape[-1] if self.weights[0].dim() == 2 else 0
        for name, w in zip("qkv", self.weights):
            _shape(w, f"conv weight_{name}", (H * d, W), torch.float32)
        st_shape = (N, W - 1, H * d)
        init = self.initial if self.initial is not None else (None, None, None)
        if len(init) != 3:
            raise ValueError("conv_state must be (q, k, v) carried inputs")
        for name, t in zip("qkv", init):
            if t is not None:
                _shape(t, f"conv_state[{name}]", st_shape, in_dt)
        fin = self.final
        if fin is None and self.with_final:
            fin = tuple(torch.empty(st_shape, dtype=in_dt, device=dev) for _ in range(3))
        fin = fin if fin is not None else (None, None, None)
        if len(fin) != 3:
            raise ValueError("conv_final_state must be (q, k, v) tensors")
        for name, t in zip("qkv", fin):
            if t is not None:
                _shape(t, f"conv_final_state[{name}]", st_shape, in_dt)
        _on_device(dev, *[(f"conv weight_{n}", w) for n, w in zip("qkv", self.weights)],
                   *[(f"conv_state[{n}]", t) for n, t in zip("qkv", init)],
                   *[(f"conv_final_state[{n}]", t) for n, t in zip("qkv", fin)])
        self.final = fin if self.with_final or self.final is not None else None
        return KdaConv(W, 1 if self.silu else 0, *[_ptr(w) for w in self.weights], *[_ptr(t) for t in init],
                       *[_ptr(t) for t in fin])


def chunk_prefill_conv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                       beta: torch.Tensor, initial_state: Optional[torch.Tensor] = None, *,
                       conv_weights, conv_state=None, conv_final_state=None, with_conv_state: bool = True,
                       activation: Optional[str] = "silu", **kw):
    """chunk_prefill on the raw q, k, v projections: the library runs their causal short
    convolution (conv_weights = (wq, wk, wv), float32 [H*d, W] each, then SiLU) inside the
    prefill.  conv_state = (q, k, v) carried inputs [N, W-1, H*d] in q's dtype (or None:
    zeros).  Returns chunk_prefill's tuple followed by the (q, k, v) carried inputs after
    the call (written into conv_final_state when given; the same tensors as conv_state
    update them in place), or None with with_conv_state=False."""
    spec = _ConvSpec(conv_weights, conv_state, conv_final_state, with_conv_state, activation)
    res = chunk_prefill(q, k, v, g, beta, initial_state, _conv=spec, **kw)
    return (*res, spec.final)


def chunk_prefill_workspace_size(B: int, T: int, H: int, dk: int, dv: int, *,
                                  num_seqs: Optional[int] = None, dtype: torch.dtype = torch.bfloat16,
                                  chunk: int = 0, states: bool = False) -> int:
    """Bytes of workspace chunk_prefill needs (with states=True: with per-token states);
    num_seqs is the sequence count when cu_seqlens packs the batch (B = 1)."""
    lib = load_library()
    p = _params(B, T, H, dk, dv, num_seqs=num_seqs or 0, chunk=chunk, in_dtype=_dtype_code(dtype),
                out_dtype=_dtype_code(dtype))
    fn = lib.kda_chunk_prefill_states_workspace_size if states else lib.kda_chunk_prefill_workspace_size
    return int(fn(ctypes.byref(p), 1 if num_seqs is not None else 0))


def chunk_prefill_status(workspace: torch.Tensor, B: int, T: int, H: int, dk: int = 128, dv: int = 128, *,
                         num_seqs: Optional[int] = None, dtype: torch.dtype = torch.bfloat16, chunk: int = 0) -> None:
    """Waits for the current stream and raises KdaError (KDA_ERR_TIMEOUT) if a bounded wait
    between the two column tiles of a head ran out in a scan that applied the gated norm
    on this workspace (y then holds NaN after that token).  num_seqs as for
    chunk_prefill_workspace_size."""
    lib = load_library()
    _dev(workspace, "workspace", workspace.device)
    p = _params(B, T, H, dk, dv, num_seqs=num_seqs or 0, chunk=chunk, in_dtype=_dtype_code(dtype),
                out_dtype=_dtype_code(dtype))
    _check(lib.kda_chunk_prefill_status(ctypes.byref(p), 1 if num_seqs is not None else 0, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(workspace.device)))


def _packing(cu_seqlens, attention_mask, B, T, dev):
    cu_dev = None
    N = B
    if cu_seqlens is not None:
        if cu_seqlens.device.type == "cpu":
            _check_cu_seqlens(cu_seqlens, T)
            cu_dev = cu_seqlens.to(device=dev, dtype=torch.int32).contiguous()
        else:
            cu_dev = _dev(cu_seqlens, "cu_seqlens", dev)
            if cu_dev.dtype != torch.int32:
                raise TypeError("cu_seqlens must be int32")
        N = cu_dev.numel() - 1
    mask_dev = None
    if attention_mask is not None:
        if attention_mask.shape != (B, T):
            raise ValueError("attention_mask must be [B, T]")
        mask_dev = (attention_mask != 0).to(device=dev, dtype=torch.uint8).contiguous()
    return cu_dev, mask_dev, N


def chunk_prepare(q: torch.Tensor, k: torch.Tensor, g: torch.Tensor, beta: torch.Tensor, *,
                  cu_seqlens: Optional[torch.Tensor] = None,
                  attention_mask: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                  use_qk_l2norm_in_kernel: bool = True, workspace: Optional[torch.Tensor] = None,
                  dv: Optional[int] = None) -> torch.Tensor:
    """First launch of the bf16, d = 128 chunked prefill: the per-chunk records (no state
    needed).  Returns the workspace that chunk_scan consumes."""
    lib = load_library()
    dev = q.device
    B, T, H, dk = q.shape
    dv = dk if dv is None else dv
    for name, t in (("q", q), ("k", k), ("g", g), ("beta", beta)):
        _dev(t, name, dev)
    if k.shape != q.shape or k.dtype != q.dtype or beta.shape != (B, T, H):
        raise ValueError("q, k must be [B,T,H,dk] of one dtype, beta [B,T,H]")
    per_head = _decay_layout(g, B, T, H, dk)
    if beta.dtype != torch.float32:
        raise TypeError("beta must be float32")
    cu_dev, mask_dev, N = _packing(cu_seqlens, attention_mask, B, T, dev)
    p = _params(B, T, H, dk, dv, num_seqs=N if cu_dev is not None else 0, scale=scale,
                use_qk_l2norm=use_qk_l2norm_in_kernel, in_dtype=_dtype_code(q.dtype), decay_per_head=per_head)
    need = lib.kda_chunk_prefill_workspace_size(ctypes.byref(p), 1 if cu_dev is not None else 0)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", dev)
    _check(lib.kda_chunk_prepare(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(cu_dev),
                                 _ptr(mask_dev), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(dev)))
    return workspace


def chunk_scan(v: torch.Tensor, workspace: torch.Tensor, initial_state: Optional[torch.Tensor] = None, *,
               cu_seqlens: Optional[torch.Tensor] = None, dk: Optional[int] = None,
               output_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
               final_state: Optional[torch.Tensor] = None, gate: Optional[torch.Tensor] = None,
               norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
               y: Optional[torch.Tensor] = None, head_outputs: bool = True):
    """Second launch of the bf16, d = 128 chunked prefill: the state scan over the records
    chunk_prepare wrote (same shapes and cu_seqlens).  Returns (o, final_state), or
    (o, final_state, y) with the gated norm (gate and norm_weight given); with the norm
    and head_outputs=False, o is not written (None).  Caller-supplied out, final_state and
    y are checked as in chunk_prefill."""
    lib = load_library()
    dev = v.device
    if v.dim() != 4:
        raise ValueError("v must be [B,T,H,dv]")
    B, T, H, dv = v.shape
    dk = dv if dk is None else dk
    N = _seq_count(cu_seqlens, B)
    if initial_state is not None:
        _shape(initial_state, "initial_state", (N, H, dk, dv), torch.float32)
    norm = gate is not None or norm_weight is not None
    if not head_outputs and not norm:
        raise ValueError("head_outputs=False needs the gated norm (gate and norm_weight)")
    if norm and (gate is None or norm_weight is None):
        raise ValueError("gate and norm_weight go together")
    out_dt = out.dtype if (out is not None and head_outputs) else (output_dtype or v.dtype)
    _dtype_code(out_dt)
    if out is not None and head_outputs:
        _shape(out, "out", (B, T, H, dv), out_dt)
    if final_state is not None:
        _shape(final_state, "final_state", (N, H, dk, dv), torch.float32)
    if norm:
        _shape(gate, "gate", (B, T, H, dv), v.dtype)
        _shape(norm_weight, "norm_weight", (dv,), torch.float32)
        if y is not None:
            _shape(y, "y", (B, T, H, dv), out_dt)
    _on_device(dev, ("v", v), ("workspace", workspace), ("initial_state", initial_state),
               ("out", out if head_outputs else None), ("final_state", final_state), ("gate", gate),
               ("norm_weight", norm_weight), ("y", y if norm else None))
    cu_dev = _seq_device(cu_seqlens, T, dev)
    o = None
    if head_outputs:
        o = out if out is not None else torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    fs = final_state if final_state is not None else torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    yy = None
    if norm:
        yy = y if y is not None else torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    p = _params(B, T, H, dk, dv, num_seqs=N if cu_dev is not None else 0, in_dtype=_dtype_code(v.dtype),
                out_dtype=_dtype_code(out_dt), norm_eps=norm_eps)
    _check(lib.kda_chunk_scan(ctypes.byref(p), _ptr(v), _ptr(initial_state), _ptr(cu_dev), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(o), _ptr(fs), _ptr(gate),
                              _ptr(norm_weight), _ptr(yy), _stream(dev)))
    return (o, fs, yy) if norm else (o, fs)


def recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                   beta: torch.Tensor, state: torch.Tensor, *,
                   attention_mask: Optional[torch.Tensor] = None,
                   gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
                   norm_eps: float = 1e-6, scale: Optional[float] = None,
                   use_qk_l2norm_in_kernel: bool = True, output_dtype: Optional[torch.dtype] = None,
                   out: Optional[torch.Tensor] = None, y: Optional[torch.Tensor] = None,
                   states: Optional[torch.Tensor] = None, _conv=None):
    """Token-by-token step(s): advances `state` ([B,H,dk,dv] fp32) in place over the T
    tokens of q/k/v and returns o (and y with the gated norm).  With `states` (a float32
    [B,T,H,dk,dv] tensor) the state after every token is stored there as well.  Caller-
    supplied out and y must be [B,T,H,dv] of one dtype (out's when out is given)."""
    lib = load_library()
    dev = q.device
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k must be [B,T,H,dk] and v [B,T,H,dv]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    in_dt = q.dtype
    for name, t in (("k", k), ("v", v)):
        if t.dtype != in_dt:
            raise TypeError(f"{name} dtype {t.dtype} differs from q's {in_dt}")
    if k.shape != q.shape or v.shape[:3] != (B, T, H):
        raise ValueError("q, k must be [B,T,H,dk] and v [B,T,H,dv]")
    per_head = _decay_layout(g, B, T, H, dk)
    _shape(beta, "beta", (B, T, H), torch.float32)
    _shape(state, "state", (B, H, dk, dv), torch.float32)
    out_dt = out.dtype if out is not None else (output_dtype or in_dt)
    _dtype_code(out_dt)
    if out is not None:
        _shape(out, "out", (B, T, H, dv), out_dt)
    norm = gate is not None or norm_weight is not None
    if norm:
        if gate is None or norm_weight is None:
            raise ValueError("the gated norm needs both gate and norm_weight")
        _shape(gate, "gate", (B, T, H, dv), in_dt)
        _shape(norm_weight, "norm_weight", (dv,), torch.float32)
        if y is not None:
            _shape(y, "y", (B, T, H, dv), out_dt)
    if states is not None:
        _shape(states, "states", (B, T, H, dk, dv), torch.float32)
    _on_device(dev, ("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state), ("out", out),
               ("gate", gate), ("norm_weight", norm_weight), ("y", y if norm else None), ("states", states))
    mask_dev = _mask_device(attention_mask, B, T, dev)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    if norm:
        y = y if y is not None else torch.empty((B, T, H, dv), dtype=out_dt, device=dev)
    else:
        y = None
    p = _params(B, T, H, dk, dv, scale=scale, use_qk_l2norm=use_qk_l2norm_in_kernel,
                in_dtype=_dtype_code(in_dt), out_dtype=_dtype_code(out_dt), norm_eps=norm_eps,
                decay_per_head=per_head)
    if _conv is not None:
        if states is not None:
            raise ValueError("the fused convolution stores no per-token states")
        cv = _conv(B, H, dk, in_dt, dev)
        _check(lib.kda_recurrent_step_conv(ctypes.byref(p), ctypes.byref(cv), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                           _ptr(beta), _ptr(state), _ptr(mask_dev), _ptr(o), _ptr(gate),
                                           _ptr(norm_weight), _ptr(y), _stream(dev)))
    elif states is None:
        _check(lib.kda_recurrent_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(state), _ptr(mask_dev), _ptr(o), _ptr(gate), _ptr(norm_weight),
                                      _ptr(y), _stream(dev)))
    else:
        _check(lib.kda_recurrent_states(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(state), _ptr(mask_dev), _ptr(o), _ptr(gate), _ptr(norm_weight),
                                        _ptr(y), _ptr(states), _stream(dev)))
    return o if y is None else (o, y)


def recurrent_step_conv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                        beta: torch.Tensor, state: torch.Tensor, *, conv_weights, conv_state=None,
                        conv_final_state=None, with_conv_state: bool = True, activation: Optional[str] = "silu",
                        **kw):
    """recurrent_step on the raw q, k, v of the new tokens: each is filtered with the row's
    carried inputs conv_state = (q, k, v) [B, W-1, H*d] (or None: zeros) inside the kernel.
    Returns recurrent_step's result and the (q, k, v) carried inputs after the call; pass the
    same tensors as conv_state and conv_final_state to update them in place (decode)."""
    spec = _ConvSpec(conv_weights, conv_state, conv_final_state, with_conv_state, activation)
    res = recurrent_step(q, k, v, g, beta, state, _conv=spec, **kw)
    return res, spec.final


def gated_rmsnorm(x: torch.Tensor, gate: torch.Tensor, weight: torch.Tensor, eps: float = 1e-6, *,
                  output_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None):
    """y = weight * x / sqrt(mean(x^2) + eps) * sigmoid(gate) over the last axis."""
    lib = load_library()
    dev = x.device
    if out is not None:
        _shape(out, "out", x.shape, out.dtype)
    _dev(x, "x", dev)
    _dev(gate, "gate", dev)
    _dev(weight, "weight", dev)
    if gate.shape != x.shape or gate.dtype != x.dtype:
        raise ValueError("gate must match x in shape and dtype")
    width = x.shape[-1]
    if weight.dtype != torch.float32 or weight.shape != (width,):
        raise ValueError("weight must be float32 [width]")
    y = out if out is not None else torch.empty(x.shape, dtype=output_dtype or x.dtype, device=dev)
    _dev(y, "out", dev)
    rows = x.numel() // width if width else 0
    _check(lib.kda_gated_rmsnorm(_ptr(x), _ptr(gate), _ptr(weight), _ptr(y), rows, width, float(eps),
                                 _dtype_code(x.dtype), _dtype_code(y.dtype), _stream(dev)))
    return y


def short_conv(x: torch.Tensor, weight: torch.Tensor, initial_state: Optional[torch.Tensor] = None, *,
               cu_seqlens: Optional[torch.Tensor] = None, attention_mask: Optional[torch.Tensor] = None,
               activation: Optional[str] = "silu", output_dtype: Optional[torch.dtype] = None,
               out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
               with_final_state: bool = True):
    """Causal short convolution over the token axis of x [B, T, D] (one width-W filter per
    channel, weight [D, W] float32), then SiLU.  initial_state / final_state [N, W-1, D] hold
    the W-1 inputs before / at the end of each sequence, oldest first, in x's dtype; pass
    the same tensor as both for an in-place decode step.  Returns (y, final_state) (or y
    alone with with_final_state=False)."""
    lib = load_library()
    dev = x.device
    _dev(x, "x", dev)
    _dev(weight, "weight", dev)
    B, T, D = x.shape
    if weight.dtype != torch.float32 or weight.dim() != 2 or weight.shape[0] != D:
        raise ValueError("weight must be float32 [D, W]")
    W = weight.shape[1]
    if activation not in ("silu", None):
        raise ValueError("activation must be 'silu' or None")
    cu_dev, mask_dev, N = _packing(cu_seqlens, attention_mask, B, T, dev)
    if initial_state is not None:
        _dev(initial_state, "initial_state", dev)
        if initial_state.dtype != x.dtype or initial_state.shape != (N, W - 1, D):
            raise ValueError(f"initial_state must be {x.dtype} [{N},{W - 1},{D}]")
    if out is not None:
        _shape(out, "out", (B, T, D), out.dtype)
    y = out if out is not None else torch.empty((B, T, D), dtype=output_dtype or x.dtype, device=dev)
    _dev(y, "out", dev)
    fs = final_state
    if fs is None and with_final_state:
        fs = torch.empty((N, W - 1, D), dtype=x.dtype, device=dev)
    if fs is not None:
        _dev(fs, "final_state", dev)
        if fs.dtype != x.dtype or fs.shape != (N, W - 1, D):
            raise ValueError(f"final_state must be {x.dtype} [{N},{W - 1},{D}]")
    p = KdaConvParams(B, T, D, N if cu_dev is not None else 0, W, 1 if activation == "silu" else 0,
                      _dtype_code(x.dtype), _dtype_code(y.dtype))
    _check(lib.kda_short_conv(ctypes.byref(p), _ptr(x), _ptr(weight), _ptr(initial_state), _ptr(cu_dev),
                              _ptr(mask_dev), _ptr(y), _ptr(fs), _stream(dev)))
    return (y, fs) if with_final_state else y


def _proj_workspace(lib, rows, K, N, dev, workspace):
    need = lib.kda_out_proj_workspace_size(rows, K, N)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None
    else:
        _dev(workspace, "workspace", dev)
    return workspace, 0 if workspace is None else workspace.numel() * workspace.element_size()


def out_proj(x: torch.Tensor, weight: torch.Tensor, *, output_dtype: Optional[torch.dtype] = None,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = x @ weight^T for bf16 x [..., in_features] and weight [out_features,
    in_features] (a Linear without bias); fp32 accumulation."""
    lib = load_library()
    dev = x.device
    _dev(x, "x", dev)
    _dev(weight, "weight", dev)
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("x and weight must be bfloat16")
    K = x.shape[-1]
    N = weight.shape[0]
    if weight.shape != (N, K):
        raise ValueError("weight must be [out_features, in_features]")
    rows = x.numel() // K if K else 0
    if out is not None:
        _shape(out, "out", x.shape[:-1] + (N,), out.dtype)
    res = out if out is not None else torch.empty(x.shape[:-1] + (N,), dtype=output_dtype or x.dtype, device=dev)
    _dev(res, "out", dev)
    ws, nbytes = _proj_workspace(lib, rows, K, N, dev, workspace)
    _check(lib.kda_out_proj(_ptr(x), _ptr(weight), _ptr(res), rows, K, N, _dtype_code(res.dtype), _ptr(ws), nbytes,
                            _stream(dev)))
    return res


def gated_norm_proj(o: torch.Tensor, gate: torch.Tensor, norm_weight: torch.Tensor, proj_weight: torch.Tensor,
                    eps: float = 1e-6, *, output_dtype: Optional[torch.dtype] = None,
                    y: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None):
    """The layer's exit: y = gated RMSNorm of each head of o ([..., heads, head_dim], bf16)
    with sigmoid(gate), then out = y_flat @ proj_weight^T (proj_weight [out_features,
    heads * head_dim] bf16).  Returns (y [..., heads * head_dim], out [..., out_features])."""
    lib = load_library()
    dev = o.device
    for name, t in (("o", o), ("gate", gate), ("norm_weight", norm_weight), ("proj_weight", proj_weight)):
        _dev(t, name, dev)
    if o.dtype != torch.bfloat16 or gate.dtype != torch.bfloat16 or proj_weight.dtype != torch.bfloat16:
        raise TypeError("o, gate and proj_weight must be bfloat16")
    if gate.shape != o.shape or o.dim() < 2:
        raise ValueError("o and gate must be [..., heads, head_dim]")
    heads, hd = o.shape[-2], o.shape[-1]
    if norm_weight.dtype != torch.float32 or norm_weight.shape != (hd,):
        raise ValueError("norm_weight must be float32 [head_dim]")
    N = proj_weight.shape[0]
    if proj_weight.shape != (N, heads * hd):
        raise ValueError("proj_weight must be [out_features, heads * head_dim]")
    rows = o.numel() // (heads * hd)
    lead = o.shape[:-2]
    if y is not None:
        _shape(y, "y", lead + (heads * hd,), torch.bfloat16)
    if out is not None:
        _shape(out, "out", lead + (N,), out.dtype)
    yy = y if y is not None else torch.empty(lead + (heads * hd,), dtype=torch.bfloat16, device=dev)
    _dev(yy, "y", dev)
    res = out if out is not None else torch.empty(lead + (N,), dtype=output_dtype or torch.bfloat16, device=dev)
    _dev(res, "out", dev)
    ws, nbytes = _proj_workspace(lib, rows, heads * hd, N, dev, workspace)
    _check(lib.kda_gated_norm_proj(_ptr(o), _ptr(gate), _ptr(norm_weight), _ptr(proj_weight), _ptr(yy), _ptr(res),
                                   rows, heads, hd, N, float(eps), _dtype_code(res.dtype), _ptr(ws), nbytes,
                                   _stream(dev)))
    return yy, res



def gated_norm_proj_noalloc(o: torch.Tensor, gate: torch.Tensor, norm_weight: torch.Tensor,
                            proj_weight: torch.Tensor, eps: float = 1e-6, *, y: torch.Tensor, out: torch.Tensor):
    """gated_norm_proj through the library's allocation-free entry point: the caller
    supplies y [..., heads * head_dim] (bf16) and out [..., out_features]; the split-K
    partial sums use the library's static per-GPU scratch (16 MiB), so neither this call
    nor the library allocates.  Calls that overlap in time on one GPU must not be issued.
    Returns (y, out)."""
    lib = load_library()
    dev = o.device
    if o.dim() < 2 or gate.shape != o.shape:
        raise ValueError("o and gate must be [..., heads, head_dim]")
    heads, hd = o.shape[-2], o.shape[-1]
    N = proj_weight.shape[0]
    lead = o.shape[:-2]
    _shape(y, "y", lead + (heads * hd,), torch.bfloat16)
    _shape(out, "out", lead + (N,), out.dtype)
    if o.dtype != torch.bfloat16 or gate.dtype != torch.bfloat16 or proj_weight.dtype != torch.bfloat16:
        raise TypeError("o, gate and proj_weight must be bfloat16")
    _shape(norm_weight, "norm_weight", (hd,), torch.float32)
    _shape(proj_weight, "proj_weight", (N, heads * hd), torch.bfloat16)
    _on_device(dev, ("o", o), ("gate", gate), ("norm_weight", norm_weight), ("proj_weight", proj_weight),
               ("y", y), ("out", out))
    rows = o.numel() // (heads * hd)
    _check(lib.kda_gated_norm_proj_noalloc(_ptr(o), _ptr(gate), _ptr(norm_weight), _ptr(proj_weight), _ptr(y),
                                           _ptr(out), rows, heads, hd, N, float(eps), _dtype_code(out.dtype),
                                           _stream(dev)))
    return y, out
