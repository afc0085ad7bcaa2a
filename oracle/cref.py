"""Build step and ctypes wrapper for the C fp64 oracle (kda_ref.c).  TEST INFRASTRUCTURE ONLY."""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "kda_ref.c")
LIB = os.path.join(_HERE, "libkda_oracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile kda_ref.c with gcc (fp64, OpenMP).  x86-64-v3 = AVX2 + FMA, which every
    recent EPYC/Xeon host has; no -ffast-math, so the fp64 arithmetic keeps IEEE order."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i = ctypes.c_int
        lib.kda_oracle_recurrence.restype = ctypes.c_int
        lib.kda_oracle_recurrence.argtypes = [
            i, i, i, i, i, i, P, P, P, P, P, P, P, i, P,
            ctypes.c_double, i, ctypes.c_double, P, i, P, P, i]
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(q, k, v, g, beta, initial_state=None, *, in_dtype: str = "f32",
               scale: Optional[float] = None, use_qk_l2norm: bool = True, l2_eps: float = 1e-6,
               mask=None, cu_seqlens=None, heads: Optional[Sequence[int]] = None,
               num_threads: int = 0):
    """C oracle.  q, k, v are fp32 arrays, or uint16 raw bf16 bits with in_dtype='bf16';
    g ([B,T,H,dk], or [B,T,H] for one decay per head), beta, initial_state fp32.  heads selects a subset of heads (outputs are laid out
    over that subset).  Returns o [B,T,len(heads),dv] and final_state [N,len(heads),dk,dv],
    both fp64."""
    lib = _load()
    bf16 = in_dtype == "bf16"
    want = np.uint16 if bf16 else np.float32
    q = np.ascontiguousarray(q, dtype=want)
    k = np.ascontiguousarray(k, dtype=want)
    v = np.ascontiguousarray(v, dtype=want)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    B, T, H, dk = q.shape
    g = np.asarray(g, dtype=np.float32)
    if g.ndim == 3:                    # one decay per head: the same factor on every key channel
        g = np.repeat(g[..., None], dk, axis=-1)
    g = np.ascontiguousarray(g)
    dv = v.shape[-1]
    init = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float32)
    cu = None if cu_seqlens is None else np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    m = None if mask is None else np.ascontiguousarray(mask, dtype=np.uint8)
    N = len(cu) - 1 if cu is not None else B
    hs = np.arange(H, dtype=np.int32) if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    nh = len(hs)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    o = np.empty((B, T, nh, dv), np.float64)
    fin = np.empty((N, nh, dk, dv), np.float64)
    rc = lib.kda_oracle_recurrence(B, T, H, dk, dv, int(bf16), _ptr(q), _ptr(k), _ptr(v),
                                   _ptr(g), _ptr(beta), _ptr(init), _ptr(cu), N, _ptr(m),
                                   float(scale), int(use_qk_l2norm), float(l2_eps),
                                   _ptr(hs), nh, _ptr(o), _ptr(fin), int(num_threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_recurrence failed with code {rc}")
    return o, fin
