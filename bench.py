"""Benchmark of the KDA mixer core on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  1. chunked prefill of one 8192-token prompt at the 96-head, 128-dim layer shape
     (bf16 q/k/v, fp32 g and beta, no initial state) -> head outputs + final state, in
     its two launches: the per-chunk preparation (kda_chunk_prepare), then the state
     scan (kda_chunk_scan);
  2. the sigmoid-gated RMSNorm over those head outputs;
  3. one decode step for 64 rows (one new token each) on an fp32 state [64, 96, 128, 128]
     produced beforehand by prefilling a 1000-token prompt per row, with the gated norm.
Inputs are resident in HBM before timing starts.  Kernel durations come from HIP events
recorded on the stream the kernels run on (torch's current stream, which the binding
passes to the library).

Prints one JSON line.  `value` is prefill tokens/s (preparation + scan + gated norm);
`roofline` prices that whole prefill against the bytes the problem moves (inputs read
once, outputs written once), with the measured HBM traffic beside it; the decode state
bandwidth and per-launch figures ride along.  --gpus above 1 is
refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0
METRIC = "KDA prefill tokens/s (H=96,d=128,T=8192) + decode-step state GB/s at B=64"

T_PREFILL, H, D = 8192, 96, 128
D_HEAD = D
B_DECODE, P_DECODE = 64, 1000


def _bytes_prefill(T: int, H: int, d: int, with_init: bool, norm: bool = False) -> int:
    """Algorithmic HBM bytes of one prefill: q, k, v (bf16), g (fp32), beta (fp32) read,
    o (bf16) written, final state (fp32) written (+ read when an initial state is given);
    with the gated norm also gate (bf16) read and y (bf16) written."""
    per_tok_head = 3 * d * 2 + d * 4 + 4 + d * 2 + (2 * d * 2 if norm else 0)
    state = H * d * d * 4
    return T * H * per_tok_head + state * (2 if with_init else 1)


REC_BYTES = 32272      # one chunk record (per 32-token chunk and head) in the workspace
XCHG_BYTES = 512       # the scan's norm-exchange words per chunk and head, cleared by the preparation
CHUNK = 32


def _bytes_prep(T: int, H: int, d: int) -> int:
    """Algorithmic bytes of one preparation launch: per chunk and head, q, k (bf16), g
    (fp32) and beta (fp32) of its 32 tokens read, its record and cleared exchange words
    written."""
    per_chunk = CHUNK * (2 * d * 2 + d * 4 + 4) + REC_BYTES + XCHG_BYTES
    return (T // CHUNK) * H * per_chunk


def _bytes_scan(T: int, H: int, d: int, with_init: bool, norm: bool = False) -> int:
    """Algorithmic bytes of one scan launch: per chunk and head, its record and v (bf16)
    read, o (bf16) written, with the gated norm also gate read and y written (bf16); the
    final state (fp32) written (+ read with an initial state).  The exchange words of the
    norm (512 B per chunk and head, written and read once) are the split into two tiles'
    own traffic and are not counted."""
    per_chunk = REC_BYTES + CHUNK * d * 2 * (4 if norm else 2)
    state = H * d * d * 4
    return (T // CHUNK) * H * per_chunk + state * (2 if with_init else 1)


def _bytes_norm(rows: int, d: int) -> int:
    return rows * d * 2 * 3 + d * 4            # o and gate read, y written (bf16)


def _bytes_conv(B: int, T: int, D: int, width: int, with_init: bool) -> int:
    """Algorithmic bytes of one short-convolution launch (bf16 in and out): x read, y
    written, the carried inputs of each row written (and read when given), the fp32 taps."""
    state = B * (width - 1) * D * 2
    return B * T * D * 2 * 2 + state * (2 if with_init else 1) + D * width * 4


def time_short_conv(kda, reps: int = 10) -> dict:
    """The short convolution in front of the kernel, timed on its own (it is not part of
    the step): the T=8192 prompt's q, k and v projections side by side (D = 3 x 96 x 128),
    and one decode token for 64 rows with the carried inputs updated in place."""
    D = 3 * H * D_HEAD
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    w = (torch.rand((D, 4), generator=gen, device="cuda") - 0.5)
    out = {}
    for name, B, T in (("prefill", 1, T_PREFILL), ("decode", B_DECODE, 1)):
        x = torch.randn((B, T, D), generator=gen, device="cuda").to(torch.bfloat16)
        y = torch.empty_like(x)
        st = torch.randn((B, 3, D), generator=gen, device="cuda").to(torch.bfloat16)
        for _ in range(2):
            kda.short_conv(x, w, st, final_state=st, out=y)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            kda.short_conv(x, w, st, final_state=st, out=y)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3 / reps
        nbytes = _bytes_conv(B, T, D, 4, True)
        out[name] = {"B": B, "T": T, "D": D, "avg_call_us": t * 1e6, "algorithmic_bytes": nbytes,
                     "achieved": nbytes / t / 1e9, "unit": "GB/s", "frac": nbytes / t / 1e9 / HBM_PEAK_GBPS}
        del x, y, st
    return out


def time_per_head_decay(kda, P, ws, o, fs, reps: int = 10) -> dict:
    """The T=8192 prefill with one decay per (token, head) (g [1, T, H]: the gated
    DeltaNet's scalar decay), both launches timed with events; not part of the step."""
    g1 = P["g"][..., 0].contiguous()
    for _ in range(2):
        kda.chunk_prepare(P["q"], P["k"], g1, P["beta"], workspace=ws)
        kda.chunk_scan(P["v"], ws, out=o, final_state=fs)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        kda.chunk_prepare(P["q"], P["k"], g1, P["beta"], workspace=ws)
        e[1].record()
        kda.chunk_scan(P["v"], ws, out=o, final_state=fs)
        e[2].record()
    torch.cuda.synchronize()
    tp = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
    ts = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e-3
    b_prep = (T_PREFILL // CHUNK) * H * (CHUNK * (2 * D * 2 + 4 + 4) + REC_BYTES)
    return {"prepare_us": tp * 1e6, "scan_us": ts * 1e6, "tokens_per_s": T_PREFILL / (tp + ts),
            "prepare_algorithmic_bytes": b_prep, "prepare_GBps": b_prep / tp / 1e9}


def _median_pair_us(fns: dict, reps: int, rounds: int = 5) -> dict:
    """Median over `rounds` of the mean time per call (us) of `reps` back-to-back calls,
    the callables taking turns round by round so that clock drift hits each alike."""
    for fn in fns.values():
        for _ in range(2):
            fn()
    torch.cuda.synchronize()
    times = {name: [] for name in fns}
    for _ in range(rounds):
        for name, fn in fns.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            times[name].append(e0.elapsed_time(e1) * 1e3 / reps)
    return {name: float(np.median(v)) for name, v in times.items()}


def time_prefill_conv(kda, P, ws, o, fs, y, reps: int = 4) -> dict:
    """The T=8192 prefill with the short convolution in front (raw q, k, v projections,
    width-4 taps, carried inputs written), with gated norm, two ways: fused into the
    preparation and the scan (kda_chunk_prefill_conv), and as three kda_short_conv passes
    followed by kda_chunk_prefill.  Not part of the step."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    C = H * D
    ws3 = tuple((torch.rand((C, 4), generator=gen, device="cuda") - 0.5) for _ in range(3))
    fin = tuple(torch.empty((1, 3, C), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    filt = tuple(torch.empty((1, T_PREFILL, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    raw = (P["q"], P["k"], P["v"])

    def fused():
        kda.chunk_prefill_conv(P["q"], P["k"], P["v"], P["g"], P["beta"], conv_weights=ws3, conv_final_state=fin,
                               gate=P["gate"], norm_weight=P["w"], norm_eps=P["eps"], out=o, final_state=fs, y=y,
                               workspace=ws)

    def separate():
        for x, w, f, yv in zip(raw, ws3, fin, filt):
            kda.short_conv(x.view(1, T_PREFILL, C), w, final_state=f, out=yv.view(1, T_PREFILL, C))
        kda.chunk_prefill(filt[0], filt[1], filt[2], P["g"], P["beta"], gate=P["gate"], norm_weight=P["w"],
                          norm_eps=P["eps"], out=o, final_state=fs, y=y, workspace=ws)

    res = {}
    for name, us in _median_pair_us({"fused": fused, "separate": separate}, reps).items():
        res[f"{name}_us"] = us
        res[f"{name}_tokens_per_s"] = T_PREFILL / (us * 1e-6)
    nb = _bytes_prefill(T_PREFILL, H, D, False, norm=True) + 3 * (3 * C * 2 + C * 4 * 4)
    res["fused_algorithmic_bytes"] = nb
    res["fused_GBps"] = nb / (res["fused_us"] * 1e-6) / 1e9
    res["saved_bytes_vs_separate"] = 3 * 2 * T_PREFILL * C * 2      # filtered q, k, v written and read back
    del filt, fin
    return res


def time_decode_conv(kda, S, state0, reps: int = 20) -> dict:
    """The B=64 decode step with the short convolution in front (raw q, k, v of the new
    token, carried inputs updated in place), with gated norm: fused into the decode kernel
    (kda_recurrent_step_conv) against three kda_short_conv passes and kda_recurrent_step.
    Not part of the step."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12)
    C = H * D
    ws3 = tuple((torch.rand((C, 4), generator=gen, device="cuda") - 0.5) for _ in range(3))
    cst = tuple(torch.randn((B_DECODE, 3, C), generator=gen, device="cuda").to(torch.bfloat16) for _ in range(3))
    filt = tuple(torch.empty((B_DECODE, 1, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    st = state0.clone()
    od = torch.empty((B_DECODE, 1, H, D), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty_like(od)
    raw = (S["q"], S["k"], S["v"])

    def fused():
        kda.recurrent_step_conv(S["q"], S["k"], S["v"], S["g"], S["beta"], st, conv_weights=ws3, conv_state=cst,
                                conv_final_state=cst, gate=S["gate"], norm_weight=S["w"], out=od, y=yd)

    def separate():
        for x, w, c, f in zip(raw, ws3, cst, filt):
            kda.short_conv(x.view(B_DECODE, 1, C), w, c, final_state=c, out=f.view(B_DECODE, 1, C),
                           with_final_state=False)
        kda.recurrent_step(filt[0], filt[1], filt[2], S["g"], S["beta"], st, gate=S["gate"], norm_weight=S["w"],
                           out=od, y=yd)

    res = {f"{name}_us": us for name, us in _median_pair_us({"fused": fused, "separate": separate}, reps).items()}
    nb = _bytes_decode_state(B_DECODE, H, D)
    res["state_GBps_fused"] = nb / (res["fused_us"] * 1e-6) / 1e9
    res["state_frac_fused"] = res["state_GBps_fused"] / HBM_PEAK_GBPS
    del st, filt
    return res


def time_recurrent_states(kda, T: int = 256, reps: int = 5) -> dict:
    """The state after every token of a T-token prompt at the 96-head, 128-dim shape (64 KB
    per token and head), two ways: the token-by-token kernel (kda_recurrent_states), and
    the chunked form (kda_chunk_prefill_states: preparation, scan, then the per-token
    fill), under "chunked".  Not part of the step."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    shp = (1, T, H, D)
    q = _unit_rows(_dev_randn(shp, gen, torch.bfloat16))
    k = _unit_rows(_dev_randn(shp, gen, torch.bfloat16))
    v = _dev_randn(shp, gen, torch.bfloat16)
    g = torch.rand(shp, generator=gen, device="cuda") * -5.0
    beta = torch.sigmoid(torch.randn((1, T, H), generator=gen, device="cuda"))
    st0 = torch.zeros((1, H, D, D), device="cuda")
    states = torch.empty((1, T, H, D, D), device="cuda")
    o = torch.empty_like(v)
    st = st0.clone()
    kda.recurrent_step(q, k, v, g, beta, st, out=o, states=states)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        st.copy_(st0)
        e0.record()
        kda.recurrent_step(q, k, v, g, beta, st, out=o, states=states)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    t = float(np.mean(ts))
    nbytes = T * H * D * D * 4 + 2 * H * D * D * 4 + T * H * (4 * D * 2 + D * 4 + 4)
    # the chunked form on the same inputs (initial state read, final state written)
    fs = torch.empty_like(st0)
    ws = torch.empty((kda.chunk_prefill_workspace_size(1, T, H, D, D, states=True),), dtype=torch.uint8,
                     device="cuda")
    run = lambda: kda.chunk_prefill(q, k, v, g, beta, st0, out=o, final_state=fs, states=states, workspace=ws)
    tc = _median_pair_us({"chunked": run}, reps=5)["chunked"] * 1e-6
    del states
    return {"T": T, "H": H, "avg_call_us": t * 1e6, "algorithmic_bytes": nbytes, "achieved": nbytes / t / 1e9,
            "unit": "GB/s", "frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
            "chunked": {"avg_call_us": tc * 1e6, "achieved": nbytes / tc / 1e9, "unit": "GB/s",
                        "frac": nbytes / tc / 1e9 / HBM_PEAK_GBPS}}


def time_layer_exit(kda, rows: int = B_DECODE, N: int = 7168, reps: int = 10) -> dict:
    """The layer's exit at decode (gated norm of the 96 heads, then the 12,288 -> 7,168
    output projection) for one new token per row, timed on its own; torch's bf16 Linear
    on the same normed rows is timed beside it for reference."""
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    K = H * D
    o = torch.randn((rows, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    gate = torch.randn((rows, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    w = (1.0 + 0.1 * torch.randn((D,), generator=gen, device="cuda")).float()
    W = ((torch.rand((N, K), generator=gen, device="cuda") * 2 - 1) / K ** 0.5).to(torch.bfloat16)
    y = torch.empty((rows, K), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((rows, N), dtype=torch.bfloat16, device="cuda")

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps
    nws = kda.load_library().kda_out_proj_workspace_size(rows, K, N)
    ws = torch.empty((max(nws, 1),), dtype=torch.uint8, device="cuda")
    t = timed(lambda: kda.gated_norm_proj(o, gate, w, W, 1e-6, y=y, out=out, workspace=ws))
    t_proj = timed(lambda: kda.out_proj(y, W, out=out, workspace=ws))
    t_ref = timed(lambda: torch.nn.functional.linear(y, W))
    nbytes = N * K * 2 + rows * K * 2 * 3 + rows * N * 2 + D * 4
    return {"rows": rows, "in_features": K, "out_features": N, "avg_call_us": t * 1e6, "algorithmic_bytes": nbytes,
            "achieved": nbytes / t / 1e9, "unit": "GB/s", "frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
            "projection_us": t_proj * 1e6, "torch_linear_us": t_ref * 1e6}


def time_fused_norm_scan(kda, P, ws, o, fs, y, reps: int = 10) -> float:
    """Average duration of the scan that applies the gated norm itself, over the records
    the step's preparation left in ws, from HIP events on the current stream."""
    def call():
        kda.chunk_scan(P["v"], ws, out=o, final_state=fs, gate=P["gate"], norm_weight=P["w"], norm_eps=P["eps"], y=y)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def time_prefill_y_only(kda, P, ws, fs, y, reps: int = 10) -> dict:
    """The T=8192 prefill with the gated norm when the caller wants y alone (no head
    outputs): the preparation, the scan writing its head outputs into y, and the norm in
    place.  Timed on its own with HIP events; not part of the step."""
    def call():
        kda.chunk_prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], gate=P["gate"], norm_weight=P["w"],
                          norm_eps=P["eps"], head_outputs=False, final_state=fs, y=y, workspace=ws)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    nbytes = _bytes_prefill(T_PREFILL, H, D, False, norm=True) - T_PREFILL * H * D * 2   # no o written
    return {"avg_call_us": t * 1e6, "tokens_per_s": T_PREFILL / t, "algorithmic_bytes": nbytes,
            "achieved_GBps": nbytes / t / 1e9}


def _bytes_decode_state(B: int, H: int, d: int) -> int:
    return 2 * B * H * d * d * 4               # state read + written (fp32)


def _bytes_decode_io(B: int, H: int, d: int) -> int:
    # q, k, v, gate (bf16) + g (fp32) + beta read; o, y (bf16) written
    return B * H * (4 * d * 2 + d * 4 + 4 + 2 * d * 2)


CSRC = os.path.join(ROOT, "linear_attention_recurrence_07_amd", "csrc")
KERNEL_SOURCES = {
    "chunk_prep_kernel": ["chunk_prep.hip", "kda_chunk.h", "kda_device.h"],
    "chunk_scan_kernel": ["chunk_scan.hip", "kda_chunk.h", "kda_device.h"],
    "recurrent_kernel": ["recurrent.hip", "kda_device.h"],
    "gated_rmsnorm_kernel": ["gated_rmsnorm.hip", "kda_device.h"],
}
COUNTERS_FILE = os.path.join(ROOT, "profiles", "bench_T8192_B64_hbm_counters.md")
MFMA_FILE = os.path.join(ROOT, "profiles", "bench_T8192_B64_mfma_counters.md")
MFMA_PEAK_TFLOPS = 2500.0     # dense bf16 / fp16


def source_digest(kernel: str) -> str:
    """First 16 hex digits of the SHA-256 of the sources a kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_lines(path: str, tag: str) -> dict:
    """Lines `tag kernel digest value...` of a committed profile summary whose kernel
    sources still match the recorded digest."""
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and f[0] == tag and f[1] in KERNEL_SOURCES and source_digest(f[1]) == f[2]:
            out[f[1]] = [float(x) for x in f[3:]]
    return out


def measured_mfma() -> dict:
    """Matrix-core work per launch from the committed rocprofv3 summary
    (SQ_INSTS_VALU_MFMA_MOPS_* x 512 flop, and SQ_VALU_MFMA_BUSY_CYCLES as a share of
    all SIMD-cycles of the launch), for kernels unchanged since it was taken."""
    return {k: {"flops_per_launch": v[0], "busy_pct": v[1]} for k, v in _profile_lines(MFMA_FILE, "mfma").items()}


def _algorithmic_flops(T: int, H: int, d: int, chunk: int) -> float:
    """Flops the chunked form needs per launch: the three state contractions (6 d^2 per
    token), the intra-chunk products (2 C (dk + dv)) and the triangular solve (C^2 / 3)."""
    return float(T) * H * (6 * d * d + 2 * chunk * 2 * d + chunk * chunk / 3.0)


def ceilings() -> dict:
    """Practical ceilings on this GPU: a plain streaming kernel (torch.neg over 1 GiB of
    bf16: 1 GiB read + 1 GiB written) and a large bf16 GEMM (torch.mm, 8192^3)."""
    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps
    src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t_copy = timed(lambda: torch.neg(src, out=dst))
    del src, dst
    n = 8192
    a = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    t_mm = timed(lambda: torch.mm(a, b, out=c))
    del a, b, c
    return {"copy_GBps": 2 * (1 << 30) / t_copy / 1e9, "gemm_bf16_TFLOPs": 2.0 * n ** 3 / t_mm / 1e12,
            "how": "torch.neg over 1 GiB bf16 (read + write); torch.mm bf16 8192x8192x8192"}


def measured_traffic() -> dict:
    """HBM bytes per launch from the committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE, each scaled by the factor a plain streaming kernel of known size gives),
    for each kernel whose sources still match the digest recorded with the counters;
    kernels changed since then get no entry (their traffic is reported as null)."""
    out = {}
    if not os.path.exists(COUNTERS_FILE):
        return out
    for line in open(COUNTERS_FILE):
        f = line.split()
        if len(f) == 4 and f[0] == "traffic" and f[1] in KERNEL_SOURCES:
            if source_digest(f[1]) == f[2]:
                out[f[1]] = int(f[3])
    return out


def _dev_randn(shape, gen, dtype, std=1.0, mean=0.0):
    return (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32) * std + mean).to(dtype)


def _unit_rows(x):
    return x / x.float().norm(dim=-1, keepdim=True).to(x.dtype)


def make_prefill_inputs(seed: int = 0):
    """The headline prompt, drawn by the shared seeded generator (numpy), then copied."""
    from gen import inputs as gi
    x = gi.prefill(T=T_PREFILL, seed=seed, norm=True)

    def t(a, bf):
        if bf:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    return dict(q=t(x.q, True), k=t(x.k, True), v=t(x.v, True), g=t(x.g, False),
                beta=t(x.beta, False), gate=t(x.gate, True), w=t(x.norm_weight, False),
                eps=x.norm_eps)


def make_decode_inputs(seed: int = 0):
    """Decode rows: a 1000-token prompt per row drawn on the device (same distributions as
    the shared generator: unit-length q/k, N(0,1) v, U[-5,0) g, sigmoid(N(0,1)) beta),
    prefilled on the GPU to produce the fp32 state, then one new token per row."""
    import linear_attention_recurrence_07_amd as kda
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 1000)
    state = torch.empty((B_DECODE, H, D, D), dtype=torch.float32, device="cuda")
    rows = 8
    for r0 in range(0, B_DECODE, rows):
        shp = (rows, P_DECODE, H, D)
        q = _unit_rows(_dev_randn(shp, gen, torch.bfloat16))
        k = _unit_rows(_dev_randn(shp, gen, torch.bfloat16))
        v = _dev_randn(shp, gen, torch.bfloat16)
        g = torch.rand(shp, generator=gen, device="cuda") * -5.0
        beta = torch.sigmoid(torch.randn((rows, P_DECODE, H), generator=gen, device="cuda"))
        # fp32 head outputs (discarded): keeps these launches apart from the timed bf16 ones
        kda.chunk_prefill(q, k, v, g, beta, final_state=state[r0:r0 + rows], output_dtype=torch.float32)
        del q, k, v, g, beta
    shp = (B_DECODE, 1, H, D)
    step = dict(q=_unit_rows(_dev_randn(shp, gen, torch.bfloat16)),
                k=_unit_rows(_dev_randn(shp, gen, torch.bfloat16)),
                v=_dev_randn(shp, gen, torch.bfloat16),
                g=torch.rand(shp, generator=gen, device="cuda") * -5.0,
                beta=torch.sigmoid(torch.randn((B_DECODE, 1, H), generator=gen, device="cuda")),
                gate=_dev_randn(shp, gen, torch.bfloat16),
                w=(1.0 + 0.1 * torch.randn((D,), generator=gen, device="cuda")).float())
    torch.cuda.synchronize()
    return state, step


def cpu_baseline(seed: int = 0, tokens: int = T_PREFILL, min_seconds: float = 10.0):
    """The fp64 oracle (C, OpenMP over heads) over the first `tokens` tokens of the same
    prompt, all 96 heads, timed on this host's cores; whole passes are repeated until at
    least `min_seconds` have elapsed."""
    from gen import inputs as gi
    from oracle import cref
    x = gi.prefill(T=tokens, seed=seed)
    threads = cref.max_threads()
    cref.recurrence(x.q[:, :64], x.k[:, :64], x.v[:, :64], x.g[:, :64], x.beta[:, :64],
                    in_dtype="bf16")                     # warm the library and threads
    passes = 0
    t0 = time.perf_counter()
    while True:
        cref.recurrence(x.q, x.k, x.v, x.g, x.beta, in_dtype="bf16", num_threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    # one thread on a short cut of the same prompt, for the per-core rate
    cut = 256
    t1 = time.perf_counter()
    cref.recurrence(x.q[:, :cut], x.k[:, :cut], x.v[:, :cut], x.g[:, :cut], x.beta[:, :cut], in_dtype="bf16",
                    num_threads=1)
    one = cut / (time.perf_counter() - t1)
    return {"value": passes * tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} pass(es) over the first {tokens} tokens of the T={T_PREFILL} prompt, "
                      f"all {H} heads (fp64 token-by-token recurrence, {dt:.1f} s)",
            "one_thread_tokens_per_s": one, "one_thread_sample": f"first {cut} tokens, all {H} heads",
            "cpu": _cpu_model()}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--counters", action="store_true",
                    help="first run a plain streaming kernel of known size (1 GiB read, 1 GiB written), "
                         "the reference for scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this build runs on one GPU "
              "(no collectives or sharding).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import linear_attention_recurrence_07_amd as kda
    kda.load_library()
    if args.counters:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    print("[bench] generating prefill inputs", file=sys.stderr, flush=True)
    P = make_prefill_inputs()
    print("[bench] generating decode state (64 x 1000-token prompts on the GPU)", file=sys.stderr, flush=True)
    state0, S = make_decode_inputs()
    state = state0.clone()
    o = torch.empty((1, T_PREFILL, H, D), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(o)
    fs = torch.empty((1, H, D, D), dtype=torch.float32, device="cuda")
    ws = torch.empty((kda.chunk_prefill_workspace_size(1, T_PREFILL, H, D, D),), dtype=torch.uint8, device="cuda")
    od = torch.empty((B_DECODE, 1, H, D), dtype=torch.bfloat16, device="cuda")
    yd = torch.empty_like(od)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        kda.chunk_prepare(P["q"], P["k"], P["g"], P["beta"], workspace=ws)
        mark(1)
        kda.chunk_scan(P["v"], ws, out=o, final_state=fs)
        mark(2)
        kda.gated_rmsnorm(o, P["gate"], P["w"], P["eps"], out=y)
        mark(3)
        kda.recurrent_step(S["q"], S["k"], S["v"], S["g"], S["beta"], state, gate=S["gate"],
                           norm_weight=S["w"], out=od, y=yd)
        mark(4)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dur = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e-3 for j in range(4)]
    t_prep, t_scan, t_nrm, t_dec = dur
    ms_step = wall * 1e3 / args.steps
    b_prep = _bytes_prep(T_PREFILL, H, D)
    b_scan = _bytes_scan(T_PREFILL, H, D, False)
    b_path = _bytes_prefill(T_PREFILL, H, D, False)
    b_nrm = _bytes_norm(T_PREFILL * H, D)
    b_dec = _bytes_decode_state(B_DECODE, H, D)
    b_dec_all = b_dec + _bytes_decode_io(B_DECODE, H, D)

    traffic = measured_traffic()
    mfma = measured_mfma()
    print("[bench] scan with its own gated norm", file=sys.stderr, flush=True)
    t_fused = time_fused_norm_scan(kda, P, ws, o, fs, y)
    print("[bench] prefill with y alone", file=sys.stderr, flush=True)
    y_only = time_prefill_y_only(kda, P, ws, fs, y)
    y_only["step_prepare_scan_norm_us"] = (t_prep + t_scan + t_nrm) * 1e6
    print("[bench] copy and GEMM ceilings", file=sys.stderr, flush=True)
    ceil = ceilings()
    print("[bench] short convolution", file=sys.stderr, flush=True)
    conv = time_short_conv(kda)
    print("[bench] prefill with the short convolution fused", file=sys.stderr, flush=True)
    pconv = time_prefill_conv(kda, P, ws, o, fs, y)
    print("[bench] decode step with the short convolution fused", file=sys.stderr, flush=True)
    dconv = time_decode_conv(kda, S, state0)
    print("[bench] prefill with one decay per head", file=sys.stderr, flush=True)
    per_head = time_per_head_decay(kda, P, ws, o, fs)
    print("[bench] per-token states", file=sys.stderr, flush=True)
    rec_states = time_recurrent_states(kda)
    print("[bench] layer exit (gated norm + output projection)", file=sys.stderr, flush=True)
    exit_ = time_layer_exit(kda)

    def roof(kernel, nbytes, t, **extra):
        gbs = nbytes / t / 1e9
        r = {"bound": "hbm", "kernel": kernel, "achieved": gbs, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": gbs / HBM_PEAK_GBPS, "traffic": traffic.get(kernel), "algorithmic_bytes_per_launch": nbytes,
             "avg_launch_us": t * 1e6, "frac_of_copy_ceiling": gbs / ceil["copy_GBps"], **extra}
        if kernel in mfma:
            tf = mfma[kernel]["flops_per_launch"] / t / 1e12
            r["mfma"] = {"flops_per_launch": mfma[kernel]["flops_per_launch"], "achieved_tflops": tf,
                         "peak_tflops": MFMA_PEAK_TFLOPS, "frac": tf / MFMA_PEAK_TFLOPS,
                         "frac_of_gemm_ceiling": tf / ceil["gemm_bf16_TFLOPs"],
                         "busy_pct_rocprof": mfma[kernel]["busy_pct"]}
        return r

    r_prep = roof("chunk_prep_kernel", b_prep, t_prep)
    r_scan = roof("chunk_scan_kernel", b_scan, t_scan)
    prefill_tok_s = T_PREFILL / (t_prep + t_scan + t_nrm)
    # The headline roofline: the whole prefill that `value` times (preparation + scan +
    # gated norm) against the bytes the problem itself moves -- q, k, v, g, beta, gate in,
    # o, y and the final state out, each once -- and the summed launch durations.  The
    # chunk records and o's second read are the design's own traffic: they show in
    # `traffic` (the calibrated counters of the three launches), not in `achieved`.
    t_path = t_prep + t_scan + t_nrm
    b_path_norm = _bytes_prefill(T_PREFILL, H, D, False, norm=True)
    path_kernels = ("chunk_prep_kernel", "chunk_scan_kernel", "gated_rmsnorm_kernel")
    path_traffic = sum(traffic[k] for k in path_kernels) if all(k in traffic for k in path_kernels) else None
    flops = _algorithmic_flops(T_PREFILL, H, D, CHUNK)
    headline = {
        "bound": "hbm", "kernel": " + ".join(path_kernels), "achieved": b_path_norm / t_path / 1e9,
        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": b_path_norm / t_path / 1e9 / HBM_PEAK_GBPS,
        "traffic": path_traffic, "traffic_over_algorithmic": None if path_traffic is None else path_traffic / b_path_norm,
        "algorithmic_bytes_per_launch": b_path_norm, "avg_launch_us": t_path * 1e6,
        "launch_us": {"chunk_prep_kernel": t_prep * 1e6, "chunk_scan_kernel": t_scan * 1e6,
                      "gated_rmsnorm_kernel": t_nrm * 1e6},
        "frac_of_copy_ceiling": b_path_norm / t_path / 1e9 / ceil["copy_GBps"],
        "mfma": {"algorithmic_flops_per_launch": flops, "achieved_tflops": flops / t_path / 1e12,
                 "peak_tflops": MFMA_PEAK_TFLOPS, "frac": flops / t_path / 1e12 / MFMA_PEAK_TFLOPS,
                 "target_frac": 0.40,
                 "busy_pct_rocprof": {k: mfma[k]["busy_pct"] for k in path_kernels if k in mfma}},
    }
    out = {
        "metric": METRIC,
        "value": prefill_tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"KDA prefill B=1 T={T_PREFILL} H={H} dk=dv={D} bf16 (+ gated RMSNorm) "
                               f"and one decode step B={B_DECODE} on an fp32 state after P={P_DECODE}",
                   "global_batch": 1, "seq_len": T_PREFILL, "heads": H, "head_dim": D,
                   "decode_batch": B_DECODE, "chunk": CHUNK, "parallelism": "single-gpu"},
        "prefill_prepare_ms": t_prep * 1e3,
        "prefill_scan_ms": t_scan * 1e3,
        "gated_norm_ms": t_nrm * 1e3,
        "decode_step_ms": t_dec * 1e3,
        "decode_state_GBps": b_dec / t_dec / 1e9,
        "decode_total_GBps": b_dec_all / t_dec / 1e9,
        # the prefill that `value` times, against the problem's own bytes (see above)
        "roofline": headline,
        # the same without the norm: preparation + scan against q, k, v, g, beta, o, state
        "roofline_prefill_without_norm": roof("chunk_prep_kernel + chunk_scan_kernel", b_path, t_prep + t_scan),
        # each launch against the bytes it moves itself, INCLUDING the workspace records
        # the preparation writes and the scan reads back (the two-launch design's traffic)
        "roofline_prepare_incl_workspace_records": r_prep,
        "roofline_scan_incl_workspace_records": r_scan,
        "roofline_decode": roof("recurrent_kernel", b_dec_all, t_dec),
        "roofline_norm": roof("gated_rmsnorm_kernel", b_nrm, t_nrm),
        # the scan applying the gated norm itself (kda_chunk_scan with gate and y), timed on
        # its own, against the step's scan + separate norm
        "scan_with_fused_norm": {"avg_call_us": t_fused * 1e6, "scan_plus_norm_us": (t_scan + t_nrm) * 1e6,
                                 "algorithmic_bytes": _bytes_scan(T_PREFILL, H, D, False, norm=True),
                                 "achieved_GBps": _bytes_scan(T_PREFILL, H, D, False, norm=True) / t_fused / 1e9},
        # the prefill + norm when only y is wanted (head outputs written into y, then the
        # norm in place), timed on its own against the step's preparation + scan + norm
        "prefill_y_only": y_only,
        "ceilings": ceil,
        # the causal short convolution in front of the kernel, timed on its own (two
        # launches per call: the filter over all tokens, then the carried-input update)
        "short_conv": conv,
        "prefill_conv": pconv,
        "decode_conv": dconv,
        # the same prefill with g [1, T, H] (one decay per head), timed on its own
        "prefill_per_head_decay": per_head,
        # the token-by-token kernel storing the state after every token, timed on its own
        "recurrent_states": rec_states,
        # the gated norm + output projection of one decode token per row, timed on its own
        "layer_exit_decode": exit_,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(tokens=args.cpu_tokens, min_seconds=args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
