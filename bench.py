"""Benchmark of the KDA mixer core on one MI355X.

One step = the whole hot path on one batch of synthetic input:
  1. chunked prefill of one 8192-token prompt at the 96-head, 128-dim layer shape
     (bf16 q/k/v, fp32 g and beta, no initial state) -> head outputs + final state;
  2. the sigmoid-gated RMSNorm over those head outputs;
  3. one decode step for 64 rows (one new token each) on an fp32 state [64, 96, 128, 128]
     produced beforehand by prefilling a 1000-token prompt per row, with the gated norm.
Inputs are resident in HBM before timing starts.  Kernel durations come from HIP events
recorded on the stream the kernels run on.

Prints one JSON line.  `value` is prefill tokens/s; the decode state bandwidth and the
per-kernel rooflines ride along.  --gpus above 1 is refused: this build runs on one GPU.
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
B_DECODE, P_DECODE = 64, 1000


def _bytes_prefill(T: int, H: int, d: int, with_init: bool) -> int:
    """Algorithmic HBM bytes of one prefill launch: q, k, v (bf16), g (fp32), beta (fp32)
    read, o (bf16) written, final state (fp32) written (+ read when an initial state is
    given)."""
    per_tok_head = 3 * d * 2 + d * 4 + 4 + d * 2
    state = H * d * d * 4
    return T * H * per_tok_head + state * (2 if with_init else 1)


def _bytes_norm(rows: int, d: int) -> int:
    return rows * d * 2 * 3 + d * 4            # o and gate read, y written (bf16)


def _bytes_decode_state(B: int, H: int, d: int) -> int:
    return 2 * B * H * d * d * 4               # state read + written (fp32)


def _bytes_decode_io(B: int, H: int, d: int) -> int:
    # q, k, v, gate (bf16) + g (fp32) + beta read; o, y (bf16) written
    return B * H * (4 * d * 2 + d * 4 + 4 + 2 * d * 2)


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
    return {"value": passes * tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} pass(es) over the first {tokens} tokens of the T={T_PREFILL} prompt, "
                      f"all {H} heads (fp64 token-by-token recurrence, {dt:.1f} s)",
            "cpu": platform.processor() or platform.machine()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
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
        if ev is not None:
            ev[0].record()
        kda.chunk_prefill(P["q"], P["k"], P["v"], P["g"], P["beta"], out=o, final_state=fs, workspace=ws)
        if ev is not None:
            ev[1].record()
        kda.gated_rmsnorm(o, P["gate"], P["w"], P["eps"], out=y)
        if ev is not None:
            ev[2].record()
        kda.recurrent_step(S["q"], S["k"], S["v"], S["g"], S["beta"], state, gate=S["gate"],
                           norm_weight=S["w"], out=od, y=yd)
        if ev is not None:
            ev[3].record()

    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pre = [e[0].elapsed_time(e[1]) for e in evs]
    nrm = [e[1].elapsed_time(e[2]) for e in evs]
    dec = [e[2].elapsed_time(e[3]) for e in evs]
    ms_step = wall * 1e3 / args.steps
    t_pre = float(np.mean(pre)) * 1e-3
    t_nrm = float(np.mean(nrm)) * 1e-3
    t_dec = float(np.mean(dec)) * 1e-3
    b_pre = _bytes_prefill(T_PREFILL, H, D, False)
    b_dec = _bytes_decode_state(B_DECODE, H, D)
    b_dec_all = b_dec + _bytes_decode_io(B_DECODE, H, D)
    prefill_tok_s = T_PREFILL / (t_pre + t_nrm)
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
                   "decode_batch": B_DECODE, "chunk": 32, "parallelism": "single-gpu"},
        "prefill_kernel_ms": t_pre * 1e3,
        "gated_norm_ms": t_nrm * 1e3,
        "decode_step_ms": t_dec * 1e3,
        "decode_state_GBps": b_dec / t_dec / 1e9,
        "decode_total_GBps": b_dec_all / t_dec / 1e9,
        "roofline": {"bound": "hbm", "kernel": "prefill_mfma_kernel", "achieved": b_pre / t_pre / 1e9,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": b_pre / t_pre / 1e9 / HBM_PEAK_GBPS,
                     "traffic": None, "algorithmic_bytes_per_launch": b_pre},
        "roofline_decode": {"bound": "hbm", "kernel": "recurrent_kernel", "achieved": b_dec_all / t_dec / 1e9,
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": b_dec_all / t_dec / 1e9 / HBM_PEAK_GBPS, "traffic": None,
                            "algorithmic_bytes_per_launch": b_dec_all},
        "roofline_norm": {"bound": "hbm", "kernel": "gated_rmsnorm_kernel",
                          "achieved": _bytes_norm(T_PREFILL * H, D) / t_nrm / 1e9, "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": _bytes_norm(T_PREFILL * H, D) / t_nrm / 1e9 / HBM_PEAK_GBPS},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(tokens=args.cpu_tokens, min_seconds=args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
