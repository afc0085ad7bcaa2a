"""GPU parity of the short convolution fused into the KDA kernels' prologue
(kda_chunk_prefill_conv, kda_recurrent_step_conv): q, k and v go in as the raw
projections and the kernels run the causal width-W filter + SiLU themselves, carrying the
last W-1 inputs of every sequence (Kimi-K3 atlas, KDA layer page, kda-init code; nnterp
Kimi-Linear page, Notes on KDA).

Every case is held to the oracle chain on the same seeded inputs: oracle/short_conv.py on
the raw q, k, v in fp64, then the C fp64 recurrence (and the fp64 gated norm) on the
filtered values, within 2e-2 of rms.  The kernels keep the filtered values in fp32 and
never round them to bf16, so the chain does not either.  (Rounding them on both sides
would compare different inputs: these head outputs are about 200 times smaller than v,
one bf16 unit of a filtered v or k at a sensitive token moves an output by 2-3% of rms,
and a value computed in fp32 on the GPU and in fp64 in the oracle lands on either side of
a bf16 rounding midpoint now and then.)  The carried inputs after the call are copies of
inputs and must match exactly, and bit for bit those of kda_short_conv.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import cref
from oracle import kda_ref as R
from oracle import short_conv as C

from tests import kda_testutil as U

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = U.BF16_TOL


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not U.gpu_available():
        pytest.fail("GPU tests need an MI355X; run them with -m gpu on a GPU host")
    import linear_attention_recurrence_07_amd as kda
    kda.load_library()


def _conv_dev(lc: gi.LayerConv, in_dtype: str):
    ws = tuple(torch.from_numpy(np.ascontiguousarray(w)).to(DEV) for w in lc.weights)
    init = None if lc.initial is None else tuple(U.to_torch(a, in_dtype, DEV) for a in lc.initial)
    return ws, init


def _kw(x: gi.KdaInputs, d: dict, norm: bool, chunk: int):
    return dict(cu_seqlens=d["cu_seqlens"], attention_mask=d["mask"], gate=d["gate"] if norm else None,
                norm_weight=d["norm_weight"] if norm else None, norm_eps=x.norm_eps, chunk=chunk,
                output_dtype=torch.float32)


def run_fused(x: gi.KdaInputs, lc: gi.LayerConv, *, norm: bool, chunk: int = 0, in_place: bool = False,
              activation="silu", head_outputs: bool = True):
    """kda_chunk_prefill_conv; returns (o, final_state, y, (q, k, v) carried inputs) on the GPU."""
    import linear_attention_recurrence_07_amd as kda
    d = U.device_inputs(x, DEV)
    ws, init = _conv_dev(lc, x.in_dtype)
    res = kda.chunk_prefill_conv(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], conv_weights=ws,
                                 conv_state=init, conv_final_state=init if in_place else None,
                                 activation=activation, head_outputs=head_outputs, **_kw(x, d, norm, chunk))
    torch.cuda.synchronize()
    o, fs = res[0], res[1]
    y = res[2] if norm else None
    return o, fs, y, res[-1]


def run_two_step(x: gi.KdaInputs, lc: gi.LayerConv, *, norm: bool, chunk: int = 0, activation="silu",
                 head_outputs: bool = True):
    """kda_short_conv on q, k and v (outputs in the input dtype), then kda_chunk_prefill."""
    import linear_attention_recurrence_07_amd as kda
    d = U.device_inputs(x, DEV)
    ws, init = _conv_dev(lc, x.in_dtype)
    filt, fins = [], []
    for i, name in enumerate("qkv"):
        t = d[name]
        B, T, H, dd = t.shape
        out = torch.zeros((B, T, H * dd), dtype=t.dtype, device=DEV)
        yv, fs = kda.short_conv(t.reshape(B, T, H * dd), ws[i], None if init is None else init[i],
                                cu_seqlens=d["cu_seqlens"], attention_mask=d["mask"], activation=activation, out=out)
        filt.append(yv.reshape(B, T, H, dd))
        fins.append(fs)
    res = kda.chunk_prefill(filt[0], filt[1], filt[2], d["g"], d["beta"], d["initial_state"],
                            head_outputs=head_outputs, **_kw(x, d, norm, chunk))
    torch.cuda.synchronize()
    return res[0], res[1], (res[2] if norm else None), tuple(fins)


def oracle_chain(x: gi.KdaInputs, lc: gi.LayerConv, heads=None, *, norm: bool, activation="silu"):
    """fp64 filters on the raw projections of `heads`, then the C fp64 recurrence and the
    gated norm on the filtered values (handed over in fp32).  Returns (o, final_state, y,
    carried inputs over the heads' channels)."""
    heads = list(range(x.H)) if heads is None else list(heads)
    filt, fins = [], []
    for i, name in enumerate("qkv"):
        dd = x.dv if name == "v" else x.dk
        ch = np.concatenate([np.arange(h * dd, (h + 1) * dd) for h in heads])
        raw = gi.to_f64(getattr(x, name)[:, :, heads], x.in_dtype).reshape(x.B, x.T, len(heads) * dd)
        init = None if lc.initial is None else gi.to_f64(lc.initial[i], x.in_dtype)[..., ch]
        y, fin = C.short_conv(raw, lc.weights[i][ch], init, cu_seqlens=x.cu_seqlens, mask=x.mask,
                              activation=activation)
        filt.append(y.reshape(x.B, x.T, len(heads), dd).astype(np.float32))
        fins.append(fin)
    init = None if x.initial_state is None else x.initial_state[:, heads]
    o, fs = cref.recurrence(filt[0], filt[1], filt[2], x.g[:, :, heads], x.beta[:, :, heads], init,
                            in_dtype=gi.F32, mask=x.mask, cu_seqlens=x.cu_seqlens)
    y = None
    if norm:
        y = R.gated_rmsnorm(o, gi.to_f64(x.gate[:, :, heads], x.in_dtype), x.norm_weight, x.norm_eps)
        if x.mask is not None:
            y[x.mask == 0] = 0.0
    return o, fs, y, fins


def _sel(t: torch.Tensor, heads, axis):
    if heads is None:
        return t
    return t.index_select(axis, torch.tensor(list(heads), device=t.device))


def _chan(t: torch.Tensor, heads, d):
    if heads is None:
        return t
    ch = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    return t.index_select(-1, torch.from_numpy(ch).to(t.device))


def check_against_oracle(tag, x, lc, fused, heads=None, *, norm: bool, activation="silu"):
    o, fs, y, fins = fused
    ro, rfs, ry, rfins = oracle_chain(x, lc, heads, norm=norm, activation=activation)
    v = U.valid_token_mask(x)
    U.assert_close(f"{tag} o", U.to_numpy64(_sel(o, heads, 2))[v], ro[v], TOL)
    U.assert_close(f"{tag} final state", U.to_numpy64(_sel(fs, heads, 1)), rfs, TOL)
    if norm:
        U.assert_close(f"{tag} y", U.to_numpy64(_sel(y, heads, 2))[v], ry[v], TOL)
    for name, got, ref, dd in zip("qkv", fins, rfins, (x.dk, x.dk, x.dv)):
        assert np.array_equal(U.to_numpy64(_chan(got, heads, dd)), ref), f"{tag}: carried {name} inputs"


def check_carried(tag, fused, two):
    """The carried inputs after the call equal kda_short_conv's bit for bit."""
    for name, a, b in zip("qkv", fused[3], two[3]):
        assert torch.equal(a, b), f"{tag}: carried {name} inputs differ from kda_short_conv's"


def _layout_case(name):
    H, d = 4, 128
    if name == "plain":
        x = gi.make_inputs("conv_plain", B=1, T=300, H=H, dk=d, dv=d, seed=11, norm=True, normalize_qk=False)
        return x, gi.layer_conv(x, seed=11), dict(norm=True)
    if name == "batched_state":
        x = gi.make_inputs("conv_batched", B=2, T=77, H=H, dk=d, dv=d, seed=12, norm=True, normalize_qk=False,
                           initial_state_std=0.02)
        return x, gi.layer_conv(x, seed=12, with_state=True), dict(norm=True)
    if name == "packed":
        lengths = [1, 2, 3, 40, 0, 97, 33]       # shorter than the window, empty, several chunks
        cu = gi.varlen_cu_seqlens(lengths)
        x = gi.make_inputs("conv_packed", B=1, T=int(cu[-1]) + 5, H=H, dk=d, dv=d, seed=13, norm=True,
                           normalize_qk=False, initial_state_std=0.02, cu_seqlens=cu)
        return x, gi.layer_conv(x, seed=13, with_state=True), dict(norm=True)
    if name == "masked":
        rng = np.random.default_rng(14)
        mask = np.ones((3, 150), np.uint8)
        mask[0, :37] = 0                          # left padding
        mask[1] = rng.random(150) > 0.3           # holes everywhere
        mask[2, 5:120] = 0                        # a long run of padding across several chunks
        x = gi.make_inputs("conv_masked", B=3, T=150, H=H, dk=d, dv=d, seed=14, norm=True, normalize_qk=False,
                           initial_state_std=0.02, mask=mask)
        return x, gi.layer_conv(x, seed=14, with_state=True), dict(norm=True)
    if name == "chunk64_head_decay":
        x = gi.make_inputs("conv_c64", B=1, T=200, H=H, dk=d, dv=d, seed=15, normalize_qk=False,
                           decay_per_head=True)
        return x, gi.layer_conv(x, seed=15, with_state=True), dict(norm=False, chunk=64)
    if name in ("width2", "width3"):
        W = int(name[-1])
        x = gi.make_inputs(f"conv_{name}", B=2, T=90, H=H, dk=d, dv=d, seed=16 + W, norm=True, normalize_qk=False)
        return x, gi.layer_conv(x, width=W, seed=16 + W, with_state=True), dict(norm=True)
    if name == "no_activation":
        x = gi.make_inputs("conv_noact", B=1, T=130, H=H, dk=d, dv=d, seed=19, normalize_qk=False)
        return x, gi.layer_conv(x, seed=19, with_state=True), dict(norm=False, activation=None)
    raise KeyError(name)


LAYOUTS = ["plain", "batched_state", "packed", "masked", "chunk64_head_decay", "width2", "width3", "no_activation"]


@pytest.mark.parametrize("name", LAYOUTS)
def test_fused_prefill_layouts(name):
    x, lc, opt = _layout_case(name)
    norm, chunk, act = opt["norm"], opt.get("chunk", 0), opt.get("activation", "silu")
    U.log(f"fused conv prefill {name}: B={x.B} T={x.T} H={x.H} W={lc.width} chunk={chunk} norm={norm}")
    fused = run_fused(x, lc, norm=norm, chunk=chunk, activation=act)
    check_carried(name, fused, run_two_step(x, lc, norm=norm, chunk=chunk, activation=act))
    check_against_oracle(name, x, lc, fused, norm=norm, activation=act)


def test_fused_prefill_in_place_and_y_only():
    x, lc, _ = _layout_case("masked")
    U.log("fused conv prefill: carried inputs updated in place; y alone")
    ref = run_fused(x, lc, norm=True)
    inp = run_fused(x, lc, norm=True, in_place=True)
    vm = torch.from_numpy(U.valid_token_mask(x)).to(DEV)
    assert torch.equal(inp[0][vm], ref[0][vm]) and torch.equal(inp[1], ref[1]) and torch.equal(inp[2][vm], ref[2][vm])
    check_carried("in place", inp, ref)
    yo = run_fused(x, lc, norm=True, head_outputs=False)
    assert yo[0] is None
    assert torch.equal(yo[1], ref[1])
    # y alone: the head outputs pass through y and are normalised there in place, the same
    # arithmetic as writing o and normalising it
    check_carried("y only", yo, ref)
    assert torch.equal(yo[2][vm], ref[2][vm])


def test_fused_prefill_config2_all_heads():
    """Single-prompt prefill shape (B=1, T=2048, H=96, d=128, chunk 64), raw projections,
    prompt start (no carried inputs, no state)."""
    x = gi.make_inputs("conv_cfg2", B=1, T=2048, H=96, dk=128, dv=128, chunk=64, seed=21, normalize_qk=False)
    lc = gi.layer_conv(x, seed=21)
    U.log("fused conv prefill config-2 shape")
    fused = run_fused(x, lc, norm=False, chunk=64)
    check_carried("cfg2", fused, run_two_step(x, lc, norm=False, chunk=64))
    check_against_oracle("cfg2", x, lc, fused, norm=False)


def test_fused_prefill_config3_packed_all_heads():
    """Batched varlen shape: lengths 8192/6000/3000/777 packed with cu_seqlens, carried
    state N(0, 0.02) and carried convolution inputs, fused gated norm; all 96 heads against
    the oracle in batches of 24."""
    cu = gi.varlen_cu_seqlens()
    x = gi.make_inputs("conv_cfg3", B=1, T=int(cu[-1]), H=96, dk=128, dv=128, chunk=64, seed=22,
                       initial_state_std=0.02, num_seqs=len(cu) - 1, norm=True, cu_seqlens=cu, normalize_qk=False)
    lc = gi.layer_conv(x, seed=22, with_state=True)
    U.log("fused conv prefill config-3 shape (packed)")
    fused = run_fused(x, lc, norm=True, chunk=64)
    check_carried("cfg3", fused, run_two_step(x, lc, norm=True, chunk=64))
    for h0 in range(0, x.H, 24):
        check_against_oracle(f"cfg3 heads {h0}..{h0 + 23}", x, lc, fused, list(range(h0, h0 + 24)), norm=True)


def test_fused_prefill_config5_long():
    """Long-context shape (T=65,536, H=96, g near the lower bound on half the heads, fused
    norm): eight heads (one per XCD residue of the scan's work-group mapping) against the
    oracle, every head's carried inputs against kda_short_conv's."""
    x = gi.make_inputs("conv_cfg5", B=1, T=65536, H=96, dk=128, dv=128, chunk=64, seed=23, normalize_qk=False,
                       norm=True, g_ranges_by_head=[(-5.0, -3.0)] * 48 + [(-0.05, 0.0)] * 48)
    lc = gi.layer_conv(x, seed=23)
    U.log("fused conv prefill config-5 shape (T=65536)")
    fused = run_fused(x, lc, norm=True, chunk=64)
    two = run_two_step(x, lc, norm=True, chunk=64)
    check_carried("cfg5", fused, two)
    del two
    check_against_oracle("cfg5", x, lc, fused, [0, 9, 18, 27, 52, 61, 70, 95], norm=True)


# --------------------------------------------------------------------------- decode
def run_decode(x: gi.KdaInputs, lc: gi.LayerConv, state0: np.ndarray, *, fused: bool, norm: bool):
    """One call of the token-by-token kernel over x's T tokens; the carried inputs (and
    the state) are updated in place.  Returns (o, y, state, carried inputs)."""
    import linear_attention_recurrence_07_amd as kda
    d = U.device_inputs(x, DEV)
    ws, init = _conv_dev(lc, x.in_dtype)
    st = torch.from_numpy(state0.copy()).to(DEV)
    kw = dict(attention_mask=d["mask"], gate=d["gate"] if norm else None,
              norm_weight=d["norm_weight"] if norm else None, norm_eps=x.norm_eps, output_dtype=torch.float32)
    if fused:
        res, fin = kda.recurrent_step_conv(d["q"], d["k"], d["v"], d["g"], d["beta"], st, conv_weights=ws,
                                           conv_state=init, conv_final_state=init, **kw)
        assert all(a is b for a, b in zip(fin, init))
    else:
        filt = []
        for i, name in enumerate("qkv"):
            t = d[name]
            B, T, H, dd = t.shape
            yv = kda.short_conv(t.reshape(B, T, H * dd), ws[i], init[i], attention_mask=d["mask"],
                                final_state=init[i], with_final_state=False)
            filt.append(yv.reshape(B, T, H, dd))
        res = kda.recurrent_step(filt[0], filt[1], filt[2], d["g"], d["beta"], st, **kw)
    torch.cuda.synchronize()
    o, y = (res, None) if not norm else res
    return o, y, st, init


@pytest.mark.parametrize("case", ["config4_B64", "tiles_T5_masked", "slabs_T3", "d64_T2"])
def test_fused_decode(case):
    if case == "config4_B64":      # one new token for each of 64 rows (whole slabs)
        x = gi.make_inputs("conv_dec", B=64, T=1, H=96, dk=128, dv=128, seed=31, norm=True, normalize_qk=False)
    elif case == "tiles_T5_masked":   # few slabs, several tokens: 16-column tiles, a padding token
        mask = np.ones((2, 5), np.uint8)
        mask[0, 2] = 0
        mask[1, 0] = 0
        x = gi.make_inputs("conv_dec_tiles", B=2, T=5, H=4, dk=128, dv=128, seed=32, norm=True,
                           normalize_qk=False, mask=mask)
    elif case == "slabs_T3":       # enough slabs for whole-slab work-groups with several tokens
        x = gi.make_inputs("conv_dec_slabs", B=6, T=3, H=96, dk=128, dv=128, seed=33, norm=True, normalize_qk=False)
    else:
        x = gi.make_inputs("conv_dec_d64", B=3, T=2, H=5, dk=64, dv=64, seed=34, norm=True, normalize_qk=False)
    lc = gi.layer_conv(x, seed=31, with_state=True)
    rng = np.random.default_rng(35)
    state0 = (rng.standard_normal((x.B, x.H, x.dk, x.dv)) * 0.05).astype(np.float32)
    x = gi.dataclasses.replace(x, initial_state=state0)
    U.log(f"fused conv decode {case}: B={x.B} T={x.T} H={x.H} d={x.dk}")
    of, yf, sf, cf = run_decode(x, lc, state0, fused=True, norm=True)
    _, _, _, ct = run_decode(x, lc, state0, fused=False, norm=True)
    check_carried(f"decode {case}", (None, None, None, cf), (None, None, None, ct))
    check_against_oracle(f"decode {case}", x, lc, (of, sf, yf, cf), norm=True)


def test_fused_decode_zero_tokens_copies_carried_inputs():
    """T = 0: no token, so the carried inputs after the call are those before it (copied
    into separate final buffers).  Called through the C ABI: the binding has no empty
    tensors to pass; the token pointers name a small real buffer that is never read."""
    import ctypes
    import linear_attention_recurrence_07_amd as kda
    lib = kda.load_library()
    x = gi.make_inputs("conv_dec0", B=3, T=1, H=2, dk=128, dv=128, seed=36, normalize_qk=False)
    lc = gi.layer_conv(x, seed=36, with_state=True)
    ws, init = _conv_dev(lc, x.in_dtype)
    fin = tuple(torch.full_like(t, 7.0) for t in init)
    st = torch.zeros((3, 2, 128, 128), dtype=torch.float32, device=DEV)
    buf = torch.zeros(4096, dtype=torch.float32, device=DEV)
    p = kda._params(3, 0, 2, 128, 128, in_dtype=kda.KDA_BF16, out_dtype=kda.KDA_BF16)
    cv = kda.KdaConv(4, 1, *[kda._ptr(w) for w in ws], *[kda._ptr(t) for t in init], *[kda._ptr(t) for t in fin])
    b = kda._ptr(buf)
    U.log("fused conv decode with T = 0")
    kda._check(lib.kda_recurrent_step_conv(ctypes.byref(p), ctypes.byref(cv), b, b, b, b, b, kda._ptr(st), None, b,
                                           None, None, None, None))
    torch.cuda.synchronize()
    for a, f in zip(init, fin):
        assert torch.equal(a, f)
    assert torch.count_nonzero(st) == 0


def test_fused_prefill_then_decode_chain():
    """A prompt through the fused prefill, then three tokens through the fused decode step
    (state and carried inputs handed over in place), against one oracle chain over all the
    tokens, and the carried inputs against the fused prefill of all the tokens."""
    import linear_attention_recurrence_07_amd as kda
    P, n = 100, 3
    x = gi.make_inputs("conv_chain", B=2, T=P + n, H=4, dk=128, dv=128, seed=37, norm=True, normalize_qk=False)
    lc = gi.layer_conv(x, seed=37)
    U.log("fused conv prefill -> decode chain")
    d = U.device_inputs(x, DEV)
    ws, _ = _conv_dev(lc, x.in_dtype)
    head = {k: (v[:, :P].contiguous() if torch.is_tensor(v) and v.dim() >= 2 and v.shape[1] == P + n else v)
            for k, v in d.items()}
    o1, s1, y1, c1 = kda.chunk_prefill_conv(head["q"], head["k"], head["v"], head["g"], head["beta"],
                                            conv_weights=ws, gate=head["gate"], norm_weight=head["norm_weight"],
                                            norm_eps=x.norm_eps, output_dtype=torch.float32)
    outs = [o1]
    for t in range(P, P + n):
        sl = {k: d[k][:, t:t + 1].contiguous() for k in ("q", "k", "v", "g", "beta", "gate")}
        (o, y), _ = kda.recurrent_step_conv(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], s1, conv_weights=ws,
                                            conv_state=c1, conv_final_state=c1, gate=sl["gate"],
                                            norm_weight=d["norm_weight"], norm_eps=x.norm_eps,
                                            output_dtype=torch.float32)
        outs.append(o)
    torch.cuda.synchronize()
    # the oracle chain over all P + n tokens
    filt = []
    for i, name in enumerate("qkv"):
        raw = gi.to_f64(getattr(x, name), x.in_dtype).reshape(x.B, x.T, x.H * 128)
        y, _ = C.short_conv(raw, lc.weights[i], None)
        filt.append(y.reshape(x.B, x.T, x.H, 128).astype(np.float32))
    ro, rfs = cref.recurrence(filt[0], filt[1], filt[2], x.g, x.beta, None, in_dtype=gi.F32)
    U.assert_close("chain prompt o", U.to_numpy64(o1), ro[:, :P], TOL)
    U.assert_close("chain decoded o", U.to_numpy64(torch.cat(outs[1:], dim=1)), ro[:, P:], TOL)
    U.assert_close("chain final state", U.to_numpy64(s1), rfs, TOL)
    full = run_fused(x, lc, norm=True)
    for a, b in zip(c1, full[3]):
        assert torch.equal(a, b), "carried inputs after prefill + decode"
