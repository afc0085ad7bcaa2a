"""GPU parity of kda_chunk_prefill_states: the state after every token, computed through
the chunked form (the scan stores each chunk's U rows and the state after its last
position; a second launch fills the chunk's other positions by rank-one updates).

The states are those a prompt yields token by token (nnterp Kimi-Linear page, support()
table, the 'states' row [batch, seq, heads, key_dim, value_dim]; Notes, "Loading").  The
reference is the oracle's fp64 recurrence with return_states (padding positions repeat
the carried state).  Bar: max|GPU - oracle| / rms(oracle) <= 2e-2, the bf16 prefill's
tolerance, over all states; o must be bit-identical to kda_chunk_prefill's on the same
inputs (the same arithmetic), and the state at each sequence's last token bit-identical
to final_state.  Cases span several chunks with ragged tails, one-token and exactly
one-chunk sequences (a chunk whose only position the scan writes), empty sequences,
padding at chunk edges, one decay per head with 64-token chunks, raw keys without the
in-kernel norm, and the 96-head shape the benchmark times (sampled heads).
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import kda_ref as R
from tests import kda_testutil as U

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 12345.0


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not U.gpu_available():
        pytest.fail("GPU tests need an MI355X; run them with -m gpu on a GPU host")
    import linear_attention_recurrence_07_amd as kda
    kda.load_library()


def _run(x, *, chunk=0, use_l2=True, scale=None, heads=None):
    """kda_chunk_prefill_states and kda_chunk_prefill on the same inputs (o and the final
    state must agree bit for bit); returns the states (restricted to `heads` on the GPU),
    o and final_state."""
    import linear_attention_recurrence_07_amd as kda
    d = U.device_inputs(x, DEV)
    states = torch.full((x.B, x.T, x.H, x.dk, x.dv), SENTINEL, device=DEV)
    kw = dict(cu_seqlens=d["cu_seqlens"], attention_mask=d["mask"], chunk=chunk, output_dtype=torch.float32,
              scale=scale, use_qk_l2norm_in_kernel=use_l2)
    U.log(f"chunk states {x.name}: B={x.B} T={x.T} H={x.H} chunk={chunk} l2={use_l2}")
    o, fs = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], states=states, **kw)
    o2, fs2 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], **kw)
    torch.cuda.synchronize()
    vm = torch.from_numpy(U.valid_token_mask(x)).to(DEV)     # tokens past a packed batch are not written
    assert torch.equal(o[vm], o2[vm]), "o differs from kda_chunk_prefill's"
    assert torch.equal(fs, fs2), "final_state differs from kda_chunk_prefill's"
    if heads is not None:
        states = states.index_select(2, torch.tensor(list(heads), device=DEV))
    return states, o, fs


def _oracle_states(x, heads=None, *, use_l2=True, scale=None):
    sel = (lambda a: a) if heads is None else (lambda a: a[:, :, list(heads)])
    init = x.initial_state
    if init is not None and heads is not None:
        init = init[:, list(heads)]
    ro, rfs, rst = R.kda_recurrence(sel(x.f64("q")), sel(x.f64("k")), sel(x.f64("v")), sel(x.f64("g")),
                                    sel(x.f64("beta")), init, mask=x.mask, cu_seqlens=x.cu_seqlens,
                                    return_states=True, use_qk_l2norm=use_l2, scale=scale)
    return ro, rfs, rst


def _last_tokens(x):
    """(row, token, sequence) of every non-empty sequence's last position."""
    if x.cu_seqlens is not None:
        cu = x.cu_seqlens
        return [(0, int(cu[n + 1]) - 1, n) for n in range(len(cu) - 1) if cu[n + 1] > cu[n]]
    return [(b, x.T - 1, b) for b in range(x.B)] if x.T > 0 else []


def _check(x, states, o, fs, *, use_l2=True, scale=None, heads=None):
    ro, rfs, rst = _oracle_states(x, heads, use_l2=use_l2, scale=scale)
    got = U.to_numpy64(states)
    vm = U.valid_token_mask(x)
    if x.cu_seqlens is not None:
        # tokens at or past the end of the packed batch are not written
        end = int(x.cu_seqlens[-1])
        assert np.all(got[0, end:] == SENTINEL), "states past the packed batch were written"
        got, rst = got[:, :end], rst[:, :end]
    U.assert_close(f"chunk states {x.name}", got, rst, U.BF16_TOL)
    if heads is None:
        U.assert_close(f"chunk states {x.name} o", U.to_numpy64(o)[vm], ro[vm], U.BF16_TOL)
        U.assert_close(f"chunk states {x.name} final", U.to_numpy64(fs), rfs, U.BF16_TOL)
        for b, t, n in _last_tokens(x):
            assert torch.equal(states[b, t], fs[n]), f"state at the last token of sequence {n} != final_state"


@pytest.mark.parametrize("case", ["plain", "masked", "packed", "per_head_chunk64", "one_chunk", "short",
                                  "padded_chunk", "packed_chunk64_per_head"])
def test_chunk_states(case):
    if case == "plain":
        x = gi.make_inputs("cs_plain", B=2, T=100, H=3, dk=128, dv=128, seed=71, initial_state_std=0.05)
        chunk = 0
    elif case == "masked":
        m = np.ones((2, 96), np.uint8)
        m[0, [0, 31, 32, 33, 63, 64, 95]] = 0       # padding at chunk edges and both ends
        m[1, 40:72] = 0                             # a padded run across a chunk boundary
        x = gi.make_inputs("cs_masked", B=2, T=96, H=2, dk=128, dv=128, seed=72, initial_state_std=0.05, mask=m)
        chunk = 32
    elif case == "packed":
        # lengths 33 (a second chunk with one position), 1, 0, 64, 45, 32, and 7 tokens
        # past the last offset
        lens = [33, 1, 0, 64, 45, 32]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = gi.make_inputs("cs_packed", B=1, T=int(cu[-1]) + 7, H=2, dk=128, dv=128, seed=73,
                           initial_state_std=0.05, cu_seqlens=cu)
        chunk = 0
    elif case == "per_head_chunk64":
        x = gi.make_inputs("cs_ph", B=1, T=150, H=2, dk=128, dv=128, seed=74, initial_state_std=0.05,
                           decay_per_head=True)
        chunk = 64
    elif case == "one_chunk":
        x = gi.make_inputs("cs_one", B=3, T=32, H=2, dk=128, dv=128, seed=75)
        chunk = 0
    elif case == "short":
        x = gi.make_inputs("cs_short", B=2, T=2, H=2, dk=128, dv=128, seed=76, initial_state_std=0.05)
        chunk = 0
    elif case == "padded_chunk":
        # a whole chunk of padding in row 1 (its positions repeat the carried state) and
        # a ragged, padded tail in row 0
        m = np.ones((2, 80), np.uint8)
        m[1, 32:64] = 0
        m[0, 70:] = 0
        x = gi.make_inputs("cs_padchunk", B=2, T=80, H=2, dk=128, dv=128, seed=80, initial_state_std=0.05, mask=m)
        chunk = 0
    else:
        lens = [70, 5, 64, 31]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = gi.make_inputs("cs_packed64", B=1, T=int(cu[-1]), H=2, dk=128, dv=128, seed=81,
                           initial_state_std=0.05, cu_seqlens=cu, decay_per_head=True)
        chunk = 64
    states, o, fs = _run(x, chunk=chunk)
    _check(x, states, o, fs)


def test_chunk_states_raw_keys_without_norm():
    """Raw (non-unit) keys and queries with the in-kernel norm switched off and a custom
    query scale: the states kernel must use the keys as given."""
    x = gi.make_inputs("cs_raw", B=1, T=70, H=3, dk=128, dv=128, seed=77, normalize_qk=False,
                       qk_scale_by_head=(0.05, 0.08, 0.03), initial_state_std=0.05)
    states, o, fs = _run(x, use_l2=False, scale=0.3)
    _check(x, states, o, fs, use_l2=False, scale=0.3)
    # the oracle tells the variants apart on these inputs
    _, _, alt = _oracle_states(x, use_l2=True, scale=0.3)
    _, _, ref = _oracle_states(x, use_l2=False, scale=0.3)
    assert R.rel_err(alt, ref) > 20 * U.BF16_TOL


def test_chunk_states_bench_shape_sampled_heads():
    """The benchmark's shape, B = 1, T = 256, H = 96 (all heads run; eight heads, one per
    XCD residue, against the oracle), and the token-by-token kernel's states on the same
    heads within the same bar."""
    import linear_attention_recurrence_07_amd as kda
    x = gi.make_inputs("cs_bench", B=1, T=256, H=96, dk=128, dv=128, seed=78)
    heads = (0, 9, 18, 27, 36, 45, 54, 95)
    states, o, fs = _run(x, heads=heads)
    _check(x, states, o, fs, heads=heads)
    d = U.device_inputs(x, DEV)
    st = torch.zeros((1, x.H, 128, 128), device=DEV)
    tok = torch.empty((1, x.T, x.H, 128, 128), device=DEV)
    U.log("token-by-token states at the benchmark shape")
    kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, output_dtype=torch.float32, states=tok)
    torch.cuda.synchronize()
    sel = torch.tensor(list(heads), device=DEV)
    U.assert_close("chunk vs token-by-token states", U.to_numpy64(states),
                   U.to_numpy64(tok.index_select(2, sel)), U.BF16_TOL)


def test_chunk_states_zero_tokens():
    """T = 0: final_state is the initial state and nothing else is written.  Called through
    the C ABI: the binding has no empty tensors to pass; the token pointers name a small
    real buffer that is never read or written."""
    import ctypes
    import linear_attention_recurrence_07_amd as kda
    lib = kda.load_library()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(79)
    init = torch.randn((2, 2, 128, 128), generator=gen, device=DEV)
    fs = torch.full_like(init, 7.0)
    buf = torch.full((4096,), 3.0, device=DEV)
    p = kda._params(2, 0, 2, 128, 128, in_dtype=kda.KDA_BF16, out_dtype=kda.KDA_F32)
    need = lib.kda_chunk_prefill_states_workspace_size(ctypes.byref(p), 0)
    assert need > 0
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    b = kda._ptr(buf)
    U.log("chunk states with T = 0")
    kda._check(lib.kda_chunk_prefill_states(ctypes.byref(p), b, b, b, b, b, kda._ptr(init), None, None, b,
                                            kda._ptr(fs), None, None, None, b, kda._ptr(ws), need, None))
    torch.cuda.synchronize()
    assert torch.equal(fs, init)
    assert torch.all(buf == 3.0)


def test_chunk_states_with_gated_norm_and_bf16_outputs():
    """bf16 o and the gated norm's y through kda_chunk_prefill_states: o, y and the final
    state bit-identical to kda_chunk_prefill's, the states against the oracle."""
    import linear_attention_recurrence_07_amd as kda
    x = gi.make_inputs("cs_norm", B=2, T=67, H=2, dk=128, dv=128, seed=82, initial_state_std=0.05, norm=True)
    d = U.device_inputs(x, DEV)
    states = torch.full((x.B, x.T, x.H, x.dk, x.dv), SENTINEL, device=DEV)
    kw = dict(gate=d["gate"], norm_weight=d["norm_weight"], norm_eps=x.norm_eps, output_dtype=torch.bfloat16)
    U.log("chunk states with the gated norm, bf16 outputs")
    o, fs, y = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], states=states, **kw)
    o2, fs2, y2 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["initial_state"], **kw)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and y.dtype == torch.bfloat16
    assert torch.equal(o, o2) and torch.equal(y, y2) and torch.equal(fs, fs2)
    _, _, rst = _oracle_states(x)
    U.assert_close("chunk states cs_norm", U.to_numpy64(states), rst, U.BF16_TOL)
