"""GPU parity of the q/k prologue: the in-kernel L2 norm of queries and keys, the query
scale, and the switch that turns the norm off.

The kernels receive queries and keys before their L2 norm and apply it themselves,
together with the 1/sqrt(key_dim) query scale (nnterp Kimi-Linear page, Notes, KDA
paragraph; section 04, family-module docstring: use_qk_l2norm_in_kernel).  Every case
here feeds rows that are NOT of unit length (per-head factors 0.05, 1 and 40 on N(0, 1)
draws), so a kernel that skipped or misplaced the norm or the scale would miss the
oracle by O(1); each case also checks on the CPU that the oracle itself tells the two
apart on these inputs.  Bar: max|GPU - oracle| / rms(oracle) <= 2e-2 (bf16 inputs) or
1e-4 (fp32), as in the other parity tests.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import kda_ref as R
from tests import kda_testutil as U

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RAW = (0.05, 1.0, 40.0)        # per-head factors on the raw q and k rows


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not U.gpu_available():
        pytest.fail("GPU tests need an MI355X; run them with -m gpu on a GPU host")
    import linear_attention_recurrence_07_amd as kda
    kda.load_library()


def _discriminates(x, ro, *, scale=None, use_l2=True, tol):
    """The oracle's result moves by far more than the tolerance if the norm (or the scale)
    is dropped: the case can tell a kernel that skips it from one that applies it."""
    if use_l2:
        alt, _, _ = U.oracle(x, norm=False, scale=scale, use_l2=False)
    else:
        alt, _, _ = U.oracle(x, norm=False, scale=None, use_l2=False)
    vm = U.valid_token_mask(x)
    e = R.rel_err(alt[vm], ro[vm])
    assert (not np.isfinite(e)) or e > 20 * tol, f"oracle does not tell the variants apart ({e:.2e})"


def _prefill_case(x, *, tol, chunk=0, scale=None, use_l2=True):
    U.log(f"prefill {x.name}: B={x.B} T={x.T} H={x.H} d={x.dk} chunk={chunk} scale={scale} l2={use_l2}")
    o, fs, y = U.run_prefill(x, DEV, chunk=chunk, scale=scale, use_l2=use_l2)
    ro, rfs, ry = U.oracle(x, scale=scale, use_l2=use_l2)
    vm = U.valid_token_mask(x)
    U.assert_close(f"{x.name} o", o[vm], ro[vm], tol)
    U.assert_close(f"{x.name} final_state", fs, rfs, tol)
    if ry is not None:
        U.assert_close(f"{x.name} y", y[vm], ry[vm], tol)
    _discriminates(x, ro, scale=scale, use_l2=use_l2, tol=tol)


# ------------------------------------------------------------------ matrix-core prefill
@pytest.mark.parametrize("layout", ["plain", "packed", "masked", "chunk64"])
def test_mfma_prefill_raw_qk(layout):
    if layout == "packed":
        x = gi.make_inputs("raw_packed", B=1, T=200, H=6, dk=128, dv=128, seed=71, normalize_qk=False,
                           qk_scale_by_head=RAW, initial_state_std=0.05, num_seqs=3, norm=True,
                           cu_seqlens=[0, 70, 103, 200])
    elif layout == "masked":
        m = np.ones((2, 90), np.uint8)
        m[0, :11] = 0            # left padding
        m[1, 40:45] = 0          # a gap
        m[1, 80:] = 0            # right padding
        x = gi.make_inputs("raw_masked", B=2, T=90, H=6, dk=128, dv=128, seed=72, normalize_qk=False,
                           qk_scale_by_head=RAW, initial_state_std=0.05, norm=True, mask=m)
    else:
        x = gi.make_inputs(f"raw_{layout}", B=1, T=150, H=6, dk=128, dv=128, seed=73, normalize_qk=False,
                           qk_scale_by_head=RAW, initial_state_std=0.05, norm=True)
    _prefill_case(x, tol=U.BF16_TOL, chunk=64 if layout == "chunk64" else 0)


@pytest.mark.parametrize("scale", [0.3, 0.01])
def test_mfma_prefill_explicit_scale(scale):
    x = gi.make_inputs(f"raw_scale{scale}", B=1, T=100, H=3, dk=128, dv=128, seed=74, normalize_qk=False,
                       qk_scale_by_head=RAW, norm=True)
    _prefill_case(x, tol=U.BF16_TOL, scale=scale)


def test_mfma_prefill_without_l2_norm():
    """use_qk_l2norm = 0 on rows that are already unit length (to bf16 rounding), with an
    explicit scale: the kernel must use q and k as given."""
    x = gi.make_inputs("nol2_mfma", B=1, T=130, H=4, dk=128, dv=128, seed=75, initial_state_std=0.05, norm=True)
    _prefill_case(x, tol=U.BF16_TOL, scale=0.2, use_l2=False)


# ------------------------------------------------------------------ vector-ALU prefill
@pytest.mark.parametrize("case", ["f32_raw", "f32_nol2", "bf16_raw_chunk16"])
def test_valu_prefill_qk_prologue(case):
    if case == "f32_raw":
        x = gi.make_inputs("valu_raw", B=1, T=64, H=3, dk=16, dv=16, chunk=16, in_dtype=gi.F32, seed=76,
                           normalize_qk=False, qk_scale_by_head=RAW, norm=True)
        _prefill_case(x, tol=U.F32_TOL, scale=0.4)
    elif case == "f32_nol2":
        x = gi.make_inputs("valu_nol2", B=1, T=64, H=2, dk=16, dv=16, chunk=16, in_dtype=gi.F32, seed=77,
                           norm=True)
        _prefill_case(x, tol=U.F32_TOL, scale=0.5, use_l2=False)
    else:
        x = gi.make_inputs("valu_raw_bf16", B=1, T=70, H=3, dk=128, dv=128, seed=78, normalize_qk=False,
                           qk_scale_by_head=RAW, initial_state_std=0.05, norm=True)
        _prefill_case(x, tol=U.BF16_TOL, chunk=16)


# ------------------------------------------------------------------ token-by-token kernel
# Layouts: one token (whole slabs), several tokens with many slabs (B * H >= 512: whole
# slabs, norm fused) and several tokens with few slabs (column tiles, norm as its own pass).
DECODE = {"one_token": (8, 1, 6), "many_slabs": (4, 3, 128), "column_tiles": (1, 9, 6)}


@pytest.mark.parametrize("layout", list(DECODE))
@pytest.mark.parametrize("mode", ["raw", "raw_scale", "nol2"])
def test_decode_qk_prologue(layout, mode):
    import linear_attention_recurrence_07_amd as kda
    B, T, H = DECODE[layout]
    raw = mode != "nol2"
    x = gi.make_inputs(f"dec_{layout}_{mode}", B=B, T=T, H=H, dk=128, dv=128, seed=79 + T + H,
                       normalize_qk=not raw, qk_scale_by_head=RAW if raw else None, initial_state_std=0.05,
                       norm=True)
    scale = None if mode == "raw" else 0.25
    use_l2 = mode != "nol2"
    d = U.device_inputs(x, DEV)
    st = d["initial_state"].clone()
    U.log(f"decode {layout} {mode}: B={B} T={T} H={H}")
    o, y = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, gate=d["gate"],
                              norm_weight=d["norm_weight"], norm_eps=x.norm_eps, scale=scale,
                              use_qk_l2norm_in_kernel=use_l2, output_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rfs, ry = U.oracle(x, scale=scale, use_l2=use_l2)
    U.assert_close(f"decode {layout} {mode} o", U.to_numpy64(o), ro, U.BF16_TOL)
    U.assert_close(f"decode {layout} {mode} y", U.to_numpy64(y), ry, U.BF16_TOL)
    U.assert_close(f"decode {layout} {mode} state", U.to_numpy64(st), rfs, U.BF16_TOL)
    _discriminates(x, ro, scale=scale, use_l2=use_l2, tol=U.BF16_TOL)


def test_per_token_states_raw_qk():
    import linear_attention_recurrence_07_amd as kda
    x = gi.make_inputs("states_raw", B=1, T=12, H=3, dk=128, dv=128, seed=80, normalize_qk=False,
                       qk_scale_by_head=RAW, initial_state_std=0.05)
    d = U.device_inputs(x, DEV)
    st = d["initial_state"].clone()
    states = torch.empty((x.B, x.T, x.H, x.dk, x.dv), device=DEV)
    U.log("per-token states with raw q/k")
    o = kda.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st, output_dtype=torch.float32,
                           states=states)
    torch.cuda.synchronize()
    ro, rfs, rst = R.kda_recurrence(x.f64("q"), x.f64("k"), x.f64("v"), x.g, x.beta, x.initial_state,
                                    return_states=True)
    U.assert_close("states raw", U.to_numpy64(states), rst, U.BF16_TOL)
    U.assert_close("states raw o", U.to_numpy64(o), ro, U.BF16_TOL)
    U.assert_close("states raw final", U.to_numpy64(st), rfs, U.BF16_TOL)
    _discriminates(x, ro, tol=U.BF16_TOL)
