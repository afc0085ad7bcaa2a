"""The allocation-free layer exit (kda_gated_norm_proj_noalloc) against the entry point
with a caller workspace (kda_gated_norm_proj), through the C ABI.

The no-alloc call keeps the split-K partial sums in the library's static per-GPU scratch,
which holds the previous call's partials: two calls in a row, the second on a smaller
problem, must each give exactly what the workspace entry point gives on the same inputs
(same kernels, same summation order), and the chain must meet the bf16 bar against the
fp64 oracle of the gated norm + projection."""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import out_proj as P
from tests import kda_testutil as U

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not U.gpu_available():
        pytest.fail("GPU tests need an MI355X; run them with -m gpu on a GPU host")
    import linear_attention_recurrence_07_amd as kda
    kda.load_library()


def _bf16(a):
    return U.to_torch(a, gi.BF16, DEV)


def test_noalloc_exit_equals_workspace_exit_twice_then_smaller():
    import linear_attention_recurrence_07_amd as kda
    # (rows, out_features): the decode exit (K split 4 ways, 7.3 MB of partials), then a
    # smaller one that leaves most of the scratch holding the first call's partials
    for rows, N, seed in ((64, 7168, 91), (3, 1024, 92)):
        x = gi.proj_inputs(f"noalloc_B{rows}", rows=rows, out_features=N, seed=seed)
        o, gate, W = _bf16(x.o), _bf16(x.gate), _bf16(x.proj_weight)
        w = torch.from_numpy(x.norm_weight).to(DEV)
        U.log(f"gated_norm_proj_noalloc rows={rows} heads=96 head_dim=128 N={N}")
        y1 = torch.empty((rows, 96 * 128), dtype=torch.bfloat16, device=DEV)
        out1 = torch.empty((rows, N), dtype=torch.float32, device=DEV)
        kda.gated_norm_proj_noalloc(o, gate, w, W, x.eps, y=y1, out=out1)
        y2, out2 = kda.gated_norm_proj(o, gate, w, W, x.eps, output_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2)
        assert torch.equal(out1, out2)
        ry, rout = P.gated_norm_proj(gi.bf16_bits_to_f32(x.o), gi.bf16_bits_to_f32(x.gate), x.norm_weight,
                                     gi.bf16_bits_to_f32(x.proj_weight), x.eps)
        U.assert_close(f"noalloc exit B{rows} out", U.to_numpy64(out1), rout, U.BF16_TOL)
        U.assert_close(f"noalloc exit B{rows} y", U.to_numpy64(y1), ry, U.BF16_TOL)
