"""GPU parity of the layer's exit (kda_gated_norm_proj, kda_out_proj) against the fp64
oracle in oracle/out_proj.py on the same seeded inputs.  The projection accumulates exact
bf16 products in fp32 (held to 1e-4 of rms); with the norm in front, its bf16 output y is
the projection's input, so the chain is held to the bf16 bar of 2e-2."""
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


@pytest.mark.parametrize("rows,K,N", [(1, 256, 64), (5, 768, 128), (64, 512, 64), (64, 4096, 192), (70, 1024, 64),
                                      (200, 1024, 128)])
def test_projection_alone(rows, K, N):
    import linear_attention_recurrence_07_amd as kda
    rng = np.random.default_rng(rows + K + N)
    x = gi.f32_to_bf16_bits(rng.standard_normal((rows, K)).astype(np.float32))
    W = gi.f32_to_bf16_bits((rng.uniform(-1, 1, (N, K)) / np.sqrt(K)).astype(np.float32))
    U.log(f"out_proj rows={rows} K={K} N={N}")
    out = kda.out_proj(_bf16(x), _bf16(W), output_dtype=torch.float32)
    outb = kda.out_proj(_bf16(x), _bf16(W))
    torch.cuda.synchronize()
    ref = P.project(gi.bf16_bits_to_f32(x), gi.bf16_bits_to_f32(W))
    U.assert_close(f"out_proj {rows}x{K}x{N}", U.to_numpy64(out), ref, 1e-4)
    assert torch.equal(outb, out.to(torch.bfloat16))


@pytest.mark.parametrize("rows", [64, 3])
def test_gated_norm_proj_decode_shape(rows):
    """The pages' decode exit: [rows, 96 x 128] -> [rows, 7168]."""
    import linear_attention_recurrence_07_amd as kda
    x = gi.proj_inputs(f"exit_B{rows}", rows=rows, seed=rows)
    U.log(f"gated_norm_proj rows={rows} heads=96 head_dim=128 N=7168")
    y, out = kda.gated_norm_proj(_bf16(x.o), _bf16(x.gate), torch.from_numpy(x.norm_weight).to(DEV),
                                 _bf16(x.proj_weight), x.eps, output_dtype=torch.float32)
    torch.cuda.synchronize()
    ry, rout = P.gated_norm_proj(gi.bf16_bits_to_f32(x.o), gi.bf16_bits_to_f32(x.gate), x.norm_weight,
                                 gi.bf16_bits_to_f32(x.proj_weight), x.eps)
    U.assert_close(f"exit B{rows} y", U.to_numpy64(y), ry, U.BF16_TOL)
    # y is the nearest bf16 of the normed value: within half a bf16 spacing (<= 2^-8 of
    # |y|) plus fp32 rounding of the norm
    yd = U.to_numpy64(y)
    bound = 2.0 ** -8 * np.abs(ry) * (1 + 1e-5) + 1e-6 * np.sqrt(np.mean(ry ** 2))
    assert np.all(np.abs(yd - ry) <= bound), float(np.max(np.abs(yd - ry) / bound))
    U.assert_close(f"exit B{rows} out", U.to_numpy64(out), rout, U.BF16_TOL)
