"""The GEMM timing module runs on small shapes: every product of the FFN
forward and backward is timed, for random and for zero operands, and the
output hash does not depend on the timing run (two runs, same bits)."""
import pytest

from _gpu import banner, needs_gpu

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_gemm_bench_times_every_product(act):
    from mixture_experts_layer_permute_amd import gemm_bench
    banner("gemm_bench", act)
    res, h1, _ = gemm_bench.run(4, 512, 128, 256, act, reps=2)
    names = {"gemm_down", "gemm_dW2", "gemm_dW1", "gemm_dX",
             "gemm_up_" + act, "gemm_dA_" + act} | ({"gemm_dW3"} if act == "swiglu" else set())
    assert set(res) == names, sorted(res)
    assert all(ms > 0 and tf > 0 for ms, tf in res.values())
    _, h2, _ = gemm_bench.run(4, 512, 128, 256, act, reps=1)
    assert h1 == h2
    res0, _, _ = gemm_bench.run(4, 512, 128, 256, act, reps=1, operands="zero")
    assert set(res0) == names
