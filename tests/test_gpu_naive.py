"""The naive three-kernel ablation matches the oracle too."""
import pytest
import torch

import seeded_inputs as si
from exact_io_aware_74_amd import binding as fa
from helpers import assert_close, assert_lse_close, to_device, to_f64, workload_inputs
import oracle

pytestmark = pytest.mark.gpu


def _naive_case(q, k, v, causal, scale):
    qd, kd, vd = (to_device(x, "bf16") for x in (q, k, v))
    o, lse = fa.naive_fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.attention(si.as_float64(q, "bf16"), si.as_float64(k, "bf16"), si.as_float64(v, "bf16"), causal,
                            scale)
    assert_close(to_f64(o), O, "bf16")
    assert_lse_close(to_f64(lse), L, "bf16")
    return qd, kd, vd, o


def test_naive_workload_bf16_b4h16_n1024_d64_causal():
    w = si.WORKLOADS["bf16_b4h16_n1024_d64_causal"]
    q, k, v = workload_inputs(w)
    qd, kd, vd, o_naive = _naive_case(q, k, v, True, w.scale)
    o_fused, _ = fa.fwd(qd, kd, vd, causal=True)
    # both within the bar of the oracle; and close to each other
    assert (o_fused.float() - o_naive.float()).abs().max().item() < 4e-2


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200])
def test_naive_ragged(d, causal, N):
    q, k, v = si.random_case(N + d + 3, 2, 2, N, d, "bf16")
    _naive_case(q, k, v, causal, fa.default_scale(d))
