"""GPU parity of the column-parallel up projection with SwiGLU
(tp_gate_up_swiglu) against the CPU oracle.

The output is bf16, so the bar is the bf16-output reading of the tolerance:
every element within max(1e-2 * rms, one bf16 ulp) of the oracle's double
value. The GPU accumulates in fp32 and forms silu in fp32, so an element
whose exact value lies near a bf16 rounding boundary can round to the other
neighbour; all others round as the oracle does, which is checked too.
"""
import numpy as np
import pytest
import torch

import oracle
from row_gemv_reduction_amd import binding as tp
from row_gemv_reduction_amd import synth
from tests.gpu_helpers import assert_bits_equal, bf16_bits_host, say, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def bf16_ulp(v):
    """Spacing of bf16 at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), np.float64(2.0 ** -126))
    return np.exp2(np.floor(np.log2(a)) - 7)


CASES = [
    # (n_ranks, batch, hidden, inter, layers): vector-ALU and matrix-core
    # steps, ragged column tiles, one split and several, tokens past 16
    (2, 1, 520, 1040, 2), (4, 3, 1024, 4352, 2), (1, 8, 264, 1000, 2),
    (4, 16, 1032, 2080, 2), (8, 64, 512, 2048, 1), (2, 5, 2048, 4096, 1),
    (4, 40, 1024, 4352, 1), (2, 24, 4104, 1024, 1),
]


@pytest.mark.parametrize("n,b,h,inter,L,per,rows", [c + (0, 0) for c in CASES] +
                         [(2, 3, 520, 1040, 5, 2, 0), (4, 17, 1024, 2080, 3, 1, 0),
                          (2, 24, 4104, 1024, 2, 0, 512), (1, 16, 2048, 640, 1, 0, 512)])
def test_gate_up_swiglu_matches_oracle(n, b, h, inter, L, per, rows):
    """per > 0 caps the layers per launch (swiglu_layers), so that a stack
    takes several launches; rows > 0 caps the tile length (step_rows), so
    that the matrix-core tiles split K instead of spanning it."""
    C = inter // n
    say("gate/up swiglu n=%d b=%d h=%d inter=%d L=%d per=%d rows=%d" % (n, b, h, inter, L, per, rows))
    kw = dict(seed=61, workload="swiglu")
    x = synth.normal_bf16((L, b, h), 1.0, tensor="x_ffn_in", **kw)
    wg = synth.normal_bf16((L, h, C), synth.WEIGHT_STD, tensor="w_gate", **kw)
    wu = synth.normal_bf16((L, h, C), synth.WEIGHT_STD, tensor="w_up", **kw)
    plan = tp.Plan(h, inter, n, b, tune={"swiglu_layers": per, "step_rows": rows})
    ws = plan.new_workspace()
    X, WG, WU = to_dev_bf16(x), to_dev_bf16(wg), to_dev_bf16(wu)
    out = torch.empty((L, b, C), dtype=torch.bfloat16, device="cuda")
    tp.tp_gate_up_swiglu(plan, L, X, WG, WU, out, ws)
    out2 = torch.empty_like(out)
    tp.tp_gate_up_swiglu(plan, L, X, WG, WU, out2, ws)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0
    got = bf16_bits_host(out)
    assert_bits_equal(bf16_bits_host(out2), got, "repeat")
    for l in range(L):
        a64, abf = oracle.gate_up_swiglu(x[l], wg[l], wu[l])
        gotf = synth.bf16_bits_to_f32(got[l]).astype(np.float64)
        rms = float(np.sqrt(np.mean(a64 ** 2)))
        bound = np.maximum(1e-2 * rms, bf16_ulp(a64))
        err = np.abs(gotf - a64)
        assert np.all(err <= bound), "layer %d: max excess %.3e" % (l, float((err - bound).max()))
        same = float(np.mean(got[l] == abf))
        assert same >= 0.97, "layer %d: only %.3f of the elements round as the oracle's" % (l, same)


def test_gate_up_swiglu_zero_gate_and_empty_stack():
    """Zero gate weights give zero (silu(0) = 0) on the GPU too; an empty
    stack does nothing."""
    n, b, h, inter = 2, 4, 520, 1040
    C = inter // n
    x = synth.normal_bf16((1, b, h), 1.0, seed=62, workload="swiglu", tensor="x_ffn_in")
    wu = synth.normal_bf16((1, h, C), synth.WEIGHT_STD, seed=62, workload="swiglu", tensor="w_up")
    plan = tp.Plan(h, inter, n, b)
    ws = plan.new_workspace()
    out = torch.full((1, b, C), 7.0, dtype=torch.bfloat16, device="cuda")
    tp.tp_gate_up_swiglu(plan, 1, to_dev_bf16(x), torch.zeros((1, h, C), dtype=torch.bfloat16,
                                                              device="cuda"),
                         to_dev_bf16(wu), out, ws)
    torch.cuda.synchronize()
    assert np.all((bf16_bits_host(out) & 0x7FFF) == 0)
    e = torch.empty((0, b, C), dtype=torch.bfloat16, device="cuda")
    tp.tp_gate_up_swiglu(plan, 0, torch.empty((0, b, h), dtype=torch.bfloat16, device="cuda"),
                         torch.empty((0, h, C), dtype=torch.bfloat16, device="cuda"),
                         torch.empty((0, h, C), dtype=torch.bfloat16, device="cuda"), e, ws)
    torch.cuda.synchronize()
