"""GPU parity of the column-parallel up projection with SwiGLU
(tp_gate_up_swiglu) against the CPU oracle.

The output is bf16, so the bar is the bf16-output reading of the tolerance:
every element within max(1e-2 * rms, one bf16 ulp) of the oracle's double
value. It is also checked to a much tighter bound derived from the
arithmetic: the GPU's gate and up sums g, u are each within 1e-5 * rms of
the exact ones (the partial tolerance), silu(g) * u is formed in fp32 with
a few roundings, and the result is rounded once to bf16. So the output is
within slack + half a bf16 ulp of the exact a = silu(g) * u, with
    slack = 1.1 * dg * |u| + |silu(g)| * du + dg * du + 8 * 2^-24 * |a|,
dg = 1e-5 * rms(g), du = 1e-5 * rms(u) (|silu'| <= 1.1). Where the exact value
lies within that slack of a bf16 rounding boundary, the GPU may round to
the other neighbour; elsewhere it must round as the exact value does.
"""
import numpy as np
import pytest
import torch

import oracle
from row_gemv_reduction_amd import binding as tp
from row_gemv_reduction_amd import synth
from tests.gpu_helpers import (assert_bf16_rounding, assert_bits_equal, bf16_bits_host, bf16_ulp,
                               say, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def swiglu_slack(x_bits, wg_bits, wu_bits, a64):
    """The derived per-element bound on the GPU's fp32 value of silu(g) * u
    (module docstring), from the oracle's exact gate and up projections."""
    g64, _ = oracle.partial(x_bits, wg_bits)
    u64, _ = oracle.partial(x_bits, wu_bits)
    dg = 1e-5 * np.sqrt(np.mean(g64 ** 2))
    du = 1e-5 * np.sqrt(np.mean(u64 ** 2))
    silu = g64 / (1.0 + np.exp(-g64))
    return 1.1 * dg * np.abs(u64) + np.abs(silu) * du + 1.1 * dg * du + 8 * 2.0 ** -24 * np.abs(a64)


def check_swiglu_layer(got_bits, x_bits, wg_bits, wu_bits, what):
    a64, abf = oracle.gate_up_swiglu(x_bits, wg_bits, wu_bits)
    gotf = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    rms = float(np.sqrt(np.mean(a64 ** 2)))
    bound = np.maximum(1e-2 * rms, bf16_ulp(a64))
    err = np.abs(gotf - a64)
    assert np.all(err <= bound), "%s: max excess %.3e" % (what, float((err - bound).max()))
    same = assert_bf16_rounding(got_bits, a64, swiglu_slack(x_bits, wg_bits, wu_bits, a64), what)
    return same


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
        same = check_swiglu_layer(got[l], x[l], wg[l], wu[l], "layer %d" % l)
        say("layer %d: %.4f of the elements round as the exact value does" % (l, same))


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


def test_gate_up_swiglu_full_size_sampled():
    """The benchmarked shape (bench.py --op swiglu at the page-1 stack: hidden
    5120, FFN 17408, N = 4, b = 1, 64 layers, weights [64][5120][4352] each)
    in the launch configuration bench.py times: layers 0, 32 and 63 on
    sampled columns, to the derived bound; repeated calls give the same bits."""
    from row_gemv_reduction_amd import workloads
    w = workloads.PAGE1
    L, b, H, C = w.layers, w.batch, w.hidden, w.ki_r
    say("gate/up swiglu full size: page-1 N=4 b=1, 64 layers, sampled columns")
    kw = dict(seed=0, workload=w.name, rank=0)
    x = synth.device_normal((L, b, H), 1.0, torch.bfloat16, tensor="x_ffn_in", **kw)
    wg = synth.device_normal((L, H, C), synth.WEIGHT_STD, torch.bfloat16, tensor="w_gate", **kw)
    wu = synth.device_normal((L, H, C), synth.WEIGHT_STD, torch.bfloat16, tensor="w_up", **kw)
    plan = tp.Plan(H, w.inter, w.n_ranks, b, k_attn=w.k_attn)
    ws = plan.new_workspace()
    out = torch.empty((L, b, C), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out)
    tp.tp_gate_up_swiglu(plan, L, x, wg, wu, out, ws)
    tp.tp_gate_up_swiglu(plan, L, x, wg, wu, out2, ws)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0
    got = bf16_bits_host(out)
    assert_bits_equal(bf16_bits_host(out2), got, "repeat")
    g = np.random.default_rng(5)
    cols = np.unique(np.concatenate([g.choice(C, 96, replace=False), [0, 255, 256, C - 1]]))
    ci = torch.from_numpy(cols).cuda()
    for l in (0, L // 2, L - 1):
        xb = bf16_bits_host(x[l])
        same = check_swiglu_layer(got[l][:, cols], xb, bf16_bits_host(wg[l].index_select(1, ci)),
                                  bf16_bits_host(wu[l].index_select(1, ci)), "layer %d" % l)
        say("layer %d: %.4f of the sampled elements round as the exact value does" % (l, same))
