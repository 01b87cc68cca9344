"""GPU parity of the column-parallel QKV projection (tp_qkv_proj) against
the CPU oracle.

The output is bf16, so the bar is the bf16-output reading of the tolerance:
every element within max(1e-2 * rms, one bf16 ulp) of the oracle's double
value. It is also checked to the bound the arithmetic gives: the GPU's fp32
sum is within 1e-5 * rms of the exact one (the partial tolerance) and is
rounded once to bf16, so every output is within 1e-5 * rms + half a bf16
ulp of the exact value; only values within 1e-5 * rms of a rounding
boundary may round to the other neighbour.
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


def check_qkv_layer(got_bits, x_bits, w_bits, what):
    a64, _ = oracle.qkv_proj(x_bits, w_bits)
    gotf = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    rms = float(np.sqrt(np.mean(a64 ** 2)))
    bound = np.maximum(1e-2 * rms, bf16_ulp(a64))
    err = np.abs(gotf - a64)
    assert np.all(err <= bound), "%s: max excess %.3e" % (what, float((err - bound).max()))
    return assert_bf16_rounding(got_bits, a64, 1e-5 * rms, what)


# (n_ranks, batch, hidden, cols, layers, swiglu_layers, step_rows): vector-ALU
# and matrix-core steps, odd and even stacks, several launches ending on a
# lone odd layer, one tile per K and split K with a ragged 32-row step
CASES = [
    (1, 1, 520, 264, 3, 0, 0), (4, 3, 1024, 1536, 4, 0, 0), (2, 8, 264, 1000, 2, 0, 0),
    (4, 16, 1032, 776, 5, 2, 0), (8, 64, 512, 384, 2, 0, 0), (2, 24, 4104, 520, 3, 0, 512),
    (1, 5, 2048, 1024, 1, 0, 0), (4, 40, 1024, 2048, 6, 4, 0),
]


@pytest.mark.parametrize("n,b,h,cols,L,per,rows", CASES)
def test_qkv_proj_matches_oracle(n, b, h, cols, L, per, rows):
    say("qkv n=%d b=%d h=%d cols=%d L=%d per=%d rows=%d" % (n, b, h, cols, L, per, rows))
    kw = dict(seed=91, workload="qkv")
    x = synth.normal_bf16((L, b, h), 1.0, tensor="x_qkv_in", **kw)
    w = synth.normal_bf16((L, h, cols), synth.WEIGHT_STD, tensor="w_qkv", **kw)
    plan = tp.Plan(h, 2048, n, b, qkv_cols=cols, tune={"swiglu_layers": per, "step_rows": rows})
    ws = plan.new_workspace()
    X, W = to_dev_bf16(x), to_dev_bf16(w)
    out = torch.empty((L, b, cols), dtype=torch.bfloat16, device="cuda")
    tp.tp_qkv_proj(plan, L, X, W, out, ws)
    out2 = torch.empty_like(out)
    tp.tp_qkv_proj(plan, L, X, W, out2, ws)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0
    got = bf16_bits_host(out)
    assert_bits_equal(bf16_bits_host(out2), got, "repeat")
    for l in range(L):
        same = check_qkv_layer(got[l], x[l], w[l], "layer %d" % l)
        say("layer %d: %.4f of the elements round as the exact value does" % (l, same))


def test_qkv_proj_needs_width_and_empty_stack():
    """Without tp_plan_set_qkv_dim the call is refused; an empty stack does
    nothing."""
    b, h, cols = 2, 520, 264
    plan = tp.Plan(h, 2048, 2, b)
    plan.qkv_cols = cols  # the Python side only: the library still has none
    ws = plan.new_workspace()
    x = torch.zeros((1, b, h), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, h, cols), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, b, cols), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tp.TPError):
        tp.tp_qkv_proj(plan, 1, x, w, out, ws)
    plan2 = tp.Plan(h, 2048, 2, b, qkv_cols=cols)
    ws2 = plan2.new_workspace()
    tp.tp_qkv_proj(plan2, 0, torch.empty((0, b, h), dtype=torch.bfloat16, device="cuda"),
                   torch.empty((0, h, cols), dtype=torch.bfloat16, device="cuda"),
                   torch.empty((0, b, cols), dtype=torch.bfloat16, device="cuda"), ws2)
    torch.cuda.synchronize()


@pytest.mark.parametrize("b,h,cols,L", [(1, 1024, 768, 4), (64, 512, 384, 3)])
def test_xcd_walk_gives_the_same_bits(b, h, cols, L):
    """The XCD-contiguous tile walk ("xcd_walk") only changes which workgroup
    takes which tile: the vector-ALU (b = 1) and matrix-core (b = 64) steps
    give the same bits either way, for the QKV projection and for the up
    projection with SwiGLU."""
    say("xcd_walk b=%d h=%d cols=%d L=%d" % (b, h, cols, L))
    kw = dict(seed=93, workload="qkv")
    x = to_dev_bf16(synth.normal_bf16((L, b, h), 1.0, tensor="x_qkv_in", **kw))
    w = to_dev_bf16(synth.normal_bf16((L, h, cols), synth.WEIGHT_STD, tensor="w_qkv", **kw))
    wu = to_dev_bf16(synth.normal_bf16((L, h, cols), synth.WEIGHT_STD, tensor="w_up", **kw))
    got = {}
    for walk in (0, 1):
        plan = tp.Plan(h, 2 * cols, 2, b, qkv_cols=cols, tune={"xcd_walk": walk})
        ws = plan.new_workspace()
        q = torch.empty((L, b, cols), dtype=torch.bfloat16, device="cuda")
        a = torch.empty((L, b, cols), dtype=torch.bfloat16, device="cuda")
        tp.tp_qkv_proj(plan, L, x, w, q, ws)
        tp.tp_gate_up_swiglu(plan, L, x, w, wu, a, ws)
        torch.cuda.synchronize()
        assert tp.tp_workspace_status(plan, ws) == 0
        got[walk] = (bf16_bits_host(q), bf16_bits_host(a))
    assert_bits_equal(got[1][0], got[0][0], "qkv")
    assert_bits_equal(got[1][1], got[0][1], "swiglu")


def test_qkv_proj_full_size_sampled():
    """The benchmarked shape (bench.py --op qkv at the page-1 stack: hidden
    5120, N = 4, b = 1, 64 layers, 1536 columns: 1280 query columns and one
    key and one value head of 128) in the launch configuration bench.py
    times: layers 0, 32 and 63 on sampled columns; repeated calls give the
    same bits."""
    from row_gemv_reduction_amd import workloads
    w = workloads.PAGE1
    L, b, H, C = w.layers, w.batch, w.hidden, 1536
    say("qkv full size: page-1 N=4 b=1, 64 layers, 1536 columns, sampled columns")
    kw = dict(seed=0, workload=w.name, rank=0)
    x = synth.device_normal((L, b, H), 1.0, torch.bfloat16, tensor="x_qkv_in", **kw)
    wq = synth.device_normal((L, H, C), synth.WEIGHT_STD, torch.bfloat16, tensor="w_qkv", **kw)
    plan = tp.Plan(H, w.inter, w.n_ranks, b, k_attn=w.k_attn, qkv_cols=C)
    ws = plan.new_workspace()
    out = torch.empty((L, b, C), dtype=torch.bfloat16, device="cuda")
    out2 = torch.empty_like(out)
    tp.tp_qkv_proj(plan, L, x, wq, out, ws)
    tp.tp_qkv_proj(plan, L, x, wq, out2, ws)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0
    got = bf16_bits_host(out)
    assert_bits_equal(bf16_bits_host(out2), got, "repeat")
    g = np.random.default_rng(6)
    cols = np.unique(np.concatenate([g.choice(C, 96, replace=False), [0, 255, 256, 1279, 1280, C - 1]]))
    ci = torch.from_numpy(cols).cuda()
    for l in (0, L // 2, L - 1):
        same = check_qkv_layer(got[l][:, cols], bf16_bits_host(x[l]),
                               bf16_bits_host(wq[l].index_select(1, ci)), "layer %d" % l)
        say("layer %d: %.4f of the sampled elements round as the exact value does" % (l, same))
