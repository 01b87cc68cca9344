"""tp_decode_layers_packed_noalloc: the packed decode step on the library's
per-GPU scratch instead of a caller's workspace, against
tp_decode_layers_packed on the same inputs, bit for bit, on two calls in a
row (the second with a smaller input, so that it runs on the first one's
leftover scratch), on both streams and both point orders."""
import numpy as np
import pytest
import torch

from row_gemv_reduction_amd import binding as tp
from row_gemv_reduction_amd import synth
from tests.gpu_helpers import assert_bits_equal, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def stack(L, n, b, h, ka, ki, rank, seed):
    kw = dict(seed=seed, workload="noalloc", rank=rank)
    xa = synth.device_normal((L, b, ka // n), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((L, ka // n, h), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    xf = synth.device_normal((L, b, ki // n), 1.0, torch.bfloat16, tensor="x_ffn", **kw)
    wd = synth.device_normal((L, ki // n, h), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down", **kw)
    slots = synth.device_normal((L, 2, n, b, h), 0.3, torch.float32, tensor="slots", seed=seed,
                                workload="noalloc")
    h0 = synth.device_normal((b, h), 1.0, torch.float32, tensor="residual", seed=seed, workload="noalloc")
    return xa, wo, xf, wd, slots, h0


def packed_inputs(plan, L, xa, wo, xf, wd):
    po = torch.empty(tp.packed_shape(plan, 0, L), dtype=torch.bfloat16, device="cuda")
    pd = torch.empty(tp.packed_shape(plan, 1, L), dtype=torch.bfloat16, device="cuda")
    tp.tp_pack_weights(plan, 0, wo, po)
    tp.tp_pack_weights(plan, 1, wd, pd)
    pa = torch.empty(tp.packed_act_shape(plan, 0, L), dtype=torch.bfloat16, device="cuda")
    pf = torch.empty(tp.packed_act_shape(plan, 1, L), dtype=torch.bfloat16, device="cuda")
    tp.tp_pack_activations(plan, xa, xf, pa, pf)
    return pa, po, pf, pd


# (kind, serial, first call (L, n, b, h, ka, ki, rank), second call, smaller)
CASES = [
    (1, 0, (6, 4, 1, 5120, 5120, 17408, 0), (2, 4, 1, 1032, 640, 2048, 3)),
    (1, 1, (5, 4, 2, 4096, 4096, 12288, 1), (3, 2, 1, 520, 512, 1376, 1)),
    (2, 0, (4, 4, 64, 4096, 4096, 12288, 2), (2, 8, 16, 1024, 1024, 4096, 5)),
    (2, 0, (3, 2, 32, 5120, 5120, 17408, 1), (2, 4, 5, 1040, 640, 2048, 0)),
]


@pytest.mark.parametrize("kind,serial,first,second", CASES)
def test_noalloc_equals_workspace_entry_point(kind, serial, first, second):
    for call, (L, n, b, h, ka, ki, rank) in enumerate((first, second)):
        say("no-alloc kind=%d serial=%d call %d: L=%d n=%d b=%d h=%d ka=%d ki=%d rank=%d"
            % (kind, serial, call, L, n, b, h, ka, ki, rank))
        xa, wo, xf, wd, slots, h0 = stack(L, n, b, h, ka, ki, rank, 81 + call)
        plan = tp.Plan(h, ki, n, b, k_attn=ka, tune={"stream_kind": kind, "serial_points": serial})
        assert plan.info()["packed_kind"] == kind
        pa, po, pf, pd = packed_inputs(plan, L, xa, wo, xf, wd)
        ws = plan.new_workspace()
        S1, H1 = slots.clone(), h0.clone()
        tp.tp_decode_layers_packed(plan, L, rank, pa, po, pf, pd, S1, H1, ws)
        S2, H2 = slots.clone(), h0.clone()
        tp.tp_decode_layers_packed_noalloc(plan, L, rank, pa, po, pf, pd, S2, H2)
        torch.cuda.synchronize()
        assert tp.tp_workspace_status(plan, ws) == 0
        assert tp.tp_workspace_status(plan, None) == 0
        assert_bits_equal(host(S2), host(S1), "slots, call %d" % call)
        assert_bits_equal(host(H2), host(H1), "hidden, call %d" % call)


def test_noalloc_rejects_plans_beyond_its_scratch():
    """hidden 5120 with 64 tokens on the matrix-core stream needs 10 MiB of
    exchange buffers, more than the 8 MiB the scratch holds: refused before
    anything is enqueued; 48 tokens (7.5 MiB) fit."""
    for b, ok in ((64, False), (48, True)):
        n, h, ka, ki, L = 2, 5120, 1024, 2048, 1
        plan = tp.Plan(h, ki, n, b, k_attn=ka, tune={"stream_kind": 2})
        xa, wo, xf, wd, slots, h0 = stack(L, n, b, h, ka, ki, 0, 90)
        pa, po, pf, pd = packed_inputs(plan, L, xa, wo, xf, wd)
        S, Hd = slots.clone(), h0.clone()
        if ok:
            tp.tp_decode_layers_packed_noalloc(plan, L, 0, pa, po, pf, pd, S, Hd)
            ws = plan.new_workspace()
            S1, H1 = slots.clone(), h0.clone()
            tp.tp_decode_layers_packed(plan, L, 0, pa, po, pf, pd, S1, H1, ws)
            torch.cuda.synchronize()
            assert_bits_equal(host(Hd), host(H1), "hidden, b=48")
        else:
            with pytest.raises(tp.TPError) as e:
                tp.tp_decode_layers_packed_noalloc(plan, L, 0, pa, po, pf, pd, S, Hd)
            assert e.value.status == tp.TP_ERR_UNSUPPORTED
            torch.cuda.synchronize()
            assert_bits_equal(host(Hd), host(h0), "untouched when refused")
