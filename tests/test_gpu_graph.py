"""Library calls replayed from a HIP graph give the eager bits.

A graph is captured once and replayed several times, with eager work and
synchronisations of the program's own between the replays; every replay's
output is compared bit for bit with the same calls issued eagerly from the
same inputs. Covered: the per-point row-parallel partial + ring sum sequence
(the MFMA skinny GEMM at 16 tokens and more, the VALU GEMV below), the
MoE layer share on two streams (routing and the rank's experts beside the
attention point, joined by the MoE ring sum) and the one-entry layer share
(tp_moe_layer_decode).
"""
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


def replay_against_eager(run, state, reset, other_work, replays=4):
    """run(): issues the calls; state(): the tensors they write; reset():
    restores the inputs they read and write in place."""
    reset()
    run()
    torch.cuda.synchronize()
    want = [host(t).copy() for t in state()]
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for r in range(replays):
        reset()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(state(), want)):
            assert_bits_equal(host(t), w, "replay %d, output %d" % (r, i))
        other_work()
        torch.cuda.synchronize()


@pytest.mark.parametrize("b", [4, 32])
def test_partial_and_ring_sequence_replays_bitwise(b):
    H, KA, KI, N, L = 1024, 2048, 4096, 4, 2
    say("graph: partial + ring, b=%d" % b)
    plan = tp.Plan(H, KI, N, b, k_attn=KA)
    ws = plan.new_workspace()
    kw = dict(seed=29, rank=1)
    xa = synth.device_normal((L, b, KA // N), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((L, KA // N, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    xf = synth.device_normal((L, b, KI // N), 1.0, torch.bfloat16, tensor="x_ffn", **kw)
    wd = synth.device_normal((L, KI // N, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down", **kw)
    s0 = synth.device_normal((L, 2, N, b, H), synth.WEIGHT_STD * 40, torch.float32, tensor="slots", seed=29)
    h0 = synth.device_normal((b, H), 1.0, torch.float32, tensor="residual", seed=29)
    slots, hidden = s0.clone(), h0.clone()
    scratch = torch.empty((b, H), dtype=torch.float32, device="cuda")

    def run():
        for l in range(L):
            tp.tp_rowparallel_partial(plan, 0, xa[l], wo[l], slots[l, 0, 1], ws)
            tp.tp_ring_reduce(plan, slots[l, 0], hidden, hidden)
            tp.tp_rowparallel_partial(plan, 1, xf[l], wd[l], slots[l, 1, 1], ws)
            tp.tp_ring_reduce(plan, slots[l, 1], hidden, hidden)

    def reset():
        slots.copy_(s0)
        hidden.copy_(h0)

    def other_work():  # eager calls of the same library on other buffers
        tp.tp_rowparallel_partial(plan, 1, xf[0], wd[0], scratch, ws)

    replay_against_eager(run, lambda: (slots, hidden), reset, other_work)
    plan.close()


def test_debug_sync_mode_eager_and_graph():
    """With the library's debug mode on (a stream wait and an error check
    after every launch) the same sequence runs eagerly, and a graph captured
    meanwhile (no waits while capturing) replays it bit for bit."""
    tp.tp_set_debug_sync(1)
    try:
        test_partial_and_ring_sequence_replays_bitwise(4)
    finally:
        tp.tp_set_debug_sync(0)


def test_moe_share_on_two_streams_replays_bitwise():
    T, E, k, I, H, ep, KA = 64, 32, 4, 512, 1024, 4, 2048
    rank = 2
    el = E // ep
    say("graph: MoE share T=%d E=%d k=%d I=%d H=%d ep=%d" % (T, E, k, I, H, ep))
    plan = tp.Plan(H, KA, ep, T, k_attn=KA, moe=dict(n_experts=E, top_k=k, ep=ep, moe_inter=I, max_tokens=T))
    kw = dict(seed=31, rank=rank)
    xa = synth.device_normal((T, KA // ep), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((KA // ep, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    logits = synth.device_normal((T, E), 1.0, torch.float32, tensor="logits", seed=31)
    u = synth.device_normal((T, k, I), 1.0, torch.bfloat16, tensor="u", **kw)
    we = synth.device_normal((el, I, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_expert", **kw)
    wp = torch.empty(tp.moe_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_experts(plan, we, wp)
    s0 = synth.device_normal((2, ep, T, H), synth.WEIGHT_STD * 40, torch.float32, tensor="slots", seed=31)
    h0 = synth.device_normal((T, H), 1.0, torch.float32, tensor="residual", seed=31)
    slots, hidden = s0.clone(), h0.clone()
    se = torch.empty((T, k), dtype=torch.int32, device="cuda")
    sw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws, ws_moe = plan.new_workspace(), plan.new_workspace()
    side = torch.cuda.Stream()
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    scratch = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def run():
        cur = torch.cuda.current_stream()
        fork.record(cur)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            tp.tp_moe_route(plan, logits, se, sw)
            tp.tp_moe_partial(plan, rank, se, sw, u, wp, slots[1, rank], ws_moe)
            join.record(side)
        tp.tp_decode_point(plan, 0, rank, xa, wo, slots[0], hidden, ws)
        cur.wait_event(join)
        tp.tp_ring_reduce(plan, slots[1], hidden, hidden)

    def reset():
        slots.copy_(s0)
        hidden.copy_(h0)
        se.fill_(-1)
        sw.fill_(float("nan"))

    def other_work():
        tp.tp_moe_partial(plan, rank, se, sw, u, wp, scratch, ws_moe)

    replay_against_eager(run, lambda: (slots, hidden, se, sw), reset, other_work)
    plan.close()


def test_moe_layer_share_entry_replays_bitwise():
    # tp_moe_layer_decode's routing counter is cleared by its own second
    # launch, so the captured pair of launches replays as often as needed
    T, E, k, I, H, ep, KA = 64, 32, 4, 512, 1024, 4, 512
    rank = 1
    el = E // ep
    say("graph: tp_moe_layer_decode T=%d E=%d k=%d I=%d H=%d ep=%d" % (T, E, k, I, H, ep))
    plan = tp.Plan(H, KA * ep, ep, T, k_attn=KA * ep,
                   moe=dict(n_experts=E, top_k=k, ep=ep, moe_inter=I, max_tokens=T))
    kw = dict(seed=37, rank=rank)
    xa = synth.device_normal((T, KA), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((KA, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    logits = synth.device_normal((T, E), 1.0, torch.float32, tensor="logits", seed=37)
    u = synth.device_normal((T, k, I), 1.0, torch.bfloat16, tensor="u", **kw)
    we = synth.device_normal((el, I, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_expert", **kw)
    wp = torch.empty(tp.moe_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_experts(plan, we, wp)
    wap = torch.empty(tp.moe_attn_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_attn(plan, wo, wap)
    s0 = synth.device_normal((2, ep, T, H), synth.WEIGHT_STD * 40, torch.float32, tensor="slots", seed=37)
    h0 = synth.device_normal((T, H), 1.0, torch.float32, tensor="residual", seed=37)
    slots, hidden = s0.clone(), h0.clone()
    se = torch.empty((T, k), dtype=torch.int32, device="cuda")
    sw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ws = plan.new_workspace()
    other = [s0.clone(), h0.clone()]

    def run():
        tp.tp_moe_layer_decode(plan, rank, logits, xa, wap, u, wp, se, sw, slots[0], slots[1], hidden, ws)

    def reset():
        slots.copy_(s0)
        hidden.copy_(h0)
        se.fill_(-1)
        sw.fill_(float("nan"))

    def other_work():  # an eager call of the same entry on other buffers and the same workspace
        tp.tp_moe_layer_decode(plan, rank, logits, xa, wap, u, wp, se, sw, other[0][0], other[0][1],
                               other[1], ws)

    replay_against_eager(run, lambda: (slots, hidden, se, sw), reset, other_work)
    assert tp.tp_workspace_status(plan, ws) == 0
    plan.close()
