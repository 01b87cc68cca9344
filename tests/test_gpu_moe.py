"""GPU parity of the expert-parallel MoE share against the CPU oracle.

Routing: the expert choice is compared exactly (both sides compare the same
fp32 logits), the weights within fp32 rounding of the oracle's double values.
Expert projections + local combine: within the projection tolerance
(1e-5 * rms of the oracle's double result), using the GPU's routing weights
on both sides so that the comparison isolates the projection and combine.
"""
import numpy as np
import pytest
import torch

import oracle
from row_gemv_reduction_amd import binding as tp
from row_gemv_reduction_amd import synth, workloads
from tests.gpu_helpers import (assert_bits_equal, assert_partial_close, bf16_bits_host, host,
                               say, to_dev_bf16, to_dev_f32)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def moe_plan(H, E, k, ep, I, T):
    return tp.Plan(H, 8 * ep, ep, 1, moe=dict(n_experts=E, top_k=k, ep=ep, moe_inter=I, max_tokens=T))


def gpu_route(plan, logits, renorm=True):
    i = plan.info()
    T = logits.shape[0]
    se = torch.full((T, i["top_k"]), -1, dtype=torch.int32, device="cuda")
    sw = torch.full((T, i["top_k"]), float("nan"), dtype=torch.float32, device="cuda")
    tp.tp_moe_route(plan, to_dev_f32(logits), se, sw, renorm=renorm)
    torch.cuda.synchronize()
    return host(se), host(sw)


def check_route(logits, k, renorm):
    T, E = logits.shape
    plan = moe_plan(64, E, k, 1, 64, T)
    se, sw = gpu_route(plan, logits, renorm)
    se_or, sw_or = oracle.moe_route(logits, k, renorm)
    assert_bits_equal(se, se_or, "selected experts")
    err = np.abs(sw.astype(np.float64) - sw_or).max()
    assert err <= 2.0 ** -23 * np.abs(sw_or).max() + 1e-30, err


@pytest.mark.parametrize("T,E,k,renorm", [(64, 128, 8, True), (64, 128, 8, False), (5, 100, 3, True),
                                          (3, 16, 16, False), (1, 2048, 32, True), (7, 65, 1, True)])
def test_route_matches_oracle(T, E, k, renorm):
    say("route T=%d E=%d k=%d renorm=%d" % (T, E, k, renorm))
    logits = synth.normal_f32((T, E), 1.0, seed=3, tensor="logits", layer=E)
    check_route(logits, k, renorm)


def test_route_ties_go_to_the_lower_index():
    say("route ties")
    logits = np.zeros((4, 128), np.float32)
    logits[1, 5:] = 1.0          # 123 equal maxima: the 8 lowest indices among them win
    logits[2, ::7] = 2.0
    logits[3, 100] = -np.inf     # -inf logits are never chosen before finite ones
    check_route(logits, 8, True)


# ---------------------------------------------------- expert projections --

def moe_inputs(T, E, k, I, H, ep, seed, host_weights=True):
    logits = synth.normal_f32((T, E), 1.0, seed=seed, tensor="logits")
    u = synth.normal_bf16((T, k, I), 1.0, seed=seed, tensor="u")
    w = synth.normal_bf16((E, I, H), synth.WEIGHT_STD, seed=seed, tensor="w_expert") if host_weights else None
    return logits, u, w


def gpu_moe_partial(plan, rank, se, sw, u_bits, w_rank_dev):
    i = plan.info()
    packed = torch.empty(tp.moe_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_experts(plan, w_rank_dev, packed)
    T = se.shape[0]
    part = torch.full((T, i["hidden"]), float("nan"), device="cuda")
    ws = plan.new_workspace()
    tp.tp_moe_partial(plan, rank, torch.from_numpy(se).cuda(), torch.from_numpy(sw).cuda(),
                      to_dev_bf16(u_bits), packed, part, ws)
    torch.cuda.synchronize()
    return host(part)


@pytest.mark.parametrize("T,E,k,I,H,ep", [(10, 16, 4, 64, 256, 2), (64, 128, 8, 1536, 1040, 4),
                                          (3, 8, 2, 24, 16, 1), (33, 32, 8, 520, 2048, 4)])
def test_moe_partial_matches_oracle_every_rank(T, E, k, I, H, ep):
    say("moe partial T=%d E=%d k=%d I=%d H=%d ep=%d" % (T, E, k, I, H, ep))
    plan = moe_plan(H, E, k, ep, I, T)
    logits, u, w = moe_inputs(T, E, k, I, H, ep, 11)
    se, sw = gpu_route(plan, logits)
    el = E // ep
    total = np.zeros((T, H))
    for r in range(ep):
        got = gpu_moe_partial(plan, r, se, sw, u, to_dev_bf16(w[r * el:(r + 1) * el]))
        ref64, _ = oracle.moe_partial(se, sw.astype(np.float64), r * el, u, w[r * el:(r + 1) * el])
        assert_partial_close(got, ref64, "rank %d" % r)
        total += got
    # the ranks' partials sum to the full combine (all experts local)
    full64, _ = oracle.moe_partial(se, sw.astype(np.float64), 0, u, w)
    assert_partial_close(total, full64, "sum over ranks")


def test_moe_expert_with_many_tokens_and_tokens_without_local_experts():
    # tokens 0..18 all pick expert 1 (19 rows: two passes of at most 16
    # rows); tokens 19..23 pick only rank 1's experts; 33 strips of 16
    # columns (a last block of one strip)
    T, E, k, I, H, ep = 24, 8, 3, 40, 528, 2
    say("moe crafted routing")
    plan = moe_plan(H, E, k, ep, I, T)
    _, u, w = moe_inputs(T, E, k, I, H, ep, 12)
    se = np.array([[1, 4 + t % 2, 6 + t % 2] if t < 19 else [5, 6, 7] for t in range(T)], np.int32)
    sw = (np.arange(T * k, dtype=np.float32).reshape(T, k) % 5 + 1) / 10
    el = E // ep
    for r in range(ep):
        got = gpu_moe_partial(plan, r, se, sw, u, to_dev_bf16(w[r * el:(r + 1) * el]))
        ref64, _ = oracle.moe_partial(se, sw.astype(np.float64), r * el, u, w[r * el:(r + 1) * el])
        assert_partial_close(got, ref64, "rank %d" % r)
        if r == 0:
            assert np.all(got[19:] == 0.0), "tokens with no local expert must give zero rows"


def test_moe_partial_is_deterministic_and_skips_unselected_experts():
    T, E, k, I, H, ep = 16, 32, 2, 128, 1024, 1
    say("moe determinism")
    plan = moe_plan(H, E, k, ep, I, T)
    logits, u, w = moe_inputs(T, E, k, I, H, ep, 13)
    se, sw = gpu_route(plan, logits)
    wd = to_dev_bf16(w)
    a = gpu_moe_partial(plan, 0, se, sw, u, wd)
    b = gpu_moe_partial(plan, 0, se, sw, u, wd)
    assert_bits_equal(a, b, "repeat")
    # poison the weights of every expert no token selected: nothing changes
    unused = sorted(set(range(E)) - set(se.ravel().tolist()))
    assert unused, "want some unselected experts"
    w2 = w.copy()
    w2[unused] = 0x7FC0  # NaN
    c = gpu_moe_partial(plan, 0, se, sw, u, to_dev_bf16(w2))
    assert_bits_equal(a, c, "unselected experts are not read")


def test_moe_config_full_size_sampled_columns():
    """The MoE decode share at its full size (hidden 4096, 128 experts of
    1536, top-8, EP=4, 64 tokens), rank 2, weights drawn on the device;
    the oracle computes sampled columns."""
    w = workloads.MOE
    T, E, k, I, H, ep = w.batch, w.n_experts, w.top_k, w.moe_inter, w.hidden, w.ep
    rank = 2
    say("moe full size, rank %d" % rank)
    plan = moe_plan(H, E, k, ep, I, T)
    logits = synth.normal_f32((T, E), 1.0, seed=0, workload=w.name, tensor="logits")
    u = synth.normal_bf16((T, k, I), 1.0, seed=0, workload=w.name, tensor="u", rank=rank)
    el = E // ep
    wdev = synth.device_normal((el, I, H), synth.WEIGHT_STD, torch.bfloat16, seed=0, workload=w.name,
                               tensor="w_expert", rank=rank)
    se, sw = gpu_route(plan, logits)
    se_or, _ = oracle.moe_route(logits, k, True)
    assert_bits_equal(se, se_or, "routing")
    got = gpu_moe_partial(plan, rank, se, sw, u, wdev)
    cols = np.array(sorted(set(np.random.default_rng(5).choice(H, 48, replace=False).tolist())
                           | {0, 255, 256, H - 1}))
    wcols = bf16_bits_host(wdev[:, :, torch.from_numpy(cols).cuda()].contiguous())
    ref64, _ = oracle.moe_partial(se, sw.astype(np.float64), rank * el, u, wcols, nthreads=8)
    assert_partial_close(got[:, cols], ref64, "sampled columns")


@pytest.mark.parametrize("T,E,k,I,H,ep", [(10, 16, 4, 64, 256, 2), (64, 128, 8, 1536, 1040, 4)])
def test_moe_decode_equals_partial_then_ring_bitwise(T, E, k, I, H, ep):
    say("moe decode T=%d E=%d k=%d I=%d H=%d ep=%d" % (T, E, k, I, H, ep))
    plan = tp.Plan(H, 8 * ep, ep, T, moe=dict(n_experts=E, top_k=k, ep=ep, moe_inter=I, max_tokens=T))
    logits, u, w = moe_inputs(T, E, k, I, H, ep, 17)
    se, sw = gpu_route(plan, logits)
    el = E // ep
    rank = ep - 1
    g = np.random.default_rng(19)
    slots = (g.standard_normal((ep, T, H)) * 0.5).astype(np.float32)
    h0 = g.standard_normal((T, H)).astype(np.float32)
    wr = to_dev_bf16(w[rank * el:(rank + 1) * el])
    packed = torch.empty(tp.moe_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_experts(plan, wr, packed)
    ws = plan.new_workspace()
    sed, swd, ud = torch.from_numpy(se).cuda(), torch.from_numpy(sw).cuda(), to_dev_bf16(u)
    # fused point
    S, hd = to_dev_f32(slots), to_dev_f32(h0)
    tp.tp_moe_decode(plan, rank, sed, swd, ud, packed, S, hd, ws)
    # composition
    P, hc = to_dev_f32(slots), to_dev_f32(h0)
    tp.tp_moe_partial(plan, rank, sed, swd, ud, packed, P[rank], ws)
    tp.tp_ring_reduce(plan, P, hc, hc)
    torch.cuda.synchronize()
    assert_bits_equal(host(S), host(P), "slots")
    assert_bits_equal(host(hd), host(hc), "hidden")
    ref64, _ = oracle.moe_partial(se, sw.astype(np.float64), rank * el, u, w[rank * el:(rank + 1) * el])
    assert_partial_close(host(S)[rank], ref64, "partial")


# ------------------------------------------------ the whole layer share --

def layer_plan(T, E, k, I, H, ep, KA):
    return tp.Plan(H, KA * ep, ep, T, k_attn=KA * ep,
                   moe=dict(n_experts=E, top_k=k, ep=ep, moe_inter=I, max_tokens=T))


def run_layer(plan, rank, logits, u, w_rank_dev, xa, wa_dev, slots_a, slots_m, h0, ws, renorm=True):
    i = plan.info()
    T, k = i["batch"], i["top_k"]
    wp = torch.empty(tp.moe_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_experts(plan, w_rank_dev, wp)
    wap = torch.empty(tp.moe_attn_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
    tp.tp_moe_pack_attn(plan, wa_dev, wap)
    se = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    sw = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    SA, SM, hd = to_dev_f32(slots_a), to_dev_f32(slots_m), to_dev_f32(h0)
    tp.tp_moe_layer_decode(plan, rank, to_dev_f32(logits), to_dev_bf16(xa), wap, to_dev_bf16(u), wp, se, sw,
                           SA, SM, hd, ws, renorm=renorm)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0, "a bounded wait timed out"
    return host(se), host(sw), host(SA), host(SM), host(hd)


def check_layer(T, E, k, I, H, ep, KA, rank, seed, renorm=True, ws=None, plan=None):
    plan = plan or layer_plan(T, E, k, I, H, ep, KA)
    ws = ws if ws is not None else plan.new_workspace()
    logits, u, w = moe_inputs(T, E, k, I, H, ep, seed)
    xa = synth.normal_bf16((T, KA), 1.0, seed=seed, tensor="x_attn")
    wa = synth.normal_bf16((KA, H), synth.WEIGHT_STD, seed=seed, tensor="w_o")
    el = E // ep
    g = np.random.default_rng(seed)
    slots_a = (g.standard_normal((ep, T, H)) * 0.5).astype(np.float32)
    slots_m = (g.standard_normal((ep, T, H)) * 0.5).astype(np.float32)
    h0 = g.standard_normal((T, H)).astype(np.float32)
    wr = w[rank * el:(rank + 1) * el]
    se, sw, SA, SM, hd = run_layer(plan, rank, logits, u, to_dev_bf16(wr), xa, to_dev_bf16(wa),
                                   slots_a, slots_m, h0, ws, renorm)
    # routing: the routing entry's bits, the oracle's choice
    se_r, sw_r = gpu_route(plan, logits, renorm)
    assert_bits_equal(se, se_r, "selected experts vs tp_moe_route")
    assert_bits_equal(sw, sw_r, "routing weights vs tp_moe_route")
    se_or, _ = oracle.moe_route(logits, k, renorm)
    assert_bits_equal(se, se_or, "selected experts vs the oracle")
    # the other ranks' slots are only read
    for r in range(ep):
        if r != rank:
            assert_bits_equal(SA[r], slots_a[r], "attention slot %d" % r)
            assert_bits_equal(SM[r], slots_m[r], "expert slot %d" % r)
    # the attention slice's partial against the oracle
    ref_a, _ = oracle.partial(xa, wa, nthreads=8)
    assert_partial_close(SA[rank], ref_a, "attention partial")
    # the experts: tp_moe_partial's bits, within tolerance of the oracle
    part = gpu_moe_partial(plan, rank, se, sw, u, to_dev_bf16(wr))
    assert_bits_equal(SM[rank], part, "expert partial vs tp_moe_partial")
    ref_m, _ = oracle.moe_partial(se, sw.astype(np.float64), rank * el, u, wr, nthreads=8)
    assert_partial_close(SM[rank], ref_m, "expert partial")
    # both ring stages, bit for bit, on the slots as written
    h1 = oracle.ring_reduce(SA, h0)
    assert_bits_equal(hd, oracle.ring_reduce(SM, h1), "hidden")
    return plan, ws


@pytest.mark.parametrize("T,E,k,I,H,ep,KA,rank", [
    (10, 16, 4, 64, 256, 2, 200, 1),       # one row group, a ragged last attention tile
    (64, 128, 8, 1536, 1040, 4, 512, 3),   # 65 strips: a last block of one strip
    (33, 100, 3, 520, 2048, 4, 264, 0),    # three row groups, 25 experts per rank
    (49, 32, 2, 64, 512, 2, 64, 1),        # four row groups, the last of one token
    (1, 8, 2, 24, 16, 1, 8, 0),            # one token, one rank, one strip
])
def test_moe_layer_share_matches_oracle_and_composition(T, E, k, I, H, ep, KA, rank):
    say("moe layer T=%d E=%d k=%d I=%d H=%d ep=%d KA=%d rank=%d" % (T, E, k, I, H, ep, KA, rank))
    check_layer(T, E, k, I, H, ep, KA, rank, 21)


def test_moe_layer_share_repeats_on_one_workspace_without_renorm():
    # the routing counter is cleared by each call's second launch: a second
    # call on the same workspace (other inputs) waits for its own routing
    T, E, k, I, H, ep, KA = 24, 64, 4, 128, 512, 4, 128
    say("moe layer repeated")
    plan, ws = check_layer(T, E, k, I, H, ep, KA, 2, 22)
    check_layer(T, E, k, I, H, ep, KA, 1, 23, renorm=False, ws=ws, plan=plan)
    check_layer(T, E, k, I, H, ep, KA, 0, 24, ws=ws, plan=plan)


def test_moe_layer_share_full_size_sampled_columns():
    """The layer share at its full size (hidden 4096, attention 8192 -> 4096
    over 4 ranks, 128 experts of 1536, top-8, EP=4, 64 tokens), rank 2,
    weights drawn on the device; the oracle computes sampled columns and
    both ring stages in full."""
    w = workloads.MOE
    T, E, k, I, H, ep, KA = w.batch, w.n_experts, w.top_k, w.moe_inter, w.hidden, w.ep, w.ka_r
    rank = 2
    el = E // ep
    say("moe layer full size, rank %d" % rank)
    plan = layer_plan(T, E, k, I, H, ep, KA)
    ws = plan.new_workspace()
    kw = dict(seed=0, workload=w.name, rank=rank)
    logits = synth.normal_f32((T, E), 1.0, seed=0, workload=w.name, tensor="logits")
    u = synth.normal_bf16((T, k, I), 1.0, tensor="u", **kw)
    xa = synth.normal_bf16((T, KA), 1.0, tensor="x_attn", **kw)
    wdev = synth.device_normal((el, I, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_expert", **kw)
    wadev = synth.device_normal((KA, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    g = np.random.default_rng(25)
    slots_a = (g.standard_normal((ep, T, H)) * 0.5).astype(np.float32)
    slots_m = (g.standard_normal((ep, T, H)) * 0.5).astype(np.float32)
    h0 = g.standard_normal((T, H)).astype(np.float32)
    se, sw, SA, SM, hd = run_layer(plan, rank, logits, u, wdev, xa, wadev, slots_a, slots_m, h0, ws)
    se_or, _ = oracle.moe_route(logits, k, True)
    assert_bits_equal(se, se_or, "routing")
    part = gpu_moe_partial(plan, rank, se, sw, u, wdev)
    assert_bits_equal(SM[rank], part, "expert partial vs tp_moe_partial")
    cols = np.array(sorted(set(np.random.default_rng(6).choice(H, 48, replace=False).tolist())
                           | {0, 127, 128, H - 1}))
    cdev = torch.from_numpy(cols).cuda()
    ref_a, _ = oracle.partial(xa, bf16_bits_host(wadev[:, cdev].contiguous()), nthreads=8)
    assert_partial_close(SA[rank][:, cols], ref_a, "attention partial, sampled columns")
    ref_m, _ = oracle.moe_partial(se, sw.astype(np.float64), rank * el, u,
                                  bf16_bits_host(wdev[:, :, cdev].contiguous()), nthreads=8)
    assert_partial_close(SM[rank][:, cols], ref_m, "expert partial, sampled columns")
    h1 = oracle.ring_reduce(SA, h0)
    assert_bits_equal(hd, oracle.ring_reduce(SM, h1), "hidden")
