"""GPU parity of the prefill (tp_prefill_layers) against the oracle: the
same reconciliation points with a whole prompt of T tokens ("Interconnects
e clusters", lesson 9.9, Conceito: a 4,096-token prompt; every collective
carries 4,096 hidden vectors).

Each point's partial is the oracle's projection of T tokens (within
1e-5 * rms); the ring stage is checked bit for bit against the oracle's
ring sum run on the GPU's own partials, chained over every point; repeated
launches give the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
from row_gemv_reduction_amd import binding as tp
from row_gemv_reduction_amd import synth, workloads
from tests.gpu_helpers import assert_bits_equal, assert_partial_close, bf16_bits_host, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def packed(plan, point, w_dev):
    p = torch.empty(tp.prefill_packed_shape(plan, point, w_dev.shape[0]), dtype=torch.bfloat16, device="cuda")
    tp.tp_prefill_pack_weights(plan, point, w_dev, p)
    return p


def ring_chain(slots_gpu, h0):
    h = np.array(h0, dtype=np.float32, copy=True)
    for l in range(slots_gpu.shape[0]):
        for pt in range(2):
            h = oracle.ring_reduce(slots_gpu[l, pt], h)
    return h


CASES = [
    # (n, tokens, hidden, k_attn, inter, rank, layers): ragged token and column
    # tiles, K_r below one 64-row tile, N = 1, 3 and 8, chunk boundaries
    # inside a token row (T*H/N not a multiple of H)
    (4, 200, 528, 512, 1024, 1, 2), (2, 128, 1024, 640, 2048, 0, 3), (8, 64, 256, 512, 1024, 5, 2),
    (1, 33, 512, 256, 512, 0, 1), (3, 96, 528, 96, 192, 2, 2), (4, 130, 272, 1024, 4096, 3, 2),
]


@pytest.mark.parametrize("n,T,h,ka,ki,rank,L", CASES)
def test_prefill_matches_oracle(n, T, h, ka, ki, rank, L):
    say("prefill n=%d T=%d h=%d ka=%d ki=%d rank=%d L=%d" % (n, T, h, ka, ki, rank, L))
    kw = dict(seed=51, workload="prefill", rank=rank)
    xa = synth.normal_bf16((L, T, ka // n), 1.0, tensor="x_attn", **kw)
    wo = synth.normal_bf16((L, ka // n, h), synth.WEIGHT_STD, tensor="w_o", **kw)
    xf = synth.normal_bf16((L, T, ki // n), 1.0, tensor="x_ffn", **kw)
    wd = synth.normal_bf16((L, ki // n, h), synth.WEIGHT_STD, tensor="w_down", **kw)
    slots = synth.normal_f32((L, 2, n, T, h), 0.3, tensor="slots", **kw)
    h0 = synth.normal_f32((T, h), 1.0, tensor="residual", **kw)
    plan = tp.Plan(h, ki, n, 1, k_attn=ka)
    po, pd = packed(plan, 0, dev_bf16(wo)), packed(plan, 1, dev_bf16(wd))
    XA, XF = dev_bf16(xa), dev_bf16(xf)
    ws = plan.new_workspace()
    outs = []
    for _ in range(2):
        S, Hd = torch.from_numpy(slots).cuda(), torch.from_numpy(h0).cuda()
        tp.tp_prefill_layers(plan, L, rank, T, XA, po, XF, pd, S, Hd, ws)
        torch.cuda.synchronize()
        assert tp.tp_workspace_status(plan, ws) == 0
        outs.append((host(S), host(Hd)))
    assert_bits_equal(outs[1][0], outs[0][0], "slots, repeat")
    assert_bits_equal(outs[1][1], outs[0][1], "hidden, repeat")
    s_gpu, h_gpu = outs[0]
    for l in range(L):
        assert_partial_close(s_gpu[l, 0, rank], oracle.partial(xa[l], wo[l])[0], "attn l=%d" % l)
        assert_partial_close(s_gpu[l, 1, rank], oracle.partial(xf[l], wd[l])[0], "ffn l=%d" % l)
    others = [r for r in range(n) if r != rank]
    assert_bits_equal(s_gpu[:, :, others], slots[:, :, others], "other ranks' slots untouched")
    assert_bits_equal(h_gpu, ring_chain(s_gpu, h0), "hidden vs the oracle's ring chain")


def sampled_ring_chain(parts, h0, e_idx, total_len):
    """The oracle's ring sum + residual chained over points, for sampled
    elements only: each element is placed in its own chunk of a payload
    whose chunks are as long as needed, so oracle.ring_reduce adds it in the
    order of the chunk it has in the full [T x H] payload.
    parts: [points][N][m] the N ranks' values of the m sampled elements."""
    n = parts.shape[1]
    C = total_len // n
    chunk = e_idx // C
    m = e_idx.size
    h = np.array(h0, dtype=np.float32, copy=True)
    for j in range(parts.shape[0]):
        out = np.empty_like(h)
        for c in np.unique(chunk):
            sel = np.flatnonzero(chunk == c)
            P = np.zeros((n, n * sel.size), np.float32)
            R = np.zeros((n * sel.size,), np.float32)
            P[:, c * sel.size:(c + 1) * sel.size] = parts[j][:, sel]
            R[c * sel.size:(c + 1) * sel.size] = h[sel]
            out[sel] = oracle.ring_reduce(P, R)[c * sel.size:(c + 1) * sel.size]
        h = out
    assert m == h.size
    return h


def test_prefill_page1_4096_tokens_sampled():
    """The pages' prefill: the page-1 stack (hidden 5120, FFN 17408, 64
    layers, N = 4, rank 0) with a 4,096-token prompt, in the launch
    configuration bench.py times; partials of layers 0, 32 and 63 and the
    whole chain on sampled tokens x columns."""
    w = workloads.PREFILL
    L, T, H, n, rank = w.layers, w.batch, w.hidden, w.n_ranks, 0
    say("prefill page-1 T=%d, 64 layers" % T)
    kw = dict(seed=0, workload=w.name, rank=rank)
    xa = synth.device_normal((L, T, w.ka_r), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((L, w.ka_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    xf = synth.device_normal((L, T, w.ki_r), 1.0, torch.bfloat16, tensor="x_ffn", **kw)
    wd = synth.device_normal((L, w.ki_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down", **kw)
    slots = synth.device_normal((L, 2, n, T, H), synth.WEIGHT_STD * np.sqrt(w.ki_r), torch.float32,
                                tensor="slots", seed=0, workload=w.name)
    h0 = synth.device_normal((T, H), 1.0, torch.float32, tensor="residual", seed=0, workload=w.name)
    plan = tp.Plan(H, w.inter, n, 1, k_attn=w.k_attn)
    po, pd = packed(plan, 0, wo), packed(plan, 1, wd)
    g = np.random.default_rng(9)
    ts = np.unique(np.concatenate([g.choice(T, 20, replace=False), [0, 127, 128, 1023, 1024, T - 1]]))
    cs = np.unique(np.concatenate([g.choice(H, 20, replace=False), [0, 255, 256, H - 1]]))
    ti, ci = torch.from_numpy(ts).cuda(), torch.from_numpy(cs).cuda()
    # the other ranks' values at the sampled elements, before the launch
    before = slots.index_select(3, ti).index_select(4, ci).cpu().numpy()   # [L][2][N][t][c]
    h0s = h0.index_select(0, ti).index_select(1, ci).cpu().numpy()
    ws = plan.new_workspace()
    Hd = h0.clone()
    tp.tp_prefill_layers(plan, L, rank, T, xa, po, xf, pd, slots, Hd, ws)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0
    after = slots.index_select(3, ti).index_select(4, ci).cpu().numpy()
    others = [r for r in range(n) if r != rank]
    assert_bits_equal(after[:, :, others], before[:, :, others], "other ranks' slots untouched")
    for l in (0, L // 2, L - 1):
        for pt, (x, W) in enumerate(((xa, wo), (xf, wd))):
            ref64, _ = oracle.partial(bf16_bits_host(x[l].index_select(0, ti)),
                                      bf16_bits_host(W[l].index_select(1, ci)), nthreads=8)
            assert_partial_close(after[l, pt, rank], ref64, "l=%d pt=%d" % (l, pt))
    e_idx = (ts[:, None] * H + cs[None, :]).ravel()
    parts = after.reshape(2 * L, n, -1)
    want = sampled_ring_chain(parts, h0s.ravel(), e_idx, T * H).reshape(ts.size, cs.size)
    got = Hd.index_select(0, ti).index_select(1, ci).cpu().numpy()
    assert_bits_equal(got, want, "hidden (sampled) vs the oracle's ring chain")
