"""GPU parity of the microscaled (MXFP8 / MXFP4) weight path against the
oracle ("Hosting Qwen on Blackwell", Quantization: weights converted once,
statically, to MXFP8; MXFP4 weighed too).

- tp_quantize_mx is byte work: codes and scales must equal the oracle's bit
  for bit (random weights over many binades, zero blocks, subnormal and
  non-finite weights, the full page-1 FFN slice).
- tp_pack_weights_mx is a layout change: checked byte for byte.
- The packed decode step on MX weights, on either stream (the vector-ALU
  stream on pair strips, the matrix-core stream on MX tiles): each partial
  within 1e-5 * rms of the oracle's exact MX projection; the ring stage bit
  for bit against the oracle's ring chain on the GPU's partials; both point
  orders, the partials-only and the no-alloc forms give the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
from row_gemv_reduction_amd import binding as tp
from row_gemv_reduction_amd import synth, workloads
from tests.gpu_helpers import assert_bits_equal, assert_partial_close, bf16_bits_host, host, say

pytestmark = pytest.mark.gpu

FMTS = [tp.TP_WEIGHTS_MXFP8, tp.TP_WEIGHTS_MXFP4]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def u8(t):
    return t.cpu().numpy().view(np.uint8)


def quantize_dev(plan, point, w_dev):
    L = w_dev.shape[0]
    codes = torch.empty(tp.mx_codes_shape(plan, point, L), dtype=torch.uint8, device="cuda")
    scales = torch.empty(tp.mx_scales_shape(plan, point, L), dtype=torch.uint8, device="cuda")
    tp.tp_quantize_mx(plan, point, w_dev, codes, scales)
    return codes, scales


def pack_mx_dev(plan, point, codes, scales):
    p = torch.empty(tp.packed_shape(plan, point, codes.shape[0]), dtype=torch.uint8, device="cuda")
    tp.tp_pack_weights_mx(plan, point, codes, scales, p)
    return p


def hard_weights(k, h, seed):
    """bf16 weights over ~60 binades per block, with an all-zero block, a
    block of bf16 subnormals, ties of the element grid and one block holding
    an infinity and one a NaN."""
    g = np.random.default_rng(seed)
    v = g.standard_normal((k, h)) * np.exp2(g.integers(-30, 31, (k // 32, h)).repeat(32, 0))
    v *= np.exp2(g.integers(-4, 5, (k, h)))
    v[0:32, 0] = 0.0
    v[32:64, 1] = g.standard_normal(32) * 2.0 ** -130
    v[0:32, 2] = np.array([256.0, 1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 480.0, 2.5, 5.0] * 4)
    v[0:32, 3] = np.inf
    v[32:64, 3] = np.nan
    return synth.f32_to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_matches_oracle_bit_for_bit(fmt):
    k, h = 256, 264
    say("MX quantise fmt=%d k=%d h=%d" % (fmt, k, h))
    w = hard_weights(k, h, 11 + fmt)
    plan = tp.Plan(h, k, 1, 1, weight_format=fmt)
    codes, scales = quantize_dev(plan, 1, dev_u16(w[None]))
    torch.cuda.synchronize()
    c_or, s_or = oracle.mx_quantize(fmt, w)
    assert_bits_equal(u8(scales)[0], s_or, "scales")
    assert_bits_equal(u8(codes)[0], c_or, "codes")


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_full_page1_ffn_slice(fmt):
    """The page-1 FFN down-projection slice of one rank (4352 x 5120), drawn as
    the benchmark draws it, two layers."""
    w = workloads.PAGE1
    say("MX quantise fmt=%d, page-1 FFN slice" % fmt)
    W = synth.device_normal((2, w.ki_r, w.hidden), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down",
                            seed=0, workload=w.name, rank=0)
    plan = tp.Plan(w.hidden, w.inter, w.n_ranks, w.batch, weight_format=fmt)
    codes, scales = quantize_dev(plan, 1, W)
    torch.cuda.synchronize()
    for l in range(2):
        c_or, s_or = oracle.mx_quantize(fmt, bf16_bits_host(W[l]))
        assert_bits_equal(u8(scales)[l], s_or, "scales l=%d" % l)
        assert_bits_equal(u8(codes)[l], c_or, "codes l=%d" % l)


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_layout(fmt):
    L, n, h, ka, ki = 2, 2, 520, 256, 1024
    plan = tp.Plan(h, ki, n, 1, k_attn=ka, weight_format=fmt)
    assert plan.info()["packed_kind"] == 1
    say("MX pack layout fmt=%d" % fmt)
    for point, k in ((0, ka // n), (1, ki // n)):
        w = synth.normal_bf16((L, k, h), synth.WEIGHT_STD, seed=12, tensor="w", layer=point)
        codes, scales = quantize_dev(plan, point, dev_u16(w))
        got = u8(pack_mx_dev(plan, point, codes, scales))
        torch.cuda.synchronize()
        c, sc = u8(codes), u8(scales)
        S = h // 4
        rows = 4  # interchange code rows per 16-byte vector: 4 FP8 rows, or 4 bytes of two FP4 rows
        kv = c.shape[1] // rows
        vec = c.reshape(L, kv, rows, S, 4).transpose(0, 3, 1, 4, 2)      # [l][s][v][col][row]
        sw = sc.reshape(L, k // 32, S, 4).transpose(0, 2, 1, 3)           # [l][s][blk][col]
        want = np.concatenate([np.ascontiguousarray(vec).ravel(), np.ascontiguousarray(sw).ravel()])
        assert_bits_equal(got, want, "packed point %d" % point)


def mx_stack(plan, L, n, b, h, ka, ki, rank, seed):
    kw = dict(seed=seed, workload="mx", rank=rank)
    xa = synth.normal_bf16((L, b, ka // n), 1.0, tensor="x_attn", **kw)
    wo = synth.normal_bf16((L, ka // n, h), synth.WEIGHT_STD, tensor="w_o", **kw)
    xf = synth.normal_bf16((L, b, ki // n), 1.0, tensor="x_ffn", **kw)
    wd = synth.normal_bf16((L, ki // n, h), synth.WEIGHT_STD, tensor="w_down", **kw)
    slots = synth.normal_f32((L, 2, n, b, h), 0.3, tensor="slots", **kw)
    h0 = synth.normal_f32((b, h), 1.0, tensor="residual", **kw)
    return xa, wo, xf, wd, slots, h0


def ring_chain(slots_gpu, h0):
    h = np.array(h0, dtype=np.float32, copy=True)
    for l in range(slots_gpu.shape[0]):
        for pt in range(2):
            h = oracle.ring_reduce(slots_gpu[l, pt], h)
    return h


MX_CASES = [
    # (n, b, hidden, k_attn, inter, rank): ragged strips per workgroup, 1..8
    # tokens, several ranks, a ring chunk starting inside a strip (b*H/N = 66)
    (4, 1, 1032, 1024, 4096, 0), (2, 3, 520, 512, 1408, 1), (8, 8, 4096, 4096, 12288, 7),
    (4, 1, 264, 512, 1024, 2), (1, 2, 256, 256, 512, 0), (4, 5, 5120, 2048, 8192, 3),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,b,h,ka,ki,rank", MX_CASES)
def test_mx_decode_matches_oracle(fmt, n, b, h, ka, ki, rank):
    L = 3
    say("MX decode fmt=%d n=%d b=%d h=%d ka=%d ki=%d rank=%d" % (fmt, n, b, h, ka, ki, rank))
    plan = tp.Plan(h, ki, n, b, k_attn=ka, weight_format=fmt, tune={"stream_kind": 1})
    assert plan.info()["packed_kind"] == 1
    xa, wo, xf, wd, slots, h0 = mx_stack(plan, L, n, b, h, ka, ki, rank, 13)
    qo = quantize_dev(plan, 0, dev_u16(wo))
    qd = quantize_dev(plan, 1, dev_u16(wd))
    po, pd = pack_mx_dev(plan, 0, *qo), pack_mx_dev(plan, 1, *qd)
    XA, XF = dev_u16(xa), dev_u16(xf)
    outs = []
    for serial in (0, 1):
        plan.tune("serial_points", serial)
        ws = plan.new_workspace()
        S, Hd = torch.from_numpy(slots).cuda(), torch.from_numpy(h0).cuda()
        tp.tp_decode_layers_packed(plan, L, rank, XA, po, XF, pd, S, Hd, ws)
        torch.cuda.synchronize()
        assert tp.tp_workspace_status(plan, ws) == 0
        outs.append((host(S), host(Hd)))
    plan.tune("serial_points", 0)
    # the dataflow order with a point per bank and with banks across points
    for flat in (0, 1):
        plan.tune("stream_flat", flat)
        ws = plan.new_workspace()
        S, Hd = torch.from_numpy(slots).cuda(), torch.from_numpy(h0).cuda()
        tp.tp_decode_layers_packed(plan, L, rank, XA, po, XF, pd, S, Hd, ws)
        torch.cuda.synchronize()
        assert tp.tp_workspace_status(plan, ws) == 0
        outs.append((host(S), host(Hd)))
    plan.tune("stream_flat", -1)
    for o, what in ((outs[1], "serial"), (outs[2], "a point per bank"), (outs[3], "banks across points")):
        assert_bits_equal(o[0], outs[0][0], "slots, %s vs dataflow" % what)
        assert_bits_equal(o[1], outs[0][1], "hidden, %s vs dataflow" % what)
    s_gpu, h_gpu = outs[0]
    # no-alloc form and partials-only form: the same bits
    S2, H2 = torch.from_numpy(slots).cuda(), torch.from_numpy(h0).cuda()
    tp.tp_decode_layers_packed_noalloc(plan, L, rank, XA, po, XF, pd, S2, H2)
    P = torch.empty((L, 2, b, h), dtype=torch.float32, device="cuda")
    ws = plan.new_workspace()
    tp.tp_rowparallel_partials_packed(plan, L, XA, po, XF, pd, P, ws)
    torch.cuda.synchronize()
    assert_bits_equal(host(S2), s_gpu, "no-alloc slots")
    assert_bits_equal(host(H2), h_gpu, "no-alloc hidden")
    assert_bits_equal(host(P), s_gpu[:, :, rank], "partials-only")
    # against the oracle: quantisation, projection, ring stage
    co, so = u8(qo[0]), u8(qo[1])
    cd, sd = u8(qd[0]), u8(qd[1])
    for l in range(L):
        c_or, s_or = oracle.mx_quantize(fmt, wo[l])
        assert_bits_equal(co[l], c_or, "codes w_o l=%d" % l)
        assert_bits_equal(so[l], s_or, "scales w_o l=%d" % l)
        assert_partial_close(s_gpu[l, 0, rank], oracle.mx_partial(fmt, xa[l], co[l], so[l])[0], "attn l=%d" % l)
        assert_partial_close(s_gpu[l, 1, rank], oracle.mx_partial(fmt, xf[l], cd[l], sd[l])[0], "ffn l=%d" % l)
    others = [r for r in range(n) if r != rank]
    assert_bits_equal(s_gpu[:, :, others], slots[:, :, others], "other ranks' slots untouched")
    assert_bits_equal(h_gpu, ring_chain(s_gpu, h0), "hidden vs the oracle's ring chain")


def test_mx_plans_refuse_what_they_cannot_run():
    """MX weights: K_r must be a multiple of 32 (else no packed kind), and
    bf16 packing or bf16 quantisation is refused."""
    p = tp.Plan(512, 1040, 2, 1, weight_format=tp.TP_WEIGHTS_MXFP8)  # K_r of the FFN point = 520
    assert p.info()["packed_kind"] == 0
    q = tp.Plan(512, 1024, 2, 1, weight_format=tp.TP_WEIGHTS_MXFP4)
    w = torch.zeros((1, 512, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tp.TPError):
        tp.tp_pack_weights(q, 1, w, torch.empty(tp.packed_shape(q, 1, 1), dtype=torch.uint8, device="cuda"))
    b = tp.Plan(512, 1024, 2, 1)
    with pytest.raises(tp.TPError):
        tp.tp_quantize_mx(b, 1, w, torch.empty(tp.mx_codes_shape(b, 1, 1), dtype=torch.uint8, device="cuda"),
                          torch.empty(tp.mx_scales_shape(b, 1, 1), dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("fmt", FMTS)
def test_mx_page1_full_size_sampled(fmt):
    """The page-1 stack (hidden 5120, FFN 17408, 64 layers, N = 4, b = 1) on
    MX weights in the launch configuration bench.py times: quantised on the
    GPU; layers 0, 32 and 63 on sampled columns: codes and scales bit for
    bit, partials against the oracle's MX projection; the whole hidden chain
    bit for bit against the oracle's ring chain."""
    w = workloads.PAGE1
    L, b, H, rank = w.layers, w.batch, w.hidden, 0
    say("MX page-1 full size fmt=%d" % fmt)
    kw = dict(seed=0, workload=w.name, rank=rank)
    xa = synth.device_normal((L, b, w.ka_r), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((L, w.ka_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    xf = synth.device_normal((L, b, w.ki_r), 1.0, torch.bfloat16, tensor="x_ffn", **kw)
    wd = synth.device_normal((L, w.ki_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down", **kw)
    slots = synth.device_normal((L, 2, w.n_ranks, b, H), synth.WEIGHT_STD * np.sqrt(w.ki_r), torch.float32,
                                tensor="slots", seed=0, workload=w.name)
    h0 = synth.device_normal((b, H), 1.0, torch.float32, tensor="residual", seed=0, workload=w.name)
    plan = tp.Plan(H, w.inter, w.n_ranks, b, k_attn=w.k_attn, weight_format=fmt)
    assert plan.info()["packed_kind"] == 1
    qo, qd = quantize_dev(plan, 0, wo), quantize_dev(plan, 1, wd)
    po, pd = pack_mx_dev(plan, 0, *qo), pack_mx_dev(plan, 1, *qd)
    ws = plan.new_workspace()
    S, Hd = slots.clone(), h0.clone()
    tp.tp_decode_layers_packed(plan, L, rank, xa, po, xf, pd, S, Hd, ws)
    torch.cuda.synchronize()
    assert tp.tp_workspace_status(plan, ws) == 0
    s_got = host(S)
    assert_bits_equal(host(Hd), ring_chain(s_got, host(h0)), "hidden vs the oracle's ring chain")
    g = np.random.default_rng(8)
    cols = np.unique(np.concatenate([g.choice(H, 48, replace=False), [0, 3, 4, H - 1]]))
    ci = torch.from_numpy(cols).cuda()
    for l in (0, L // 2, L - 1):
        for pt, (x, W, (codes, scales)) in enumerate(((xa, wo, qo), (xf, wd, qd))):
            wcols = bf16_bits_host(W[l].index_select(1, ci))
            c_or, s_or = oracle.mx_quantize(fmt, wcols)
            c_got = u8(codes[l].index_select(1, ci))
            s_got_ = u8(scales[l].index_select(1, ci))
            assert_bits_equal(c_got, c_or, "codes l=%d pt=%d" % (l, pt))
            assert_bits_equal(s_got_, s_or, "scales l=%d pt=%d" % (l, pt))
            ref64, _ = oracle.mx_partial(fmt, bf16_bits_host(x[l]), c_or, s_or)
            assert_partial_close(s_got[l, pt, rank][:, cols], ref64, "partial l=%d pt=%d" % (l, pt))


# ------------------------------------------- the matrix-core stream (MX tiles)

@pytest.mark.parametrize("fmt", FMTS)
def test_pack_layout_mfma_tiles(fmt):
    """MX tiles of the matrix-core stream, byte for byte: per tile of 64 rows
    x 16 columns the codes lane-major (lane l: rows 16(l/16) .. +15 of column
    l%16; FP8 one byte a row, FP4 two rows a byte), then the 32 scale bytes
    [block][column]; zero past K (K_r = 160: a half tile)."""
    L, n, h, ka, ki = 2, 2, 528, 320, 1024
    plan = tp.Plan(h, ki, n, 1, k_attn=ka, weight_format=fmt, tune={"stream_kind": 2})
    assert plan.info()["packed_kind"] == 2
    say("MX tile layout fmt=%d" % fmt)
    for point, k in ((0, ka // n), (1, ki // n)):
        w = synth.normal_bf16((L, k, h), synth.WEIGHT_STD, seed=14, tensor="w", layer=point)
        codes, scales = quantize_dev(plan, point, dev_u16(w))
        got = u8(pack_mx_dev(plan, point, codes, scales))
        torch.cuda.synchronize()
        c, sc = u8(codes), u8(scales)
        nkb, S = (k + 63) // 64, h // 16
        if fmt == tp.TP_WEIGHTS_MXFP8:
            cz = np.zeros((L, 64 * nkb, h), np.uint8)
            cz[:, :k] = c
            # rows 64kb + 16g + i, columns 16s + col -> [l][s][kb][g][col][i]
            cw = cz.reshape(L, nkb, 4, 16, S, 16).transpose(0, 4, 1, 2, 5, 3).reshape(L, S, nkb, 1024)
        else:
            cz = np.zeros((L, 32 * nkb, h), np.uint8)
            cz[:, :k // 2] = c
            cw = cz.reshape(L, nkb, 4, 8, S, 16).transpose(0, 4, 1, 2, 5, 3).reshape(L, S, nkb, 512)
        sz = np.zeros((L, 2 * nkb, h), np.uint8)
        sz[:, :k // 32] = sc
        sw = sz.reshape(L, nkb, 2, S, 16).transpose(0, 3, 1, 2, 4).reshape(L, S, nkb, 32)
        want = np.concatenate([cw, sw], axis=3)
        assert_bits_equal(got, want.ravel(), "tiles point %d" % point)


MX_MFMA_CASES = [
    # (n, b, hidden, k_attn, inter, rank): the H4096 N=8 slices; K_r of 160
    # and 512 (a half tile) with 65 strips and activations in A-operand
    # order; 672 rows (ragged) at 3 tokens row-major; 16 tokens; one rank
    (8, 1, 4096, 4096, 12288, 7), (4, 5, 1040, 640, 2048, 1), (2, 3, 528, 512, 1344, 0),
    (4, 16, 256, 512, 1024, 2), (1, 2, 64, 64, 128, 0),
]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,b,h,ka,ki,rank", MX_MFMA_CASES)
def test_mx_mfma_stream_matches_oracle(fmt, n, b, h, ka, ki, rank):
    """The matrix-core stream on MX tiles: each partial within 1e-5 * rms of
    the oracle's exact MX projection, the ring stage bit for bit against the
    oracle's ring chain on the GPU's partials, in both ways of holding the
    tiles in registers (a bank per segment, a ring of slots) and both
    activation layouts; the no-alloc form gives the same bits."""
    L = 3
    say("MX matrix-core stream fmt=%d n=%d b=%d h=%d ka=%d ki=%d rank=%d" % (fmt, n, b, h, ka, ki, rank))
    plan = tp.Plan(h, ki, n, b, k_attn=ka, weight_format=fmt, tune={"stream_kind": 2})
    assert plan.info()["packed_kind"] == 2
    xa, wo, xf, wd, slots, h0 = mx_stack(plan, L, n, b, h, ka, ki, rank, 15)
    qo = quantize_dev(plan, 0, dev_u16(wo))
    qd = quantize_dev(plan, 1, dev_u16(wd))
    po, pd = pack_mx_dev(plan, 0, *qo), pack_mx_dev(plan, 1, *qd)
    co, so = u8(qo[0]), u8(qo[1])
    cd, sd = u8(qd[0]), u8(qd[1])
    refs = [(oracle.mx_partial(fmt, xa[l], co[l], so[l])[0], oracle.mx_partial(fmt, xf[l], cd[l], sd[l])[0])
            for l in range(L)]
    others = [r for r in range(n) if r != rank]
    for flat in (0, 1):
        for acts in ((1, 2) if b <= 16 else (2,)):
            plan.tune("mfma_flat", flat)
            plan.tune("mfma_acts", acts)
            XA, XF = dev_u16(xa), dev_u16(xf)
            pa = torch.empty(tp.packed_act_shape(plan, 0, L), dtype=torch.bfloat16, device="cuda")
            pf = torch.empty(tp.packed_act_shape(plan, 1, L), dtype=torch.bfloat16, device="cuda")
            tp.tp_pack_activations(plan, XA, XF, pa, pf)
            ws = plan.new_workspace()
            S, Hd = torch.from_numpy(slots).cuda(), torch.from_numpy(h0).cuda()
            tp.tp_decode_layers_packed(plan, L, rank, pa, po, pf, pd, S, Hd, ws)
            S2, H2 = torch.from_numpy(slots).cuda(), torch.from_numpy(h0).cuda()
            tp.tp_decode_layers_packed_noalloc(plan, L, rank, pa, po, pf, pd, S2, H2)
            torch.cuda.synchronize()
            assert tp.tp_workspace_status(plan, ws) == 0
            s_gpu, h_gpu = host(S), host(Hd)
            what = "flat=%d acts=%d" % (flat, acts)
            assert_bits_equal(host(S2), s_gpu, "no-alloc slots " + what)
            assert_bits_equal(host(H2), h_gpu, "no-alloc hidden " + what)
            for l in range(L):
                assert_partial_close(s_gpu[l, 0, rank], refs[l][0], "attn l=%d %s" % (l, what))
                assert_partial_close(s_gpu[l, 1, rank], refs[l][1], "ffn l=%d %s" % (l, what))
            assert_bits_equal(s_gpu[:, :, others], slots[:, :, others], "other ranks' slots untouched")
            assert_bits_equal(h_gpu, ring_chain(s_gpu, h0), "hidden vs the oracle's ring chain " + what)
