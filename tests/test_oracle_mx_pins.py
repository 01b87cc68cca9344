"""Pins of the oracle's microscaled (MX) weight formats against what the
formats and the mathematics fix ("Hosting Qwen on Blackwell", Quantization:
weights converted statically to MXFP8; MXFP4 weighed too).

Independent references: torch's float8_e4m3fn and float8_e8m0fnu dtypes
(element and scale decoding, and round-to-nearest-even conversion to E4M3
where no saturation is involved); E2M1 through its embedding in E4M3 (the
same sign, an exponent offset by 6 and the mantissa bit shifted left by
two) decoded by torch; exact rational arithmetic; blocks built from
representable values; ties and saturation derived by hand.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from row_gemv_reduction_amd import synth

F8, F4 = oracle.MXFP8, oracle.MXFP4


def torch_e4m3(codes):
    return torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_e8m0(scales):
    return torch.tensor(np.asarray(scales, np.uint8)).view(torch.float8_e8m0fnu).double().numpy()


def e2m1_as_e4m3(code):
    """The E4M3 code of the same value as E2M1 `code`: sign kept, exponent
    field + 6 (bias 1 -> 7), mantissa bit -> the top of three; the E2M1
    subnormal 0.5 is the E4M3 normal 2^-1, and zero stays zero."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    if e == 0:
        mag = 0 if m == 0 else (6 << 3)
    else:
        mag = ((e + 6) << 3) | (m << 2)
    return (s << 7) | mag


def unpack_fp4(codes, k):
    """[K/2][H] bytes (even row in the low nibble) -> [K][H] codes."""
    out = np.empty((k, codes.shape[1]), np.uint8)
    out[0::2] = codes & 0xF
    out[1::2] = codes >> 4
    return out


def decode(fmt, codes, scales, k):
    """Exact weights (float64) through torch's decoders."""
    c = codes if fmt == F8 else np.vectorize(e2m1_as_e4m3)(unpack_fp4(codes, k)).astype(np.uint8)
    return torch_e4m3(c) * np.repeat(torch_e8m0(scales), 32, axis=0)


# ------------------------------------------------------------ elements --

def test_e4m3_values_match_torch():
    got = np.array([oracle.mx_element_value(F8, c) for c in range(256)])
    want = torch_e4m3(np.arange(256))
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))  # -0 for 0x80
    assert np.isnan(want[[0x7F, 0xFF]]).all() and np.nanmax(want) == 448.0


def test_e2m1_values_through_their_e4m3_embedding():
    got = np.array([oracle.mx_element_value(F4, c) for c in range(16)])
    want = torch_e4m3([e2m1_as_e4m3(c) for c in range(16)])
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))
    assert got.max() == 6.0 and sorted(set(np.abs(got).tolist())) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


# ------------------------------------------------------------ quantise --

def random_weights(k, h, seed, spread=6):
    g = np.random.default_rng(seed)
    v = g.standard_normal((k, h)) * 0.02 * np.exp2(g.integers(-spread, spread + 1, (k // 32, h)).repeat(32, 0))
    return synth.f32_to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("fmt", [F8, F4])
def test_scaled_block_maximum_lands_in_the_top_binade(fmt):
    k, h = 256, 40
    w = random_weights(k, h, 1)
    codes, scales = oracle.mx_quantize(fmt, w)
    X = torch_e8m0(scales)
    amax = np.abs(synth.bf16_bits_to_f32(w).astype(np.float64)).reshape(k // 32, 32, h).max(axis=1)
    emax = 8 if fmt == F8 else 2
    r = amax / X
    assert np.all((r >= 2.0 ** emax) & (r < 2.0 ** (emax + 1)))


def test_e4m3_elements_round_as_torch_converts_them():
    """Element codes of MXFP8 are the nearest-even E4M3 values of w / X
    (torch's conversion), except that values beyond 448 saturate to 448
    where torch gives NaN."""
    k, h = 512, 64
    w = random_weights(k, h, 2)
    codes, scales = oracle.mx_quantize(F8, w)
    X = np.repeat(torch_e8m0(scales), 32, axis=0)
    v = synth.bf16_bits_to_f32(w).astype(np.float64) / X
    conv = torch.tensor(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    big = np.abs(v) > 448.0
    assert np.array_equal(codes[~big], conv[~big])
    assert np.all((codes[big] & 0x7F) == 0x7E)
    assert big.any()  # some block maxima do round past 448


@pytest.mark.parametrize("fmt", [F8, F4])
def test_representable_blocks_round_trip(fmt):
    """Weights built as element * 2^(E-127), with each block's largest
    element in the format's top binade, quantise back to the same codes and
    scales."""
    g = np.random.default_rng(3)
    k, h = 128, 24
    top = [0x78, 0x7E] if fmt == F8 else [0x6, 0x7]      # 256..448 / 4..6
    ncodes = 0x7F if fmt == F8 else 0x8
    el = g.integers(0, ncodes, (k, h)).astype(np.uint8)
    el |= (g.integers(0, 2, (k, h)) << (7 if fmt == F8 else 3)).astype(np.uint8)
    rows = g.integers(0, 32, (k // 32, h))
    for kb in range(k // 32):
        for n in range(h):
            el[kb * 32 + rows[kb, n], n] = g.integers(top[0], top[1] + 1)
    E = g.integers(100, 130, (k // 32, h)).astype(np.uint8)
    vals = (torch_e4m3(el) if fmt == F8 else torch_e4m3(np.vectorize(e2m1_as_e4m3)(el).astype(np.uint8)))
    w = synth.f32_to_bf16_bits((vals * np.repeat(torch_e8m0(E), 32, axis=0)).astype(np.float32))
    codes, scales = oracle.mx_quantize(fmt, w)
    assert np.array_equal(scales, E)
    got = codes if fmt == F8 else unpack_fp4(codes, k)
    assert np.array_equal(got, el)


@pytest.mark.parametrize("fmt,values,want", [
    # one block, X = 1 (largest 256 or 4): ties to the even code, saturation
    # 256 = 2^8 (e 15, m 0); 1.0625 halfway 1 | 1.125 -> 1; 1.1875 halfway
    # 1.125 | 1.25 -> 1.25; 2^-10 halfway 0 | 2^-9 -> 0; 3 * 2^-10 halfway
    # 2^-9 | 2^-8 -> 2^-8; 240 = 1.875 * 2^7 (e 14, m 7)
    (F8, [256.0, 1.0625, 1.1875, -1.0625, 2.0 ** -10, 3 * 2.0 ** -10, 240.0], [0x78, 0x38, 0x3A, 0xB8, 0x00, 0x02, 0x77]),
    (F8, [480.0, -500.0, 449.0], [0x7E, 0xFE, 0x7E]),
    # 2.5 halfway 2 | 3 -> 2; 5 halfway 4 | 6 -> 4; 0.25 halfway 0 | 0.5 -> 0;
    # 0.75 halfway 0.5 | 1 -> 1; 1.25 halfway 1 | 1.5 -> 1; 1.75 -> 2; 3.5 -> 4
    (F4, [4.0, 2.5, 5.0, 0.25, 0.75, -1.25, 1.75, 3.5], [0x6, 0x4, 0x6, 0x0, 0x2, 0xA, 0x4, 0x6]),
    (F4, [7.5, -7.0, 6.5], [0x7, 0xF, 0x7]),
])
def test_ties_and_saturation(fmt, values, want):
    k, h = 32, 1
    col = np.zeros((k,), np.float32)
    col[:len(values)] = values
    codes, scales = oracle.mx_quantize(fmt, synth.f32_to_bf16_bits(col.reshape(k, h)))
    assert scales[0, 0] == 127  # largest element in [2^emax, 2^(emax+1)): X = 1
    got = codes[:, 0] if fmt == F8 else unpack_fp4(codes, k)[:, 0]
    assert got[:len(values)].tolist() == want


@pytest.mark.parametrize("fmt", [F8, F4])
def test_quantisation_error_is_within_half_a_spacing(fmt):
    k, h = 256, 32
    w = random_weights(k, h, 4)
    codes, scales = oracle.mx_quantize(fmt, w)
    deq = decode(fmt, codes, scales, k)
    wf = synth.bf16_bits_to_f32(w).astype(np.float64)
    X = np.repeat(torch_e8m0(scales), 32, axis=0)
    v = np.abs(wf / X)
    mbits = 3 if fmt == F8 else 1
    emin = -6 if fmt == F8 else 0
    vmax = 448.0 if fmt == F8 else 6.0
    spacing = np.exp2(np.maximum(np.floor(np.log2(np.maximum(v, 2.0 ** -30))), emin) - mbits)
    sat = v > vmax
    assert np.all(np.abs(deq - wf)[~sat] <= 0.5 * spacing[~sat] * X[~sat])
    assert np.all(np.abs(deq[sat]) == vmax * X[sat])


def test_zero_and_nonfinite_blocks():
    w = np.zeros((64, 2), np.uint16)
    w[32:, 1] = synth.f32_to_bf16_bits(np.array([np.inf], np.float32))[0]
    for fmt in (F8, F4):
        codes, scales = oracle.mx_quantize(fmt, w)
        assert scales[0].tolist() == [0, 0] and scales[1].tolist() == [0, 255]
        assert not codes.any()


# ------------------------------------------------------------- product --

@pytest.mark.parametrize("fmt", [F8, F4])
def test_unit_scales_reduce_to_the_bf16_projection(fmt):
    """With every scale 127 (X = 1) the MX weights are their element values,
    each a bf16 value: the MX product equals oracle.partial on those bf16
    weights bit for bit."""
    g = np.random.default_rng(5)
    b, k, h = 3, 96, 40
    x = synth.normal_bf16((b, k), 1.0, seed=5, tensor="x")
    el = g.integers(0, 256 if fmt == F8 else 16, (k, h)).astype(np.uint8)
    if fmt == F8:
        el[(el & 0x7F) == 0x7F] = 0x11  # no NaN codes
        codes, vals = el, torch_e4m3(el)
    else:
        codes = (el[0::2] | (el[1::2] << 4)).astype(np.uint8)
        vals = torch_e4m3(np.vectorize(e2m1_as_e4m3)(el).astype(np.uint8))
    scales = np.full((k // 32, h), 127, np.uint8)
    _, y32 = oracle.mx_partial(fmt, x, codes, scales)
    _, ref32 = oracle.partial(x, synth.f32_to_bf16_bits(vals.astype(np.float32)))
    assert np.array_equal(y32.view(np.uint32), ref32.view(np.uint32))


@pytest.mark.parametrize("fmt", [F8, F4])
def test_raising_every_scale_doubles_the_product(fmt):
    k, h = 128, 16
    x = synth.normal_bf16((2, k), 1.0, seed=6, tensor="x")
    codes, scales = oracle.mx_quantize(fmt, random_weights(k, h, 6))
    y64, _ = oracle.mx_partial(fmt, x, codes, scales)
    y64b, _ = oracle.mx_partial(fmt, x, codes, (scales + 1).astype(np.uint8))
    assert np.array_equal(y64b, 2 * y64)


@pytest.mark.parametrize("fmt", [F8, F4])
def test_product_exact_bruteforce_tiny(fmt):
    b, k, h = 2, 64, 3
    x = synth.normal_bf16((b, k), 1.0, seed=7, tensor="x")
    codes, scales = oracle.mx_quantize(fmt, random_weights(k, h, 7, spread=3))
    W = decode(fmt, codes, scales, k)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    y64, y32 = oracle.mx_partial(fmt, x, codes, scales)
    for i in range(b):
        for n in range(h):
            exact = sum((Fraction(xf[i, kk]) * Fraction(W[kk, n]) for kk in range(k)), Fraction(0))
            absum = sum((abs(Fraction(xf[i, kk]) * Fraction(W[kk, n])) for kk in range(k)), Fraction(0))
            assert abs(Fraction(y64[i, n]) - exact) <= absum * k * Fraction(2) ** -53
            # the float result is the double one rounded once
            assert y32[i, n] == np.float32(y64[i, n])


def test_fp4_rows_pair_up_along_k():
    """MXFP4 holds two rows of a column per byte, the even row in the low
    nibble: a weight in an odd row must multiply x's odd column."""
    k, h = 32, 1
    w = np.zeros((k, h), np.float32)
    w[0, 0], w[1, 0] = 4.0, 1.0
    codes, scales = oracle.mx_quantize(F4, synth.f32_to_bf16_bits(w))
    x = np.zeros((1, k), np.float32)
    x[0, 1] = 1.0
    y64, _ = oracle.mx_partial(F4, synth.f32_to_bf16_bits(x), codes, scales)
    assert y64[0, 0] == 1.0
