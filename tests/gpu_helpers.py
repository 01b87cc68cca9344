"""Shared helpers of the GPU parity tests: host<->device copies of bf16 bit
patterns and the parity tolerances.

Tolerances (the acceptance bar of this path):
  * fp32 partial projections: max|got - ref| <= 1e-5 * rms(ref), with ref
    the oracle's double-accumulated value (normwise; a per-element relative
    error is undefined near zero).
  * ring-order reduction: bit-exact, given identical partials.
  * bf16 outputs: |got - ref| <= max(1e-2 * rms(ref), one bf16 ulp of ref)
    per element (correct rounding of the exact value already moves an
    element by up to half an ulp, which at |y| ~ 4-5 rms is ~1-2 % of rms).
"""
import sys

import numpy as np
import torch

PARTIAL_RTOL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bf16_bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_partial_close(got, ref64, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref64 ** 2)))
    err = float(np.abs(got - ref64).max()) if got.size else 0.0
    assert err <= PARTIAL_RTOL * rms, "%s: max|d|=%.3e > %.0e*rms=%.3e" % (
        what, err, PARTIAL_RTOL, PARTIAL_RTOL * rms)
    return err / rms if rms else 0.0


def assert_bits_equal(got, want, what=""):
    got = np.ascontiguousarray(got)
    want = np.ascontiguousarray(want)
    assert got.shape == want.shape, what
    gb = got.view(np.uint32 if got.dtype == np.float32 else np.uint16)
    wb = want.view(np.uint32 if want.dtype == np.float32 else np.uint16)
    bad = np.flatnonzero(gb.ravel() != wb.ravel())
    assert bad.size == 0, "%s: %d elements differ, first at %d: %r vs %r" % (
        what, bad.size, bad[0], got.ravel()[bad[0]], want.ravel()[bad[0]])


def bf16_ulp(v):
    """Spacing of bf16 at |v| (8 significant bits; subnormal spacing below 2^-126)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), np.float64(2.0 ** -126))
    return np.exp2(np.floor(np.log2(a)) - 7)


def assert_bf16_rounding(got_bits, a64, slack, what=""):
    """A bf16 output rounded once from a GPU fp32 value v: got = RNE_bf16(v)
    with |v - a64| <= slack (per element, a bound on the fp32 value's error
    against the exact a64). Then |got - a64| <= slack + half a bf16 ulp (at
    the larger of the two magnitudes, for values next to a power of two).
    Returns the fraction of elements equal to RNE_bf16 of the exact value's
    fp32 rounding (reported, not a bar)."""
    from row_gemv_reduction_amd import synth
    got = synth.bf16_bits_to_f32(got_bits).astype(np.float64)
    a64 = np.asarray(a64, dtype=np.float64)
    half = 0.5 * np.maximum(bf16_ulp(a64), bf16_ulp(got))
    bound = np.asarray(slack, dtype=np.float64) + half
    err = np.abs(got - a64)
    bad = np.flatnonzero(~(err <= bound))
    assert bad.size == 0, "%s: %d elements beyond slack + half ulp, first at %d: got %r exact %r " \
        "(slack %r)" % (what, bad.size, bad[0], got.ravel()[bad[0]], a64.ravel()[bad[0]],
                        np.broadcast_to(slack, a64.shape).ravel()[bad[0]])
    rne = synth.f32_to_bf16_bits(a64.astype(np.float32))
    return float(np.mean(np.asarray(got_bits) == rne))
