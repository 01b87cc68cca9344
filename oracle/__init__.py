"""CPU oracle for one tensor-parallel rank's share of a decode step.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this; the product path never does.
The arithmetic lives in ``oracle.c`` (plain C, double accumulation); this
module only builds it with gcc and marshals numpy arrays through ctypes.
It shares no code with the HIP library.

Every wrapper takes and returns numpy arrays. bf16 data is carried as
``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
          "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no -ffast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.oracle_abi_version.restype = ctypes.c_int
        L.oracle_partial.argtypes = [vp, i64, vp, i64, i64, i64, vp, vp, ctypes.c_int]
        L.oracle_partial.restype = None
        L.oracle_ring_reduce.argtypes = [vp, i32, i64, vp, vp, vp]
        L.oracle_ring_reduce.restype = ctypes.c_int
        L.oracle_ring_wire_bytes_per_rank.argtypes = [i32, i64, i32]
        L.oracle_ring_wire_bytes_per_rank.restype = i64
        L.oracle_split_allreduce_total_bytes.argtypes = [i32, i64]
        L.oracle_split_allreduce_total_bytes.restype = i64
        L.oracle_naive_allreduce_total_bytes.argtypes = [i32, i64]
        L.oracle_naive_allreduce_total_bytes.restype = i64
        L.oracle_decode_layers.argtypes = [i32, i32, i32, i64, i64, i64, i64,
                                           vp, vp, vp, vp, vp, vp, ctypes.c_int]
        L.oracle_decode_layers.restype = ctypes.c_int
        L.oracle_moe_route.argtypes = [vp, i32, i32, i32, i32, vp, vp]
        L.oracle_moe_route.restype = ctypes.c_int
        L.oracle_moe_partial.argtypes = [i32, i32, vp, vp, i32, i32, vp, vp, i64, i64,
                                         vp, vp, ctypes.c_int]
        L.oracle_moe_partial.restype = ctypes.c_int
        L.oracle_gate_up_swiglu.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, ctypes.c_int]
        L.oracle_gate_up_swiglu.restype = ctypes.c_int
        L.oracle_qkv_proj.argtypes = [vp, vp, i64, i64, i64, vp, vp, ctypes.c_int]
        L.oracle_qkv_proj.restype = ctypes.c_int
        L.oracle_mx_element_value.argtypes = [i32, ctypes.c_uint32]
        L.oracle_mx_element_value.restype = ctypes.c_double
        L.oracle_mx_quantize.argtypes = [i32, vp, i64, i64, vp, vp]
        L.oracle_mx_quantize.restype = ctypes.c_int
        L.oracle_mx_partial.argtypes = [i32, vp, i64, i64, i64, vp, vp, vp, vp, ctypes.c_int]
        L.oracle_mx_partial.restype = ctypes.c_int
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (dtype, a.dtype))
    return np.ascontiguousarray(a)


def partial(x_bits, w_bits, nthreads: int = 1):
    """p[b, n] = sum_k x[b, k] * w[k, n]; returns (double, float) arrays.

    x_bits: uint16 [batch, k] (bf16); w_bits: uint16 [k, hidden] (bf16).
    """
    x = _c(x_bits, np.uint16)
    w = _c(w_bits, np.uint16)
    b, k = x.shape
    k2, h = w.shape
    if k != k2:
        raise ValueError("x and w disagree on k")
    y64 = np.empty((b, h), np.float64)
    y32 = np.empty((b, h), np.float32)
    lib().oracle_partial(_ptr(x), k, _ptr(w), b, k, h, _ptr(y64), _ptr(y32), nthreads)
    return y64, y32


def ring_reduce(partials, residual, want_bf16: bool = False):
    """out = ring-order sum of partials [N, ...] plus residual (float32)."""
    p = _c(partials, np.float32)
    r = _c(residual, np.float32)
    n = p.shape[0]
    length = r.size
    if p.size != n * length:
        raise ValueError("partials must be [N, *residual.shape]")
    out = np.empty_like(r)
    ob = np.empty(r.shape, np.uint16) if want_bf16 else None
    rc = lib().oracle_ring_reduce(_ptr(p), n, length, _ptr(r), _ptr(out), _ptr(ob))
    if rc != 0:
        raise ValueError("ring_reduce: N must divide the payload")
    return (out, ob) if want_bf16 else out


def ring_wire_bytes_per_rank(n_ranks: int, payload_elems: int, elem_bytes: int) -> int:
    return int(lib().oracle_ring_wire_bytes_per_rank(n_ranks, payload_elems, elem_bytes))


def split_allreduce_total_bytes(n_ranks: int, payload_bytes: int) -> int:
    return int(lib().oracle_split_allreduce_total_bytes(n_ranks, payload_bytes))


def naive_allreduce_total_bytes(n_ranks: int, payload_bytes: int) -> int:
    return int(lib().oracle_naive_allreduce_total_bytes(n_ranks, payload_bytes))


def decode_layers(rank, x_attn, w_o, x_ffn, w_down, slots, hidden_state, nthreads: int = 1):
    """Run the 2L reconciliation points; returns (slots, hidden_state) copies.

    x_attn [L, b, ka_r], w_o [L, ka_r, H], x_ffn [L, b, ki_r], w_down [L, ki_r, H]
    (uint16 bf16 bits); slots float32 [L, 2, N, b, H]; hidden_state float32 [b, H].
    """
    xa = _c(x_attn, np.uint16)
    wo = _c(w_o, np.uint16)
    xf = _c(x_ffn, np.uint16)
    wd = _c(w_down, np.uint16)
    s = _c(slots, np.float32).copy()
    h = _c(hidden_state, np.float32).copy()
    L, b, ka = xa.shape
    ki = xf.shape[2]
    n = s.shape[2]
    hid = h.shape[-1]
    rc = lib().oracle_decode_layers(L, n, rank, b, hid, ka, ki, _ptr(xa), _ptr(wo),
                                    _ptr(xf), _ptr(wd), _ptr(s), _ptr(h), nthreads)
    if rc != 0:
        raise ValueError("decode_layers: bad sizes")
    return s, h


def moe_route(logits, top_k: int, renorm: bool = True):
    """Top-k routing; returns (sel_expert int32 [T, k], sel_weight float64 [T, k])."""
    z = _c(logits, np.float32)
    t, e = z.shape
    se = np.empty((t, top_k), np.int32)
    sw = np.empty((t, top_k), np.float64)
    rc = lib().oracle_moe_route(_ptr(z), t, e, top_k, 1 if renorm else 0, _ptr(se), _ptr(sw))
    if rc != 0:
        raise ValueError("moe_route: bad sizes")
    return se, sw


def moe_partial(sel_expert, sel_weight, e_begin, u_bits, w_local_bits, nthreads: int = 1):
    """One rank's expert down projection + local weighted combine.

    u_bits uint16 [T, k, moe_inter]; w_local_bits uint16 [E_local, moe_inter, H].
    Returns (double, float) [T, H].
    """
    se = _c(sel_expert, np.int32)
    sw = _c(sel_weight, np.float64)
    u = _c(u_bits, np.uint16)
    w = _c(w_local_bits, np.uint16)
    t, k = se.shape
    el, mi, h = w.shape
    p64 = np.empty((t, h), np.float64)
    p32 = np.empty((t, h), np.float32)
    rc = lib().oracle_moe_partial(t, k, _ptr(se), _ptr(sw), e_begin, e_begin + el,
                                  _ptr(u), _ptr(w), mi, h, _ptr(p64), _ptr(p32), nthreads)
    if rc != 0:
        raise ValueError("moe_partial: bad sizes")
    return p64, p32


def gate_up_swiglu(x_bits, w_gate_bits, w_up_bits, nthreads: int = 1):
    """a = silu(x . W_gate) * (x . W_up); returns (double array, bf16 bits).

    x_bits: uint16 [batch, hidden]; w_gate_bits, w_up_bits: uint16
    [hidden, cols] (bf16).
    """
    x = _c(x_bits, np.uint16)
    wg = _c(w_gate_bits, np.uint16)
    wu = _c(w_up_bits, np.uint16)
    b, h = x.shape
    if wg.shape != wu.shape or wg.shape[0] != h:
        raise ValueError("x, w_gate and w_up disagree")
    c = wg.shape[1]
    a64 = np.empty((b, c), np.float64)
    abf = np.empty((b, c), np.uint16)
    rc = lib().oracle_gate_up_swiglu(_ptr(x), _ptr(wg), _ptr(wu), b, h, c, _ptr(a64), _ptr(abf),
                                     nthreads)
    if rc != 0:
        raise ValueError("gate_up_swiglu: bad sizes")
    return a64, abf


def qkv_proj(x_bits, w_bits, nthreads: int = 1):
    """a = x . W_qkv (the rank's columns); returns (double array, bf16 bits).

    x_bits: uint16 [batch, hidden]; w_bits: uint16 [hidden, cols] (bf16).
    """
    x = _c(x_bits, np.uint16)
    w = _c(w_bits, np.uint16)
    b, h = x.shape
    if w.shape[0] != h:
        raise ValueError("x and w disagree on hidden")
    c = w.shape[1]
    a64 = np.empty((b, c), np.float64)
    abf = np.empty((b, c), np.uint16)
    rc = lib().oracle_qkv_proj(_ptr(x), _ptr(w), b, h, c, _ptr(a64), _ptr(abf), nthreads)
    if rc != 0:
        raise ValueError("qkv_proj: bad sizes")
    return a64, abf


def bf16_to_f32(bits) -> float:
    return float(lib().oracle_bf16_to_f32(int(bits)))


def f32_to_bf16(value) -> int:
    return int(lib().oracle_f32_to_bf16(float(np.float32(value))))


MXFP8, MXFP4 = 1, 2
MX_BLOCK = 32


def mx_element_value(fmt: int, code: int) -> float:
    """Value of one MX element code (fmt 1: FP8 E4M3, fmt 2: FP4 E2M1)."""
    return float(lib().oracle_mx_element_value(fmt, int(code)))


def mx_codes_shape(fmt: int, k: int, h: int):
    return (k, h) if fmt == MXFP8 else (k // 2, h)


def mx_quantize(fmt: int, w_bits):
    """bf16 weights [K, H] -> (codes uint8, scales uint8 [K/32, H]) in the MX
    interchange layout (fmt 1: codes [K, H]; fmt 2: [K/2, H], two rows of a
    column per byte, the even row in the low nibble)."""
    w = _c(w_bits, np.uint16)
    k, h = w.shape
    codes = np.empty(mx_codes_shape(fmt, k, h), np.uint8)
    scales = np.empty((k // MX_BLOCK, h), np.uint8)
    if lib().oracle_mx_quantize(fmt, _ptr(w), k, h, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("mx_quantize: bad format or size (K must be a multiple of 32)")
    return codes, scales


def mx_partial(fmt: int, x_bits, codes, scales, nthreads: int = 1):
    """p = x . W for MX weights W (codes, scales as mx_quantize gives them);
    returns (double, float) arrays [batch, H]."""
    x = _c(x_bits, np.uint16)
    c = _c(codes, np.uint8)
    sc = _c(scales, np.uint8)
    b, k = x.shape
    h = sc.shape[1]
    if sc.shape[0] * MX_BLOCK != k or c.shape != mx_codes_shape(fmt, k, h):
        raise ValueError("mx_partial: codes / scales do not match x")
    y64 = np.empty((b, h), np.float64)
    y32 = np.empty((b, h), np.float32)
    if lib().oracle_mx_partial(fmt, _ptr(x), b, k, h, _ptr(c), _ptr(sc), _ptr(y64), _ptr(y32),
                               nthreads) != 0:
        raise ValueError("mx_partial: bad format or size")
    return y64, y32
