"""The C interface on the host: the library loads, exports every declared
symbol, and its plan logic and argument validation behave as documented.
No compute call is made here (no GPU in this suite)."""
import ctypes
import os
import re

import pytest

from row_gemv_reduction_amd import binding
from row_gemv_reduction_amd.binding import (TP_ERR_ALIGNMENT, TP_ERR_INVALID_ARG,
                                            TP_ERR_UNSUPPORTED, TP_OK, Plan, TPError)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tp_decode.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(tp_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 13
    lib = binding._lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTS)


def test_plan_validation():
    L = binding._lib()
    h = ctypes.c_void_p()
    bad = [(0, 8, 1, 1), (8, 0, 1, 1), (8, 8, 0, 1), (8, 8, 1, 0),
           (5120, 17408, 3, 1),   # N does not divide I (or H)
           (24, 24, 3, 1),        # fine for K, but...
           ]
    for args in bad[:5]:
        assert L.tp_plan(*args, ctypes.byref(h)) == TP_ERR_INVALID_ARG, args
    assert L.tp_plan(24, 24, 3, 1, ctypes.byref(h)) == TP_OK  # 3 | 24 and 3 | 24
    L.tp_plan_destroy(h)
    assert L.tp_plan(16, 32, 32, 1, ctypes.byref(h)) == TP_ERR_INVALID_ARG  # N=32 does not divide H=16
    assert L.tp_plan(20, 40, 4, 1, ctypes.byref(h)) == TP_ERR_UNSUPPORTED   # H % 8 != 0
    assert L.tp_plan(512, 512, 2, 65, ctypes.byref(h)) == TP_ERR_UNSUPPORTED  # batch > 64
    assert L.tp_plan(512, 512, 2, 1, None) == TP_ERR_INVALID_ARG
    for s in range(6):
        assert L.tp_status_str(s)


def test_plan_rejects_ring_payload_not_divisible():
    # b*H must split into N equal chunks; H=8, N=8... use H=8*3=24, N=16? N must divide H too
    with pytest.raises(TPError):
        Plan(24, 48, 16, 1)


def test_plan_info_reproduces_the_pages_wire_bytes():
    mib = 1 << 20
    for n, want in ((2, 1.25), (4, 1.875)):
        i = Plan(5120, 17408, n, 1).info()
        assert i["wire_bytes_bf16"] * 128 == want * mib
        assert i["wire_bytes_fp32"] == 2 * i["wire_bytes_bf16"]
        assert i["chunk_elems"] == 5120 // n
        assert i["k_rank"] == [5120 // n, 17408 // n]


def test_plan_geometry_covers_every_row():
    for (H, I, N, b) in [(512, 1376, 2, 1), (5120, 17408, 4, 1), (5120, 17408, 2, 32),
                         (4096, 12288, 8, 64), (1032, 2000, 2, 3), (8, 8, 1, 1)]:
        p = Plan(H, I, N, b)
        i = p.info()
        for pt in (0, 1):
            assert i["path"][pt] == (1 if b >= 16 else 0)
            assert i["splits"][pt] >= 1
        assert i["workspace_bytes"] >= 64 * 1024


def test_plan_attn_dim_moe_and_tuning():
    p = Plan(4096, 4096, 4, 64, k_attn=8192,
             moe=dict(n_experts=128, top_k=8, ep=4, moe_inter=1536, max_tokens=64))
    i = p.info()
    assert i["k_attn"] == 8192 and i["k_rank"][0] == 2048
    assert i["local_experts"] == 32 and i["top_k"] == 8
    with pytest.raises(TPError):
        Plan(4096, 4096, 4, 1, k_attn=8191)
    with pytest.raises(TPError):
        Plan(4096, 4096, 4, 1, moe=dict(n_experts=128, top_k=8, ep=3, moe_inter=1536, max_tokens=64))
    with pytest.raises(TPError):
        Plan(4096, 4096, 4, 1, tune={"no_such_knob": 1})
    with pytest.raises(TPError):
        Plan(4096, 4096, 4, 1, tune={"valu_cols": 100})
    q = Plan(4096, 4096, 4, 1, tune={"splits_attn": 16, "valu_cols": 512})
    assert q.info()["splits"][0] == 16
    # the register-resident tile bounds the rows per split: 96 rows at 512 columns
    assert Plan(4096, 4096, 4, 1, tune={"splits_attn": 3, "valu_cols": 512}).info()["splits"][0] == 11


def test_matrix_core_stream_workgroups():
    # the matrix-core stream shares each point's tiles among one workgroup per
    # CU (at most one per 16-column strip, at least one per two strips)
    assert Plan(5120, 17408, 2, 16).info()["stream_wgs"] == 256
    assert Plan(1024, 4096, 4, 17).info()["stream_wgs"] == 64
    assert Plan(5120, 17408, 2, 16, tune={"stream_wgs": 200}).info()["stream_wgs"] == 200
    assert Plan(5120, 17408, 4, 1).info()["stream_wgs"] == 0  # vector-ALU stream
    # 320 strips need at least 160 workgroups: b = 4 falls back to the
    # vector-ALU stream, b = 16 has no streamed step
    p = Plan(5120, 17408, 2, 4, tune={"stream_kind": 2, "stream_wgs": 100})
    assert p.info()["packed_kind"] == 0
    p = Plan(5120, 17408, 2, 4, tune={"stream_wgs": 100})
    assert p.info()["packed_kind"] == 1 and p.info()["stream_wgs"] == 0
    assert Plan(5120, 17408, 2, 16, tune={"stream_wgs": 100}).info()["packed_kind"] == 0
    with pytest.raises(TPError):
        Plan(5120, 17408, 2, 16, tune={"stream_wgs": 257})
    # the workspace does not depend on the knob
    a = Plan(4096, 12288, 8, 64).info()["workspace_bytes"]
    assert Plan(4096, 12288, 8, 64, tune={"stream_wgs": 200}).info()["workspace_bytes"] == a


def test_entry_points_validate_before_launching():
    """Null and misaligned pointers are rejected on the host; nothing is
    enqueued (these addresses are never dereferenced)."""
    L = binding._lib()
    p = Plan(512, 1376, 2, 1)
    h = p.handle
    A, M = 4096, 4097  # an aligned and a misaligned fake address
    vp = ctypes.c_void_p
    assert L.tp_rowparallel_partial(h, 0, None, vp(A), vp(A), vp(A), None) == TP_ERR_INVALID_ARG
    assert L.tp_rowparallel_partial(h, 2, vp(A), vp(A), vp(A), vp(A), None) == TP_ERR_INVALID_ARG
    assert L.tp_rowparallel_partial(h, 0, vp(M), vp(A), vp(A), vp(A), None) == TP_ERR_ALIGNMENT
    assert L.tp_ring_reduce(h, vp(A), None, vp(A), None, None) == TP_ERR_INVALID_ARG
    assert L.tp_ring_reduce(h, vp(A), vp(A), vp(M), None, None) == TP_ERR_ALIGNMENT
    assert L.tp_decode_layers(h, 1, 2, *[vp(A)] * 8) == TP_ERR_INVALID_ARG  # rank >= N
    assert L.tp_decode_layers(h, -1, 0, *[vp(A)] * 8) == TP_ERR_INVALID_ARG
    assert L.tp_decode_layers(h, 1, 0, *[vp(A)] * 5, vp(M), vp(A), vp(A)) == TP_ERR_ALIGNMENT
    assert L.tp_workspace_init(h, None, None) == TP_ERR_INVALID_ARG


def test_weight_format_plans():
    """MX weight formats: the packed step needs K_r of both points to be a
    multiple of 32 and runs on the vector-ALU stream; the packed stack's
    bytes are the code vectors plus one scale byte per 32 rows of a column."""
    for fmt, rows_per_vec in ((binding.TP_WEIGHTS_MXFP8, 4), (binding.TP_WEIGHTS_MXFP4, 8)):
        i = Plan(5120, 17408, 4, 1, weight_format=fmt).info()
        assert i["weight_format"] == fmt and i["packed_kind"] == 1
        for pt, kr in enumerate((1280, 4352)):
            assert i["packed_layer_bytes"][pt] == (5120 // 4) * (kr // rows_per_vec * 16 + kr // 32 * 4)
            # codes + scales = K_r*H*(1 or 1/2) + K_r*H/32
            assert i["packed_layer_bytes"][pt] == kr * 5120 * (2 if fmt == 1 else 1) // 2 + kr // 32 * 5120
        assert Plan(512, 1040, 2, 1, weight_format=fmt).info()["packed_kind"] == 0  # K_r 520
        assert Plan(4096, 12288, 8, 64, weight_format=fmt).info()["packed_kind"] == 0  # batch > 8
    assert Plan(5120, 17408, 4, 1).info()["packed_layer_bytes"][1] == 5120 // 4 * 2176 * 16
    L = binding._lib()
    h = ctypes.c_void_p()
    assert L.tp_plan(512, 512, 2, 1, ctypes.byref(h)) == TP_OK
    assert L.tp_plan_set_weight_format(h, 3) == TP_ERR_INVALID_ARG
    assert L.tp_plan_set_weight_format(h, -1) == TP_ERR_INVALID_ARG
    assert L.tp_plan_set_weight_format(h, 1) == TP_OK
    L.tp_plan_destroy(h)


def test_debug_sync_switch():
    """The debug mode's switch takes 0 and 1 and refuses anything else (no
    device call is made: the mode only acts at the next launch)."""
    binding.tp_set_debug_sync(1)
    binding.tp_set_debug_sync(0)
    with pytest.raises(binding.TPError):
        binding.tp_set_debug_sync(2)
