"""ctypes binding of libtpdecode.so (the C interface in include/tp_decode.h).

Argument marshalling only: every function checks dtype, shape, contiguity
and device of the torch tensors it is given, then passes raw device
pointers and the current HIP stream to the library. All arithmetic runs in
the library's HIP kernels. Loading fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtpdecode.so")

TP_OK, TP_ERR_INVALID_ARG, TP_ERR_UNSUPPORTED, TP_ERR_ALIGNMENT, TP_ERR_DEVICE, TP_ERR_OOM = range(6)
TP_POINT_ATTN_OUT, TP_POINT_FFN_DOWN = 0, 1
TP_PATH_VALU, TP_PATH_MFMA = 0, 1
TP_WEIGHTS_BF16, TP_WEIGHTS_MXFP8, TP_WEIGHTS_MXFP4 = 0, 1, 2
MX_BLOCK = 32


class TPError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib().tp_status_str(status).decode() if _LIB is not None else str(status)
        super().__init__("%s failed: %s (status %d)" % (where, msg, status))


class tp_plan_info(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64), ("k_attn", ctypes.c_int64),
        ("n_ranks", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("k_rank", ctypes.c_int64 * 2), ("path", ctypes.c_int32 * 2),
        ("splits", ctypes.c_int32 * 2),
        ("chunk_elems", ctypes.c_int64), ("wire_bytes_bf16", ctypes.c_int64),
        ("wire_bytes_fp32", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("ep", ctypes.c_int32),
        ("local_experts", ctypes.c_int32), ("moe_inter", ctypes.c_int64),
        ("max_tokens", ctypes.c_int32), ("packed_kind", ctypes.c_int32),
        ("stream_wgs", ctypes.c_int32), ("weight_format", ctypes.c_int32),
        ("acts_layout", ctypes.c_int32), ("packed_layer_bytes", ctypes.c_int64 * 2),
    ]


_LIB = None

EXPORTS = {
    # name: (restype, argtypes)
    "tp_plan": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                               ctypes.POINTER(ctypes.c_void_p)]),
    "tp_plan_set_attn_dim": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64]),
    "tp_plan_set_qkv_dim": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64]),
    "tp_plan_set_moe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]),
    "tp_plan_tune": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_char_p, ctypes.c_int64]),
    "tp_plan_set_weight_format": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    "tp_quantize_mx": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                       + [ctypes.c_void_p] * 4),
    "tp_pack_weights_mx": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                           + [ctypes.c_void_p] * 4),
    "tp_plan_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(tp_plan_info)]),
    "tp_plan_info_get": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(tp_plan_info)]),
    "tp_plan_destroy": (None, [ctypes.c_void_p]),
    "tp_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "tp_workspace_init": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tp_workspace_status": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.POINTER(ctypes.c_int32)]),
    "tp_rowparallel_partial": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p]),
    "tp_rowparallel_partials": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]
                                + [ctypes.c_void_p] * 7),
    "tp_gate_up_swiglu": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 6),
    "tp_qkv_proj": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 5),
    "tp_ring_reduce": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tp_decode_layers": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                         + [ctypes.c_void_p] * 8),
    "tp_decode_point": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                        + [ctypes.c_void_p] * 6),
    "tp_pack_weights": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "tp_pack_activations": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 5),
    "tp_decode_layers_packed": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                                + [ctypes.c_void_p] * 8),
    "tp_rowparallel_partials_packed": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]
                                       + [ctypes.c_void_p] * 7),
    "tp_decode_layers_packed_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                                        + [ctypes.c_void_p] * 7),
    "tp_moe_route": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]),
    "tp_moe_pack_experts": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "tp_moe_partial": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p]),
    "tp_moe_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 8),
    "tp_moe_pack_attn": (ctypes.c_int, [ctypes.c_void_p] * 4),
    "tp_moe_layer_decode": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32]
                            + [ctypes.c_void_p] * 11),
    "tp_prefill_pack_weights": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
                                + [ctypes.c_void_p] * 3),
    "tp_prefill_layers": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
                          + [ctypes.c_void_p] * 8),
    "tp_stream_read_probe": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_int32, ctypes.c_void_p]),
    "tp_set_debug_sync": (ctypes.c_int, [ctypes.c_int32]),
}


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libtpdecode.so is not built (%s); run `python -m row_gemv_reduction_amd.build` "
                "or __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status, where):
    if status != TP_OK:
        raise TPError(status, where)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    return ctypes.c_void_p(t.data_ptr())


class Plan:
    """Owns a tp_plan_t. Sizes follow tp_plan(); optional k_attn, MoE share
    and tuning knobs are applied before first use."""

    def __init__(self, hidden, inter, n_ranks, batch, k_attn=None, moe=None, tune=None,
                 qkv_cols=None, weight_format=TP_WEIGHTS_BF16):
        h = ctypes.c_void_p()
        _check(_lib().tp_plan(hidden, inter, n_ranks, batch, ctypes.byref(h)), "tp_plan")
        self._h = h
        self._info = None  # tp_plan_info, read once per state of the plan
        self.qkv_cols = qkv_cols  # the rank's Q, K and V columns (tp_plan_set_qkv_dim)
        try:
            if qkv_cols is not None:
                _check(_lib().tp_plan_set_qkv_dim(h, qkv_cols), "tp_plan_set_qkv_dim")
            if k_attn is not None:
                _check(_lib().tp_plan_set_attn_dim(h, k_attn), "tp_plan_set_attn_dim")
            if weight_format != TP_WEIGHTS_BF16:
                _check(_lib().tp_plan_set_weight_format(h, weight_format), "tp_plan_set_weight_format")
            if moe is not None:
                _check(_lib().tp_plan_set_moe(h, moe["n_experts"], moe["top_k"], moe["ep"],
                                              moe["moe_inter"], moe["max_tokens"]),
                       "tp_plan_set_moe")
            for k, v in (tune or {}).items():
                _check(_lib().tp_plan_tune(h, k.encode(), int(v)), "tp_plan_tune(%s)" % k)
        except Exception:
            self.close()
            raise

    def tune(self, key, value):
        """Set a tuning knob (tp_plan_tune)."""
        self._info = None
        _check(_lib().tp_plan_tune(self.handle, key.encode(), int(value)), "tp_plan_tune(%s)" % key)

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("plan is closed")
        return self._h

    def info(self) -> dict:
        """tp_plan_info as a dict (a copy the caller may change)."""
        return {k: (list(v) if isinstance(v, list) else v) for k, v in self._plan_info().items()}

    def _plan_info(self) -> dict:
        # The binding's calls read the plan's info on every call; it only
        # changes with tune(), so it is fetched once per state.
        if self._info is None:
            i = tp_plan_info()
            _check(_lib().tp_plan_info(self.handle, ctypes.byref(i)), "tp_plan_info")
            d = {}
            for name, _ in tp_plan_info._fields_:
                v = getattr(i, name)
                d[name] = list(v) if hasattr(v, "__len__") else v
            self._info = d
        return self._info

    def new_workspace(self, device="cuda"):
        """Allocate (torch) and prepare a workspace for this plan."""
        nbytes = max(self._plan_info()["workspace_bytes"], 256)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        tp_workspace_init(self, ws)
        return ws

    def close(self):
        if getattr(self, "_h", None) is not None and _LIB is not None:
            _LIB.tp_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tp_plan(hidden, inter, n_ranks, batch, **kw) -> Plan:
    return Plan(hidden, inter, n_ranks, batch, **kw)


def tp_workspace_init(plan: Plan, workspace):
    _check(_lib().tp_workspace_init(plan.handle, _dev(workspace, "workspace", torch.uint8),
                                    _stream()), "tp_workspace_init")


def tp_workspace_status(plan: Plan, workspace) -> int:
    """The workspace's error word; workspace=None reads that of the no-alloc
    entry point's scratch on the current device."""
    flags = ctypes.c_int32(0)
    ws = None if workspace is None else _dev(workspace, "workspace", torch.uint8)
    _check(_lib().tp_workspace_status(plan.handle, ws, ctypes.byref(flags)), "tp_workspace_status")
    return flags.value


def tp_rowparallel_partial(plan: Plan, point, x, w, p, workspace):
    i = plan._plan_info()
    b, H, kr = i["batch"], i["hidden"], i["k_rank"][point] if point in (0, 1) else -1
    if point not in (0, 1):
        raise ValueError("point must be 0 (attention out) or 1 (FFN down)")
    args = (_dev(x, "x", torch.bfloat16, (b, kr)), _dev(w, "w", torch.bfloat16, (kr, H)),
            _dev(p, "p", torch.float32, (b, H)), _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_rowparallel_partial(plan.handle, point, *args, _stream()),
           "tp_rowparallel_partial")


def tp_rowparallel_partials(plan: Plan, n_layers, x_attn, w_o, x_ffn, w_down, p, workspace):
    """The 2L partials of a layer stack in one call: p [L][2][batch][hidden]."""
    i = plan._plan_info()
    b, H = i["batch"], i["hidden"]
    ka, ki = i["k_rank"]
    L = n_layers
    args = (_dev(x_attn, "x_attn", torch.bfloat16, (L, b, ka)),
            _dev(w_o, "w_o", torch.bfloat16, (L, ka, H)),
            _dev(x_ffn, "x_ffn", torch.bfloat16, (L, b, ki)),
            _dev(w_down, "w_down", torch.bfloat16, (L, ki, H)),
            _dev(p, "p", torch.float32, (L, 2, b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_rowparallel_partials(plan.handle, L, *args, _stream()),
           "tp_rowparallel_partials")


def tp_gate_up_swiglu(plan: Plan, n_layers, x, w_gate, w_up, out, workspace):
    """out[l] = bf16(silu(x[l] . w_gate[l]) * (x[l] . w_up[l])), the rank's columns."""
    i = plan._plan_info()
    b, H, n = i["batch"], i["hidden"], i["n_ranks"]
    C = i["inter"] // n
    L = n_layers
    args = (_dev(x, "x", torch.bfloat16, (L, b, H)),
            _dev(w_gate, "w_gate", torch.bfloat16, (L, H, C)),
            _dev(w_up, "w_up", torch.bfloat16, (L, H, C)),
            _dev(out, "out", torch.bfloat16, (L, b, C)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_gate_up_swiglu(plan.handle, L, *args, _stream()), "tp_gate_up_swiglu")


def tp_qkv_proj(plan: Plan, n_layers, x, w_qkv, out, workspace):
    """out[l] = bf16(x[l] . w_qkv[l]), the rank's Q, K and V columns."""
    if plan.qkv_cols is None:
        raise ValueError("the plan has no QKV width (Plan(..., qkv_cols=...))")
    i = plan._plan_info()
    b, H, C = i["batch"], i["hidden"], plan.qkv_cols
    L = n_layers
    args = (_dev(x, "x", torch.bfloat16, (L, b, H)),
            _dev(w_qkv, "w_qkv", torch.bfloat16, (L, H, C)),
            _dev(out, "out", torch.bfloat16, (L, b, C)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_qkv_proj(plan.handle, L, *args, _stream()), "tp_qkv_proj")


def tp_ring_reduce(plan: Plan, partials, residual, out, out_bf16=None):
    i = plan._plan_info()
    n, b, H = i["n_ranks"], i["batch"], i["hidden"]
    ob = None if out_bf16 is None else _dev(out_bf16, "out_bf16", torch.bfloat16, (b, H))
    _check(_lib().tp_ring_reduce(plan.handle, _dev(partials, "partials", torch.float32, (n, b, H)),
                                 _dev(residual, "residual", torch.float32, (b, H)),
                                 _dev(out, "out", torch.float32, (b, H)), ob, _stream()),
           "tp_ring_reduce")


def tp_decode_layers(plan: Plan, n_layers, rank, x_attn, w_o, x_ffn, w_down, slots, hidden,
                     workspace):
    i = plan._plan_info()
    n, b, H = i["n_ranks"], i["batch"], i["hidden"]
    ka, ki = i["k_rank"]
    L = n_layers
    args = (_dev(x_attn, "x_attn", torch.bfloat16, (L, b, ka)),
            _dev(w_o, "w_o", torch.bfloat16, (L, ka, H)),
            _dev(x_ffn, "x_ffn", torch.bfloat16, (L, b, ki)),
            _dev(w_down, "w_down", torch.bfloat16, (L, ki, H)),
            _dev(slots, "slots", torch.float32, (L, 2, n, b, H)),
            _dev(hidden, "hidden", torch.float32, (b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_decode_layers(plan.handle, L, rank, *args, _stream()), "tp_decode_layers")


def tp_decode_point(plan: Plan, point, rank, x, w, slots, hidden, workspace):
    """One reconciliation point: partial into slots[rank], then hidden <- ring_sum(slots) + hidden."""
    i = plan._plan_info()
    if point not in (0, 1):
        raise ValueError("point must be 0 (attention out) or 1 (FFN down)")
    n, b, H, kr = i["n_ranks"], i["batch"], i["hidden"], i["k_rank"][point]
    args = (_dev(x, "x", torch.bfloat16, (b, kr)), _dev(w, "w", torch.bfloat16, (kr, H)),
            _dev(slots, "slots", torch.float32, (n, b, H)), _dev(hidden, "hidden", torch.float32, (b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_decode_point(plan.handle, point, rank, *args, _stream()), "tp_decode_point")


def packed_dtype(plan: Plan):
    """bf16 for bf16 weights; uint8 bytes for MX weights."""
    return torch.bfloat16 if plan._plan_info()["weight_format"] == TP_WEIGHTS_BF16 else torch.uint8


def packed_shape(plan: Plan, point, n_layers):
    """Shape of a packed weight stack for the plan's streamed step:
    pair strips [L, H/4, ceil(K_r/2), 8] or MFMA tiles [L, H/16, ceil(K_r/64), 2, 64, 8]
    (bf16); for MX weights the stack's bytes [L * packed_layer_bytes] (uint8)."""
    if point not in (0, 1):
        raise ValueError("point must be 0 or 1")
    i = plan._plan_info()
    kr, H = i["k_rank"][point], i["hidden"]
    if i["packed_kind"] in (1, 2) and i["weight_format"] != TP_WEIGHTS_BF16:
        return (n_layers * i["packed_layer_bytes"][point],)
    if i["packed_kind"] == 1:
        return (n_layers, H // 4, (kr + 1) // 2, 8)
    if i["packed_kind"] == 2:
        return (n_layers, H // 16, (kr + 63) // 64, 2, 64, 8)
    raise TPError(TP_ERR_UNSUPPORTED, "packed_shape")


def packed_act_shape(plan: Plan, point, n_layers):
    """Shape of a step's activation slices as tp_decode_layers_packed reads them:
    row-major [L, b, K_r] (info acts_layout 0) or the matrix-core stream's
    A-operand order [L, ceil(K_r/64), ceil(b/16), 2, 64, 8] (acts_layout 1)."""
    if point not in (0, 1):
        raise ValueError("point must be 0 or 1")
    i = plan._plan_info()
    kr, b = i["k_rank"][point], i["batch"]
    if i["packed_kind"] == 1 or (i["packed_kind"] == 2 and i["acts_layout"] == 0):
        return (n_layers, b, kr)
    if i["packed_kind"] == 2:
        return (n_layers, (kr + 63) // 64, (b + 15) // 16, 2, 64, 8)
    raise TPError(TP_ERR_UNSUPPORTED, "packed_act_shape")


def tp_pack_activations(plan: Plan, x_attn, x_ffn, xa_packed, xf_packed):
    """Lay a step's activation slices [L, b, K_r] out as packed_act_shape() (tp_pack_activations)."""
    i = plan._plan_info()
    b = i["batch"]
    ka, ki = i["k_rank"]
    L = x_attn.shape[0]
    _check(_lib().tp_pack_activations(plan.handle, L, _dev(x_attn, "x_attn", torch.bfloat16, (L, b, ka)),
                                      _dev(x_ffn, "x_ffn", torch.bfloat16, (L, b, ki)),
                                      _dev(xa_packed, "xa_packed", torch.bfloat16, packed_act_shape(plan, 0, L)),
                                      _dev(xf_packed, "xf_packed", torch.bfloat16, packed_act_shape(plan, 1, L)),
                                      _stream()), "tp_pack_activations")


def mx_codes_shape(plan: Plan, point, n_layers):
    """Interchange layout of a point's MX codes: [L, K_r, H] (MXFP8) or [L, K_r/2, H] (MXFP4)."""
    i = plan._plan_info()
    kr, H = i["k_rank"][point], i["hidden"]
    return (n_layers, kr if i["weight_format"] == TP_WEIGHTS_MXFP8 else kr // 2, H)


def mx_scales_shape(plan: Plan, point, n_layers):
    i = plan._plan_info()
    return (n_layers, i["k_rank"][point] // MX_BLOCK, i["hidden"])


def tp_quantize_mx(plan: Plan, point, w, codes, scales):
    """bf16 weights [L, K_r, H] -> MX codes and scales (the plan's format)."""
    if point not in (0, 1):
        raise ValueError("point must be 0 or 1")
    L = w.shape[0]
    i = plan._plan_info()
    _check(_lib().tp_quantize_mx(plan.handle, point, L,
                                 _dev(w, "w", torch.bfloat16, (L, i["k_rank"][point], i["hidden"])),
                                 _dev(codes, "codes", torch.uint8, mx_codes_shape(plan, point, L)),
                                 _dev(scales, "scales", torch.uint8, mx_scales_shape(plan, point, L)),
                                 _stream()), "tp_quantize_mx")


def tp_pack_weights_mx(plan: Plan, point, codes, scales, w_packed):
    """MX codes and scales of a stack -> the packed step's layout (packed_shape, uint8)."""
    if point not in (0, 1):
        raise ValueError("point must be 0 or 1")
    L = codes.shape[0]
    _check(_lib().tp_pack_weights_mx(plan.handle, point, L,
                                     _dev(codes, "codes", torch.uint8, mx_codes_shape(plan, point, L)),
                                     _dev(scales, "scales", torch.uint8, mx_scales_shape(plan, point, L)),
                                     _dev(w_packed, "w_packed", torch.uint8, packed_shape(plan, point, L)),
                                     _stream()), "tp_pack_weights_mx")


def tp_pack_weights(plan: Plan, point, w, w_packed):
    """Pack a stack of row-major weight slices [L, K_r, H] -> packed_shape()."""
    L = w.shape[0]
    shape = packed_shape(plan, point, L)
    kr, H = plan._plan_info()["k_rank"][point], plan._plan_info()["hidden"]
    _check(_lib().tp_pack_weights(plan.handle, point, L, _dev(w, "w", torch.bfloat16, (L, kr, H)),
                                  _dev(w_packed, "w_packed", packed_dtype(plan), shape),
                                  _stream()), "tp_pack_weights")


def tp_decode_layers_packed(plan: Plan, n_layers, rank, x_attn, w_o_packed, x_ffn, w_down_packed,
                            slots, hidden, workspace):
    """The streamed decode step; x_attn / x_ffn as tp_pack_activations lays them out."""
    i = plan._plan_info()
    n, b, H = i["n_ranks"], i["batch"], i["hidden"]
    ka, ki = i["k_rank"]
    L = n_layers
    args = (_dev(x_attn, "x_attn", torch.bfloat16, packed_act_shape(plan, 0, L)),
            _dev(w_o_packed, "w_o_packed", packed_dtype(plan), packed_shape(plan, 0, L)),
            _dev(x_ffn, "x_ffn", torch.bfloat16, packed_act_shape(plan, 1, L)),
            _dev(w_down_packed, "w_down_packed", packed_dtype(plan), packed_shape(plan, 1, L)),
            _dev(slots, "slots", torch.float32, (L, 2, n, b, H)),
            _dev(hidden, "hidden", torch.float32, (b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_decode_layers_packed(plan.handle, L, rank, *args, _stream()),
           "tp_decode_layers_packed")


def tp_decode_layers_packed_noalloc(plan: Plan, n_layers, rank, x_attn, w_o_packed, x_ffn,
                                    w_down_packed, slots, hidden):
    """tp_decode_layers_packed with the library's per-GPU scratch instead of a workspace."""
    i = plan._plan_info()
    n, b, H = i["n_ranks"], i["batch"], i["hidden"]
    L = n_layers
    args = (_dev(x_attn, "x_attn", torch.bfloat16, packed_act_shape(plan, 0, L)),
            _dev(w_o_packed, "w_o_packed", packed_dtype(plan), packed_shape(plan, 0, L)),
            _dev(x_ffn, "x_ffn", torch.bfloat16, packed_act_shape(plan, 1, L)),
            _dev(w_down_packed, "w_down_packed", packed_dtype(plan), packed_shape(plan, 1, L)),
            _dev(slots, "slots", torch.float32, (L, 2, n, b, H)),
            _dev(hidden, "hidden", torch.float32, (b, H)))
    _check(_lib().tp_decode_layers_packed_noalloc(plan.handle, L, rank, *args, _stream()),
           "tp_decode_layers_packed_noalloc")


def tp_rowparallel_partials_packed(plan: Plan, n_layers, x_attn, w_o_packed, x_ffn, w_down_packed,
                                   p, workspace):
    """The 2L partials of a stack on packed weights in one call (packed_kind 1):
    p [L][2][batch][hidden]."""
    i = plan._plan_info()
    b, H = i["batch"], i["hidden"]
    L = n_layers
    args = (_dev(x_attn, "x_attn", torch.bfloat16, packed_act_shape(plan, 0, L)),
            _dev(w_o_packed, "w_o_packed", packed_dtype(plan), packed_shape(plan, 0, L)),
            _dev(x_ffn, "x_ffn", torch.bfloat16, packed_act_shape(plan, 1, L)),
            _dev(w_down_packed, "w_down_packed", packed_dtype(plan), packed_shape(plan, 1, L)),
            _dev(p, "p", torch.float32, (L, 2, b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_rowparallel_partials_packed(plan.handle, L, *args, _stream()),
           "tp_rowparallel_partials_packed")


def tp_moe_route(plan: Plan, logits, sel_expert, sel_weight, renorm=True):
    i = plan._plan_info()
    t = logits.shape[0]
    k, e = i["top_k"], i["n_experts"]
    _check(_lib().tp_moe_route(plan.handle, _dev(logits, "logits", torch.float32, (t, e)), t,
                               1 if renorm else 0,
                               _dev(sel_expert, "sel_expert", torch.int32, (t, k)),
                               _dev(sel_weight, "sel_weight", torch.float32, (t, k)), _stream()),
           "tp_moe_route")


def moe_packed_shape(plan: Plan):
    """Shape of a rank's packed experts: [E/ep, H/16, ceil(moe_inter/64), 1024]
    (2 KB matrix-core tiles of 64 rows x 16 columns)."""
    i = plan._plan_info()
    return (i["local_experts"], i["hidden"] // 16, (i["moe_inter"] + 63) // 64, 1024)


def tp_moe_pack_experts(plan: Plan, w_local, w_packed):
    i = plan._plan_info()
    le, mi, H = i["local_experts"], i["moe_inter"], i["hidden"]
    _check(_lib().tp_moe_pack_experts(plan.handle, _dev(w_local, "w_local", torch.bfloat16, (le, mi, H)),
                                      _dev(w_packed, "w_packed", torch.bfloat16, moe_packed_shape(plan)),
                                      _stream()), "tp_moe_pack_experts")


def tp_moe_partial(plan: Plan, rank, sel_expert, sel_weight, u, w_packed, part, workspace):
    i = plan._plan_info()
    t = sel_expert.shape[0]
    k, mi, H = i["top_k"], i["moe_inter"], i["hidden"]
    args = (_dev(sel_expert, "sel_expert", torch.int32, (t, k)),
            _dev(sel_weight, "sel_weight", torch.float32, (t, k)))
    rest = (_dev(u, "u", torch.bfloat16, (t, k, mi)),
            _dev(w_packed, "w_packed", torch.bfloat16, moe_packed_shape(plan)),
            _dev(part, "part", torch.float32, (t, H)), _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_moe_partial(plan.handle, rank, *args, t, *rest, _stream()), "tp_moe_partial")


def tp_moe_decode(plan: Plan, rank, sel_expert, sel_weight, u, w_packed, slots, hidden, workspace):
    """The MoE point: the rank's experts for the plan's batch, the combine into slots[rank], then
    hidden <- ring_sum(slots) + hidden."""
    i = plan._plan_info()
    n, b, k, mi, H = i["n_ranks"], i["batch"], i["top_k"], i["moe_inter"], i["hidden"]
    args = (_dev(sel_expert, "sel_expert", torch.int32, (b, k)),
            _dev(sel_weight, "sel_weight", torch.float32, (b, k)),
            _dev(u, "u", torch.bfloat16, (b, k, mi)),
            _dev(w_packed, "w_packed", torch.bfloat16, moe_packed_shape(plan)),
            _dev(slots, "slots", torch.float32, (n, b, H)), _dev(hidden, "hidden", torch.float32, (b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_moe_decode(plan.handle, rank, *args, _stream()), "tp_moe_decode")


def moe_attn_packed_shape(plan: Plan):
    """Shape of a rank's attention slice packed by tp_moe_pack_attn:
    [H/16, ceil(k_attn/N / 64), 1024] (bf16)."""
    i = plan._plan_info()
    return (i["hidden"] // 16, (i["k_attn"] // i["n_ranks"] + 63) // 64, 1024)


def tp_moe_pack_attn(plan: Plan, w, w_packed):
    i = plan._plan_info()
    ka = i["k_attn"] // i["n_ranks"]
    _check(_lib().tp_moe_pack_attn(plan.handle, _dev(w, "w", torch.bfloat16, (ka, i["hidden"])),
                                   _dev(w_packed, "w_packed", torch.bfloat16, moe_attn_packed_shape(plan)),
                                   _stream()), "tp_moe_pack_attn")


def tp_moe_layer_decode(plan: Plan, rank, logits, x_attn, w_attn_packed, u, w_packed, sel_expert,
                        sel_weight, slots_attn, slots_moe, hidden, workspace, renorm=True):
    """One MoE layer's decode share: routing, the attention slice's partial into
    slots_attn[rank] and its ring sum into hidden, the rank's experts into
    slots_moe[rank] and their ring sum into hidden."""
    i = plan._plan_info()
    n, b, k, mi, H = i["n_ranks"], i["batch"], i["top_k"], i["moe_inter"], i["hidden"]
    ka = i["k_attn"] // n
    lg = _dev(logits, "logits", torch.float32, (b, i["n_experts"]))
    args = (_dev(x_attn, "x_attn", torch.bfloat16, (b, ka)),
            _dev(w_attn_packed, "w_attn_packed", torch.bfloat16, moe_attn_packed_shape(plan)),
            _dev(u, "u", torch.bfloat16, (b, k, mi)),
            _dev(w_packed, "w_packed", torch.bfloat16, moe_packed_shape(plan)),
            _dev(sel_expert, "sel_expert", torch.int32, (b, k)),
            _dev(sel_weight, "sel_weight", torch.float32, (b, k)),
            _dev(slots_attn, "slots_attn", torch.float32, (n, b, H)),
            _dev(slots_moe, "slots_moe", torch.float32, (n, b, H)),
            _dev(hidden, "hidden", torch.float32, (b, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_moe_layer_decode(plan.handle, rank, lg, 1 if renorm else 0, *args, _stream()),
           "tp_moe_layer_decode")


def tp_set_debug_sync(on) -> None:
    """Debug mode, process-wide: each entry point waits for its stream after
    every kernel launch and raises from the call whose kernel failed (not
    while the stream is captured into a graph). `on` is 0/1 or a bool."""
    _check(_lib().tp_set_debug_sync(int(on)), "tp_set_debug_sync")


def tp_stream_read_probe(buf, sink):
    """Read all of `buf` (any dtype, contiguous, on the GPU) with the library's
    streaming-read probe; `sink` is a uint32 tensor with one word per
    workgroup (its length is the workgroup count)."""
    if not isinstance(buf, torch.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    _check(_lib().tp_stream_read_probe(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                       _dev(sink, "sink", torch.uint32), sink.numel(), _stream()),
           "tp_stream_read_probe")


def prefill_packed_shape(plan: Plan, point, n_layers):
    """Shape of a point's weight stack packed for tp_prefill_layers:
    [L, H/16, ceil(K_r/64), 2, 64, 8] (bf16)."""
    i = plan._plan_info()
    return (n_layers, i["hidden"] // 16, (i["k_rank"][point] + 63) // 64, 2, 64, 8)


def tp_prefill_pack_weights(plan: Plan, point, w, w_packed):
    if point not in (0, 1):
        raise ValueError("point must be 0 or 1")
    i = plan._plan_info()
    L = w.shape[0]
    _check(_lib().tp_prefill_pack_weights(
        plan.handle, point, L, _dev(w, "w", torch.bfloat16, (L, i["k_rank"][point], i["hidden"])),
        _dev(w_packed, "w_packed", torch.bfloat16, prefill_packed_shape(plan, point, L)), _stream()),
        "tp_prefill_pack_weights")


def tp_prefill_layers(plan: Plan, n_layers, rank, tokens, x_attn, w_o_packed, x_ffn, w_down_packed,
                      slots, hidden, workspace):
    """The prefill of `tokens` tokens: per point the rank's partial into its slot, then
    hidden <- ring_sum(slots) + hidden."""
    i = plan._plan_info()
    n, H = i["n_ranks"], i["hidden"]
    ka, ki = i["k_rank"]
    L, T = n_layers, tokens
    args = (_dev(x_attn, "x_attn", torch.bfloat16, (L, T, ka)),
            _dev(w_o_packed, "w_o_packed", torch.bfloat16, prefill_packed_shape(plan, 0, L)),
            _dev(x_ffn, "x_ffn", torch.bfloat16, (L, T, ki)),
            _dev(w_down_packed, "w_down_packed", torch.bfloat16, prefill_packed_shape(plan, 1, L)),
            _dev(slots, "slots", torch.float32, (L, 2, n, T, H)),
            _dev(hidden, "hidden", torch.float32, (T, H)),
            _dev(workspace, "workspace", torch.uint8))
    if workspace.numel() < i["workspace_bytes"]:
        raise ValueError("workspace too small")
    _check(_lib().tp_prefill_layers(plan.handle, L, rank, T, *args, _stream()), "tp_prefill_layers")
