"""ctypes binding of the C ABI in include/moe.h (argument marshalling only).

Each function has the name and argument order of the C entry point, takes
torch tensors (device memory) where the C call takes device pointers, and
raises MoEError on a non-zero status.  Every step of the layer runs in the
HIP library; nothing here computes.  The library must be built
(router_gemm_amd.build): there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

from .build import LIB, LIB_SAN

# MOE_SANITIZED_HOST=1: load the build whose host code carries AddressSanitizer
# and UBSan (CPU tests of the argument validation only; tests/run_sanitized.py)
if os.environ.get("MOE_SANITIZED_HOST", "") == "1":
    LIB = LIB_SAN

MOE_BF16 = 1
MOE_FP8_E4M3FN = 2
MOE_F32 = 3
MOE_MXFP4_E2M1 = 4

EXPERT_DTYPE = {"bf16": MOE_BF16, "fp8": MOE_FP8_E4M3FN, "mxfp4": MOE_MXFP4_E2M1}

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = range(5)
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILE16 = 0, 1

_DT = {torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}


class MoEError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"status {status}: {detail}")
        self.status = status
        self.detail = detail


class MoELayerC(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("num_experts", C.c_int32),
                ("top_k", C.c_int32), ("shared_inter", C.c_int32), ("expert_dtype", C.c_int32),
                ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("w_gate_up", C.c_void_p), ("s_gate_up", C.c_void_p),
                ("w_down", C.c_void_p), ("s_down", C.c_void_p),
                ("w_shared_gate_up", C.c_void_p), ("w_shared_down", C.c_void_p),
                ("weight_layout", C.c_int32)]


EXPORTS = ["moe_workspace_bytes", "moe_route", "moe_permute", "moe_expert_ffn", "moe_combine",
           "moe_forward", "moe_forward_routed", "moe_forward_noalloc", "moe_saved_z_floats", "moe_forward_train", "moe_backward_workspace_bytes",
           "moe_backward", "moe_pack_weights", "moe_status_string",
           "moe_last_error", "moe_timing_arm", "moe_timing_read"]

_lib = None


def lib() -> C.CDLL:
    """Load the in-tree HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is missing: build it with router_gemm_amd.build.build()")
        L = C.CDLL(LIB)
        vp, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [vp, i64, i64]
        L.moe_route.restype = C.c_int
        L.moe_route.argtypes = [vp, vp, i64, vp, vp, vp, vp, sz, vp]
        L.moe_permute.restype = C.c_int
        L.moe_permute.argtypes = [vp, vp, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_ffn.restype = C.c_int
        L.moe_expert_ffn.argtypes = [vp, vp, vp, vp, i64, vp, i32, vp, sz, vp]
        L.moe_combine.restype = C.c_int
        L.moe_combine.argtypes = [vp, vp, i32, vp, vp, vp, i64, vp, i32, i64, vp, i32, vp, sz, vp]
        L.moe_forward.restype = C.c_int
        L.moe_forward.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp, sz, vp]
        L.moe_forward_routed.restype = C.c_int
        L.moe_forward_routed.argtypes = [vp, vp, i64, vp, vp, vp, i64, vp, i32, vp, sz, vp]
        L.moe_forward_noalloc.restype = C.c_int
        L.moe_forward_noalloc.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp]
        L.moe_backward_workspace_bytes.restype = sz
        L.moe_backward_workspace_bytes.argtypes = [vp, i64]
        L.moe_backward.restype = C.c_int
        L.moe_backward.argtypes = [vp, vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_saved_z_floats.restype = sz
        L.moe_saved_z_floats.argtypes = [vp, i64]
        L.moe_forward_train.restype = C.c_int
        L.moe_forward_train.argtypes = [vp, vp, i64, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_pack_weights.restype = C.c_int
        L.moe_pack_weights.argtypes = [vp, vp, i64, i64, i64, vp]
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [C.c_int]
        L.moe_last_error.restype = C.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_timing_arm.restype = C.c_int
        L.moe_timing_arm.argtypes = [i32, i32]
        L.moe_timing_read.restype = C.c_int
        L.moe_timing_read.argtypes = [i32, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(status: int):
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error().decode())


def dtype_code(t: torch.Tensor) -> int:
    return _DT[t.dtype]


class Layer:
    """Holds a moe_layer struct and keeps its tensors alive."""

    def __init__(self, hidden, inter, num_experts, top_k, expert_dtype, w_gate_up, w_down,
                 s_gate_up=None, s_down=None, w_router=None, router_bias=None,
                 w_shared_gate_up=None, w_shared_down=None, shared_inter=0, weight_layout=MOE_LAYOUT_ROWS):
        self.tensors = [w_gate_up, w_down, s_gate_up, s_down, w_router, router_bias,
                        w_shared_gate_up, w_shared_down]
        self.c = MoELayerC(hidden, inter, num_experts, top_k, shared_inter, expert_dtype,
                           _ptr(w_router), _ptr(router_bias), _ptr(w_gate_up), _ptr(s_gate_up),
                           _ptr(w_down), _ptr(s_down), _ptr(w_shared_gate_up), _ptr(w_shared_down),
                           weight_layout)

    @property
    def ref(self):
        return C.byref(self.c)

    @classmethod
    def from_tensors(cls, lt, top_k: Optional[int] = None) -> "Layer":
        """Routed layer from workloads.LayerTensors."""
        cfg = lt.cfg
        return cls(cfg.H, cfg.I, cfg.E, cfg.k if top_k is None else top_k,
                   EXPERT_DTYPE[cfg.expert_dtype], lt.w_gate_up, lt.w_down,
                   lt.s_gate_up, lt.s_down, lt.w_router, lt.router_bias,
                   lt.w_shared_gate_up, lt.w_shared_down, cfg.Is if lt.w_shared_gate_up is not None else 0)

    def packed(self, stream=None) -> "Layer":
        """The same layer with the routed experts' weights repacked into
        MOE_LAYOUT_TILE16 (new device tensors; this layer is unchanged)."""
        c = self.c
        wgu, wd = self.tensors[0], self.tensors[1]
        esz = 1 if c.expert_dtype == MOE_FP8_E4M3FN else 2
        pgu = pack_weights(wgu, c.num_experts, 2 * c.inter, c.hidden * esz, stream)
        pd = pack_weights(wd, c.num_experts, c.hidden, c.inter * esz, stream)
        t = self.tensors
        return Layer(c.hidden, c.inter, c.num_experts, c.top_k, c.expert_dtype, pgu, pd, t[2], t[3], t[4], t[5],
                     t[6], t[7], c.shared_inter, MOE_LAYOUT_TILE16)

    def with_router_bias(self, router_bias: Optional[torch.Tensor]) -> "Layer":
        """The same layer (same weight tensors and layout) with another router bias."""
        c, t = self.c, self.tensors
        return Layer(c.hidden, c.inter, c.num_experts, c.top_k, c.expert_dtype, t[0], t[1], t[2], t[3], t[4],
                     router_bias, t[6], t[7], c.shared_inter, c.weight_layout)

    @classmethod
    def shared_view(cls, lt) -> "Layer":
        """The shared expert as a one-expert bf16 layer (for moe_expert_ffn)."""
        cfg = lt.cfg
        return cls(cfg.H, cfg.Is, 1, 1, MOE_BF16, lt.w_shared_gate_up, lt.w_shared_down)


def moe_workspace_bytes(layer: Layer, T: int, N: int) -> int:
    return int(lib().moe_workspace_bytes(layer.ref, T, N))


def workspace(layer: Layer, T: int, N: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_workspace_bytes(layer, T, N), 256), dtype=torch.uint8, device=device)


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def moe_route(layer: Layer, x, T, topk_ids, topk_gates, logits=None, ws=None, stream=None):
    w, nb = _ws(ws)
    _check(lib().moe_route(layer.ref, _ptr(x), T, _ptr(topk_ids), _ptr(topk_gates), _ptr(logits),
                           w, nb, _stream(stream)))


def moe_permute(layer: Layer, x, T, assign_expert, assign_token, N, expert_offsets, perm_src,
                perm_pos, x_perm, x_scale=None, ws=None, stream=None):
    w, nb = _ws(ws)
    _check(lib().moe_permute(layer.ref, _ptr(x), T, _ptr(assign_expert), _ptr(assign_token), N,
                             _ptr(expert_offsets), _ptr(perm_src), _ptr(perm_pos), _ptr(x_perm),
                             _ptr(x_scale), w, nb, _stream(stream)))


def moe_expert_ffn(layer: Layer, expert_offsets, x_perm, x_scale, N, y_perm, y_dtype=None,
                   ws=None, stream=None):
    w, nb = _ws(ws)
    yd = dtype_code(y_perm) if y_dtype is None else y_dtype
    _check(lib().moe_expert_ffn(layer.ref, _ptr(expert_offsets), _ptr(x_perm), _ptr(x_scale), N,
                                _ptr(y_perm), yd, w, nb, _stream(stream)))


def moe_combine(layer: Layer, y_perm, y_dtype, perm_pos, assign_token, gates, N, shared_out,
                shared_dtype, T, y, out_dtype, ws=None, stream=None):
    w, nb = _ws(ws)
    _check(lib().moe_combine(layer.ref, _ptr(y_perm), y_dtype, _ptr(perm_pos), _ptr(assign_token),
                             _ptr(gates), N, _ptr(shared_out), shared_dtype, T, _ptr(y), out_dtype,
                             w, nb, _stream(stream)))


def moe_forward(layer: Layer, x, T, y, out_dtype=None, topk_ids=None, topk_gates=None, ws=None,
                stream=None):
    w, nb = _ws(ws)
    od = dtype_code(y) if out_dtype is None else out_dtype
    _check(lib().moe_forward(layer.ref, _ptr(x), T, _ptr(y), od, _ptr(topk_ids), _ptr(topk_gates),
                             w, nb, _stream(stream)))


def moe_forward_routed(layer: Layer, x, T, assign_expert, assign_token, gates, N, y, out_dtype=None, ws=None,
                       stream=None):
    w, nb = _ws(ws)
    od = dtype_code(y) if out_dtype is None else out_dtype
    _check(lib().moe_forward_routed(layer.ref, _ptr(x), T, _ptr(assign_expert), _ptr(assign_token), _ptr(gates), N,
                                    _ptr(y), od, w, nb, _stream(stream)))


def moe_forward_noalloc(layer: Layer, x, T, y, out_dtype=None, topk_ids=None, topk_gates=None, stream=None):
    od = dtype_code(y) if out_dtype is None else out_dtype
    _check(lib().moe_forward_noalloc(layer.ref, _ptr(x), T, _ptr(y), od, _ptr(topk_ids), _ptr(topk_gates),
                                     _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # include/moe.h


def moe_pack_weights(src, dst, count: int, rows: int, row_bytes: int, stream=None):
    _check(lib().moe_pack_weights(_ptr(src), _ptr(dst), count, rows, row_bytes, _stream(stream)))


def pack_weights(w: torch.Tensor, count: int, rows: int, row_bytes: int, stream=None) -> torch.Tensor:
    """A new tensor holding w (count row-major [rows, row_bytes]-byte
    matrices) in the MOE_LAYOUT_TILE16 layout (same dtype and shape as w)."""
    if w.numel() * w.element_size() != count * rows * row_bytes:
        raise ValueError("pack_weights: count * rows * row_bytes does not match the tensor")
    out = torch.empty_like(w)
    moe_pack_weights(w, out, count, rows, row_bytes, stream)
    return out


def moe_backward_workspace_bytes(layer: Layer, T: int) -> int:
    return int(lib().moe_backward_workspace_bytes(layer.ref, T))


def backward_workspace(layer: Layer, T: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(moe_backward_workspace_bytes(layer, T), 256), dtype=torch.uint8, device=device)


def moe_saved_z_floats(layer: Layer, T: int) -> int:
    return int(lib().moe_saved_z_floats(layer.ref, T))


def moe_forward_train(layer: Layer, x, T, y, topk_ids, topk_gates, z_saved, out_dtype=None, ws=None,
                      stream=None):
    w, nb = _ws(ws)
    od = dtype_code(y) if out_dtype is None else out_dtype
    _check(lib().moe_forward_train(layer.ref, _ptr(x), T, _ptr(y), od, _ptr(topk_ids), _ptr(topk_gates),
                                   _ptr(z_saved), w, nb, _stream(stream)))


def moe_backward(layer: Layer, x, T, topk_ids, topk_gates, dy, dx, dw_gate_up, dw_down,
                 dw_shared_gate_up, dw_shared_down, dw_router, dbias=None, z_saved=None, ws=None,
                 stream=None):
    w, nb = _ws(ws)
    _check(lib().moe_backward(layer.ref, _ptr(x), T, _ptr(topk_ids), _ptr(topk_gates), _ptr(dy),
                              _ptr(z_saved), _ptr(dx), _ptr(dw_gate_up), _ptr(dw_down), _ptr(dw_shared_gate_up),
                              _ptr(dw_shared_down), _ptr(dw_router), _ptr(dbias), w, nb,
                              _stream(stream)))


def timing_arm(site: int, capacity: int):
    _check(lib().moe_timing_arm(site, capacity))


def timing_read(site: int):
    """-> (total milliseconds, number of timed launches) for an armed site."""
    ms, n = C.c_double(0.0), C.c_int32(0)
    _check(lib().moe_timing_read(site, C.byref(ms), C.byref(n)))
    return ms.value, n.value
