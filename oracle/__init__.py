"""fp64 CPU oracle of the routed MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``router_gemm_amd``)
never imports it and shares no code with it.

This module is a thin ctypes wrapper over ``moe_oracle.c`` (plain C, fp64,
OpenMP over independent tokens).  Every array goes in and out as numpy.  The
definitions each function follows are stated in ``moe_oracle.h``:

  y[t] = Shared(x[t]) + sum_{e in TopK(t)} g[t,e] FFN_e(x[t]),
  FFN(a) = (silu(a Wg^T) * (a Wu^T)) Wd^T

("Step-5-Preview", NeMo AutoModel model coverage, section "Model
Architecture"; "Step-5 minimal inference", introduction: block-scaled FP8
expert GEMM).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "moe_oracle.c")
# MOE_ORACLE_SANITIZE=1 selects the AddressSanitizer + UBSan build (CPU tests
# only; the process must preload gcc's libasan, see tests/run_sanitized.py).
SANITIZE = os.environ.get("MOE_ORACLE_SANITIZE", "") == "1"
LIB_PATH = os.path.join(_HERE, "libmoe_oracle_san.so" if SANITIZE else "libmoe_oracle.so")

_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def build(sanitize: bool = SANITIZE) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction); with
    `sanitize`, the AddressSanitizer + UBSan build (-O1, aborts on the first
    report) next to the plain one."""
    out = os.path.join(_HERE, "libmoe_oracle_san.so" if sanitize else "libmoe_oracle.so")
    opt = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined"] if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-Wall", "-Wpointer-arith", SRC_PATH, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class _Layer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("num_experts", C.c_int32),
                ("top_k", C.c_int32), ("shared_inter", C.c_int32), ("expert_format", C.c_int32),
                ("w_router", C.c_void_p), ("router_bias", C.c_void_p),
                ("w_gate_up", C.c_void_p), ("s_gate_up", C.c_void_p),
                ("w_down", C.c_void_p), ("s_down", C.c_void_p),
                ("w_shared_gate_up", C.c_void_p), ("w_shared_down", C.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
        L.oref_bf16_decode.restype = C.c_double
        L.oref_bf16_decode.argtypes = [C.c_uint16]
        L.oref_bf16_encode.restype = C.c_uint16
        L.oref_bf16_encode.argtypes = [C.c_double]
        L.oref_e4m3_decode.restype = C.c_double
        L.oref_e4m3_decode.argtypes = [C.c_uint8]
        L.oref_e4m3_encode.restype = C.c_uint8
        L.oref_e4m3_encode.argtypes = [C.c_float]
        L.oref_e2m1_decode.restype = C.c_double
        L.oref_e2m1_decode.argtypes = [C.c_uint8]
        L.oref_e8m0_decode.restype = C.c_double
        L.oref_e8m0_decode.argtypes = [C.c_uint8]
        for name, args in {
            "oref_quant_row": [vp, i64, vp, vp],
            "oref_e4m3_encode_array": [vp, i64, vp],
            "oref_bf16_encode_array": [vp, i64, vp],
            "oref_quant_bf16_rows": [vp, i64, i64, vp, vp],
            "oref_route": [vp, vp, i64, vp, i64, vp, vp, vp, vp],
            "oref_gates_for_ids": [vp, vp, i64, vp, i64, vp, vp],
            "oref_expert_row": [vp, i32, vp, vp, vp, vp],
            "oref_expert_gate_up_factored": [vp, i32, vp, vp, vp, vp],
            "oref_expert_gate_up_dequant": [vp, i32, vp, vp, vp, vp],
            "oref_expert_gate_up_mx_factored": [vp, i32, vp, vp, vp, vp],
            "oref_shared_row": [vp, vp, vp],
            "oref_expert_ffn": [vp, vp, vp, vp, i64, vp],
            "oref_forward": [vp, vp, i64, vp, i64, vp, vp, vp, vp],
            "oref_forward_with_ids": [vp, vp, i64, vp, i64, vp, vp],
            "oref_forward_triples": [vp, vp, i64, vp, vp, vp, i64, vp, i64, vp],
            "oref_combine": [vp, vp, vp, i32, vp, i64, vp, i64, i64, vp],
            "oref_backward": [vp, vp, i64, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp],
        }.items():
            f = getattr(L, name)
            f.restype = None
            f.argtypes = args
        L.oref_permute.restype = C.c_int64
        L.oref_permute.argtypes = [vp, i64, i32, vp, vp, vp]
        L.oref_num_threads.restype = C.c_int
        L.oref_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


BF16, FP8, MXFP4 = 0, 1, 2
_FORMATS = {"bf16": BF16, "fp8": FP8, "mxfp4": MXFP4}


class Layer:
    """Host copy of one MoE layer for the oracle (numpy arrays).

    w_router uint16 (bf16 bits) [E,H]; router_bias float32 [E] or None;
    expert_format: "bf16" / "fp8" / "mxfp4" (or False / True / 2):
      bf16:  w_gate_up uint16 [E,2I,H], w_down uint16 [E,H,I];
      fp8:   w_gate_up uint8 (e4m3fn) [E,2I,H], w_down [E,H,I],
             s_gate_up float32 [E,2I/128,H/128], s_down float32 [E,H/128,I/128];
      mxfp4: w_gate_up uint8 [E,2I,H/2], w_down uint8 [E,H,I/2] (two E2M1
             codes per byte, even input in the low nibble),
             s_gate_up uint8 (E8M0) [E,2I,H/32], s_down uint8 [E,H,I/32];
    w_shared_gate_up uint16 [2Is,H], w_shared_down uint16 [H,Is] or None.
    """

    def __init__(self, hidden, inter, num_experts, top_k, expert_format, w_router, w_gate_up,
                 w_down, s_gate_up=None, s_down=None, router_bias=None,
                 w_shared_gate_up=None, w_shared_down=None, shared_inter=None):
        self.H, self.I, self.E, self.k = int(hidden), int(inter), int(num_experts), int(top_k)
        fmt = _FORMATS[expert_format] if isinstance(expert_format, str) else int(expert_format)
        assert fmt in (BF16, FP8, MXFP4)
        self.format = fmt
        self.mx = fmt == MXFP4
        self.fp8 = fmt != BF16          # activations and h stored as e4m3 + 1x128 scales
        wdt = np.uint16 if fmt == BF16 else np.uint8
        sdt = np.uint8 if self.mx else np.float32
        self.w_router = _c(w_router, np.uint16)
        self.router_bias = _c(router_bias, np.float32)
        self.w_gate_up = _c(w_gate_up, wdt)
        self.w_down = _c(w_down, wdt)
        self.s_gate_up = _c(s_gate_up, sdt)
        self.s_down = _c(s_down, sdt)
        self.w_shared_gate_up = _c(w_shared_gate_up, np.uint16)
        self.w_shared_down = _c(w_shared_down, np.uint16)
        if shared_inter is None:
            shared_inter = 0 if w_shared_gate_up is None else self.w_shared_gate_up.shape[0] // 2
        self.Is = int(shared_inter)
        if self.fp8:
            assert self.s_gate_up is not None and self.s_down is not None
            assert self.H % 128 == 0 and self.I % 128 == 0
        if self.mx:
            E, H, I = self.E, self.H, self.I
            assert self.w_gate_up.shape == (E, 2 * I, H // 2) and self.w_down.shape == (E, H, I // 2)
            assert self.s_gate_up.shape == (E, 2 * I, H // 32) and self.s_down.shape == (E, H, I // 32)
        self._s = _Layer(self.H, self.I, self.E, self.k, self.Is, fmt,
                         _p(self.w_router), _p(self.router_bias), _p(self.w_gate_up),
                         _p(self.s_gate_up), _p(self.w_down), _p(self.s_down),
                         _p(self.w_shared_gate_up), _p(self.w_shared_down))

    @property
    def ref(self):
        return C.byref(self._s)


# ---------------------------------------------------------------- codecs

def bf16_decode(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return np.array([lib().oref_bf16_decode(int(v)) for v in b.ravel()]).reshape(b.shape)


def bf16_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oref_bf16_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    table = np.array([lib().oref_e4m3_decode(i) for i in range(256)])
    return table[c]


def e4m3_encode(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oref_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e2m1_decode(c) -> np.ndarray:
    """E2M1 value of the low nibble of each code."""
    c = np.asarray(c, dtype=np.uint8)
    table = np.array([lib().oref_e2m1_decode(i) for i in range(16)])
    return table[c & 0x0F]


def e8m0_decode(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    table = np.array([lib().oref_e8m0_decode(i) for i in range(256)])
    return table[c]


def quant_row(v):
    """1x128 group quantisation of a float32 vector -> (codes uint8, scales float32)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.ndim == 1 and v.size % 128 == 0
    q = np.empty(v.size, dtype=np.uint8)
    s = np.empty(v.size // 128, dtype=np.float32)
    lib().oref_quant_row(_p(v), v.size, _p(q), _p(s))
    return q, s


def quant_bf16_rows(x):
    """Per-row 1x128 quantisation of bf16 rows [R, n] -> codes [R, n], scales [R, n/128]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    R, n = x.shape
    q = np.empty((R, n), dtype=np.uint8)
    s = np.empty((R, n // 128), dtype=np.float32)
    lib().oref_quant_bf16_rows(_p(x), R, n, _p(q), _p(s))
    return q, s


# ---------------------------------------------------------------- routing

def _tokens(token_list, T):
    if token_list is None:
        return None, T
    tl = np.ascontiguousarray(token_list, dtype=np.int64)
    assert tl.size == 0 or (tl.min() >= 0 and tl.max() < T)
    return tl, tl.size


def route(layer: Layer, x, token_list=None, want_logits=False):
    """-> ids int32 [n,k] (ascending), gates float64 [n,k], gap float64 [n], logits or None."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    tl, n = _tokens(token_list, T)
    ids = np.empty((n, layer.k), dtype=np.int32)
    gates = np.empty((n, layer.k), dtype=np.float64)
    gap = np.empty(n, dtype=np.float64)
    logits = np.empty((n, layer.E), dtype=np.float64) if want_logits else None
    lib().oref_route(layer.ref, _p(x), T, _p(tl), n, _p(ids), _p(gates), _p(logits), _p(gap))
    return ids, gates, gap, logits


def gates_for_ids(layer: Layer, x, ids, token_list=None):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    tl, n = _tokens(token_list, T)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, layer.k)
    g = np.empty((n, layer.k), dtype=np.float64)
    lib().oref_gates_for_ids(layer.ref, _p(x), T, _p(tl), n, _p(ids), _p(g))
    return g


# ---------------------------------------------------------------- grouping

def permute(keys, E):
    """Stable counting sort -> (offsets [E+1], perm_src [N], perm_pos [N], dropped)."""
    keys = np.ascontiguousarray(keys, dtype=np.int32).ravel()
    N = keys.size
    off = np.empty(E + 1, dtype=np.int32)
    src = np.full(max(N, 1), -1, dtype=np.int32)[:N]
    pos = np.empty(N, dtype=np.int32)
    dropped = lib().oref_permute(_p(keys), N, E, _p(off), _p(src), _p(pos))
    return off, src, pos, int(dropped)


# ---------------------------------------------------------------- FFN

def expert_row(layer: Layer, e, a, a_scale=None):
    """Routed expert e on one stored input row -> (out fp64 [H], stored h fp64 [I])."""
    a = np.ascontiguousarray(a, dtype=np.uint8 if layer.fp8 else np.uint16)
    sc = _c(a_scale, np.float32)
    out = np.empty(layer.H)
    h = np.empty(layer.I)
    lib().oref_expert_row(layer.ref, int(e), _p(a), _p(sc), _p(out), _p(h))
    return out, h


def expert_gate_up(layer: Layer, e, a, a_scale, factored: bool):
    """Gate/up pre-activations (fp8 or mxfp4 layer) -> zg [I], zu [I]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    sc = np.ascontiguousarray(a_scale, dtype=np.float32)
    zg = np.empty(layer.I)
    zu = np.empty(layer.I)
    if factored:
        f = lib().oref_expert_gate_up_mx_factored if layer.mx else lib().oref_expert_gate_up_factored
    else:
        f = lib().oref_expert_gate_up_dequant
    f(layer.ref, int(e), _p(a), _p(sc), _p(zg), _p(zu))
    return zg, zu


def shared_row(layer: Layer, x_row):
    x_row = np.ascontiguousarray(x_row, dtype=np.uint16)
    out = np.empty(layer.H)
    lib().oref_shared_row(layer.ref, _p(x_row), _p(out))
    return out


def expert_ffn(layer: Layer, offsets, a_rows, a_scale=None):
    """moe_expert_ffn definition on grouped rows -> out fp64 [N,H]."""
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    a_rows = np.ascontiguousarray(a_rows, dtype=np.uint8 if layer.fp8 else np.uint16)
    sc = _c(a_scale, np.float32)
    N = a_rows.shape[0]
    out = np.empty((N, layer.H))
    lib().oref_expert_ffn(layer.ref, _p(offsets), _p(a_rows), _p(sc), N, _p(out))
    return out


# ---------------------------------------------------------------- layer

def forward(layer: Layer, x, token_list=None):
    """-> y fp64 [n,H], ids [n,k], gates [n,k], gap [n] for the listed tokens."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    tl, n = _tokens(token_list, T)
    y = np.empty((n, layer.H))
    ids = np.empty((n, layer.k), dtype=np.int32)
    gates = np.empty((n, layer.k))
    gap = np.empty(n)
    lib().oref_forward(layer.ref, _p(x), T, _p(tl), n, _p(y), _p(ids), _p(gates), _p(gap))
    return y, ids, gates, gap


def forward_with_ids(layer: Layer, x, ids, token_list=None):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    tl, n = _tokens(token_list, T)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, layer.k)
    y = np.empty((n, layer.H))
    lib().oref_forward_with_ids(layer.ref, _p(x), T, _p(tl), n, _p(ids), _p(y))
    return y


def forward_triples(layer: Layer, x, tok, expert, gate, token_list=None):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    tl, n = _tokens(token_list, T)
    tok = np.ascontiguousarray(tok, dtype=np.int32)
    expert = np.ascontiguousarray(expert, dtype=np.int32)
    gate = np.ascontiguousarray(gate, dtype=np.float32)
    y = np.empty((n, layer.H))
    lib().oref_forward_triples(layer.ref, _p(x), T, _p(tok), _p(expert), _p(gate), tok.size,
                               _p(tl), n, _p(y))
    return y


def combine(y_perm, perm_pos, gates, T, k=1, tok=None, shared=None):
    """moe_combine definition in fp64 -> y [T,H]."""
    y_perm = np.ascontiguousarray(y_perm, dtype=np.float64)
    perm_pos = np.ascontiguousarray(perm_pos, dtype=np.int32).ravel()
    gates = np.ascontiguousarray(gates, dtype=np.float32).ravel()
    tok = _c(tok, np.int32)
    shared = _c(shared, np.float64)
    H = y_perm.shape[1]
    y = np.empty((T, H))
    lib().oref_combine(_p(y_perm), _p(perm_pos), _p(tok), int(k), _p(gates), perm_pos.size,
                       _p(shared), T, H, _p(y))
    return y


def backward(layer: Layer, x, ids, dy, token_list=None, weights=True):
    """Backward of the layer (bf16 experts) with experts fixed to ids -> dict of fp64 gradients:
    dx [n,H], dw_gate_up [E,2I,H], dw_down [E,H,I], dw_shared_gate_up [2Is,H], dw_shared_down [H,Is],
    dw_router [E,H], dbias [E] (weight gradients summed over the listed tokens).
    weights=False: dx only (the weight gradients are not formed; they are None)."""
    assert layer.format == BF16, "the backward oracle covers bf16 experts"
    x = np.ascontiguousarray(x, dtype=np.uint16)
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    T = x.shape[0]
    tl, n = _tokens(token_list, T)
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(T, layer.k)
    E, H, I, Is = layer.E, layer.H, layer.I, layer.Is
    w = weights
    out = dict(dx=np.empty((n, H)), dw_gate_up=np.empty((E, 2 * I, H)) if w else None,
               dw_down=np.empty((E, H, I)) if w else None,
               dw_shared_gate_up=np.empty((2 * Is, H)) if Is and w else None,
               dw_shared_down=np.empty((H, Is)) if Is and w else None,
               dw_router=np.empty((E, H)) if w else None, dbias=np.empty(E) if w else None)
    lib().oref_backward(layer.ref, _p(x), T, _p(ids), _p(dy), _p(tl), n, _p(out["dx"]), _p(out["dw_gate_up"]),
                        _p(out["dw_down"]), _p(out["dw_shared_gate_up"]), _p(out["dw_shared_down"]),
                        _p(out["dw_router"]), _p(out["dbias"]))
    return out


def _bf16_f64(b) -> np.ndarray:
    """bf16 bits -> fp64: a bf16 value is the binary32 value with the same top 16 bits."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def expert_weight_grads(layer: Layer, x, ids, dy, e):
    """dW_gate_up[e] [2I,H] and dW_down[e] [H,I] (fp64) of the layer's backward
    (bf16 experts, experts fixed to ids), summed over every token routed to e.

    Only expert e's slots enter these two gradients: with g the slot's gate
    (softmax over the token's chosen logits) the expert sees output gradient
    g dy, so dW_down = sum (g dy) h^T and dW_gate_up = sum dz x^T with the
    SwiGLU backward dz.  numpy matmuls serve as the products, one batch of
    the expert's tokens (for sizes where the whole backward is out of reach)."""
    assert layer.format == BF16
    x = np.ascontiguousarray(x, dtype=np.uint16)
    T = x.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(T, layer.k)
    H, I = layer.H, layer.I
    ts, js = np.nonzero(ids == e)
    if ts.size == 0:
        return np.zeros((2 * I, H)), np.zeros((H, I))
    g = gates_for_ids(layer, x, ids[ts], token_list=ts)[np.arange(ts.size), js]
    X = _bf16_f64(x[ts])
    dO = g[:, None] * _bf16_f64(np.asarray(dy, dtype=np.uint16)[ts])
    wgu = _bf16_f64(layer.w_gate_up[e])
    wd = _bf16_f64(layer.w_down[e])
    z = X @ wgu.T
    zg, zu = z[:, :I], z[:, I:]
    sg = 1.0 / (1.0 + np.exp(-zg))
    h = zg * sg * zu
    dh = dO @ wd
    dz = np.concatenate([dh * zu * sg * (1.0 + zg * (1.0 - sg)), dh * zg * sg], axis=1)
    return dz.T @ X, dO.T @ h


def num_threads() -> int:
    return int(lib().oref_num_threads())
