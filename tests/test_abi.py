"""The C-ABI library loads, exports every entry point include/moe.h declares,
and refuses bad arguments on the host before launching anything (so these run
without a GPU: every call below fails validation, or is a T == 0 no-op)."""
import ctypes as C
import os
import re

import pytest

from router_gemm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # never dereferenced: validation fails first


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(B.EXPORTS), names
    lib = B.lib()
    for n in names:
        assert hasattr(lib, n), n


def layer(H=4096, I=1536, E=352, k=8, dtype=B.MOE_FP8_E4M3FN, Is=1536):
    return B.MoELayerC(H, I, E, k, Is, dtype, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def route(L, T=64, ws=FAKE, nb=1 << 40, x=FAKE):
    return B.lib().moe_route(C.byref(L), x, T, FAKE, FAKE, None, ws, nb, None)


def test_status_strings():
    lib = B.lib()
    for s in range(5):
        assert lib.moe_status_string(s).startswith(b"MOE_")


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), B.MOE_EINVAL), (dict(k=33), B.MOE_EINVAL), (dict(E=4, k=5), B.MOE_EINVAL),
    (dict(H=4000), B.MOE_EUNSUPPORTED), (dict(E=1025), B.MOE_EUNSUPPORTED),
    (dict(I=1600), B.MOE_EUNSUPPORTED),                              # fp8 needs I % 128 == 0
    (dict(I=1600, dtype=B.MOE_BF16), B.MOE_OK),                       # bf16 allows I % 64 == 0 (T=0 below)
    (dict(I=1568, dtype=B.MOE_BF16), B.MOE_EUNSUPPORTED),
    (dict(dtype=7), B.MOE_EUNSUPPORTED), (dict(Is=100), B.MOE_EUNSUPPORTED),
    (dict(H=0), B.MOE_EINVAL), (dict(E=-1), B.MOE_EINVAL),
    (dict(H=16384 + 128), B.MOE_EUNSUPPORTED), (dict(I=16384 + 128), B.MOE_EUNSUPPORTED),
    (dict(Is=16384 + 64), B.MOE_EUNSUPPORTED), (dict(H=16384, I=16384, Is=16384), B.MOE_OK),
    (dict(dtype=B.MOE_MXFP4_E2M1), B.MOE_OK),
    (dict(dtype=B.MOE_MXFP4_E2M1, I=1600), B.MOE_EUNSUPPORTED),      # mxfp4 needs I % 128 == 0
    (dict(dtype=B.MOE_MXFP4_E2M1, H=4000), B.MOE_EUNSUPPORTED),
])
def test_layer_validation(kw, status):
    L = layer(**kw)
    assert route(L, T=0) == status, B.lib().moe_last_error()


def test_null_layer_and_pointers():
    lib = B.lib()
    assert lib.moe_route(None, FAKE, 4, FAKE, FAKE, None, FAKE, 1 << 30, None) == B.MOE_EINVAL
    assert route(layer(), x=None) == B.MOE_EINVAL
    assert route(layer(), x=FAKE + 2) == B.MOE_EINVAL          # misaligned
    assert route(layer(), T=-1) == B.MOE_EINVAL


def test_workspace_refusal():
    L = layer()
    need = B.lib().moe_workspace_bytes(C.byref(L), 64, 512)
    assert need > 0
    assert route(L, nb=0) == B.MOE_EWORKSPACE
    assert route(L, ws=None, nb=1 << 40) == B.MOE_EINVAL
    assert route(L, ws=FAKE + 64) == B.MOE_EINVAL              # workspace must be 256-byte aligned
    assert b"workspace" in B.lib().moe_last_error()
    bad = layer(k=0)
    assert B.lib().moe_workspace_bytes(C.byref(bad), 64, 512) > 0   # k = 0 allowed for pre-routed calls
    assert B.lib().moe_workspace_bytes(C.byref(layer(H=100)), 64, 512) == 0


def test_permute_combine_ffn_refusals():
    lib, L = B.lib(), layer()
    r = lib.moe_permute(C.byref(L), FAKE, 64, FAKE, None, 500, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert r == B.MOE_EINVAL and b"T*k" in lib.moe_last_error()
    r = lib.moe_permute(C.byref(L), FAKE, 64, FAKE, None, 512, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert r == B.MOE_EINVAL and b"x_scale" in lib.moe_last_error()
    r = lib.moe_expert_ffn(C.byref(L), FAKE, FAKE, FAKE, 100, FAKE, 9, FAKE, 1 << 40, None)
    assert r == B.MOE_EUNSUPPORTED
    r = lib.moe_expert_ffn(C.byref(L), FAKE, FAKE, FAKE, 100, FAKE, B.MOE_F32, FAKE, 16, None)
    assert r == B.MOE_EWORKSPACE
    r = lib.moe_expert_ffn(C.byref(L), FAKE, FAKE, FAKE, 0, FAKE, B.MOE_F32, None, 0, None)
    assert r == B.MOE_OK                                       # N == 0: no-op
    Lk0 = layer(k=0)
    r = lib.moe_combine(C.byref(Lk0), FAKE, B.MOE_BF16, FAKE, None, FAKE, 10, None, 0, 10, FAKE, B.MOE_BF16,
                        FAKE, 1 << 40, None)
    assert r == B.MOE_EINVAL
    r = lib.moe_combine(C.byref(L), FAKE, B.MOE_BF16, FAKE, FAKE, FAKE, 10, None, 0, 10, FAKE, B.MOE_FP8_E4M3FN,
                        FAKE, 1 << 40, None)
    assert r == B.MOE_EUNSUPPORTED
    r = lib.moe_forward(C.byref(L), FAKE, 0, FAKE, B.MOE_BF16, None, None, None, 0, None)
    assert r == B.MOE_OK                                       # T == 0: no-op
    r = lib.moe_forward(C.byref(L), FAKE, 8, FAKE, B.MOE_F32, None, None, FAKE, 1024, None)
    assert r == B.MOE_EWORKSPACE


def test_timing_sites_validate_without_gpu():
    lib = B.lib()
    assert lib.moe_timing_arm(-1, 4) == B.MOE_EINVAL
    assert lib.moe_timing_arm(11, 4) == B.MOE_EINVAL          # MOE_SITE_COUNT
    assert lib.moe_timing_arm(4, 0) == B.MOE_EINVAL
    ms, n = C.c_double(1.0), C.c_int32(7)
    assert lib.moe_timing_read(5, C.byref(ms), C.byref(n)) == B.MOE_OK
    assert ms.value == 0.0 and n.value == 0


def test_mxfp4_scale_refusals():
    """MX FP4 layers need both E8M0 scale tensors, 16-byte aligned."""
    lib = B.lib()
    for sgu, sd, what in ((None, FAKE, b"s_gate_up"), (FAKE, None, b"s_gate_up"), (FAKE + 4, FAKE, b"aligned"),
                          (FAKE, FAKE + 8, b"aligned")):
        L = B.MoELayerC(4096, 1536, 352, 8, 0, B.MOE_MXFP4_E2M1, FAKE, None, FAKE, sgu, FAKE, sd, None, None)
        r = lib.moe_expert_ffn(C.byref(L), FAKE, FAKE, FAKE, 100, FAKE, B.MOE_F32, FAKE, 1 << 40, None)
        assert r == B.MOE_EINVAL and what in lib.moe_last_error(), lib.moe_last_error()
    # activations of an mxfp4 layer are e4m3 with 1x128 scales: x_scale is required
    L = layer(dtype=B.MOE_MXFP4_E2M1)
    r = lib.moe_permute(C.byref(L), FAKE, 64, FAKE, None, 512, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert r == B.MOE_EINVAL and b"x_scale" in lib.moe_last_error()


def test_backward_refusals_without_gpu():
    """moe_backward: bf16 experts only, router and outputs required, its own
    workspace size (moe_workspace_bytes does not cover it)."""
    lib = B.lib()
    L = layer(dtype=B.MOE_BF16)
    args = lambda T=64, dx=FAKE, dsgu=FAKE, ws=FAKE, nb=1 << 40, z=None: (
        C.byref(L), FAKE, T, FAKE, FAKE, FAKE, z, dx, FAKE, FAKE, dsgu, FAKE, FAKE, None, ws, nb, None)
    need = lib.moe_backward_workspace_bytes(C.byref(L), 64)
    assert need > lib.moe_workspace_bytes(C.byref(L), 64, 512)
    assert lib.moe_backward(*args(nb=need - 1)) == B.MOE_EWORKSPACE
    assert lib.moe_backward(*args(dx=None)) == B.MOE_EINVAL
    assert lib.moe_backward(*args(dx=FAKE + 4)) == B.MOE_EINVAL and b"aligned" in lib.moe_last_error()
    assert lib.moe_backward(*args(z=FAKE + 8)) == B.MOE_EINVAL and b"aligned" in lib.moe_last_error()
    assert lib.moe_backward(*args(dsgu=None)) == B.MOE_EINVAL and b"shared" in lib.moe_last_error()
    assert lib.moe_backward(*args(T=0, ws=None, nb=0)) == B.MOE_OK        # no-op
    L = layer(dtype=B.MOE_FP8_E4M3FN)
    assert lib.moe_backward(*args()) == B.MOE_EUNSUPPORTED and b"bf16" in lib.moe_last_error()
    L = layer(dtype=B.MOE_BF16, k=0)
    assert lib.moe_backward(*args()) == B.MOE_EINVAL
    assert lib.moe_backward_workspace_bytes(C.byref(L), 64) == 0


def test_forward_train_refusals_without_gpu():
    """moe_forward_train: bf16 experts, ids/gates/z_saved required; the saved
    pre-activation buffer holds T*k*2I + T*2Is floats."""
    lib = B.lib()
    L = layer(dtype=B.MOE_BF16)
    assert lib.moe_saved_z_floats(C.byref(L), 64) == 64 * 8 * 2 * 1536 + 64 * 2 * 1536
    call = lambda ids=FAKE, z=FAKE: lib.moe_forward_train(C.byref(L), FAKE, 64, FAKE, B.MOE_BF16, ids, FAKE, z,
                                                         FAKE, 1 << 40, None)
    assert call(z=None) == B.MOE_EINVAL
    assert call(ids=None) == B.MOE_EINVAL
    assert call(z=FAKE + 4) == B.MOE_EINVAL and b"aligned" in lib.moe_last_error()
    L = layer(dtype=B.MOE_FP8_E4M3FN)
    assert call() == B.MOE_EUNSUPPORTED


def test_weight_layout_and_pack_refusals_without_gpu():
    """weight_layout is 0 or 1, tile16 is refused for MX weights and for the
    training calls; moe_pack_weights validates pointers and sizes first."""
    lib = B.lib()

    def with_layout(v, **kw):
        L = layer(**kw)
        L.weight_layout = v
        return L

    assert route(with_layout(B.MOE_LAYOUT_TILE16), T=0) == B.MOE_OK
    assert route(with_layout(B.MOE_LAYOUT_TILE16, dtype=B.MOE_BF16), T=0) == B.MOE_OK
    assert route(with_layout(2), T=0) == B.MOE_EINVAL
    assert route(with_layout(-1), T=0) == B.MOE_EINVAL
    assert route(with_layout(B.MOE_LAYOUT_TILE16, dtype=B.MOE_MXFP4_E2M1), T=0) == B.MOE_EUNSUPPORTED
    L = with_layout(B.MOE_LAYOUT_TILE16, dtype=B.MOE_BF16)
    r = lib.moe_backward(C.byref(L), FAKE, 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                         FAKE, 1 << 40, None)
    assert r == B.MOE_EUNSUPPORTED and b"row-major" in lib.moe_last_error()
    r = lib.moe_forward_train(C.byref(L), FAKE, 64, FAKE, B.MOE_BF16, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert r == B.MOE_EUNSUPPORTED and b"row-major" in lib.moe_last_error()
    pack = lambda src=FAKE, dst=FAKE + (1 << 24), n=1, rows=16, rb=128: lib.moe_pack_weights(src, dst, n, rows, rb,
                                                                                              None)
    assert pack(src=None) == B.MOE_EINVAL
    assert pack(dst=None) == B.MOE_EINVAL
    assert pack(src=FAKE + 8) == B.MOE_EINVAL and b"aligned" in lib.moe_last_error()
    for n, rows, rb in ((1, 15, 128), (1, 0, 128), (1, -16, 128), (1, 16, 64), (1, 16, 0), (1, 32, 200), (0, 16, 128),
                        (-1, 16, 128), (1 << 40, 1 << 20, 1 << 20)):
        assert pack(n=n, rows=rows, rb=rb) == B.MOE_EINVAL, (n, rows, rb)
    assert pack(dst=FAKE + 1024) == B.MOE_EINVAL and b"overlap" in lib.moe_last_error()
    assert pack(n=2, dst=FAKE + 2048) == B.MOE_EINVAL and b"overlap" in lib.moe_last_error()


def test_forward_routed_refusals():
    lib = B.lib()
    L = layer()
    f = lambda L=L, T=16, N=20, x=FAKE, ae=FAKE, at=FAKE, g=FAKE, y=FAKE, od=B.MOE_BF16, ws=FAKE, nb=1 << 40: \
        lib.moe_forward_routed(C.byref(L), x, T, ae, at, g, N, y, od, ws, nb, None)
    assert f(x=None) == B.MOE_EINVAL
    assert f(ae=None) == B.MOE_EINVAL and f(at=None) == B.MOE_EINVAL and f(g=None) == B.MOE_EINVAL
    assert f(od=7) == B.MOE_EUNSUPPORTED
    assert f(T=-1) == B.MOE_EINVAL
    assert f(nb=16) == B.MOE_EWORKSPACE
    assert f(x=FAKE + 4) == B.MOE_EINVAL                     # misaligned
    assert f(T=0, x=None, y=None) == B.MOE_OK                # no-op
    bad = layer(H=100)
    assert f(L=bad) == B.MOE_EUNSUPPORTED
