"""moe_forward_noalloc (include/moe.h): the forward with the library's static
scratch array instead of a workspace, for callers that cannot allocate.  On
the GPU it must give moe_forward's outputs bit for bit (same kernels), on two
calls in a row -- the second with fewer tokens, so it runs on what the first
left in the array -- and again after moe_forward has run in between; on the
CPU, a call too large for the array is refused before the device is touched."""
import numpy as np
import pytest
import torch

from router_gemm_amd import binding as B
from router_gemm_amd import workloads as W

from conftest import gpu_available
from gpu_util import dev


def _layer_c(dtype, H=4096, I=1536, E=352, k=8, Is=1536):
    FAKE = 0x100000   # never dereferenced: the size check refuses first
    return B.MoELayerC(H, I, E, k, Is, dtype, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


@pytest.mark.parametrize("dtype,T_ok,T_big", [(B.MOE_FP8_E4M3FN, 469, 470), (B.MOE_BF16, 359, 360)])
def test_noalloc_refuses_calls_beyond_the_scratch_array(dtype, T_ok, T_big):
    import ctypes as C
    L = _layer_c(dtype)
    lib = B.lib()
    assert lib.moe_workspace_bytes(C.byref(L), T_ok, T_ok * 8) <= B.MOE_NOALLOC_SCRATCH_BYTES
    for T in (T_big, 8192):
        st = lib.moe_forward_noalloc(C.byref(L), 0x100000, T, 0x100000, B.MOE_BF16, None, None, None)
        assert st == B.MOE_EWORKSPACE, (T, st)
        assert b"scratch" in lib.moe_last_error()
    bad = _layer_c(dtype, H=100)           # invalid layer: the usual host-side refusal
    assert lib.moe_forward_noalloc(C.byref(bad), 0x100000, 8, 0x100000, B.MOE_BF16, None, None, None) \
        == B.MOE_EUNSUPPORTED


def _run_both(lt, x, out_dtype):
    cfg = lt.cfg
    T = x.shape[0]
    layer = B.Layer.from_tensors(lt)
    d = x.device
    outs = []
    for use_ws in (True, False):
        y = torch.full((T, cfg.H), float("nan"), dtype=out_dtype, device=d)
        ids = torch.full((T, cfg.k), -7, dtype=torch.int32, device=d)
        gates = torch.full((T, cfg.k), float("nan"), dtype=torch.float32, device=d)
        if use_ws:
            B.moe_forward(layer, x, T, y, topk_ids=ids, topk_gates=gates, ws=B.workspace(layer, T, T * cfg.k, d))
        else:
            B.moe_forward_noalloc(layer, x, T, y, topk_ids=ids, topk_gates=gates)
        torch.cuda.synchronize()
        outs.append((y, ids, gates))
    return outs


@pytest.mark.gpu
@pytest.mark.skipif(not gpu_available(), reason="needs a GPU")
@pytest.mark.parametrize("name,Ts,out_dtype", [
    ("decode_fp8", (64, 17), torch.bfloat16),          # the decode layer: 352 fp8 experts, streaming kernels
    ("decode_fp8", (4, 1), torch.bfloat16),            # the shared expert's K split 4, then 8 ways
    ("decode_bf16", (64, 5), torch.float32),            # bf16 experts
    ("small_fp8", (300, 30), torch.float32),   # LDS-tiled kernels (mean 75 rows), then streaming (7.5)
    ("small_bf16", (128, 31), torch.bfloat16),
])
def test_noalloc_matches_moe_forward_on_consecutive_calls(name, Ts, out_dtype):
    cfg = W.get_config(name)
    lt = W.make_layer(cfg, dev())
    for T in Ts:
        x = W.make_x(cfg, dev(), T=T)
        (ya, ia, ga), (yb, ib, gb) = _run_both(lt, x, out_dtype)
        assert torch.equal(ia, ib) and torch.equal(ga, gb), (name, T)
        assert torch.equal(ya, yb), (name, T, float((ya.float() - yb.float()).abs().max()))
        assert not torch.isnan(yb.float()).any()
    # and once more at the first size, after the smaller call and a moe_forward in between
    x = W.make_x(cfg, dev(), T=Ts[0])
    (ya, _, _), (yb, _, _) = _run_both(lt, x, out_dtype)
    assert torch.equal(ya, yb)
