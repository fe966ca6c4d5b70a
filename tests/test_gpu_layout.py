"""The 16-row tile weight layout (MOE_LAYOUT_TILE16, moe_pack_weights).

The packing is a byte permutation, checked against a numpy restatement of
the layout that include/moe.h documents.  Every forward path that reads
packed weights -- the streaming kernels (bf16 with one and two gate tiles
per wave, fp8), the LDS-tiled kernels with 128- and 256-row token tiles,
moe_expert_ffn on a one-expert layer, and the full-size decode and prefill
layers -- must give the row-major path's outputs bit for bit: the kernels
do the same arithmetic on the same values, only their addresses differ.
The row-major path itself is held to the fp64 oracle by the parity tests.
"""
import dataclasses

import numpy as np
import pytest
import torch

from router_gemm_amd import binding as B
from router_gemm_amd import workloads as W

from conftest import gpu_available
from gpu_util import dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def np_pack(a: np.ndarray) -> np.ndarray:
    """tile16 bytes of count row-major uint8 [rows, row_bytes] matrices
    a[count, rows, row_bytes]: tile (t, c) of a matrix at (c * rows/16 + t)
    * 2048, byte b of its row i at 1024 ((b / 16) % 2) + 16 (i + 16 (b / 32))
    + b % 16."""
    count, rows, K = a.shape
    v = a.reshape(count, rows // 16, 16, K // 128, 4, 2, 16)   # [m, t, i, c, g = b/32, q = (b/16)%2, b%16]
    return np.ascontiguousarray(v.transpose(0, 3, 1, 5, 4, 2, 6)).reshape(-1)


@pytest.mark.parametrize("count,rows,row_bytes", [(1, 16, 128), (3, 48, 384), (5, 64, 1024)])
def test_pack_is_the_documented_permutation(count, rows, row_bytes):
    rng = np.random.default_rng(rows + row_bytes)
    a = rng.integers(0, 256, (count, rows, row_bytes), dtype=np.uint8)
    src = torch.from_numpy(a).to(dev())
    dst = torch.full_like(src, 0x5A)
    B.moe_pack_weights(src, dst, count, rows, row_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy().reshape(-1), np_pack(a))


def _forward(layer, x, cfg):
    T = x.shape[0]
    y = torch.empty((T, cfg.H), dtype=torch.float32, device=x.device)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device=x.device)
    gates = torch.empty((T, cfg.k), dtype=torch.float32, device=x.device)
    B.moe_forward(layer, x, T, y, topk_ids=ids, topk_gates=gates, ws=B.workspace(layer, T, T * cfg.k, x.device))
    torch.cuda.synchronize()
    return y, ids


CASES = [
    ("small_bf16", {}),                                   # streaming, bf16, two gate tiles per wave
    ("small_bf16", dict(I=192, Is=64)),                   # streaming, bf16, I % 128 != 0: one gate tile per wave
    ("small_fp8", {}),                                    # streaming, fp8
    ("small_bf16", dict(T=1)),                            # one token
    ("small_fp8", dict(T=1, E=4, k=1)),                   # one token, one expert per token
    ("small_bf16", dict(I=64, Is=64)),                    # the narrowest bf16 experts (one 64-column tile)
    ("small_bf16", dict(T=517, I=128, Is=128)),           # LDS-tiled, 128-row token tiles
    ("small_fp8", dict(T=389)),                           # LDS-tiled, 128-row token tiles, fp8
    ("small_bf16", dict(T=1500, I=256, Is=128)),          # LDS-tiled, 256-row token tiles
    ("small_fp8", dict(T=1100, zipf_s=1.1, zipf_beta=0.6)),  # 256-row token tiles, skewed loads
]


@pytest.mark.parametrize("name,over", CASES)
def test_packed_forward_equals_row_major(name, over):
    cfg = dataclasses.replace(W.get_config(name), **over)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    y0, i0 = _forward(layer, x, cfg)
    y1, i1 = _forward(layer.packed(), x, cfg)
    assert torch.equal(i0, i1)
    assert torch.equal(y0, y1), float((y0 - y1).abs().max())


@pytest.mark.parametrize("name,over", [("small_bf16", {}), ("small_fp8", dict(T=777))])
def test_packed_forward_bf16_output(name, over):
    """bf16 output (the rounding of the combine's fp32 sums) is the same too."""
    cfg = dataclasses.replace(W.get_config(name), **over)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    out = []
    for L in (layer, layer.packed()):
        y = torch.empty((cfg.T, cfg.H), dtype=torch.bfloat16, device=dev())
        B.moe_forward(L, x, cfg.T, y, ws=B.workspace(L, cfg.T, cfg.N, dev()))
        torch.cuda.synchronize()
        out.append(y)
    assert torch.equal(out[0], out[1])


def test_packed_pre_routed_expert_ffn():
    """moe_expert_ffn on pre-routed rows of many experts (the expert-parallel
    share's call): 44 fp8 experts, 3000 rows with Zipf-like loads."""
    cfg = dataclasses.replace(W.get_config("small_fp8"), E=44, k=0)
    lt = W.make_layer(cfg, dev())
    rng = np.random.default_rng(9)
    counts = np.maximum(1, (3000 / np.arange(1, 45) ** 1.1 / np.sum(1 / np.arange(1, 45) ** 1.1))).astype(int)
    N = int(counts.sum())
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev())
    xq = torch.from_numpy(rng.integers(0, 0x7f, (N, cfg.H), dtype=np.uint8)).to(dev())   # finite e4m3 codes
    xs = torch.from_numpy(rng.uniform(0.5, 2.0, (N, cfg.H // 128)).astype(np.float32)).to(dev())
    layer = B.Layer.from_tensors(lt, top_k=0)
    out = []
    for L in (layer, layer.packed()):
        y = torch.empty((N, cfg.H), dtype=torch.float32, device=dev())
        B.moe_expert_ffn(L, off, xq, xs, N, y, ws=B.workspace(L, N, N, dev()))
        torch.cuda.synchronize()
        out.append(y)
    assert torch.isfinite(out[0]).all()
    assert torch.equal(out[0], out[1])


def test_packed_expert_ffn_one_expert():
    """moe_expert_ffn on a one-expert layer (the dense FF layer's call): 300
    rows over a 2560-wide intermediate, bf16."""
    H, I, T = 1024, 2560, 300
    g = torch.Generator(device="cpu").manual_seed(5)
    wgu = (torch.randn(1, 2 * I, H, generator=g) * 0.02).to(torch.bfloat16).to(dev())
    wd = (torch.randn(1, H, I, generator=g) * 0.02).to(torch.bfloat16).to(dev())
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).to(dev())
    layer = B.Layer(H, I, 1, 1, B.MOE_BF16, wgu, wd)
    off = torch.tensor([0, T], dtype=torch.int32, device=dev())
    out = []
    for L in (layer, layer.packed()):
        y = torch.empty((T, H), dtype=torch.float32, device=dev())
        B.moe_expert_ffn(L, off, x, None, T, y, ws=B.workspace(L, T, T, dev()))
        torch.cuda.synchronize()
        out.append(y)
    assert torch.equal(out[0], out[1])


@pytest.mark.parametrize("name", ["decode_bf16", "decode_fp8", "prefill_fp8"])
def test_packed_full_size_layers_equal_row_major(name):
    cfg = W.get_config(name)
    print("case", name, flush=True)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    layer = B.Layer.from_tensors(lt)
    y0, i0 = _forward(layer, x, cfg)
    packed = layer.packed()
    y1, i1 = _forward(packed, x, cfg)
    assert torch.equal(i0, i1)
    assert torch.equal(y0, y1), float((y0 - y1).abs().max())
