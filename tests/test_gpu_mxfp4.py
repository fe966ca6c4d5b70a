"""GPU parity of the MX FP4 expert-weight format (E2M1 codes, one E8M0 scale
per 32 inputs) against the fp64 oracle: the grouped expert FFN on its own
(every token-tile height the streaming kernels have, ragged K with an odd
number of 128-input chunks, empty experts, both output dtypes) and the whole
layer (routing, grouping with e4m3 activations, MX expert GEMMs, the bf16
shared expert in the same launch, combine)."""
import numpy as np
import pytest
import torch

import oracle
from router_gemm_amd import binding as B
from router_gemm_amd import workloads as W

from conftest import gpu_available
from gpu_util import TOL, check_forward, dev, oracle_layer, rel_err_rows, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _print(*a):
    print(*a, flush=True)


def _grouped_e4m3_rows(E, N, H, rng, empty_frac=0.3):
    counts = rng.multinomial(N, rng.dirichlet(np.ones(E) * 0.5))
    counts[rng.random(E) < empty_frac] = 0
    counts[0] += N - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    codes = rng.integers(0, 0x7E, size=(N, H)).astype(np.uint8) | (rng.integers(0, 2, (N, H)) << 7).astype(np.uint8)
    scales = (rng.random((N, H // 128)) * 0.01 + 1e-3).astype(np.float32)
    return off, codes, scales


@pytest.mark.parametrize("E,N,H,I,ydt", [
    (64, 200, 512, 256, torch.float32),     # ~3 rows per expert: 16-row token tiles
    (16, 300, 512, 256, torch.float32),     # ~19: 32-row tiles
    (3, 2000, 384, 128, torch.bfloat16),    # ~667: 64-row tiles; 3 and 1 chunks of 128 inputs (odd)
    (8, 517, 640, 384, torch.bfloat16),     # 5 and 3 chunks
    (1, 100, 512, 1536, torch.float32),     # one expert, the routed width (tiled: 100 rows)
    (32, 150, 768, 640, torch.float32),     # 16-row tiles: 6 gate/up chunks (pipelined steps + a lone last step), 5 down chunks
    (8, 200, 1024, 512, torch.bfloat16),    # 32-row tiles: 8 and 4 chunks
    # LDS-tiled MX kernels, 64-row token tiles (48..127 rows per expert, H and I multiples of 256):
    (16, 1100, 512, 256, torch.bfloat16),   # ~69 rows: 2 and 1 stages; ragged last token tiles
    (12, 1000, 1024, 768, torch.float32),   # ~83: 4 and 3 (odd) stages
    # 256 x 256 MX items (128 or more rows per expert), three-stage ring of 128-input chunks:
    (6, 1500, 1024, 768, torch.bfloat16),   # several 256-row token tiles per expert; 8 and 6 chunks
    (3, 700, 512, 256, torch.float32),      # 4 and 2 chunks (the down items' two chunks are both issued ahead)
    (2, 1300, 768, 512, torch.bfloat16),    # ~650 rows: bands of token tiles; 6 and 4 chunks, 3 down column tiles
    (1, 300, 512, 1536, torch.float32),     # one expert, the routed width: 12 gate/up column tiles, 12 down chunks
])
def test_mx_expert_ffn_matches_oracle(E, N, H, I, ydt):
    rng = np.random.default_rng(E * N + H)
    cfg = W.MoEConfig("t", T=N, H=H, E=E, k=1, I=I, Is=0, expert_dtype="mxfp4", router_std=0.05, seed=4)
    _print(f"[mx expert_ffn E={E} N={N} H={H} I={I}]")
    lt = W.make_layer(cfg, dev())
    off, a, s = _grouped_e4m3_rows(E, N, H, rng)
    d = dev()
    layer = B.Layer.from_tensors(lt)
    y = torch.full((N, H), float("nan"), dtype=ydt, device=d)
    B.moe_expert_ffn(layer, torch.from_numpy(off).to(d), torch.from_numpy(a).to(d), torch.from_numpy(s).to(d),
                     N, y, ws=B.workspace(layer, N, N, d))
    torch.cuda.synchronize()
    y_ref = oracle.expert_ffn(oracle_layer(lt), off, a, s)
    err = rel_err_rows(to_np(y), y_ref)
    _print(f"  max rel err {err.max():.3e} mean {err.mean():.3e}")
    assert err.max() < TOL["mxfp4"]


# 136, 1, 17: streaming kernels; 389: 64-row MX tiles and the shared expert's
# own tiled launch; 600 and 1100: 256 x 256 MX items with the bf16 shared
# expert's items in the same launches
@pytest.mark.parametrize("T", [136, 1, 17, 389, 600, 1100])
def test_mx_forward_matches_oracle(T):
    cfg = W.get_config("small_mxfp4", T=T)
    _print(f"[mx forward T={T}]")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x)
    _print(f"  {st}")


def test_mx_forward_bf16_output_without_shared_expert():
    cfg = W.get_config("small_mxfp4", Is=0, T=64)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x, out_dtype=torch.bfloat16)
    _print(f"[mx forward bf16 out, no shared] {st}")


@pytest.mark.parametrize("over", [dict(T=1100), dict(T=1100, Is=0), dict(T=900, zipf_s=1.1, zipf_beta=0.6)])
def test_mx_wide_forward_bitwise_repeatable(over):
    """The 256 x 256 MX items: the same output bits on every call, whatever
    the workspace held before (no order-dependent sums; every padding row and
    stale LDS byte stays out of the stored results), and within tolerance of
    the oracle."""
    cfg = W.get_config("small_mxfp4", **over)
    _print(f"[mx wide repeat {over}]")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    check_forward(lt, x)
    layer = B.Layer.from_tensors(lt)
    ws = B.workspace(layer, cfg.T, cfg.N, dev())
    outs = []
    for rep in range(5):
        ws.fill_(rep * 53 % 256)
        y = torch.empty((cfg.T, cfg.H), dtype=torch.float32, device=dev())
        B.moe_forward(layer, x, cfg.T, y, ws=ws)
        torch.cuda.synchronize()
        outs.append(y)
    for y in outs[1:]:
        assert torch.equal(y, outs[0])


def test_mx_weights_are_read_as_stored():
    """Swapping the two nibbles of every weight byte changes the GPU result the
    way it changes the oracle's (a kernel reading the wrong nibble would match
    the swapped layer instead)."""
    cfg = W.get_config("small_mxfp4", T=32, Is=0)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    check_forward(lt, x)
    sw = lambda t: ((t >> 4) | (t << 4)).contiguous()
    lt2 = W.LayerTensors(cfg, lt.w_router, lt.router_bias, sw(lt.w_gate_up), sw(lt.w_down), lt.s_gate_up,
                         lt.s_down, None, None)
    check_forward(lt2, x)


def test_mx_primitives_with_pre_routed_triples():
    """An expert-parallel share with MX FP4 experts driven through the four
    primitives: permute (e4m3 rows + 1x128 scales), the MX expert FFN, the
    shared expert as a one-expert bf16 layer, combine; against the oracle's
    pre-routed-triples form of the layer."""
    cfg = W.MoEConfig("mx_triples", T=300, H=512, E=12, k=0, I=256, Is=128, expert_dtype="mxfp4",
                      router_std=0.05, zipf_s=1.1, triples=700, seed=5)
    _print("[mx triples]")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    tok, exp, gate = W.make_triples(cfg)
    exp[:3] = [cfg.E, -1, cfg.E + 7]          # out of range: dropped
    d = dev()
    T, N, E, H = cfg.T, cfg.N, cfg.E, cfg.H
    layer = B.Layer.from_tensors(lt, top_k=0)
    shared = B.Layer.shared_view(lt)
    ws = torch.empty(max(B.moe_workspace_bytes(layer, T, N), B.moe_workspace_bytes(shared, T, T)),
                     dtype=torch.uint8, device=d)
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    src = torch.empty(N, dtype=torch.int32, device=d)
    pos = torch.empty(N, dtype=torch.int32, device=d)
    xp = torch.empty((N, H), dtype=torch.uint8, device=d)
    xs = torch.empty((N, H // 128), dtype=torch.float32, device=d)
    tok_g, exp_g, gate_g = (torch.from_numpy(a).to(d) for a in (tok, exp, gate))
    B.moe_permute(layer, x, T, exp_g, tok_g, N, off, src, pos, xp, xs, ws=ws)
    yp = torch.empty((N, H), dtype=torch.bfloat16, device=d)
    B.moe_expert_ffn(layer, off, xp, xs, N, yp, ws=ws)
    s_out = torch.empty((T, H), dtype=torch.float32, device=d)
    B.moe_expert_ffn(shared, torch.tensor([0, T], dtype=torch.int32, device=d), x, None, T, s_out, ws=ws)
    y = torch.empty((T, H), dtype=torch.float32, device=d)
    B.moe_combine(layer, yp, B.MOE_BF16, pos, tok_g, gate_g, N, s_out, B.MOE_F32, T, y, B.MOE_F32, ws=ws)
    torch.cuda.synchronize()
    off_r, src_r, pos_r, dropped = oracle.permute(exp, E)
    assert dropped == 3
    assert np.array_equal(off.cpu().numpy(), off_r) and np.array_equal(pos.cpu().numpy(), pos_r)
    # the e4m3 rows and scales are bit-exact: quantisation decisions in fp32 on both sides
    q_tok, s_tok = oracle.quant_bf16_rows(W.bf16_bits(x))
    nv = int(off_r[-1])
    assert np.array_equal(xp.cpu().numpy()[:nv], q_tok[tok[src_r[:nv]]])
    assert np.array_equal(xs.cpu().numpy()[:nv], s_tok[tok[src_r[:nv]]])
    y_ref = oracle.forward_triples(oracle_layer(lt), W.bf16_bits(x), tok, exp, gate)
    err = rel_err_rows(to_np(y), y_ref)
    _print(f"  max rel err {err.max():.3e} over {T} tokens")
    assert err.max() < TOL["mxfp4"]
