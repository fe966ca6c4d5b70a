"""GPU parity at the full Step-5 layer sizes, in the launch configuration the
benchmark times: decode T=64 (bf16, FP8 and MX FP4 experts), prefill T=8192 with the
Zipf-biased router (FP8), and one expert-parallel share driven through the four
primitives with pre-routed triples.  Routing, grouping and the fp8 x_perm bytes
are checked for every token; outputs on every token where the oracle is quick
(decode) and on a seeded sample of tokens otherwise."""
import numpy as np
import pytest
import torch

import oracle
from router_gemm_amd import binding as B
from router_gemm_amd import workloads as W

from conftest import gpu_available
from gpu_util import TOL, check_forward, check_ids, dev, oracle_layer, rel_err_rows, run_forward, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.mark.parametrize("name", ["c1", "c2", "decode_mxfp4"])
def test_decode_full_parity(name):
    cfg = W.get_config(name)
    print(f"[{cfg.name}] building layer", flush=True)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    st = check_forward(lt, x)
    print(f"[{cfg.name}] {st}", flush=True)


def test_prefill_routing_grouping_and_sampled_outputs():
    cfg = W.get_config("c3")
    print("[prefill_fp8] building layer", flush=True)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    OL = oracle_layer(lt)
    sample = np.random.default_rng(0).choice(cfg.T, 24, replace=False)
    st = check_forward(lt, x, OL=OL, sample=sample)
    print(f"[prefill_fp8] {st}", flush=True)
    # grouping of the GPU's own ids, bit-exact, plus every fp8 byte of x_perm
    _, ids, _ = run_forward(lt, x)
    layer = B.Layer.from_tensors(lt)
    N, E, H = cfg.N, cfg.E, cfg.H
    d = dev()
    off = torch.empty(E + 1, dtype=torch.int32, device=d)
    src = torch.empty(N, dtype=torch.int32, device=d)
    pos = torch.empty(N, dtype=torch.int32, device=d)
    xp = torch.empty((N, H), dtype=torch.uint8, device=d)
    xs = torch.empty((N, H // 128), dtype=torch.float32, device=d)
    B.moe_permute(layer, x, cfg.T, ids, None, N, off, src, pos, xp, xs, ws=B.workspace(layer, cfg.T, N, d))
    torch.cuda.synchronize()
    ids_np = ids.cpu().numpy().ravel()
    off_r, src_r, pos_r, _ = oracle.permute(ids_np, E)
    assert np.array_equal(off.cpu().numpy(), off_r)
    assert np.array_equal(src.cpu().numpy(), src_r) and np.array_equal(pos.cpu().numpy(), pos_r)
    counts = np.diff(off_r)
    print(f"[prefill_fp8] expert load max/mean {counts.max() / counts.mean():.2f}, "
          f"max {counts.max()}, min {counts.min()}", flush=True)
    q_tok, s_tok = oracle.quant_bf16_rows(W.bf16_bits(x))
    toks = src_r // cfg.k
    assert np.array_equal(xp.cpu().numpy(), q_tok[toks])
    assert np.array_equal(xs.cpu().numpy(), s_tok[toks])


def test_prefill_mxfp4_sampled_outputs():
    """The prefill layer with MX FP4 experts (LDS-tiled MX kernels, 64-row token
    tiles; the bf16 shared expert on its own tiled launch): routing of every
    token, outputs of a seeded sample of tokens plus the tokens routed to the
    most loaded expert."""
    cfg = W.get_config("prefill_mxfp4")
    print("[prefill_mxfp4] building layer", flush=True)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    OL = oracle_layer(lt)
    ids_all, _, _, _ = oracle.route(OL, W.bf16_bits(x))
    hot = np.bincount(ids_all.ravel(), minlength=cfg.E).argmax()
    hot_tokens = np.nonzero((ids_all == hot).any(1))[0][:4]
    sample = np.concatenate([np.random.default_rng(2).choice(cfg.T, 20, replace=False), hot_tokens])
    st = check_forward(lt, x, OL=OL, sample=np.unique(sample))
    print(f"[prefill_mxfp4] {st}", flush=True)


def test_ep_share_primitives_with_triples():
    cfg = W.get_config("c4")
    print("[ep8_share_fp8] building layer", flush=True)
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    tok, exp, gate = W.make_triples(cfg)
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
    assert dropped == 0
    assert np.array_equal(off.cpu().numpy(), off_r) and np.array_equal(pos.cpu().numpy(), pos_r)
    OL = oracle_layer(lt)
    rng = np.random.default_rng(1)
    hot = np.bincount(tok, minlength=T)
    sample = np.concatenate([rng.choice(T, 16, replace=False), np.argsort(-hot)[:4], np.nonzero(hot == 0)[0][:2]])
    y_ref = oracle.forward_triples(OL, W.bf16_bits(x), tok, exp, gate, token_list=sample)
    err = rel_err_rows(to_np(y)[sample], y_ref)
    print(f"[ep8_share_fp8] max rel err {err.max():.3e} over {len(sample)} tokens", flush=True)
    assert err.max() < TOL["fp8"]
