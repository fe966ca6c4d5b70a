"""GPU parity of moe_backward (bf16 experts) against the fp64 oracle.

Every gradient is compared block by block with the inf-norm relative error
max |gpu - ref| / max |ref| (dx per token; dW_gate_up, dW_down and dW_router
per expert; the shared expert's gradients and dbias as whole tensors) against
the bf16 tolerance of the layer, 2e-2.  Gradients the mathematics makes zero
(an expert that receives no token; the router when k = 1) must be exactly 0.
The GPU takes the forward's ids and gates (moe_forward on the same x); the
oracle recomputes the gates from x in fp64.

Small layers: every gradient against oracle.backward.  The training workload
(8192 tokens at the full Step-5 shape, the launch the benchmark times): dx of
sampled tokens (oracle.backward, dx only), the weight gradients of the least
and the most loaded expert (oracle.expert_weight_grads), and two identities
of the softmax backward that hold at any size: each token's logit gradients
sum to zero, so the bias gradients and the router-weight gradients summed
over experts vanish.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from router_gemm_amd import binding as B
from router_gemm_amd import workloads as W

from conftest import gpu_available
from gpu_util import dev, oracle_layer, rel_err_rows, run_forward

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

TOL = 2e-2   # bf16 tolerance (inf-norm relative)


def _print(*a):
    print(*a, flush=True)


def _rel(a, ref):
    den = np.abs(ref).max(initial=0.0)
    if den == 0:
        return float(np.abs(a).max(initial=0.0))   # must be exactly 0
    return float(np.abs(a - ref).max() / den)


def _outputs(cfg, T, device):
    nan = float("nan")
    f = lambda *s: torch.full(s, nan, dtype=torch.float32, device=device)
    return dict(dx=f(T, cfg.H), dw_gate_up=f(cfg.E, 2 * cfg.I, cfg.H), dw_down=f(cfg.E, cfg.H, cfg.I),
                dw_shared_gate_up=f(2 * cfg.Is, cfg.H) if cfg.Is else None,
                dw_shared_down=f(cfg.H, cfg.Is) if cfg.Is else None,
                dw_router=f(cfg.E, cfg.H), dbias=f(cfg.E))


def run_backward(lt, x, dy, ids, gates, ws=None, z_saved=None):
    cfg = lt.cfg
    layer = B.Layer.from_tensors(lt)
    T = x.shape[0]
    out = _outputs(cfg, T, x.device)
    ws = B.backward_workspace(layer, T, x.device) if ws is None else ws
    B.moe_backward(layer, x, T, ids, gates, dy, z_saved=z_saved, ws=ws, **out)
    torch.cuda.synchronize()
    return out


def run_forward_train(lt, x):
    """moe_forward_train -> (y f32, ids, gates, z_saved)."""
    cfg = lt.cfg
    layer = B.Layer.from_tensors(lt)
    T = x.shape[0]
    y = torch.empty((T, cfg.H), dtype=torch.float32, device=x.device)
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device=x.device)
    gates = torch.empty((T, cfg.k), dtype=torch.float32, device=x.device)
    z = torch.full((B.moe_saved_z_floats(layer, T),), float("nan"), dtype=torch.float32, device=x.device)
    B.moe_forward_train(layer, x, T, y, ids, gates, z, ws=B.workspace(layer, T, T * cfg.k, x.device))
    torch.cuda.synchronize()
    return y, ids, gates, z


def _np(t):
    return None if t is None else t.cpu().numpy().astype(np.float64)


def _cfg(base, **kw):
    return dataclasses.replace(W.get_config(base), **kw)


def check_small(cfg, saved=False):
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    dy = W.make_dy(cfg, dev())
    y, ids, gates = run_forward(lt, x)
    z = None
    if saved:   # the training forward: same outputs, plus the pre-activations
        y2, ids2, gates2, z = run_forward_train(lt, x)
        assert torch.equal(y, y2) and torch.equal(ids, ids2) and torch.equal(gates, gates2)
    out = {k: _np(v) for k, v in run_backward(lt, x, dy, ids, gates, z_saved=z).items()}
    OL = oracle_layer(lt)
    ref = oracle.backward(OL, W.bf16_bits(x), ids.cpu().numpy(), W.bf16_bits(dy))
    errs = {}
    errs["dx"] = float(rel_err_rows(out["dx"], ref["dx"]).max())
    used = np.bincount(ids.cpu().numpy().ravel(), minlength=cfg.E) > 0
    for name in ("dw_gate_up", "dw_down", "dw_router"):
        per = [_rel(out[name][e], ref[name][e]) for e in range(cfg.E)]
        errs[name] = max(per)
        for e in np.nonzero(~used)[0]:
            assert not out[name][e].any(), (name, e)      # no token: exactly zero
    errs["dbias"] = _rel(out["dbias"], ref["dbias"])
    if cfg.Is:
        errs["dw_shared_gate_up"] = _rel(out["dw_shared_gate_up"], ref["dw_shared_gate_up"])
        errs["dw_shared_down"] = _rel(out["dw_shared_down"], ref["dw_shared_down"])
    _print(cfg.name, "saved z" if saved else "recomputed z", "T", cfg.T, "unused experts", int((~used).sum()),
           {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v < TOL, (k, v)
    if cfg.k == 1:   # one chosen logit: the gate is 1 and the router gets no gradient
        assert not out["dw_router"].any() and not out["dbias"].any()
    return out


@pytest.mark.parametrize("saved", [False, True])
def test_backward_small_full_parity(saved):
    check_small(W.get_config("small_bf16"), saved)


@pytest.mark.parametrize("saved", [False, True])
def test_backward_ragged_tiles_bias_and_unused_experts(saved):
    # H = 3 x 128, I = 2.5 column tiles, 200 tokens, Zipf-biased router (bias
    # gradient checked), 40 experts of which several get no token
    check_small(_cfg("small_bf16", name="bwd_ragged", T=200, H=384, E=40, k=3, I=320, Is=128,
                     zipf_s=1.1, zipf_beta=0.6, router_std=1.0 / np.sqrt(384)), saved)


@pytest.mark.parametrize("saved", [False, True])
def test_backward_k1_no_shared_expert_single_token_tiles(saved):
    check_small(_cfg("small_bf16", name="bwd_k1", T=37, E=64, k=1, Is=0), saved)


def test_forward_train_tiled_path_saves_pre_activations():
    # 2048 tokens over 16 experts: the training forward takes the LDS-tiled
    # expert kernels (rows read through the sort permutation)
    check_small(_cfg("small_bf16", name="bwd_tiled", T=2048, E=16, k=2, I=256, Is=128), True)


def test_backward_deterministic_and_zero_tokens():
    cfg = W.get_config("small_bf16")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    dy = W.make_dy(cfg, dev())
    _, ids, gates = run_forward(lt, x)
    a = run_backward(lt, x, dy, ids, gates)
    ws = B.backward_workspace(B.Layer.from_tensors(lt), cfg.T, dev())
    ws.fill_(0x5A)
    b = run_backward(lt, x, dy, ids, gates, ws=ws)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    # T == 0: no-op, outputs untouched
    layer = B.Layer.from_tensors(lt)
    out = _outputs(cfg, 1, dev())
    B.moe_backward(layer, x, 0, ids, gates, dy, ws=None, **out)
    torch.cuda.synchronize()
    assert torch.isnan(out["dx"]).all()


@pytest.mark.parametrize("saved", [True, False])
def test_backward_training_workload_sampled(saved):
    """The training workload at full size (moe_forward_train then moe_backward
    with the saved pre-activations, the benchmark's step; and with the
    recompute): dx of sampled tokens, weight gradients of the least and most
    loaded experts, softmax identities."""
    cfg = W.get_config("train_bf16")
    _print("case", cfg.name, "T", cfg.T, "saved z" if saved else "recomputed z")
    lt = W.make_layer(cfg, dev())
    x = W.make_x(cfg, dev())
    dy = W.make_dy(cfg, dev())
    if saved:
        y, ids, gates, z = run_forward_train(lt, x)
    else:
        (y, ids, gates), z = run_forward(lt, x), None
    out = run_backward(lt, x, dy, ids, gates, z_saved=z)
    del z
    for k, v in out.items():
        if v is not None:
            assert not torch.isnan(v).any(), k
    OL = oracle_layer(lt)
    xb, dyb, idn = W.bf16_bits(x), W.bf16_bits(dy), ids.cpu().numpy()
    tl = np.array([0, 1, cfg.T // 2 + 3, cfg.T - 1])
    # the training forward's own output (moe_forward_train, or moe_forward for
    # the recompute case) on the sampled tokens plus two of the most loaded
    # expert's tokens, against the oracle with the same ids
    hot = np.bincount(idn.ravel(), minlength=cfg.E).argmax()
    tly = np.unique(np.concatenate([tl, np.nonzero((idn == hot).any(1))[0][:2]]))
    y_ref = oracle.forward_with_ids(OL, xb, idn[tly], token_list=tly)
    e_y = rel_err_rows(_np(y)[tly], y_ref)
    _print(cfg.name, "forward y max rel err", f"{e_y.max():.2e}", "over", len(tly), "tokens")
    assert e_y.max() < TOL
    assert e_y.max() < 2e-3              # regression bar (observed 6.9e-4)
    ref = oracle.backward(OL, xb, idn, dyb, token_list=tl, weights=False)
    e_dx = rel_err_rows(out["dx"][torch.from_numpy(tl).to(dev())].cpu().numpy(), ref["dx"])
    load = np.bincount(idn.ravel(), minlength=cfg.E)
    errs = {"dx": float(e_dx.max())}
    for e in (int(load.argmin()), int(load.argmax())):
        dgu, dd = oracle.expert_weight_grads(OL, xb, idn, dyb, e)
        errs[f"dw_gate_up[{e}] ({load[e]} rows)"] = _rel(_np(out["dw_gate_up"][e]), dgu)
        errs[f"dw_down[{e}]"] = _rel(_np(out["dw_down"][e]), dd)
    db = _np(out["dbias"])
    dwr = _np(out["dw_router"])
    errs["sum dbias / sum |dbias|"] = abs(db.sum()) / np.abs(db).sum()
    errs["col sums dW_router"] = float((np.abs(dwr.sum(0)) / np.abs(dwr).sum(0)).max())
    _print(cfg.name, "loads", int(load.min()), int(load.max()), {k: f"{v:.2e}" for k, v in errs.items()})
    for k, v in errs.items():
        assert v < (1e-4 if k.startswith(("sum", "col")) else TOL), (k, v)
