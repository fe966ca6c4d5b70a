"""Seeded synthetic workloads for the routed MoE layer (inputs only).

This module draws inputs and nothing else: it holds none of the layer's
arithmetic (no routing, grouping, FFN or combine).  Both the HIP path and the
fp64 oracle consume the bytes it produces.

Shapes follow the Step-5-Preview MoE layer ("Step-5-Preview", NeMo AutoModel
model coverage, section "Model Architecture": hidden 4,096, 352 routed
experts, top-8, one shared expert, expert intermediate 1,536) plus a scaled
-down case.  Expert weights are bf16, or OCP E4M3 with one fp32 scale per
128x128 block ("Step-5 minimal inference", introduction: block-scaled FP8
expert GEMM; section "Install": FP8 E4M3).

Recipe (all draws seeded):
  * small tensors (x, router, router bias, shared expert, pre-routed triples)
    come from numpy PCG64 streams keyed by (seed, stream id), so they are the
    same bytes whichever device the layer is built on;
  * routed expert weights (up to 13 GB) come from torch's generator on the
    target device, one generator per (expert, matrix) keyed by the seed;
  * every value is drawn in fp32 and rounded to bf16 (nearest even), or, for
    fp8 experts, scaled per 128x128 block by s = amax/448 and rounded to E4M3,
    or, for MX FP4 experts, given one power-of-two scale per 32 inputs of a
    row and rounded to E2M1 (see quantize_mxfp4).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int                 # tokens
    H: int                 # hidden
    E: int                 # routed experts held by this GPU
    k: int                 # top-k (0 for pre-routed triples)
    I: int                 # routed expert intermediate
    Is: int                # shared expert intermediate (0 = none)
    expert_dtype: str      # "bf16" | "fp8" | "mxfp4"
    router_std: float      # std of the router weights
    expert_std: float = 0.02
    zipf_s: float = 0.0    # > 0: router bias skews loads by Zipf(s) ranks
    zipf_beta: float = 0.0 # strength of that bias (see zipf_bias)
    triples: int = 0       # > 0: number of pre-routed (token, expert, gate) triples
    dense: bool = False    # a dense SwiGLU FF layer: one "expert" applied to every token
    seed: int = 0
    description: str = ""

    @property
    def N(self) -> int:
        return self.triples if self.triples else self.T * self.k


# The Zipf strength for the prefill case: chosen once (bisection on seed 0
# with this module's x and router draws) so that the hottest expert receives
# about 10x the mean number of rows under top-8 routing.
_ZIPF_BETA_PREFILL = 0.2436

CONFIGS = {
    "small_bf16": MoEConfig(
        "small_bf16", T=128, H=512, E=32, k=4, I=192, Is=192, expert_dtype="bf16",
        router_std=1.0 / math.sqrt(512),
        description="scaled-down MoE layer, bf16, T=128, H=512, 32 experts top-4, I=192"),
    "small_fp8": MoEConfig(
        "small_fp8", T=200, H=512, E=16, k=4, I=256, Is=128, expert_dtype="fp8",
        router_std=1.0 / math.sqrt(512),
        description="scaled-down MoE layer, FP8 experts, T=200 (ragged), H=512, 16 experts top-4, I=256"),
    "decode_bf16": MoEConfig(
        "decode_bf16", T=64, H=4096, E=352, k=8, I=1536, Is=1536, expert_dtype="bf16",
        router_std=1.0 / 64,
        description="Step-5 MoE layer, bf16 experts, decode T=64, unbiased router"),
    "decode_fp8": MoEConfig(
        "decode_fp8", T=64, H=4096, E=352, k=8, I=1536, Is=1536, expert_dtype="fp8",
        router_std=1.0 / 64,
        description="Step-5 MoE layer, FP8 E4M3 experts (128x128 block scales), decode T=64"),
    "prefill_fp8": MoEConfig(
        "prefill_fp8", T=8192, H=4096, E=352, k=8, I=1536, Is=1536, expert_dtype="fp8",
        router_std=1.0 / 64, zipf_s=1.1, zipf_beta=_ZIPF_BETA_PREFILL,
        description="Step-5 MoE layer, FP8 experts, prefill T=8192, Zipf(1.1)-biased router"),
    "ep8_share_fp8": MoEConfig(
        "ep8_share_fp8", T=16384, H=4096, E=44, k=0, I=1536, Is=1536, expert_dtype="fp8",
        router_std=1.0 / 64, zipf_s=1.1, triples=16384,
        description="one rank's EP=8 share: 44 FP8 experts, 16384 pre-routed Zipf(1.1) "
                    "triples, bf16 shared expert on 16384 tokens"),
    "small_mxfp4": MoEConfig(
        "small_mxfp4", T=136, H=512, E=16, k=4, I=256, Is=128, expert_dtype="mxfp4",
        router_std=1.0 / math.sqrt(512),
        description="scaled-down MoE layer, MX FP4 experts, T=136, H=512, 16 experts top-4, I=256"),
    "decode_mxfp4": MoEConfig(
        "decode_mxfp4", T=64, H=4096, E=352, k=8, I=1536, Is=1536, expert_dtype="mxfp4",
        router_std=1.0 / 64,
        description="Step-5 MoE shape with MX FP4 expert weights (E2M1, E8M0 per 32), decode T=64"),
    "prefill_mxfp4": MoEConfig(
        "prefill_mxfp4", T=8192, H=4096, E=352, k=8, I=1536, Is=1536, expert_dtype="mxfp4",
        router_std=1.0 / 64, zipf_s=1.1, zipf_beta=_ZIPF_BETA_PREFILL,
        description="the prefill layer with MX FP4 experts, T=8192, Zipf(1.1)-biased router"),
    "dense_ff_bf16": MoEConfig(
        "dense_ff_bf16", T=8192, H=4096, E=1, k=1, I=13824, Is=0, expert_dtype="bf16",
        router_std=1.0 / 64, dense=True,
        description="the model's dense SwiGLU FF layers (0-2 and 91): intermediate 13824, bf16, "
                    "8192 tokens, as one expert through moe_expert_ffn"),
    "train_bf16": MoEConfig(
        "train_bf16", T=8192, H=4096, E=352, k=8, I=1536, Is=1536, expert_dtype="bf16",
        router_std=1.0 / 64,
        description="training step of the Step-5 MoE layer in BF16 (forward + backward), one "
                    "8192-token sequence, unbiased router on random inputs (near-balanced loads)"),
}
# Short aliases by position in the workload list.
def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return dataclasses.replace(cfg, **overrides) if overrides else cfg


# ----------------------------------------------------------------- draws

def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def _bf16_bits(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy array -> torch bfloat16 (round to nearest even), CPU."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def quantize_blocks_e4m3(w: torch.Tensor):
    """Input-side weight quantiser: [R, C] fp32 -> (uint8 e4m3 codes [R,C], fp32 [R/128, C/128]).

    Scale s = amax(block)/448 (1 for an all-zero block); code = e4m3(w/s),
    clamped to the finite range first.  This prepares stored weights the way
    a block-scaled FP8 checkpoint holds them; it is not part of the layer.
    """
    R, Cc = w.shape
    assert R % 128 == 0 and Cc % 128 == 0
    blk = w.float().reshape(R // 128, 128, Cc // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / s[:, None, :, None]).clamp(-448.0, 448.0).reshape(R, Cc)
    return q.to(torch.float8_e4m3fn).view(torch.uint8), s.contiguous()


# E2M1 magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7).  Rounding to
# nearest: a magnitude goes to code i when it lies between the midpoints
# around value i; at a midpoint the even code wins (ties to even).
_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (0.75, 1.75, 3.5)   # midpoints whose even neighbour is the upper code


def quantize_mxfp4(w: torch.Tensor):
    """Input-side weight quantiser to OCP MX FP4: [R, C] fp32 ->
    (uint8 [R, C/2]: two E2M1 codes per byte, input 2j in the low nibble of
    byte j; uint8 [R, C/32]: E8M0 scale bytes).

    Per 32 inputs of a row: the scale is 2^(floor(log2 amax) - 2) (E2M1's
    largest exponent is 2), byte = exponent + 127 clamped to [0, 254] (127
    for an all-zero block); code = E2M1(w / scale), nearest with ties to
    even, magnitudes above 6 saturated to 6.  This prepares stored weights
    the way an MX checkpoint holds them; it is not part of the layer.
    """
    R, Cc = w.shape
    assert Cc % 32 == 0
    blk = w.float().reshape(R, Cc // 32, 32)
    amax = blk.abs().amax(dim=2)
    _, ex = torch.frexp(amax)                  # amax = m * 2^ex, m in [0.5, 1)
    e = ex.to(torch.int32) - 1 - 2             # floor(log2 amax) - 2
    sbyte = torch.where(amax > 0, (e + 127).clamp(0, 254), torch.full_like(e, 127))
    scale = torch.exp2((sbyte - 127).float())
    v = (blk / scale[..., None]).abs().clamp(max=6.0)
    mid = torch.tensor(_E2M1_MID, dtype=torch.float32, device=w.device)
    code = torch.bucketize(v, mid, right=False)
    for t in _E2M1_TIE_UP:
        code = code + (v == t).to(code.dtype)
    code = code | (((blk < 0) & (code > 0)).to(code.dtype) << 3)
    code = code.to(torch.uint8).reshape(R, Cc)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    return packed.contiguous(), sbyte.to(torch.uint8).contiguous()


def zipf_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    """Per-expert router bias: b_e = -beta * s * ln(r_e), r = seeded permutation of 1..E."""
    if cfg.zipf_s <= 0 or cfg.triples:
        return None
    ranks = _rng(cfg.seed, 3).permutation(cfg.E) + 1
    return (-cfg.zipf_beta * cfg.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)


@dataclasses.dataclass
class LayerTensors:
    cfg: MoEConfig
    w_router: torch.Tensor                 # bf16 [E,H]
    router_bias: Optional[torch.Tensor]    # f32 [E]
    w_gate_up: torch.Tensor                # bf16 or uint8(e4m3) [E,2I,H]; mxfp4: uint8 [E,2I,H/2]
    w_down: torch.Tensor                   # bf16 or uint8(e4m3) [E,H,I]; mxfp4: uint8 [E,H,I/2]
    s_gate_up: Optional[torch.Tensor]      # f32 [E,2I/128,H/128]; mxfp4: uint8 (E8M0) [E,2I,H/32]
    s_down: Optional[torch.Tensor]         # f32 [E,H/128,I/128]; mxfp4: uint8 (E8M0) [E,H,I/32]
    w_shared_gate_up: Optional[torch.Tensor]  # bf16 [2Is,H]
    w_shared_down: Optional[torch.Tensor]     # bf16 [H,Is]

    @property
    def fp8(self) -> bool:
        """Activations and h are stored as e4m3 + 1x128 scales (fp8 and mxfp4 experts)."""
        return self.cfg.expert_dtype != "bf16"

    @property
    def mx(self) -> bool:
        return self.cfg.expert_dtype == "mxfp4"


def _expert_gen(device, seed: int, e: int, which: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 1_000_003 + 7919) * 4099 + e * 2 + which) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def make_layer(cfg: MoEConfig, device="cpu") -> LayerTensors:
    """Draw the layer's weights on `device`."""
    dev = torch.device(device)
    E, H, I, Is = cfg.E, cfg.H, cfg.I, cfg.Is
    fp8 = cfg.expert_dtype == "fp8"
    mx = cfg.expert_dtype == "mxfp4"
    if fp8 or mx:
        assert H % 128 == 0 and I % 128 == 0, "fp8 and mxfp4 experts need H and I multiples of 128"
    w_router = _bf16_bits(_rng(cfg.seed, 2).standard_normal((E, H), dtype=np.float32)
                          * np.float32(cfg.router_std)).to(dev)
    b = zipf_bias(cfg)
    router_bias = None if b is None else torch.from_numpy(b).to(dev)
    wdt = torch.bfloat16 if not (fp8 or mx) else torch.uint8
    pk = 2 if mx else 1
    w_gu = torch.empty((E, 2 * I, H // pk), dtype=wdt, device=dev)
    w_d = torch.empty((E, H, I // pk), dtype=wdt, device=dev)
    s_gu = s_d = None
    if fp8:
        s_gu = torch.empty((E, 2 * I // 128, H // 128), dtype=torch.float32, device=dev)
        s_d = torch.empty((E, H // 128, I // 128), dtype=torch.float32, device=dev)
    elif mx:
        s_gu = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device=dev)
        s_d = torch.empty((E, H, I // 32), dtype=torch.uint8, device=dev)
    for e in range(E):
        for which, (shape, dst) in enumerate((((2 * I, H), w_gu), ((H, I), w_d))):
            w = torch.randn(shape, generator=_expert_gen(dev, cfg.seed, e, which), device=dev,
                            dtype=torch.float32) * cfg.expert_std
            if fp8 or mx:
                q, s = quantize_mxfp4(w) if mx else quantize_blocks_e4m3(w)
                dst[e].copy_(q)
                (s_gu if which == 0 else s_d)[e].copy_(s)
            else:
                dst[e].copy_(w.to(torch.bfloat16))
    wsg = wsd = None
    if Is > 0:
        wsg = (_bf16_bits(_rng(cfg.seed, 5).standard_normal((2 * Is, H), dtype=np.float32)
                          * np.float32(cfg.expert_std))).to(dev)
        wsd = (_bf16_bits(_rng(cfg.seed, 6).standard_normal((H, Is), dtype=np.float32)
                          * np.float32(cfg.expert_std))).to(dev)
    return LayerTensors(cfg, w_router, router_bias, w_gu, w_d, s_gu, s_d, wsg, wsd)


def make_x(cfg: MoEConfig, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Token activations x ~ N(0,1), bf16 [T,H]."""
    T = cfg.T if T is None else T
    return _bf16_bits(_rng(cfg.seed, 1).standard_normal((T, cfg.H), dtype=np.float32)).to(device)


def make_dy(cfg: MoEConfig, device="cpu", T: Optional[int] = None) -> torch.Tensor:
    """Gradient of the layer output for the backward, dy ~ N(0,1), bf16 [T,H]."""
    T = cfg.T if T is None else T
    return _bf16_bits(_rng(cfg.seed, 8).standard_normal((T, cfg.H), dtype=np.float32)).to(device)


def make_triples(cfg: MoEConfig):
    """Pre-routed assignments for one EP rank: (token int32 [N], expert int32 [N], gate f32 [N]).

    expert ~ Zipf(s) over ranks 1..E mapped through a seeded shuffle;
    token ~ U[0, T) with no repeated (token, expert) pair; gate ~ U(0, 1).
    The triples are in draw order (not sorted by token or expert).
    """
    assert cfg.triples > 0
    rng = _rng(cfg.seed, 7)
    N, E, T = cfg.triples, cfg.E, cfg.T
    p = np.arange(1, E + 1, dtype=np.float64) ** (-cfg.zipf_s)
    p /= p.sum()
    rank_to_expert = rng.permutation(E)
    expert = rank_to_expert[rng.choice(E, size=N, p=p)].astype(np.int32)
    token = rng.integers(0, T, size=N).astype(np.int32)
    for _ in range(100):
        key = token.astype(np.int64) * E + expert
        _, first = np.unique(key, return_index=True)
        dup = np.ones(N, dtype=bool)
        dup[first] = False
        if not dup.any():
            break
        token[dup] = rng.integers(0, T, size=int(dup.sum())).astype(np.int32)
    gate = rng.random(N, dtype=np.float32)
    gate = np.where(gate == 0, np.float32(0.5), gate).astype(np.float32)
    return token, expert, gate


def host_layer_arrays(lt: LayerTensors) -> dict:
    """numpy views (bit patterns) of a layer's tensors, for host-side consumers."""
    def bits(t):
        if t is None:
            return None
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()
    return dict(w_router=bits(lt.w_router), router_bias=bits(lt.router_bias),
                w_gate_up=bits(lt.w_gate_up), w_down=bits(lt.w_down),
                s_gate_up=bits(lt.s_gate_up), s_down=bits(lt.s_down),
                w_shared_gate_up=bits(lt.w_shared_gate_up), w_shared_down=bits(lt.w_shared_down))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
