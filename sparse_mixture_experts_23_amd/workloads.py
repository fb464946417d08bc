"""Seeded synthetic workloads for the sparse MoE layer forward.

This module only describes layer shapes and draws seeded random inputs; it
holds none of the layer's arithmetic.  Both the HIP path and the CPU oracle
receive the tensors it draws.

Shapes follow the model families the pages discuss:
  * tiny fp32 layer (d=64, m=128, E=8, k=2) for element-by-element checks;
  * Switch-style top-1 with capacity factor 1.25 ("MoE token routing", §6;
    "LLM from scratch" ch. 36 §36.2 Switch convention);
  * Mixtral-shaped layer d=4096, m=14336, E=8, k=2 ("MoE token routing", §4);
  * Qwen3-style many-expert layer E=128, k=8 ("MoE token routing", §4);
  * DeepSeek-V3-style E=256, k=8 plus one shared expert
    ("Sizzling MoE skewer analogy", DeepSeek-V3 table and formula).
Inputs: x ~ N(0,1); every projection ~ N(0, 1/fan_in) (fan_in = d for the
router, gate and up projections, m for the down projection).  bf16 tensors
are drawn in fp32 and rounded to bf16 (round-to-nearest-even, by torch).
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

GATE_RENORM = 0
GATE_SWITCH = 1


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    m: int
    E: int
    k: int
    dtype: str                    # "f32" or "bf16" (x and expert weights); router is fp32
    gate_mode: int                # GATE_RENORM or GATE_SWITCH
    cf: Optional[Tuple[int, int]]  # capacity factor num/den, None = unlimited
    bias: str = "none"            # "none" | "first_two_plus2" | "zipf"
    m_shared: int = 0
    renorm_form: str = "softmax_then_renorm"   # the oracle's literal weight form
    cfg_id: int = 0
    accept_by_gate: bool = False      # overflow variant: capacity competition by routing weight
    renorm_survivors: bool = False    # overflow variant: weights renormalised over accepted paths
    reroute: bool = False             # overflow variant: rejected paths go to the next-choice expert

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_tokens(self, T: int) -> "MoEConfig":
        return MoEConfig(**{**self.__dict__, "T": T})

    def scaled(self, **kw) -> "MoEConfig":
        return MoEConfig(**{**self.__dict__, **kw})


CONFIGS = {
    "tiny_fp32": MoEConfig("tiny_fp32", T=128, d=64, m=128, E=8, k=2, dtype="f32",
                           gate_mode=GATE_RENORM, cf=None, cfg_id=1),
    "switch_top1": MoEConfig("switch_top1", T=1024, d=1024, m=4096, E=8, k=1, dtype="bf16",
                             gate_mode=GATE_SWITCH, cf=(5, 4), bias="first_two_plus2", cfg_id=2),
    "mixtral": MoEConfig("mixtral", T=4096, d=4096, m=14336, E=8, k=2, dtype="bf16",
                         gate_mode=GATE_RENORM, cf=None, renorm_form="topk_then_softmax", cfg_id=3),
    "qwen3_like": MoEConfig("qwen3_like", T=8192, d=4096, m=1536, E=128, k=8, dtype="bf16",
                            gate_mode=GATE_RENORM, cf=(5, 4), bias="zipf", cfg_id=4),
    "dsv3_like": MoEConfig("dsv3_like", T=4096, d=7168, m=2048, E=256, k=8, dtype="bf16",
                           gate_mode=GATE_RENORM, cf=None, m_shared=2048, cfg_id=5),
}

BASE_SEED = 2023

# tensor ids used in the seed of each tensor
_TID = dict(x=0, w_r=1, w_gate=2, w_up=3, w_down=4, s_gate=5, s_up=6, s_down=7)


def _gen(cfg: MoEConfig, tensor: str, seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((BASE_SEED * 1000003 + cfg.cfg_id) * 1000003 + seed) * 64 + _TID[tensor])
    return g


def _normal(shape, std, gen, device, dtype, chunk_rows=None):
    """N(0, std^2) drawn in fp32 then rounded to `dtype`; chunked along dim 0
    to bound fp32 temporaries for very large weight tensors."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    step = n0 if chunk_rows is None else max(1, chunk_rows)
    for i in range(0, n0, step):
        j = min(n0, i + step)
        tmp = torch.randn((j - i,) + tuple(shape[1:]), generator=gen, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        out[i:j].copy_(tmp)
    return out


def router_bias(cfg: MoEConfig, device="cpu") -> Optional[torch.Tensor]:
    """Router bias as the workload defines it (fp32), or None."""
    if cfg.bias == "none":
        return None
    if cfg.bias == "first_two_plus2":
        b = torch.zeros(cfg.E, dtype=torch.float32)
        b[:2] = 2.0
        return b.to(device)
    if cfg.bias == "zipf":
        b = torch.tensor([1.5 * math.log(1.0 / (e + 1)) for e in range(cfg.E)],
                         dtype=torch.float64).to(torch.float32)
        return b.to(device)
    raise ValueError(cfg.bias)


@dataclass
class MoEInputs:
    cfg: MoEConfig
    x: torch.Tensor          # [T, d]   cfg dtype
    w_r: torch.Tensor        # [E, d]   fp32
    b_r: Optional[torch.Tensor]  # [E] fp32 or None
    w_gate: torch.Tensor     # [E, m, d] cfg dtype
    w_up: torch.Tensor       # [E, m, d]
    w_down: torch.Tensor     # [E, d, m]
    s_gate: Optional[torch.Tensor] = None   # [m_s, d]
    s_up: Optional[torch.Tensor] = None     # [m_s, d]
    s_down: Optional[torch.Tensor] = None   # [d, m_s]


def make_inputs(cfg: MoEConfig, seed: int = 0, device="cpu") -> MoEInputs:
    dt = cfg.torch_dtype
    T, d, m, E = cfg.T, cfg.d, cfg.m, cfg.E
    per_expert = max(1, (1 << 26) // max(1, m * d))  # ~256 MiB fp32 temporaries
    x = _normal((T, d), 1.0, _gen(cfg, "x", seed, device), device, dt)
    w_r = _normal((E, d), 1.0 / math.sqrt(d), _gen(cfg, "w_r", seed, device), device, torch.float32)
    w_gate = _normal((E, m, d), 1.0 / math.sqrt(d), _gen(cfg, "w_gate", seed, device), device, dt, per_expert)
    w_up = _normal((E, m, d), 1.0 / math.sqrt(d), _gen(cfg, "w_up", seed, device), device, dt, per_expert)
    w_down = _normal((E, d, m), 1.0 / math.sqrt(m), _gen(cfg, "w_down", seed, device), device, dt, per_expert)
    inp = MoEInputs(cfg, x, w_r, router_bias(cfg, device), w_gate, w_up, w_down)
    if cfg.m_shared:
        ms = cfg.m_shared
        inp.s_gate = _normal((ms, d), 1.0 / math.sqrt(d), _gen(cfg, "s_gate", seed, device), device, dt)
        inp.s_up = _normal((ms, d), 1.0 / math.sqrt(d), _gen(cfg, "s_up", seed, device), device, dt)
        inp.s_down = _normal((d, ms), 1.0 / math.sqrt(ms), _gen(cfg, "s_down", seed, device), device, dt)
    return inp
