"""Seeded synthetic workloads for the MoE layer forward.

This module only draws random inputs; it holds none of the layer's
arithmetic.  The same tensors feed the HIP library and, in tests, the CPU
oracle.

The five main presets follow the workloads the pages describe: the LSTM
language model layer with thousands of experts (positions flattened into one
batch), its two-level variant, a Switch-style top-1 router with expert
capacity and a fine-grained routed-expert layer with a gated (SwiGLU) FFN.  A
sixth gives the fine-grained layer the sigmoid gate with a selection-only bias
and one always-active shared expert of the routed experts' width.  No dataset
is used; every tensor is a seeded draw:

* x ~ N(0, 1); gate and expert weights ~ N(0, 1/fan_in) (variance);
* noise ~ N(0, 1) per (token, expert), supplied as a tensor;
* per-expert logit bias: N(0, 0.5) variance (LM layer), N(0, 1) (Switch),
  or Zipf(1.1) as b_i = -1.1 ln(rank_i) over a seeded rank permutation;
* bf16 expert weights are fp32 draws rounded once to bf16.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import torch

GATE_TOPK_SOFTMAX = 0
GATE_SWITCH_TOP1 = 1
GATE_SIGMOID_BIAS = 2
ACT_RELU = 0
ACT_SWIGLU = 1
DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_FP8 = 2   # the library packs the bf16 draws into E4M3 codes with per-row scales


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d_model: int
    d_hidden: int
    n_experts: int
    k: int
    gate: int = GATE_TOPK_SOFTMAX
    act: int = ACT_RELU
    expert_dtype: int = DTYPE_BF16
    noisy: bool = True
    capacity_factor: float = 0.0
    w_importance: float = 0.1
    w_load: float = 0.1
    alpha_switch: float = 1.0
    w_z: float = 1.0           # router z-loss weight (1: the raw mean statistic)
    w_entropy: float = 1.0     # gate-entropy loss weight
    d_hidden_shared: int = 0   # shared expert's hidden width (0: none)
    n_groups: int = 0          # hierarchical: a
    k_groups: int = 0          # hierarchical: k1 (k = k1 * k2)
    logit_bias: str = "none"   # none | normal0.5 | normal1 | zipf1.1
    zero_expert_bias: bool = False
    expert_bias_std: float = 0.0  # > 0: ReLU expert biases b1, b2 ~ N(0, std^2)
    seed: int = 1000

    @property
    def hierarchical(self) -> bool:
        return self.n_groups > 0

    @property
    def b(self) -> int:
        return self.n_experts // self.n_groups if self.n_groups else self.n_experts

    @property
    def k2(self) -> int:
        return self.k // self.k_groups if self.k_groups else self.k

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


PRESETS = {
    "tiny_f32": MoEConfig("tiny_f32", T=512, d_model=64, d_hidden=128, n_experts=16, k=2,
                          expert_dtype=DTYPE_F32, zero_expert_bias=True, seed=1001),
    "lm_layer": MoEConfig("lm_layer", T=8192, d_model=512, d_hidden=1024, n_experts=256, k=4,
                          logit_bias="normal0.5", seed=1002),
    "hierarchical": MoEConfig("hierarchical", T=16384, d_model=512, d_hidden=1024,
                              n_experts=4096, k=4, n_groups=64, k_groups=2, seed=1003),
    "switch_cf": MoEConfig("switch_cf", T=32768, d_model=768, d_hidden=3072, n_experts=128, k=1,
                           gate=GATE_SWITCH_TOP1, noisy=False, capacity_factor=1.25,
                           logit_bias="normal1", seed=1004),
    "fine_swiglu": MoEConfig("fine_swiglu", T=4096, d_model=7168, d_hidden=2048, n_experts=256,
                             k=8, act=ACT_SWIGLU, noisy=False, logit_bias="zipf1.1", seed=1005),
    "lm_layer_fp8": MoEConfig("lm_layer_fp8", T=8192, d_model=512, d_hidden=1024, n_experts=256,
                              k=4, expert_dtype=DTYPE_FP8, logit_bias="normal0.5", seed=1002),
    "fine_swiglu_fp8": MoEConfig("fine_swiglu_fp8", T=4096, d_model=7168, d_hidden=2048,
                                 n_experts=256, k=8, act=ACT_SWIGLU, expert_dtype=DTYPE_FP8,
                                 noisy=False, logit_bias="zipf1.1", seed=1005),
    "sigmoid_shared": MoEConfig("sigmoid_shared", T=4096, d_model=7168, d_hidden=2048,
                                n_experts=256, k=8, act=ACT_SWIGLU, gate=GATE_SIGMOID_BIAS,
                                noisy=False, logit_bias="normal0.5", d_hidden_shared=2048,
                                seed=1006),
}
CONFIG_ORDER = ["tiny_f32", "lm_layer", "hierarchical", "switch_cf", "fine_swiglu"]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & ((1 << 63) - 1))
    return g


def _normal(shape, std, device, seed):
    return torch.randn(shape, generator=_gen(device, seed), device=device,
                       dtype=torch.float32) * std


def _derived(seed, tensor_id, e=0):
    return seed * (1 << 32) + tensor_id * (1 << 16) + e


def _logit_bias(cfg: MoEConfig, n: int, device):
    if cfg.logit_bias == "none":
        return None
    if cfg.logit_bias == "normal0.5":
        return _normal((n,), math.sqrt(0.5), device, _derived(cfg.seed, 4))
    if cfg.logit_bias == "normal1":
        return _normal((n,), 1.0, device, _derived(cfg.seed, 4))
    if cfg.logit_bias == "zipf1.1":
        g = _gen("cpu", _derived(cfg.seed, 4))
        ranks = torch.randperm(n, generator=g).to(torch.float64) + 1.0
        return (-1.1 * torch.log(ranks)).to(torch.float32).to(device)
    raise ValueError(cfg.logit_bias)


def make_inputs(cfg: MoEConfig, device="cpu", T: int | None = None):
    """All layer inputs for ``cfg`` as torch tensors on ``device``.

    Returns a dict with x, w_gate, b_gate, w_noise, noise, (w_gate2, w_noise2,
    noise2 for the hierarchical preset), w1, w3, w2, b1, b2, (ws1, ws3, ws2 of
    the shared expert).  Absent inputs are None.  Expert weights are drawn per (tensor, expert) with derived seeds, in
    bf16 when the preset's experts are bf16.
    """
    T = cfg.T if T is None else T
    d, h, n = cfg.d_model, cfg.d_hidden, cfg.n_experts
    s = cfg.seed
    out = {}
    out["x"] = _normal((T, d), 1.0, device, _derived(s, 1))
    n_gate = cfg.n_groups if cfg.hierarchical else n
    out["w_gate"] = _normal((n_gate, d), 1.0 / math.sqrt(d), device, _derived(s, 2))
    out["w_noise"] = (_normal((n_gate, d), 1.0 / math.sqrt(d), device, _derived(s, 3))
                      if cfg.noisy else None)
    out["b_gate"] = _logit_bias(cfg, n_gate, device)
    out["noise"] = _normal((T, n_gate), 1.0, device, _derived(s, 5)) if cfg.noisy else None
    if cfg.hierarchical:
        a, b, k1 = cfg.n_groups, cfg.b, cfg.k_groups
        out["w_gate2"] = _normal((a, b, d), 1.0 / math.sqrt(d), device, _derived(s, 6))
        out["w_noise2"] = (_normal((a, b, d), 1.0 / math.sqrt(d), device, _derived(s, 7))
                           if cfg.noisy else None)
        out["noise2"] = _normal((T, k1, b), 1.0, device, _derived(s, 8)) if cfg.noisy else None
    wdt = torch.float32 if cfg.expert_dtype == DTYPE_F32 else torch.bfloat16

    def experts(tensor_id, shape, fan_in):
        buf = torch.empty((n,) + shape, dtype=wdt, device=device)
        for e in range(n):
            buf[e] = _normal(shape, 1.0 / math.sqrt(fan_in), device,
                             _derived(s, tensor_id, e)).to(wdt)
        return buf

    out["w1"] = experts(10, (h, d), d)
    out["w3"] = experts(11, (h, d), d) if cfg.act == ACT_SWIGLU else None
    out["w2"] = experts(12, (d, h), h)
    hs = cfg.d_hidden_shared
    if hs:
        out["ws1"] = _normal((hs, d), 1.0 / math.sqrt(d), device, _derived(s, 13)).to(wdt)
        out["ws3"] = (_normal((hs, d), 1.0 / math.sqrt(d), device, _derived(s, 14)).to(wdt)
                      if cfg.act == ACT_SWIGLU else None)
        out["ws2"] = _normal((d, hs), 1.0 / math.sqrt(hs), device, _derived(s, 15)).to(wdt)
    if cfg.zero_expert_bias:
        out["b1"] = torch.zeros((n, h), dtype=torch.float32, device=device)
        out["b2"] = torch.zeros((n, d), dtype=torch.float32, device=device)
    elif cfg.expert_bias_std > 0:
        out["b1"] = _normal((n, h), cfg.expert_bias_std, device, _derived(s, 16))
        out["b2"] = _normal((n, d), cfg.expert_bias_std, device, _derived(s, 17))
    else:
        out["b1"] = None
        out["b2"] = None
    return out


def make_grad_inputs(cfg: MoEConfig, device="cpu", T: int | None = None):
    """Upstream gradients for the backward pass: dy ~ N(0, 1) [T, d] and
    dlosses ~ N(0, 1) [5] (one per auxiliary loss)."""
    T = cfg.T if T is None else T
    dy = _normal((T, cfg.d_model), 1.0, device, _derived(cfg.seed, 20))
    dlosses = _normal((5,), 1.0, device, _derived(cfg.seed, 21))
    return dy, dlosses


def to_numpy64(t):
    """Host float64 copy of an input tensor (None passes through)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()
