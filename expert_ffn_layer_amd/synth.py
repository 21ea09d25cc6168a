"""Seeded synthetic MoE layers: shapes, value distributions and draw order.

This module only draws random tensors.  It holds none of the layer's
arithmetic (no routing, no FFN), so that both the CPU oracle and the GPU path
can be fed the same inputs from it without sharing any computation.

Shapes follow the models the source pages discuss:

* Qwen 3.5-397B (pwwt.cn, "Qwen 3.5 on Ironwood" §2.1 and §4.2): hidden size
  4096, 512 routed experts, top-k 10.
* Ling-2.6-1T (lumevalley.com, SGLang-JAX Ling-2.6-1T article, opening
  paragraph): 256 routed experts, top-8, plus one always-on shared expert.

The pages give no expert intermediate size and no value distributions; the
ones used here are fixed below.

Storage layout (the "Linear" convention, [out_features, in_features]):

* ``x``      [T, H]        activations
* ``wg``     [H, E] fp32   router projection (logits = x @ wg + bias)
* ``w_gu``   [E, 2I, H]    rows 0..I-1 are W_gate^T, rows I..2I-1 are W_up^T
* ``w_dn``   [E, H, I]     W_down^T
* ``ws_gu``  [2I_s, H], ``ws_dn`` [H, I_s]  shared expert (optional)

Every weight entry is an independent normal draw, so storing the transpose of
the [H, I] / [I, H] math-layout matrices does not change the distribution.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# Zipf bias strength for the hot-expert workload.  Chosen so that the top 10%
# of experts receive ~60% of the routed assignments at seed 0; found by
# oracle/calibrate_skew.py (bisection over the oracle's router) and frozen
# here so that generating inputs never runs any routing arithmetic.
SKEW_ZIPF_S = 1.2
SKEW_ALPHA = 0.508


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    I_shared: int = 0
    x_std: float = 1.0
    wg_std: float = 0.02
    w_std: float = 0.02
    fp32_values: bool = False      # tiny case: values drawn and kept in fp32
    zipf_s: float = 0.0            # > 0: add a Zipf(s) log-bias to the logits
    zipf_alpha: float = 0.0
    renorm: int = 1

    @property
    def A(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "LayerConfig":
        return dataclasses.replace(self, T=T)


CONFIGS = {
    # Tiny layer, fp32 throughout: seeds the oracle's own checks.
    "tiny": LayerConfig("tiny", T=16, H=64, E=8, k=2, I=32,
                        wg_std=0.1, w_std=0.05, fp32_values=True),
    # One decode step at concurrency 64 on Qwen-3.5-like dims: HBM-bound on
    # streaming the touched experts' weights.
    "decode": LayerConfig("decode", T=64, H=4096, E=512, k=10, I=1024),
    # Prefill chunk of 8192 tokens on the same dims.
    "prefill": LayerConfig("prefill", T=8192, H=4096, E=512, k=10, I=1024),
    # Same dims at 32768 tokens: ~640 rows per expert, MFMA-bound FFN.
    "prefill_long": LayerConfig("prefill_long", T=32768, H=4096, E=512, k=10, I=1024),
    # Ling-like: 256 experts, top-8, I=2048, plus one shared expert.
    "ling": LayerConfig("ling", T=4096, H=8192, E=256, k=8, I=2048, I_shared=2048),
    # Hot-expert skew on the decode dims, Zipf(1.2) log-bias on the logits.
    "skew": LayerConfig("skew", T=4096, H=4096, E=512, k=10, I=1024,
                        zipf_s=SKEW_ZIPF_S, zipf_alpha=SKEW_ALPHA),
}


def workload_name(cfg: LayerConfig) -> str:
    s = f"{cfg.name}_T{cfg.T}_H{cfg.H}_E{cfg.E}_k{cfg.k}_I{cfg.I}"
    if cfg.I_shared:
        s += f"_Is{cfg.I_shared}"
    return s


@dataclasses.dataclass
class Layer:
    cfg: LayerConfig
    x: torch.Tensor
    wg: torch.Tensor
    bias: Optional[torch.Tensor]
    w_gu: torch.Tensor
    w_dn: torch.Tensor
    ws_gu: Optional[torch.Tensor] = None
    ws_dn: Optional[torch.Tensor] = None

    def to(self, device) -> "Layer":
        f = lambda t: None if t is None else t.to(device)
        return Layer(self.cfg, f(self.x), f(self.wg), f(self.bias), f(self.w_gu),
                     f(self.w_dn), f(self.ws_gu), f(self.ws_dn))

    def rounded_to_bf16(self) -> "Layer":
        """Activations and expert weights rounded (RNE) to bf16; router stays fp32."""
        f = lambda t: None if t is None else t.to(torch.bfloat16)
        return Layer(self.cfg, f(self.x), self.wg, self.bias, f(self.w_gu),
                     f(self.w_dn), f(self.ws_gu), f(self.ws_dn))


def zipf_bias(E: int, s: float, alpha: float, gen: torch.Generator,
              device) -> torch.Tensor:
    """Log-Zipf(s) bias over a seeded random ranking of the expert ids.

    Expert with rank r (1 = hottest) gets alpha * log(r^-s).
    """
    ranks = torch.randperm(E, generator=gen, device=gen.device).to(device) + 1
    return (-alpha * s) * torch.log(ranks.to(torch.float64)).to(torch.float32)


def make_layer(cfg: LayerConfig | str, seed: int = 0, device="cpu",
               router_only: bool = False) -> Layer:
    """Draw one layer.

    Two generators, so that the routing of a given seed is the same whichever
    device holds the experts:

    * a CPU generator seeded ``seed`` draws x, wg and (skew workloads) the
      Zipf ranking, in that order;
    * a generator on ``device`` seeded ``seed + 1`` draws, per expert, the
      gate|up block then the down block, then the shared expert.

    Values are fp32 draws scaled by the stated standard deviation, then
    rounded to bf16 (round-to-nearest-even) unless ``cfg.fp32_values``.
    ``router_only`` stops after the router inputs (expert tensors empty).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    dev = torch.device(device)
    cpu_gen = torch.Generator(device="cpu")
    cpu_gen.manual_seed(seed)
    wdt = torch.float32 if cfg.fp32_values else torch.bfloat16

    def draw(gen, shape, std, dtype):
        t = torch.randn(shape, generator=gen, device=gen.device, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t if dtype == torch.float32 else t.to(dtype)

    x = draw(cpu_gen, (cfg.T, cfg.H), cfg.x_std, wdt).to(dev)
    wg = draw(cpu_gen, (cfg.H, cfg.E), cfg.wg_std, torch.float32).to(dev)
    bias = None
    if cfg.zipf_s > 0:
        bias = zipf_bias(cfg.E, cfg.zipf_s, cfg.zipf_alpha, cpu_gen, dev)
    if router_only:
        empty = torch.empty((0,), dtype=wdt, device=dev)
        return Layer(cfg, x, wg, bias, empty, empty)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 1)
    w_gu = torch.empty((cfg.E, 2 * cfg.I, cfg.H), dtype=wdt, device=dev)
    w_dn = torch.empty((cfg.E, cfg.H, cfg.I), dtype=wdt, device=dev)
    for e in range(cfg.E):
        w_gu[e] = draw(gen, (2 * cfg.I, cfg.H), cfg.w_std, wdt)
        w_dn[e] = draw(gen, (cfg.H, cfg.I), cfg.w_std, wdt)
    ws_gu = ws_dn = None
    if cfg.I_shared:
        ws_gu = draw(gen, (2 * cfg.I_shared, cfg.H), cfg.w_std, wdt)
        ws_dn = draw(gen, (cfg.H, cfg.I_shared), cfg.w_std, wdt)
    return Layer(cfg, x, wg, bias, w_gu, w_dn, ws_gu, ws_dn)


def custom_config(name="custom", **kw) -> LayerConfig:
    return LayerConfig(name, **kw)
