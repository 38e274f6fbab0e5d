"""Workload shapes for the any-precision MoE expert layer.

Pure data: experts, hidden/intermediate sizes, top-k, token count and the
per-expert bitwidth recipe.  The shapes stand in for the three MoE models the
PagedWeight summary measures on (a 60-expert Qwen1.5-MoE-A2.7B, the 8-expert
Mixtral-8x7B and a 128-expert fine-grained model; zhichai.net page, section
"数据说话"); the sizes themselves are not given by the pages and are fixed here.

Nothing in this module computes any part of the layer.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

# Bitwidths an expert may run at: the nested 3/4/5/6-bit any-precision codes and
# the plain fp16 fallback (zhichai.net page, section "核心洞察").
VALID_BITS = (3, 4, 5, 6, 16)
N_PLANES = 6          # every quantized matrix stores all six bit-planes
LUT_BITS = (3, 4, 5, 6)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    E: int                      # routed experts
    H: int                      # hidden size
    I: int                      # expert SwiGLU intermediate size
    k: int                      # top-k
    T: int                      # tokens in the batch
    bits_mode: str              # "fixed" | "uniform" | "planner_zipf"
    bits: Optional[Tuple[int, ...]] = None   # for bits_mode == "fixed"
    logit_scale: float = 1.0
    router_bias: Optional[str] = None        # None | "zipf"
    zipf_s: float = 1.1
    shared_I: int = 0           # intermediate size of an always-on fp16 expert (0 = none)
    x_std: float = 1.0
    w_std: float = 0.02         # router, LUT draws and fp16 weights
    note: str = ""

    @property
    def slots(self) -> int:
        return self.T * self.k

    def with_tokens(self, T: int) -> "LayerConfig":
        return replace(self, T=T, name=f"{self.name.rsplit('_t', 1)[0]}_t{T}")


CONFIGS = {
    # Tiny single layer: every bitwidth present twice, launch-bound.
    "tiny": LayerConfig("tiny", E=8, H=256, I=512, k=2, T=16, bits_mode="fixed",
                        bits=(3, 4, 5, 6, 3, 4, 5, 6)),
    # Qwen1.5-MoE-A2.7B-shaped decode step: 60 experts, Zipf(1.1) routing skew
    # through a router bias, bitwidths chosen by the greedy planner, plus one
    # always-on fp16 shared expert.
    "qwen_decode": LayerConfig("qwen_decode", E=60, H=2048, I=1408, k=4, T=64,
                               bits_mode="planner_zipf", router_bias="zipf",
                               shared_I=5632),
    # Mixtral-8x7B-shaped decode at 1, 8 and 32 tokens; expert 0 is fp16.
    "mixtral_decode_t1": LayerConfig("mixtral_decode_t1", E=8, H=4096, I=14336, k=2, T=1,
                                     bits_mode="fixed", bits=(16, 6, 6, 5, 4, 4, 3, 3)),
    "mixtral_decode_t8": LayerConfig("mixtral_decode_t8", E=8, H=4096, I=14336, k=2, T=8,
                                     bits_mode="fixed", bits=(16, 6, 6, 5, 4, 4, 3, 3)),
    "mixtral_decode_t32": LayerConfig("mixtral_decode_t32", E=8, H=4096, I=14336, k=2, T=32,
                                      bits_mode="fixed", bits=(16, 6, 6, 5, 4, 4, 3, 3)),
    # 128 fine-grained experts, logits scaled by 4, bitwidths uniform over 3..6.
    "e128_decode": LayerConfig("e128_decode", E=128, H=2816, I=704, k=8, T=256,
                               bits_mode="uniform", logit_scale=4.0),
    # Mixtral-shaped prefill, about 2048 tokens per expert.
    "mixtral_prefill": LayerConfig("mixtral_prefill", E=8, H=4096, I=14336, k=2, T=8192,
                                   bits_mode="fixed", bits=(6, 6, 5, 5, 4, 4, 3, 3)),
}

# Order in which the five published workloads are listed.
CONFIG_ORDER = ("tiny", "qwen_decode", "mixtral_decode_t1", "mixtral_decode_t8",
                "mixtral_decode_t32", "e128_decode", "mixtral_prefill")


def custom(name: str, E: int, H: int, I: int, k: int, T: int, bits, **kw) -> LayerConfig:
    """A small fixed-bitwidth layer for tests (several tiles plus ragged tails)."""
    return LayerConfig(name, E=E, H=H, I=I, k=k, T=T, bits_mode="fixed",
                       bits=tuple(int(b) for b in bits), **kw)


def get(name: str) -> LayerConfig:
    return CONFIGS[name]
