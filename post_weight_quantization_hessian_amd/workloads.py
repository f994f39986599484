"""The five layer workloads (shapes, calibration size, bit widths, groups).

Layers that read the same input share one Hessian; they are quantized
together by stacking their rows (rows are independent given the Hessian).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Layer:
    name: str
    rows: int          # output channels
    hessian: str       # name of the input it reads
    outlier_frac: float = 0.0


@dataclass(frozen=True)
class HessianInput:
    name: str
    dim: int
    kind: str = "cone"            # "cone" or "silu_gated"
    lognormal_sigma: float = 0.0


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    inputs: tuple
    layers: tuple
    n_tokens: int
    token_chunk: int
    bits: tuple
    group_size: int
    act_order: bool
    damp: float = 0.01
    notes: str = field(default="", compare=False)

    def input(self, name):
        for h in self.inputs:
            if h.name == name:
                return h
        raise KeyError(name)

    def layers_of(self, hname):
        return [l for l in self.layers if l.hessian == hname]

    def weights_per_step(self):
        return sum(l.rows * self.input(l.hessian).dim for l in self.layers) * len(self.bits)


WORKLOADS = {
    "smollm_q576": Workload(
        0, "smollm_q576",
        inputs=(HessianInput("x", 576),),
        layers=(Layer("q_proj", 576, "x"),),
        n_tokens=2048, token_chunk=2048, bits=(4,), group_size=128, act_order=False,
        notes="576x576 q_proj, 2048 tokens, 4-bit g128, no act-order"),
    "qwen05b_mlp": Workload(
        1, "qwen05b_mlp",
        inputs=(HessianInput("mlp_in", 896), HessianInput("down_in", 4864, kind="silu_gated")),
        layers=(Layer("gate_proj", 4864, "mlp_in"), Layer("up_proj", 4864, "mlp_in"),
                Layer("down_proj", 896, "down_in")),
        n_tokens=2048, token_chunk=2048, bits=(4,), group_size=128, act_order=False,
        notes="Qwen2.5-0.5B MLP shapes, 2048 tokens, 4-bit g128"),
    "tinyllama_block": Workload(
        2, "tinyllama_block",
        inputs=(HessianInput("attn_in", 2048), HessianInput("o_in", 2048),
                HessianInput("mlp_in", 2048), HessianInput("down_in", 5632)),
        layers=(Layer("q_proj", 2048, "attn_in"), Layer("k_proj", 256, "attn_in"),
                Layer("v_proj", 256, "attn_in"), Layer("o_proj", 2048, "o_in"),
                Layer("gate_proj", 5632, "mlp_in"), Layer("up_proj", 5632, "mlp_in"),
                Layer("down_proj", 2048, "down_in")),
        n_tokens=2048, token_chunk=2048, bits=(4, 3), group_size=128, act_order=True,
        notes="TinyLlama-1.1B block, 2048 tokens, 4-bit and 3-bit g128, act-order"),
    "llama8b_down": Workload(
        3, "llama8b_down",
        inputs=(HessianInput("down_in", 14336),),
        layers=(Layer("down_proj", 4096, "down_in", outlier_frac=0.001),),
        n_tokens=131072, token_chunk=8192, bits=(3,), group_size=128, act_order=True,
        notes="8B-shape down_proj 4096x14336, 0.1% outlier input columns x20, "
              "131072 tokens streamed in 8192-token chunks, 3-bit g128, act-order"),
    "llama70b_down": Workload(
        4, "llama70b_down",
        inputs=(HessianInput("down_in", 28672, lognormal_sigma=1.0),),
        layers=(Layer("down_proj", 8192, "down_in"),),
        n_tokens=65536, token_chunk=65536, bits=(2, 4), group_size=64, act_order=True,
        notes="70B-shape down_proj 8192x28672, 65536 tokens with log-normal channel "
              "scales, 2-bit and 4-bit g64, act-order, one H/U for both widths"),
}

ORDER = ["smollm_q576", "qwen05b_mlp", "tinyllama_block", "llama8b_down", "llama70b_down"]
