"""Registry of the synthetic layer workloads (shapes, input distributions, quantizer).

Five workloads, numbered 1..5:

1. a single 256x256 fp32 layer, 2048 tokens of correlated Gaussian
   activations with 4 outlier channels x20; 4-bit asymmetric, per-row,
   natural order.
2. OPT-125m-shaped fp16 layers (768x768, 3072x768, 768x3072); 262144 tokens
   of Student-t(4) activations, 1% outlier channels x30; 4-bit, group 128.
3. LLaMA-7B-shaped bf16 layers (4096x4096, 11008x4096, 4096x11008); 262144
   tokens Student-t(4), 0.5% outlier channels x50; 4-bit, group 128,
   act-order.  The 4096x11008 "down" layer is the headline shape.
4. LLaMA-13B-shaped bf16 layers (5120x5120, 13824x5120, 5120x13824); same
   activations; 3-bit and 2-bit, group 64, act-order, packed.
5. OPT-175B-shaped fp16 block (12288-wide q/k/v/out, 49152x12288 fc1,
   12288x49152 fc2), quantized in sequence; X0 Student-t(4) with 0.1%
   outlier channels x100; 3-bit, group 128.

All use block 128 and damp 0.01.  Token count 128 sequences x 2048 = 262144
except workload 1 (2048).
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Quant:
    bits: int = 4
    group_size: int = 128
    sym: bool = False
    act_order: bool = False
    block: int = 128
    damp: float = 0.01


@dataclasses.dataclass(frozen=True)
class Workload:
    config: int
    name: str
    dtype: str
    sigma_w: float
    dist: str
    outlier_frac: float
    outlier_scale: float
    n_tok: int
    layers: tuple           # (name, d_out, d_in, x_layer)
    quants: tuple           # one or more Quant


N_TOK = 128 * 2048

WORKLOADS = {
    1: Workload(1, "single-256", "f32", 0.02, "gauss_mix", 4 / 256, 20.0, 2048,
                (("fc", 256, 256, 0),),
                (Quant(bits=4, group_size=-1, act_order=False),)),
    2: Workload(2, "opt-125m", "f16", 0.02, "t4", 0.01, 30.0, N_TOK,
                (("q", 768, 768, 0), ("k", 768, 768, 0), ("v", 768, 768, 0),
                 ("out", 768, 768, 3), ("fc1", 3072, 768, 4), ("fc2", 768, 3072, 5)),
                (Quant(bits=4, group_size=128, act_order=False),)),
    3: Workload(3, "llama-7b", "bf16", 0.02, "t4", 0.005, 50.0, N_TOK,
                (("q", 4096, 4096, 0), ("k", 4096, 4096, 0), ("v", 4096, 4096, 0),
                 ("o", 4096, 4096, 3), ("gate", 11008, 4096, 4), ("up", 11008, 4096, 4),
                 ("down", 4096, 11008, 6)),
                (Quant(bits=4, group_size=128, act_order=True),)),
    4: Workload(4, "llama-13b", "bf16", 0.02, "t4", 0.005, 50.0, N_TOK,
                (("q", 5120, 5120, 0), ("gate", 13824, 5120, 4), ("down", 5120, 13824, 6)),
                (Quant(bits=3, group_size=64, act_order=True),
                 Quant(bits=2, group_size=64, act_order=True))),
    5: Workload(5, "opt-175b-block", "f16", 0.01, "t4", 0.001, 100.0, N_TOK,
                (("q", 12288, 12288, 0), ("k", 12288, 12288, 0), ("v", 12288, 12288, 0),
                 ("out", 12288, 12288, 3), ("fc1", 49152, 12288, 4), ("fc2", 12288, 49152, 5)),
                (Quant(bits=3, group_size=128, act_order=False),)),
}

# The shape the headline metric is quoted on: workload 3's down projection.
HEADLINE = (3, "down")


def layer_spec(config: int, name: str):
    wl = WORKLOADS[config]
    for i, (n, d_out, d_in, xl) in enumerate(wl.layers):
        if n == name:
            return wl, i, d_out, d_in, xl
    raise KeyError(name)
