"""The five workloads of the W4A16 linear path, as data.

Layer shapes (K, N) are fused projections of Llama-3.1-8B (QKV 4096x6144,
O 4096x4096, gate+up 4096x28672, down 14336x4096) and Qwen3-4B (QKV
2560x6144, O 4096x2560, gate+up 2560x19456, down 9728x2560), the two model
families the W4A16 pages tune their tiles on.  Token counts M mirror the
pages' decode (one token per step) and prompt lengths (128 and 1920).
"""
from __future__ import annotations

import dataclasses
from typing import Iterator

F16 = 0
BF16 = 1


@dataclasses.dataclass(frozen=True)
class Layer:
    K: int
    N: int


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    layers: tuple
    Ms: tuple
    groups: tuple
    symmetric: tuple      # tuple of bools to cover
    dtypes: tuple
    bias: tuple           # tuple of bools to cover


LLAMA_DECODE = (Layer(4096, 6144), Layer(4096, 4096), Layer(4096, 28672), Layer(14336, 4096))
QWEN_DECODE = (Layer(2560, 6144), Layer(4096, 2560), Layer(2560, 19456), Layer(9728, 2560))
LLAMA_PREFILL = (Layer(4096, 6144), Layer(4096, 28672), Layer(14336, 4096))
SWEEP = (Layer(4096, 14336), Layer(28672, 4096))

CONFIGS = {
    "tiny": Config("tiny", (Layer(256, 256),), (1,), (32,), (True,), (F16,), (False,)),
    "llama8b_decode": Config("llama8b_decode", LLAMA_DECODE, (1, 2, 3, 4, 5), (128,),
                             (False,), (BF16,), (False,)),
    "qwen3_4b_decode": Config("qwen3_4b_decode", QWEN_DECODE, (1, 2, 4), (128,),
                              (True,), (F16,), (False, True)),
    "llama8b_prefill": Config("llama8b_prefill", LLAMA_PREFILL, (128, 1920), (128,),
                              (False,), (BF16,), (False,)),
    "sweep": Config("sweep", SWEEP, (1, 2, 4, 5, 8, 16, 32, 64, 128, 256), (32, 64, 128),
                    (True, False), (F16, BF16), (False,)),
}


def config_cases(name: str) -> Iterator[dict]:
    """Every (layer, M, group, symmetric, dtype, bias) point of one config."""
    c = CONFIGS[name]
    for li, layer in enumerate(c.layers):
        for g in c.groups:
            for sym in c.symmetric:
                for dt in c.dtypes:
                    for b in c.bias:
                        for M in c.Ms:
                            yield dict(config=name, layer=li, K=layer.K, N=layer.N, M=M,
                                       group=g, symmetric=sym, dtype=dt, bias=b)
