"""The five synthetic workloads the sharded step is tested and timed on.

Shapes only: every config is a list of parameter groups (one group per
``fully_shard`` call, registered bottom-up so the root group holds what is left
over) with parameters in registration order, a simulated world size N and the
AdamW hyperparameters.  Nothing here computes any part of the method.

Sources of the shapes (cited by page title and section):

* "Sharded Training: FSDP2, DTensor, Tensor and Pipeline Parallelism"
  (course module 27), the ZeroRedundancyOptimizer paragraph: the two-rank probe
  on Linear(16, 32) -> Linear(32, 4); the fully_shard paragraph: one group per
  call, blocks first, then the root with embeddings, final norm and LM head;
  the lab: AdamW at lr 3e-4, a (1, 32) head with a (1,) bias.
* "Introduction to PyTorch FSDP2 Backend Features", section DTensor: a
  [4096, 4096] weight held as [512, 4096] per GPU on 8 ranks.
* "PyTorch FSDP2 Guide: Distributed LLM Training with DTensor", sections "The
  Problem" (LLaMA-3.1 70B state) and "Production Benchmarks" (Llama-3 70B on
  64 GPUs); irregular MoE experts in "The FlatParameter Monolith".

Where the task description of a config and its listed shapes disagree, the
listed shapes win (the MLP has 676 parameters, the 7B-shaped model with
ff = 14336 holds 1,005,879,808 parameters per rank at N = 8).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Tuple

Shape = Tuple[int, ...]


@dataclass(frozen=True)
class Param:
    name: str
    shape: Shape

    @property
    def rows(self) -> int:
        return self.shape[0]

    @property
    def cols(self) -> int:
        c = 1
        for d in self.shape[1:]:
            c *= d
        return c

    @property
    def numel(self) -> int:
        return self.rows * self.cols


@dataclass(frozen=True)
class Group:
    name: str
    params: Tuple[Param, ...]


@dataclass(frozen=True)
class AdamW:
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    world: int
    groups: Tuple[Group, ...]
    timing_rank: int = 0
    steps: int = 3
    hp: AdamW = field(default_factory=AdamW)
    master_std: float = 0.02
    grad_std: float = 1e-3

    @property
    def params(self) -> List[Param]:
        return [p for g in self.groups for p in g.params]

    @property
    def numel(self) -> int:
        return sum(p.numel for p in self.params)


def _g(name: str, *params: Tuple[str, Shape]) -> Group:
    return Group(name, tuple(Param(n, tuple(s)) for n, s in params))


def llama_block(prefix: str, d: int, ff: int, kv: int | None = None) -> Group:
    """One decoder block: attention norm, Wq/Wk/Wv/Wo, FFN norm, gate/up/down.

    nn.Linear stores (out_features, in_features); Shard(0) splits dim 0.
    """
    kv = d if kv is None else kv
    return _g(prefix,
              (f"{prefix}.attn_norm", (d,)),
              (f"{prefix}.wq", (d, d)),
              (f"{prefix}.wk", (kv, d)),
              (f"{prefix}.wv", (kv, d)),
              (f"{prefix}.wo", (d, d)),
              (f"{prefix}.ffn_norm", (d,)),
              (f"{prefix}.gate", (ff, d)),
              (f"{prefix}.up", (ff, d)),
              (f"{prefix}.down", (d, ff)))


def mlp_probe() -> Config:
    """Linear(16,32) -> Linear(32,4) with biases, N = 2, one group."""
    g = _g("root", ("0.weight", (32, 16)), ("0.bias", (32,)),
           ("1.weight", (4, 32)), ("1.bias", (4,)))
    return Config(0, "mlp-16-32-4 N=2", 2, (g,))


def llama_one_block(d: int = 4096, ff: int = 14336) -> Config:
    return Config(1, f"llama-block d={d} ff={ff} N=8", 8,
                  (llama_block("layers.0", d, ff),))


def llama_7b(ff: int = 14336, vocab: int = 32000, d: int = 4096,
             layers: int = 32) -> Config:
    groups = [llama_block(f"layers.{i}", d, ff) for i in range(layers)]
    groups.append(_g("root", ("tok_embeddings", (vocab, d)), ("norm", (d,)),
                     ("output", (vocab, d))))
    return Config(2, f"llama-7B-shaped d={d} ff={ff} L={layers} N=8", 8,
                  tuple(groups))


def moe_ragged(experts: int = 64, d: int = 2048, ffe: int = 1408,
               vocab: int = 32001) -> Config:
    """Ragged MoE-style groups at N = 6.

    The MoE group holds, per expert, gate/up [1408, 2048], down [2048, 1408]
    and a down bias [2048]; then the router [64, 2048], two norms [2048] and a
    (1, 2048) head with a (1,) bias, which leave ranks 1..5 with empty
    chunks.  The root group holds the embedding [32001, 2048] and final norm.
    Timing is quoted for rank 5, which owns short last chunks and two empty
    ones.
    """
    ps = []
    for e in range(experts):
        ps += [(f"moe.experts.{e}.gate", (ffe, d)),
               (f"moe.experts.{e}.up", (ffe, d)),
               (f"moe.experts.{e}.down", (d, ffe)),
               (f"moe.experts.{e}.down_bias", (d,))]
    ps += [("moe.router", (experts, d)), ("moe.norm_in", (d,)),
           ("moe.norm_out", (d,)), ("moe.head", (1, d)), ("moe.head_bias", (1,))]
    moe = _g("moe", *ps)
    root = _g("root", ("tok_embeddings", (vocab, d)), ("norm", (d,)))
    return Config(3, "moe-ragged 64x(1408x2048) N=6", 6, (moe, root), timing_rank=5)


def llama_70b(layers: int = 80, d: int = 8192, kv: int = 1024, ff: int = 28672,
              vocab: int = 128256) -> Config:
    groups = [llama_block(f"layers.{i}", d, ff, kv) for i in range(layers)]
    groups.append(_g("root", ("tok_embeddings", (vocab, d)), ("norm", (d,)),
                     ("output", (vocab, d))))
    return Config(4, f"llama-70B-shaped d={d} GQA kv={kv} ff={ff} L={layers} N=64",
                  64, tuple(groups))


def get(index: int) -> Config:
    return [mlp_probe, llama_one_block, llama_7b, moe_ragged, llama_70b][index]()


ALL = (0, 1, 2, 3, 4)
