"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module draws random numbers and nothing else: it holds none of the
sharded step's arithmetic (no chunking, packing, reduction or optimizer math).
Values follow the workloads' stated distributions, with the second parameter of
N(mean, s) read as the standard deviation:

* fp32 master shards ~ N(0, 0.02);
* gradient contributions drawn in fp32 ~ N(0, 1e-3), then handed to torch's
  own library cast to bfloat16 (round to nearest even) so the inputs are bf16;
* all-gather rows: bf16 of N(0, 0.02);
* padding slots of a synthetic [N, S] buffer hold the sentinel 0x7FC1 (a quiet
  NaN), so any read of padding shows up in the outputs.

Every draw is keyed by a tuple (config, group, role, rank-or-source, step, ...)
hashed to a 63-bit seed, so each input is reproducible on its own.  A torch
generator on the requested device makes the numbers: CPU draws for the sizes the
oracle checks whole, device draws for the full-size workloads (the oracle then
reads back only the sampled inputs it needs).
"""
from __future__ import annotations

import hashlib

import torch

ROLE_MASTER = 0
ROLE_GRAD = 1
ROLE_AG = 2
ROLE_FULLW = 3
ROLE_STATE = 4

SENTINEL_BF16 = 0x7FC1


def seed_for(*key) -> int:
    h = hashlib.blake2b(repr(tuple(key)).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _gen(key, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(*key))
    return g


def normal_f32(n: int, std: float, key, device="cpu") -> torch.Tensor:
    """n fp32 draws from N(0, std), seeded by ``key``."""
    out = torch.randn(int(n), generator=_gen(key, device), device=device,
                      dtype=torch.float32)
    out.mul_(std)
    return out


def normal_bf16_bits(n: int, std: float, key, device="cpu") -> torch.Tensor:
    """n bfloat16 draws (as int16 bit patterns) of N(0, std), seeded by ``key``."""
    return normal_f32(n, std, key, device).to(torch.bfloat16).view(torch.int16)


def fill_normal_bf16_bits_(dst: torch.Tensor, std: float, key,
                           chunk: int = 1 << 28) -> torch.Tensor:
    """Fill an int16 device tensor with bf16 draws in bounded-size chunks."""
    flat = dst.view(-1)
    n = flat.numel()
    for i, s in enumerate(range(0, n, chunk)):
        e = min(n, s + chunk)
        flat[s:e] = normal_bf16_bits(e - s, std, tuple(key) + (i,), dst.device)
    return dst


def fill_normal_f32_(dst: torch.Tensor, std: float, key,
                     chunk: int = 1 << 28) -> torch.Tensor:
    flat = dst.view(-1)
    n = flat.numel()
    for i, s in enumerate(range(0, n, chunk)):
        e = min(n, s + chunk)
        flat[s:e] = normal_f32(e - s, std, tuple(key) + (i,), dst.device)
    return dst


def bf16_bits_to_u16(t: torch.Tensor):
    """int16 bit patterns -> numpy uint16 (host copy)."""
    return t.detach().cpu().numpy().view("uint16")
