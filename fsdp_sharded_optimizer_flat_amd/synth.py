"""Seeded synthetic inputs for the step: gradients and fp32 master weights.

Random numbers only -- this module holds none of the step's arithmetic.  The
same bytes feed both the HIP library and, in tests, the CPU oracle (tensors
are generated once and copied), so the generator itself need not agree
across devices.  Values: master ~ N(0, 0.02) in fp32; gradients ~ N(0, 1e-3)
or Student-t(3) x 1e-3 (Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3)), rounded to bf16
by torch's round-to-nearest-even cast, or kept in fp32.
"""
from __future__ import annotations

import torch

_CHUNK = 1 << 26   # elements generated per pass (256 MB of fp32 scratch)

# tags keep the streams of different tensors apart
TAG_MASTER, TAG_GRAD = 1, 2


def seed_of(base: int, tag: int, step: int = 0, rank: int = 0) -> int:
    x = (base * 1_000_003 + tag * 10_007 + step * 101 + rank) & ((1 << 62) - 1)
    return x


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


@torch.no_grad()
def fill_normal_(out: torch.Tensor, std: float, seed: int) -> torch.Tensor:
    """out (fp32 or bf16, contiguous) <- N(0, std^2), rounded to out's dtype."""
    g = _gen(out.device, seed)
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - s)
        tmp = torch.randn(n, generator=g, device=out.device, dtype=torch.float32)
        tmp.mul_(std)
        flat[s:s + n].copy_(tmp)
    return out


@torch.no_grad()
def fill_student_t3_(out: torch.Tensor, scale: float, seed: int) -> torch.Tensor:
    """out <- scale * Student-t with 3 degrees of freedom."""
    g = _gen(out.device, seed)
    flat = out.view(-1)
    for s in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - s)
        z = torch.randn(4, n, generator=g, device=out.device, dtype=torch.float32)
        chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
        t = z[0] / torch.sqrt(chi)
        t.mul_(scale)
        flat[s:s + n].copy_(t)
    return out


def fill_grad_(out: torch.Tensor, dist: str, scale: float, seed: int) -> torch.Tensor:
    if dist == "normal":
        return fill_normal_(out, scale, seed)
    if dist == "student_t3":
        return fill_student_t3_(out, scale, seed)
    raise ValueError(dist)


@torch.no_grad()
def zero_padding_(flat: torch.Tensor, unit_table) -> torch.Tensor:
    """Zero the padding of every unit in a GLOBAL flat buffer (the packer's
    contract: padding holds zeros in parameters, gradients and state).
    unit_table rows: numel, padded, shard, offset, local_offset."""
    for numel, padded, _shard, offset, _loff in unit_table:
        if padded > numel:
            flat[int(offset + numel):int(offset + padded)].zero_()
    return flat


@torch.no_grad()
def zero_padding_local_(shard_buf: torch.Tensor, unit_table, n_ranks: int, rank: int) -> torch.Tensor:
    """Zero the elements of rank `rank`'s LOCAL shard that are padding."""
    for numel, padded, shard, offset, loff in unit_table:
        if padded == numel:
            continue
        a = rank * shard                 # rank's slice, relative to the unit start
        lo, hi = max(a, numel), min(a + shard, padded)
        if lo < hi:
            shard_buf[int(loff + lo - a):int(loff + hi - a)].zero_()
    return shard_buf
