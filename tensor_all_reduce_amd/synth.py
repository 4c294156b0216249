"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the reduction's arithmetic: it only draws seeded
random numbers and converts them to bf16 bit patterns with PyTorch's own
float32 -> bfloat16 conversion (a library routine).  Both the HIP path and the
CPU oracle consume what it returns; neither is imported here.

Value distributions (stand-ins for the activations the pages reduce; no
dataset or model weights are involved):

* ``normal``  -- N(0, 1), the decode and prefill hidden-state workloads;
* ``logmag``  -- sign * 2**U with U ~ Uniform[-8, 8] and a fair sign bit,
  magnitudes spread over 16 binades to stress fp32 accumulation;
* ``integers`` -- uniform integers in [lo, hi]; small enough that every
  partial sum is exact in bf16, so any reduction order gives the same bits.

Host generation uses ``numpy.random.default_rng(seed_words)``; device
generation (full-size bench inputs) uses a seeded ``torch.Generator`` on the
GPU.  Host and device draws are different streams and are never mixed.
"""
from __future__ import annotations

import numpy as np
import torch


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def rng(*seed_words: int) -> np.random.Generator:
    return np.random.default_rng([int(s) for s in seed_words])


def normal(n: int, *seed_words: int) -> np.ndarray:
    """n bf16 bit patterns of N(0,1) samples."""
    return _f32_to_bf16_bits(rng(*seed_words).standard_normal(n, dtype=np.float32))


def logmag(n: int, *seed_words: int) -> np.ndarray:
    """n bf16 bit patterns of sign * 2**U, U ~ Uniform[-8, 8]."""
    g = rng(*seed_words)
    u = g.uniform(-8.0, 8.0, n)
    sign = np.where(g.integers(0, 2, n) == 1, -1.0, 1.0)
    return _f32_to_bf16_bits((sign * np.exp2(u)).astype(np.float32))


def integers(n: int, lo: int, hi: int, *seed_words: int) -> np.ndarray:
    """n bf16 bit patterns of integers drawn uniformly from [lo, hi]."""
    v = rng(*seed_words).integers(lo, hi + 1, n).astype(np.float32)
    return _f32_to_bf16_bits(v)


def rank_buffers(kind: str, P: int, n: int, *seed_words: int) -> list[np.ndarray]:
    """P rank buffers; rank p is drawn from seed (*seed_words, p)."""
    out = []
    for p in range(P):
        if kind == "normal":
            out.append(normal(n, *seed_words, p))
        elif kind == "logmag":
            out.append(logmag(n, *seed_words, p))
        elif kind == "integers":
            out.append(integers(n, -16, 16, *seed_words, p))
        else:
            raise ValueError(f"unknown distribution {kind!r}")
    return out


def device_rank_buffers(kind: str, P: int, n: int, seed: int, device="cuda") -> list[torch.Tensor]:
    """P bf16 tensors of n elements drawn on the GPU from a seeded generator.

    Used where host generation of several GiB would dominate the run time.
    Returns contiguous ``torch.bfloat16`` tensors.
    """
    g = torch.Generator(device=device)
    out = []
    for p in range(P):
        g.manual_seed(int(seed) * 1000003 + p)
        if kind == "normal":
            x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
        elif kind == "logmag":
            u = torch.rand(n, generator=g, device=device, dtype=torch.float32) * 16.0 - 8.0
            s = torch.randint(0, 2, (n,), generator=g, device=device, dtype=torch.int8)
            x = torch.exp2(u) * (1.0 - 2.0 * s.to(torch.float32))
            del u, s
        else:
            raise ValueError(f"unknown distribution {kind!r}")
        out.append(x.to(torch.bfloat16))
        del x
    return out
