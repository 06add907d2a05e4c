"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no re-layout arithmetic: it only makes flat buffers of a
given element count.  Both the HIP path and the CPU oracle consume the same
bytes, so the generator cannot affect parity.

* ``normal_bf16``: N(0, 1) drawn in float32 from a seeded CPU generator, then
  rounded to bfloat16 (round-to-nearest-even), as the attention activations
  of the Llama/Qwen models the pages train are bf16 when training in mixed
  precision.
* ``tags_int32``: consecutive int32 tags ``base, base+1, ...``.  Every element
  is unique, so an output element names the input element it came from.

Seeds of the four activation buffers: Q = 0, K = 1, V = 2, O = 3.
"""
from __future__ import annotations

import torch

SEED_Q, SEED_K, SEED_V, SEED_O = 0, 1, 2, 3


def tensor_numel(B: int, S: int, H: int, d: int) -> int:
    """Elements of one activation tensor over all ranks: B sequences of S
    tokens, H heads of d channels."""
    return B * S * H * d


def normal_bf16(numel: int, seed: int) -> torch.Tensor:
    """Flat CPU bfloat16 tensor of N(0, 1) samples from ``seed``."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return torch.randn(numel, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def tags_int32(numel: int, base: int = 0, device: str = "cpu") -> torch.Tensor:
    """Flat int32 tensor ``base .. base+numel-1`` (on ``device``)."""
    if base < 0 or base + numel > 2**31:
        raise ValueError("int32 tags must lie in [0, 2^31)")
    return torch.arange(base, base + numel, dtype=torch.int32, device=device)


def all_bf16_patterns() -> torch.Tensor:
    """All 65536 bfloat16 bit patterns (NaN payloads, +-0, +-inf, subnormals),
    in a seeded random order."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(65536)
    perm = torch.randperm(65536, generator=gen)
    return (perm.to(torch.int32) - 32768).to(torch.int16).view(torch.bfloat16)


def raw_bits(t: torch.Tensor):
    """NumPy view of a CPU tensor's raw bits (uint16 for 2-byte, uint32 for
    4-byte types): what the oracle consumes."""
    import numpy as np
    t = t.contiguous()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise ValueError("unsupported element size %d" % t.element_size())
