"""Seeded synthetic inputs for the AdamW / AMSGrad step.

This module is the only code shared by the oracle side and the HIP side of
the tests and the benchmark.  It holds random draws, dtype conversions of the
draws and parameter-list shapes -- none of the optimizer's arithmetic.

Every draw is keyed by a tuple (seed, workload, tensor, call, field) hashed
into an independent torch generator seed, so the same element always sees the
same value whichever side asks for it and whatever else was drawn before.
Gradients stored in 16 bits are rounded from FP32 draws to nearest-even by
torch's dtype conversion.
"""
from __future__ import annotations

import hashlib
from typing import Iterable

import numpy as np
import torch

GRAD_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def derive_seed(*key) -> int:
    """63-bit seed from an arbitrary tuple of ints/strings."""
    h = hashlib.blake2b(repr(key).encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & ((1 << 63) - 1)


def _generator(device, key) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(*key))
    return g


def normal(n: int, std: float, key, device="cpu", mean: float = 0.0) -> torch.Tensor:
    """FP32 N(mean, std^2) draws (std is the standard deviation)."""
    out = torch.empty(n, dtype=torch.float32, device=device)
    if n:
        out.normal_(mean, std, generator=_generator(device, key))
    return out


def uniform(n: int, lo: float, hi: float, key, device="cpu") -> torch.Tensor:
    out = torch.empty(n, dtype=torch.float32, device=device)
    if n:
        out.uniform_(lo, hi, generator=_generator(device, key))
    return out


def stored_grad(n: int, std: float, multiplier: float, gdt: str, key, device="cpu") -> torch.Tensor:
    """Gradient as stored by a mixed-precision backward: FP32 draw of N(0, std^2)
    times ``multiplier`` (the loss scale), rounded into the storage dtype."""
    x = normal(n, std, key, device)
    if multiplier != 1.0:
        x.mul_(multiplier)
    return x.to(GRAD_TORCH_DTYPES[gdt])


def grad_numpy(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a stored gradient: float32, or raw uint16 bits for 16-bit dtypes."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def steady_state(n: int, key, amsgrad: bool, device="cpu", m_std=1e-4, v_root_std=1e-3):
    """Pre-warmed moments: m ~ N(0, m_std^2), v = N(0, v_root_std^2)^2,
    v_max = v * U(1, 1.5) when AMSGrad is on."""
    m = normal(n, m_std, key + ("m",), device)
    v = normal(n, v_root_std, key + ("v",), device)
    v.mul_(v)
    vmax = None
    if amsgrad:
        vmax = uniform(n, 1.0, 1.5, key + ("vmax",), device).mul_(v)
    return m, v, vmax


def nonfinite_positions(total: int, k: int, key) -> np.ndarray:
    """k distinct positions in [0, total), seeded, sorted (sampling without
    replacement by rejection of repeats)."""
    rng = np.random.Generator(np.random.PCG64(derive_seed(*key)))
    chosen: set[int] = set()
    while len(chosen) < k:
        for x in rng.integers(0, total, size=k - len(chosen) + 16):
            if len(chosen) < k:
                chosen.add(int(x))
    return np.array(sorted(chosen), dtype=np.int64)


def nonfinite_values(k: int) -> list[float]:
    """Alternating +inf / NaN, the injected values."""
    return [float("inf") if i % 2 == 0 else float("nan") for i in range(k)]


# ---------------------------------------------------------------- shapes --

def decoder_1b_shapes(odd_norms: bool = False) -> list[tuple[str, int]]:
    """(name, numel) of a 1.1B-parameter decoder: d_model 2048, 22 layers,
    q/k/v/o 2048x2048, gate/up 2048x5632, down 5632x2048, two RMSNorm vectors
    per layer, 32000x2048 embedding and untied head, final norm.  With
    ``odd_norms`` the 45 norm vectors alternate 2047 / 2049 elements."""
    d, ff, vocab, layers = 2048, 5632, 32000, 22
    shapes = [("embed", vocab * d)]
    norm_i = 0

    def norm_size():
        nonlocal norm_i
        size = d if not odd_norms else (d - 1 if norm_i % 2 == 0 else d + 1)
        norm_i += 1
        return size

    for layer in range(layers):
        shapes.append((f"l{layer}.attn_norm", norm_size()))
        for proj in ("q", "k", "v", "o"):
            shapes.append((f"l{layer}.{proj}", d * d))
        shapes.append((f"l{layer}.ffn_norm", norm_size()))
        shapes.append((f"l{layer}.gate", d * ff))
        shapes.append((f"l{layer}.up", d * ff))
        shapes.append((f"l{layer}.down", ff * d))
    shapes.append(("final_norm", norm_size()))
    shapes.append(("head", vocab * d))
    return shapes


def decoder_7b_shapes() -> list[tuple[str, int]]:
    """(name, numel) of a 6.7B-parameter decoder: d_model 4096, 32 layers,
    FFN 11008, vocab 32000, untied head."""
    d, ff, vocab, layers = 4096, 11008, 32000, 32
    shapes = [("embed", vocab * d)]
    for layer in range(layers):
        shapes.append((f"l{layer}.attn_norm", d))
        for proj in ("q", "k", "v", "o"):
            shapes.append((f"l{layer}.{proj}", d * d))
        shapes.append((f"l{layer}.ffn_norm", d))
        shapes.append((f"l{layer}.gate", d * ff))
        shapes.append((f"l{layer}.up", d * ff))
        shapes.append((f"l{layer}.down", ff * d))
    shapes.append(("final_norm", d))
    shapes.append(("head", vocab * d))
    return shapes


def total(shapes: Iterable[tuple[str, int]]) -> int:
    return sum(n for _, n in shapes)
