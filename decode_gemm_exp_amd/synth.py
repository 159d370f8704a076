"""Seeded synthetic inputs: bf16 weight matrices and activations.

This module draws random numbers and nothing else; it holds none of the
codec's or the GEMM's arithmetic, so the oracle and the HIP path can both be
fed from it.  Weights stand in for trained Llama MLP projections: the pages
measured real Llama 3.1 8B weights, which are not available here, so
N(0, 0.02) values at the same shapes (plus a stated fraction of power-of-two
scaled outliers where a workload asks for verbatim rows) take their place.

Recipe (all draws from ``torch.Generator`` seeded per tensor):
  * w = bf16(round-to-nearest-even(sigma * N(0,1) in fp32));
  * outliers: exactly round(frac * numel) distinct positions (a random
    permutation prefix), multiplied by 2**shift -- exact in bf16 for normal
    values, so the outlier keeps its mantissa and gains ``shift`` in exponent;
  * x = bf16(N(0,1));
  * FP8 weights (the already-quantised case): N(0, sigma) in fp32 scaled per
    tensor by 448 / max|w| (448 = the largest finite E4M3 value, the usual
    per-tensor FP8 checkpoint scale) and converted by torch to E4M3
    (round to nearest even), returned as raw bytes.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

SEED_BASE = 0x55570000


@dataclass(frozen=True)
class Workload:
    name: str
    # stored arrays: (rows, cols) of what is handed to the compressor
    mats: tuple            # tuple of (label, n, k, layout) ; layout 0 = stored W[N][K], 1 = W^T[K][N]
    sigma: float = 0.02
    outlier_frac: float = 0.0
    outlier_shift: int = 0
    batches: tuple = (1,)
    layers: int = 1
    seed: int = SEED_BASE
    notes: str = ""
    extra: dict = field(default_factory=dict)


# The five MLP workloads (shapes of Llama-3.1-8B / Llama-70B MLP projections),
# then the attention projections of the same two models (q/o: hidden x
# hidden; k/v: 8 key-value heads of 128, stored [N][K] as nn.Linear keeps
# them), the next step after the MLP: the same codec on new shapes.
WORKLOADS = {
    "w256x512": Workload(
        "w256x512", mats=(("w", 256, 512, 0),), outlier_frac=0.002, outlier_shift=12,
        batches=(1,), seed=SEED_BASE + 1,
        notes="single 256x512 matrix, 0.2% outliers x2^12; compress + full decode + B=1 GEMM"),
    "gate8b": Workload(
        "gate8b", mats=(("gate", 14336, 4096, 0),), outlier_frac=0.0005, outlier_shift=10,
        batches=(1,), seed=SEED_BASE + 2,
        notes="Llama-3.1-8B gate 14336x4096, 0.05% outliers x2^10; full + exponent decode, B=1"),
    "gateup8b": Workload(
        "gateup8b", mats=(("gate", 14336, 4096, 0), ("up", 14336, 4096, 0)),
        batches=(1, 8, 64), seed=SEED_BASE + 3,
        notes="fused gate+up 2x(14336x4096); palette transcode + direct palette"),
    "down8b": Workload(
        "down8b", mats=(("down", 4096, 14336, 1),), batches=(256, 1024), seed=SEED_BASE + 4,
        notes="down 4096x14336 stored transposed [K=14336][N=4096]; exponent + palette recon"),
    "mlp70b": Workload(
        "mlp70b", mats=(("gate", 28672, 8192, 0), ("up", 28672, 8192, 0),
                        ("down", 8192, 28672, 1)),
        batches=(1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024), layers=80, seed=SEED_BASE + 5,
        notes="80 layers of Llama-70B MLP, compressed-resident; autotuned"),
    "attn8b": Workload(
        "attn8b", mats=(("q", 4096, 4096, 0), ("k", 1024, 4096, 0), ("v", 1024, 4096, 0), ("o", 4096, 4096, 0)),
        outlier_frac=0.0002, outlier_shift=8, batches=(1, 8, 64), seed=SEED_BASE + 6,
        notes="Llama-3.1-8B attention q/k/v/o, 0.02% outliers x2^8; fused q+k+v and o at B=1, 8, 64"),
    "attn70b": Workload(
        "attn70b", mats=(("q", 8192, 8192, 0), ("k", 1024, 8192, 0), ("v", 1024, 8192, 0), ("o", 8192, 8192, 0)),
        outlier_frac=0.0002, outlier_shift=8, batches=(1, 64, 1024), seed=SEED_BASE + 7,
        notes="Llama-70B attention q/k/v/o, 0.02% outliers x2^8; fused q+k+v and o at B=1, 64, 1024"),
}


def stored_shape(n: int, k: int, layout: int) -> tuple[int, int]:
    return (n, k) if layout == 0 else (k, n)


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def weights(rows: int, cols: int, sigma: float = 0.02, outlier_frac: float = 0.0,
            outlier_shift: int = 0, seed: int = SEED_BASE, stream: int = 0,
            device="cpu") -> torch.Tensor:
    """bf16 tensor [rows][cols] (the stored array)."""
    g = _gen(seed, stream, device)
    w = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    w.mul_(sigma)
    n_out = int(round(outlier_frac * rows * cols))
    if n_out > 0:
        idx = torch.randperm(rows * cols, generator=g, device=device)[:n_out]
        flat = w.view(-1)
        flat[idx] = flat[idx] * float(2 ** outlier_shift)
    return w.to(torch.bfloat16)


def fp8_weights(rows: int, cols: int, sigma: float = 0.02, seed: int = SEED_BASE, stream: int = 500,
                device="cpu") -> torch.Tensor:
    """uint8 tensor [rows][cols] of FP8 E4M3 bytes (the stored array)."""
    g = _gen(seed, stream, device)
    w = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    w.mul_(sigma)
    w.mul_(448.0 / float(w.abs().max().clamp_min(1e-30)))
    return w.to(torch.float8_e4m3fn).view(torch.uint8)


def activations(batch: int, k: int, seed: int = SEED_BASE, stream: int = 1_000,
                device="cpu") -> torch.Tensor:
    g = _gen(seed, stream, device)
    return torch.randn(batch, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def random_bits(rows: int, cols: int, seed: int = 7, device="cpu") -> torch.Tensor:
    """Uniform random 16-bit patterns (any bf16 value incl. NaN/Inf/subnormal)."""
    g = _gen(seed, 77, device)
    return torch.randint(-32768, 32768, (rows, cols), generator=g, device=device,
                         dtype=torch.int32).to(torch.int16).view(torch.bfloat16)


def workload_weights(wl: Workload, mat_index: int, layer: int = 0, device="cpu") -> torch.Tensor:
    label, n, k, layout = wl.mats[mat_index]
    r, c = stored_shape(n, k, layout)
    return weights(r, c, wl.sigma, wl.outlier_frac, wl.outlier_shift, seed=wl.seed,
                   stream=layer * 16 + mat_index, device=device)


def bits_numpy(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
