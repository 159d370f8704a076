"""Seeded synthetic inputs: bf16 weight matrices and activations.

This module draws random numbers and nothing else; it holds none of the
codec's or the GEMM's arithmetic, so the oracle and the HIP path can both be
fed from it.  Weights stand in for trained Llama MLP projections: the pages
measured real Llama 3.1 8B weights, which are not available here, so
N(0, 0.02) values at the same shapes (plus a stated fraction of power-of-two
scaled outliers where a workload asks for verbatim rows) take their place.

Every draw is counter-based, so a tensor is the same on any device: element
i of stream (seed, stream, purpose) is SplitMix64 (Steele, Lea and Flood,
"Fast splittable pseudorandom number generators", OOPSLA 2014; the finaliser
with Vigna's constants) of a key mixed from those three and i, computed in
64-bit integer arithmetic that wraps the same way on the CPU and the GPU.
Recipe:
  * N(0,1): Box-Muller on two such draws, u1 = (h1 >> 11 + 1) 2^-53 in
    (0, 1] and u2 = (h2 >> 11) 2^-53, z = sqrt(-2 ln u1) cos(2 pi u2) in
    float64 (the CPU and GPU library functions differ by at most an ulp of
    float64 there, far below the float32 and bf16 roundings that follow);
  * w = bf16(fp32(sigma * z)), each step round-to-nearest-even;
  * outliers: exactly round(frac * numel) distinct positions drawn by Floyd's
    sampling algorithm (Bentley and Floyd, "A sample of brilliance", CACM
    1987) from the counter stream, each multiplied by 2**shift -- exact in
    bf16 for normal values, so the outlier keeps its mantissa and gains
    ``shift`` in exponent;
  * x = bf16(fp32(z));
  * FP8 weights (the already-quantised case): sigma * z in fp32 scaled per
    tensor by 448 / max|w| (448 = the largest finite E4M3 value, the usual
    per-tensor FP8 checkpoint scale) and converted by torch to E4M3
    (round to nearest even), returned as raw bytes;
  * uniform 16-bit patterns: the low 16 bits of a draw.
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


_M64 = (1 << 64) - 1


def _i64(v: int) -> int:
    """A 64-bit pattern as the signed value torch's int64 holds."""
    v &= _M64
    return v - (1 << 64) if v >> 63 else v


def _shr(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of int64 patterns (torch's >> is arithmetic)."""
    return (x >> s) & ((1 << (64 - s)) - 1)


_GAMMA = _i64(0x9E3779B97F4A7C15)
_MUL1 = _i64(0xBF58476D1CE4E5B9)
_MUL2 = _i64(0x94D049BB133111EB)


def _mix(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64's finaliser on int64 patterns (multiplications wrap)."""
    z = (z ^ _shr(z, 30)) * _MUL1
    z = (z ^ _shr(z, 27)) * _MUL2
    return z ^ _shr(z, 31)


def _key(seed: int, stream: int, purpose: int) -> int:
    k = (seed * 0x100000001B3 + stream * 0x9E3779B1 + purpose * 0x85EBCA77) & _M64
    k = _mix(torch.tensor([_i64(k)], dtype=torch.int64))
    return int(k.item())


def _draws(key: int, start: int, count: int, device) -> torch.Tensor:
    """int64 patterns of elements start .. start + count - 1 of one stream."""
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    return _mix((i + 1) * _GAMMA + key)


_CHUNK = 1 << 24


def _normal(key1: int, key2: int, numel: int, device) -> torch.Tensor:
    """float64 N(0,1) values, elements 0 .. numel - 1 of the (key1, key2) streams."""
    out = torch.empty(numel, dtype=torch.float64, device=device)
    for s0 in range(0, numel, _CHUNK):
        n = min(_CHUNK, numel - s0)
        u1 = (_shr(_draws(key1, s0, n, device), 11) + 1).to(torch.float64) * 2.0 ** -53
        u2 = _shr(_draws(key2, s0, n, device), 11).to(torch.float64) * 2.0 ** -53
        out[s0:s0 + n] = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * np.pi) * u2)
    return out


def _floyd(key: int, numel: int, count: int) -> np.ndarray:
    """count distinct positions in [0, numel), Floyd's sampling algorithm: for
    j = numel - count .. numel - 1 draw t in [0, j]; take t unless already
    taken, else j."""
    if count <= 0:
        return np.zeros(0, np.int64)
    j0 = numel - count
    h = _draws(key, 0, count, "cpu").numpy().view(np.uint64)
    chosen = set()
    order = []
    for c in range(count):
        j = j0 + c
        t = int(h[c] % np.uint64(j + 1))
        pick = j if t in chosen else t
        chosen.add(pick)
        order.append(pick)
    return np.array(order, np.int64)


def weights(rows: int, cols: int, sigma: float = 0.02, outlier_frac: float = 0.0,
            outlier_shift: int = 0, seed: int = SEED_BASE, stream: int = 0,
            device="cpu") -> torch.Tensor:
    """bf16 tensor [rows][cols] (the stored array)."""
    numel = rows * cols
    z = _normal(_key(seed, stream, 1), _key(seed, stream, 2), numel, device)
    w = (z * sigma).to(torch.float32)
    del z
    n_out = int(round(outlier_frac * numel))
    if n_out > 0:
        idx = torch.from_numpy(_floyd(_key(seed, stream, 3), numel, n_out)).to(device)
        w[idx] = w[idx] * float(2 ** outlier_shift)
    return w.to(torch.bfloat16).view(rows, cols)


def fp8_weights(rows: int, cols: int, sigma: float = 0.02, seed: int = SEED_BASE, stream: int = 500,
                device="cpu") -> torch.Tensor:
    """uint8 tensor [rows][cols] of FP8 E4M3 bytes (the stored array)."""
    z = _normal(_key(seed, stream, 1), _key(seed, stream, 2), rows * cols, device)
    w = (z * sigma).to(torch.float32).view(rows, cols)
    w.mul_(448.0 / float(w.abs().max().clamp_min(1e-30)))
    return w.to(torch.float8_e4m3fn).view(torch.uint8)


def activations(batch: int, k: int, seed: int = SEED_BASE, stream: int = 1_000,
                device="cpu") -> torch.Tensor:
    z = _normal(_key(seed, stream, 1), _key(seed, stream, 2), batch * k, device)
    return z.to(torch.float32).to(torch.bfloat16).view(batch, k)


def random_bits(rows: int, cols: int, seed: int = 7, device="cpu") -> torch.Tensor:
    """Uniform random 16-bit patterns (any bf16 value incl. NaN/Inf/subnormal)."""
    h = _draws(_key(seed, 77, 4), 0, rows * cols, device)
    return (h & 0xFFFF).to(torch.int32).to(torch.int16).view(rows, cols).view(torch.bfloat16)


def workload_weights(wl: Workload, mat_index: int, layer: int = 0, device="cpu") -> torch.Tensor:
    label, n, k, layout = wl.mats[mat_index]
    r, c = stored_shape(n, k, layout)
    return weights(r, c, wl.sigma, wl.outlier_frac, wl.outlier_shift, seed=wl.seed,
                   stream=layer * 16 + mat_index, device=device)


def bits_numpy(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
