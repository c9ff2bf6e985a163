"""Seeded synthetic inputs shared by the tests and the benchmark.

This module holds no quantization arithmetic: it only draws numbers.  Every draw comes from
a counter-based generator, so element i of a stream is a pure function of (seed, stream, i)
and does not depend on chunking, thread count or device:

    key   = mix64(seed * 2^32 + stream)
    u64_i = mix64(key + (i + 1) * 0x9E3779B97F4A7C15)            (mod 2^64)

where mix64 is the SplitMix64 output function (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014).  A uniform in [0, 1) takes the top 53 bits
times 2^-53; normals use the Box-Muller transform on index pairs (2j, 2j+1), in binary64,
then are rounded to binary32 and then to the target dtype (torch's round-to-nearest-even).

Workload recipes (see the test and bench files for the sizes they use):
  * blockwise inputs: N(0, std) values; optional outliers (x50 with probability p_out) and
    non-finite elements (probability p_nf, NaN / +Inf / -Inf one third each);
  * 16-entry code table: {-1, 0, 1} and 13 uniform draws in (-1, 1), distinct, sorted,
    min gap >= 2^-6, every nonzero |c| >= 2^-20;
  * 256-entry code table: symmetric {-p_128..-p_1, p_1..p_128}, p_128 = 1,
    p_j = ((j - 1 + u_j) / 128)^2 with u_j ~ U(0.4, 0.6) (denser near 0);
  * GGUF-style blocks: fp16 scale d = |N(0, 0.01)| rounded to fp16, little-endian, then 16
    bytes of uniform nibbles (18-byte block) or 32 uniform int8 (34-byte block).

Streams: 0 values, 1 outlier mask, 2 non-finite mask, 3 non-finite kind, 4 codes,
5 scales, 6 table draws.
"""
from __future__ import annotations

import math

import numpy as np
import torch

_M64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Two's-complement int64 value of an unsigned 64-bit constant."""
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


_GAMMA = _s64(0x9E3779B97F4A7C15)
_C1 = _s64(0xBF58476D1CE4E5B9)
_C2 = _s64(0x94D049BB133111EB)


def _srl(x: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 tensors."""
    return (x >> k) & ((1 << (64 - k)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _srl(z, 30)) * _C1
    z = (z ^ _srl(z, 27)) * _C2
    return z ^ _srl(z, 31)


def _mix64_int(z: int) -> int:
    z &= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return _s64(_mix64_int((seed << 32) + stream))


def u64(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Raw 64-bit draws (as int64) for indices start .. start+count-1."""
    idx = torch.arange(start + 1, start + count + 1, dtype=torch.int64, device=device)
    return _mix64(stream_key(seed, stream) + idx * _GAMMA)


def uniform(seed: int, stream: int, start: int, count: int, device="cpu") -> torch.Tensor:
    """Uniform binary64 values in [0, 1)."""
    top53 = _srl(u64(seed, stream, start, count, device), 11)
    return top53.to(torch.float64) * (2.0 ** -53)


def normal(seed: int, stream: int, start: int, count: int, std: float = 1.0,
           device="cpu") -> torch.Tensor:
    """N(0, std^2) binary64 values for element indices start .. start+count-1."""
    j0 = start // 2
    j1 = (start + count + 1) // 2
    u = uniform(seed, stream, 2 * j0, 2 * (j1 - j0), device).view(-1, 2)
    r = torch.sqrt(-2.0 * torch.log1p(-u[:, 0]))
    th = (2.0 * math.pi) * u[:, 1]
    z = torch.stack([r * torch.cos(th), r * torch.sin(th)], dim=1).reshape(-1)
    off = start - 2 * j0
    return z[off:off + count] * std


_TORCH_DT = {"float32": torch.float32, "float16": torch.float16, "bfloat16": torch.bfloat16}


def blockwise_input(n: int, dtype: str, seed: int, std: float = 1.0, p_out: float = 0.0,
                    p_nf: float = 0.0, device="cpu", chunk: int = 1 << 24) -> torch.Tensor:
    """1-D tensor of n elements of `dtype` drawn per the blockwise recipe."""
    out = torch.empty(n, dtype=_TORCH_DT[dtype], device=device)
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        v = normal(seed, 0, s, c, std, device)
        if p_out > 0:
            v = torch.where(uniform(seed, 1, s, c, device) < p_out, v * 50.0, v)
        if p_nf > 0:
            nf = uniform(seed, 2, s, c, device) < p_nf
            kind = uniform(seed, 3, s, c, device)
            special = torch.where(kind < 1.0 / 3.0, torch.full_like(v, float("nan")),
                                  torch.where(kind < 2.0 / 3.0, torch.full_like(v, float("inf")),
                                              torch.full_like(v, float("-inf"))))
            v = torch.where(nf, special, v)
        out[s:s + c] = v.to(torch.float32).to(out.dtype)
    return out


def table16(seed: int = 16) -> np.ndarray:
    """Sorted 16-entry code table in [-1, 1] holding -1, 0 and 1."""
    attempt = 0
    while True:
        u = uniform(seed, 6, attempt * 13, 13).numpy()
        vals = np.float32(2.0 * u - 1.0)
        t = np.unique(np.concatenate([np.float32([-1.0, 0.0, 1.0]), vals]).astype(np.float32))
        nz = t[t != 0]
        if (len(t) == 16 and np.min(np.diff(t.astype(np.float64))) >= 2.0 ** -6
                and np.min(np.abs(nz)) >= 2.0 ** -20):
            return t.astype(np.float32)
        attempt += 1


def table256(seed: int = 256) -> np.ndarray:
    """Sorted symmetric 256-entry code table, denser near 0, no zero entry."""
    u = 0.4 + 0.2 * uniform(seed, 6, 0, 127).numpy()
    j = np.arange(1, 128, dtype=np.float64)
    p = np.concatenate([((j - 1.0 + u) / 128.0) ** 2, [1.0]]).astype(np.float32)
    t = np.concatenate([-p[::-1], p]).astype(np.float32)
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    return t


def dyadic_table(K: int) -> np.ndarray:
    """Uniform dyadic table c_k = -1 + 2k/K, k = 0..K-1 (exact in binary32)."""
    return (-1.0 + 2.0 * np.arange(K, dtype=np.float64) / K).astype(np.float32)


def q32_blocks(nblocks: int, fmt: str, seed: int, device="cpu") -> torch.Tensor:
    """uint8 tensor of nblocks serialized GGUF-style blocks (fmt 'q4': 18 B, 'q8': 34 B)."""
    nbytes = 16 if fmt == "q4" else 32
    bs = 2 + nbytes
    d = normal(seed, 5, 0, nblocks, 0.01, device).abs().to(torch.float32).to(torch.float16)
    dbits = d.view(torch.int16).to(torch.int32) & 0xFFFF
    payload = (_srl(u64(seed, 4, 0, nblocks * nbytes, device), 56)).to(torch.uint8)
    out = torch.empty(nblocks, bs, dtype=torch.uint8, device=device)
    out[:, 0] = (dbits & 0xFF).to(torch.uint8)
    out[:, 1] = (dbits >> 8).to(torch.uint8)
    out[:, 2:] = payload.view(nblocks, nbytes)
    return out.reshape(-1)


def iq2xs_grid(seed: int = 512, alphabet=(8, 25, 43)) -> np.ndarray:
    """512 distinct grid entries of 8 magnitude bytes drawn from `alphabet` (the byte values the
    IQ2_XS grid uses; the grid itself is the caller's), as a (512, 8) uint8 array."""
    rows, out, start = set(), [], 0
    k = len(alphabet)
    while len(out) < 512:
        idx = (_srl(u64(seed, 7, start, 8), 33) % k).numpy()
        start += 8
        r = tuple(int(alphabet[i]) for i in idx)
        if r not in rows:
            rows.add(r)
            out.append(r)
    return np.array(out, np.uint8)


def iq1s_grid(seed: int = 2048) -> np.ndarray:
    """2048 distinct grid entries of 8 signed ternary bytes (-1, 0, +1: the IQ1_S alphabet;
    the grid itself is the caller's), as a (2048, 8) int8 array."""
    rows, out, start = set(), [], 0
    while len(out) < 2048:
        idx = (_srl(u64(seed, 10, start, 8), 33) % 3).numpy()
        start += 8
        r = tuple(int(i) - 1 for i in idx)
        if r not in rows:
            rows.add(r)
            out.append(r)
    return np.array(out, np.int8)


def iq2xs_scales(x: torch.Tensor, ratio: float = 0.8) -> torch.Tensor:
    """A caller's binary16 superblock scales for x (n a multiple of 256): ratio * (largest
    finite |x| of the superblock) / 166.625, 166.625 being the largest decoded magnitude per
    unit scale (15.5 / 4 * 43).  Returned as int16 bit patterns on x's device."""
    a = x.to(torch.float32).reshape(-1, 256).abs()
    a = torch.where(torch.isfinite(a), a, torch.zeros_like(a)).amax(dim=1)
    return (a * (ratio / 166.625)).to(torch.float16).view(torch.int16)


def to_bits16(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a 16-bit tensor (for the oracle's numpy interface)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
