"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path.

This module holds no arithmetic of the attention layer. It only draws numbers
and stores them as bf16. The same numbers can be drawn on the host (NumPy) and
on a device (PyTorch integer ops), bit for bit, because every step is integer
arithmetic or an exact float conversion:

* Counter-based uniform bits: the SplitMix64 output function (Steele, Lea and
  Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014),
  applied to ``key + n * GAMMA`` for the n-th 64-bit word of a stream.
* Approximately standard-normal values: the classic sum of twelve uniforms
  minus six (Irwin-Hall with n = 12, mean 0, variance 1, support [-6, 6]).
  Three 64-bit words give twelve 16-bit uniforms; the centred sum is an
  integer below 2**21 in magnitude, converted exactly to float32 and scaled
  by the exact power of two 2**-17.
* bf16 storage: float32 rounded to bfloat16 with round-to-nearest-even,
  done on the bit pattern.

Streams are named by small integers (``stream_id``) so every tensor of a
workload has its own independent sequence, addressed by the element's flat
index in a canonical layout; that makes any slice reproducible on its own.
"""
from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _mix64_int(z: int) -> int:
    """SplitMix64 output mix on a Python int (host scalar form)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * _M1) & MASK64
    z = ((z ^ (z >> 27)) * _M2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream_id: int) -> int:
    """64-bit key of stream ``stream_id`` under ``seed``."""
    return _mix64_int(_mix64_int(seed * GAMMA + 0x5EED) ^ (stream_id * 0xD1B54A32D192ED03 & MASK64))


# ----------------------------------------------------------------------------
# NumPy (host) form
# ----------------------------------------------------------------------------

def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * np.uint64(_M1)
    z = z ^ (z >> np.uint64(27))
    z = z * np.uint64(_M2)
    return z ^ (z >> np.uint64(31))


def _normal_int_np(key: int, idx: np.ndarray) -> np.ndarray:
    """Centred Irwin-Hall(12) sum as int64, in units of 2**-17."""
    idx = idx.astype(np.uint64)
    total = np.zeros(idx.shape, dtype=np.int64)
    with np.errstate(over="ignore"):
        base = np.uint64(key) + idx * np.uint64(3 * GAMMA & MASK64)
        for w in range(3):
            h = _mix64_np(base + np.uint64(w * GAMMA & MASK64))
            for part in range(4):
                u = ((h >> np.uint64(16 * part)) & np.uint64(0xFFFF)).astype(np.int64)
                total += 2 * u + 1
    return total - 12 * 65536


def normal_f32(seed: int, stream_id: int, idx) -> np.ndarray:
    """Approximately N(0,1) float32 values for flat indices ``idx`` of a stream."""
    idx = np.asarray(idx, dtype=np.int64)
    out = np.empty(idx.shape, dtype=np.float32)
    flat_i = idx.reshape(-1)
    flat_o = out.reshape(-1)
    chunk = 1 << 22
    key = stream_key(seed, stream_id)
    for s in range(0, flat_i.size, chunk):
        n = _normal_int_np(key, flat_i[s:s + chunk])
        flat_o[s:s + chunk] = n.astype(np.float32) * np.float32(2.0 ** -17)
    return out


def e4m3_codes(seed: int, stream_id: int, idx) -> np.ndarray:
    """uint8 codes for flat indices ``idx``: one 64-bit word per index; the
    low 16 bits pick a magnitude code in 0x20 .. 0x47 (0.125 .. 3.75 in the
    OCP E4M3 encoding), bit 16 the sign.  Data only: no rounding of values."""
    idx = np.asarray(idx, dtype=np.int64).astype(np.uint64)
    key = np.uint64(stream_key(seed, stream_id))
    with np.errstate(over="ignore"):
        h = _mix64_np(key + idx * np.uint64(GAMMA))
    mag = (h & np.uint64(0xFFFF)) % np.uint64(40) + np.uint64(0x20)
    sign = ((h >> np.uint64(16)) & np.uint64(1)) << np.uint64(7)
    return (mag | sign).astype(np.uint8)


def sign_bf16_bits(seed: int, stream_id: int, idx) -> np.ndarray:
    """bf16 bit patterns of +1 or -1 for flat indices ``idx``: bit 0 of one
    64-bit word per index picks the sign.  A row of D such entries has mean
    square exactly 1, and every value is exact in bf16 and in E4M3."""
    idx = np.asarray(idx, dtype=np.int64).astype(np.uint64)
    key = np.uint64(stream_key(seed, stream_id))
    with np.errstate(over="ignore"):
        h = _mix64_np(key + idx * np.uint64(GAMMA))
    return np.where((h & np.uint64(1)) == 1, np.uint16(0xBF80), np.uint16(0x3F80)).astype(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def normal_bf16_bits(seed: int, stream_id: int, shape, offset: int = 0) -> np.ndarray:
    """A whole tensor of bf16 N(0,1)-like values, canonical row-major indexing."""
    n = int(np.prod(shape))
    idx = np.arange(offset, offset + n, dtype=np.int64)
    return f32_to_bf16_bits(normal_f32(seed, stream_id, idx)).reshape(shape)


# ----------------------------------------------------------------------------
# PyTorch (device) form: identical integer steps on int64 tensors.
# int64 multiplication wraps modulo 2**64 on both CPU and GPU, and every right
# shift is masked so that it acts as the logical (unsigned) shift.
# ----------------------------------------------------------------------------

def _as_i64(v: int) -> int:
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _lsr(t, s: int):
    return (t >> s) & ((1 << (64 - s)) - 1)


def _mix64_torch(z):
    z = z ^ _lsr(z, 30)
    z = z * _as_i64(_M1)
    z = z ^ _lsr(z, 27)
    z = z * _as_i64(_M2)
    return z ^ _lsr(z, 31)


def normal_bf16_torch(seed: int, stream_id: int, idx):
    """bf16 tensor (torch.bfloat16) for int64 flat indices ``idx`` (any device)."""
    import torch
    key = stream_key(seed, stream_id)
    base = idx.to(torch.int64) * _as_i64(3 * GAMMA) + _as_i64(key)
    total = torch.zeros_like(base)
    for w in range(3):
        h = _mix64_torch(base + _as_i64(w * GAMMA))
        for part in range(4):
            total += 2 * (_lsr(h, 16 * part) & 0xFFFF) + 1
    total -= 12 * 65536
    f = total.to(torch.float32) * (2.0 ** -17)
    bits = f.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    r = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    r = torch.where(r >= 32768, r - 65536, r).to(torch.int16)
    return r.view(torch.bfloat16)


def e4m3_codes_torch(seed: int, stream_id: int, idx):
    """The same codes as ``e4m3_codes`` as a uint8 tensor (any device)."""
    import torch
    key = stream_key(seed, stream_id)
    h = _mix64_torch(idx.to(torch.int64) * _as_i64(GAMMA) + _as_i64(key))
    mag = torch.remainder(h & 0xFFFF, 40) + 0x20
    sign = (_lsr(h, 16) & 1) << 7
    return (mag | sign).to(torch.uint8)


def sign_bf16_torch(seed: int, stream_id: int, idx):
    """The same signs as ``sign_bf16_bits`` as a bfloat16 tensor (any device)."""
    import torch
    key = stream_key(seed, stream_id)
    h = _mix64_torch(idx.to(torch.int64) * _as_i64(GAMMA) + _as_i64(key))
    bits = torch.where((h & 1) == 1, torch.full_like(h, 0xBF80 - 65536), torch.full_like(h, 0x3F80))
    return bits.to(torch.int16).view(torch.bfloat16)


def normal_bf16_torch_tensor(seed: int, stream_id: int, shape, device, offset: int = 0):
    import torch
    n = 1
    for s in shape:
        n *= int(s)
    out = torch.empty(n, dtype=torch.bfloat16, device=device)
    chunk = 1 << 26
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(offset + s, offset + e, dtype=torch.int64, device=device)
        out[s:e] = normal_bf16_torch(seed, stream_id, idx)
    return out.view(*shape)
