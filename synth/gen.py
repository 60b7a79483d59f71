"""Seeded synthetic inputs, host side (numpy).

This module holds none of the attention method's arithmetic.  It only makes
inputs: counter-based pseudo-random numbers, rounding of those numbers to the
storage formats the kernels read (bf16, OCP FP8 E4M3 with a per-token fp32
scale), and the low-rank construction used for the 32K workload.

Random numbers
--------------
Every element is a pure function of (seed, tensor_id, flat index), so any
slice of any tensor can be regenerated without generating the rest.  The bit
source is SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; constants as in Vigna's public-domain
reference): the n-th output of a stream started at state X is
mix64(X + n * GAMMA).

  stream(seed, tid) = mix64(seed * GAMMA + tid)
  draw(e, j)        = mix64(stream + (6 * e + j + 1) * GAMMA),   j = 0..5

Each 64-bit draw yields two 20-bit uniforms (bits 0..19 and 32..51).  The
twelve uniforms of element e are summed as an integer (Irwin-Hall of order
12) and centred:

  z = (sum - 6 * 2^20) * 2^-20

The sum is below 2^24, so the conversion to float32 is exact; z has mean 0,
variance 1 - 2^-40 and support [-6, 6].  The device generator in
``gen_device.hip`` evaluates the same definition and must agree bit for bit.
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_U20 = np.uint64(0xFFFFF)

# Tensor ids: one fixed id per named tensor, shared with the device generator.
TID = {
    "q_idx": 1,   # indexer queries q^I (before FP8 quantisation)
    "w_idx": 2,   # indexer head weights w^I
    "k_idx": 3,   # indexer keys k^I (before FP8 quantisation)
    "q": 4,       # absorbed per-head attention queries (576-d)
    "kv": 5,      # latent cache rows c_s (576-d)
    "lr_z": 6,    # low-rank factor shared by kv and k_idx
    "lr_ac": 7,   # low-rank loading for kv
    "lr_ak": 8,   # low-rank loading for k_idx
    "lr_ec": 9,   # noise for kv
    "lr_ek": 10,  # noise for k_idx
    "q_mha": 11,  # MHA-mode per-head queries [q_nope | q_rope]
    "w_uk": 12,   # MHA-mode key decompression matrices
    "w_uv": 13,   # MHA-mode value decompression matrices
}

E4M3_MAX = 448.0


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(seed: int, tid: int) -> np.uint64:
    with np.errstate(over="ignore"):
        x = np.array([seed], dtype=np.uint64) * GAMMA + np.uint64(tid)
        return _mix64(x)[0]


def normal_f32(seed: int, tid: int, start: int, count: int) -> np.ndarray:
    """z for flat indices [start, start+count) of tensor `tid` (float32)."""
    e = np.arange(start, start + count, dtype=np.uint64)
    base = stream_key(seed, tid)
    acc = np.zeros(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        e6 = e * np.uint64(6)
        for j in range(6):
            x = _mix64(base + (e6 + np.uint64(j + 1)) * GAMMA)
            acc += (x & _U20) + ((x >> np.uint64(32)) & _U20)
    z = acc.astype(np.int64) - np.int64(6 << 20)
    return (z.astype(np.float32) * np.float32(2.0 ** -20)).astype(np.float32)


def normal_at(seed: int, tid: int, shape, index_ranges) -> np.ndarray:
    """Generate the sub-block of a row-major tensor of `shape` selected by
    `index_ranges` along axis 0 (a list/array of row indices)."""
    rows = np.asarray(index_ranges, dtype=np.int64)
    row_len = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((len(rows), row_len), dtype=np.float32)
    for n, r in enumerate(rows):
        out[n] = normal_f32(seed, tid, int(r) * row_len, row_len)
    return out.reshape((len(rows),) + tuple(shape[1:]))


# ---------------------------------------------------------------- bfloat16
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit pattern (uint16).
    Inputs here are finite (the generators never make NaN/inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- FP8 E4M3
def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP FP8 E4M3 (E4M3FN) byte, round-to-nearest-even,
    saturating to +-448.  Layout S.EEEE.MMM, bias 7, no infinities; the
    only NaN codes (S.1111.111) are never produced for finite input."""
    x = np.asarray(x, dtype=np.float32)
    sign = (x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    a = np.abs(x).astype(np.float64)  # exact copy of the float32 magnitude
    code = np.zeros(x.shape, dtype=np.int64)
    # Normal range: |x| >= 2^-6.  Choose exponent, round mantissa (3 bits) RNE.
    norm = a >= 2.0 ** -6
    if np.any(norm):
        an = a[norm]
        e = np.floor(np.log2(an)).astype(np.int64)
        # guard against log2 rounding at exact powers of two
        e = np.where(2.0 ** e > an, e - 1, e)
        e = np.where(2.0 ** (e + 1) <= an, e + 1, e)
        m_real = an / 2.0 ** e * 8.0 - 8.0          # in [0, 8), exact in float64
        m = np.rint(m_real).astype(np.int64)         # numpy rint = round half to even
        carry = m == 8
        m = np.where(carry, 0, m)
        e = np.where(carry, e + 1, e)
        c = (e + 7) * 8 + m
        c = np.minimum(c, 0x7E)                      # saturate at 448 = 0.1111.110
        code[norm] = c
    sub = ~norm
    if np.any(sub):
        m = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)  # 0..8; 8 becomes 2^-6 (code 8)
        code[sub] = m
    return (code.astype(np.uint8) | (sign << np.uint8(7))).astype(np.uint8)


def quantize_tokens_e4m3(x: np.ndarray):
    """Per-token FP8 quantisation.  x: [..., tok_len] float32.
    scale = amax / 448 (float32, correctly rounded; 1.0 for an all-zero token),
    code  = e4m3_encode(x / scale) with the division in float32.
    Returns (codes uint8 [..., tok_len], scales float32 [...])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    return e4m3_encode(y), scale


# ---------------------------------------------------------------- low rank
def low_rank_rows(seed: int, n_rows: int, rank: int, dim_c: int, dim_k: int, noise: float = 0.3):
    """Seeded low-rank latents for the 32K workload: a shared factor Z [n, r]
    makes both the latent rows c and the indexer keys k^I correlated across
    tokens, so the top-k sets have structure.

        c   = Z A_c / sqrt(r) + noise * eps_c
        k^I = Z A_k / sqrt(r) + noise * eps_k

    computed in float64 and rounded once to float32."""
    z = normal_f32(seed, TID["lr_z"], 0, n_rows * rank).astype(np.float64).reshape(n_rows, rank)
    ac = normal_f32(seed, TID["lr_ac"], 0, rank * dim_c).astype(np.float64).reshape(rank, dim_c)
    ak = normal_f32(seed, TID["lr_ak"], 0, rank * dim_k).astype(np.float64).reshape(rank, dim_k)
    ec = normal_f32(seed, TID["lr_ec"], 0, n_rows * dim_c).astype(np.float64).reshape(n_rows, dim_c)
    ek = normal_f32(seed, TID["lr_ek"], 0, n_rows * dim_k).astype(np.float64).reshape(n_rows, dim_k)
    c = z @ ac / np.sqrt(rank) + noise * ec
    k = z @ ak / np.sqrt(rank) + noise * ek
    return c.astype(np.float32), k.astype(np.float32)
