"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers (numpy PCG64 via ``default_rng``), rounds fp32 to bf16 with
round-to-nearest-even, and writes NaN poison into padding.  Both the GPU path
and the CPU oracle are fed from here.

Workloads (sizes of the five standard configurations):

1. single-query fp32: q ~ N(0,1) (64,), K, V ~ N(0,1) (4096, 64), no scale,
   keys processed in 64-key pieces; plus the rows [1,3,2,0] and [2,5,1,7].
2. row softmax fp32: 4096 x 32000, N(0, 3^2) plus one spike per row drawn
   uniform in [20, 90) at a uniform column.
3. attention forward bf16: B=4, H=32, N=4096, d=128, N(0,1), non-causal.
4. attention forward bf16, causal + key padding: B=8, H=16, N=8192, d=128,
   valid lengths uniform integers in [1024, 8192], NaN poison past them in
   Q, K and V.
5. split-KV decode bf16: B=16, Hq=32, Hkv=8, d=128, one query token, KV
   lengths uniform integers in [4096, 32768] (cache allocated at 32768),
   NaN poison past them, 256-key pieces.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

SEED_BASE = 1000


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-to-nearest-even, returned as uint16 bits.
    NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _e4m3_table() -> np.ndarray:
    """fp32 value of each OCP FP8 E4M3 code: sign, 4 exponent bits (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m 2^-9); S.1111.111 is NaN and
    there are no infinities (largest finite 448)."""
    t = np.empty(256, np.float32)
    for v in range(256):
        sgn, e, m = v >> 7, (v >> 3) & 15, v & 7
        if e == 15 and m == 7:
            x = np.nan
        elif e == 0:
            x = m * 2.0 ** -9
        else:
            x = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        t[v] = -x if sgn else x
    return t


E4M3 = _e4m3_table()
_E4M3_POS = E4M3[:127]                 # codes 0x00..0x7e: 0 .. 448, increasing


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> OCP FP8 E4M3 codes (uint8), round to nearest, ties to the even
    code; magnitudes beyond 448 saturate to +-448; NaN -> 0x7f."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x), np.float32(448.0))
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)   # first code >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | np.uint8(0x80), code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def e4m3_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of OCP FP8 E4M3 codes to fp32."""
    return E4M3[np.ascontiguousarray(b, dtype=np.uint8)]


def normal_f32(g: np.random.Generator, shape, sigma: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


# ---------------------------------------------------------------------------
# row softmax
# ---------------------------------------------------------------------------
def softmax_rows_input(rows: int, cols: int, seed: int, sigma: float = 3.0,
                       spike_lo: float = 20.0, spike_hi: float = 90.0,
                       spikes: bool = True) -> np.ndarray:
    """fp32 [rows, cols]: N(0, sigma^2) with one spike per row, uniform in
    [spike_lo, spike_hi), at a uniformly drawn column."""
    g = rng(seed)
    x = normal_f32(g, (rows, cols), sigma)
    if spikes and cols > 0:
        col = g.integers(0, cols, size=rows)
        val = g.uniform(spike_lo, spike_hi, size=rows).astype(np.float32)
        x[np.arange(rows), col] = val
    return x


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
@dataclass
class AttnInputs:
    q: np.ndarray            # fp32 [B, Hq, Nq, d] or uint16 bf16 bits
    k: np.ndarray            # [B, Hkv, Nk, d]
    v: np.ndarray
    dtype: str               # "bf16", "f32" or "fp8" (OCP E4M3 codes)
    seqlens_q: np.ndarray | None
    seqlens_k: np.ndarray | None
    scale: float
    causal: bool

    def widened(self):
        """(q, k, v) as exact fp32 arrays, for the oracle."""
        if self.dtype == "bf16":
            return tuple(bf16_bits_to_f32(a) for a in (self.q, self.k, self.v))
        if self.dtype == "fp8":
            return tuple(e4m3_bits_to_f32(a) for a in (self.q, self.k, self.v))
        return self.q, self.k, self.v


def uniform_lengths(g: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in [lo, hi], both ends inclusive."""
    return g.integers(lo, hi + 1, size=n).astype(np.int32)


def poison_tail(x: np.ndarray, lens: np.ndarray, axis_len: int) -> None:
    """Write NaN into positions >= lens[b] along axis 2 of [B, H, N, d]."""
    for b, L in enumerate(lens):
        if L < axis_len:
            x[b, :, int(L):, :] = np.nan


def attention_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int, *,
                     dtype: str = "bf16", scale: float | None = None, causal: bool = False,
                     seqlens_q=None, seqlens_k=None, poison: bool = False) -> AttnInputs:
    """Q, K, V ~ N(0, 1) (rounded to bf16 for dtype "bf16"); optional NaN
    poison at padded positions (>= the valid length)."""
    g = rng(seed)
    q = normal_f32(g, (B, Hq, Nq, d))
    k = normal_f32(g, (B, Hkv, Nk, d))
    v = normal_f32(g, (B, Hkv, Nk, d))
    sq = None if seqlens_q is None else np.asarray(seqlens_q, np.int32)
    sk = None if seqlens_k is None else np.asarray(seqlens_k, np.int32)
    if poison:
        if sq is not None:
            poison_tail(q, sq, Nq)
        if sk is not None:
            poison_tail(k, sk, Nk)
            poison_tail(v, sk, Nk)
    if dtype == "bf16":
        q, k, v = to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
    elif dtype == "fp8":
        q, k, v = to_e4m3_bits(q), to_e4m3_bits(k), to_e4m3_bits(v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return AttnInputs(q, k, v, dtype, sq, sk, float(scale), bool(causal))


def output_grad(B: int, Hq: int, Nq: int, d: int, seed: int, *, seqlens_q=None,
                poison: bool = False) -> np.ndarray:
    """An output gradient dO ~ N(0, 1) [B, Hq, Nq, d] as bf16 bits, with
    optional NaN poison in rows past the valid query length."""
    g = rng(seed)
    do = normal_f32(g, (B, Hq, Nq, d))
    if poison and seqlens_q is not None:
        poison_tail(do, np.asarray(seqlens_q, np.int32), Nq)
    return to_bf16_bits(do)


def causal_padded_inputs(B: int, H: int, N: int, d: int, seed: int, lo: int, hi: int,
                         poison: bool = True) -> AttnInputs:
    """Self-attention with right padding: valid lengths uniform in [lo, hi],
    seqlens_q = seqlens_k = L_b, causal, NaN poison in Q/K/V past L_b."""
    lens = uniform_lengths(rng(seed + 7919), B, lo, hi)
    return attention_inputs(B, H, H, N, N, d, seed, dtype="bf16", causal=True,
                            seqlens_q=lens, seqlens_k=lens, poison=poison)


def decode_inputs(B: int, Hq: int, Hkv: int, Lmax: int, d: int, seed: int, lo: int, hi: int,
                  *, dtype: str = "bf16", scale: float | None = None,
                  poison: bool = True) -> AttnInputs:
    """One query token per (batch, head); KV cache [B, Hkv, Lmax, d] whose
    valid prefix length is uniform in [lo, hi]; NaN poison past it."""
    lens = uniform_lengths(rng(seed + 7919), B, lo, hi)
    return attention_inputs(B, Hq, Hkv, 1, Lmax, d, seed, dtype=dtype, scale=scale,
                            seqlens_k=lens, poison=poison)


# ---------------------------------------------------------------------------
# the five standard configurations
# ---------------------------------------------------------------------------
WORKED_ROWS = ([1.0, 3.0, 2.0, 0.0], [2.0, 5.0, 1.0, 7.0])


def config1(seed: int = SEED_BASE + 1) -> AttnInputs:
    """q (64,), K, V (4096, 64) fp32, no scale, as a 1-batch 1-head decode."""
    return attention_inputs(1, 1, 1, 1, 4096, 64, seed, dtype="f32", scale=1.0,
                            seqlens_k=np.array([4096], np.int32))


def config2(seed: int = SEED_BASE + 2) -> np.ndarray:
    return softmax_rows_input(4096, 32000, seed)


def config3(seed: int = SEED_BASE + 3) -> AttnInputs:
    return attention_inputs(4, 32, 32, 4096, 4096, 128, seed, dtype="bf16")


def config4(seed: int = SEED_BASE + 4) -> AttnInputs:
    return causal_padded_inputs(8, 16, 8192, 128, seed, 1024, 8192)


def config5(seed: int = SEED_BASE + 5) -> AttnInputs:
    return decode_inputs(16, 32, 8, 32768, 128, seed, 4096, 32768)


def random_partials(rows: int, splits: int, d: int, seed: int, empty_frac: float = 0.25):
    """Arbitrary partial triples for the standalone merge: m ~ N(0, 4),
    l ~ U[1, 64], o~ ~ N(0, 1) * l; a fraction of pieces are the empty set
    (m = -inf, l = 0, o~ = 0).  fp32."""
    g = rng(seed)
    m = normal_f32(g, (rows, splits), 2.0)
    l = g.uniform(1.0, 64.0, size=(rows, splits)).astype(np.float32)
    o = normal_f32(g, (rows, splits, d)) * l[..., None]
    empty = g.random((rows, splits)) < empty_frac
    m[empty] = -np.inf
    l[empty] = 0.0
    o[empty] = 0.0
    return m, l, o.astype(np.float32)


def lse_parts(parts: int, rows: int, d: int, seed: int, *, dtype: str = "f32",
              empty_frac: float = 0.0, poison: bool = False):
    """Normalized results of `parts` disjoint key sets for the log-sum-exp
    merge: o_s ~ N(0, 1) [parts, rows, d] (bf16 bits for dtype "bf16", else
    fp32), lse_s ~ U[-8, 8] fp32 [parts, rows]; a fraction of the pieces are
    the empty set (lse = -inf), whose o is NaN when `poison` (it must never
    be read) and 0 otherwise."""
    g = rng(seed)
    o = normal_f32(g, (parts, rows, d))
    lse = g.uniform(-8.0, 8.0, size=(parts, rows)).astype(np.float32)
    empty = g.random((parts, rows)) < empty_frac
    lse[empty] = -np.inf
    o[empty] = np.nan if poison else 0.0
    if dtype == "bf16":
        o = to_bf16_bits(o)
    return o, lse


def tiled_rows(n_rows: int, d: int, seed: int, *, dtype: str = "bf16", table_rows: int = 4096):
    """Rows for tensors too large to draw element by element in a test:
    row j is table[idx[j]], with the table's rows N(0, 1) (rounded to bf16
    bits, or E4M3 codes for dtype "fp8") and idx uniform over the table.
    Neighbouring positions hold different rows, so reading the wrong
    position changes the result.  Returns (table [table_rows, d], idx
    int64 [n_rows]); the caller gathers (on the host or on the device)."""
    g = rng(seed)
    t = normal_f32(g, (table_rows, d))
    table = to_e4m3_bits(t) if dtype == "fp8" else to_bf16_bits(t)
    idx = g.integers(0, table_rows, size=n_rows, dtype=np.int64)
    return table, idx
