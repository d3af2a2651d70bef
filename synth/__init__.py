"""Seeded synthetic inputs for KV-cache attention.

This module only draws numbers and lays them out. It holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path can be fed
from it without sharing any part of the method.

Recipe (the same for tests and the benchmark):

* every floating-point input is drawn as float32 N(0, 1) from
  ``numpy.random.default_rng(seed)``; draw order is q, then K, then V;
* bf16 inputs are the float32 draws rounded to nearest-even bf16; the
  rounded values are what both sides read;
* cache rows past the valid length are overwritten with NaN after the draw
  when ``poison`` is set, so a kernel that reads them produces NaN;
* ragged batches draw the lengths first from ``default_rng(seed)`` and then
  every sequence from its own ``default_rng([seed, b])`` so one sequence can
  be regenerated without the others;
* "needle" inputs (``plant_needles``) overwrite a few keys of each
  sequence and kv head after the draw with one key that the head's query
  group scores far above the rest, so that those rows carry nearly all the
  attention weight and the output stays of order one at any length.

bf16 tensors are returned as ``uint16`` bit patterns; ``bf16_to_f32`` gives
their exact float32 values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterator, Optional

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bf16 encoding helpers (pure bit manipulation, no attention arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, BF16_QNAN, r)
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _draw(rng: np.random.Generator, shape, dtype: str):
    """Draw N(0,1) float32 and encode as the requested storage dtype."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def _nan_of(dtype: str):
    return BF16_QNAN if dtype == "bf16" else np.float32(np.nan)


def as_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values of an input array stored as ``dtype``."""
    return bf16_to_f32(arr) if dtype == "bf16" else np.asarray(arr, np.float32)


# ----------------------------------------------------------------------------
# Decode inputs
# ----------------------------------------------------------------------------
@dataclass
class DecodeInputs:
    dtype: str
    q: np.ndarray            # [B, Hq, D]
    k_cache: np.ndarray      # [B, Hkv, max_length, D]
    v_cache: np.ndarray      # [B, Hkv, max_length, D]
    position_id: Optional[int] = None      # uniform: rows [0, position_id]
    seq_lens: Optional[np.ndarray] = None  # ragged: rows [0, seq_lens[b])
    scale: Optional[float] = None

    @property
    def shape(self):
        B, Hq, D = self.q.shape
        _, Hkv, max_length, _ = self.k_cache.shape
        return B, Hq, Hkv, D, max_length


def decode_uniform(seed: int, B: int, Hq: int, Hkv: int, D: int,
                   max_length: int, position_id: int, dtype: str,
                   poison: bool = True, scale: Optional[float] = None
                   ) -> DecodeInputs:
    """Single position for the whole batch; rows > position_id poisoned."""
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, D), dtype)
    k = _draw(rng, (B, Hkv, max_length, D), dtype)
    v = _draw(rng, (B, Hkv, max_length, D), dtype)
    if poison and position_id + 1 < max_length:
        k[:, :, position_id + 1:, :] = _nan_of(dtype)
        v[:, :, position_id + 1:, :] = _nan_of(dtype)
    return DecodeInputs(dtype, q, k, v, position_id=position_id, scale=scale)


def ragged_lengths(seed: int, B: int, max_length: int,
                   low: int = 1) -> np.ndarray:
    """Per-sequence valid lengths, uniform in [low, max_length]."""
    rng = np.random.default_rng(seed)
    return rng.integers(low, max_length + 1, size=B).astype(np.int32)


def ragged_sequence(seed: int, b: int, Hq: int, Hkv: int, D: int, L: int,
                    dtype: str):
    """(q_b [Hq, D], K_b [Hkv, L, D], V_b [Hkv, L, D]) for sequence b."""
    r = np.random.default_rng([seed, b])
    q = _draw(r, (Hq, D), dtype)
    k = _draw(r, (Hkv, L, D), dtype)
    v = _draw(r, (Hkv, L, D), dtype)
    return q, k, v


def decode_ragged(seed: int, B: int, Hq: int, Hkv: int, D: int,
                  max_length: int, dtype: str,
                  lengths: Optional[np.ndarray] = None, poison: bool = True,
                  scale: Optional[float] = None) -> DecodeInputs:
    """Ragged batch, materialised in full (use for sizes that fit host RAM)."""
    if lengths is None:
        lengths = ragged_lengths(seed, B, max_length)
    lengths = np.asarray(lengths, dtype=np.int32)
    store = np.uint16 if dtype == "bf16" else np.float32
    fill = _nan_of(dtype) if poison else store(0)
    q = np.empty((B, Hq, D), store)
    k = np.full((B, Hkv, max_length, D), fill, store)
    v = np.full((B, Hkv, max_length, D), fill, store)
    for b in range(B):
        L = int(min(max(int(lengths[b]), 0), max_length))
        qb, kb, vb = ragged_sequence(seed, b, Hq, Hkv, D, L, dtype)
        q[b] = qb
        k[b, :, :L] = kb
        v[b, :, :L] = vb
    return DecodeInputs(dtype, q, k, v, seq_lens=lengths, scale=scale)


def iter_ragged(seed: int, B: int, Hq: int, Hkv: int, D: int,
                max_length: int, dtype: str,
                lengths: Optional[np.ndarray] = None) -> Iterator[tuple]:
    """Yield (b, L, q_b, K_b, V_b) one sequence at a time (bounded memory)."""
    if lengths is None:
        lengths = ragged_lengths(seed, B, max_length)
    for b in range(B):
        L = int(min(max(int(lengths[b]), 0), max_length))
        yield (b, L) + ragged_sequence(seed, b, Hq, Hkv, D, L, dtype)


def plant_needles(seed: int, q: np.ndarray, k_cache: np.ndarray,
                  lengths: np.ndarray, dtype: str, n_rows: int = 3,
                  margin: float = 8.0) -> np.ndarray:
    """Overwrite keys of a drawn decode batch (in place) with needles.

    q [B, Hq, D] and k_cache [B, Hkv, M, D] as stored; query heads
    g*G .. g*G+G-1 share kv head g (G = Hq / Hkv). For every sequence b of
    length L > 0 (lengths clamped to [0, M]) and kv head g, let u be the unit
    vector along the sum of the group's queries and m the smallest product
    q_h . u over the group; the needle key is alpha * u with alpha chosen so
    that m * alpha / sqrt(D) = log(L) + margin. Against L keys whose scaled
    products are about N(0, 1) the needles then hold all but about
    e^(0.5 - margin) of the weight. The rows overwritten are min(n_rows, L)
    distinct valid rows drawn from ``default_rng([seed, 11])`` plus row 0
    (even g) or row L - 1 (odd g). Returns the needle keys [B, Hkv, D] as
    stored (zero for empty sequences)."""
    B, Hq, D = q.shape
    Hkv, M = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    qf = as_f32(q, dtype).astype(np.float64)
    rng = np.random.default_rng([seed, 11])
    keys = np.zeros((B, Hkv, D), k_cache.dtype)
    for b in range(B):
        L = int(min(max(int(lengths[b]), 0), M))
        if L == 0:
            continue
        for g in range(Hkv):
            grp = qf[b, g * G:(g + 1) * G]
            u = grp.sum(0)
            u /= np.linalg.norm(u)
            m = float((grp @ u).min())
            if m <= 1.0:
                raise ValueError(f"query group ({b}, {g}) has no common direction")
            alpha = (np.log(L) + margin) * np.sqrt(D) / m
            key = (alpha * u).astype(np.float32)
            enc = f32_to_bf16_bits(key) if dtype == "bf16" else key
            rows = set(rng.choice(L, size=min(n_rows, L), replace=False).tolist())
            rows.add(0 if g % 2 == 0 else L - 1)
            keys[b, g] = enc
            for r in rows:
                k_cache[b, g, r] = enc
    return keys


def new_token_kv(seed: int, B: int, Hkv: int, D: int, dtype: str):
    """(k_new, v_new), each [B, Hkv, D]: the current token's key and value for
    a fused append."""
    rng = np.random.default_rng([seed, 10**6])
    return _draw(rng, (B, Hkv, D), dtype), _draw(rng, (B, Hkv, D), dtype)


def paginate(k_cache: np.ndarray, v_cache: np.ndarray, page_size: int,
             seed: int, extra_pages: int = 3, dtype: str = "bf16",
             layout: str = "token"):
    """Scatter a contiguous cache [B, Hkv, M, D] (M a multiple of page_size)
    into pages in a seeded random order, token-major [num_pages, page_size,
    Hkv, D] or head-major [num_pages, Hkv, page_size, D], with `extra_pages`
    unreferenced pages filled with NaN. Returns (k_pages, v_pages,
    block_table int32 [B, M / page_size])."""
    B, Hkv, M, D = k_cache.shape
    assert M % page_size == 0
    nb = M // page_size
    num_pages = B * nb + extra_pages
    rng = np.random.default_rng([seed, 7])
    perm = rng.permutation(num_pages)
    table = perm[:B * nb].reshape(B, nb).astype(np.int32)
    shape = ((num_pages, page_size, Hkv, D) if layout == "token"
             else (num_pages, Hkv, page_size, D))
    kp = np.full(shape, _nan_of(dtype), k_cache.dtype)
    vp = np.full(shape, _nan_of(dtype), v_cache.dtype)
    for b in range(B):
        for blk in range(nb):
            rows = slice(blk * page_size, (blk + 1) * page_size)
            kb, vb = k_cache[b, :, rows, :], v_cache[b, :, rows, :]
            if layout == "token":
                kb, vb = kb.transpose(1, 0, 2), vb.transpose(1, 0, 2)
            kp[table[b, blk]] = kb
            vp[table[b, blk]] = vb
    return kp, vp, table


# ----------------------------------------------------------------------------
# Prefill inputs
# ----------------------------------------------------------------------------
@dataclass
class PrefillInputs:
    dtype: str
    q: np.ndarray            # [B, Hq, Lq, D]
    k_cache: np.ndarray      # [B, Hkv, max_length, D]
    v_cache: np.ndarray
    prefix_len: int
    scale: Optional[float] = None

    @property
    def shape(self):
        B, Hq, Lq, D = self.q.shape
        _, Hkv, max_length, _ = self.k_cache.shape
        return B, Hq, Hkv, D, max_length, Lq


def prefill(seed: int, B: int, Hq: int, Hkv: int, D: int, Lq: int,
            prefix_len: int, max_length: Optional[int] = None,
            dtype: str = "bf16", poison: bool = True,
            scale: Optional[float] = None) -> PrefillInputs:
    """Prefix rows [0, prefix_len) plus the new tokens' rows
    [prefix_len, prefix_len+Lq) are drawn; rows beyond are poisoned."""
    if max_length is None:
        max_length = prefix_len + Lq
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, Hq, Lq, D), dtype)
    k = _draw(rng, (B, Hkv, max_length, D), dtype)
    v = _draw(rng, (B, Hkv, max_length, D), dtype)
    T = prefix_len + Lq
    if poison and T < max_length:
        k[:, :, T:, :] = _nan_of(dtype)
        v[:, :, T:, :] = _nan_of(dtype)
    return PrefillInputs(dtype, q, k, v, prefix_len, scale)


# ----------------------------------------------------------------------------
# Top-k inputs
# ----------------------------------------------------------------------------
@dataclass
class TopkInputs:
    q: np.ndarray   # [b, h, n, d] float32
    k: np.ndarray
    v: np.ndarray
    topk: int


def topk(seed: int, b: int, h: int, n: int, d: int, k: int) -> TopkInputs:
    rng = np.random.default_rng(seed)
    q = _draw(rng, (b, h, n, d), "f32")
    kk = _draw(rng, (b, h, n, d), "f32")
    v = _draw(rng, (b, h, n, d), "f32")
    return TopkInputs(q, kk, v, k)


# ----------------------------------------------------------------------------
# The five named workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    params: dict = field(default_factory=dict)


WORKLOADS = {
    "decode_f32_tiny": Workload("decode_f32_tiny", dict(
        seed=1, B=1, Hq=2, Hkv=1, D=64, max_length=32, position_id=15,
        dtype="f32", scale=1.0 / 8.0)),
    "decode_gqa_static": Workload("decode_gqa_static", dict(
        seed=2, B=1, Hq=32, Hkv=8, D=128, max_length=8192,
        positions=(0, 100, 1000, 4000, 8000), dtype="bf16",
        scale=1.0 / np.sqrt(128.0))),
    "decode_ragged_b64": Workload("decode_ragged_b64", dict(
        seed=3, B=64, Hq=32, Hkv=8, D=128, max_length=8192, dtype="bf16",
        scale=1.0 / np.sqrt(128.0))),
    "prefill_prefix3072": Workload("prefill_prefix3072", dict(
        seed=4, B=1, Hq=16, Hkv=16, D=64, Lq=1024, prefix_len=3072,
        max_length=4096, dtype="bf16", scale=1.0 / 8.0)),
    "topk_c2psa": Workload("topk_c2psa", dict(
        seed=5, b=32, h=3, n=512, d=64, topk=64)),
}
