"""Plain fp64 definitions of the three attention cases — TEST INFRASTRUCTURE.

This is the oracle the HIP kernels are checked against. It is deliberately
slow and literal: every quantity is upcast losslessly to float64 (bf16 and
float32 inputs are exact in float64) and the definitions are written out
with NumPy primitives, with no blocking, fusion or reordering.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg use it. It shares no code with the HIP path.

Sources (cited by page title and section):

* [P1] "MiniCPM4 forward_step Attention Performance Fix" (VoxCPM issue 293):
  §3 (the fix) passes only cache rows [0, position_id] to SDPA with no mask,
  and argues this equals the lower-triangular mask and that position 0
  reduces to the identity; §4.1 (patched ``forward_step``) gives the head
  layout and ``enable_gqa=True``; §2.1/§2.3 give the original masked
  full-cache form.
* [P2] "step14_3 — batched attention: removing the per-head Python loop"
  (mini-vllm tutorial): the problem section (per-head loop), the solution
  section (bmm over heads, scale 1/sqrt(d_head), -inf mask, softmax, bmm)
  and the "going further" section (SDPA with ``is_causal``).
* [P3] "c2psa multi-head self-attention high-concurrency inference"
  (blog post): core implementation §2 (dynamic top-k sparsification:
  q·kᵀ, top-k per row, scatter into zeros, product with v) and the full
  C2PSA class (topk=64 default, grouped heads).

Readings where the pages are silent are listed in the design notes of the
repository; the ones that shape this file are stated next to the code.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def default_scale(D: int) -> float:
    """1/sqrt(D): SDPA's default scale [P1 §4.1] and the explicit
    ``/ math.sqrt(d_head)`` of [P2, solution section]."""
    return 1.0 / math.sqrt(D)


def _softmax(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis, max-subtracted (mathematically identical
    to the unshifted form; -inf entries get weight exactly 0)."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ----------------------------------------------------------------------------
# Decode  [P1 §3, §4.1]
# ----------------------------------------------------------------------------
def decode_sequence(q_b: np.ndarray, K_b: np.ndarray, V_b: np.ndarray,
                    L: int, scale: float) -> np.ndarray:
    """One sequence of a decode step.

    q_b: [Hq, D]; K_b, V_b: [Hkv, >=L, D]. Query head h reads kv head
    h // (Hq/Hkv) — consecutive query heads share a kv head, the grouping
    ``enable_gqa=True`` performs [P1 §4.1]. Only rows [0, L) are read; the
    slice bound is the causal mask [P1 §3]. L == 0 gives a zero row (reading:
    the pages never reach it; a zero row rather than NaN).
    """
    Hq, D = q_b.shape
    Hkv = K_b.shape[0]
    G = Hq // Hkv
    out = np.zeros((Hq, D), dtype=np.float64)
    if L <= 0:
        return out
    for g in range(Hkv):
        K = np.asarray(K_b[g, :L], dtype=np.float64)          # [L, D]
        V = np.asarray(V_b[g, :L], dtype=np.float64)          # [L, D]
        for h in range(g * G, (g + 1) * G):
            qh = np.asarray(q_b[h], dtype=np.float64)          # [D]
            s = scale * (K @ qh)                               # [L]
            out[h] = _softmax(s) @ V                           # [D]
    return out


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
           position_id: Optional[int] = None,
           seq_lens: Optional[np.ndarray] = None,
           scale: Optional[float] = None) -> np.ndarray:
    """Single-token decode over a static cache.

    q: [B, Hq, D]; k_cache, v_cache: [B, Hkv, max_length, D].
    With ``position_id`` every sequence attends to rows [0, position_id]
    (inclusive: the current token's K/V were written at ``position_id``
    before attending [P1 §4.1]). With ``seq_lens`` sequence b attends to
    rows [0, seq_lens[b]) clamped to [0, max_length].
    Returns float64 [B, Hq, D].
    """
    B, Hq, D = q.shape
    max_length = k_cache.shape[2]
    if scale is None:
        scale = default_scale(D)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        if seq_lens is None:
            L = position_id + 1
        else:
            L = int(min(max(int(seq_lens[b]), 0), max_length))
        out[b] = decode_sequence(q[b], k_cache[b], v_cache[b], L, scale)
    return out


def decode_append(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                  k_cache: np.ndarray, v_cache: np.ndarray,
                  position_id: Optional[int] = None,
                  seq_lens: Optional[np.ndarray] = None,
                  scale: Optional[float] = None):
    """The patched ``forward_step`` order [P1 §4.1]: first store the current
    token's key and value at its cache row, then attend over the valid rows.

    k_new, v_new: [B, Hkv, D]. The row of sequence b is ``position_id``, or
    ``seq_lens[b] - 1`` for a ragged batch (lengths clamped to
    [0, max_length]; a length-0 sequence has no current token, so nothing is
    stored — reading). Returns (out, k_cache', v_cache') with the caches
    copied, not modified in place.
    """
    B = q.shape[0]
    max_length = k_cache.shape[2]
    k2 = np.array(k_cache, copy=True)
    v2 = np.array(v_cache, copy=True)
    for b in range(B):
        if seq_lens is None:
            r = position_id
        else:
            r = int(min(max(int(seq_lens[b]), 0), max_length)) - 1
        if r >= 0:
            k2[b, :, r, :] = k_new[b]
            v2[b, :, r, :] = v_new[b]
    out = decode(q, k2, v2, position_id=position_id, seq_lens=seq_lens,
                 scale=scale)
    return out, k2, v2


def gather_pages(k_pages: np.ndarray, v_pages: np.ndarray,
                 block_table: np.ndarray, layout: str = "token"):
    """The logical caches [B, Hkv, max_blocks * page_size, D] of a paged
    cache: pages [num_pages, page_size, Hkv, D] hold rows token-major (the
    head after the token, as the prefix cache of [P2, problem section]
    stores K and V), or [num_pages, Hkv, page_size, D] head-major; row r of
    sequence b is row r % page_size of page block_table[b, r // page_size]
    (reading: the block-table indirection is not spelled out on the pages).
    Page indices are clamped to the pages that exist, as the library does.
    """
    if layout == "token":
        num_pages, page_size, Hkv, D = k_pages.shape
    else:
        num_pages, Hkv, page_size, D = k_pages.shape
    B, max_blocks = block_table.shape
    M = max_blocks * page_size
    k = np.empty((B, Hkv, M, D), dtype=k_pages.dtype)
    v = np.empty((B, Hkv, M, D), dtype=v_pages.dtype)
    for b in range(B):
        for r in range(M):
            pg = int(min(max(int(block_table[b, r // page_size]), 0),
                         num_pages - 1))
            if layout == "token":
                k[b, :, r, :] = k_pages[pg, r % page_size]
                v[b, :, r, :] = v_pages[pg, r % page_size]
            else:
                k[b, :, r, :] = k_pages[pg, :, r % page_size]
                v[b, :, r, :] = v_pages[pg, :, r % page_size]
    return k, v


def decode_paged(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                 block_table: np.ndarray,
                 position_id: Optional[int] = None,
                 seq_lens: Optional[np.ndarray] = None,
                 scale: Optional[float] = None,
                 layout: str = "token") -> np.ndarray:
    """Decode over a paged cache: the logical cache is gathered row by row
    (``gather_pages``) and attended to as in ``decode``."""
    k, v = gather_pages(k_pages, v_pages, block_table, layout)
    return decode(q, k, v, position_id=position_id, seq_lens=seq_lens,
                  scale=scale)


def rope_rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotary position embedding of the last axis in float64, no rounding.

    [P1 §4.1] applies ``apply_rotary_pos_emb(q, k, cos, sin)`` to the
    current token's query and key before the cache write; the function body
    is not on the page. Reading: the rotate-half convention, element j paired
    with element j + D/2: out = x * cos + rotate_half(x) * sin with
    rotate_half(x) = (-x[D/2:], x[:D/2]). ``cos`` and ``sin`` broadcast
    against x (full length D).
    """
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    rh = np.concatenate([-x[..., h:], x[..., :h]], axis=-1)
    return x * np.asarray(cos, np.float64) + rh * np.asarray(sin, np.float64)


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, to nearest even, to the storage type
    ``dtype`` ("bf16": 8 significant bits, float32's exponent range; "f32"),
    returned as float64."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    e = np.floor(np.log2(np.abs(x[fin])))
    # guard log2 rounding at exact powers of two
    e = np.where(np.abs(x[fin]) < 2.0 ** e, e - 1, e)
    e = np.where(np.abs(x[fin]) >= 2.0 ** (e + 1), e + 1, e)
    ulp = 2.0 ** (np.maximum(e, -126.0) - 7.0)
    out[fin] = np.rint(x[fin] / ulp) * ulp
    big = np.abs(out) > 3.3895313892515355e38    # beyond the largest bf16
    out[big] = np.sign(out[big]) * np.inf
    return out


def decode_append_rope(q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                       cos: np.ndarray, sin: np.ndarray,
                       k_cache: np.ndarray, v_cache: np.ndarray,
                       dtype: str,
                       position_id: Optional[int] = None,
                       seq_lens: Optional[np.ndarray] = None,
                       scale: Optional[float] = None):
    """The patched ``forward_step`` with its position embedding [P1 §4.1]:
    rotate the query and the new key (``rope_rotate``; ``cos``, ``sin``
    [B, D] give sequence b's current position, shared by all heads), round
    both to the storage type (reading: the rotated tensors are the model's
    dtype, as SDPA and the cache receive them), then store and attend as in
    ``decode_append``. Returns (out, k_cache', v_cache')."""
    c = np.asarray(cos, np.float64)[:, None, :]
    s = np.asarray(sin, np.float64)[:, None, :]
    q_r = round_to_storage(rope_rotate(q, c, s), dtype)
    k_r = round_to_storage(rope_rotate(k_new, c, s), dtype)
    return decode_append(q_r, k_r, v_new, k_cache, v_cache,
                         position_id=position_id, seq_lens=seq_lens,
                         scale=scale)


# ----------------------------------------------------------------------------
# Causal prefill against a cached prefix  [P2 solution section]
# ----------------------------------------------------------------------------
def prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
            prefix_len: int, scale: Optional[float] = None) -> np.ndarray:
    """Prefill of Lq new tokens whose K/V sit at cache rows
    [prefix_len, prefix_len + Lq).

    q: [B, Hq, Lq, D] (head-major, the SDPA convention of [P1 §4.1] and
    [P2 going-further section]); caches [B, Hkv, max_length, D].
    New token i attends to rows [0, prefix_len + i] (reading: the mask is
    aligned to the bottom-right, so with prefix_len == 0 it is the ordinary
    causal mask). For each head: scores = Q·Kᵀ·scale over all valid rows,
    masked entries set to -inf, softmax per row, then ·V [P2 solution].
    Returns float64 [B, Hq, Lq, D].
    """
    B, Hq, Lq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = default_scale(D)
    T = prefix_len + Lq
    i = np.arange(Lq)[:, None]
    j = np.arange(T)[None, :]
    masked = j > prefix_len + i                                # [Lq, T]
    out = np.zeros((B, Hq, Lq, D), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            Q = np.asarray(q[b, h], dtype=np.float64)            # [Lq, D]
            K = np.asarray(k_cache[b, g, :T], dtype=np.float64)  # [T, D]
            V = np.asarray(v_cache[b, g, :T], dtype=np.float64)
            s = (Q @ K.T) * scale                                # [Lq, T]
            s = np.where(masked, -np.inf, s)
            out[b, h] = _softmax(s) @ V
    return out


def prefill_paged(q: np.ndarray, k_pages: np.ndarray, v_pages: np.ndarray,
                  block_table: np.ndarray, prefix_len: int,
                  scale: Optional[float] = None,
                  layout: str = "token") -> np.ndarray:
    """Prefill whose cache is paged (the prefix cache of [P2, problem
    section] keeps K and V per token): the logical cache is gathered
    (``gather_pages``) and ``prefill`` runs on it."""
    k, v = gather_pages(k_pages, v_pages, block_table, layout)
    return prefill(q, k, v, prefix_len, scale)


# ----------------------------------------------------------------------------
# Top-k sparsified scores  [P3 core implementation §2]
# ----------------------------------------------------------------------------
def topk_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """s[i, j] = Σ_d q[i, d]·k[j, d] in float64, no scale [P3 §2].

    q, k: [n, d] float32. Each product of two float32 values is exact in
    float64; the sum runs over d in ascending order for every (i, j), so
    identical key rows give bit-identical scores (needed for exact ties).
    """
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    s = np.zeros((q64.shape[0], k64.shape[0]), dtype=np.float64)
    for d in range(q64.shape[1]):
        s += q64[:, d, None] * k64[None, :, d]
    return s


def topk_select(s: np.ndarray, topk: int) -> np.ndarray:
    """Indices of the ``topk`` largest scores per row, ordered by (score
    descending, index ascending) — ties go to the lower index (reading: the
    page's ``torch.topk`` leaves equal scores unordered). Returned sorted
    ascending per row. -0.0 and +0.0 compare equal here."""
    order = np.argsort(-s, axis=-1, kind="stable")[:, :topk]
    return np.sort(order, axis=-1)


def topk_sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray, topk: int,
                return_details: bool = False):
    """Top-k sparse attention [P3 §2]: scores q·kᵀ (no scale), keep the
    ``topk`` largest per row, zero the rest, multiply by v. No softmax: the
    page's code applies none (its prose says "before softmax" but the listed
    function returns ``sparse_attn @ v`` directly; the code is followed).

    q, k, v: [b, h, n, d] float32. Returns float64 [b, h, n, d], and with
    ``return_details`` also the selected indices [b, h, n, topk] (ascending)
    and the gap between the topk-th and (topk+1)-th largest scores per row
    (+inf when topk == n).
    """
    bsz, H, n, d = q.shape
    out = np.zeros((bsz, H, n, d), dtype=np.float64)
    idx_all = np.zeros((bsz, H, n, topk), dtype=np.int64)
    gap_all = np.full((bsz, H, n), np.inf, dtype=np.float64)
    for b in range(bsz):
        for h in range(H):
            s = topk_scores(q[b, h], k[b, h])                    # [n, n]
            idx = topk_select(s, topk)                           # [n, topk]
            sel = np.take_along_axis(s, idx, axis=-1)            # [n, topk]
            v64 = np.asarray(v[b, h], dtype=np.float64)          # [n, d]
            out[b, h] = np.einsum("it,itd->id", sel, v64[idx])
            idx_all[b, h] = idx
            if topk < n:
                srt = -np.sort(-s, axis=-1)
                gap_all[b, h] = srt[:, topk - 1] - srt[:, topk]
    if return_details:
        return out, idx_all, gap_all
    return out


def topk_causal_select(s_row: np.ndarray, i: int, topk: int) -> np.ndarray:
    """Key indices row i keeps in the decoder form of top-k sparsification
    [P3 "further thoughts": a causal model attends only to the tokens on its
    left, and each query keeps its most recent k/2 tokens]. Reading:

    * the candidates are j <= i (the query's own token included);
    * when i + 1 <= topk every candidate is kept (nothing to sparsify);
    * otherwise the r = floor(topk / 2) most recent keys, j in (i - r, i],
      are kept unconditionally and the remaining topk - r slots go to the
      largest scores among the older keys j <= i - r, equal scores to the
      lower index (as in ``topk_select``).

    Returns the kept indices in ascending order (min(topk, i + 1) of them).
    """
    if i + 1 <= topk:
        return np.arange(i + 1)
    r = topk // 2
    older = s_row[: i + 1 - r]
    best = np.argsort(-older, kind="stable")[: topk - r]
    return np.sort(np.concatenate([best, np.arange(i + 1 - r, i + 1)]))


def topk_causal_sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                       topk: int, return_details: bool = False):
    """Decoder-causal top-k sparse attention: the scores of [P3 §2] (q·kᵀ,
    no scale, no softmax), with row i keeping the keys chosen by
    ``topk_causal_select``; every other entry of row i is zero, and the
    output row is the kept scores times the kept rows of v.

    q, k, v: [b, h, n, d] float32. Returns float64 [b, h, n, d]; with
    ``return_details`` also the kept indices [b, h, n, topk] (ascending,
    padded with -1 when a row keeps fewer than topk) and, per row, the gap
    between the last older score taken and the first one left out (+inf
    when the row keeps every candidate or no older key is left out).
    """
    bsz, H, n, d = q.shape
    out = np.zeros((bsz, H, n, d), dtype=np.float64)
    idx_all = np.full((bsz, H, n, topk), -1, dtype=np.int64)
    gap_all = np.full((bsz, H, n), np.inf, dtype=np.float64)
    r = topk // 2
    for b in range(bsz):
        for h in range(H):
            s = topk_scores(q[b, h], k[b, h])                    # [n, n]
            v64 = np.asarray(v[b, h], dtype=np.float64)
            for i in range(n):
                sel = topk_causal_select(s[i], i, topk)
                out[b, h, i] = s[i, sel] @ v64[sel]
                idx_all[b, h, i, : len(sel)] = sel
                n_old = i + 1 - r
                if i + 1 > topk and topk - r < n_old:
                    srt = -np.sort(-s[i, :n_old])
                    gap_all[b, h, i] = srt[topk - r - 1] - srt[topk - r]
    if return_details:
        return out, idx_all, gap_all
    return out
