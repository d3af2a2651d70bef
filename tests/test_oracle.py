"""Pins for the fp64 oracle (CPU only).

None of these re-types the oracle's formula. Each checks it against
something fixed independently of it:

* hand-worked examples from the pages' definitions (``tests/golden``);
* closed forms (single row, uniform weights, constant V, k=1, k=n);
* library routines the pages themselves call: PyTorch's CPU
  ``scaled_dot_product_attention`` in float64 (sliced cache with
  ``enable_gqa``, the original full-cache bool mask, ``is_causal``);
* the definitions in an independent form: all heads in one batched product
  with the causal condition applied by selection; top-k as a keep mask
  ("score >= the row's k-th largest") times v;
* invariants the pages state (slice == mask, batched == per-head results,
  GQA == MHA with repeated K/V, position 0 == identity);
* brute force over all k-subsets for top-k on tiny inputs.

A plausible slip in the oracle (dropped scale, off-by-one length, wrong head
map, transposed operand, softmax applied in top-k, wrong tie order) fails at
least one test here.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


def _sdpa_sliced(q, k_cache, v_cache, L, scale=None):
    """The pages' patched decode: SDPA over cache rows [0, L), enable_gqa."""
    qt = _t(q)[:, :, None, :]                       # [B, Hq, 1, D]
    kt = _t(k_cache[:, :, :L, :])
    vt = _t(v_cache[:, :, :L, :])
    o = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True,
                                       scale=scale)
    return o[:, :, 0, :].numpy()


# ----------------------------------------------------------------------------
# Golden hand-worked examples
# ----------------------------------------------------------------------------
def test_decode_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "decode_hand.json")))
    q = np.array(g["q"])
    max_len = g["max_length"]
    D = q.shape[-1]
    k = np.full((1, 1, max_len, D), np.nan)
    v = np.full((1, 1, max_len, D), np.nan)
    n = len(g["k_rows"])
    k[0, 0, :n] = g["k_rows"]
    v[0, 0, :n] = g["v_rows"]
    out = oracle.decode(q, k, v, position_id=g["position_id"])
    np.testing.assert_allclose(out, np.array(g["expected"]),
                               rtol=0, atol=g["tolerance"])


def test_prefill_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "prefill_hand.json")))
    q = np.array(g["q"])
    k = np.array(g["k_rows"])[None, None]
    v = np.array(g["v_rows"])[None, None]
    out = oracle.prefill(q, k, v, prefix_len=g["prefix_len"])
    np.testing.assert_allclose(out, np.array(g["expected"]),
                               rtol=0, atol=g["tolerance"])


def test_topk_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "topk_hand.json")))
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    v = np.array(g["v"], np.float32)
    for case in g["cases"]:
        out, idx, _ = oracle.topk_sparse(q, k, v, case["topk"],
                                         return_details=True)
        rows = case["rows"]
        np.testing.assert_allclose(out[0, 0, rows], np.array(case["expected"]),
                                   rtol=0, atol=g["tolerance"])
        assert idx[0, 0, rows].tolist() == case["indices"]


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_position0_returns_v0_exactly(dtype):
    inp = synth.decode_uniform(11, B=2, Hq=8, Hkv=2, D=64, max_length=16,
                               position_id=0, dtype=dtype)
    q = synth.as_f32(inp.q, dtype)
    k = synth.as_f32(inp.k_cache, dtype)
    v = synth.as_f32(inp.v_cache, dtype)
    out = oracle.decode(q, k, v, position_id=0)
    expect = np.repeat(v[:, :, 0, :], 4, axis=1).astype(np.float64)
    assert np.array_equal(out, expect)


def test_decode_zero_query_gives_mean_of_valid_rows():
    # q = 0 makes every score 0, so the weights are uniform over exactly the
    # valid rows: an off-by-one in the length shows as a different mean.
    rng = np.random.default_rng(0)
    B, Hq, Hkv, D, M = 1, 4, 2, 8, 20
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    q = np.zeros((B, Hq, D))
    for p in (0, 1, 7, 19):
        out = oracle.decode(q, k, v, position_id=p)
        mean = v[:, :, :p + 1, :].mean(axis=2)
        np.testing.assert_allclose(out, np.repeat(mean, 2, axis=1),
                                   rtol=0, atol=1e-14)


def test_decode_constant_v_rows_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 6, 16)) * 3
    k = rng.standard_normal((2, 3, 40, 16)) * 3
    v = np.full((2, 3, 40, 16), 2.5)
    out = oracle.decode(q, k, v, seq_lens=np.array([40, 5]))
    np.testing.assert_allclose(out, 2.5, rtol=0, atol=1e-13)


@pytest.mark.parametrize("B,Hq,Hkv,D,M,p", [
    (1, 2, 1, 64, 32, 15), (2, 32, 8, 128, 64, 40), (1, 4, 4, 8, 9, 8),
    (3, 6, 2, 16, 10, 0)])
def test_decode_matches_torch_sdpa_on_sliced_cache(B, Hq, Hkv, D, M, p):
    rng = np.random.default_rng(B * 1000 + p)
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    out = oracle.decode(q, k, v, position_id=p)
    ref = _sdpa_sliced(q, k, v, p + 1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # an explicit scale is honoured, not replaced by the default
    out2 = oracle.decode(q, k, v, position_id=p, scale=0.37)
    ref2 = _sdpa_sliced(q, k, v, p + 1, scale=0.37)
    np.testing.assert_allclose(out2, ref2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("p", [0, 5, 11])
def test_decode_append_follows_the_page_forward_step(p):
    # [P1 §4.1]: key_cache[:, :, position_id, :] = key_states (same for V),
    # then SDPA over the slice [0, position_id] with enable_gqa. Row p of the
    # incoming caches holds NaN: only the stored values may reach the output.
    rng = np.random.default_rng(500 + p)
    B, Hq, Hkv, D, M = 2, 4, 2, 8, 12
    q = rng.standard_normal((B, Hq, D))
    kn = rng.standard_normal((B, Hkv, D))
    vn = rng.standard_normal((B, Hkv, D))
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    k[:, :, p] = np.nan
    v[:, :, p] = np.nan
    out, k2, v2 = oracle.decode_append(q, kn, vn, k, v, position_id=p)
    kt, vt = _t(k).clone(), _t(v).clone()
    kt[:, :, p, :] = _t(kn)
    vt[:, :, p, :] = _t(vn)
    ref = _sdpa_sliced(q, kt.numpy(), vt.numpy(), p + 1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(k2, kt.numpy())
    np.testing.assert_array_equal(v2, vt.numpy())
    assert np.isnan(k[:, :, p]).all()  # the inputs are not modified


def test_decode_append_ragged_rows_and_empty_sequence():
    rng = np.random.default_rng(77)
    B, Hq, Hkv, D, M = 3, 2, 1, 4, 6
    q = rng.standard_normal((B, Hq, D))
    kn = rng.standard_normal((B, Hkv, D))
    vn = rng.standard_normal((B, Hkv, D))
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    lens = np.array([0, 1, 6])
    out, k2, v2 = oracle.decode_append(q, kn, vn, k, v, seq_lens=lens)
    # length 0: nothing stored, zero output
    np.testing.assert_array_equal(k2[0], k[0])
    assert np.all(out[0] == 0)
    # otherwise the new token is the last valid row, the rest is untouched
    for b, r in ((1, 0), (2, 5)):
        np.testing.assert_array_equal(k2[b, :, r], kn[b])
        np.testing.assert_array_equal(v2[b, :, r], vn[b])
        keep = [i for i in range(M) if i != r]
        np.testing.assert_array_equal(k2[b][:, keep], k[b][:, keep])
        ref = _sdpa_sliced(q[b:b + 1], k2[b:b + 1], v2[b:b + 1], int(lens[b]))
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)
    # length 1 attends to the new row alone: output = v_new
    np.testing.assert_allclose(out[1], np.repeat(vn[1], Hq, axis=0),
                               rtol=0, atol=1e-15)


def _rope_tables(positions, D, base=10000.0):
    """Standard rotary tables: angle pos * base^(-2j/D) for pair j, the same
    angle on elements j and j + D/2."""
    inv = base ** (-np.arange(0, D, 2) / D)
    ang = np.asarray(positions, np.float64)[:, None] * inv[None, :]
    ang = np.concatenate([ang, ang], axis=-1)
    return np.cos(ang), np.sin(ang)


def test_rope_quarter_and_half_turns():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    assert oracle.rope_rotate(x, np.zeros(4), np.ones(4)).tolist() == \
        [-3.0, -4.0, 1.0, 2.0]
    assert oracle.rope_rotate(x, -np.ones(4), np.zeros(4)).tolist() == \
        [-1.0, -2.0, -3.0, -4.0]
    assert oracle.rope_rotate(x, np.ones(4), np.zeros(4)).tolist() == \
        x.tolist()


def test_rope_is_complex_multiplication_of_half_pairs():
    # element j and j + D/2 as the complex number x_j + i x_{j+D/2}, turned
    # by e^{i theta_j}
    rng = np.random.default_rng(60)
    D = 16
    x = rng.standard_normal((5, 3, D))
    c, s = _rope_tables([0, 1, 7, 100, 4095], D)
    got = oracle.rope_rotate(x, c[:, None, :], s[:, None, :])
    z = (x[..., :D // 2] + 1j * x[..., D // 2:]) * \
        np.exp(1j * np.arctan2(s, c)[:, None, :D // 2])
    np.testing.assert_allclose(got, np.concatenate([z.real, z.imag], -1),
                               rtol=0, atol=1e-13)


def test_rope_scores_depend_on_the_position_difference_only():
    rng = np.random.default_rng(61)
    D = 32
    q = rng.standard_normal(D)
    k = rng.standard_normal(D)
    pos = np.array([5, 2, 105, 102, 3000, 2997])
    c, s = _rope_tables(pos, D)
    qr = oracle.rope_rotate(q, c, s)
    kr = oracle.rope_rotate(k, c, s)
    d1 = qr[0] @ kr[1]
    assert abs(qr[2] @ kr[3] - d1) < 1e-10
    assert abs(qr[4] @ kr[5] - d1) < 1e-10
    assert abs(q @ k - d1) > 1e-3  # the rotation does change the score


def test_round_to_storage_bf16_ties_and_library_encoder():
    one = 1.0
    r = oracle.round_to_storage(np.array([one + 2.0 ** -8, one + 3 * 2.0 ** -8,
                                          -(one + 2.0 ** -8 + 2.0 ** -30),
                                          2.0 ** -130, 0.0, -0.0]), "bf16")
    assert r[0] == 1.0                      # tie to even (down)
    assert r[1] == 1.0 + 2.0 ** -6          # tie to even (up)
    assert r[2] == -(1.0 + 2.0 ** -7)       # above the tie: away from 1
    assert r[3] == 2.0 ** -130              # subnormal, exact
    assert r[4] == 0.0 and np.signbit(r[5])
    # against the bit-level float32 -> bf16 encoder on float32 values
    rng = np.random.default_rng(62)
    x = (rng.standard_normal(20000) *
         np.exp(rng.uniform(-40, 40, 20000))).astype(np.float32)
    ref = synth.bf16_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(
        oracle.round_to_storage(x.astype(np.float64), "bf16"), ref)


def test_decode_append_rope_with_identity_tables_is_the_plain_append():
    rng = np.random.default_rng(63)
    B, Hq, Hkv, D, M = 3, 4, 2, 8, 10
    enc = lambda a: synth.bf16_to_f32(synth.f32_to_bf16_bits(
        a.astype(np.float32))).astype(np.float64)
    q = enc(rng.standard_normal((B, Hq, D)))
    kn = enc(rng.standard_normal((B, Hkv, D)))
    vn = enc(rng.standard_normal((B, Hkv, D)))
    k = enc(rng.standard_normal((B, Hkv, M, D)))
    v = enc(rng.standard_normal((B, Hkv, M, D)))
    lens = np.array([1, 10, 4])
    a = oracle.decode_append(q, kn, vn, k, v, seq_lens=lens)
    b = oracle.decode_append_rope(q, kn, vn, np.ones((B, D)),
                                  np.zeros((B, D)), k, v, "bf16",
                                  seq_lens=lens)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("p", [0, 6])
def test_decode_append_rope_follows_the_page_forward_step(p):
    # [P1 §4.1]: rotate q and k, store k (and v) at position_id, SDPA over
    # [0, position_id]. Rotation by complex multiplication, rounding to
    # float32 by numpy, attention by torch's SDPA.
    rng = np.random.default_rng(64 + p)
    B, Hq, Hkv, D, M = 2, 4, 2, 8, 9
    f = lambda a: a.astype(np.float32).astype(np.float64)
    q = f(rng.standard_normal((B, Hq, D)))
    kn = f(rng.standard_normal((B, Hkv, D)))
    vn = f(rng.standard_normal((B, Hkv, D)))
    k = f(rng.standard_normal((B, Hkv, M, D)))
    v = f(rng.standard_normal((B, Hkv, M, D)))
    k[:, :, p] = np.nan
    c, s = _rope_tables([p, p], D)
    out, k2, v2 = oracle.decode_append_rope(q, kn, vn, c, s, k, v, "f32",
                                            position_id=p)
    th = np.arctan2(s, c)[:, None, :D // 2]
    turn = lambda a: (lambda z: np.concatenate([z.real, z.imag], -1))(
        (a[..., :D // 2] + 1j * a[..., D // 2:]) * np.exp(1j * th))
    qr, kr = f(turn(q)), f(turn(kn))
    kt = np.array(k, copy=True)
    kt[:, :, p] = kr
    vt = np.array(v, copy=True)
    vt[:, :, p] = vn
    ref = _sdpa_sliced(qr, kt, vt, p + 1)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(k2, kt)
    np.testing.assert_array_equal(v2, vt)


def test_decode_paged_equals_contiguous_and_sdpa():
    # a contiguous cache scattered over shuffled token-major pages (spare
    # pages hold NaN): the paged oracle must see exactly the same rows
    rng = np.random.default_rng(91)
    B, Hq, Hkv, D, M, ps = 3, 4, 2, 8, 24, 8
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, M, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, M, D)).astype(np.float32)
    kp, vp, table = synth.paginate(k, v, ps, seed=91, dtype="f32")
    assert len(set(table.ravel().tolist())) == B * M // ps
    lens = np.array([M, 1, 13])
    out = oracle.decode_paged(q, kp, vp, table, seq_lens=lens)
    np.testing.assert_array_equal(out, oracle.decode(q, k, v, seq_lens=lens))
    # head-major pages hold the same rows: kp_h[p, g, r] == kp[p, r, g]
    kh, vh, th = synth.paginate(k, v, ps, seed=91, dtype="f32", layout="head")
    np.testing.assert_array_equal(th, table)
    np.testing.assert_array_equal(kh, kp.transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(
        oracle.decode_paged(q, kh, vh, th, seq_lens=lens, layout="head"), out)
    for b in range(B):
        ref = _sdpa_sliced(q[b:b + 1], k[b:b + 1], v[b:b + 1], int(lens[b]))
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)
    # the page of row r is table[b, r // ps]: swapping two table entries of
    # a sequence swaps those blocks of rows
    t2 = table.copy()
    t2[0, [0, 2]] = t2[0, [2, 0]]
    k2 = k.copy()
    k2[0, :, 0:8], k2[0, :, 16:24] = k[0, :, 16:24], k[0, :, 0:8]
    v2 = v.copy()
    v2[0, :, 0:8], v2[0, :, 16:24] = v[0, :, 16:24], v[0, :, 0:8]
    np.testing.assert_array_equal(
        oracle.decode_paged(q, kp, vp, t2, position_id=M - 1),
        oracle.decode(q, k2, v2, position_id=M - 1))


def test_decode_sliced_equals_masked_full_cache():
    # The page's original form: full cache, bool mask arange(max) <= pos.
    rng = np.random.default_rng(2)
    B, Hq, Hkv, D, M = 2, 8, 2, 32, 50
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    for p in (0, 13, 49):
        mask = (torch.arange(M) <= p)[None, :]   # [1 query, max_length]
        ref = F.scaled_dot_product_attention(
            _t(q)[:, :, None], _t(k), _t(v), attn_mask=mask,
            enable_gqa=True)[:, :, 0].numpy()
        out = oracle.decode(q, k, v, position_id=p)
        np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_decode_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, D, M = 2, 12, 3, 16, 30
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    kr = torch.repeat_interleave(_t(k), Hq // Hkv, dim=1).numpy()
    vr = torch.repeat_interleave(_t(v), Hq // Hkv, dim=1).numpy()
    lens = np.array([30, 11])
    np.testing.assert_allclose(oracle.decode(q, k, v, seq_lens=lens),
                               oracle.decode(q, kr, vr, seq_lens=lens),
                               rtol=0, atol=1e-14)


def test_decode_ragged_equals_per_sequence_sdpa():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, D, M = 4, 8, 4, 32, 33
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, M, D))
    v = rng.standard_normal((B, Hkv, M, D))
    lens = np.array([1, 33, 17, 2])
    out = oracle.decode(q, k, v, seq_lens=lens)
    for b in range(B):
        ref = _sdpa_sliced(q[b:b + 1], k[b:b + 1], v[b:b + 1], lens[b])
        np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)


def test_decode_length_zero_and_clamp():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 2, 8))
    k = rng.standard_normal((3, 1, 6, 8))
    v = rng.standard_normal((3, 1, 6, 8))
    out = oracle.decode(q, k, v, seq_lens=np.array([0, 100, -4]))
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    ref = _sdpa_sliced(q[1:2], k[1:2], v[1:2], 6)
    np.testing.assert_allclose(out[1:2], ref, rtol=0, atol=1e-12)


def test_decode_two_row_logistic_closed_form():
    # L = 2: weights are the logistic function of the score difference.
    rng = np.random.default_rng(6)
    D = 16
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, 2, D))
    v = rng.standard_normal((1, 1, 2, D))
    s = (k[0, 0] @ q[0, 0]) / math.sqrt(D)
    w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    expect = w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1]
    out = oracle.decode(q, k, v, position_id=1)
    np.testing.assert_allclose(out[0, 0], expect, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
# Prefill
# ----------------------------------------------------------------------------
def _bottom_right_mask(Lq, prefix):
    i = torch.arange(Lq)[:, None]
    j = torch.arange(prefix + Lq)[None, :]
    return j <= prefix + i


@pytest.mark.parametrize("B,Hq,Hkv,D,Lq,prefix", [
    (1, 4, 4, 16, 7, 9), (2, 8, 2, 32, 33, 0), (1, 2, 1, 8, 1, 20),
    (1, 16, 16, 64, 40, 64)])
def test_prefill_matches_torch_sdpa_bottom_right_mask(B, Hq, Hkv, D, Lq,
                                                      prefix):
    rng = np.random.default_rng(Lq * 100 + prefix)
    T = prefix + Lq
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, T + 3, D))
    v = rng.standard_normal((B, Hkv, T + 3, D))
    out = oracle.prefill(q, k, v, prefix_len=prefix)
    ref = F.scaled_dot_product_attention(
        _t(q), _t(k[:, :, :T]), _t(v[:, :, :T]),
        attn_mask=_bottom_right_mask(Lq, prefix), enable_gqa=True).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("layout", ["token", "head"])
def test_prefill_paged_equals_contiguous_and_sdpa(layout):
    # a prefix cache cut into shuffled pages (spare pages and rows past the
    # new tokens hold NaN): the paged prefill sees exactly the contiguous rows
    rng = np.random.default_rng(95)
    B, Hq, Hkv, D, ps, Lq, prefix = 2, 4, 2, 8, 8, 11, 13
    M = 32
    q = rng.standard_normal((B, Hq, Lq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, M, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, M, D)).astype(np.float32)
    k[:, :, prefix + Lq:] = np.nan
    v[:, :, prefix + Lq:] = np.nan
    kp, vp, table = synth.paginate(k, v, ps, seed=95, dtype="f32",
                                   layout=layout)
    out = oracle.prefill_paged(q, kp, vp, table, prefix, layout=layout)
    np.testing.assert_array_equal(out, oracle.prefill(q, k, v, prefix))
    T = prefix + Lq
    ref = F.scaled_dot_product_attention(
        _t(q), _t(k[:, :, :T]), _t(v[:, :, :T]),
        attn_mask=_bottom_right_mask(Lq, prefix), enable_gqa=True).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # swapping two blocks' table entries swaps those rows of the cache
    t2 = table.copy()
    t2[1, [0, 1]] = t2[1, [1, 0]]
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 0:8], k2[1, :, 8:16] = k[1, :, 8:16], k[1, :, 0:8]
    v2[1, :, 0:8], v2[1, :, 8:16] = v[1, :, 8:16], v[1, :, 0:8]
    np.testing.assert_array_equal(
        oracle.prefill_paged(q, kp, vp, t2, prefix, layout=layout),
        oracle.prefill(q, k2, v2, prefix))


def test_prefill_prefix0_equals_is_causal():
    # The going-further section's SDPA call with is_causal=True is exact
    # when there is no prefix.
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 4, 24, 16))
    k = rng.standard_normal((1, 4, 24, 16))
    v = rng.standard_normal((1, 4, 24, 16))
    ref = F.scaled_dot_product_attention(_t(q), _t(k), _t(v),
                                         is_causal=True).numpy()
    np.testing.assert_allclose(oracle.prefill(q, k, v, 0), ref,
                               rtol=0, atol=1e-12)


def test_prefill_row_equals_decode_at_prefix_plus_i():
    rng = np.random.default_rng(8)
    B, Hq, Hkv, D, Lq, prefix = 2, 8, 4, 16, 5, 11
    q = rng.standard_normal((B, Hq, Lq, D))
    k = rng.standard_normal((B, Hkv, prefix + Lq, D))
    v = rng.standard_normal((B, Hkv, prefix + Lq, D))
    out = oracle.prefill(q, k, v, prefix)
    for i in range(Lq):
        dec = oracle.decode(q[:, :, i], k, v, position_id=prefix + i)
        np.testing.assert_allclose(out[:, :, i], dec, rtol=0, atol=1e-14)


def test_prefill_token_major_all_heads_at_once():
    # "step14_3 — batched attention", solution section: every head in one
    # batched product over token-major Q [seq, H, d], K/V [total, H, d], the
    # bottom-right causal condition (new token t sees key s iff s <= prefix
    # + t) applied by selection, and the heads' outputs side by side in
    # [seq, H*d]. Written as one batched contraction per step, not per head.
    rng = np.random.default_rng(9)
    H, d, Lq, prefix = 6, 16, 9, 13
    T = prefix + Lq
    Q = rng.standard_normal((Lq, H, d))
    Kf = rng.standard_normal((T, H, d))
    Vf = rng.standard_normal((T, H, d))
    sc = torch.einsum("thd,shd->hts", _t(Q), _t(Kf)) / math.sqrt(d)
    allowed = torch.arange(T)[None, :] <= prefix + torch.arange(Lq)[:, None]
    sc = torch.where(allowed[None], sc, torch.tensor(float("-inf"),
                                                     dtype=sc.dtype))
    w = torch.exp(sc - sc.amax(dim=-1, keepdim=True))
    w = w / w.sum(dim=-1, keepdim=True)
    ref = torch.einsum("hts,shd->thd", w, _t(Vf)).reshape(Lq, H * d).numpy()
    out = oracle.prefill(Q.transpose(1, 0, 2)[None], Kf.transpose(1, 0, 2)[None],
                         Vf.transpose(1, 0, 2)[None], prefix)
    out_tm = out[0].transpose(1, 0, 2).reshape(Lq, H * d)
    np.testing.assert_allclose(out_tm, ref, rtol=0, atol=1e-12)


def test_prefill_never_reads_past_new_tokens():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 2, 4, 8))
    k = rng.standard_normal((1, 2, 12, 8))
    v = rng.standard_normal((1, 2, 12, 8))
    k[:, :, 7:] = np.nan
    v[:, :, 7:] = np.nan
    out = oracle.prefill(q, k, v, prefix_len=3)
    assert np.all(np.isfinite(out))


# ----------------------------------------------------------------------------
# Top-k
# ----------------------------------------------------------------------------
def test_topk_k_equals_n_is_dense_product_without_softmax():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 3, 20, 8)).astype(np.float32)
    k = rng.standard_normal((2, 3, 20, 8)).astype(np.float32)
    v = rng.standard_normal((2, 3, 20, 8)).astype(np.float32)
    out = oracle.topk_sparse(q, k, v, 20)
    qt, kt, vt = _t(q), _t(k), _t(v)
    ref = torch.matmul(torch.matmul(qt, kt.transpose(-2, -1)), vt).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)


def test_topk_k1_is_max_score_times_argmax_row():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    k = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    v = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    out = oracle.topk_sparse(q, k, v, 1)
    s = torch.matmul(_t(q), _t(k).transpose(-2, -1))
    smax, arg = s.max(dim=-1)
    ref = smax[..., None] * torch.gather(
        _t(v), 2, arg[..., None].expand(-1, -1, -1, 8))
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


def test_topk_keep_mask_product_form():
    # c2psa page, core implementation §2: keep each row's k largest scores,
    # zero the rest, multiply by v (no scale, no softmax). Here the kept set
    # is a boolean mask "score >= the row's k-th largest score" (tie-free
    # random data, so the mask holds exactly k entries) and the product is
    # the masked score matrix times v.
    rng = np.random.default_rng(14)
    q = rng.standard_normal((2, 3, 64, 16)).astype(np.float32)
    k = rng.standard_normal((2, 3, 64, 16)).astype(np.float32)
    v = rng.standard_normal((2, 3, 64, 16)).astype(np.float32)
    kk = 10
    s64 = q.astype(np.float64) @ np.swapaxes(k.astype(np.float64), -1, -2)
    kth = -np.partition(-s64, kk - 1, axis=-1)[..., kk - 1:kk]
    keep = s64 >= kth
    assert np.all(keep.sum(axis=-1) == kk)
    ref = np.where(keep, s64, 0.0) @ v.astype(np.float64)
    out, myidx, _ = oracle.topk_sparse(q, k, v, kk, return_details=True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)
    kept_idx = np.nonzero(keep)[-1].reshape(2, 3, 64, kk)
    assert np.array_equal(kept_idx, myidx)


def test_topk_brute_force_over_all_subsets():
    # The top-k set is the k-subset with the largest score sum; among equal
    # sums the lexicographically smallest sorted index tuple (lower indices
    # win ties). Enumerate every subset.
    rng = np.random.default_rng(15)
    n, d = 8, 3
    for trial in range(6):
        q = rng.integers(-3, 4, (1, 1, n, d)).astype(np.float32)
        k = rng.integers(-3, 4, (1, 1, n, d)).astype(np.float32)
        v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        for topk in (1, 3, 5, 8):
            out, idx, _ = oracle.topk_sparse(q, k, v, topk,
                                             return_details=True)
            for i in range(n):
                s = [float(np.dot(q[0, 0, i].astype(np.float64),
                                  k[0, 0, j].astype(np.float64)))
                     for j in range(n)]
                best = None
                for sub in itertools.combinations(range(n), topk):
                    key = tuple(sorted((-s[j], j) for j in sub))
                    if best is None or key < best[0]:
                        best = (key, sub)
                assert tuple(idx[0, 0, i]) == best[1]
                expect = sum(s[j] * v[0, 0, j].astype(np.float64)
                             for j in best[1])
                np.testing.assert_allclose(out[0, 0, i], expect, rtol=0,
                                           atol=1e-12)


def test_topk_exact_ties_go_to_lower_index():
    rng = np.random.default_rng(16)
    n, d = 32, 8
    q = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    k = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    k[0, 0, 20] = k[0, 0, 3]          # keys 3 and 20 tie for every query
    k[0, 0, 27] = k[0, 0, 3]
    v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
    s = oracle.topk_scores(q[0, 0], k[0, 0])
    assert np.array_equal(s[:, 3], s[:, 20]) and np.array_equal(s[:, 3],
                                                                s[:, 27])
    for topk in range(1, n + 1):
        _, idx, _ = oracle.topk_sparse(q, k, v, topk, return_details=True)
        for i in range(n):
            sel = set(idx[0, 0, i].tolist())
            # whenever a later copy is in, every earlier copy is in too
            if 27 in sel:
                assert 20 in sel and 3 in sel
            if 20 in sel:
                assert 3 in sel


def test_topk_zero_query_selects_first_indices():
    q = np.zeros((1, 1, 4, 8), np.float32)
    rng = np.random.default_rng(17)
    k = rng.standard_normal((1, 1, 4, 8)).astype(np.float32)
    k[0, 0, 1] *= -1  # negative zero products appear
    v = rng.standard_normal((1, 1, 4, 8)).astype(np.float32)
    out, idx, _ = oracle.topk_sparse(q, k, v, 2, return_details=True)
    assert idx[0, 0].tolist() == [[0, 1]] * 4
    assert np.all(out == 0)


# ----------------------------------------------------------------------------
# Decoder-causal top-k (c2psa page, further thoughts)
# ----------------------------------------------------------------------------
def test_topk_causal_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "topk_causal_hand.json")))
    q = np.array(g["q"], np.float32)
    k = np.array(g["k"], np.float32)
    v = np.array(g["v"], np.float32)
    for case in g["cases"]:
        out, idx, _ = oracle.topk_causal_sparse(q, k, v, case["topk"],
                                                return_details=True)
        np.testing.assert_allclose(out[0, 0], np.array(case["expected"]),
                                   rtol=0, atol=g["tolerance"])
        assert idx[0, 0].tolist() == case["indices"]


def test_topk_causal_brute_force_over_admissible_subsets():
    # Row i keeps c = min(topk, i+1) keys among j <= i; when i+1 > topk the
    # r = topk//2 most recent are forced. Among every admissible c-subset,
    # the kept one has the largest older scores, ties to the lower index
    # (lexicographically smallest sorted (-score, index) tuple of its older
    # part). Enumerate all of them on integer data full of ties.
    rng = np.random.default_rng(41)
    n, d = 8, 3
    for trial in range(4):
        q = rng.integers(-2, 3, (1, 1, n, d)).astype(np.float32)
        k = rng.integers(-2, 3, (1, 1, n, d)).astype(np.float32)
        v = rng.standard_normal((1, 1, n, d)).astype(np.float32)
        for topk in (1, 2, 3, 4, 5, 8):
            out, idx, _ = oracle.topk_causal_sparse(q, k, v, topk,
                                                    return_details=True)
            r = topk // 2
            for i in range(n):
                s = [float(np.dot(q[0, 0, i].astype(np.float64),
                                  k[0, 0, j].astype(np.float64)))
                     for j in range(n)]
                c = min(topk, i + 1)
                forced = set(range(i + 1 - r, i + 1)) if i + 1 > topk else set()
                best = None
                for sub in itertools.combinations(range(i + 1), c):
                    if not forced <= set(sub):
                        continue
                    key = tuple(sorted((-s[j], j) for j in sub
                                       if j not in forced))
                    if best is None or key < best[0]:
                        best = (key, sub)
                assert tuple(idx[0, 0, i, :c]) == best[1]
                assert np.all(idx[0, 0, i, c:] == -1)
                expect = sum(s[j] * v[0, 0, j].astype(np.float64)
                             for j in best[1])
                np.testing.assert_allclose(out[0, 0, i], expect, rtol=0,
                                           atol=1e-12)


def test_topk_causal_k_at_least_n_is_lower_triangular_product():
    rng = np.random.default_rng(42)
    q = rng.standard_normal((2, 3, 20, 8)).astype(np.float32)
    k = rng.standard_normal((2, 3, 20, 8)).astype(np.float32)
    v = rng.standard_normal((2, 3, 20, 8)).astype(np.float32)
    out = oracle.topk_causal_sparse(q, k, v, 20)
    s = torch.matmul(_t(q), _t(k).transpose(-2, -1))
    ref = torch.matmul(torch.tril(s), _t(v)).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)


def test_topk_causal_k1_is_causal_max_times_its_row():
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    k = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    v = rng.standard_normal((1, 2, 16, 8)).astype(np.float32)
    out = oracle.topk_causal_sparse(q, k, v, 1)
    s = torch.matmul(_t(q), _t(k).transpose(-2, -1))
    s = s.masked_fill(torch.ones(16, 16, dtype=torch.bool).triu(1),
                      float("-inf"))
    smax, arg = s.max(dim=-1)
    ref = smax[..., None] * torch.gather(
        _t(v), 2, arg[..., None].expand(-1, -1, -1, 8))
    np.testing.assert_allclose(out, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("topk", [2, 7, 10, 16])
def test_topk_causal_keep_mask_form(topk):
    # Reading of the c2psa page's further thoughts as a keep mask: a row with
    # i+1 <= topk keeps its whole lower triangle; a longer row keeps its r
    # most recent keys (i-r, i] and, among the older keys j <= i-r, those
    # scoring at least the (topk-r)-th largest older score (tie-free data);
    # the output is the masked score matrix times v.
    rng = np.random.default_rng(44)
    n = 40
    q = rng.standard_normal((2, 2, n, 16)).astype(np.float32)
    k = rng.standard_normal((2, 2, n, 16)).astype(np.float32)
    v = rng.standard_normal((2, 2, n, 16)).astype(np.float32)
    r = topk // 2
    s64 = q.astype(np.float64) @ np.swapaxes(k.astype(np.float64), -1, -2)
    ii = np.arange(n)[:, None]
    jj = np.arange(n)[None, :]
    older = jj <= ii - r
    keep = np.zeros(s64.shape, bool)
    for i in range(n):
        if i + 1 <= topk:
            keep[..., i, :i + 1] = True
            continue
        cand = s64[..., i, :i - r + 1]
        kth = -np.partition(-cand, topk - r - 1, axis=-1)[..., topk - r - 1]
        keep[..., i, :i - r + 1] = cand >= kth[..., None]
        keep[..., i, i - r + 1:i + 1] = True
    assert np.all(keep.sum(-1) == np.minimum(topk, np.arange(n) + 1))
    assert not np.any(keep & (jj > ii))
    assert np.all(keep[..., (jj <= ii) & ~older & (ii + 1 > topk)])
    ref = np.where(keep, s64, 0.0) @ v.astype(np.float64)
    out, myidx, gap = oracle.topk_causal_sparse(q, k, v, topk,
                                                return_details=True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-11)
    for i in range(n):
        c = min(topk, i + 1)
        got = myidx[..., i, :c]
        assert np.array_equal(got, np.nonzero(keep[..., i, :])[-1].reshape(
            got.shape))
        assert np.all(myidx[..., i, c:] == -1)
    assert np.all(np.isinf(gap[..., :topk])) and np.all(gap[..., topk:] > 0)


def test_topk_causal_rows_respect_order_and_recency():
    rng = np.random.default_rng(45)
    n, topk = 50, 12
    q = rng.standard_normal((1, 1, n, 8)).astype(np.float32)
    k = rng.standard_normal((1, 1, n, 8)).astype(np.float32)
    v = rng.standard_normal((1, 1, n, 8)).astype(np.float32)
    _, idx, _ = oracle.topk_causal_sparse(q, k, v, topk, return_details=True)
    s = oracle.topk_scores(q[0, 0], k[0, 0])
    for i in range(n):
        row = [j for j in idx[0, 0, i].tolist() if j >= 0]
        assert len(row) == min(topk, i + 1) and row == sorted(set(row))
        assert max(row) <= i                      # no key to the right
        if i + 1 > topk:
            assert set(range(i - topk // 2 + 1, i + 1)) <= set(row)
            old_in = [j for j in row if j <= i - topk // 2]
            old_out = [j for j in range(i - topk // 2 + 1) if j not in row]
            assert min(s[i, old_in]) >= max(s[i, old_out])


@pytest.mark.slow
def test_fp32_accumulation_is_not_enough_for_topk_tolerance():
    # Why the kernel accumulates top-k scores and outputs in fp64: on the
    # C2PSA shape an fp32-accumulated path misses the 1e-4 fp32 tolerance.
    # (fp32 scores, keep mask "score >= the row's 64th largest fp32 score",
    # fp32 product of the masked scores with v)
    inp = synth.topk(5, 4, 3, 512, 64, 64)
    q, k, v = (torch.from_numpy(x) for x in (inp.q, inp.k, inp.v))
    attn = torch.matmul(q, k.transpose(-2, -1))
    kth = attn.sort(dim=-1, descending=True).values[..., 63:64]
    out32 = torch.matmul(torch.where(attn >= kth, attn, 0.0), v).double().numpy()
    ref = oracle.topk_sparse(inp.q, inp.k, inp.v, 64)
    assert np.max(np.abs(out32 - ref)) > 1e-4
    # while rounding the exact result to fp32 alone stays well inside it
    assert np.max(np.abs(ref.astype(np.float32).astype(np.float64) - ref)) \
        < 5e-5


# ----------------------------------------------------------------------------
# Input generators (not the oracle, but both sides depend on them)
# ----------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(18)
    x = rng.standard_normal(100000).astype(np.float32) * 10
    x[:4] = [0.0, -0.0, 1e-40, -3.4e38]
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.int16), ref)
    back = synth.bf16_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16)
                          .float().numpy())


def test_generators_are_seeded_and_poisoned():
    a = synth.decode_uniform(2, 1, 4, 2, 16, 10, 3, "bf16")
    b = synth.decode_uniform(2, 1, 4, 2, 16, 10, 3, "bf16")
    assert np.array_equal(a.k_cache, b.k_cache)
    kf = synth.bf16_to_f32(a.k_cache)
    assert np.all(np.isnan(kf[:, :, 4:])) and np.all(np.isfinite(kf[:, :, :4]))
    r = synth.decode_ragged(3, 4, 4, 2, 16, 12, "f32")
    for bb in range(4):
        L = r.seq_lens[bb]
        assert np.all(np.isfinite(r.k_cache[bb, :, :L]))
        assert np.all(np.isnan(r.k_cache[bb, :, L:]))
