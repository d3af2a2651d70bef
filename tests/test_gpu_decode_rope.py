"""GPU parity of attn_decode_append_rope (rotary embedding of the query and
the new key fused into the append + decode launch) against the fp64 oracle.

The kernel rotates in fp32 and rounds once to the storage type; the oracle
rotates in fp64 and rounds once. The stored key may therefore differ by one
unit in the last place of the storage type where the exact value sits within
the fp32 error of a rounding tie; every other cache element must be
unchanged bit for bit, and the output must meet the dtype's tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import max_abs_err, say, to_dev, to_host64, tol

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def _rows(inp):
    B, _, _, _, max_length = inp.shape
    if inp.seq_lens is None:
        return np.full(B, inp.position_id)
    return np.clip(inp.seq_lens.astype(np.int64), 0, max_length) - 1


def rope_tables(rows, D, base=10000.0):
    """fp32 cos / sin [B, D] of each sequence's current row (rotate-half
    layout: the same angle on j and j + D/2)."""
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.maximum(np.asarray(rows, np.float64), 0)[:, None] * inv[None, :]
    ang = np.concatenate([ang, ang], axis=-1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _bits(t, dt):
    return t.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()


def check_rope(inp, kn, vn, cos, sin, split_rows=0):
    dt = inp.dtype
    q = to_dev(inp.q, dt)
    k = to_dev(inp.k_cache, dt)
    v = to_dev(inp.v_cache, dt)
    k0 = _bits(k, dt)
    v0 = _bits(v, dt)
    sl = None
    if inp.seq_lens is not None:
        sl = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out = tas.attn_decode_append_rope(
        q, to_dev(kn, dt), to_dev(vn, dt), torch.from_numpy(cos).cuda(),
        torch.from_numpy(sin).cuda(), k, v, position_id=inp.position_id,
        seq_lens=sl, scale=inp.scale, split_rows=split_rows)
    torch.cuda.synchronize()
    ref, k2, v2 = oracle.decode_append_rope(
        synth.as_f32(inp.q, dt), synth.as_f32(kn, dt), synth.as_f32(vn, dt),
        cos.astype(np.float64), sin.astype(np.float64),
        synth.as_f32(inp.k_cache, dt), synth.as_f32(inp.v_cache, dt), dt,
        position_id=inp.position_id, seq_lens=inp.seq_lens, scale=inp.scale)
    k1, v1 = _bits(k, dt), _bits(v, dt)
    kv = to_host64(k)
    unit = 2.0 ** -7 if dt == "bf16" else 2.0 ** -23
    # magnitudes of the two fp32 terms of each rotated key element
    x = synth.as_f32(kn, dt).astype(np.float64)
    h = x.shape[-1] // 2
    rh = np.concatenate([-x[..., h:], x[..., :h]], axis=-1)
    terms = np.abs(x * cos[:, None, :]) + np.abs(rh * sin[:, None, :])
    for b, r in enumerate(_rows(inp)):
        keep = np.ones(k0.shape[2], bool)
        if r >= 0:
            keep[r] = False
            # v stored unchanged; k rotated: one unit in the last place of the
            # storage type plus the fp32 rounding of the product and the fma
            np.testing.assert_array_equal(to_host64(v)[b, :, r], v2[b, :, r])
            got, want = kv[b, :, r], k2[b, :, r]
            ulp = unit * 2.0 ** np.floor(np.log2(np.maximum(np.abs(want),
                                                            2.0 ** -126)))
            bound = ulp + 2.0 ** -23 * terms[b]
            assert np.all(np.abs(got - want) <= bound), \
                np.max(np.abs(got - want) / bound)
        assert np.array_equal(k1[b][:, keep], k0[b][:, keep])
        assert np.array_equal(v1[b][:, keep], v0[b][:, keep])
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol(dt), err
    return out


@pytest.mark.parametrize("pos", [0, 4000, 8191])
def test_rope_append_gqa_static(pos):
    inp = synth.decode_uniform(71, 1, 32, 8, 128, 8192, pos, "bf16",
                               poison=True, scale=128 ** -0.5)
    inp.k_cache[:, :, pos] = synth.BF16_QNAN
    inp.v_cache[:, :, pos] = synth.BF16_QNAN
    kn, vn = synth.new_token_kv(71, 1, 8, 128, "bf16")
    cos, sin = rope_tables([pos], 128)
    say(f"decode_append_rope bf16 B=1 Hq=32 Hkv=8 D=128 pos={pos}")
    check_rope(inp, kn, vn, cos, sin)


def test_rope_append_f32_tiny_nan_tail():
    inp = synth.decode_uniform(72, 1, 2, 1, 64, 32, 15, "f32", poison=True,
                               scale=0.125)
    inp.k_cache[:, :, 15] = np.nan
    inp.v_cache[:, :, 15] = np.nan
    kn, vn = synth.new_token_kv(72, 1, 1, 64, "f32")
    cos, sin = rope_tables([15], 64)
    say("decode_append_rope f32 B=1 Hq=2 Hkv=1 D=64 pos=15")
    check_rope(inp, kn, vn, cos, sin)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D,Hq,Hkv", [(64, 8, 8), (128, 8, 2), (64, 16, 2)])
@pytest.mark.parametrize("split_rows", [0, 64, 100])
def test_rope_append_ragged_with_empty_sequences(dtype, D, Hq, Hkv, split_rows):
    lens = np.array([0, 1, 64, 65, 128, 200, 333, 0, 100, 640], np.int32)
    inp = synth.decode_ragged(73, B=len(lens), Hq=Hq, Hkv=Hkv, D=D,
                              max_length=640, dtype=dtype, lengths=lens)
    kn, vn = synth.new_token_kv(73, len(lens), Hkv, D, dtype)
    # arbitrary tables (not unit-norm pairs) exercise every product
    rng = np.random.default_rng(730 + D)
    cos = rng.standard_normal((len(lens), D)).astype(np.float32)
    sin = rng.standard_normal((len(lens), D)).astype(np.float32)
    say(f"decode_append_rope {dtype} D={D} G={Hq // Hkv} ragged split_rows={split_rows}")
    check_rope(inp, kn, vn, cos, sin, split_rows=split_rows)


@pytest.mark.parametrize("seed", range(12))
def test_rope_append_random_batches(seed):
    # Seeded random batch sizes (balanced schedule and plain grid), head
    # counts, dtypes, least run lengths and table kinds (standard angles of
    # each sequence's row, or arbitrary values that exercise every product).
    rng = np.random.default_rng(94000 + seed)
    B = int(rng.choice([1, 2, 5, 64, 100, 300]))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    M = int(rng.integers(1, 700))
    dt = "f32" if rng.random() < 0.25 else "bf16"
    sr = int(rng.choice([0, 1, 64]))
    lens = rng.integers(0, M + 1, B).astype(np.int32)
    lens[rng.random(B) < 0.1] = 0
    lens[rng.random(B) < 0.1] = M
    inp = synth.decode_ragged(95000 + seed, B=B, Hq=G * Hkv, Hkv=Hkv, D=D,
                              max_length=M, dtype=dt, lengths=lens)
    kn, vn = synth.new_token_kv(95000 + seed, B, Hkv, D, dt)
    if rng.random() < 0.5:
        cos, sin = rope_tables(_rows(inp), D)
    else:
        cos = rng.standard_normal((B, D)).astype(np.float32)
        sin = rng.standard_normal((B, D)).astype(np.float32)
    say(f"decode_append_rope random seed={seed} B={B} Hkv={Hkv} G={G} D={D} "
        f"M={M} {dt} split_rows={sr}")
    check_rope(inp, kn, vn, cos, sin, split_rows=sr)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rope_identity_tables_equal_the_plain_append(dtype):
    lens = np.array([3, 700, 1, 4096, 2048], np.int32)
    inp = synth.decode_ragged(74, B=5, Hq=32, Hkv=8, D=128, max_length=4096,
                              dtype=dtype, lengths=lens)
    kn, vn = synth.new_token_kv(74, 5, 8, 128, dtype)
    q = to_dev(inp.q, dtype)
    sl = torch.from_numpy(lens).cuda()
    outs, caches = [], []
    for rope in (False, True):
        k, v = to_dev(inp.k_cache, dtype), to_dev(inp.v_cache, dtype)
        if rope:
            ones = torch.ones(5, 128, dtype=torch.float32, device="cuda")
            outs.append(tas.attn_decode_append_rope(
                q, to_dev(kn, dtype), to_dev(vn, dtype), ones,
                torch.zeros_like(ones), k, v, seq_lens=sl, scale=0.09))
        else:
            outs.append(tas.attn_decode_append(
                q, to_dev(kn, dtype), to_dev(vn, dtype), k, v, seq_lens=sl,
                scale=0.09))
        caches.append((k, v))
    torch.cuda.synchronize()
    say(f"decode_append_rope identity tables {dtype}")
    assert torch.equal(outs[0], outs[1])
    # bit patterns: the caches hold NaN past each sequence's length
    assert np.array_equal(_bits(caches[0][0], dtype), _bits(caches[1][0], dtype))
    assert np.array_equal(_bits(caches[0][1], dtype), _bits(caches[1][1], dtype))


def test_rope_append_ragged_standard_tables():
    rng = np.random.default_rng(75)
    lens = rng.integers(1, 2049, 16).astype(np.int32)
    inp = synth.decode_ragged(75, B=16, Hq=32, Hkv=8, D=128, max_length=2048,
                              dtype="bf16", lengths=lens)
    kn, vn = synth.new_token_kv(75, 16, 8, 128, "bf16")
    cos, sin = rope_tables(_rows(inp), 128)
    say("decode_append_rope bf16 ragged B=16 max=2048 standard tables")
    check_rope(inp, kn, vn, cos, sin)


def test_rope_append_more_sequences_than_the_device_work_map():
    rng = np.random.default_rng(76)
    lens = rng.integers(0, 150, 300).astype(np.int32)
    inp = synth.decode_ragged(76, B=300, Hq=4, Hkv=2, D=64, max_length=150,
                              dtype="bf16", lengths=lens)
    kn, vn = synth.new_token_kv(76, 300, 2, 64, "bf16")
    cos, sin = rope_tables(_rows(inp), 64)
    say("decode_append_rope bf16 ragged B=300 split_rows=32")
    check_rope(inp, kn, vn, cos, sin, split_rows=32)
