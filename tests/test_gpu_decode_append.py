"""GPU parity of attn_decode_append (the cache append fused into the decode
launch) against the fp64 oracle, and against a separate copy followed by
attn_decode."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import max_abs_err, say, to_dev, to_host64, tol

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def _rows(inp):
    """Row receiving the new token per sequence (-1: none)."""
    B, _, _, _, max_length = inp.shape
    if inp.seq_lens is None:
        return np.full(B, inp.position_id)
    return np.clip(inp.seq_lens.astype(np.int64), 0, max_length) - 1


def check_append(inp, kn, vn, split_rows=0):
    dt = inp.dtype
    q = to_dev(inp.q, dt)
    k = to_dev(inp.k_cache, dt)
    v = to_dev(inp.v_cache, dt)
    k_new, v_new = to_dev(kn, dt), to_dev(vn, dt)
    sl = None
    if inp.seq_lens is not None:
        sl = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    # reference on the device path: copy, then the plain decode
    k_ref, v_ref = k.clone(), v.clone()
    for b, r in enumerate(_rows(inp)):
        if r >= 0:
            k_ref[b, :, r] = k_new[b]
            v_ref[b, :, r] = v_new[b]
    out_ref = tas.attn_decode(q, k_ref, v_ref, position_id=inp.position_id,
                              seq_lens=sl, scale=inp.scale,
                              split_rows=split_rows)
    out = tas.attn_decode_append(q, k_new, v_new, k, v,
                                 position_id=inp.position_id, seq_lens=sl,
                                 scale=inp.scale, split_rows=split_rows)
    torch.cuda.synchronize()
    # the caches now equal the copied ones, bit for bit
    assert torch.equal(k.view(torch.int16) if dt == "bf16" else k.view(torch.int32),
                       k_ref.view(torch.int16) if dt == "bf16" else k_ref.view(torch.int32))
    assert torch.equal(v.view(torch.int16) if dt == "bf16" else v.view(torch.int32),
                       v_ref.view(torch.int16) if dt == "bf16" else v_ref.view(torch.int32))
    # same values, same reduction order: identical to copy + decode
    assert torch.equal(out, out_ref)
    ref, _, _ = oracle.decode_append(
        synth.as_f32(inp.q, dt), synth.as_f32(kn, dt), synth.as_f32(vn, dt),
        synth.as_f32(inp.k_cache, dt), synth.as_f32(inp.v_cache, dt),
        position_id=inp.position_id, seq_lens=inp.seq_lens, scale=inp.scale)
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol(dt), err


@pytest.mark.parametrize("pos", [0, 4000, 8191])
def test_append_gqa_static(pos):
    # the single-sequence workload shape; the row being written holds NaN
    # before the call, so a read of the stale row would show
    inp = synth.decode_uniform(41, 1, 32, 8, 128, 8192, pos, "bf16",
                               poison=True, scale=128 ** -0.5)
    inp.k_cache[:, :, pos] = synth.BF16_QNAN
    inp.v_cache[:, :, pos] = synth.BF16_QNAN
    kn, vn = synth.new_token_kv(41, 1, 8, 128, "bf16")
    say(f"decode_append bf16 B=1 Hq=32 Hkv=8 D=128 max=8192 pos={pos}")
    check_append(inp, kn, vn)


def test_append_f32_tiny_nan_tail():
    inp = synth.decode_uniform(42, 1, 2, 1, 64, 32, 15, "f32", poison=True,
                               scale=0.125)
    inp.k_cache[:, :, 15] = np.nan
    inp.v_cache[:, :, 15] = np.nan
    kn, vn = synth.new_token_kv(42, 1, 1, 64, "f32")
    say("decode_append f32 B=1 Hq=2 Hkv=1 D=64 max=32 pos=15")
    check_append(inp, kn, vn)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("split_rows", [0, 64, 100])
def test_append_ragged_with_empty_sequences(dtype, D, split_rows):
    # lengths put the new row at the start, middle and end of a split and in
    # single-split sequences; length 0 gets no append and a zero row
    lens = np.array([0, 1, 64, 65, 128, 200, 333, 0, 100, 640], np.int32)
    inp = synth.decode_ragged(43, B=len(lens), Hq=8, Hkv=2, D=D,
                              max_length=640, dtype=dtype, lengths=lens)
    kn, vn = synth.new_token_kv(43, len(lens), 2, D, dtype)
    say(f"decode_append {dtype} D={D} ragged split_rows={split_rows}")
    check_append(inp, kn, vn, split_rows=split_rows)


@pytest.mark.parametrize("seed", range(16))
def test_append_random_batches(seed):
    # Seeded random batch sizes (balanced schedule and plain grid), head
    # counts, dtypes and least run lengths: the caches and the output equal
    # copy + decode bit for bit, and the oracle within the tolerance.
    rng = np.random.default_rng(92000 + seed)
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
    inp = synth.decode_ragged(93000 + seed, B=B, Hq=G * Hkv, Hkv=Hkv, D=D,
                              max_length=M, dtype=dt, lengths=lens)
    kn, vn = synth.new_token_kv(93000 + seed, B, Hkv, D, dt)
    say(f"decode_append random seed={seed} B={B} Hkv={Hkv} G={G} D={D} M={M} "
        f"{dt} split_rows={sr}")
    check_append(inp, kn, vn, split_rows=sr)


def test_append_ragged_batch_over_reorder_limit():
    # more than 256 sequences: the plain grid order instead of the on-device
    # work map
    rng = np.random.default_rng(44)
    lens = rng.integers(0, 150, 300).astype(np.int32)
    inp = synth.decode_ragged(44, B=300, Hq=4, Hkv=2, D=64, max_length=150,
                              dtype="bf16", lengths=lens)
    kn, vn = synth.new_token_kv(44, 300, 2, 64, "bf16")
    say("decode_append bf16 ragged B=300 split_rows=32")
    check_append(inp, kn, vn, split_rows=32)
