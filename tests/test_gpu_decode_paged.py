"""GPU parity of attn_decode_paged (decode over a paged, token-major cache)
against the fp64 oracle, and bitwise against attn_decode on the contiguous
cache the pages were cut from."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import max_abs_err, say, to_dev, to_host64, tol

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def run_paged(inp, kp, vp, table, split_rows=0, layout="token"):
    q = to_dev(inp.q, "bf16")
    k_pages, v_pages = to_dev(kp, "bf16"), to_dev(vp, "bf16")
    bt = torch.from_numpy(table).cuda()
    sl = None
    if inp.seq_lens is not None:
        sl = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out = tas.attn_decode_paged(q, k_pages, v_pages, bt, layout=layout,
                                position_id=inp.position_id, seq_lens=sl,
                                scale=inp.scale, split_rows=split_rows)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("D,page_size", [(64, 64), (64, 256), (128, 32),
                                         (128, 128), (128, 512)])
@pytest.mark.parametrize("G", [1, 4, 8])
@pytest.mark.parametrize("layout", ["token", "head"])
def test_paged_ragged_with_empty_sequences(D, page_size, G, layout):
    M = 1024
    lens = np.array([0, 1, 31, 32, 33, 300, 1000, 1024, 0, 517], np.int32)
    inp = synth.decode_ragged(61, B=len(lens), Hq=2 * G, Hkv=2, D=D,
                              max_length=M, dtype="bf16", lengths=lens)
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, page_size, 61,
                                   layout=layout)
    say(f"decode_paged bf16 D={D} page={page_size} G={G} {layout}-major")
    out = to_host64(run_paged(inp, kp, vp, table, layout=layout))
    assert np.all(out[lens == 0] == 0)
    ref = oracle.decode_paged(synth.as_f32(inp.q, "bf16"),
                              synth.as_f32(kp, "bf16"),
                              synth.as_f32(vp, "bf16"), table,
                              seq_lens=lens, scale=inp.scale, layout=layout)
    err = max_abs_err(out, ref)
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("seed", range(16))
def test_paged_random_batches(seed):
    # Seeded random page sizes, page counts, layouts, batch sizes (balanced
    # schedule and plain grid), head counts and least run lengths, against
    # the oracle. Bitwise equal to the contiguous decode wherever the two
    # plans coincide: balanced batches, or splits already whole wave tiles
    # (the plain grid otherwise rounds paged splits up to whole tiles, so
    # that no tile straddles a page).
    rng = np.random.default_rng(94000 + seed)
    D = int(rng.choice([64, 128]))
    tile = 4096 // D
    ps = tile * int(rng.choice([1, 2, 4]))
    M = ps * int(rng.integers(1, 9))
    B = int(rng.choice([1, 2, 9, 64, 256, 260]))
    Hkv = int(rng.integers(1, 9))
    G = int(rng.choice([1, 2, 4, 8]))
    layout = str(rng.choice(["token", "head"]))
    sr = int(rng.choice([0, 1, 100, tile]))
    lens = rng.integers(0, M + 1, B).astype(np.int32)
    lens[rng.random(B) < 0.1] = 0
    lens[rng.random(B) < 0.1] = M
    inp = synth.decode_ragged(95000 + seed, B=B, Hq=G * Hkv, Hkv=Hkv, D=D,
                              max_length=M, dtype="bf16", lengths=lens)
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, ps, 95000 + seed,
                                   layout=layout)
    say(f"decode_paged random seed={seed} B={B} Hkv={Hkv} G={G} D={D} "
        f"page_size={ps} M={M} {layout}-major split_rows={sr}")
    a = run_paged(inp, kp, vp, table, split_rows=sr, layout=layout)
    sl = torch.from_numpy(lens).cuda()
    b = tas.attn_decode(to_dev(inp.q, "bf16"), to_dev(inp.k_cache, "bf16"),
                        to_dev(inp.v_cache, "bf16"), seq_lens=sl,
                        scale=inp.scale, split_rows=sr)
    torch.cuda.synchronize()
    if 2 <= B <= 256 or sr % tile == 0:
        assert torch.equal(a, b)
    ref = oracle.decode(synth.as_f32(inp.q, "bf16"),
                        synth.as_f32(inp.k_cache, "bf16"),
                        synth.as_f32(inp.v_cache, "bf16"), seq_lens=lens,
                        scale=inp.scale)
    err = max_abs_err(to_host64(a), ref)
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("split_rows", [0, 128, 640])
@pytest.mark.parametrize("layout", ["token", "head"])
def test_paged_equals_contiguous_bitwise(split_rows, layout):
    # same rows, same split plan: the same reductions in the same order
    M, ps = 2048, 128
    lens = np.array([2048, 1, 777, 1500], np.int32)
    inp = synth.decode_ragged(62, B=4, Hq=32, Hkv=8, D=128, max_length=M,
                              dtype="bf16", lengths=lens)
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, ps, 62,
                                   layout=layout)
    say(f"decode_paged vs contiguous split_rows={split_rows} {layout}-major")
    a = run_paged(inp, kp, vp, table, split_rows=split_rows, layout=layout)
    sl = torch.from_numpy(lens).cuda()
    b = tas.attn_decode(to_dev(inp.q, "bf16"), to_dev(inp.k_cache, "bf16"),
                        to_dev(inp.v_cache, "bf16"), seq_lens=sl,
                        scale=inp.scale, split_rows=split_rows)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_paged_uniform_position_and_reused_pages():
    # every sequence at one position; two sequences share their first page
    M, ps = 512, 64
    inp = synth.decode_uniform(63, B=3, Hq=8, Hkv=2, D=64, max_length=M,
                               position_id=300, dtype="bf16", poison=True)
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, ps, 63)
    table[2, 0] = table[1, 0]
    k2, v2 = inp.k_cache.copy(), inp.v_cache.copy()
    k2[2, :, :ps], v2[2, :, :ps] = k2[1, :, :ps], v2[1, :, :ps]
    say("decode_paged uniform position 300, shared page")
    out = to_host64(run_paged(inp, kp, vp, table))
    ref = oracle.decode(synth.as_f32(inp.q, "bf16"), synth.as_f32(k2, "bf16"),
                        synth.as_f32(v2, "bf16"), position_id=300,
                        scale=inp.scale)
    err = max_abs_err(out, ref)
    assert err <= tol("bf16"), err


def test_paged_out_of_range_table_entries_are_clamped():
    # entries past the last page or negative read the last / first page, never
    # outside the pages (the oracle clamps the same way)
    M, ps = 256, 64
    lens = np.array([256, 200], np.int32)
    inp = synth.decode_ragged(64, B=2, Hq=4, Hkv=1, D=64, max_length=M,
                              dtype="bf16", lengths=lens)
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, ps, 64,
                                   extra_pages=0)
    table[0, 1] = 10 ** 6
    table[1, 2] = -5
    say("decode_paged clamped table entries")
    out = to_host64(run_paged(inp, kp, vp, table))
    ref = oracle.decode_paged(synth.as_f32(inp.q, "bf16"),
                              synth.as_f32(kp, "bf16"),
                              synth.as_f32(vp, "bf16"), table,
                              seq_lens=lens, scale=inp.scale)
    err = max_abs_err(out, ref)
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("layout", ["token", "head"])
def test_paged_more_sequences_than_the_device_work_map(layout):
    # more than 256 sequences: the grid's plain order instead of the
    # on-device work map; still the contiguous decode bit for bit
    rng = np.random.default_rng(65)
    lens = rng.integers(0, 257, 300).astype(np.int32)
    inp = synth.decode_ragged(65, B=300, Hq=4, Hkv=2, D=64, max_length=256,
                              dtype="bf16", lengths=lens)
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, 64, 65,
                                   layout=layout)
    say(f"decode_paged bf16 B=300 {layout}-major")
    out = run_paged(inp, kp, vp, table, split_rows=64, layout=layout)
    ref = tas.attn_decode(to_dev(inp.q, "bf16"), to_dev(inp.k_cache, "bf16"),
                          to_dev(inp.v_cache, "bf16"),
                          seq_lens=torch.from_numpy(lens).cuda(),
                          scale=inp.scale, split_rows=64)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
