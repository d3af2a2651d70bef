"""GPU parity of attn_decode against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (assert_discriminating, max_abs_err, say, to_dev,
                         to_host64, tol)

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def run_decode(inp, split_rows=0, seq_lens_dev=None):
    q = to_dev(inp.q, inp.dtype)
    k = to_dev(inp.k_cache, inp.dtype)
    v = to_dev(inp.v_cache, inp.dtype)
    if inp.seq_lens is not None and seq_lens_dev is None:
        seq_lens_dev = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out = tas.attn_decode(q, k, v, position_id=inp.position_id,
                          seq_lens=seq_lens_dev, scale=inp.scale,
                          split_rows=split_rows)
    torch.cuda.synchronize()
    return out


def oracle_of(inp):
    return oracle.decode(synth.as_f32(inp.q, inp.dtype),
                         synth.as_f32(inp.k_cache, inp.dtype),
                         synth.as_f32(inp.v_cache, inp.dtype),
                         position_id=inp.position_id, seq_lens=inp.seq_lens,
                         scale=inp.scale)


# ----------------------------------------------------------------------------
# The named workloads at full size
# ----------------------------------------------------------------------------
def test_decode_f32_tiny_nan_poisoned():
    p = synth.WORKLOADS["decode_f32_tiny"].params
    inp = synth.decode_uniform(p["seed"], p["B"], p["Hq"], p["Hkv"], p["D"],
                               p["max_length"], p["position_id"], "f32",
                               poison=True, scale=p["scale"])
    assert np.isnan(inp.k_cache[0, 0, 16:]).all()
    say("decode f32 B=1 Hq=2 Hkv=1 D=64 max=32 pos=15")
    out = to_host64(run_decode(inp))
    err = max_abs_err(out, oracle_of(inp))
    assert err <= tol("f32"), err


@pytest.fixture(scope="module")
def gqa_static():
    p = synth.WORKLOADS["decode_gqa_static"].params
    inp = synth.decode_uniform(p["seed"], p["B"], p["Hq"], p["Hkv"], p["D"],
                               p["max_length"], p["max_length"] - 1, "bf16",
                               poison=False, scale=p["scale"])
    dev = dict(q=to_dev(inp.q, "bf16"), k=to_dev(inp.k_cache, "bf16"),
               v=to_dev(inp.v_cache, "bf16"))
    return p, inp, dev


@pytest.mark.parametrize("pos", [0, 100, 1000, 4000, 8000])
def test_decode_gqa_static_positions(gqa_static, pos):
    p, inp, dev = gqa_static
    # rows past pos are poisoned on the device for this call
    k = dev["k"].clone()
    v = dev["v"].clone()
    k[:, :, pos + 1:] = float("nan")
    v[:, :, pos + 1:] = float("nan")
    say(f"decode bf16 B=1 Hq=32 Hkv=8 D=128 max=8192 pos={pos}")
    out = tas.attn_decode(dev["q"], k, v, position_id=pos, scale=p["scale"])
    torch.cuda.synchronize()
    got = to_host64(out)
    ref = oracle.decode(synth.as_f32(inp.q, "bf16"),
                        synth.as_f32(inp.k_cache[:, :, :pos + 1], "bf16"),
                        synth.as_f32(inp.v_cache[:, :, :pos + 1], "bf16"),
                        position_id=pos, scale=p["scale"])
    err = max_abs_err(got, ref)
    assert err <= tol("bf16"), err
    if pos == 0:
        # softmax over one row is the identity: out == V[b, h // G, 0] bitwise
        v0 = dev["v"][:, :, 0, :].repeat_interleave(4, dim=1)
        assert torch.equal(out, v0)


def test_decode_ragged_batch64_full():
    p = synth.WORKLOADS["decode_ragged_b64"].params
    B, Hq, Hkv, D, M = p["B"], p["Hq"], p["Hkv"], p["D"], p["max_length"]
    lens = synth.ragged_lengths(p["seed"], B, M)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.full((B, Hkv, M, D), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    v = torch.full_like(k, float("nan"))
    refs = []
    for b, L, qb, kb, vb in synth.iter_ragged(p["seed"], B, Hq, Hkv, D, M,
                                               "bf16", lens):
        q[b] = to_dev(qb, "bf16")
        k[b, :, :L] = to_dev(kb, "bf16")
        v[b, :, :L] = to_dev(vb, "bf16")
        refs.append(oracle.decode_sequence(synth.as_f32(qb, "bf16"),
                                           synth.as_f32(kb, "bf16"),
                                           synth.as_f32(vb, "bf16"), L,
                                           p["scale"]))
    sl = torch.from_numpy(lens).cuda()
    say(f"decode bf16 ragged B=64 sum(L)={int(lens.sum())}")
    out = tas.attn_decode(q, k, v, seq_lens=sl, scale=p["scale"])
    torch.cuda.synchronize()
    err = max_abs_err(to_host64(out), np.stack(refs))
    assert err <= tol("bf16"), err


def test_decode_ragged_batch64_full_needles():
    # The same workload with needle keys: over thousands of random keys the
    # output shrinks to about the bf16 tolerance, while needles keep it of
    # order one, so a split or tile that is skipped or read at the wrong rows
    # shows up.
    p = synth.WORKLOADS["decode_ragged_b64"].params
    B, Hq, Hkv, D, M = p["B"], p["Hq"], p["Hkv"], p["D"], p["max_length"]
    lens = synth.ragged_lengths(p["seed"], B, M)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.full((B, Hkv, M, D), float("nan"), dtype=torch.bfloat16,
                   device="cuda")
    v = torch.full_like(k, float("nan"))
    refs = []
    for b, L, qb, kb, vb in synth.iter_ragged(p["seed"], B, Hq, Hkv, D, M,
                                               "bf16", lens):
        synth.plant_needles(p["seed"] + b, qb[None], kb[None],
                            np.array([L]), "bf16", n_rows=4)
        q[b] = to_dev(qb, "bf16")
        k[b, :, :L] = to_dev(kb, "bf16")
        v[b, :, :L] = to_dev(vb, "bf16")
        refs.append(oracle.decode_sequence(synth.as_f32(qb, "bf16"),
                                           synth.as_f32(kb, "bf16"),
                                           synth.as_f32(vb, "bf16"), L,
                                           p["scale"]))
    ref = np.stack(refs)
    assert_discriminating(ref, "bf16")
    sl = torch.from_numpy(lens).cuda()
    say(f"decode bf16 ragged B=64 needles sum(L)={int(lens.sum())}")
    out = tas.attn_decode(q, k, v, seq_lens=sl, scale=p["scale"])
    torch.cuda.synchronize()
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("pos", [1000, 8000])
def test_decode_gqa_static_needles(pos):
    p = synth.WORKLOADS["decode_gqa_static"].params
    inp = synth.decode_uniform(p["seed"], p["B"], p["Hq"], p["Hkv"], p["D"],
                               p["max_length"], pos, "bf16", poison=True,
                               scale=p["scale"])
    synth.plant_needles(p["seed"], inp.q, inp.k_cache,
                        np.full(p["B"], pos + 1), "bf16")
    ref = oracle_of(inp)
    assert_discriminating(ref, "bf16")
    say(f"decode bf16 static position={pos} needles")
    err = max_abs_err(to_host64(run_decode(inp)), ref)
    assert err <= tol("bf16"), err


# ----------------------------------------------------------------------------
# Shapes, group sizes, ragged tails
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_group_sizes_and_dims(dtype, D, G):
    Hkv = 2
    inp = synth.decode_ragged(100 + G, B=3, Hq=G * Hkv, Hkv=Hkv, D=D,
                              max_length=700, dtype=dtype,
                              lengths=np.array([700, 1, 333]))
    say(f"decode {dtype} D={D} G={G} lens=700,1,333")
    err = max_abs_err(to_host64(run_decode(inp)), oracle_of(inp))
    assert err <= tol(dtype), err


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hkv", [3, 4, 6, 12])
def test_decode_balanced_kv_head_counts(D, Hkv):
    # Ragged bf16 batches run the balanced schedule: with Hkv a multiple of 4
    # a workgroup takes four neighbouring kv heads (one per wave), otherwise
    # every wave takes one kv head of its own. Both orders on head counts that
    # are not powers of two, with an empty sequence and runs of one tile
    # (split_rows 1) as well as the planner's.
    lens = np.array([1, 700, 333, 0, 64, 129])
    inp = synth.decode_ragged(110 + Hkv, B=6, Hq=2 * Hkv, Hkv=Hkv, D=D,
                              max_length=700, dtype="bf16", lengths=lens)
    ref = oracle_of(inp)
    for split_rows in (0, 1):
        say(f"decode bf16 balanced D={D} Hkv={Hkv} split_rows={split_rows}")
        out = to_host64(run_decode(inp, split_rows=split_rows))
        assert np.all(out[3] == 0)
        err = max_abs_err(out, ref)
        assert err <= tol("bf16"), (split_rows, err)


@pytest.mark.parametrize("seed", range(24))
def test_decode_balanced_random_batches(seed):
    # Seeded random batch compositions for the balanced schedule's work
    # order (runs crossing sequence and kv-head ends, slots, the combine's
    # recount of the pieces): batch size, kv heads, group size, head size,
    # lengths with zeros and full rows, and the least run length.
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.choice([2, 3, 5, 17, 64, 100, 256]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    M = int(rng.integers(1, 700))
    lens = rng.integers(0, M + 1, B).astype(np.int32)
    lens[rng.random(B) < 0.1] = 0
    lens[rng.random(B) < 0.1] = M
    split_rows = int(rng.choice([0, 1, 33, 64, 257]))
    inp = synth.decode_ragged(2000 + seed, B=B, Hq=G * Hkv, Hkv=Hkv, D=D,
                              max_length=M, dtype="bf16", lengths=lens)
    say(f"decode bf16 balanced random seed={seed} B={B} Hkv={Hkv} G={G} "
        f"D={D} M={M} split_rows={split_rows}")
    out = to_host64(run_decode(inp, split_rows=split_rows))
    assert np.all(out[lens == 0] == 0)
    err = max_abs_err(out, oracle_of(inp))
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("split_rows", [1, 7, 64, 100, 128, 1000, 5000])
def test_decode_split_invariance(split_rows):
    inp = synth.decode_ragged(21, B=2, Hq=8, Hkv=2, D=128, max_length=3000,
                              dtype="bf16", lengths=np.array([2999, 1234]))
    say(f"decode split_rows={split_rows}")
    a = run_decode(inp, split_rows=split_rows)
    b = run_decode(inp, split_rows=split_rows)
    assert torch.equal(a, b), "not bitwise repeatable"
    err = max_abs_err(to_host64(a), oracle_of(inp))
    assert err <= tol("bf16"), err


def test_decode_edge_lengths_clamped():
    # 0 -> zero row; beyond max_length and negative are clamped on the device
    lens = np.array([0, 1, 64, 65, 10**6, -3], dtype=np.int32)
    inp = synth.decode_ragged(22, B=6, Hq=4, Hkv=1, D=64, max_length=65,
                              dtype="f32", lengths=np.clip(lens, 0, 65))
    inp.seq_lens = lens
    say("decode edge lengths 0,1,64,65,1e6,-3")
    out = to_host64(run_decode(inp))
    assert np.all(out[0] == 0) and np.all(out[5] == 0)
    err = max_abs_err(out, oracle_of(inp))
    assert err <= tol("f32"), err


@pytest.mark.parametrize("B", [63, 65, 256, 300])
def test_decode_many_sequences_with_zero_lengths(B):
    # Batches around the sizes where the ragged work order changes (one or
    # more 64-sequence chunks of the on-device scan; above 256 sequences the
    # plain grid order is used), with every length category present: zero,
    # shorter than one split, whole splits, and whole splits plus a tail.
    rng = np.random.default_rng(B)
    lens = rng.integers(0, 200, B).astype(np.int32)
    lens[::7] = 0
    lens[1::11] = 64
    lens[2::13] = 128
    inp = synth.decode_ragged(30 + B, B=B, Hq=4, Hkv=2, D=64, max_length=200,
                              dtype="bf16", lengths=lens)
    say(f"decode bf16 ragged B={B} with zero lengths, split_rows=64")
    out = to_host64(run_decode(inp, split_rows=64))
    assert np.all(out[lens == 0] == 0)
    err = max_abs_err(out, oracle_of(inp))
    assert err <= tol("bf16"), err


def test_decode_position_is_last_row():
    inp = synth.decode_uniform(23, B=2, Hq=16, Hkv=4, D=128, max_length=777,
                               position_id=776, dtype="bf16")
    say("decode position_id = max_length - 1")
    err = max_abs_err(to_host64(run_decode(inp)), oracle_of(inp))
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("lens", [[513], [513, 200]])
def test_decode_gqa_equals_mha_with_repeated_kv(lens):
    # One sequence runs the plain split grid, whose splits do not depend on
    # Hkv: the same reductions in the same order, so equal to 1e-6. A ragged
    # batch runs the balanced schedule, which cuts the batch's rows by their
    # position in the (sequence, kv head) order, so the pieces differ with
    # Hkv. Each side then rounds its probabilities to bf16 relative to its own
    # pieces' running maxima (relative error 2^-9 each, weighted by |v|) and
    # its output to bf16 (half a unit in the last place, at most 2^-8 of the
    # value): the two may differ by 2^-7 * max|out| + 2^-8 * sum_j w_j |v_j|.
    B = len(lens)
    inp = synth.decode_ragged(24, B=B, Hq=16, Hkv=4, D=128, max_length=513,
                              dtype="bf16", lengths=np.array(lens))
    q = to_dev(inp.q, "bf16")
    k = to_dev(inp.k_cache, "bf16")
    v = to_dev(inp.v_cache, "bf16")
    sl = torch.from_numpy(inp.seq_lens).cuda()
    say(f"decode GQA vs repeated-KV MHA lens={lens}")
    gqa = tas.attn_decode(q, k, v, seq_lens=sl, split_rows=128)
    mha = tas.attn_decode(q, k.repeat_interleave(4, dim=1).contiguous(),
                          v.repeat_interleave(4, dim=1).contiguous(),
                          seq_lens=sl, split_rows=128)
    torch.cuda.synchronize()
    a, b = to_host64(gqa), to_host64(mha)
    if B == 1:
        assert max_abs_err(a, b) <= 1e-6
    else:
        absv = oracle.decode(synth.as_f32(inp.q, "bf16"),
                             synth.as_f32(inp.k_cache, "bf16"),
                             np.abs(synth.as_f32(inp.v_cache, "bf16")),
                             seq_lens=inp.seq_lens)  # sum_j w_j |v_j|
        bound = np.maximum(np.abs(a), np.abs(b)) * 2.0 ** -7 + absv * 2.0 ** -8
        assert np.all(np.abs(a - b) <= bound), float(np.max(np.abs(a - b) - bound))
    assert max_abs_err(a, oracle_of(inp)) <= tol("bf16")


def test_decode_batched_equals_per_sequence_launches():
    inp = synth.decode_ragged(25, B=4, Hq=8, Hkv=2, D=64, max_length=300,
                              dtype="bf16", lengths=np.array([300, 5, 77, 1]))
    q = to_dev(inp.q, "bf16")
    k = to_dev(inp.k_cache, "bf16")
    v = to_dev(inp.v_cache, "bf16")
    sl = torch.from_numpy(inp.seq_lens).cuda()
    say("decode one launch for the batch vs per-sequence launches")
    full = tas.attn_decode(q, k, v, seq_lens=sl, split_rows=64)
    parts = [tas.attn_decode(q[b:b + 1].contiguous(),
                             k[b:b + 1].contiguous(),
                             v[b:b + 1].contiguous(), seq_lens=sl[b:b + 1],
                             split_rows=64) for b in range(4)]
    torch.cuda.synchronize()
    assert torch.equal(full, torch.cat(parts, 0))


def test_decode_sliced_equals_masked_full_via_positions():
    # the same cache at position p and a cache truncated to p+1 rows
    inp = synth.decode_uniform(26, B=1, Hq=8, Hkv=2, D=128, max_length=1024,
                               position_id=1023, dtype="bf16", poison=False)
    q = to_dev(inp.q, "bf16")
    k = to_dev(inp.k_cache, "bf16")
    v = to_dev(inp.v_cache, "bf16")
    say("decode full cache at pos=300 vs cache truncated to 301 rows")
    a = tas.attn_decode(q, k, v, position_id=300, split_rows=64)
    b = tas.attn_decode(q, k[:, :, :301].contiguous(),
                        v[:, :, :301].contiguous(), position_id=300,
                        split_rows=64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_empty_batch_is_noop():
    q = torch.empty(0, 4, 64, device="cuda")
    k = torch.empty(0, 1, 8, 64, device="cuda")
    out = tas.attn_decode(q, k, k.clone(), position_id=0)
    assert out.shape == (0, 4, 64)


def test_decode_on_side_stream_keeps_its_workspace():
    # The binding allocates the workspace (and out) itself on the current
    # stream while the kernels run on `stream`. A long matrix product queued
    # first keeps the side stream busy; the binding then returns and the
    # test allocates and overwrites memory of the same size on the current
    # stream. Unless the binding recorded the side stream's use, the
    # allocator can hand that block over while split and combine still use
    # it, and the output is corrupted.
    inp = synth.decode_ragged(77, B=8, Hq=8, Hkv=2, D=128, max_length=4096,
                              dtype="bf16")
    q = to_dev(inp.q, "bf16")
    k = to_dev(inp.k_cache, "bf16")
    v = to_dev(inp.v_cache, "bf16")
    lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    need = tas.attn_decode_workspace_bytes(8, 8, 2, 128, 4096, 128)
    ref = oracle_of(inp)
    side = torch.cuda.Stream()
    big = torch.randn(4096, 4096, device="cuda")
    torch.cuda.synchronize()
    say("decode on a side stream, allocations on the current stream")
    for stream_arg in (side, side.cuda_stream):
        with torch.cuda.stream(side):
            for _ in range(8):
                big = big @ big * 1e-3
        out = tas.attn_decode(q, k, v, seq_lens=lens, scale=inp.scale,
                              split_rows=128, stream=stream_arg)
        junk = [torch.full((need,), 255, dtype=torch.uint8,
                           device="cuda") for _ in range(4)]
        junk.append(torch.full(out.shape, float("nan"), dtype=out.dtype,
                               device="cuda"))
        torch.cuda.synchronize()
        err = max_abs_err(to_host64(out), ref)
        assert err <= tol("bf16"), err
        del junk
