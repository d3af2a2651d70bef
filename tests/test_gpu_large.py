"""GPU parity at the size limits a 288 GB device makes ordinary: caches whose
byte offsets pass 2^32 (the sequence, kv head or page that is read starts
beyond 4 GiB), a single sequence of 2^20 rows at the cap of 1024 splits per
sequence, and prefill after a prefix of 65536 tokens. Every cache row that
holds no data is NaN, so an offset that lands on the wrong row shows up as a
non-finite output. Expected values come from the fp64 oracle run on a small
host copy of the rows that are read (the oracle reads no others).

Over thousands of random keys an attention output is the mean of many values
and shrinks towards zero (to about 0.002 at 2^20 rows), below the bf16
tolerance, so a kernel that skipped whole tiles would still pass. The inputs
here are therefore shaped so that few rows carry the weight: decode plants
"needle" keys (``synth.plant_needles``) at chosen rows, the first or last
valid row among them; prefill uses the score scale 1.0, which makes each
query's softmax peak on its own key, spread over the whole cache. Each test
asserts that the expected output is large against the tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import (assert_discriminating, max_abs_err, say, to_dev,
                         to_host64, tol)

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)

GIB = 1 << 30
TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}
ESIZE = {"bf16": 2, "f32": 4}


def nan_tensor(shape, dtype):
    return torch.full(shape, float("nan"), dtype=TORCH_DTYPE[dtype],
                      device="cuda")


@pytest.fixture(autouse=True)
def release_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# Contiguous caches past 4 GiB
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,B", [("bf16", 3), ("f32", 2)])
def test_decode_cache_beyond_4gib(dtype, B):
    Hq, Hkv, D, M = 32, 8, 128, 1 << 20
    lens = np.zeros(B, np.int32)
    lens[0], lens[-1] = 1, 5000
    # the last sequence starts at byte 4 GiB of each cache
    assert (B - 1) * Hkv * M * D * ESIZE[dtype] >= 4 * GIB
    k = nan_tensor((B, Hkv, M, D), dtype)
    v = nan_tensor((B, Hkv, M, D), dtype)
    Lh = int(lens.max())
    inp = synth.decode_ragged(71, B, Hq, Hkv, D, Lh, dtype, lengths=lens)
    synth.plant_needles(71, inp.q, inp.k_cache, lens, dtype)
    k[:, :, :Lh] = to_dev(inp.k_cache, dtype)
    v[:, :, :Lh] = to_dev(inp.v_cache, dtype)
    ref = oracle.decode(synth.as_f32(inp.q, dtype),
                        synth.as_f32(inp.k_cache, dtype),
                        synth.as_f32(inp.v_cache, dtype), seq_lens=lens)
    assert_discriminating(ref, dtype)
    sl = torch.from_numpy(lens).cuda()
    for split_rows in (0, 256):
        say(f"decode {dtype} cache {B * Hkv * M * D * ESIZE[dtype] / GIB:.0f}"
            f" GiB lens={lens.tolist()} split_rows={split_rows}")
        out = tas.attn_decode(to_dev(inp.q, dtype), k, v, seq_lens=sl,
                              split_rows=split_rows)
        torch.cuda.synchronize()
        out = to_host64(out)
        assert np.all(out[1:-1] == 0)
        err = max_abs_err(out, ref)
        assert err <= tol(dtype), (split_rows, err)


def test_decode_append_beyond_4gib():
    # the current token's row is written beyond 4 GiB and read back in the
    # same call
    B, Hq, Hkv, D, M = 3, 16, 8, 128, 1 << 20
    lens = np.array([700, 0, 4097], np.int32)
    k = nan_tensor((B, Hkv, M, D), "bf16")
    v = nan_tensor((B, Hkv, M, D), "bf16")
    Lh = int(lens.max())
    inp = synth.decode_ragged(72, B, Hq, Hkv, D, Lh, "bf16", lengths=lens)
    needles = synth.plant_needles(72, inp.q, inp.k_cache, lens, "bf16")
    k[:, :, :Lh] = to_dev(inp.k_cache, "bf16")
    v[:, :, :Lh] = to_dev(inp.v_cache, "bf16")
    kn, vn = synth.new_token_kv(72, B, Hkv, D, "bf16")
    # the appended key is a needle too (for even kv heads row L-1 held none)
    kn[lens > 0] = needles[lens > 0]
    ref, k2, v2 = oracle.decode_append(
        synth.as_f32(inp.q, "bf16"), synth.as_f32(kn, "bf16"),
        synth.as_f32(vn, "bf16"), synth.as_f32(inp.k_cache, "bf16"),
        synth.as_f32(inp.v_cache, "bf16"), seq_lens=lens)
    assert_discriminating(ref, "bf16")
    say(f"decode_append bf16 cache 6 GiB lens={lens.tolist()}")
    out = tas.attn_decode_append(to_dev(inp.q, "bf16"), to_dev(kn, "bf16"),
                                 to_dev(vn, "bf16"), k, v,
                                 seq_lens=torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err
    kd = k[:, :, :Lh].float().cpu().numpy()
    vd = v[:, :, :Lh].float().cpu().numpy()
    assert np.array_equal(kd, k2, equal_nan=True)
    assert np.array_equal(vd, v2, equal_nan=True)
    # nothing written past each sequence's current row
    assert torch.isnan(k[2, :, 4097:8192]).all()
    assert torch.isnan(k[1, :, :64]).all()


def test_prefill_cache_beyond_4gib():
    B, Hq, Hkv, D, M = 3, 16, 8, 128, 1 << 20
    prefix, Lq = 3000, 200
    inp = synth.prefill(73, B, Hq, Hkv, D, Lq, prefix, dtype="bf16")
    T = prefix + Lq
    k = nan_tensor((B, Hkv, M, D), "bf16")
    v = nan_tensor((B, Hkv, M, D), "bf16")
    k[:, :, :T] = to_dev(inp.k_cache, "bf16")
    v[:, :, :T] = to_dev(inp.v_cache, "bf16")
    say(f"prefill bf16 cache 6 GiB B={B} prefix={prefix} Lq={Lq}")
    out = tas.attn_prefill(to_dev(inp.q, "bf16"), k, v, prefix_len=prefix,
                           scale=1.0)
    torch.cuda.synchronize()
    ref = oracle.prefill(synth.as_f32(inp.q, "bf16"),
                         synth.as_f32(inp.k_cache, "bf16"),
                         synth.as_f32(inp.v_cache, "bf16"), prefix, scale=1.0)
    assert_discriminating(ref, "bf16")
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err


# ----------------------------------------------------------------------------
# Page pools past 4 GiB: the pages that are read sit at the pool's far end
# ----------------------------------------------------------------------------
def big_pool(kp, vp, num_pages, layout):
    """Device pools of num_pages NaN pages holding host page p at
    num_pages - 1 - p; returns (k_pages, v_pages, page map)."""
    n = kp.shape[0]
    assert n <= num_pages
    shape = (num_pages,) + kp.shape[1:]
    k = nan_tensor(shape, "bf16")
    v = nan_tensor(shape, "bf16")
    where = torch.arange(num_pages - 1, num_pages - 1 - n, -1, device="cuda")
    k[where] = to_dev(kp, "bf16")
    v[where] = to_dev(vp, "bf16")
    return k, v, (num_pages - 1 - np.arange(n)).astype(np.int32)


@pytest.mark.parametrize("layout", ["token", "head"])
def test_decode_paged_pool_beyond_4gib(layout):
    Hq, Hkv, D, ps, M = 32, 8, 128, 128, 4096
    num_pages = 20480  # 256 KiB pages: a 5 GiB pool per cache
    lens = np.array([4096, 1, 0, 2500], np.int32)
    inp = synth.decode_ragged(74, len(lens), Hq, Hkv, D, M, "bf16",
                              lengths=lens)
    synth.plant_needles(74, inp.q, inp.k_cache, lens, "bf16")
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, ps, 74,
                                   layout=layout)
    k, v, remap = big_pool(kp, vp, num_pages, layout)
    ref = oracle.decode_paged(synth.as_f32(inp.q, "bf16"),
                              synth.as_f32(kp, "bf16"),
                              synth.as_f32(vp, "bf16"), table,
                              seq_lens=lens, layout=layout)
    assert_discriminating(ref, "bf16")
    bt = torch.from_numpy(remap[table]).cuda()
    say(f"decode_paged bf16 {layout}-major pool 5 GiB lens={lens.tolist()}")
    out = tas.attn_decode_paged(to_dev(inp.q, "bf16"), k, v, bt,
                                layout=layout,
                                seq_lens=torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("layout", ["token", "head"])
def test_prefill_paged_pool_beyond_4gib(layout):
    B, Hq, Hkv, D, ps = 2, 16, 8, 128, 128
    prefix, Lq = 1500, 300
    num_pages = 20480
    M = ((prefix + Lq + ps - 1) // ps) * ps
    inp = synth.prefill(75, B, Hq, Hkv, D, Lq, prefix, max_length=M,
                        dtype="bf16")
    kp, vp, table = synth.paginate(inp.k_cache, inp.v_cache, ps, 75,
                                   layout=layout)
    k, v, remap = big_pool(kp, vp, num_pages, layout)
    ref = oracle.prefill_paged(synth.as_f32(inp.q, "bf16"),
                               synth.as_f32(kp, "bf16"),
                               synth.as_f32(vp, "bf16"), table, prefix,
                               scale=1.0, layout=layout)
    assert_discriminating(ref, "bf16")
    bt = torch.from_numpy(remap[table]).cuda()
    say(f"prefill_paged bf16 {layout}-major pool 5 GiB prefix={prefix} "
        f"Lq={Lq}")
    out = tas.attn_prefill_paged(to_dev(inp.q, "bf16"), k, v, bt,
                                 prefix_len=prefix, layout=layout,
                                 scale=1.0)
    torch.cuda.synchronize()
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err


# ----------------------------------------------------------------------------
# Long single sequences
# ----------------------------------------------------------------------------
@pytest.fixture(scope="module", params=["bf16", "f32"])
def million_rows(request):
    dtype = request.param
    lens = np.array([1 << 20, 777_777], np.int32)
    inp = synth.decode_ragged(76, B=2, Hq=8, Hkv=1, D=128, max_length=1 << 20,
                              dtype=dtype, lengths=lens)
    synth.plant_needles(76, inp.q, inp.k_cache, lens, dtype, n_rows=8)
    ref = oracle.decode(synth.as_f32(inp.q, dtype),
                        synth.as_f32(inp.k_cache, dtype),
                        synth.as_f32(inp.v_cache, dtype), seq_lens=lens)
    assert_discriminating(ref, dtype)
    dev = (to_dev(inp.q, dtype), to_dev(inp.k_cache, dtype),
           to_dev(inp.v_cache, dtype), torch.from_numpy(lens).cuda())
    yield dtype, dev, ref
    del dev
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# 0: the automatic plan (1024 splits of 1024 rows, the cap); 1: raised to the
# cap's floor of 1024 rows; 100000: 11 long splits
@pytest.mark.parametrize("split_rows", [0, 1, 100_000])
def test_decode_million_rows(million_rows, split_rows):
    dtype, (q, k, v, sl), ref = million_rows
    say(f"decode {dtype} B=2 Hkv=1 lens=2^20,777777 split_rows={split_rows}")
    out = tas.attn_decode(q, k, v, seq_lens=sl, split_rows=split_rows)
    torch.cuda.synchronize()
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol(dtype), err


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 8, 2), (128, 8, 8)])
def test_prefill_prefix_65536(D, Hq, Hkv):
    prefix, Lq = 65536, 257
    inp = synth.prefill(77 + D, 1, Hq, Hkv, D, Lq, prefix, dtype="bf16")
    say(f"prefill bf16 D={D} Hq={Hq} Hkv={Hkv} prefix={prefix} Lq={Lq}")
    out = tas.attn_prefill(to_dev(inp.q, "bf16"), to_dev(inp.k_cache, "bf16"),
                           to_dev(inp.v_cache, "bf16"), prefix_len=prefix,
                           scale=1.0)
    torch.cuda.synchronize()
    ref = oracle.prefill(synth.as_f32(inp.q, "bf16"),
                         synth.as_f32(inp.k_cache, "bf16"),
                         synth.as_f32(inp.v_cache, "bf16"), prefix, scale=1.0)
    assert_discriminating(ref, "bf16")
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err
