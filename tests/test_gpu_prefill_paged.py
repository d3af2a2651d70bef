"""GPU parity of attn_prefill_paged (causal prefill over a paged prefix
cache) against attn_prefill on the contiguous cache (bit for bit: the same
kernel arithmetic on the same rows) and against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import max_abs_err, say, to_dev, to_host64, tol

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def _padded(inp, page_size):
    """The contiguous caches padded with NaN rows to a whole number of pages."""
    B, Hkv, M, D = inp.k_cache.shape
    M2 = -(-M // page_size) * page_size
    if M2 == M:
        return inp.k_cache, inp.v_cache
    pad = np.full((B, Hkv, M2 - M, D), synth.BF16_QNAN, inp.k_cache.dtype)
    return (np.concatenate([inp.k_cache, pad], axis=2),
            np.concatenate([inp.v_cache, pad], axis=2))


def check_paged(inp, page_size, layout, seed, with_oracle=True, table_fix=None,
                extra_pages=3):
    k, v = _padded(inp, page_size)
    kp, vp, table = synth.paginate(k, v, page_size, seed, layout=layout,
                                   extra_pages=extra_pages)
    if table_fix is not None:
        table = table_fix(table)
    q = to_dev(inp.q, "bf16")
    out = tas.attn_prefill_paged(
        q, to_dev(kp, "bf16"), to_dev(vp, "bf16"),
        torch.from_numpy(table).cuda(), prefix_len=inp.prefix_len,
        layout=layout, scale=inp.scale)
    # the same rows, contiguous
    kc, vc = oracle.gather_pages(kp, vp, table, layout)
    ref_dev = tas.attn_prefill(q, to_dev(kc, "bf16"), to_dev(vc, "bf16"),
                               prefix_len=inp.prefix_len, scale=inp.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_dev)
    if with_oracle:
        ref = oracle.prefill_paged(
            synth.as_f32(inp.q, "bf16"), synth.as_f32(kp, "bf16"),
            synth.as_f32(vp, "bf16"), table, inp.prefix_len, scale=inp.scale,
            layout=layout)
        err = max_abs_err(to_host64(out), ref)
        assert err <= tol("bf16"), err


@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("page_size", [64, 256])
def test_prefill_paged_prefix3072(layout, page_size):
    p = synth.WORKLOADS["prefill_prefix3072"].params
    inp = synth.prefill(p["seed"], p["B"], p["Hq"], p["Hkv"], p["D"], p["Lq"],
                        p["prefix_len"], p["max_length"], "bf16",
                        scale=p["scale"])
    say(f"prefill_paged 16 heads D=64 prefix=3072 Lq=1024 page={page_size} {layout}")
    check_paged(inp, page_size, layout, 81, with_oracle=page_size == 64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("layout", ["token", "head"])
@pytest.mark.parametrize("B,Hq,Hkv,Lq,prefix,extra,ps", [
    (1, 2, 2, 1, 0, 0, 64),        # single token, no prefix
    (1, 2, 1, 1, 37, 5, 64),       # single token after a prefix
    (2, 4, 2, 100, 0, 9, 128),     # pure causal, ragged query tile, GQA
    (1, 3, 3, 64, 64, 0, 64),      # tile-aligned
    (1, 8, 2, 65, 63, 30, 192),    # one past a tile
    (1, 4, 4, 33, 31, 3, 96),      # D=128 tiles: 32-row page multiples
    (2, 2, 2, 200, 333, 17, 64),   # ragged everything, several sequences
])
def test_prefill_paged_shapes(D, layout, B, Hq, Hkv, Lq, prefix, extra, ps):
    inp = synth.prefill(2000 + Lq + prefix, B, Hq, Hkv, D, Lq, prefix,
                        max_length=prefix + Lq + extra, dtype="bf16")
    if ps % (4096 // D):
        # pages must hold whole key tiles (4096 / D rows): the call is
        # refused before any launch
        k, v = _padded(inp, ps)
        kp, vp, table = synth.paginate(k, v, ps, 82 + Lq, layout=layout)
        with pytest.raises(tas.AttnArgError) as ei:
            tas.attn_prefill_paged(
                to_dev(inp.q, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16"),
                torch.from_numpy(table).cuda(), prefix_len=inp.prefix_len,
                layout=layout, scale=inp.scale)
        assert ei.value.status == tas.ATTN_E_UNSUPPORTED
        return
    say(f"prefill_paged D={D} B={B} Hq={Hq} Hkv={Hkv} Lq={Lq} prefix={prefix} "
        f"page={ps} {layout}")
    check_paged(inp, ps, layout, 82 + Lq)


@pytest.mark.parametrize("seed", range(12))
def test_prefill_paged_random_shapes(seed):
    # Seeded random shapes across the kernel forms (D 64 and 128; grids of
    # one and of two or more workgroups per CU; GQA groups; prefixes on and
    # off the key tile; ragged last query tiles), page sizes of one to six
    # key tiles and both page layouts: bit for bit against the contiguous
    # prefill and within the tolerance of the oracle.
    rng = np.random.default_rng(96000 + seed)
    while True:
        B = int(rng.choice([1, 2, 3]))
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        D = int(rng.choice([64, 128]))
        Lq = int(rng.integers(1, 700))
        prefix = int(rng.choice([0, 64, 128, int(rng.integers(1, 1200))]))
        if seed % 2 == 0:  # grids of two or more workgroups per CU (>= 768)
            Hkv = int(rng.choice([2, 4, 8]))
            Hq = 64
            B = 3
            Lq = int(rng.integers(200, 400))
            prefix = int(rng.integers(0, 200))
        if B * Hq * Lq * (prefix + Lq) <= 5e7:
            break
    extra = int(rng.integers(0, 50))
    ps = (4096 // D) * int(rng.integers(1, 7))
    layout = "token" if rng.random() < 0.5 else "head"
    inp = synth.prefill(97000 + seed, B, Hq, Hkv, D, Lq, prefix,
                        max_length=prefix + Lq + extra, dtype="bf16")
    say(f"prefill_paged random seed={seed} D={D} B={B} Hq={Hq} Hkv={Hkv} "
        f"Lq={Lq} prefix={prefix} extra={extra} page={ps} {layout}")
    check_paged(inp, ps, layout, 97000 + seed)


def test_prefill_paged_clamped_and_shared_pages():
    # entries past the last page or negative are clamped; two sequences may
    # share pages (a common prefix). Every page holds finite rows (no spare
    # pages, no rows past the new tokens), so any clamped page is readable.
    inp = synth.prefill(83, 2, 4, 4, 64, 70, 250, max_length=320, dtype="bf16")

    def fix(table):
        t = table.copy()
        t[1, 0] = t[0, 0]           # shared first page
        t[0, 2] = 10 ** 6           # clamped to the last page
        t[1, 3] = -7                # clamped to page 0
        return t
    say("prefill_paged clamped and shared pages")
    check_paged(inp, 64, "token", 84, table_fix=fix, extra_pages=0)


@pytest.mark.parametrize("layout", ["token", "head"])
def test_prefill_paged_d128_long(layout):
    inp = synth.prefill(85, 1, 8, 2, 128, 300, 1000, max_length=1400,
                        dtype="bf16")
    say(f"prefill_paged D=128 Hq=8 Hkv=2 Lq=300 prefix=1000 page=32 {layout}")
    check_paged(inp, 32, layout, 86)


@pytest.mark.parametrize("D,prefix,ps", [(64, 16500, 256), (128, 8300, 128)])
def test_prefill_paged_past_the_lane_table(D, prefix, ps):
    # a wave keeps the page offsets of its first 64 iterations in lanes;
    # later tiles (past 64 iterations x 4 quarters x 4096/D rows) are looked
    # up one by one
    inp = synth.prefill(87 + D, 1, 2, 1, D, 100, prefix,
                        max_length=prefix + 100 + 60, dtype="bf16")
    say(f"prefill_paged D={D} prefix={prefix} Lq=100 page={ps} (lookup path)")
    check_paged(inp, ps, "token", 88, with_oracle=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("layout", ["token", "head"])
def test_prefill_paged_two_workgroups_per_cu(D, layout):
    # 512 workgroups: the half-LDS kernels read the pages
    inp = synth.prefill(89 + D, 1, 64, 8, D, 512, 100, max_length=640,
                        dtype="bf16")
    say(f"prefill_paged D={D} Hq=64 Hkv=8 Lq=512 prefix=100 page=64 {layout}")
    check_paged(inp, 64, layout, 90)
