"""attn_decode_noalloc, the decode whose split partials live in the
library's static scratch array, against attn_decode with a caller
workspace: two calls in a row on one GPU, the second smaller than the first
(so the scratch holds the first call's partials when the second starts),
each bit for bit equal to attn_decode on the same inputs and within the bf16
bound of the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import max_abs_err, say, to_dev, to_host64, tol

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def check(inp, split_rows):
    q, k, v = (to_dev(x, inp.dtype) for x in (inp.q, inp.k_cache, inp.v_cache))
    lens = None
    if inp.seq_lens is not None:
        lens = torch.from_numpy(inp.seq_lens.astype(np.int32)).cuda()
    out = torch.empty_like(q)
    got = tas.attn_decode_noalloc(q, k, v, out, position_id=inp.position_id,
                                  seq_lens=lens, scale=inp.scale,
                                  split_rows=split_rows)
    ref_dev = tas.attn_decode(q, k, v, position_id=inp.position_id,
                              seq_lens=lens, scale=inp.scale,
                              split_rows=split_rows)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got, ref_dev)
    ref = oracle.decode(synth.as_f32(inp.q, inp.dtype),
                        synth.as_f32(inp.k_cache, inp.dtype),
                        synth.as_f32(inp.v_cache, inp.dtype),
                        position_id=inp.position_id, seq_lens=inp.seq_lens,
                        scale=inp.scale)
    err = max_abs_err(to_host64(got), ref)
    assert err <= tol(inp.dtype), err


def test_noalloc_two_calls_second_smaller():
    big = synth.decode_ragged(91, B=16, Hq=32, Hkv=8, D=128, max_length=4096,
                              dtype="bf16")
    say("decode_noalloc bf16 B=16 Hq=32 Hkv=8 D=128 max=4096 ragged, split 256")
    check(big, 256)
    small = synth.decode_uniform(92, 2, 8, 2, 64, 1024, 700, "f32",
                                 poison=True)
    say("decode_noalloc f32 B=2 Hq=8 Hkv=2 D=64 max=1024 pos=700, split 64")
    check(small, 64)
    say("decode_noalloc bf16 B=16 again after the smaller call")
    check(big, 0)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, 8, 256, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(64, dtype=torch.int32, device="cuda")
    with pytest.raises(tas.AttnArgError) as ei:
        # 1-row splits of 64 sequences of 256 rows: partials far beyond 64 MiB
        tas.attn_decode_noalloc(q, k, k, torch.empty_like(q), seq_lens=lens,
                                split_rows=1)
    assert ei.value.status == tas.ATTN_E_WORKSPACE
