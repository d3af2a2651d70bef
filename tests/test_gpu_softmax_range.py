"""The online softmax of decode and prefill under score ranges far from
N(0, 1): keys scaled up along the sequence (the running maximum keeps
moving, so the rescale of the output and the row sum is taken many times,
also in later tiles and splits), keys scaled down along it (the maximum
settles early), and scores in the thousands (one key dominates; the others
underflow to zero weight). Every case is checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import max_abs_err, say, to_dev, to_host64, tol

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)

PROFILES = {
    "growing": lambda x: 1.0 + 6.0 * x,          # max moves up to the end
    "shrinking": lambda x: 7.0 - 6.0 * x,        # max found early
    "huge": lambda x: 60.0 + 0.0 * x,            # scores in the thousands
}


def scaled(arr, dtype, factors):
    """Cache [B, Hkv, M, D] with row r multiplied by factors[r]; bf16 values
    are rounded again to bf16."""
    x = synth.as_f32(arr, dtype) * factors[None, None, :, None].astype(np.float32)
    return synth.f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float32)


@pytest.mark.parametrize("profile", sorted(PROFILES))
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_decode_score_ranges(profile, dtype, D):
    lens = np.array([1, 300, 2048, 1500], np.int32)
    inp = synth.decode_ragged(501, B=4, Hq=8, Hkv=2, D=D, max_length=2048,
                              dtype=dtype, lengths=lens)
    q, kc = inp.q, inp.k_cache
    if dtype == "f32" and profile == "huge":
        # Scores in the thousands: an fp32 dot product there is off by up to
        # ~1e-4 from rounding alone, which no fp32 result can keep under the
        # 1e-4 bound. With integer-valued q and keys every product and partial
        # sum is an integer below 2^24, so the fp32 scores are exact in any
        # summation order and the case tests the softmax, not the rounding.
        q = np.round(q * 4).astype(np.float32)
        kc = np.where(np.isnan(kc), kc, np.round(kc * 4)).astype(np.float32)
    f = PROFILES[profile](np.arange(2048) / 2048.0)
    k = scaled(kc, dtype, f)
    say(f"decode {dtype} D={D} keys {profile}")
    for split_rows in (0, 128):
        out = tas.attn_decode(to_dev(q, dtype), to_dev(k, dtype),
                              to_dev(inp.v_cache, dtype),
                              seq_lens=torch.from_numpy(lens).cuda(),
                              split_rows=split_rows)
        torch.cuda.synchronize()
        ref = oracle.decode(synth.as_f32(q, dtype), synth.as_f32(k, dtype),
                            synth.as_f32(inp.v_cache, dtype), seq_lens=lens)
        err = max_abs_err(to_host64(out), ref)
        assert err <= tol(dtype), (split_rows, err)


@pytest.mark.parametrize("profile", sorted(PROFILES))
@pytest.mark.parametrize("D,Hq,Hkv,Lq,prefix", [
    (64, 4, 4, 200, 900),      # 8 KiB tiles, one workgroup per CU
    (128, 4, 2, 130, 700),
    (64, 64, 8, 512, 300),     # 4 KiB tiles, two workgroups per CU
])
def test_prefill_score_ranges(profile, D, Hq, Hkv, Lq, prefix):
    inp = synth.prefill(502 + D, 1, Hq, Hkv, D, Lq, prefix, dtype="bf16")
    T = prefix + Lq
    f = PROFILES[profile](np.arange(T) / T)
    k = scaled(inp.k_cache, "bf16", f)
    say(f"prefill D={D} Hq={Hq} keys {profile}")
    out = tas.attn_prefill(to_dev(inp.q, "bf16"), to_dev(k, "bf16"),
                           to_dev(inp.v_cache, "bf16"), prefix_len=prefix)
    torch.cuda.synchronize()
    ref = oracle.prefill(synth.as_f32(inp.q, "bf16"), synth.as_f32(k, "bf16"),
                         synth.as_f32(inp.v_cache, "bf16"), prefix)
    err = max_abs_err(to_host64(out), ref)
    assert err <= tol("bf16"), err
