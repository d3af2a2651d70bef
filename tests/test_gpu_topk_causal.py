"""GPU parity of attn_topk_causal (decoder form of top-k) against the fp64
oracle.

Index sets, including the -1 padding of short rows, are compared exactly
wherever the oracle's gap between the last older score taken and the first
one left out exceeds what two fp64 summation orders can disagree by; in rows
where it does not, the GPU's set only has to be a valid choice under the
oracle's scores (same forced recent keys, older keys taken no worse than
those left out).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import F32_TOL, max_abs_err, say, to_dev

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def run(q, k, v, topk):
    qd, kd, vd = (to_dev(x, "f32") for x in (q, k, v))
    b, h, n, _ = q.shape
    idx = torch.full((b, h, n, topk), 12345, dtype=torch.int32, device="cuda")
    out = tas.attn_topk_causal(qd, kd, vd, topk, idx_out=idx)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), idx.cpu().numpy()


def check(q, k, v, topk, out, idx, ulp_allowance=False):
    """Exact index sets (outside ambiguous rows) and max abs error <= 1e-4;
    ulp_allowance adds one fp32 unit in the last place of the value, for the
    outlier-key outputs (~1e5) that no fp32 value can hold to 1e-4."""
    ref, ref_idx, gap = oracle.topk_causal_sparse(q, k, v, topk,
                                                  return_details=True)
    b, h, n, _ = q.shape
    r = topk // 2
    ambiguous = 0
    for bb in range(b):
        for hh in range(h):
            s = oracle.topk_scores(q[bb, hh], k[bb, hh])
            eps = 1e-10 * (1.0 + np.max(np.abs(s), axis=-1))
            amb = gap[bb, hh] <= eps
            ambiguous += int(amb.sum())
            clear = ~amb
            assert np.array_equal(idx[bb, hh][clear], ref_idx[bb, hh][clear])
            for i in np.nonzero(amb)[0]:
                got = idx[bb, hh, i]
                c = min(topk, i + 1)
                assert np.all(got[c:] == -1)
                sel = got[:c]
                assert np.all(np.diff(sel) > 0) and sel.min() >= 0
                assert sel.max() <= i
                assert set(range(i + 1 - r, i + 1)) <= set(sel.tolist())
                old = np.zeros(i + 1 - r, bool)
                old[sel[sel <= i - r]] = True
                assert s[i, :i + 1 - r][old].min() >= \
                    s[i, :i + 1 - r][~old].max() - eps[i]
                ref[bb, hh, i] = s[i, sel] @ v[bb, hh, sel].astype(np.float64)
    err = max_abs_err(out, ref)
    if ulp_allowance:
        excess = np.max(np.abs(out - ref) - 2.0 ** -23 * np.abs(ref))
        assert excess <= F32_TOL, (err, excess)
    else:
        assert err <= F32_TOL, err
    return ambiguous


def test_topk_causal_c2psa_shape():
    p = synth.WORKLOADS["topk_c2psa"].params
    inp = synth.topk(p["seed"], p["b"], p["h"], p["n"], p["d"], p["topk"])
    say("topk_causal b=32 h=3 n=512 d=64 topk=64")
    out, idx = run(inp.q, inp.k, inp.v, inp.topk)
    assert check(inp.q, inp.k, inp.v, inp.topk, out, idx) == 0


@pytest.mark.parametrize("n,topk", [
    (1, 1), (5, 2), (16, 16), (17, 16), (63, 7), (64, 64), (65, 1),
    (100, 33), (200, 3), (512, 512), (512, 2), (700, 64), (1024, 64),
    (1024, 1000)])
def test_topk_causal_sizes(n, topk):
    inp = synth.topk(140 + n, 2, 2, n, 64, topk)
    say(f"topk_causal n={n} topk={topk}")
    out, idx = run(inp.q, inp.k, inp.v, topk)
    check(inp.q, inp.k, inp.v, topk, out, idx)


@pytest.mark.parametrize("seed", range(12))
def test_topk_causal_random_shapes(seed):
    # Seeded random (b, h, n, topk) across the row-length classes of the
    # kernel (one to sixteen 64-key slots per lane), with topk from 1 to n so
    # that dense rows, the recent-key split and the score selection all meet
    # row tiles of every length.
    rng = np.random.default_rng(8000 + seed)
    b = int(rng.choice([1, 2, 3]))
    h = int(rng.choice([1, 2, 3]))
    n = int(rng.choice([int(rng.integers(1, 1025)), 64, 65, 128, 1023, 1024]))
    topk = int(rng.choice([1, 2, 3, int(rng.integers(1, n + 1)), min(n, 64), n]))
    inp = synth.topk(9000 + seed, b, h, n, 64, topk)
    say(f"topk_causal random seed={seed} b={b} h={h} n={n} topk={topk}")
    out, idx = run(inp.q, inp.k, inp.v, inp.topk)
    check(inp.q, inp.k, inp.v, inp.topk, out, idx)


def test_topk_causal_k_equals_n_is_lower_triangular():
    inp = synth.topk(150, 1, 3, 200, 64, 200)
    say("topk_causal k=n")
    out, idx = run(inp.q, inp.k, inp.v, 200)
    q, k, v = (x.astype(np.float64) for x in (inp.q, inp.k, inp.v))
    ref = np.tril(q @ np.swapaxes(k, -1, -2)) @ v
    assert max_abs_err(out, ref) <= F32_TOL
    for i in range(200):
        assert np.array_equal(idx[0, 0, i, :i + 1], np.arange(i + 1))
        assert np.all(idx[0, 0, i, i + 1:] == -1)


def test_topk_causal_exact_ties_lower_index_wins():
    inp = synth.topk(151, 1, 2, 256, 64, 40)
    k = inp.k.copy()
    for j in range(0, 256, 7):
        k[:, :, j] = k[:, :, 3]
    k[:, :, 200:230] = k[:, :, 100:101]
    say("topk_causal exact ties")
    for topk in (1, 10, 40, 37, 100):
        out, idx = run(inp.q, k, inp.v, topk)
        ref, ref_idx, _ = oracle.topk_causal_sparse(inp.q, k, inp.v, topk,
                                                    return_details=True)
        assert np.array_equal(idx, ref_idx), topk
        assert max_abs_err(out, ref) <= F32_TOL


@pytest.mark.parametrize("topk", [5, 64, 300])
def test_topk_causal_outlier_key_forces_exact_ranking(topk):
    inp = synth.topk(153, 1, 2, 512, 64, topk)
    k = inp.k.copy()
    k[:, :, 17] *= np.float32(1e5)
    say(f"topk_causal outlier key, topk={topk}")
    out, idx = run(inp.q, k, inp.v, topk)
    check(inp.q, k, inp.v, topk, out, idx, ulp_allowance=True)


def test_topk_causal_zero_queries_take_the_oldest_keys():
    inp = synth.topk(152, 1, 1, 130, 64, 9)
    q = inp.q.copy()
    q[0, 0, 20:40] = 0.0
    q[0, 0, 40:45] = -0.0
    say("topk_causal zero queries")
    out, idx = run(q, inp.k, inp.v, 9)
    for i in range(20, 45):  # all scores 0: older keys 0..4, recent i-3..i
        assert idx[0, 0, i].tolist() == list(range(5)) + list(range(i - 3, i + 1))
    assert np.all(out[0, 0, 20:45] == 0)
    check(q, inp.k, inp.v, 9, out, idx)


def test_topk_causal_repeatable_and_without_index_output():
    inp = synth.topk(154, 2, 3, 512, 64, 64)
    qd, kd, vd = (to_dev(x, "f32") for x in (inp.q, inp.k, inp.v))
    say("topk_causal repeatability")
    a = tas.attn_topk_causal(qd, kd, vd, 64)
    b = tas.attn_topk_causal(qd, kd, vd, 64)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    out, _ = run(inp.q, inp.k, inp.v, 64)
    assert np.array_equal(a.cpu().numpy().astype(np.float64), out)
