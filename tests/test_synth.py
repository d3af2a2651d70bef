"""CPU checks of the input recipes in ``synth`` that shape inputs beyond
plain draws."""
import numpy as np

import oracle
import synth


def test_needles_carry_the_weight():
    # With V = 1 on the rows plant_needles overwrote and 0 elsewhere, the
    # oracle's output is the softmax weight on those rows, for every head.
    lens = np.array([1, 2, 700, 0, 5000], np.int32)
    B, Hq, Hkv, D, M = len(lens), 8, 2, 128, 5000
    inp = synth.decode_ragged(5, B, Hq, Hkv, D, M, "bf16", lengths=lens)
    before = inp.k_cache.copy()
    keys = synth.plant_needles(5, inp.q, inp.k_cache, lens, "bf16")
    changed = np.any(inp.k_cache != before, axis=-1)        # [B, Hkv, M]
    for b, L in enumerate(lens):
        assert not changed[b, :, L:].any()
        for g in range(Hkv):
            rows = np.flatnonzero(np.all(inp.k_cache[b, g] == keys[b, g], -1))
            if L == 0:
                assert rows.size == 0
                continue
            assert 1 <= rows.size <= 4 and rows.max() < L
            assert (0 if g % 2 == 0 else L - 1) in rows
    ind = np.zeros((B, Hkv, M, D), np.float32)
    for b in range(B):
        for g in range(Hkv):
            ind[b, g, np.all(inp.k_cache[b, g] == keys[b, g], -1)] = 1.0
    w = oracle.decode(synth.as_f32(inp.q, "bf16"),
                      synth.as_f32(inp.k_cache, "bf16"), ind, seq_lens=lens)
    assert np.all(w[lens == 0] == 0)
    assert w[lens > 0].min() > 0.99, w[lens > 0].min()
