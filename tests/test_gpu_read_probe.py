"""The streaming-read probe reads every 16-byte word of its range exactly
once: the XOR each workgroup reports equals the XOR of its chunk computed on
the host, for ragged and empty chunks."""
import numpy as np
import pytest
import torch

from gpu_helpers import say

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


@pytest.mark.parametrize("n16,workgroups", [
    (1, 1), (1000, 7), (65536 + 3, 300), (5, 64), (0, 3), (1 << 20, 4096),
])
def test_read_probe_xor_per_chunk(n16, workgroups):
    rng = np.random.default_rng(n16 + workgroups)
    words = rng.integers(-2**31, 2**31, size=(n16, 4), dtype=np.int64).astype(np.int32)
    say(f"read probe n16={n16} workgroups={workgroups}")
    src = torch.from_numpy(words).cuda() if n16 else torch.empty((0, 4), dtype=torch.int32, device="cuda")
    sink = torch.full((workgroups, 4), -1, dtype=torch.int32, device="cuda")
    tas.attn_read_probe(src, workgroups, sink=sink)
    torch.cuda.synchronize()
    per = -(-n16 // workgroups) if n16 else 0
    want = np.zeros((workgroups, 4), np.int32)
    for w in range(workgroups):
        chunk = words[w * per:min((w + 1) * per, n16)]
        if len(chunk):
            want[w] = np.bitwise_xor.reduce(chunk, axis=0)
    assert np.array_equal(sink.cpu().numpy(), want)
