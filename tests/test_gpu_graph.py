"""Every entry point is capturable in a HIP graph (it allocates nothing,
synchronises nothing and enqueues only kernels on the given stream): a graph
of decode (split + combine), fused append, RoPE append, paged decode,
prefill, paged prefill and both top-k forms is replayed several times, with
eager work in between, and every replay must equal the eager results bit
for bit."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import say, to_dev

pytestmark = pytest.mark.gpu

import transformer_attention_split_amd as tas  # noqa: E402 (no skip: a missing library fails)


def test_graph_replays_equal_eager_calls():
    lens = np.array([1, 700, 4096, 2048], np.int32)
    dec = synth.decode_ragged(91, B=4, Hq=32, Hkv=8, D=128, max_length=4096,
                              dtype="bf16", lengths=lens)
    q, k, v = (to_dev(x, "bf16") for x in (dec.q, dec.k_cache, dec.v_cache))
    sl = torch.from_numpy(lens).cuda()
    kn, vn = (to_dev(x, "bf16") for x in synth.new_token_kv(91, 4, 8, 128, "bf16"))
    rng = np.random.default_rng(91)
    cos = torch.from_numpy(rng.standard_normal((4, 128)).astype(np.float32)).cuda()
    sin = torch.from_numpy(rng.standard_normal((4, 128)).astype(np.float32)).cuda()
    kp_np, vp_np, tab_np = synth.paginate(dec.k_cache, dec.v_cache, 256, 92,
                                          layout="head")
    kp, vp = to_dev(kp_np, "bf16"), to_dev(vp_np, "bf16")
    tab = torch.from_numpy(tab_np).cuda()
    pre = synth.prefill(93, 1, 4, 2, 64, 200, 300, dtype="bf16")
    pq, pk, pv = (to_dev(x, "bf16") for x in (pre.q, pre.k_cache, pre.v_cache))
    # paged prefill over the same prefix cache (500 rows -> 512, NaN padded)
    pad = np.full((1, 2, 12, 64), synth.BF16_QNAN, pre.k_cache.dtype)
    ppk_np, ppv_np, ptab_np = synth.paginate(
        np.concatenate([pre.k_cache, pad], 2), np.concatenate([pre.v_cache, pad], 2),
        64, 94)
    ppk, ppv = to_dev(ppk_np, "bf16"), to_dev(ppv_np, "bf16")
    ptab = torch.from_numpy(ptab_np).cuda()
    tk = synth.topk(95, 2, 3, 300, 64, 32)
    tq, tkk, tv = (torch.from_numpy(x).cuda() for x in (tk.q, tk.k, tk.v))

    need = tas.attn_decode_workspace_bytes(4, 32, 8, 128, 4096)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    k_app, v_app = k.clone(), v.clone()
    k_rope, v_rope = k.clone(), v.clone()

    def calls(o):
        tas.attn_decode(q, k, v, seq_lens=sl, out=o["dec"], workspace=ws)
        tas.attn_decode_append(q, kn, vn, k_app, v_app, seq_lens=sl,
                               out=o["app"], workspace=ws)
        tas.attn_decode_append_rope(q, kn, vn, cos, sin, k_rope, v_rope,
                                    seq_lens=sl, out=o["rope"], workspace=ws)
        tas.attn_decode_paged(q, kp, vp, tab, layout="head", seq_lens=sl,
                              out=o["paged"], workspace=ws)
        tas.attn_prefill(pq, pk, pv, prefix_len=300, out=o["pre"])
        tas.attn_prefill_paged(pq, ppk, ppv, ptab, prefix_len=300,
                               out=o["ppre"])
        tas.attn_topk(tq, tkk, tv, 32, out=o["topk"])
        tas.attn_topk_causal(tq, tkk, tv, 32, out=o["topkc"])

    shapes = dict(dec=q, app=q, rope=q, paged=q, pre=pq, ppre=pq, topk=tq,
                  topkc=tq)
    eager = {n: torch.empty_like(t) for n, t in shapes.items()}
    graph_out = {n: torch.empty_like(t) for n, t in shapes.items()}
    say("graph: eager reference")
    calls(eager)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        calls(graph_out)  # warm-up outside capture
    torch.cuda.synchronize()
    say("graph: capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        calls(graph_out)
    for r in range(4):
        for t in graph_out.values():
            t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        say(f"graph: replay {r}")
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for n in eager:
            assert torch.equal(graph_out[n], eager[n]), (r, n)
