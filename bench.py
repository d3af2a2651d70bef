#!/usr/bin/env python3
"""Benchmark of the KV-cache attention hot path on one MI355X.

One step runs every operation of the path once over resident synthetic
inputs, on the stream the library launches on:

  decode   ragged batch: B=64, Hq=32, Hkv=8, D=128, bf16, static cache of
           max_length 8192, per-sequence lengths uniform in [1, 8192]
           (one attn_decode call for the whole batch)              <- headline
  prefill  causal prefill: 16 heads, D=64, prefix 3072 + 1024 new tokens
  topk     top-k sparse scores: b=32, 3 head groups, n=512, d=64, topk=64

`value` is the decode KV-read bandwidth: algorithmic bytes (every valid K and
V row once per kv head, plus q and out) divided by the decode time measured
with HIP events around each decode call. Prefill TFLOP/s (causal FLOPs) and
top-k figures are reported beside it. Inputs are synthetic (seeded N(0,1),
bf16 rounded to nearest even), generated once and resident in HBM before the
timed region starts.

Unless --no-secondary is given, the `secondary` object also times the fused
append (plain and with the rotary embedding), the paged decode and the
fp32 decode on the decode batch, the decoder-causal top-k, the paged prefill, the prefill shape
at head size 128 and with 32 heads, and the single-sequence decode at
position 8000 (cold and warm, from a captured graph; --no-single skips only
that part).

The `context` object holds the read bandwidth a compute-free streaming read
over 4 GiB attains (attn_read_probe), against which the decode bandwidth can
be read, and the GPU's clock levels, performance level, power and
temperatures (sysfs) just before and after the timed steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-secondary | --no-single] [--calib-copy]
"""
import argparse
import glob
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FP64_PEAK_TFLOPS = 78.6         # MI355X fp64 (vector and matrix)
METRIC = ("decode KV-read GB/s (% HBM peak) at ctx 8192; "
          "prefill TFLOP/s (% MFMA peak)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip every secondary figure (fused append, paged "
                         "forms, other prefill shapes, single-sequence decode)")
    ap.add_argument("--no-single", action="store_true",
                    help="skip only the single-sequence position-8000 figures "
                         "(graph replays of thousands of calls)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy (counter calibration)")
    return ap.parse_args()


# ----------------------------------------------------------------------------
# Inputs
# ----------------------------------------------------------------------------
def bf16_dev(arr, torch):
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def make_decode(torch, synth, tas):
    import numpy as np
    p = synth.WORKLOADS["decode_ragged_b64"].params
    B, Hq, Hkv, D, M = p["B"], p["Hq"], p["Hkv"], p["D"], p["max_length"]
    lens = synth.ragged_lengths(p["seed"], B, M)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(B, Hkv, M, D, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    for b, L, qb, kb, vb in synth.iter_ragged(p["seed"], B, Hq, Hkv, D, M,
                                               "bf16", lens):
        q[b] = bf16_dev(qb, torch)
        k[b, :, :L] = bf16_dev(kb, torch)
        v[b, :, :L] = bf16_dev(vb, torch)
    sl = torch.from_numpy(lens.astype(np.int32)).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(1, tas.attn_decode_workspace_bytes(B, Hq, Hkv, D, M)),
                     dtype=torch.uint8, device="cuda")
    nbytes = 2 * Hkv * D * 2 * int(lens.sum()) + 2 * B * Hq * D * 2
    return dict(p=p, q=q, k=k, v=v, seq_lens=sl, lens=lens, out=out, ws=ws,
                bytes=nbytes)


def make_prefill(torch, synth):
    p = synth.WORKLOADS["prefill_prefix3072"].params
    inp = synth.prefill(p["seed"], p["B"], p["Hq"], p["Hkv"], p["D"], p["Lq"],
                        p["prefix_len"], p["max_length"], "bf16",
                        poison=False, scale=p["scale"])
    q, k, v = (bf16_dev(x, torch) for x in (inp.q, inp.k_cache, inp.v_cache))
    D, H, Lq, P = p["D"], p["Hq"], p["Lq"], p["prefix_len"]
    flops = 4 * D * H * p["B"] * sum(P + i + 1 for i in range(Lq))
    return dict(p=p, q=q, k=k, v=v, out=torch.empty_like(q), flops=flops)


def make_topk(torch, synth):
    import numpy as np
    p = synth.WORKLOADS["topk_c2psa"].params
    inp = synth.topk(p["seed"], p["b"], p["h"], p["n"], p["d"], p["topk"])
    q, k, v = (torch.from_numpy(x).cuda() for x in (inp.q, inp.k, inp.v))
    b, h, n, d, kk = p["b"], p["h"], p["n"], p["d"], p["topk"]
    flops = b * h * (2 * n * n * d + 2 * n * kk * d)
    # decoder-causal form: row i scores keys j <= i and sums min(k, i+1) rows
    rows = np.arange(1, n + 1)
    flops_causal = int(b * h * 2 * d * (rows.sum() + np.minimum(kk, rows).sum()))
    return dict(p=p, q=q, k=k, v=v, out=torch.empty_like(q), flops=flops,
                flops_causal=flops_causal)


# ----------------------------------------------------------------------------
# Secondary: one sequence at position 8000 of an 8192-row cache
# ----------------------------------------------------------------------------
def bench_single_position(torch, tas, synth, copies=32, reps=20):
    """Single-sequence GQA decode (B=1, Hq=32, Hkv=8, D=128, bf16) at
    position 8000, replayed from a captured graph of `copies` calls. Cold:
    each call reads a different cache copy (copies * 32 MiB, well past the
    256 MiB MALL). Warm: every call reads the same copy."""
    import numpy as np
    p = synth.WORKLOADS["decode_gqa_static"].params
    pos = 8000
    inp = synth.decode_uniform(p["seed"], 1, p["Hq"], p["Hkv"], p["D"],
                               p["max_length"], pos, "bf16", poison=False)
    q = bf16_dev(inp.q, torch)
    k0 = bf16_dev(inp.k_cache, torch)
    v0 = bf16_dev(inp.v_cache, torch)
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    out = torch.empty_like(q)
    ws = torch.zeros(tas.attn_decode_workspace_bytes(1, 32, 8, 128, 8192),
                     dtype=torch.uint8, device="cuda")
    nbytes = 2 * 8 * 128 * 2 * (pos + 1) + 2 * 32 * 128 * 2
    res = {}
    s = torch.cuda.Stream()
    for mode in ("cold", "warm"):
        idx = list(range(copies)) if mode == "cold" else [0] * copies
        with torch.cuda.stream(s):
            for i in idx[:4]:  # warm-up outside capture
                tas.attn_decode(q, ks[i], vs[i], position_id=pos,
                                scale=p["scale"], out=out, workspace=ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in idx:
                tas.attn_decode(q, ks[i], vs[i], position_id=pos,
                                scale=p["scale"], out=out, workspace=ws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):  # replay and events on the same stream
            g.replay()
            torch.cuda.synchronize()
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * copies)
        res[mode] = dict(us_per_call=round(us, 3),
                         GBps=round(nbytes / (us * 1e-6) / 1e9, 1))
        del g
    ref = out.float().cpu().numpy()
    assert np.all(np.isfinite(ref))
    del ks, vs
    # Time against position (warm, one cache): the work of a call is
    # proportional to the valid rows, so the time should be affine in p+1.
    sweep = []
    for pp in (0, 100, 1000, 4000, 8000):
        with torch.cuda.stream(s):
            for _ in range(4):
                tas.attn_decode(q, k0, v0, position_id=pp, scale=p["scale"],
                                out=out, workspace=ws)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(copies):
                tas.attn_decode(q, k0, v0, position_id=pp, scale=p["scale"],
                                out=out, workspace=ws)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            g.replay()
            torch.cuda.synchronize()
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        sweep.append((pp, e0.elapsed_time(e1) * 1e3 / (reps * copies)))
        del g
    xs = np.array([pp + 1 for pp, _ in sweep], dtype=np.float64)
    ys = np.array([us for _, us in sweep])
    slope, icpt = np.polyfit(xs[1:], ys[1:], 1)  # p >= 100
    torch.cuda.empty_cache()
    return dict(workload="decode_gqa_static_pos8000", bytes=nbytes,
                calls_per_graph=copies, **res,
                warm_us_by_position={str(pp): round(us, 3) for pp, us in sweep},
                warm_fit_us=dict(per_1000_rows=round(slope * 1000, 4),
                                 intercept=round(icpt, 3)))


# ----------------------------------------------------------------------------
# Secondary: the cache append fused into the decode call
# ----------------------------------------------------------------------------
def bench_append(torch, tas, dec, steps):
    """attn_decode_append on the ragged batch (each call stores one new K/V
    row per (sequence, kv head) and attends to it) against attn_decode on the
    same inputs, alternating calls, HIP events around each. The caches keep
    the appended rows afterwards; the decode output buffer is not touched."""
    import numpy as np
    p = dec["p"]
    B, Hkv, D = p["B"], p["Hkv"], p["D"]
    g = torch.Generator(device="cuda").manual_seed(1234)
    k_new = torch.randn(B, Hkv, D, device="cuda", generator=g).bfloat16()
    v_new = torch.randn(B, Hkv, D, device="cuda", generator=g).bfloat16()
    out = torch.empty_like(dec["out"])
    kw = dict(seq_lens=dec["seq_lens"], scale=p["scale"], out=out,
              workspace=dec["ws"])
    # rotary tables of each sequence's current row (rotate-half layout)
    rows = torch.clamp(dec["seq_lens"].long() - 1, min=0).double()
    inv = 10000.0 ** (-torch.arange(0, D, 2, device="cuda").double() / D)
    ang = rows[:, None] * inv[None, :]
    ang = torch.cat([ang, ang], dim=-1)
    cos, sin = ang.cos().float().contiguous(), ang.sin().float().contiguous()
    calls = (
        lambda: tas.attn_decode_append(dec["q"], k_new, v_new, dec["k"],
                                       dec["v"], **kw),
        lambda: tas.attn_decode_append_rope(dec["q"], k_new, v_new, cos, sin,
                                            dec["k"], dec["v"], **kw),
        lambda: tas.attn_decode(dec["q"], dec["k"], dec["v"], **kw),
    )
    for _ in range(5):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
          for _ in range(steps)]
    for e in ev:
        for i, c in enumerate(calls):
            e[i].record()
            c()
        e[3].record()
    torch.cuda.synchronize()
    ta, tr, td = (float(np.median([e[i].elapsed_time(e[i + 1]) * 1e3
                                   for e in ev])) for i in range(3))
    return dict(workload="decode_ragged_b64 + append of one row per "
                         "(sequence, kv head)",
                us_p50_append_decode=round(ta, 2),
                us_p50_rope_append_decode=round(tr, 2),
                us_p50_decode=round(td, 2),
                GBps_append_decode=round(dec["bytes"] / (ta * 1e-6) / 1e9, 1),
                GBps_rope_append_decode=round(dec["bytes"] / (tr * 1e-6) / 1e9, 1))


def bench_decode_f32(torch, tas, dec, steps):
    """The ragged decode batch with fp32 caches (the bf16 values upcast, so
    twice the bytes): the vector-ALU kernel on the plain split grid, HIP
    events around each call."""
    import numpy as np
    p = dec["p"]
    q, k, v = dec["q"].float(), dec["k"].float(), dec["v"].float()
    out = torch.empty_like(q)
    kw = dict(seq_lens=dec["seq_lens"], scale=p["scale"], out=out,
              workspace=dec["ws"])
    for _ in range(3):
        tas.attn_decode(q, k, v, **kw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
          for _ in range(steps)]
    for e in ev:
        e[0].record()
        tas.attn_decode(q, k, v, **kw)
        e[1].record()
    torch.cuda.synchronize()
    t = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in ev]))
    nbytes = 2 * dec["bytes"]
    del q, k, v, out
    torch.cuda.empty_cache()
    gbps = nbytes / (t * 1e-6) / 1e9
    return dict(workload="decode_ragged_b64 with fp32 caches",
                us_p50=round(t, 2), bytes=nbytes, GBps=round(gbps, 1),
                frac_of_hbm_peak=round(gbps / HBM_PEAK_GBPS, 4))


def bench_paged(torch, tas, dec, steps, page_size, layout):
    """attn_decode_paged on the ragged batch cut into pages of `page_size`
    rows (token- or head-major) in a shuffled order, built on the device from
    the contiguous cache, against attn_decode on the contiguous cache."""
    import numpy as np
    p = dec["p"]
    B, Hkv, D, M = p["B"], p["Hkv"], p["D"], p["max_length"]
    nb = M // page_size
    g = torch.Generator(device="cpu").manual_seed(4321)
    perm = torch.randperm(B * nb, generator=g).to(torch.int32)
    table = perm.view(B, nb).cuda()
    perm_dims = (0, 2, 3, 1, 4) if layout == "token" else (0, 2, 1, 3, 4)
    src_k = dec["k"].view(B, Hkv, nb, page_size, D).permute(*perm_dims)
    src_v = dec["v"].view(B, Hkv, nb, page_size, D).permute(*perm_dims)
    kp = torch.empty((B * nb,) + tuple(src_k.shape[2:]), dtype=torch.bfloat16,
                     device="cuda")
    vp = torch.empty_like(kp)
    idx = table.view(-1).long()
    kp[idx] = src_k.reshape(kp.shape)
    vp[idx] = src_v.reshape(vp.shape)
    out = torch.empty_like(dec["out"])
    kw = dict(seq_lens=dec["seq_lens"], scale=p["scale"], out=out,
              workspace=dec["ws"])
    for _ in range(5):
        tas.attn_decode_paged(dec["q"], kp, vp, table, layout=layout, **kw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
          for _ in range(steps)]
    for e in ev:
        e[0].record()
        tas.attn_decode_paged(dec["q"], kp, vp, table, layout=layout, **kw)
        e[1].record()
        tas.attn_decode(dec["q"], dec["k"], dec["v"], **kw)
        e[2].record()
    torch.cuda.synchronize()
    tp = float(np.median([e[0].elapsed_time(e[1]) * 1e3 for e in ev]))
    td = float(np.median([e[1].elapsed_time(e[2]) * 1e3 for e in ev]))
    del kp, vp
    torch.cuda.empty_cache()
    return dict(workload=f"decode_ragged_b64 in shuffled {page_size}-row "
                         f"{layout}-major pages",
                us_p50_paged=round(tp, 2), us_p50_contiguous=round(td, 2),
                GBps_paged=round(dec["bytes"] / (tp * 1e-6) / 1e9, 1))


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the decode workload
# ----------------------------------------------------------------------------
def bench_prefill_shape(torch, tas, synth, D, H, n=20, Hkv=None):
    """The prefill workload's prefix and new tokens with head size D, H query
    heads over Hkv kv heads (default H), n back-to-back calls between two
    events."""
    p = synth.WORKLOADS["prefill_prefix3072"].params
    Hkv = H if Hkv is None else Hkv
    inp = synth.prefill(p["seed"], 1, H, Hkv, D, p["Lq"], p["prefix_len"],
                        p["max_length"], "bf16", poison=False, scale=D ** -0.5)
    q, k, v = (bf16_dev(x, torch) for x in (inp.q, inp.k_cache, inp.v_cache))
    out = torch.empty_like(q)

    def fn():
        tas.attn_prefill(q, k, v, prefix_len=p["prefix_len"], scale=D ** -0.5,
                         out=out)
    for _ in range(3):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n
    flops = 4 * D * H * sum(p["prefix_len"] + i + 1 for i in range(p["Lq"]))
    del q, k, v, out
    torch.cuda.empty_cache()
    return dict(workload=f"prefill_prefix3072 at D={D} ({H} query heads over "
                         f"{Hkv} kv heads)",
                us_back_to_back=round(us, 2), flops=flops,
                TFLOPs_back_to_back=round(flops / us / 1e6, 1),
                frac_of_bf16_mfma_peak=round(flops / us / 1e6
                                             / BF16_MFMA_PEAK_TFLOPS, 4))


def bench_prefill_paged(torch, tas, pre, page_size, layout, n=20):
    """attn_prefill_paged on the prefill workload's cache cut into shuffled
    pages of `page_size` rows, against attn_prefill on the contiguous cache:
    n back-to-back calls of each between two events."""
    p = pre["p"]
    B, Hkv, D, M = p["B"], p["Hkv"], p["D"], p["max_length"]
    nb = M // page_size
    g = torch.Generator(device="cpu").manual_seed(4322)
    table = torch.randperm(B * nb, generator=g).to(torch.int32).view(B, nb).cuda()
    perm_dims = (0, 2, 3, 1, 4) if layout == "token" else (0, 2, 1, 3, 4)
    src_k = pre["k"].view(B, Hkv, nb, page_size, D).permute(*perm_dims)
    src_v = pre["v"].view(B, Hkv, nb, page_size, D).permute(*perm_dims)
    kp = torch.empty((B * nb,) + tuple(src_k.shape[2:]), dtype=torch.bfloat16,
                     device="cuda")
    vp = torch.empty_like(kp)
    idx = table.view(-1).long()
    kp[idx] = src_k.reshape(kp.shape)
    vp[idx] = src_v.reshape(vp.shape)
    out = torch.empty_like(pre["out"])

    def timed(fn):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n
    tp = timed(lambda: tas.attn_prefill_paged(
        pre["q"], kp, vp, table, prefix_len=p["prefix_len"], layout=layout,
        scale=p["scale"], out=out))
    tc = timed(lambda: tas.attn_prefill(
        pre["q"], pre["k"], pre["v"], prefix_len=p["prefix_len"],
        scale=p["scale"], out=out))
    del kp, vp
    torch.cuda.empty_cache()
    return dict(workload=f"prefill_prefix3072 in shuffled {page_size}-row "
                         f"{layout}-major pages",
                us_back_to_back_paged=round(tp, 2),
                us_back_to_back_contiguous=round(tc, 2),
                TFLOPs_paged=round(pre["flops"] / tp / 1e6, 1))


def gpu_state(torch):
    """Clock levels in use, performance level, power and temperatures of
    cuda:0, read from sysfs (the state beside a measurement); None where the
    files cannot be read."""
    try:
        pr = torch.cuda.get_device_properties(0)
        dev = (f"/sys/bus/pci/devices/{pr.pci_domain_id:04x}:"
               f"{pr.pci_bus_id:02x}:{pr.pci_device_id:02x}.0")
    except Exception:
        return None
    if not os.path.isdir(dev):
        return None

    def read(path):
        try:
            with open(path) as f:
                return f.read().strip()
        except OSError:
            return None

    def level(name):
        text = read(os.path.join(dev, name))
        for ln in (text or "").splitlines():
            if ln.rstrip().endswith("*"):
                return ln.split(":", 1)[-1].rstrip("* ").strip()
        return None

    st = {"pci": os.path.basename(dev), "sclk": level("pp_dpm_sclk"),
          "mclk": level("pp_dpm_mclk"), "fclk": level("pp_dpm_fclk"),
          "performance_level": read(os.path.join(
              dev, "power_dpm_force_performance_level"))}
    for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
        for name in ("power1_average", "power1_input"):
            v = read(os.path.join(hw, name))
            if v and "power_w" not in st:
                st["power_w"] = round(int(v) * 1e-6, 1)
        for tin in sorted(glob.glob(os.path.join(hw, "temp*_input"))):
            v = read(tin)
            lab = read(tin.replace("_input", "_label")) or os.path.basename(tin)
            if v:
                st[f"temp_{lab}_c"] = round(int(v) * 1e-3, 1)
    return st


def bench_read_probe(torch, tas, gib=4, reps=20):
    """Attainable HBM read bandwidth: attn_read_probe over `gib` GiB (every
    byte read once with 16-byte non-temporal loads) at three grid sizes,
    `reps` back-to-back calls each between two events."""
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    by_wg = {}
    for wg in (2048, 4096, 8192):
        sink = torch.empty((wg, 4), dtype=torch.int32, device="cuda")
        for _ in range(3):
            tas.attn_read_probe(buf, wg, sink=sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            tas.attn_read_probe(buf, wg, sink=sink)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        by_wg[str(wg)] = round(nbytes / us / 1e3, 1)
    del buf
    torch.cuda.empty_cache()
    best = max(by_wg.values())
    return dict(bytes=nbytes, GBps=best,
                frac_of_hbm_peak=round(best / HBM_PEAK_GBPS, 4),
                GBps_by_workgroups=by_wg)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return platform.processor() or "unknown"


def cpu_baseline(dec, synth):
    """The fp64 NumPy oracle, as it stands, timed on this machine's host
    cores on a bounded sample of every configuration point: one warm-up run
    and the median of three, once with as many BLAS threads as the process
    may use and once with one, reported in the numerators of the GPU line
    (decode bytes per second, prefill and top-k FLOP per second). Inputs are
    generated and converted to float before the timed runs."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits

    W = synth.WORKLOADS
    f32 = synth.as_f32
    points = []  # (name, fn, numerator, unit, sample)

    p1 = W["decode_f32_tiny"].params
    c1 = synth.decode_uniform(p1["seed"], p1["B"], p1["Hq"], p1["Hkv"], p1["D"],
                              p1["max_length"], p1["position_id"], "f32",
                              poison=True, scale=p1["scale"])
    nb1 = 2 * p1["Hkv"] * p1["D"] * 4 * (p1["position_id"] + 1) + \
        2 * p1["Hq"] * p1["D"] * 4
    points.append(("decode_f32_tiny", lambda: oracle.decode(
        c1.q, c1.k_cache, c1.v_cache, position_id=p1["position_id"],
        scale=p1["scale"]), nb1, "GB/s", "whole workload"))

    p2 = W["decode_gqa_static"].params
    c2 = synth.decode_uniform(p2["seed"], p2["B"], p2["Hq"], p2["Hkv"], p2["D"],
                              p2["max_length"], p2["max_length"] - 1, "bf16",
                              poison=False, scale=p2["scale"])
    q2, k2, v2 = (f32(x, "bf16") for x in (c2.q, c2.k_cache, c2.v_cache))
    for pos in p2["positions"]:
        nb = 2 * p2["Hkv"] * p2["D"] * 2 * (pos + 1) + 2 * p2["Hq"] * p2["D"] * 2
        points.append((f"decode_gqa_static_p{pos}", lambda pos=pos: oracle.decode(
            q2, k2, v2, position_id=pos, scale=p2["scale"]), nb, "GB/s",
            "whole workload"))

    p3 = dec["p"]
    n3 = p3["B"]
    seqs = []
    nb3 = 0
    for b in range(n3):
        L = int(dec["lens"][b])
        qb, kb, vb = synth.ragged_sequence(p3["seed"], b, p3["Hq"], p3["Hkv"],
                                           p3["D"], L, "bf16")
        seqs.append((L,) + tuple(synth.bf16_to_f32(x) for x in (qb, kb, vb)))
        nb3 += 2 * p3["Hkv"] * p3["D"] * 2 * L + 2 * p3["Hq"] * p3["D"] * 2
    outs3 = []

    def run3():
        outs3.clear()
        for L, qf, kf, vf in seqs:
            outs3.append(oracle.decode_sequence(qf, kf, vf, L, p3["scale"]))
    points.append(("decode_ragged_b64", run3, nb3, "GB/s",
                   f"all {n3} sequences ({sum(x[0] for x in seqs)} rows)"))

    p4 = W["prefill_prefix3072"].params
    c4 = synth.prefill(p4["seed"], p4["B"], p4["Hq"], p4["Hkv"], p4["D"],
                       p4["Lq"], p4["prefix_len"], p4["max_length"], "bf16",
                       scale=p4["scale"])
    h4 = p4["Hq"]
    q4, k4, v4 = (np.ascontiguousarray(f32(x, "bf16")[:, :h4])
                  for x in (c4.q, c4.k_cache, c4.v_cache))
    fl4 = 4 * p4["D"] * h4 * sum(p4["prefix_len"] + i + 1 for i in range(p4["Lq"]))
    points.append(("prefill_prefix3072", lambda: oracle.prefill(
        q4, k4, v4, p4["prefix_len"], scale=p4["scale"]), fl4, "GFLOP/s",
        f"all {h4} heads"))

    p5 = W["topk_c2psa"].params
    c5 = synth.topk(p5["seed"], p5["b"], p5["h"], p5["n"], p5["d"], p5["topk"])
    b5 = 8
    q5, k5, v5 = (np.ascontiguousarray(x[:b5]) for x in (c5.q, c5.k, c5.v))
    fl5 = b5 * p5["h"] * p5["n"] * (2 * p5["n"] * p5["d"] + 2 * p5["topk"] * p5["d"])
    points.append(("topk_c2psa", lambda: oracle.topk_sparse(
        q5, k5, v5, p5["topk"]), fl5, "GFLOP/s",
        f"batches 0-{b5 - 1} of {p5['b']} ({b5 * p5['h']} of {p5['b'] * p5['h']} (b, h))"))

    def median3(fn):
        fn()  # warm-up
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    cores = len(os.sched_getaffinity(0))
    res = {}
    t_start = time.perf_counter()
    for threads in (cores, 1):
        key = "all_cores" if threads == cores else "one_thread"
        with threadpool_limits(limits=threads):
            for name, fn, num, unit, sample in points:
                sec = median3(fn)
                r = res.setdefault(name, {"unit": unit, "sample": sample,
                                          "numerator": num})
                r[key] = {"s": round(sec, 6), "rate": round(num / sec / 1e9, 4)}
    wall = time.perf_counter() - t_start
    # spot check of the GPU's ragged-batch output against the sampled oracle
    gpu_out = dec["out"].float().cpu().numpy().astype(np.float64)
    err = max(float(np.max(np.abs(o - gpu_out[b]))) for b, o in enumerate(outs3))
    head = res["decode_ragged_b64"]
    return dict(value=head["all_cores"]["rate"], unit="GB/s", cores=cores,
                kind="oracle",
                sample=(f"fp64 NumPy oracle on the ragged decode batch "
                        f"({head['sample']}, {head['numerator']} algorithmic "
                        "bytes); median of 3 after 1 warm-up"),
                one_thread=head["one_thread"]["rate"], cpu_model=cpu_model(),
                threads={"all_cores": cores, "one_thread": 1},
                points=res, wall_s=round(wall, 1),
                spot_check_max_abs_err=err)


# ----------------------------------------------------------------------------
# HBM traffic from committed counter summaries
# ----------------------------------------------------------------------------
def kernel_source_hash(names):
    """First 16 hex digits of the SHA-256 over the named csrc/ files, in
    order: the kernel and the host code that plans its launch."""
    h = hashlib.sha256()
    for name in names:
        path = os.path.join(ROOT, "transformer_attention_split_amd", "csrc", name)
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


# the decode kernels, their shared helpers, and the host side of the split plan
DECODE_SOURCES = ("decode.hip", "common.h", "launch.h", "api.cpp")


def committed_traffic(summary, sources):
    """Bytes per launch from a profiles/ summary, if it was taken on the
    current sources (the summary records their hash)."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("source_sha256_16") != kernel_source_hash(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        log(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): "
            "the attention path here has no multi-GPU component.")
        sys.exit(2)
    import numpy as np
    import torch

    import synth
    import transformer_attention_split_amd as tas

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log("building inputs ...")
    dec = make_decode(torch, synth, tas)
    pre = make_prefill(torch, synth)
    tk = make_topk(torch, synth)
    torch.cuda.synchronize()
    dp, pp = dec["p"], pre["p"]

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("calibration copy: 1 GiB device-to-device done")

    def step(ev=None):
        if ev:
            ev[0].record()
        tas.attn_decode(dec["q"], dec["k"], dec["v"], seq_lens=dec["seq_lens"],
                        scale=dp["scale"], out=dec["out"], workspace=dec["ws"])
        if ev:
            ev[1].record()
        tas.attn_prefill(pre["q"], pre["k"], pre["v"],
                         prefix_len=pp["prefix_len"], scale=pp["scale"],
                         out=pre["out"])
        if ev:
            ev[2].record()
        tas.attn_topk(tk["q"], tk["k"], tk["v"], tk["p"]["topk"],
                      out=tk["out"])
        if ev:
            ev[3].record()

    log(f"warmup {args.warmup} steps ...")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(args.steps)]
    log(f"timing {args.steps} steps ...")
    state_before = gpu_state(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    state_after = gpu_state(torch)
    t_dec = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps * 1e-3
    t_pre = sum(e[1].elapsed_time(e[2]) for e in evs) / args.steps * 1e-3
    t_tk = sum(e[2].elapsed_time(e[3]) for e in evs) / args.steps * 1e-3
    def back_to_back(fn, n=20):
        """Per-call time of n consecutive calls between two events (the
        launch gap after a different kernel is then paid once, not per call)."""
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    t_pre_b2b = back_to_back(lambda: tas.attn_prefill(
        pre["q"], pre["k"], pre["v"], prefix_len=pp["prefix_len"],
        scale=pp["scale"], out=pre["out"]))
    t_tk_b2b = back_to_back(lambda: tas.attn_topk(
        tk["q"], tk["k"], tk["v"], tk["p"]["topk"], out=tk["out"]))
    t_tkc_b2b = back_to_back(lambda: tas.attn_topk_causal(
        tk["q"], tk["k"], tk["v"], tk["p"]["topk"], out=tk["out"]))

    def pct(i):
        xs = np.array([e[i].elapsed_time(e[i + 1]) * 1e3 for e in evs])
        return {k: round(float(np.percentile(xs, q)), 2)
                for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}
    dec_pct, pre_pct, tk_pct = pct(0), pct(1), pct(2)
    dec_gbps = dec["bytes"] / t_dec / 1e9
    pre_tflops = pre["flops"] / t_pre / 1e12
    tk_tflops = tk["flops"] / t_tk / 1e12
    log(f"decode {t_dec * 1e6:.1f} us  {dec_gbps:.1f} GB/s | prefill "
        f"{t_pre * 1e6:.1f} us {pre_tflops:.1f} TFLOP/s | topk "
        f"{t_tk * 1e6:.1f} us {tk_tflops:.2f} TFLOP/s")

    secondary = {
        "prefill": dict(workload="prefill_prefix3072", us=round(t_pre * 1e6, 2),
                        TFLOPs=round(pre_tflops, 2),
                        frac_of_bf16_mfma_peak=round(
                            pre_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                        flops=pre["flops"], us_percentiles=pre_pct,
                        us_back_to_back=round(t_pre_b2b, 2),
                        TFLOPs_back_to_back=round(pre["flops"] / t_pre_b2b / 1e6, 2),
                        frac_back_to_back=round(pre["flops"] / t_pre_b2b / 1e6
                                                / BF16_MFMA_PEAK_TFLOPS, 4)),
        "topk": dict(workload="topk_c2psa", us=round(t_tk * 1e6, 2),
                     TFLOPs=round(tk_tflops, 3),
                     frac_of_fp64_peak=round(tk_tflops / FP64_PEAK_TFLOPS, 4),
                     flops=tk["flops"], us_percentiles=tk_pct,
                     us_back_to_back=round(t_tk_b2b, 2)),
        "topk_causal": dict(workload="topk_c2psa, decoder-causal form",
                            us_back_to_back=round(t_tkc_b2b, 2),
                            flops=tk["flops_causal"],
                            TFLOPs_back_to_back=round(
                                tk["flops_causal"] / t_tkc_b2b / 1e6, 3)),
    }
    if not args.no_secondary:
        log("fused append + decode on the ragged batch ...")
        secondary["decode_append_ragged_b64"] = bench_append(torch, tas, dec,
                                                             args.steps)
        log("fp32 decode on the ragged batch ...")
        secondary["decode_f32_ragged_b64"] = bench_decode_f32(torch, tas, dec,
                                                              args.steps)
        log("paged decode on the ragged batch ...")
        secondary["decode_paged_ragged_b64"] = [
            bench_paged(torch, tas, dec, args.steps, ps, lay)
            for lay in ("token", "head") for ps in (64, 256)]
        log("prefill at D=128 (16 heads; 32 over 8 kv heads) and with 32 heads ...")
        secondary["prefill_d128_prefix3072"] = bench_prefill_shape(
            torch, tas, synth, 128, 16)
        secondary["prefill_h32_prefix3072"] = bench_prefill_shape(
            torch, tas, synth, 64, 32)
        secondary["prefill_d128_gqa32x8_prefix3072"] = bench_prefill_shape(
            torch, tas, synth, 128, 32, Hkv=8)
        log("paged prefill ...")
        secondary["prefill_paged_prefix3072"] = [
            bench_prefill_paged(torch, tas, pre, ps, lay)
            for lay in ("token", "head") for ps in (64, 256)]
    if not args.no_secondary and not args.no_single:
        log("single-sequence position-8000 decode (graph replay) ...")
        secondary["decode_single_pos8000"] = bench_single_position(
            torch, tas, synth)

    log("streaming-read probe over 4 GiB ...")
    context = {"read_probe": bench_read_probe(torch, tas),
               "gpu_state_before": state_before,
               "gpu_state_after": state_after}

    traffic = committed_traffic("decode_ragged_b64_traffic.txt",
                                DECODE_SOURCES)
    roofline = {
        "kernel": "decode_bf16_kernel<128, 4, 0, true> + decode_combine_kernel<true, 128> (one attn_decode call)",
        "bound": "hbm", "achieved": round(dec_gbps, 1),
        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "algorithmic_bytes_per_launch": dec["bytes"],
        "avg_launch_us": round(t_dec * 1e6, 2),
        "launch_us_percentiles": dec_pct,
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(dec, synth)

    line = {
        "metric": METRIC,
        "value": round(dec_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "decode_ragged_b64",
            "B": dp["B"], "Hq": dp["Hq"], "Hkv": dp["Hkv"], "D": dp["D"],
            "max_length": dp["max_length"],
            "sum_valid_rows": int(dec["lens"].sum()),
            "step_also_runs": ["prefill_prefix3072", "topk_c2psa"],
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
        "context": context,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
