#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache hot path on one MI355X (gfx950).

A step is one decode step of the whole path on the decode workload (batch 32,
32 query / 8 KV heads, head_dim 128, 8192 cached tokens per sequence,
3-bit Lloyd-Max keys + 1-bit QJL, 4-bit group-32 values, paged through a
permuted block table): tq_quantize_store of the step's new token for every
sequence and KV head, then tq_decode_attention over the 8192 cached tokens,
launched eagerly (the same step replayed from a HIP graph is reported beside
it).

Printed as ONE JSON line:
  value     = KV bytes the decode must read per step (every packed record byte
              of every cached token-head, 148 B each) / mean step time over
              the K timed steps, in TB/s;
  roofline  = the split kernel (the streaming kernel): median time of one
              launch over back-to-back split-only launches, against the
              8 TB/s HBM peak;
  workloads = the other workloads timed the same way (median of launches):
              the long-context d=256 decode, the ragged mixed-preset decode
              with a bf16 window, the quantise workload (65536 new bf16
              tokens x 8 KV heads, K3V4 and K3V2), MSE-only keys, and a
              check that repeated decode calls are bit-identical;
  cpu_baseline = the fp64 CPU oracle on bounded samples of the decode and
              quantise workloads, on this host's cores.
Caches smaller than a few times the 256 MB last-level cache are rotated over
several copies so that repeated launches cannot be served from it.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TQ decode attn: KV-bytes TB/s (% HBM peak) + tokens/s; quantize Mtok/s"
HBM_PEAK_TBS = 8.0
REC_BYTES_K3V4 = 148  # per token-head: 48 code + 16 sign + 4 meta + 64 value + 16 value-meta bytes


def _kernel_source_sha():
    h = hashlib.sha256()
    for name in ("csrc/tq_decode.hip", "csrc/tq_common.hip.h", "build.py"):
        with open(os.path.join(ROOT, "kv_cache_vector_03_amd", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_record(per_launch_units):
    """HBM bytes per split launch from the committed PMC summary, if it was
    taken on the current decode source and build flags; else None."""
    path = os.path.join(ROOT, "profiles", "decode_split_b32_ctx8192_k3v4_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != _kernel_source_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------- graphs --
def capture(torch, fn):
    """Run ``fn`` once on a side stream (torch's warm-up recipe), then capture
    it into a HIP graph on torch's capture stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_total(torch, graphs, reps):
    """Mean ms per replay over ``reps`` back-to-back replays (graphs taken
    round-robin), bracketed by synchronisations and two events."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# --------------------------------------------------------- decode workload --
def setup_decode(torch, tq, synth, chunk, copies, mse_only=False, kb=3, vb=4, uniform=False):
    d, B, Hq, Hkv, L, nb, seed = 128, 32, 32, 8, 8192, 16384, 3
    signs1, signs2, S = synth.method_params(seed, d)
    import numpy as np
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([signs1, signs2]), S=S, mse_only=mse_only, uniform=uniform)
    bt_np = synth.block_table(seed, B, L // 16, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pools = [torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda") for _ in range(copies)]
    t = torch.arange(L, device="cuda")
    for b in range(B):
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        k = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b)
        v = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b + 1)
        for p in pools:
            tq.tq_quantize_store(ctx, k, v, slots, p)
    torch.cuda.synchronize()
    # the step's new token: position L-1 of every sequence (rewritten each step)
    knew = synth.torch_normal_bf16((B, Hkv, d), seed * 7 + 1)
    vnew = synth.torch_normal_bf16((B, Hkv, d), seed * 7 + 2)
    slot_new = (bt[:, (L - 1) // 16].long() * 16 + (L - 1) % 16).to(torch.int32).contiguous()
    q = synth.torch_normal_bf16((B, Hq, d), seed * 7 + 3)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    nbytes = tq.tq_decode_workspace_bytes(q, [ctx], [pools[0]], bt, lens, out, chunk_tokens=chunk, max_seq_len=L)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    return dict(ctx=ctx, bt=bt, pools=pools, knew=knew, vnew=vnew, slot_new=slot_new, q=q, lens=lens, out=out, ws=ws,
                B=B, Hq=Hq, Hkv=Hkv, d=d, L=L, chunk=chunk, kv_bytes=B * Hkv * L * (ctx.block_bytes // 16),
                units=B * Hkv * L)


def _prepared(tq, s):
    """Prepared (validated-once) store and decode calls per pool copy: the
    timed loop's host cost per launch is one ctypes call, so the launches
    queue up ahead of the GPU."""
    if "prep" not in s:
        s["prep"] = [tq.PreparedDecode(s["q"], [s["ctx"]], [p], s["bt"], s["lens"], s["out"], s["ws"],
                                       chunk_tokens=s["chunk"], max_seq_len=s["L"]) for p in s["pools"]]
        s["prep_store"] = [tq.PreparedQuantize(s["ctx"], s["knew"], s["vnew"], s["slot_new"], p) for p in s["pools"]]
    return s


def decode_only(tq, s, i):
    _prepared(tq, s)["prep"][i % len(s["pools"])]()


def decode_step(tq, s, i):
    _prepared(tq, s)["prep_store"][i % len(s["pools"])]()
    decode_only(tq, s, i)


def decode_step_current_stream(tq, s, i):
    """The same step through the plain calls, which launch on torch's current
    stream (the form a HIP graph capture records)."""
    pool = s["pools"][i % len(s["pools"])]
    tq.tq_quantize_store(s["ctx"], s["knew"], s["vnew"], s["slot_new"], pool)
    tq.tq_decode_attention(s["q"], [s["ctx"]], [pool], s["bt"], s["lens"], s["out"], s["ws"],
                           chunk_tokens=s["chunk"], max_seq_len=s["L"])


def spin_up(torch, fn, seconds=0.25, batch=50):
    """Untimed launches of ``fn`` for at least ``seconds`` of wall time.  The
    GPU's clocks ramp up under load: after set-up or a pause of a second or
    two, the first ~150-300 decode launches run 15-25 % slower than the
    steady state (measured on the split kernel), which a warm-up of a few
    steps does not cover."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(batch):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def time_eager(torch, fn, reps):
    """Eager launches of ``fn`` (one step each): the mean over ``reps``
    back-to-back steps between two events and two synchronisations, then the
    median of a second pass with an event between consecutive steps (the
    host enqueues ahead of the GPU, so an event marks where one step's
    kernels end and the next one's begin)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / reps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(reps):
        fn(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    each = [evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]
    return mean, each


def time_decode(torch, tq, s, steps, warmup):
    """The step (store + decode, eager launches): mean over exactly ``steps``
    steps and the median step; the same step replayed from HIP graphs for
    comparison; the split kernel's median launch time from back-to-back
    decode-only launches."""
    spin_up(torch, lambda i: decode_step(tq, s, i))
    for i in range(warmup):
        decode_step(tq, s, i)
    torch.cuda.synchronize()
    # the timed region: exactly `steps` steps between two synchronisations
    ms_step, each = time_eager(torch, lambda i: decode_step(tq, s, i), steps)
    n = len(s["pools"])
    step_graphs = [capture(torch, (lambda j: (lambda: decode_step_current_stream(tq, s, j)))(j)) for j in range(n)]
    spin_up(torch, lambda i: step_graphs[i % n].replay(), seconds=0.05)
    graph_ms = time_total(torch, step_graphs, steps)
    del step_graphs
    spin_up(torch, lambda i: decode_only(tq, s, i), seconds=0.1)
    for i in range(warmup):
        decode_only(tq, s, i)
    split_mean, split_each = time_eager(torch, lambda i: decode_only(tq, s, i), steps)
    return {"ms_per_step": ms_step, "median_ms_per_step": _median(each), "graph_ms_per_step": graph_ms,
            "split_mean_ms": split_mean, "split_median_ms": _median(split_each), "split_min_ms": min(split_each),
            "split_max_ms": max(split_each)}


def repeat_bit_identical(torch, tq, s):
    """Two decode calls on the same inputs give bit-identical outputs (every
    wave takes its steps in a fixed order)."""
    outs = []
    for i in range(2):
        decode_only(tq, s, 0)
        torch.cuda.synchronize()
        outs.append(s["out"].clone())
    return bool(torch.equal(outs[0], outs[1]))


# ----------------------------------------------------- long / ragged decode --
def setup_long(torch, tq, synth):
    """B=8, Hq=16, Hkv=4, d=256, 131072 cached tokens, K4V4 (one 1.36 GB pool
    copy: five times the last-level cache)."""
    import numpy as np
    d, B, Hq, Hkv, L, kb, vb, nb, seed = 256, 8, 16, 4, 131072, 4, 4, 65536, 4
    s1, s2, S = synth.method_params(seed, d)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([s1, s2]), S=S)
    bt = torch.from_numpy(synth.block_table(seed, B, L // 16, nb)).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    t = torch.arange(L, device="cuda")
    for b in range(B):
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        k = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b)
        v = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b + 1)
        tq.tq_quantize_store(ctx, k, v, slots, pool)
        del k, v
    q = synth.torch_normal_bf16((B, Hq, d), seed * 7 + 3)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    kw = dict(chunk_tokens=8192, max_seq_len=L)
    ws = torch.empty(tq.tq_decode_workspace_bytes(q, [ctx], [pool], bt, lens, out, **kw), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    fn = tq.PreparedDecode(q, [ctx], [pool], bt, lens, out, ws, **kw)
    return dict(keep=[ctx, bt, pool, q, lens, out, ws], fn=fn, B=B,
                kv_bytes=B * Hkv * L * (ctx.block_bytes // 16),
                workload="decode-b8-hq16-hkv4-d256-ctx131072-k4v4", chunk_tokens=8192)


def setup_ragged(torch, tq, synth):
    """B=64, Hq=32, Hkv=8, d=128, lognormal lengths in [1024, 131072]; the last
    128 tokens of each sequence as a bf16 window, the rest quantised K3V2
    (even sequences) or K4V4 (odd); N(0,1) with 0.5% x20 outliers."""
    import numpy as np
    d, B, Hq, Hkv, W, seed = 128, 64, 32, 8, 128, 5
    presets = [(3, 2), (4, 4)]
    total = synth.ragged_lengths(seed, B)
    cached = np.maximum(total - W, 0)
    rlens = np.minimum(total, W)
    seq_preset = (np.arange(B) % 2).astype(np.int8)
    ctxs = []
    for i, (kb, vb) in enumerate(presets):
        s1, s2, S = synth.method_params(seed + 10 * i, d)
        ctxs.append(tq.tq_codebook_init(d, kb, vb, signs=np.stack([s1, s2]), S=S))
    mb = int(np.ceil(cached.max() / 16))
    bt_np = np.zeros((B, mb), dtype=np.int32)
    pools = []
    for pr in range(2):
        seqs = [b for b in range(B) if seq_preset[b] == pr]
        need = [int(np.ceil(cached[b] / 16)) for b in seqs]
        nbp = sum(need) + 1
        perm = np.random.default_rng([seed, pr, 0xB10C]).permutation(nbp).astype(np.int32)
        off = 0
        for b, n in zip(seqs, need):
            bt_np[b, :n] = perm[off:off + n]
            off += n
        pools.append(torch.zeros((nbp, Hkv, ctxs[pr].block_bytes), dtype=torch.uint8, device="cuda"))
    bt = torch.from_numpy(bt_np).cuda()
    for b in range(B):
        L = int(cached[b])
        t = torch.arange(L, device="cuda")
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        k = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b, p=0.005)
        v = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b + 1, p=0.005)
        tq.tq_quantize_store(ctxs[seq_preset[b]], k, v, slots, pools[seq_preset[b]])
        del k, v
    rk = synth.torch_normal_bf16((B, Hkv, W, d), seed * 7 + 5, p=0.005)
    rv = synth.torch_normal_bf16((B, Hkv, W, d), seed * 7 + 6, p=0.005)
    q = synth.torch_normal_bf16((B, Hq, d), seed * 7 + 3)
    lens = torch.from_numpy(cached.astype(np.int32)).cuda()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    kw = dict(seq_preset=torch.from_numpy(seq_preset).cuda(), recent_k=rk, recent_v=rv,
              recent_lens=torch.from_numpy(rlens.astype(np.int32)).cuda(), chunk_tokens=8192, max_seq_len=mb * 16)
    ws = torch.empty(tq.tq_decode_workspace_bytes(q, ctxs, pools, bt, lens, out, **kw), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    fn = tq.PreparedDecode(q, ctxs, pools, bt, lens, out, ws, **kw)
    rec = [ctxs[p].block_bytes // 16 for p in range(2)]
    kv = int(sum(Hkv * (int(cached[b]) * rec[seq_preset[b]] + int(rlens[b]) * 2 * d * 2) for b in range(B)))
    return dict(keep=[ctxs, bt, pools, rk, rv, q, lens, out, ws, kw], fn=fn, B=B, kv_bytes=kv,
                workload="decode-ragged-b64-hq32-hkv8-d128-k3v2|k4v4-recent128", chunk_tokens=8192,
                mean_len=float(total.mean()))


def time_workload(torch, w, reps):
    spin_up(torch, lambda i: w["fn"](), batch=10)
    _, each = time_eager(torch, lambda i: w["fn"](), reps)
    ms = _median(each)
    tbs = w["kv_bytes"] / (ms * 1e-3) / 1e12
    res = {"workload": w["workload"], "kv_bytes_per_call": w["kv_bytes"], "median_ms": round(ms, 5),
           "tbs": round(tbs, 4), "hbm_frac": round(tbs / HBM_PEAK_TBS, 4),
           "decode_tokens_per_s": round(w["B"] / (ms * 1e-3), 1), "chunk_tokens": w["chunk_tokens"]}
    if "mean_len" in w:
        res["mean_tokens_per_seq"] = round(w["mean_len"], 1)
    return res


# ---------------------------------------------------------- prefill workload --
EXTEND_FLOPS_PER_PREFIX = 6 * 128  # per (query row, prefix token): q~.c, p.sign and the value product, 2 flops per MAC
EXTEND_FLOPS_PER_CHUNK = 4 * 128   # per (query row, visible chunk token): q.k and the value product


def setup_prefill(torch, tq, synth):
    """B=4, Hq=32, Hkv=8, d=128: an 8192-token K3V4 prefix per sequence in the
    paged pool and a 512-token bf16 chunk per sequence (0.5% x20 outliers).
    A step stores the chunk compressed (tq_quantize_store into positions
    8192..8703) and runs the extend attention of its 512 x 32 query rows."""
    import numpy as np
    d, B, Hq, Hkv, P, C, kb, vb, seed = 128, 4, 32, 8, 8192, 512, 3, 4, 6
    s1, s2, S = synth.method_params(seed, d)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([s1, s2]), S=S)
    mb = (P + C) // 16
    bt = torch.from_numpy(synth.block_table(seed, B, mb, B * mb)).cuda()
    pool = torch.zeros((B * mb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    t = torch.arange(P, device="cuda")
    for b in range(B):
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        k = synth.torch_normal_bf16((P, Hkv, d), seed * 1000003 + 2 * b, p=0.005)
        v = synth.torch_normal_bf16((P, Hkv, d), seed * 1000003 + 2 * b + 1, p=0.005)
        tq.tq_quantize_store(ctx, k, v, slots, pool)
    q = synth.torch_normal_bf16((B * C, Hq, d), seed * 7 + 1)
    kc = synth.torch_normal_bf16((B * C, Hkv, d), seed * 7 + 2, p=0.005)
    vc = synth.torch_normal_bf16((B * C, Hkv, d), seed * 7 + 3, p=0.005)
    tc = torch.arange(P, P + C, device="cuda")
    slot_chunk = torch.cat([(bt[b][tc // 16].long() * 16 + tc % 16) for b in range(B)]).to(torch.int32).contiguous()
    cu = (torch.arange(B + 1, dtype=torch.int32, device="cuda") * C).contiguous()
    plen = torch.full((B,), P, dtype=torch.int32, device="cuda")
    out = torch.empty((B * C, Hq, d), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    store = tq.PreparedQuantize(ctx, kc, vc, slot_chunk, pool)
    ext = tq.PreparedExtend(q, kc, vc, cu, ctx, pool, bt, plen, out, max_chunk=C, max_prefix_len=P)
    rows = B * C * Hq
    flops = rows * P * EXTEND_FLOPS_PER_PREFIX + B * Hq * (C * (C + 1) // 2) * EXTEND_FLOPS_PER_CHUNK
    return dict(keep=[ctx, bt, pool, q, kc, vc, slot_chunk, cu, plen, out], store=store, ext=ext, B=B, C=C,
                flops=flops)


def time_prefill(torch, w, reps):
    spin_up(torch, lambda i: (w["store"](), w["ext"]()), batch=10)
    _, each = time_eager(torch, lambda i: w["ext"](), reps)
    ext_ms = _median(each)
    _, each = time_eager(torch, lambda i: (w["store"](), w["ext"]()), reps)
    step_ms = _median(each)
    tflops = w["flops"] / (ext_ms * 1e-3) / 1e12
    return {"workload": "prefill-b4-hq32-hkv8-d128-prefix8192-chunk512-k3v4: store the chunk + extend attention",
            "chunk_tokens_per_step": w["B"] * w["C"], "median_ms_per_step": round(step_ms, 5),
            "prefill_tokens_per_s": round(w["B"] * w["C"] / (step_ms * 1e-3), 1),
            "extend_median_ms": round(ext_ms, 5), "extend_algorithmic_flops": w["flops"],
            "extend_tflops": round(tflops, 2), "mfma_peak_tflops": 2500.0,
            "extend_mfma_frac": round(tflops / 2500.0, 4)}


# ------------------------------------------------------- quantise workload --
def bench_quantize(torch, tq, synth, reps):
    import numpy as np
    d, T, Hkv, nb, seed = 128, 65536, 8, 4096, 2
    signs1, signs2, S = synth.method_params(seed, d)
    bt_np = synth.block_table(seed, 1, nb, nb)[0]
    t = np.arange(T)
    slots = torch.from_numpy((bt_np[t // 16].astype(np.int64) * 16 + t % 16).astype(np.int32)).cuda()
    res = {}
    copies = 2
    ks = [synth.torch_normal_bf16((T, Hkv, d), 200 + c, p=0.005) for c in range(copies)]
    vs = [synth.torch_normal_bf16((T, Hkv, d), 300 + c, p=0.005) for c in range(copies)]
    for kb, vb in ((3, 4), (3, 2)):
        ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([signs1, signs2]), S=S)
        pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
        prep = [tq.PreparedQuantize(ctx, ks[c], vs[c], slots, pool) for c in range(copies)]
        fn = lambda i: prep[i % copies]()  # noqa: E731
        spin_up(torch, fn, batch=20)
        # the kernel's average launch duration: back-to-back launches between
        # two events (as the kernel trace measures it); the median of
        # per-launch event intervals, which carry the events' own packets,
        # beside it
        mean, each = time_eager(torch, fn, reps)
        hbm = T * Hkv * (2 * d * 2 + ctx.block_bytes // 16) + T * 4
        res[f"k{kb}v{vb}"] = {"mean_ms": round(mean, 5), "median_event_interval_ms": round(_median(each), 5),
                              "mtok_per_s": round(T / mean / 1e3, 2),
                              "hbm_bytes": hbm, "hbm_tbs": round(hbm / mean / 1e9, 3),
                              "hbm_frac": round(hbm / mean / 1e9 / HBM_PEAK_TBS, 4)}
        ctx.close()
    return {"workload": "quantize-65536tok-hkv8-d128-bf16-outliers0.5%x20", **res}


# --------------------------------------------------------------- oracle --
def cpu_baseline(synth, seqs=32, quant_tokens=16384):
    """The oracle on bounded samples: its decode of ``seqs`` sequences of the
    decode workload (cache encoded by the oracle first, not timed), and its
    encoding of ``quant_tokens`` tokens x 8 KV heads of the quantise workload."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attention, codebook, keys, paged, values

    cores = len(os.sched_getaffinity(0))
    d, Hq, Hkv, L, kb, vb, seed = 128, 32, 8, 8192, 3, 4, 3
    signs1, signs2, S = synth.method_params(seed, d)
    c32, t32 = codebook.tables_fp32(d, kb)
    prm = {"d1": signs1.astype(np.float64), "d2": signs2.astype(np.float64), "S": S, "c32": c32}
    lay = paged.layout(d, kb, vb)
    bt = synth.block_table(seed, seqs, L // 16, seqs * L // 16)
    pool = paged.new_pool(seqs * L // 16, Hkv, lay)

    def encode(i):  # untimed set-up: the oracle writes the cache (disjoint records per (b, h))
        b, h = divmod(i, Hkv)
        K, V = synth.seq_kv(seed, b, h, L, d)
        ke = keys.encode_keys(K.astype(np.float64), prm["d1"], prm["d2"], S, c32, t32)
        ve = values.encode_values(V, vb)
        tt = np.arange(L)
        paged.write_tokens(pool, bt[b][tt // 16].astype(np.int64) * 16 + tt % 16, h, ke, ve, lay)

    from concurrent.futures import ThreadPoolExecutor
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=min(16, cores)) as ex:
        list(ex.map(encode, range(seqs * Hkv)))
    q = synth.queries(seed, seqs, Hq, d)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for b in range(seqs):
            fields = [paged.read_tokens(pool, bt[b], L, h, lay) for h in range(Hkv)]
            attention.decode_one_sequence(q[b].astype(np.float64), fields, prm)
        dt = time.perf_counter() - t0
        # quantise: encode + pack + scatter of quant_tokens x 8 heads (K3V4)
        qs1, qs2, qS = synth.method_params(2, d)
        rng = np.random.default_rng([2, 0xC0])
        Kq = synth.normal_with_outliers(rng, (quant_tokens, Hkv, d))
        Vq = synth.normal_with_outliers(rng, (quant_tokens, Hkv, d))
        qpool = paged.new_pool(quant_tokens // 16, Hkv, lay)
        t1 = time.perf_counter()
        for h in range(Hkv):
            ke = keys.encode_keys(Kq[:, h].astype(np.float64), qs1.astype(np.float64), qs2.astype(np.float64), qS,
                                  c32, t32)
            ve = values.encode_values(Vq[:, h], vb)
            paged.write_tokens(qpool, np.arange(quant_tokens), h, ke, ve, lay)
        dq = time.perf_counter() - t1
    kv = seqs * Hkv * L * REC_BYTES_K3V4
    return {"value": kv / dt / 1e12, "unit": "TB/s", "cores": cores, "kind": "oracle",
            "sample": f"{seqs} of the 32 sequences of the decode workload (all 8 KV heads x 8192 tokens, "
                      f"32 query heads; the oracle reads the records back from an oracle-written pool and "
                      f"decodes them, one sequence at a time): {dt:.2f} s, "
                      f"{seqs / dt:.3f} sequences/s; BLAS threads = cores, numpy elementwise work single-threaded",
            "decode_tokens_per_s": seqs / dt,
            "quantize": {"mtok_per_s": quant_tokens / dq / 1e6, "seconds": dq,
                         "sample": f"{quant_tokens} tokens x 8 KV heads of the quantise workload's shape "
                                   f"(K3 + QJL, V4, bf16 N(0,1) with 0.5% x20 outliers), oracle encode + pack "
                                   f"+ paged write"}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--chunk", type=int, default=8192, help="tokens per decode split (fixed grid)")
    ap.add_argument("--skip-cpu", action="store_true", help="leave out the CPU oracle baseline")
    ap.add_argument("--decode-only", action="store_true",
                    help="time the decode workload alone (for profiler runs of the split kernel)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="finish with three 256 MiB device-to-device copies (the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by KV head or "
              f"sequence with no cross-GPU step in this build", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_vector_03_amd as tq
    import synth

    tq.load()
    torch.cuda.init()
    log(f"device {torch.cuda.get_device_name(0)}; building the decode cache")
    s = setup_decode(torch, tq, synth, args.chunk, copies=3)
    dec = time_decode(torch, tq, s, args.steps, args.warmup)
    ms_step = dec["ms_per_step"]
    value = s["kv_bytes"] / (ms_step * 1e-3) / 1e12
    # the kernel's average launch duration: back-to-back split-only launches
    # between two events (no events between the launches, whose own packets
    # add a few microseconds to each interval: the kernel trace's average
    # duration agrees with this figure)
    split_ms = dec["split_mean_ms"]
    achieved = s["kv_bytes"] / (split_ms * 1e-3) / 1e9
    log(f"decode step {ms_step * 1e3:.1f} us (median {dec['median_ms_per_step'] * 1e3:.1f}, graph replay "
        f"{dec['graph_ms_per_step'] * 1e3:.1f}), split kernel mean {split_ms * 1e3:.1f} us "
        f"(median of event intervals {dec['split_median_ms'] * 1e3:.1f})")
    det_equal = repeat_bit_identical(torch, tq, s)
    log(f"repeated decode calls bit-identical: {det_equal}")
    for p in s["pools"]:
        del p
    s.clear()
    torch.cuda.empty_cache()

    workloads = {"determinism": {"bit_identical_repeat": det_equal,
                                 "schedule": "every wave takes its 32-token steps in a fixed order in every call"}}
    if not args.decode_only:
        log("decode workload, MSE-only keys")
        s = setup_decode(torch, tq, synth, args.chunk, copies=3, mse_only=True)
        m = time_decode(torch, tq, s, max(20, args.steps // 2), 3)
        workloads["mse_only"] = {
            "workload": "decode-b32-hq32-hkv8-d128-ctx8192-k3v4-mse-only: store 1 new token + attend 8192",
            "kv_bytes_per_step": s["kv_bytes"], "ms_per_step": round(m["ms_per_step"], 5),
            "tbs": round(s["kv_bytes"] / (m["ms_per_step"] * 1e-3) / 1e12, 4),
            "split_mean_ms": round(m["split_mean_ms"], 5), "split_median_ms": round(m["split_median_ms"], 5),
            "split_hbm_frac": round(s["kv_bytes"] / (m["split_mean_ms"] * 1e-3) / 1e12 / HBM_PEAK_TBS, 4)}
        log(f"MSE-only step {m['ms_per_step'] * 1e3:.1f} us, split median {m['split_median_ms'] * 1e3:.1f} us")
        s.clear()
        torch.cuda.empty_cache()
        # the same decode workload at K4V4 with the Lloyd-Max codebook (scores
        # through the LDS pair table) and with the equally spaced one (scores
        # from the codes arithmetically)
        cmp = {}
        for name, uni in (("lloyd_max", False), ("uniform", True)):
            s = setup_decode(torch, tq, synth, args.chunk, copies=3, kb=4, vb=4, uniform=uni)
            m = time_decode(torch, tq, s, max(20, args.steps // 2), 3)
            cmp[name] = {"split_median_ms": round(m["split_median_ms"], 5),
                         "tbs": round(s["kv_bytes"] / (m["split_median_ms"] * 1e-3) / 1e12, 4)}
            cmp["kv_bytes_per_call"] = s["kv_bytes"]
            s.clear()
            torch.cuda.empty_cache()
        cmp["workload"] = "decode-b32-hq32-hkv8-d128-ctx8192-k4v4, Lloyd-Max (pair table) vs uniform (arithmetic)"
        # 8-bit MSE-only keys (K8V4): one-code table lookups, 210 B per token-head
        s = setup_decode(torch, tq, synth, args.chunk, copies=3, kb=8, vb=4, mse_only=True)
        m = time_decode(torch, tq, s, max(20, args.steps // 2), 3)
        workloads["k8v4_mse_only"] = {
            "workload": "decode-b32-hq32-hkv8-d128-ctx8192-k8v4-mse-only: store 1 new token + attend 8192",
            "kv_bytes_per_step": s["kv_bytes"], "ms_per_step": round(m["ms_per_step"], 5),
            "split_mean_ms": round(m["split_mean_ms"], 5),
            "split_hbm_frac": round(s["kv_bytes"] / (m["split_mean_ms"] * 1e-3) / 1e12 / HBM_PEAK_TBS, 4)}
        log(f"K8V4 MSE-only step {m['ms_per_step'] * 1e3:.1f} us, split mean {m['split_mean_ms'] * 1e3:.1f} us")
        s.clear()
        torch.cuda.empty_cache()
        cmp["uniform_speedup"] = round(cmp["lloyd_max"]["split_median_ms"] / cmp["uniform"]["split_median_ms"], 4)
        workloads["codebook_k4v4"] = cmp
        log(f"K4V4 split median: Lloyd-Max {cmp['lloyd_max']['split_median_ms'] * 1e3:.1f} us, "
            f"uniform {cmp['uniform']['split_median_ms'] * 1e3:.1f} us")
        for name, setup in (("long_d256", setup_long), ("ragged_hybrid", setup_ragged)):
            log(f"workload {name}")
            w = setup(torch, tq, synth)
            workloads[name] = time_workload(torch, w, max(20, args.steps // 2))
            log(f"{name}: {workloads[name]['median_ms'] * 1e3:.1f} us, {workloads[name]['tbs']:.3f} TB/s")
            w.clear()
            torch.cuda.empty_cache()
        log("prefill workload (extend attention)")
        w = setup_prefill(torch, tq, synth)
        workloads["prefill_extend"] = time_prefill(torch, w, max(10, args.steps // 5))
        log(f"prefill: extend {workloads['prefill_extend']['extend_median_ms'] * 1e3:.1f} us, "
            f"{workloads['prefill_extend']['extend_tflops']:.1f} TFLOP/s")
        w.clear()
        torch.cuda.empty_cache()
        log("quantise workload")
        workloads["quantize"] = bench_quantize(torch, tq, synth, reps=max(20, args.steps // 2))
        log(f"quantise K3V4 {workloads['quantize']['k3v4']['mean_ms'] * 1e3:.1f} us mean over back-to-back launches "
            f"({workloads['quantize']['k3v4']['median_event_interval_ms'] * 1e3:.1f} us median of event intervals)")
    cpu = None
    if not args.skip_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(synth)

    traffic = _traffic_record(None)
    kv_bytes = 32 * 8 * 8192 * REC_BYTES_K3V4
    line = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32acc-bf16x2",
        "data": "synthetic",
        "config": {"workload": "decode-b32-hq32-hkv8-d128-ctx8192-k3v4: store 1 new token + attend 8192",
                   "batch": 32, "q_heads": 32, "kv_heads": 8, "head_dim": 128, "context": 8192,
                   "k_bits": 3, "v_bits": 4, "chunk_tokens": args.chunk, "pool_copies": 3},
        "hbm_frac": round(value / HBM_PEAK_TBS, 4),
        "decode_tokens_per_s": round(32 / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "median_ms_per_step": round(dec["median_ms_per_step"], 5),
        "graph_replay_ms_per_step": round(dec["graph_ms_per_step"], 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_TBS * 1000, "unit": "GB/s",
                     "frac": round(achieved / (HBM_PEAK_TBS * 1000), 4), "traffic": traffic,
                     "kernel": "decode_split_kernel<128,4,3,4,true,false>", "bytes_per_launch": kv_bytes,
                     "mean_launch_ms": round(split_ms, 5),
                     "median_event_interval_ms": round(dec["split_median_ms"], 5),
                     "min_event_interval_ms": round(dec["split_min_ms"], 5),
                     "timing": "mean launch duration over K back-to-back eager split-only launches (3 pool "
                               "copies in turn) between two events; the per-launch event intervals of a "
                               "second pass (events between the library calls) are reported beside it",
                     "consistent_with_step": bool(split_ms <= ms_step and achieved >= kv_bytes / (ms_step * 1e-3) / 1e9)},
        "workloads": workloads,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_calibration:
        x = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
