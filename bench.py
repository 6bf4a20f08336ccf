#!/usr/bin/env python3
"""Benchmark of the TurboQuant KV-cache hot path on one MI355X (gfx950).

A step is one decode step of the whole path on the decode workload (batch 32,
32 query / 8 KV heads, head_dim 128, 8192 cached tokens per sequence,
3-bit Lloyd-Max keys + 1-bit QJL, 4-bit group-32 values, paged through a
permuted block table): tq_quantize_store of the step's new token for every
sequence and KV head, then tq_decode_attention over the 8192 cached tokens.

Printed as ONE JSON line:
  value     = KV bytes the decode must read per step (every packed record byte
              of every cached token-head, 148 B each) / step time, in TB/s;
  roofline  = the split kernel (the streaming kernel) timed live with HIP
              events around its launch, against the 8 TB/s HBM peak;
  quantize  = tq_quantize_store throughput on the quantise workload (65536
              new bf16 tokens x 8 KV heads, 0.5% x20 outliers, K3V4 and K3V2);
  mse_only  = the same decode step with MSE-only keys (no QJL sketch, 130 B
              per token-head): step and split-kernel times, TB/s of its KV bytes;
  cpu_baseline = the fp64 CPU oracle on a bounded sample of the decode
              workload, on this host's cores.
The cache pool is rotated over several copies so that the 256 MB last-level
cache cannot serve repeated reads of one pool.
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


def setup_decode(torch, tq, synth, chunk, copies, mse_only=False):
    d, B, Hq, Hkv, L, kb, vb, nb, seed = 128, 32, 32, 8, 8192, 3, 4, 16384, 3
    signs1, signs2, S = synth.method_params(seed, d)
    import numpy as np
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([signs1, signs2]), S=S, mse_only=mse_only)
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


def decode_step(tq, s, i, events=None):
    pool = s["pools"][i % len(s["pools"])]
    tq.tq_quantize_store(s["ctx"], s["knew"], s["vnew"], s["slot_new"], pool)
    tq.tq_decode_attention(s["q"], [s["ctx"]], [pool], s["bt"], s["lens"], s["out"], s["ws"],
                           chunk_tokens=s["chunk"], max_seq_len=s["L"], split_events=events)


def time_decode(torch, tq, s, steps, warmup):
    """Average step time (store + decode) over `steps` steps, then the split
    kernel's average launch duration from HIP events on its stream."""
    for i in range(warmup):
        decode_step(tq, s, i)
    torch.cuda.synchronize()
    # timed region: K steps of the whole path (store + decode), nothing else
    # on the stream.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        decode_step(tq, s, i)
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    # the same K steps again with the split (streaming) kernel bracketed by
    # HIP events on its own stream each step, for its average launch duration
    # (kept out of the step timing: an event record between launches adds a
    # few microseconds of idle time to the step).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:  # create the underlying HIP events
        a.record()
        b.record()
    torch.cuda.synchronize()
    for i in range(steps):
        decode_step(tq, s, i, events=(evs[i][0].cuda_event, evs[i][1].cuda_event))
    torch.cuda.synchronize()
    split_ms = sorted(a.elapsed_time(b) for a, b in evs)
    return ms_step, sum(split_ms) / len(split_ms), split_ms


def bench_quantize(torch, tq, synth, steps, warmup):
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
        for i in range(warmup):
            tq.tq_quantize_store(ctx, ks[i % copies], vs[i % copies], slots, pool)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            tq.tq_quantize_store(ctx, ks[i % copies], vs[i % copies], slots, pool)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        hbm = T * Hkv * (2 * d * 2 + ctx.block_bytes // 16) + T * 4
        res[f"k{kb}v{vb}"] = {"ms": round(ms, 4), "mtok_per_s": round(T / ms / 1e3, 2),
                              "hbm_bytes": hbm, "hbm_tbs": round(hbm / ms / 1e9, 3),
                              "hbm_frac": round(hbm / ms / 1e9 / HBM_PEAK_TBS, 4)}
        ctx.close()
    return {"workload": "quantize-65536tok-hkv8-d128-bf16-outliers0.5%x20", **res}


def cpu_baseline(synth, seqs=24):
    """The oracle on a bounded sample of the decode workload: cache encoded
    by the oracle (not timed), then its decode of `seqs` sequences timed."""
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
    for b in range(seqs):
        for h in range(Hkv):
            K, V = synth.seq_kv(seed, b, h, L, d)
            ke = keys.encode_keys(K.astype(np.float64), prm["d1"], prm["d2"], S, c32, t32)
            ve = values.encode_values(V, vb)
            tt = np.arange(L)
            paged.write_tokens(pool, bt[b][tt // 16].astype(np.int64) * 16 + tt % 16, h, ke, ve, lay)
    q = synth.queries(seed, seqs, Hq, d)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        for b in range(seqs):
            fields = [paged.read_tokens(pool, bt[b], L, h, lay) for h in range(Hkv)]
            attention.decode_one_sequence(q[b].astype(np.float64), fields, prm)
        dt = time.perf_counter() - t0
    kv = seqs * Hkv * L * REC_BYTES_K3V4
    return {"value": kv / dt / 1e12, "unit": "TB/s", "cores": cores, "kind": "oracle",
            "sample": f"{seqs} of the 32 sequences of the decode workload (all 8 KV heads x 8192 tokens, "
                      f"32 query heads), oracle decode from an oracle-written pool: {dt:.2f} s, "
                      f"{seqs / dt:.3f} sequences/s; BLAS threads = cores, numpy elementwise work single-threaded"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--chunk", type=int, default=8192, help="tokens per decode split (fixed grid)")
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
    print(f"[bench] device {torch.cuda.get_device_name(0)}; building the decode cache", file=sys.stderr, flush=True)
    s = setup_decode(torch, tq, synth, args.chunk, copies=3)
    ms_step, split_avg, split_ms = time_decode(torch, tq, s, args.steps, args.warmup)
    value = s["kv_bytes"] / (ms_step * 1e-3) / 1e12
    achieved = s["kv_bytes"] / (split_avg * 1e-3) / 1e9
    print(f"[bench] decode step {ms_step * 1e3:.1f} us, split kernel avg {split_avg * 1e3:.1f} us "
          f"(median {split_ms[len(split_ms) // 2] * 1e3:.1f})", file=sys.stderr, flush=True)
    for p in s["pools"]:
        del p
    s.clear()
    torch.cuda.empty_cache()

    # the same workload with MSE-only keys (no QJL sketch: 130 B per token-head)
    print("[bench] decode workload, MSE-only keys", file=sys.stderr, flush=True)
    s = setup_decode(torch, tq, synth, args.chunk, copies=3, mse_only=True)
    m_step, m_split, _ = time_decode(torch, tq, s, args.steps, args.warmup)
    mse = {"workload": "decode-b32-hq32-hkv8-d128-ctx8192-k3v4-mse-only: store 1 new token + attend 8192",
           "kv_bytes_per_step": s["kv_bytes"], "ms_per_step": round(m_step, 5),
           "tbs": round(s["kv_bytes"] / (m_step * 1e-3) / 1e12, 4),
           "split_avg_ms": round(m_split, 5),
           "split_hbm_frac": round(s["kv_bytes"] / (m_split * 1e-3) / 1e12 / HBM_PEAK_TBS, 4),
           "decode_tokens_per_s": round(32 / (m_step * 1e-3), 1)}
    print(f"[bench] MSE-only decode step {m_step * 1e3:.1f} us, split kernel avg {m_split * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    for p in s["pools"]:
        del p
    s.clear()
    torch.cuda.empty_cache()

    print("[bench] quantise workload", file=sys.stderr, flush=True)
    qres = bench_quantize(torch, tq, synth, steps=max(5, args.steps // 5), warmup=3)
    print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
    cpu = cpu_baseline(synth)

    traffic = _traffic_record(None)
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
        "kv_bytes_per_step": 32 * 8 * 8192 * REC_BYTES_K3V4,
        "quantize": qres,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_TBS * 1000, "unit": "GB/s",
                     "frac": round(achieved / (HBM_PEAK_TBS * 1000), 4), "traffic": traffic,
                     "kernel": "decode_split_kernel<128,4,3,4,true>", "bytes_per_launch": 32 * 8 * 8192 * REC_BYTES_K3V4,
                     "avg_launch_ms": round(split_avg, 5)},
        "mse_only": mse,
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
