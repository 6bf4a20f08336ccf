"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark uses (chunk_tokens = 8192), on every output.

The whole cache is written by tq_quantize_store from seeded inputs generated
on the device.  The decode reads that pool; the oracle reads the same pool
back (``paged.read_tokens`` on a host copy) and runs its fp64 attention for
every (sequence, KV head) pair, so both sides decode the same GPU-written
records.  Every pair's outputs (within 1e-3 relative per row) and every score
(within 1e-3 of max(|ref|, rms(ref row))) are compared, including the recent
bf16 window's.  The pairs run on a host thread pool with one BLAS thread each.

Workloads:
  * decode: B=32, Hq=32, Hkv=8, d=128, 8192 cached tokens, K3V4, a
    16384-block pool through a permuted block table (QJL and MSE-only
    keys); the same shape with 8-bit MSE-only keys
    (K8V4) and with a 4-bit equally spaced key codebook (K4V4, the
    arithmetic score path);
  * long: B=8, Hq=16, Hkv=4, d=256, 131072 cached tokens, K4V4, a
    65536-block pool;
  * ragged: B=64, Hq=32, Hkv=8, d=128, lognormal lengths (median 16384,
    clipped to [1024, 131072]), K3V2 for even and K4V4 for odd sequences, the
    last 128 tokens of each sequence as a bf16 window, 0.5% x20 outliers.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import kv_cache_vector_03_amd as tq
import synth
from oracle import attention, paged
from parity import oracle_params, output_errors, score_errors

pytestmark = pytest.mark.gpu

TOL = 1e-3
CHUNK = 8192
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def _fill(ctx, pool, bt, lens, Hkv, d, seed, p, factor, only=None):
    """Quantise every sequence (of ``only``, if given) into ``pool`` on the GPU."""
    for b in range(len(lens)):
        L = int(lens[b])
        if L == 0 or (only is not None and b not in only):
            continue
        k = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b, p=p, factor=factor)
        v = synth.torch_normal_bf16((L, Hkv, d), seed * 1000003 + 2 * b + 1, p=p, factor=factor)
        t = torch.arange(L, device="cuda")
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        tq.tq_quantize_store(ctx, k, v, slots, pool)
        del k, v
    torch.cuda.synchronize()


def _decode(qd, ctxs, pools, btd, lensd, msl, W=0, **kw):
    B, Hq, d = qd.shape
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    scores = torch.full((B, Hq, msl + W), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = tq.tq_decode_workspace_bytes(qd, ctxs, pools, btd, lensd, out, chunk_tokens=CHUNK, max_seq_len=msl, **kw)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    tq.tq_decode_attention(qd, ctxs, pools, btd, lensd, out, ws, chunk_tokens=CHUNK, max_seq_len=msl,
                           scores_out=scores, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy(), scores.cpu().numpy()


def _check_all_pairs(label, pools_host, lays, prms, bt_np, cached, q, G, out, scores, seq_preset=None,
                     rk=None, rv=None, rlens=None):
    """Oracle decode of every (sequence, KV head) from the GPU-written pools;
    asserts every output row and every score."""
    B, Hq, d = q.shape
    Hkv = Hq // G

    def pair(i):
        b, h = divmod(i, Hkv)
        pr = int(seq_preset[b]) if seq_preset is not None else 0
        L = int(cached[b])
        fields = paged.read_tokens(pools_host[pr], bt_np[b], L, h, lays[pr])
        R = int(rlens[b]) if rk is not None else 0
        rkk = rk[b, h:h + 1, :R].astype(np.float64) if rk is not None else None
        rvv = rv[b, h:h + 1, :R].astype(np.float64) if rk is not None else None
        ref_out, ref_sc = attention.decode_one_sequence(q[b, h * G:(h + 1) * G].astype(np.float64), [fields],
                                                        prms[pr], rkk, rvv)
        got = out[b, h * G:(h + 1) * G].astype(np.float64)
        oe = output_errors(got, ref_out) if np.all(np.isfinite(got)) else np.inf
        sc = scores[b, h * G:(h + 1) * G, :L + R].astype(np.float64)
        se = score_errors(sc, ref_sc) if np.all(np.isfinite(sc)) else np.inf
        return b, h, L + R, oe, se

    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=WORKERS) as ex:
        res = list(ex.map(pair, range(B * Hkv)))
    worst_o = max(res, key=lambda r: r[3])
    worst_s = max(res, key=lambda r: r[4])
    print(f"[full-size parity {label}] {len(res)} (sequence, KV head) pairs, {sum(r[2] for r in res) * G} "
          f"scores: max out err {worst_o[3]:.2e} (b={worst_o[0]} h={worst_o[1]} len={worst_o[2]}), "
          f"max score err {worst_s[4]:.2e} (b={worst_s[0]} h={worst_s[1]})", flush=True)
    bad = [r for r in res if not (r[3] <= TOL and r[4] <= TOL)]
    assert not bad, f"{len(bad)} pairs out of tolerance, first {bad[:4]}"


@pytest.mark.parametrize("mse_only,kb", [(False, 3), (True, 3), (True, 8)])
def test_decode_workload_full_size_all_pairs(mse_only, kb):
    """The benchmark's decode workload, with QJL keys and with MSE-only keys
    (the benchmark's mse_only section), and with 8-bit MSE-only keys (K8V4)."""
    d, B, Hq, Hkv, L, vb, nb, seed = 128, 32, 32, 8, 8192, 4, 16384, 3
    G = Hq // Hkv
    prm = oracle_params(seed, d, kb)
    prm["qjl"] = not mse_only
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=mse_only)
    bt_np = synth.block_table(seed, B, L // 16, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    lens = np.full(B, L)
    _fill(ctx, pool, bt, lens, Hkv, d, seed, 0.0, 20.0)
    q = synth.bf16_round(synth.queries(seed, B, Hq, d))
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    out, scores = _decode(qd, [ctx], [pool], bt, torch.from_numpy(lens.astype(np.int32)).cuda(), L)
    label = f"decode b32 ctx8192 k{kb}v4{' mse-only' if mse_only else ''}"
    _check_all_pairs(label, [pool.cpu().numpy()], [paged.layout(d, kb, vb, qjl=not mse_only)], [prm], bt_np, lens,
                     q, G, out, scores)
    ctx.close()


def test_uniform_k4v4_decode_workload_full_size_all_pairs():
    """The decode workload's shape with a 4-bit equally spaced key codebook,
    which the decode scores arithmetically (c0 + idx * step, no pair table)."""
    d, B, Hq, Hkv, L, kb, vb, nb, seed = 128, 32, 32, 8, 8192, 4, 4, 16384, 6
    G = Hq // Hkv
    prm = oracle_params(seed, d, kb, uniform=True)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], uniform=True)
    bt_np = synth.block_table(seed, B, L // 16, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    lens = np.full(B, L)
    _fill(ctx, pool, bt, lens, Hkv, d, seed, 0.005, 20.0)
    q = synth.bf16_round(synth.queries(seed, B, Hq, d))
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    out, scores = _decode(qd, [ctx], [pool], bt, torch.from_numpy(lens.astype(np.int32)).cuda(), L)
    _check_all_pairs("decode b32 ctx8192 uniform k4v4", [pool.cpu().numpy()], [paged.layout(d, kb, vb)], [prm], bt_np,
                     lens, q, G, out, scores)
    ctx.close()


def test_long_context_d256_full_size_all_pairs():
    d, B, Hq, Hkv, L, kb, vb, nb, seed = 256, 8, 16, 4, 131072, 4, 4, 65536, 4
    G = Hq // Hkv
    prm = oracle_params(seed, d, kb)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"])
    bt_np = synth.block_table(seed, B, L // 16, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    lens = np.full(B, L)
    _fill(ctx, pool, bt, lens, Hkv, d, seed, 0.0, 20.0)
    q = synth.bf16_round(synth.queries(seed, B, Hq, d))
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    out, scores = _decode(qd, [ctx], [pool], bt, torch.from_numpy(lens.astype(np.int32)).cuda(), L)
    _check_all_pairs("long d256 ctx131072 k4v4", [pool.cpu().numpy()], [paged.layout(d, kb, vb)], [prm], bt_np,
                     lens, q, G, out, scores)
    ctx.close()


@pytest.mark.parametrize("mse_only,kb", [(False, 3), (True, 4)])
def test_long_context_d256_gqa8_all_pairs(mse_only, kb):
    """d = 256 with eight query heads per KV head (the variants that keep one
    wave per SIMD and hold the most registers) over 65,536- and 40,001-token
    sequences: every output row and score against the oracle decode of the
    GPU-written pool."""
    d, B, Hq, Hkv, vb, seed = 256, 2, 32, 4, 4, 7
    lens = np.array([65536, 40001])
    L = int(lens.max())
    nb = B * (L // 16) + 8
    G = Hq // Hkv
    prm = oracle_params(seed, d, kb)
    prm["qjl"] = not mse_only
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=mse_only)
    bt_np = synth.block_table(seed, B, L // 16, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    _fill(ctx, pool, bt, lens, Hkv, d, seed, 0.005, 20.0)
    q = synth.bf16_round(synth.queries(seed, B, Hq, d))
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    out, scores = _decode(qd, [ctx], [pool], bt, torch.from_numpy(lens.astype(np.int32)).cuda(), L)
    _check_all_pairs(f"long d256 G8 k{kb}v4{' mse-only' if mse_only else ''}", [pool.cpu().numpy()],
                     [paged.layout(d, kb, vb, qjl=not mse_only)], [prm], bt_np, lens, q, G, out, scores)
    ctx.close()


def test_ragged_mixed_presets_recent_window_full_size_all_pairs():
    d, B, Hq, Hkv, W, seed = 128, 64, 32, 8, 128, 5
    G = Hq // Hkv
    presets = [(3, 2), (4, 4)]
    total = synth.ragged_lengths(seed, B)             # tokens per sequence
    cached = np.maximum(total - W, 0)                 # quantised part
    rlens = np.minimum(total, W)                      # bf16 window
    seq_preset = (np.arange(B) % 2).astype(np.int8)   # K3V2 even, K4V4 odd
    prms = [oracle_params(seed + 10 * i, d, kb) for i, (kb, vb) in enumerate(presets)]
    ctxs = [tq.tq_codebook_init(d, kb, vb, signs=prms[i]["signs"], S=prms[i]["S"]) for i, (kb, vb) in enumerate(presets)]
    mb = int(np.ceil(cached.max() / 16))
    # per preset: its sequences' blocks are a permutation of that preset's pool
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
    for pr in range(2):
        _fill(ctxs[pr], pools[pr], bt, np.where(seq_preset == pr, cached, 0), Hkv, d, seed, 0.005, 20.0)
    rng = np.random.default_rng([seed, 0x3EC])
    rk32 = synth.bf16_round(rng.standard_normal((B, Hkv, W, d)).astype(np.float32))
    rv32 = synth.bf16_round(rng.standard_normal((B, Hkv, W, d)).astype(np.float32))
    kw = dict(seq_preset=torch.from_numpy(seq_preset).cuda(),
              recent_k=torch.from_numpy(synth.bf16_bits(rk32).view(np.int16)).cuda().view(torch.bfloat16),
              recent_v=torch.from_numpy(synth.bf16_bits(rv32).view(np.int16)).cuda().view(torch.bfloat16),
              recent_lens=torch.from_numpy(rlens.astype(np.int32)).cuda())
    q = synth.bf16_round(synth.queries(seed, B, Hq, d))
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    msl = mb * 16
    out, scores = _decode(qd, ctxs, pools, bt, torch.from_numpy(cached.astype(np.int32)).cuda(), msl, W=W, **kw)
    # the window's scores follow each sequence's cached tokens (columns L .. L+R-1)
    _check_all_pairs("ragged k3v2|k4v4 + bf16 window", [p.cpu().numpy() for p in pools],
                     [paged.layout(d, kb, vb) for kb, vb in presets], prms, bt_np, cached, q, G, out, scores,
                     seq_preset=seq_preset, rk=rk32, rv=rv32, rlens=rlens)
    for c in ctxs:
        c.close()
