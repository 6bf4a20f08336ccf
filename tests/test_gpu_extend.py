"""GPU parity of tq_extend_attention (extend / chunked prefill attention over
the compressed prefix plus the chunk's own bf16 keys and values, causal)
against the oracle's extend attention, on pools written by the oracle (small
cases: every row of every chunk) and by the GPU quantiser (the prefill
workload's shape: every chunk's rows sampled, checked against the decode
oracle with the chunk's tokens up to the row as its recent window, which the
oracle pins show is the same function).  Outputs within 1e-3 relative per
row."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import kv_cache_vector_03_amd as tq
import synth
from oracle import attention, paged
from parity import oracle_cache, oracle_params, output_errors

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _bf16(rng, shape, p=0.0):
    return synth.normal_with_outliers(rng, shape, p, 20.0)


def _to_dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("kb,vb,G,mse_only", [(3, 4, 4, False), (4, 2, 1, False), (2, 4, 8, False),
                                              (3, 2, 2, True), (4, 4, 4, True)])
def test_extend_small_every_row(kb, vb, G, mse_only):
    d, Hkv = 128, 2
    Hq = G * Hkv
    seed = 70 + kb * 10 + G
    prefix = np.array([100, 0, 37, 250, 16])
    chunk = np.array([40, 17, 1, 70, 33])
    B = len(prefix)
    prm = oracle_params(seed, d, kb)
    prm["qjl"] = not mse_only
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=mse_only)
    mb = int(np.ceil(max(prefix.max(), 1) / 16))
    nb = B * mb + 3
    bt = synth.block_table(seed, B, mb, nb)
    pool = paged.new_pool(nb, Hkv, paged.layout(d, kb, vb, qjl=not mse_only))
    fields = oracle_cache(prm, d, kb, vb, prefix, Hkv, bt, pool, seed, p=0.005, qjl=not mse_only)
    rng = np.random.default_rng(seed)
    T = int(chunk.sum())
    q = _bf16(rng, (T, Hq, d))
    k = _bf16(rng, (T, Hkv, d), 0.005)
    v = _bf16(rng, (T, Hkv, d), 0.005)
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    out = torch.full((T, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_extend_attention(_to_dev_bf16(q), _to_dev_bf16(k), _to_dev_bf16(v), torch.from_numpy(cu).cuda(), ctx,
                           torch.from_numpy(pool).cuda(), torch.from_numpy(bt.astype(np.int32)).cuda(),
                           torch.from_numpy(prefix.astype(np.int32)).cuda(), out, max_chunk=int(chunk.max()))
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    worst = 0.0
    for b in range(B):
        sl = slice(cu[b], cu[b + 1])
        ref = attention.extend_one_sequence(q[sl].astype(np.float64), fields[b], k[sl], v[sl], prm)
        e = max(output_errors(got[sl][:, hq], ref[:, hq]) for hq in range(Hq))
        worst = max(worst, e)
        assert np.all(np.isfinite(got[sl]))
    print(f"[extend parity k{kb}v{vb} G={G}{' mse-only' if mse_only else ''}] {T} chunk tokens, "
          f"max out err {worst:.2e}", flush=True)
    assert worst <= TOL
    ctx.close()


def test_extend_prefill_workload_gpu_written_prefix_sampled_rows():
    """The prefill workload: B=4, Hq=32, Hkv=8, d=128, an 8192-token K3V4
    prefix per sequence written by tq_quantize_store through a permuted block
    table, a 512-token chunk per sequence; for every sequence and KV head,
    rows 0, 1, 63, 64, 255 and 511 of the chunk (all 4 query heads) against
    the oracle reading the GPU-written pool."""
    d, B, Hq, Hkv, P, C, kb, vb, seed = 128, 4, 32, 8, 8192, 512, 3, 4, 6
    G = Hq // Hkv
    prm = oracle_params(seed, d, kb)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"])
    mb = (P + C) // 16
    nb = B * mb
    bt_np = synth.block_table(seed, B, mb, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    t = torch.arange(P, device="cuda")
    for b in range(B):
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        kk = synth.torch_normal_bf16((P, Hkv, d), seed * 1000003 + 2 * b, p=0.005)
        vv = synth.torch_normal_bf16((P, Hkv, d), seed * 1000003 + 2 * b + 1, p=0.005)
        tq.tq_quantize_store(ctx, kk, vv, slots, pool)
    rng = np.random.default_rng(seed)
    q = _bf16(rng, (B * C, Hq, d))
    k = _bf16(rng, (B * C, Hkv, d), 0.005)
    v = _bf16(rng, (B * C, Hkv, d), 0.005)
    cu = (np.arange(B + 1) * C).astype(np.int32)
    out = torch.full((B * C, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_extend_attention(_to_dev_bf16(q), _to_dev_bf16(k), _to_dev_bf16(v), torch.from_numpy(cu).cuda(), ctx, pool,
                           bt, torch.full((B,), P, dtype=torch.int32, device="cuda"), out, max_chunk=C)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    host_pool = pool.cpu().numpy()
    lay = paged.layout(d, kb, vb)
    rows = [0, 1, 63, 64, 255, 511]

    def pair(i):
        b, h = divmod(i, Hkv)
        f = paged.read_tokens(host_pool, bt_np[b], P, h, lay)
        worst = 0.0
        for r in rows:
            tok = b * C + r
            rk = k[b * C:tok + 1, h][None].astype(np.float64)
            rv = v[b * C:tok + 1, h][None].astype(np.float64)
            ref, _ = attention.decode_one_sequence(q[tok, h * G:(h + 1) * G].astype(np.float64), [f], prm, rk, rv)
            worst = max(worst, output_errors(got[tok, h * G:(h + 1) * G], ref))
        return worst

    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=max(1, min(16, len(os.sched_getaffinity(0))))) as ex:
        errs = list(ex.map(pair, range(B * Hkv)))
    print(f"[extend parity prefill b4 prefix8192 chunk512 k3v4] {B * Hkv * len(rows) * G} rows sampled, "
          f"max out err {max(errs):.2e}; all outputs finite: {bool(np.all(np.isfinite(got)))}", flush=True)
    assert np.all(np.isfinite(got))
    assert max(errs) <= TOL
    ctx.close()
