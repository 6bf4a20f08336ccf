"""GPU parity of 8-bit MSE-only keys (the K8V4 preset the iThome page lists
among vLLM's presets, "which path vLLM takes": Hadamard rotation and
MSE-quantised keys, no QJL sketch) against the oracle.

Records bit-exact outside the 1e-6 decision band through all three store
kernels (the MFMA kernel for large bf16 batches at head_dim 128, the tiled
kernel for fp32 inputs and head_dim 256, the row kernel for small batches),
whose 8-bit index is a binary search over the 255 thresholds; decode scores
and outputs within 1e-3 on oracle-written caches (one-code table lookups),
at head_dim 128 and 256 with four and eight query heads per KV head.  The
extend kernel rejects 8-bit keys."""

import numpy as np
import pytest
import torch

import kv_cache_vector_03_amd as tq
import synth
from oracle import attention, paged
from parity import compare_pools, expected_records, oracle_cache, oracle_params, output_errors, score_errors

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.mark.parametrize("d,vb,T,Hkv,dtype", [
    (128, 4, 1500, 8, torch.bfloat16),   # MFMA store kernel (more than 2048 token-heads)
    (128, 2, 700, 4, torch.float32),     # tiled kernel (fp32 input)
    (256, 4, 601, 4, torch.bfloat16),    # tiled kernel (head_dim 256)
    (128, 4, 5, 8, torch.bfloat16),      # row kernel
    (256, 2, 37, 2, torch.float32),      # row kernel, head_dim 256
])
def test_k8_quantize_every_store_kernel(d, vb, T, Hkv, dtype):
    kb, seed = 8, 80 + vb
    prm = oracle_params(seed, d, kb)
    rng = np.random.default_rng([808, d, vb, T])
    K = synth.normal_with_outliers(rng, (T, Hkv, d), 0.005, 20.0)
    V = synth.normal_with_outliers(rng, (T, Hkv, d), 0.005, 20.0)
    nb = (T + 15) // 16 + 3
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=True)
    c, t, _, _ = tq.tq_ctx_tables(ctx)
    assert np.array_equal(c, prm["c32"]) and np.array_equal(t, prm["t32"])
    k = torch.from_numpy(K).to(dtype).cuda()
    v = torch.from_numpy(V).to(dtype).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    tq.tq_quantize_store(ctx, k, v, torch.from_numpy(slots.astype(np.int32)).cuda(), pool)
    torch.cuda.synchronize()
    gpu = pool.cpu().numpy()
    ctx.close()
    lay = paged.layout(d, kb, vb, qjl=False)
    exp = paged.new_pool(nb, Hkv, lay)
    mask = paged.new_pool(nb, Hkv, lay)
    Kx = k.float().cpu().numpy().astype(np.float64)
    Vx = v.float().cpu().numpy()
    counts = {}
    for h in range(Hkv):
        cnt = expected_records(Kx[:, h], Vx[:, h], slots, h, prm, d, kb, vb, exp, mask, qjl=False)
        for key, val in cnt.items():
            counts[key] = counts.get(key, 0) + val
    outside, inside = compare_pools(gpu, exp, mask)
    print(f"[k8 quantize parity d{d} k8v{vb} T={T}x{Hkv} {str(dtype)[6:]}] exempt={counts} "
          f"differing bits outside band={outside} inside band={inside}", flush=True)
    assert outside == 0


@pytest.mark.parametrize("d,Hq,vb,chunk", [(128, 8, 4, 512), (128, 16, 2, 1024), (256, 8, 4, 256), (256, 16, 4, 4096)])
def test_k8_decode(d, Hq, vb, chunk):
    kb, seed, B, Hkv = 8, 88, 4, 2
    lens = np.array([1000, 33, 0, 2000])
    prm = oracle_params(seed, d, kb)
    prm["qjl"] = False
    mb = int(np.ceil(lens.max() / 16))
    nb = B * mb + 3
    bt = synth.block_table(seed, B, mb, nb)
    pool = paged.new_pool(nb, Hkv, paged.layout(d, kb, vb, qjl=False))
    fields = oracle_cache(prm, d, kb, vb, lens, Hkv, bt, pool, seed, p=0.005, qjl=False)
    q = synth.queries(seed, B, Hq, d)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=True)
    qd = torch.from_numpy(q).cuda()
    pd = torch.from_numpy(pool).cuda()
    btd = torch.from_numpy(bt.astype(np.int32)).cuda()
    lensd = torch.from_numpy(lens.astype(np.int32)).cuda()
    msl = mb * 16
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, msl), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = tq.tq_decode_workspace_bytes(qd, [ctx], [pd], btd, lensd, out, chunk_tokens=chunk, max_seq_len=msl)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    tq.tq_decode_attention(qd, [ctx], [pd], btd, lensd, out, ws, chunk_tokens=chunk, max_seq_len=msl, scores_out=sc)
    torch.cuda.synchronize()
    out, sc = out.cpu().numpy(), sc.cpu().numpy()
    ctx.close()
    ref, errs = [], []
    for b in range(B):
        o, s = attention.decode_one_sequence(q[b].astype(np.float64), fields[b], prm)
        ref.append(o)
        if s.shape[1]:
            errs.append(score_errors(sc[b, :, :s.shape[1]].astype(np.float64), s))
    se, oe = max(errs), output_errors(out.astype(np.float64), np.stack(ref))
    print(f"[k8 decode parity d{d} G{Hq // Hkv} k8v{vb} chunk {chunk}] max score err {se:.2e} max out err {oe:.2e}",
          flush=True)
    assert np.all(np.isfinite(out)) and se <= TOL and oe <= TOL


def test_extend_rejects_8_bit_keys():
    d, B, Hq, Hkv, C = 128, 1, 4, 1, 16
    ctx = tq.tq_codebook_init(d, 8, 4, mse_only=True)
    q = torch.zeros((B * C, Hq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B * C, Hkv, d), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((2, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    cu = torch.tensor([0, C], dtype=torch.int32, device="cuda")
    bt = torch.zeros((B, 2), dtype=torch.int32, device="cuda")
    plen = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.empty((B * C, Hq, d), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="8-bit keys"):
        tq.tq_extend_attention(q, k, k, cu, ctx, pool, bt, plen, out, max_chunk=C)
    ctx.close()
