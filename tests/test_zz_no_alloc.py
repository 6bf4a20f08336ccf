"""The decode entry point that allocates nothing (tq_decode_attention_noalloc,
for callers that cannot call hipMalloc) against tq_decode_attention on the
same inputs, through the C ABI: two calls in a row, the second with a smaller
batch and shorter sequences, both with several splits per sequence (so the
partials live in the library's static scratch) and a recent bf16 window.  On
the deterministic schedule both entry points form every sum in the same order,
so the outputs and scores must be identical.  A call whose partials exceed the
scratch is rejected on the host."""

import numpy as np
import pytest
import torch

import kv_cache_vector_03_amd as tq
import synth

pytestmark = pytest.mark.gpu


def _case(ctx, seed, B, Hq, Hkv, d, lens, W):
    mb = int(np.ceil(max(lens) / 16))
    nb = B * mb + 1
    bt_np = synth.block_table(seed, B, mb, nb)
    bt = torch.from_numpy(bt_np).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    for b in range(B):
        L = int(lens[b])
        t = torch.arange(L, device="cuda")
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        k = synth.torch_normal_bf16((L, Hkv, d), seed * 1000 + 2 * b, p=0.005)
        v = synth.torch_normal_bf16((L, Hkv, d), seed * 1000 + 2 * b + 1, p=0.005)
        tq.tq_quantize_store(ctx, k, v, slots, pool)
    rk = synth.torch_normal_bf16((B, Hkv, W, d), seed + 5)
    rv = synth.torch_normal_bf16((B, Hkv, W, d), seed + 6)
    rlens = torch.from_numpy(np.minimum(np.asarray(lens) // 7, W).astype(np.int32)).cuda()
    q = synth.torch_normal_bf16((B, Hq, d), seed + 3)
    lensd = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    kw = dict(recent_k=rk, recent_v=rv, recent_lens=rlens, chunk_tokens=256, max_seq_len=mb * 16,
              deterministic=True)
    return q, pool, bt, lensd, kw, mb * 16 + W


def test_noalloc_matches_workspace_entry_point_twice():
    d, kb, vb, Hq, Hkv = 128, 3, 4, 16, 4
    s1, s2, S = synth.method_params(91, d)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([s1, s2]), S=S)
    for call, (seed, B, lens) in enumerate(((92, 6, [3000, 511, 2049, 0, 1200, 700]), (93, 3, [900, 33, 260]))):
        q, pool, bt, lensd, kw, ncol = _case(ctx, seed, B, Hq, Hkv, d, lens, 64)
        outs, scs = [], []
        for noalloc in (False, True):
            out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
            sc = torch.full((B, Hq, ncol), float("nan"), dtype=torch.float32, device="cuda")
            if noalloc:
                tq.tq_decode_attention_noalloc(q, [ctx], [pool], bt, lensd, out, scores_out=sc, **kw)
            else:
                nbytes = tq.tq_decode_workspace_bytes(q, [ctx], [pool], bt, lensd, out, **kw)
                ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
                tq.tq_decode_attention(q, [ctx], [pool], bt, lensd, out, ws, scores_out=sc, **kw)
            torch.cuda.synchronize()
            outs.append(out)
            scs.append(sc)
        print(f"[noalloc call {call}] B={B} max |noalloc - workspace| = "
              f"{float((outs[1] - outs[0]).abs().max()):.3e}", flush=True)
        assert torch.isfinite(outs[1]).all()
        assert torch.equal(outs[0], outs[1])
        assert torch.equal(torch.nan_to_num(scs[0], nan=0.0), torch.nan_to_num(scs[1], nan=0.0))
    ctx.close()


def test_noalloc_rejects_partials_beyond_the_scratch():
    d, kb, vb, B, Hq, Hkv = 128, 3, 4, 64, 32, 8
    s1, s2, S = synth.method_params(94, d)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([s1, s2]), S=S)
    msl = 32 * 1000  # 1000 splits of 32 tokens per sequence
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((2, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    bt = torch.zeros((B, msl // 16), dtype=torch.int32, device="cuda")
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    need = tq.tq_decode_workspace_bytes(q, [ctx], [pool], bt, lens, out, chunk_tokens=32, max_seq_len=msl)
    assert need > tq.NOALLOC_SCRATCH_BYTES
    with pytest.raises(tq.TqError) as e:
        tq.tq_decode_attention_noalloc(q, [ctx], [pool], bt, lens, out, chunk_tokens=32, max_seq_len=msl)
    assert e.value.code == tq.TQ_EINVAL and "scratch" in str(e.value)
    ctx.close()
