"""A decode step (store the new token of every sequence, then decode
attention over the compressed cache) captured in a HIP graph and replayed
(Roadmap §3.1 and §7: a fixed split grid and caller-owned workspace so that
the path can run under graph capture; the library allocates nothing and
records no memset inside its calls).

Every replay is compared with the same step run eagerly on the same inputs,
with eager work and synchronisations between the replays, and the query
buffer is rewritten between replays to check that each replay reads the
current inputs.  Both launch shapes are covered: one split per sequence
(direct output) and several splits with the combine launch, with one preset
and with two (one split launch per preset, both captured).

Every wave of the split kernel takes its cache steps in a fixed order, so
every replay must equal the eager run bit for bit, with or without
TQ_DECODE_DETERMINISTIC (accepted, no further effect); a stale replay (new
queries) fails that by orders of magnitude.
"""

import numpy as np
import pytest
import torch

import kv_cache_vector_03_amd as tq
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("two_presets", [False, True])
@pytest.mark.parametrize("chunk", [8192, 256])
def test_captured_decode_step_replays_match_eager(chunk, two_presets, deterministic):
    d, B, Hq, Hkv, L, kb, vb, seed = 128, 4, 8, 2, 1024, 3, 4, 160
    s1, s2, S = synth.method_params(seed, d)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=np.stack([s1, s2]), S=S)
    ctx2 = tq.tq_codebook_init(d, 4, 2, signs=np.stack([s1, s2]), S=S, mse_only=True) if two_presets else None
    nb = B * (L // 16) + 2
    bt = torch.from_numpy(synth.block_table(seed, B, L // 16, nb)).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    pool2 = torch.zeros((nb, Hkv, ctx2.block_bytes), dtype=torch.uint8, device="cuda") if two_presets else None
    preset_of = [b % 2 if two_presets else 0 for b in range(B)]
    t = torch.arange(L, device="cuda")
    for b in range(B):
        slots = (bt[b][t // 16].long() * 16 + t % 16).to(torch.int32)
        k = synth.torch_normal_bf16((L, Hkv, d), seed * 100 + 2 * b)
        v = synth.torch_normal_bf16((L, Hkv, d), seed * 100 + 2 * b + 1)
        if preset_of[b] == 0:
            tq.tq_quantize_store(ctx, k, v, slots, pool)
        else:
            tq.tq_quantize_store(ctx2, k, v, slots, pool2)
    knew = synth.torch_normal_bf16((B, Hkv, d), seed + 1)
    vnew = synth.torch_normal_bf16((B, Hkv, d), seed + 2)
    slot_new = (bt[:, (L - 1) // 16].long() * 16 + (L - 1) % 16).to(torch.int32).contiguous()
    # the new token of each preset's sequences goes to that preset's pool
    sel = [torch.tensor([b for b in range(B) if preset_of[b] == p], dtype=torch.long, device="cuda") for p in (0, 1)]
    kw = {"deterministic": deterministic}
    if two_presets:
        kw["seq_preset"] = torch.tensor(preset_of, dtype=torch.int8, device="cuda")
    ctxs = [ctx, ctx2] if two_presets else [ctx]
    pools = [pool, pool2] if two_presets else [pool]
    knew_p = [knew[s_].contiguous() for s_ in sel]
    vnew_p = [vnew[s_].contiguous() for s_ in sel]
    slot_p = [slot_new[s_].contiguous() for s_ in sel]
    q = synth.torch_normal_bf16((B, Hq, d), seed + 3)
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    nbytes = tq.tq_decode_workspace_bytes(q, ctxs, pools, bt, lens, out, chunk_tokens=chunk, max_seq_len=L, **kw)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        for p in range(len(ctxs)):
            if len(sel[p]):
                tq.tq_quantize_store(ctxs[p], knew_p[p], vnew_p[p], slot_p[p], pools[p])
        tq.tq_decode_attention(q, ctxs, pools, bt, lens, out, ws, chunk_tokens=chunk, max_seq_len=L, **kw)

    # warm up on a side stream (torch's recipe before capture), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for r in range(4):
        if r >= 2:  # new queries in the captured buffer
            q.copy_(synth.torch_normal_bf16((B, Hq, d), seed + 10 + r))
        step()  # eager reference on the same inputs
        torch.cuda.synchronize()
        ref = out.clone()
        out.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.clone()
        print(f"[graph chunk {chunk} presets {len(ctxs)} deterministic {deterministic}] replay {r}: "
              f"max |replay - eager| = {float((got - ref).abs().max()):.3e}", flush=True)
        assert torch.isfinite(got).all()
        assert torch.equal(got, ref)
    del g
    ctx.close()
    if ctx2 is not None:
        ctx2.close()
