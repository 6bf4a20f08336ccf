"""Seeded random sweep of decode, store and extend configurations against the
oracle, to reach the combinations the targeted tests do not enumerate: any
number of query heads per KV head up to 8 (odd ones included), one or two
presets per batch (every key width, both value widths, QJL / MSE-only /
equally spaced keys), empty and ragged sequences, split sizes from 32 to
8192 tokens, recent windows of any length, both step schedules, fp32 and
bf16 queries; the store path with random token counts, head counts, skipped
slots and both input dtypes; extend with random chunk and prefix lengths.
Every configuration is printed before it runs.  Tolerances are the
contract's: records bit-exact outside the 1e-6 band, scores and outputs
within 1e-3."""

import numpy as np
import pytest
import torch

import kv_cache_vector_03_amd as tq
import synth
from oracle import attention, paged
from parity import (compare_pools, expected_records, oracle_cache, oracle_params, output_errors,
                    score_errors)

pytestmark = pytest.mark.gpu

TOL = 1e-3
KINDS = [(2, 2, "qjl"), (2, 4, "qjl"), (3, 2, "qjl"), (3, 4, "qjl"), (4, 2, "qjl"), (4, 4, "qjl"),
         (3, 4, "mse"), (4, 2, "mse"), (2, 4, "mse"), (8, 4, "mse"), (8, 2, "mse"),
         (4, 4, "uniform"), (3, 2, "uniform"), (4, 2, "uniform-mse")]


def _kind_flags(kind):
    return dict(mse_only="mse" in kind, uniform="uniform" in kind)


def _decode_case(i):
    rng = np.random.default_rng([2026, 12, i])
    d = int(rng.choice([128, 256]))
    G = int(rng.integers(1, 9))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.integers(1, 5))
    npre = 2 if (B >= 2 and rng.random() < 0.4) else 1
    kinds = [KINDS[j] for j in rng.choice(len(KINDS), npre, replace=False)]
    lens = rng.integers(0, 1300, B)
    lens[rng.random(B) < 0.2] = 0
    chunk = int(rng.choice([32, 64, 96, 256, 1024, 8192]))
    W = int(rng.choice([0, 0, 16, 128]))
    det = bool(rng.random() < 0.3)
    q_bf16 = bool(rng.random() < 0.6)
    return dict(d=d, G=G, Hkv=Hkv, B=B, kinds=kinds, lens=lens, chunk=chunk, W=W, det=det, q_bf16=q_bf16)


@pytest.mark.parametrize("i", range(24))
def test_random_decode_configuration(i):
    c = _decode_case(i)
    d, G, Hkv, B, kinds, lens, chunk, W = c["d"], c["G"], c["Hkv"], c["B"], c["kinds"], c["lens"], c["chunk"], c["W"]
    Hq = G * Hkv
    print(f"[random decode {i}] d={d} G={G} Hkv={Hkv} B={B} presets={kinds} lens={lens.tolist()} chunk={chunk} "
          f"W={W} det={c['det']} q_bf16={c['q_bf16']}", flush=True)
    seed = 9000 + i
    npre = len(kinds)
    seq_preset = (np.arange(B) % npre).astype(np.int8)
    prms, ctxs, pools, fields = [], [], [], {}
    mb = max(1, int(np.ceil(lens.max() / 16)))
    nb = B * mb + 2
    bt = synth.block_table(seed, B, mb, nb)
    for p, (kb, vb, kind) in enumerate(kinds):
        fl = _kind_flags(kind)
        prm = oracle_params(seed + 7 * p, d, kb, uniform=fl["uniform"])
        prm["qjl"] = not fl["mse_only"]
        pool = paged.new_pool(nb, Hkv, paged.layout(d, kb, vb, qjl=not fl["mse_only"]))
        seqs = [b for b in range(B) if seq_preset[b] == p]
        fields.update(oracle_cache(prm, d, kb, vb, lens, Hkv, bt, pool, seed, p=0.005, seqs=seqs,
                                   qjl=not fl["mse_only"]))
        prms.append(prm)
        pools.append(pool)
        ctxs.append(tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], **fl))
    rng = np.random.default_rng([seed, 1])
    kw = {}
    rlens = np.zeros(B, dtype=np.int64)
    rk32 = rv32 = None
    if W:
        rlens = rng.integers(0, W + 1, B)
        rk32 = synth.bf16_round(rng.standard_normal((B, Hkv, W, d)).astype(np.float32))
        rv32 = synth.bf16_round(rng.standard_normal((B, Hkv, W, d)).astype(np.float32))
        kw.update(recent_k=torch.from_numpy(synth.bf16_bits(rk32).view(np.int16)).cuda().view(torch.bfloat16),
                  recent_v=torch.from_numpy(synth.bf16_bits(rv32).view(np.int16)).cuda().view(torch.bfloat16),
                  recent_lens=torch.from_numpy(rlens.astype(np.int32)).cuda())
    if npre == 2:
        kw["seq_preset"] = torch.from_numpy(seq_preset).cuda()
    q = synth.queries(seed, B, Hq, d)
    if c["q_bf16"]:
        q = synth.bf16_round(q)
        qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    else:
        qd = torch.from_numpy(q).cuda()
    pd = [torch.from_numpy(p).cuda() for p in pools]
    btd = torch.from_numpy(bt.astype(np.int32)).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    msl = mb * 16
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, msl + W), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = tq.tq_decode_workspace_bytes(qd, ctxs, pd, btd, ld, out, chunk_tokens=chunk, max_seq_len=msl, **kw)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    tq.tq_decode_attention(qd, ctxs, pd, btd, ld, out, ws, chunk_tokens=chunk, max_seq_len=msl, scores_out=sc,
                           deterministic=c["det"], **kw)
    torch.cuda.synchronize()
    out, sc = out.cpu().numpy(), sc.cpu().numpy()
    for cx in ctxs:
        cx.close()
    ref, serr = [], []
    for b in range(B):
        pr = int(seq_preset[b])
        R = int(rlens[b])
        rkk = rk32[b, :, :R].astype(np.float64) if R else None
        rvv = rv32[b, :, :R].astype(np.float64) if R else None
        o, s = attention.decode_one_sequence(q[b].astype(np.float64), fields[b], prms[pr], rkk, rvv)
        ref.append(o)
        L = int(lens[b])
        if L + R:
            got = np.concatenate([sc[b, :, :L], sc[b, :, L:L + R]], axis=1)
            serr.append(score_errors(got.astype(np.float64), s))
    oe = output_errors(out.astype(np.float64), np.stack(ref))
    se = max(serr) if serr else 0.0
    print(f"[random decode {i}] max score err {se:.2e} max out err {oe:.2e}", flush=True)
    assert np.all(np.isfinite(out)) and se <= TOL and oe <= TOL


@pytest.mark.parametrize("i", range(12))
def test_random_store_configuration(i):
    rng = np.random.default_rng([2026, 13, i])
    d = int(rng.choice([128, 256]))
    kb, vb, kind = KINDS[int(rng.integers(len(KINDS)))]
    fl = _kind_flags(kind)
    T = int(rng.choice([1, 3, 17, 255, 700, 1500, 2600]))
    Hkv = int(rng.integers(1, 9))
    dtype = torch.bfloat16 if rng.random() < 0.6 else torch.float32
    print(f"[random store {i}] d={d} k{kb}v{vb} {kind} T={T} Hkv={Hkv} {str(dtype)[6:]}", flush=True)
    seed = 9500 + i
    prm = oracle_params(seed, d, kb, uniform=fl["uniform"])
    K = synth.normal_with_outliers(rng, (T, Hkv, d), 0.005, 20.0)
    V = synth.normal_with_outliers(rng, (T, Hkv, d), 0.005, 20.0)
    nb = (T + 15) // 16 + 2
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[rng.random(T) < 0.05] = -1  # skipped tokens
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], **fl)
    k = torch.from_numpy(K).to(dtype).cuda()
    v = torch.from_numpy(V).to(dtype).cuda()
    pool = torch.zeros((nb, Hkv, ctx.block_bytes), dtype=torch.uint8, device="cuda")
    tq.tq_quantize_store(ctx, k, v, torch.from_numpy(slots.astype(np.int32)).cuda(), pool)
    torch.cuda.synchronize()
    gpu = pool.cpu().numpy()
    ctx.close()
    lay = paged.layout(d, kb, vb, qjl=not fl["mse_only"])
    exp = paged.new_pool(nb, Hkv, lay)
    mask = paged.new_pool(nb, Hkv, lay)
    keep = slots >= 0
    Kx = k.float().cpu().numpy().astype(np.float64)
    Vx = v.float().cpu().numpy()
    for h in range(Hkv):
        expected_records(Kx[keep, h], Vx[keep, h], slots[keep], h, prm, d, kb, vb, exp, mask,
                         qjl=not fl["mse_only"])
    outside, inside = compare_pools(gpu, exp, mask)
    print(f"[random store {i}] differing bits outside band={outside} inside band={inside}", flush=True)
    assert outside == 0


@pytest.mark.parametrize("i", range(8))
def test_random_extend_configuration(i):
    rng = np.random.default_rng([2026, 14, i])
    d = 128
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2]))
    Hq = G * Hkv
    kb, vb, kind = [x for x in KINDS if x[0] <= 4 and "uniform" not in x[2]][int(rng.integers(9))]
    mse = kind == "mse"
    B = int(rng.integers(1, 4))
    plens = rng.integers(0, 600, B)
    clens = rng.integers(1, 90, B)
    print(f"[random extend {i}] G={G} Hkv={Hkv} k{kb}v{vb} {kind} prefix={plens.tolist()} chunk={clens.tolist()}",
          flush=True)
    seed = 9800 + i
    prm = oracle_params(seed, d, kb)
    prm["qjl"] = not mse
    mb = max(1, int(np.ceil(plens.max() / 16)))
    nb = B * mb + 2
    bt = synth.block_table(seed, B, mb, nb)
    pool = paged.new_pool(nb, Hkv, paged.layout(d, kb, vb, qjl=not mse))
    fields = oracle_cache(prm, d, kb, vb, plens, Hkv, bt, pool, seed, p=0.005, qjl=not mse)
    ctx = tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=mse)
    cu = np.concatenate([[0], np.cumsum(clens)]).astype(np.int32)
    N = int(cu[-1])
    q = synth.bf16_round(rng.standard_normal((N, Hq, d)).astype(np.float32))
    kc = synth.bf16_round(synth.normal_with_outliers(rng, (N, Hkv, d), 0.005, 20.0))
    vc = synth.bf16_round(synth.normal_with_outliers(rng, (N, Hkv, d), 0.005, 20.0))
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()  # noqa: E731
    out = torch.full((N, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    tq.tq_extend_attention(to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(cu).cuda(), ctx,
                           torch.from_numpy(pool).cuda(), torch.from_numpy(bt.astype(np.int32)).cuda(),
                           torch.from_numpy(plens.astype(np.int32)).cuda(), out, max_chunk=int(clens.max()))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ctx.close()
    worst = 0.0
    for b in range(B):
        rows = slice(int(cu[b]), int(cu[b + 1]))
        ref = attention.extend_one_sequence(q[rows].astype(np.float64), fields[b], kc[rows], vc[rows], prm)
        worst = max(worst, output_errors(out[rows].astype(np.float64).reshape(-1, d), ref.reshape(-1, d)))
    print(f"[random extend {i}] max out err {worst:.2e}", flush=True)
    assert np.all(np.isfinite(out)) and worst <= TOL


@pytest.mark.parametrize("Hq,mse_first", [(64, False), (32, True)])
def test_gqa8_many_items_per_workgroup(Hq, mse_first):
    """Many split items per workgroup (so the score operands kept in LDS are
    reused and rebuilt across consecutive items), two presets, ragged
    lengths, 64-token splits and a bf16 recent window.  Eight query heads
    per KV head: K3V4 (operands in LDS, 8-wave workgroups) beside K4V4 with
    the sketch (operands in registers).  Four: K3V4 with MSE-only keys
    (operands in LDS, 12-wave workgroups) beside K4V4 with the sketch."""
    d, B, Hkv, W, chunk, seed = 128, 16, 8, 32, 64, 9900 if Hq == 64 else 9932
    kinds = [(3, 4, not mse_first), (4, 4, True)]
    lens = synth.ragged_lengths(seed, B, lo=100, hi=3000, median=1200.0)
    lens[3] = 0
    print(f"[many items G{Hq // Hkv}] lens={lens.tolist()} chunk={chunk} W={W}", flush=True)
    seq_preset = (np.arange(B) % 2).astype(np.int8)
    mb = int(np.ceil(lens.max() / 16))
    nb = B * mb + 2
    bt = synth.block_table(seed, B, mb, nb)
    prms, ctxs, pools, fields = [], [], [], {}
    for p, (kb, vb, qjl) in enumerate(kinds):
        prm = oracle_params(seed + 7 * p, d, kb)
        prm["qjl"] = qjl
        pool = paged.new_pool(nb, Hkv, paged.layout(d, kb, vb, qjl=qjl))
        seqs = [b for b in range(B) if seq_preset[b] == p]
        fields.update(oracle_cache(prm, d, kb, vb, lens, Hkv, bt, pool, seed, p=0.005, seqs=seqs, qjl=qjl))
        prms.append(prm)
        pools.append(pool)
        ctxs.append(tq.tq_codebook_init(d, kb, vb, signs=prm["signs"], S=prm["S"], mse_only=not qjl))
    rng = np.random.default_rng([seed, 1])
    rlens = rng.integers(0, W + 1, B)
    rk32 = synth.bf16_round(rng.standard_normal((B, Hkv, W, d)).astype(np.float32))
    rv32 = synth.bf16_round(rng.standard_normal((B, Hkv, W, d)).astype(np.float32))
    kw = dict(seq_preset=torch.from_numpy(seq_preset).cuda(),
              recent_k=torch.from_numpy(synth.bf16_bits(rk32).view(np.int16)).cuda().view(torch.bfloat16),
              recent_v=torch.from_numpy(synth.bf16_bits(rv32).view(np.int16)).cuda().view(torch.bfloat16),
              recent_lens=torch.from_numpy(rlens.astype(np.int32)).cuda())
    q = synth.bf16_round(synth.queries(seed, B, Hq, d))
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    pd = [torch.from_numpy(p).cuda() for p in pools]
    btd = torch.from_numpy(bt.astype(np.int32)).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    msl = mb * 16
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    sc = torch.full((B, Hq, msl + W), float("nan"), dtype=torch.float32, device="cuda")
    nbytes = tq.tq_decode_workspace_bytes(qd, ctxs, pd, btd, ld, out, chunk_tokens=chunk, max_seq_len=msl, **kw)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    tq.tq_decode_attention(qd, ctxs, pd, btd, ld, out, ws, chunk_tokens=chunk, max_seq_len=msl, scores_out=sc, **kw)
    torch.cuda.synchronize()
    out, sc = out.cpu().numpy(), sc.cpu().numpy()
    for cx in ctxs:
        cx.close()
    ref, serr = [], []
    for b in range(B):
        pr, R, L = int(seq_preset[b]), int(rlens[b]), int(lens[b])
        o, s = attention.decode_one_sequence(q[b].astype(np.float64), fields[b], prms[pr],
                                             rk32[b, :, :R].astype(np.float64), rv32[b, :, :R].astype(np.float64))
        ref.append(o)
        if L + R:
            got = np.concatenate([sc[b, :, :L], sc[b, :, L:L + R]], axis=1)
            serr.append(score_errors(got.astype(np.float64), s))
    oe = output_errors(out.astype(np.float64), np.stack(ref))
    print(f"[many items G{Hq // Hkv}] max score err {max(serr):.2e} max out err {oe:.2e}", flush=True)
    assert np.all(np.isfinite(out)) and max(serr) <= TOL and oe <= TOL
