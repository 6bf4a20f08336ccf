"""CPU checks of the decode binding's argument validation: every tensor the C
ABI would trust as a device pointer is checked for device, dtype, layout and
shape before the library is called, so a mismatched call raises instead of
reaching a kernel.  The tensors here are CPU tensors with the device check
stubbed out; nothing reaches the library."""

import pytest
import torch

import kv_cache_vector_03_amd as tq


class _Ctx:
    """Stand-in for a Context (no device tables are needed for validation)."""

    def __init__(self, d=128, block_bytes=2368):
        self.handle, self.head_dim, self.block_bytes = 1, d, block_bytes


def _valid(B=2, Hq=8, Hkv=2, d=128, W=16, two=False):
    ctxs = [_Ctx(d)] + ([_Ctx(d, 2624)] if two else [])
    kw = dict(
        q=torch.zeros(B, Hq, d, dtype=torch.bfloat16),
        ctxs=ctxs,
        pools=[torch.zeros(4, Hkv, c.block_bytes, dtype=torch.uint8) for c in ctxs],
        block_tables=torch.zeros(B, 4, dtype=torch.int32),
        seq_lens=torch.zeros(B, dtype=torch.int32),
        out=torch.zeros(B, Hq, d, dtype=torch.float32),
        workspace=torch.zeros(1024, dtype=torch.uint8),
        recent_k=torch.zeros(B, Hkv, W, d, dtype=torch.bfloat16),
        recent_v=torch.zeros(B, Hkv, W, d, dtype=torch.bfloat16),
        recent_lens=torch.zeros(B, dtype=torch.int32),
        scores_out=torch.zeros(B, Hq, 64 + W, dtype=torch.float32),
        seq_preset=torch.zeros(B, dtype=torch.int8) if two else None,
    )
    return kw


def _call(kw):
    kw = dict(kw)
    return tq._decode_args(kw.pop("q"), kw.pop("ctxs"), kw.pop("pools"), kw.pop("block_tables"),
                           kw.pop("seq_lens"), kw.pop("out"), **kw)


@pytest.fixture
def on_device(monkeypatch):
    monkeypatch.setattr(tq, "_on_device", lambda t: True)


def test_valid_arguments_marshal(on_device):
    a = _call(_valid())
    assert a.batch == 2 and a.num_q_heads == 8 and a.num_kv_heads == 2 and a.recent_window == 16
    assert a.scores_stride == 80 and a.flags == 0
    a = _call(dict(_valid(two=True), deterministic=True))
    assert a.num_presets == 2 and a.flags == tq.TQ_DECODE_DETERMINISTIC


def test_cpu_tensors_are_rejected():
    with pytest.raises(ValueError, match="device"):
        _call(_valid())


BAD = {
    "q head_dim vs context": lambda kw: kw.update(q=torch.zeros(2, 8, 256, dtype=torch.bfloat16)),
    "q dtype": lambda kw: kw.update(q=torch.zeros(2, 8, 128, dtype=torch.float16)),
    "q non-contiguous": lambda kw: kw.update(q=torch.zeros(2, 128, 8, dtype=torch.bfloat16).transpose(1, 2)),
    "out dtype": lambda kw: kw.update(out=torch.zeros(2, 8, 128, dtype=torch.bfloat16)),
    "out shape": lambda kw: kw.update(out=torch.zeros(2, 4, 128, dtype=torch.float32)),
    "pool record size": lambda kw: kw.update(pools=[torch.zeros(4, 2, 2000, dtype=torch.uint8)]),
    "pool dtype": lambda kw: kw.update(pools=[torch.zeros(4, 2, 592, dtype=torch.int32)]),
    "heads not a multiple": lambda kw: kw.update(pools=[torch.zeros(4, 3, 2368, dtype=torch.uint8)]),
    "block_tables rows": lambda kw: kw.update(block_tables=torch.zeros(3, 4, dtype=torch.int32)),
    "block_tables dtype": lambda kw: kw.update(block_tables=torch.zeros(2, 4, dtype=torch.int64)),
    "seq_lens rows": lambda kw: kw.update(seq_lens=torch.zeros(1, dtype=torch.int32)),
    "seq_lens dtype": lambda kw: kw.update(seq_lens=torch.zeros(2, dtype=torch.int64)),
    "recent_k shape": lambda kw: kw.update(recent_k=torch.zeros(2, 1, 16, 128, dtype=torch.bfloat16)),
    "recent_k dtype": lambda kw: kw.update(recent_k=torch.zeros(2, 2, 16, 128, dtype=torch.float32)),
    "recent_v shape": lambda kw: kw.update(recent_v=torch.zeros(2, 2, 8, 128, dtype=torch.bfloat16)),
    "recent_lens dtype": lambda kw: kw.update(recent_lens=torch.zeros(2, dtype=torch.int64)),
    "recent partial": lambda kw: kw.update(recent_v=None),
    "scores_out too narrow": lambda kw: kw.update(scores_out=torch.zeros(2, 8, 40, dtype=torch.float32)),
    "scores_out heads": lambda kw: kw.update(scores_out=torch.zeros(2, 4, 80, dtype=torch.float32)),
    "workspace missing": lambda kw: kw.update(workspace=None),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_mismatched_arguments_are_rejected(on_device, case):
    kw = _valid()
    BAD[case](kw)
    with pytest.raises(ValueError):
        _call(kw)


def test_two_presets_need_int8_seq_preset(on_device):
    kw = _valid(two=True)
    kw["seq_preset"] = None
    with pytest.raises(ValueError, match="seq_preset"):
        _call(kw)
    kw = _valid(two=True)
    kw["seq_preset"] = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError):
        _call(kw)


def test_prepared_decode_validates_once_and_keeps_its_tensors(on_device, monkeypatch):
    """PreparedDecode marshals (and validates) at construction; launching it
    only calls the library with the stored argument struct."""
    calls = []

    class _Lib:
        def tq_decode_attention(self, ref, stream):
            calls.append(("ws", stream))
            return tq.TQ_OK

        def tq_decode_attention_noalloc(self, ref, stream):
            calls.append(("noalloc", stream))
            return tq.TQ_OK

    monkeypatch.setattr(tq, "load", lambda path=None: _Lib())
    kw = _valid()
    q = kw.pop("q")
    ctxs, pools, bt, lens, out = kw.pop("ctxs"), kw.pop("pools"), kw.pop("block_tables"), kw.pop("seq_lens"), kw.pop("out")
    ws = kw.pop("workspace")
    p = tq.PreparedDecode(q, ctxs, pools, bt, lens, out, ws, stream=7, **kw)
    p()
    p()
    assert calls == [("ws", 7), ("ws", 7)]
    assert p._args.q == q.data_ptr() and p._args.workspace == ws.data_ptr()
    pn = tq.PreparedDecode(q, ctxs, pools, bt, lens, out, stream=9, noalloc=True, **kw)
    pn()
    assert calls[-1] == ("noalloc", 9) and not pn._args.workspace
    with pytest.raises(ValueError):
        tq.PreparedDecode(q, ctxs, pools, bt, lens, out, None, stream=7, **kw)  # workspace required
