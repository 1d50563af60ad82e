"""The one-call decode / verify entry points against the two-stage calls, and
the combine fused into the vector-ALU partition launch ([I1] "FlashDecoding":
the partials of a row are merged with the online-softmax rescaling; here the
work item that finishes a row's last partition does it, counting partitions
in the workspace).  The matrix-core (stream-K) cases run the separate reduce
and check that the one-call path and a shared workspace leave the counters
alone.

Checked: every row against the oracle (tolerance max(2e-3, 1e-2 * |oracle|)),
the one-call result against the two-stage calls, the counter region left at
zero after every call (whatever other calls share the workspace), bit-identical
outputs from repeated calls, and the rows of sequences with unusable lengths.
"""
import numpy as np
import pytest
import torch

from kv_cached_decode_kvc_amd import kvc, synth
from gpu_harness import GpuCache, assert_close, oracle_outputs, queries_dev

pytestmark = pytest.mark.gpu

CNT_WORDS = (256 << 10) // 4  # the counter region at the start of every workspace

# (name, dtype, D, Hq, Hkv, block_size, n_q, len_lo, len_hi, B, kv)
CASES = [
    ("mha-bf16-d128-contig", "bf16", 128, 4, 4, 0, 1, 1, 900, 6, ""),       # vector ALU, per row
    ("mha-f32-d64-paged", "f32", 64, 4, 4, 16, 1, 1, 600, 5, ""),
    ("verify5-mha-bf16-paged", "bf16", 128, 2, 2, 16, 5, 5, 700, 4, ""),
    ("mha-fp8e4m3-d128-paged", "bf16", 128, 4, 4, 16, 1, 1, 800, 4, "e4m3"),
    ("gqa4-bf16-d128-paged", "bf16", 128, 8, 2, 16, 1, 1, 900, 7, ""),      # stream-K: separate reduce
    ("verify5-gqa4-bf16-paged", "bf16", 128, 8, 2, 16, 5, 5, 900, 6, ""),
    ("gqa8-bf16-d64-contig-long", "bf16", 64, 8, 1, 0, 1, 1, 6000, 3, ""),  # segments over many workers
    ("verify3-gqa4-fp8e5m2-paged", "bf16", 128, 8, 2, 16, 3, 3, 700, 5, "e5m2"),
]


def _build(case, seed=0):
    name, dtype, D, Hq, Hkv, bs, n_q, lo, hi, B, kv = case
    w = synth.custom(name=name, seed=3000 + seed, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     block_size=bs, n_q=n_q, len_lo=lo, len_hi=hi, kv=kv)
    lengths = synth.final_lengths(w)
    cached = lengths - n_q
    gc = GpuCache(w, block_size=bs if bs else None)
    gc.prefill(cached)
    gc.step_rows(0)
    return w, gc, cached


def _one_call(gc, q, n_q, ws, lens=None):
    w = gc.w
    out = torch.empty((w.B, n_q, w.Hq, w.D), dtype=torch.float32, device="cuda")
    kvc.kvc_verify_attn(gc.desc, q, n_q, gc.k, gc.v, gc.seq_lens if lens is None else lens,
                        gc.table, gc.scale, out, ws, gc.status)
    return out


def _counters_zero(ws):
    torch.cuda.synchronize()
    return int(torch.count_nonzero(ws[:CNT_WORDS].view(torch.int32)).item()) == 0


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_one_call_equals_oracle_and_two_stage(ref, case):
    w, gc, cached = _build(case)
    n_q = w.n_q
    # one launch: one query row per KV row (vector ALU), a small grid
    one = w.dtype == "f32" or (w.Hq == w.Hkv and n_q == 1)
    assert kvc.kvc_attn_launches(gc.desc, n_q) == (1 if one else 2)
    q = queries_dev(w)
    ws = gc.workspace(n_q)
    fused = _one_call(gc, q, n_q, ws)
    assert gc.dev_status() == 0
    assert _counters_zero(ws)
    ws2 = gc.workspace(n_q)
    two = torch.empty_like(fused)
    gc.partition(q, n_q, gc.seq_lens, ws2)
    gc.reduce(n_q, gc.seq_lens, ws2, two)
    assert gc.dev_status() == 0
    want = oracle_outputs(ref, w, range(w.B), cached)
    f, t = fused.cpu().numpy(), two.cpu().numpy()
    for b in range(w.B):
        assert_close(f[b], want[b], "%s one call b=%d" % (w.name, b))
        assert_close(t[b], want[b], "%s two stages b=%d" % (w.name, b))
    # the two combines differ only in the order of their sums
    assert float(np.abs(f - t).max()) <= 1e-5 * max(1.0, float(np.abs(t).max()))


def test_shared_workspace_any_shape_and_repeatable(ref):
    """One workspace serves every case in turn (and, in between, an MLA call
    and two-stage calls of other shapes, which must leave the counters
    alone); every one-call result is bit-identical to the same call on a
    fresh workspace and to itself repeated, and the counters are zero after
    each call."""
    built = [_build(c, seed=1) for c in CASES]
    need = max(kvc.kvc_attn_workspace_bytes(gc.desc, w.n_q) for w, gc, _ in built)
    mla = synth.custom(name="ws-mla", seed=77, B=3, Hq=16, Hkv=1, D=576, dtype="bf16",
                       block_size=64, n_q=1, len_lo=1, len_hi=700, dv=512)
    mc = GpuCache(mla)
    mc.prefill(synth.final_lengths(mla) - 1)
    mc.step_rows(0)
    need = max(need, kvc.kvc_mla_workspace_bytes(mc.desc, 1, 512))
    shared = torch.zeros(need // 4 + 1, dtype=torch.float32, device="cuda")
    fresh = {}
    for w, gc, _ in built:
        fresh[w.name] = _one_call(gc, queries_dev(w), w.n_q, gc.workspace(w.n_q))
    for rnd in range(2):
        for i, (w, gc, cached) in enumerate(built):
            got = _one_call(gc, queries_dev(w), w.n_q, shared)
            assert gc.dev_status() == 0
            assert _counters_zero(shared), (w.name, rnd)
            assert torch.equal(got, fresh[w.name]), (w.name, rnd)
            # something of another shape in between: MLA, then a two-stage call
            mo = torch.empty((mla.B, 1, mla.Hq, 512), dtype=torch.float32, device="cuda")
            kvc.kvc_mla_attn(mc.desc, queries_dev(mla), 1, mc.k, mc.seq_lens, mc.table, 512,
                             mc.scale, mo, shared, mc.status)
            ow, og, _ = built[(i + 3) % len(built)]
            two = torch.empty((ow.B, ow.n_q, ow.Hq, ow.D), dtype=torch.float32, device="cuda")
            og.partition(queries_dev(ow), ow.n_q, og.seq_lens, shared)
            og.reduce(ow.n_q, og.seq_lens, shared, two)
            assert mc.dev_status() == 0 and og.dev_status() == 0
            assert _counters_zero(shared), (w.name, rnd, "after other shapes")
    for w, gc, cached in built[:3]:
        want = oracle_outputs(ref, w, range(w.B), cached)
        got = fresh[w.name].cpu().numpy()
        for b in range(w.B):
            assert_close(got[b], want[b], "%s b=%d" % (w.name, b))


@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[5]], ids=["valu", "sk16", "sk32"])
def test_unusable_length_gives_zero_rows(ref, case):
    """A length past the capacity: that sequence's rows are zeros, the status
    says KVC_ERR_DATA, the counters end at zero and the next call on the same
    workspace, with good lengths, is right."""
    w, gc, cached = _build(case, seed=2)
    ws = gc.workspace(w.n_q)
    bad = gc.seq_lens.clone()
    bad[1] = gc.cap + 1
    out = _one_call(gc, queries_dev(w), w.n_q, ws, lens=bad)
    assert gc.dev_status() == -8
    assert _counters_zero(ws)
    got = out.cpu().numpy()
    assert float(np.abs(got[1]).max()) == 0.0
    want = oracle_outputs(ref, w, [b for b in range(w.B) if b != 1], cached)
    for b, o in want.items():
        assert_close(got[b], o, "%s b=%d next to a bad length" % (w.name, b))
    gc.status.zero_()
    out = _one_call(gc, queries_dev(w), w.n_q, ws).cpu().numpy()
    assert gc.dev_status() == 0
    want = oracle_outputs(ref, w, [1], cached)
    assert_close(out[1], want[1], "%s b=1 after the bad call" % w.name)
