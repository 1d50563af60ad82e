"""GPU parity of decode and verify attention against the CPU oracle.

Tolerance: per element |gpu - oracle| <= max(2e-3, 1e-2 * |oracle|) (bf16
inputs, fp32 accumulation; fp32 output unless stated).  The oracle is evaluated in
float64 on the generator's rows, never on anything the GPU wrote.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvc_amd import kvc, synth
from gpu_harness import (GpuCache, assert_close, i32, logical_rows, oracle_outputs, queries_dev,
                         to_dev)

pytestmark = pytest.mark.gpu

# (name, dtype, D, Hq, Hkv, block_size, n_q, len_lo, len_hi, B, partition_tokens)
CASES = [
    ("mha-bf16-d128-contig", "bf16", 128, 4, 4, 0, 1, 1, 700, 5, 0),
    ("mha-bf16-d64-contig", "bf16", 64, 3, 3, 0, 1, 1, 700, 4, 0),
    ("mha-f32-d64-contig", "f32", 64, 4, 4, 0, 1, 1, 600, 3, 0),
    ("mha-f32-d128-paged", "f32", 128, 2, 2, 16, 1, 1, 600, 4, 0),
    ("mha-bf16-d128-paged", "bf16", 128, 4, 4, 16, 1, 1, 900, 6, 0),
    ("mha-bf16-d128-paged-bs32", "bf16", 128, 2, 2, 32, 1, 1, 500, 3, 0),
    ("gqa4-bf16-d128-paged", "bf16", 128, 8, 2, 16, 1, 1, 900, 5, 0),
    ("gqa8-bf16-d64-contig", "bf16", 64, 8, 1, 0, 1, 1, 700, 3, 0),
    ("gqa4-bf16-d128-contig-P16", "bf16", 128, 8, 2, 0, 1, 1, 300, 4, 16),
    ("mha-bf16-d128-contig-P48", "bf16", 128, 2, 2, 0, 1, 1, 300, 4, 48),
    ("verify5-gqa4-bf16-d128-paged", "bf16", 128, 8, 2, 16, 5, 5, 900, 5, 0),
    ("verify5-mha-bf16-d128-paged", "bf16", 128, 2, 2, 16, 5, 5, 600, 4, 0),
    ("verify2-gqa8-bf16-d64-contig", "bf16", 64, 16, 2, 0, 2, 2, 400, 3, 0),
    ("verify8-gqa4-bf16-d128-paged-rb", "bf16", 128, 8, 1, 16, 8, 8, 500, 3, 0),
    ("verify16-mha-bf16-d64-paged", "bf16", 64, 2, 2, 16, 16, 16, 300, 2, 0),
    ("verify5-f32-d64-paged", "f32", 64, 4, 2, 16, 5, 5, 300, 3, 0),
    ("verify3-gqa4-bf16-d128-P32", "bf16", 128, 8, 2, 16, 3, 3, 200, 4, 32),
    # up to 94 partitions a row: the combine's eight-at-a-time loads and its
    # second pass over partitions beyond 64
    ("mha-bf16-d128-contig-P16-long", "bf16", 128, 4, 4, 0, 1, 1000, 1500, 3, 16),
    ("verify4-gqa4-bf16-d64-paged-P16-long", "bf16", 64, 8, 2, 16, 4, 1000, 1500, 3, 16),
]


def _run_case(ref, case, seed=0, out_dtype=torch.float32):
    name, dtype, D, Hq, Hkv, bs, n_q, lo, hi, B, P = case
    w = synth.custom(name=name, seed=1000 + seed, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     block_size=bs, n_q=n_q, len_lo=lo, len_hi=hi)
    lengths = synth.final_lengths(w)
    cached = lengths - n_q
    gc = GpuCache(w, partition_tokens=P, block_size=bs if bs else None)
    gc.prefill(cached)
    gc.step_rows(0)
    out = gc.attend(queries_dev(w), n_q, out_dtype=out_dtype)
    assert gc.dev_status() == 0
    want = oracle_outputs(ref, w, range(B), cached)
    return w, gc, out, want


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_attention_parity(ref, case):
    w, gc, out, want = _run_case(ref, case)
    got = out.cpu().numpy()
    for b in range(w.B):
        assert_close(got[b], want[b], "%s b=%d L=%d" % (case[0], b, int(gc.seq_lens[b])))


def test_bf16_output(ref):
    """bf16 output: within tolerance of the oracle (one extra bf16 ulp allowed)."""
    case = CASES[6]
    w, gc, out, want = _run_case(ref, case, seed=3, out_dtype=torch.bfloat16)
    got = out.float().cpu().numpy()
    for b in range(w.B):
        assert_close(got[b], want[b], "bf16 out b=%d" % b, bf16_out=True)


def test_tiny_gptlite_32_steps_equal_recompute(ref):
    """Tiny GPTlite-shaped workload (fp32, contiguous, 256 cached tokens): 32
    decode steps of append + attend on the GPU, each step checked against the
    oracle's causal attention recomputed over the whole sequence with no cache.
    The fp32 path stays at the float32 rounding scale (~1e-6, as the online
    softmax worked example prints), far inside the tolerance."""
    w = synth.get("C1")
    cached = synth.cached_lengths(w)
    S = synth.capacity_tokens(w)
    gc = GpuCache(w)
    gc.prefill(cached)
    scale = 1.0 / math.sqrt(w.D)
    outs = []
    for s in range(w.steps):
        gc.step_rows(s)
        outs.append(gc.attend(queries_dev(w, s), 1).cpu().numpy())
    assert gc.dev_status() == 0
    worst = 0.0
    for b in range(w.B):
        k = logical_rows(w, b, "k", int(cached[b]), w.steps)
        v = logical_rows(w, b, "v", int(cached[b]), w.steps)
        qfull = np.zeros((S, w.Hq, w.D), np.float32)
        for s in range(w.steps):
            qfull[cached[b] + s] = synth.queries(w, b, s)[0]
        full = ref.attention(qfull, k, v, scale, "f32")  # causal over all S positions
        for s in range(w.steps):
            worst = max(worst, assert_close(outs[s][b, 0], full[cached[b] + s], "step %d" % s))
    assert worst < 2e-5, worst


def test_paged_equals_contiguous_bitwise():
    """Same rows, same partition length: the paged cache read through a permuted
    block table gives bit-identical outputs to the contiguous cache."""
    for n_q, Hq, Hkv in ((1, 4, 4), (1, 8, 2), (5, 8, 2)):
        w = synth.custom(seed=11, B=6, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", block_size=16, n_q=n_q,
                         len_lo=n_q, len_hi=777)
        lengths = synth.final_lengths(w)
        cap = synth.capacity_tokens(w)
        outs = []
        for bs in (0, 16):
            wc = synth.custom(seed=11, B=6, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", block_size=bs,
                              n_q=n_q, len_lo=n_q, len_hi=777)
            gc = GpuCache(wc, partition_tokens=64, block_size=bs if bs else None, capacity=cap)
            gc.prefill(lengths - n_q)
            gc.step_rows(0)
            outs.append(gc.attend(queries_dev(wc), n_q))
            assert gc.dev_status() == 0
        assert torch.equal(outs[0], outs[1])


def test_nan_poisoned_unused_slots(ref):
    """Every cache slot beyond a sequence's length, and every pool block never
    handed out, holds NaN: outputs are unchanged (the mask stops at the length)."""
    for bs in (0, 16):
        for n_q, Hq, Hkv in ((1, 4, 4), (1, 8, 2), (5, 8, 2)):
            w = synth.custom(seed=12, B=4, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16", block_size=bs,
                             n_q=n_q, len_lo=n_q, len_hi=500)
            lengths = synth.final_lengths(w)
            res = []
            for poison in (False, True):
                gc = GpuCache(w, block_size=bs if bs else None, poison_nan=poison)
                gc.prefill(lengths - n_q)
                gc.step_rows(0)
                res.append(gc.attend(queries_dev(w), n_q))
            assert torch.equal(res[0], res[1]) and bool(torch.isfinite(res[1]).all())


def test_verify_rows_equal_decodes():
    """Verify row r equals a decode over the first L - n_q + r + 1 keys (within
    tolerance: a different grouping of the same keys)."""
    w = synth.custom(seed=13, B=4, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=16, n_q=5,
                     len_lo=5, len_hi=700)
    lengths = synth.final_lengths(w)
    gc = GpuCache(w, block_size=16)
    gc.prefill(lengths - 5)
    gc.step_rows(0)
    q = queries_dev(w)
    ver = gc.attend(q, 5).cpu().numpy()
    for r in range(5):
        cut = gc.seq_lens - 5 + r + 1
        dec = gc.attend(q[:, r:r + 1].contiguous(), 1, seq_lens=cut).cpu().numpy()
        assert_close(ver[:, r], dec[:, 0].astype(np.float64), "row %d" % r)


def test_edge_lengths(ref):
    """Lengths 1, 15, 16, 17, a partition multiple, and the full capacity."""
    for bs in (0, 16):
        w = synth.custom(seed=14, B=7, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=bs, n_q=1,
                         len_lo=1, len_hi=1)
        lengths = np.array([1, 15, 16, 17, 256, 257, 512], np.int32)
        gc = GpuCache(w, partition_tokens=256, block_size=bs if bs else None, capacity=512)
        gc.prefill(lengths - 1)
        gc.step_rows(0)
        out = gc.attend(queries_dev(w), 1).cpu().numpy()
        assert gc.dev_status() == 0
        want = oracle_outputs(ref, w, range(w.B), lengths - 1)
        for b in range(w.B):
            assert_close(out[b], want[b], "L=%d" % lengths[b])
        # L = 1: the output is the single value row of the head's group
        v0 = oracle.widen(logical_rows(w, 0, "v", 0, 1)[:, 0], w.dtype)  # [Hkv, D]
        np.testing.assert_allclose(out[0, 0], np.repeat(v0, w.G, axis=0), rtol=0, atol=1e-6)


def test_verify_with_empty_cache_is_causal(ref):
    """n_q = L: ordinary causal attention over the new rows only."""
    w = synth.custom(seed=15, B=3, Hq=4, Hkv=2, D=64, dtype="bf16", block_size=16, n_q=9,
                     len_lo=9, len_hi=9)
    gc = GpuCache(w, block_size=16)
    gc.step_rows(0)
    out = gc.attend(queries_dev(w), 9).cpu().numpy()
    want = oracle_outputs(ref, w, range(3), np.zeros(3, np.int32))
    for b in range(3):
        assert_close(out[b], want[b])


def test_values_all_one_give_one():
    """Softmax rows sum to one: with every value row equal to 1 the output is 1."""
    w = synth.custom(seed=16, B=3, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=16, n_q=5,
                     len_lo=5, len_hi=600)
    lengths = synth.final_lengths(w)
    gc = GpuCache(w, block_size=16)
    gc.prefill(lengths - 5)
    gc.step_rows(0)
    gc.v.fill_(1.0)
    out = gc.attend(queries_dev(w), 5)
    assert float((out - 1).abs().max()) <= 1e-5  # weights and their sum use the same rounding


def test_bad_block_id_reports_and_does_not_fault():
    w = synth.custom(seed=17, B=2, Hq=4, Hkv=4, D=128, dtype="bf16", block_size=16, n_q=1,
                     len_lo=40, len_hi=40)
    gc = GpuCache(w, block_size=16)
    gc.prefill([39, 39])
    gc.step_rows(0)
    gc.table[1, 1] = gc.N + 5  # outside the pool
    out = gc.attend(queries_dev(w), 1)
    assert gc.dev_status() == -8
    assert bool(torch.isfinite(out).all())


def test_length_beyond_capacity_reports():
    w = synth.custom(seed=18, B=2, Hq=4, Hkv=1, D=64, dtype="bf16", block_size=0, n_q=1,
                     len_lo=10, len_hi=10)
    gc = GpuCache(w, capacity=32)
    gc.prefill([9, 9])
    gc.step_rows(0)
    bad = i32([10, 33])
    out = gc.attend(queries_dev(w), 1, seq_lens=bad)
    assert gc.dev_status() == -8
    assert float(out[1].abs().max()) == 0.0  # invalid sequence gives zeros


def test_workspace_too_small_is_refused():
    w = synth.custom(seed=19, B=2, Hq=4, Hkv=4, D=128, dtype="bf16", block_size=0, n_q=1,
                     len_lo=10, len_hi=10)
    gc = GpuCache(w)
    q = queries_dev(w)
    out = torch.empty((2, 1, 4, 128), dtype=torch.float32, device="cuda")
    small = torch.empty(4, dtype=torch.float32, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_decode_attn(gc.desc, q, gc.k, gc.v, gc.seq_lens, None, 0.1, out, small)
    assert e.value.status == -4


@pytest.mark.parametrize("n_q", [1, 5])
def test_peaked_weights_large_values(ref, n_q):
    """Matrix-core path on short contexts where a few keys take nearly all the
    weight and value rows are large (|v| up to ~16): the error the weights
    carry into the value product shows up undamped here, so this case bounds
    the precision of the probabilities in that product."""
    D, Hq, Hkv, B = 128, 8, 2, 24
    w = synth.custom(name="peaked", seed=31 + n_q, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                     block_size=0, n_q=n_q, len_lo=n_q, len_hi=40)
    lengths = synth.final_lengths(w)
    rng = np.random.default_rng(4242 + n_q)
    total = int(lengths.sum())
    k = synth.to_bf16_bits(rng.standard_normal((total, Hkv, D), dtype=np.float32))
    v = synth.to_bf16_bits(4.0 * rng.standard_normal((total, Hkv, D), dtype=np.float32))
    q = synth.to_bf16_bits(rng.standard_normal((B, n_q, Hq, D), dtype=np.float32))
    scale = 3.0 / math.sqrt(D)  # scores spread ~3x wider than 1/sqrt(D) gives
    gc = GpuCache(w, capacity=48)
    gc.add_tokens(k, v, lengths)
    got = gc.attend(to_dev(q, "bf16"), n_q, scale=scale).cpu().numpy()
    assert gc.dev_status() == 0
    kc = np.zeros((B, Hkv, 48, D), np.uint16)
    vc = np.zeros_like(kc)
    st, lens = ref.append(k, v, np.zeros(B, np.int32), synth.cu_from_counts(lengths), kc, vc)
    assert st == 0
    st, want = ref.cache_attention(q, kc, vc, lens, scale, "bf16")
    assert st == 0
    assert_close(got, want, "peaked n_q=%d" % n_q)


@pytest.mark.parametrize("dv", [0, 512])
def test_stale_workspace_bytes_do_not_matter(dv):
    """The reduce requests every partition slot of a row before it knows the
    row's partition count and discards the extra slots by selection: a
    workspace full of NaN (stale bytes) past its counter region (which must
    be zero) gives the same outputs bit for bit.  Lengths from 1 to 700 with
    32-key partitions give rows with 1 to 22 partitions (past the 16 the
    reduce fetches early) next to unused slots."""
    if dv:
        w = synth.custom(name="ws-mla", seed=77, B=5, Hq=16, Hkv=1, D=576, dtype="bf16",
                         block_size=64, n_q=1, len_lo=1, len_hi=700, dv=512)
    else:
        w = synth.custom(name="ws", seed=77, B=5, Hq=8, Hkv=2, D=128, dtype="bf16",
                         block_size=16, n_q=1, len_lo=1, len_hi=700)
    lengths = synth.final_lengths(w)
    for P in (32, 0):
        gc = GpuCache(w, partition_tokens=P)
        gc.prefill(lengths - 1)
        gc.step_rows(0)
        q = queries_dev(w)
        outs = []
        for fill in (0.0, float("nan")):
            ws = gc.workspace(1)
            ws.fill_(fill)
            ws[:(256 << 10) // 4].zero_()  # the combine counters
            out = torch.empty((w.B, 1, w.Hq, w.out_dim), dtype=torch.float32, device="cuda")
            if dv:
                kvc.kvc_mla_attn(gc.desc, q, 1, gc.k, gc.seq_lens, gc.table, dv, gc.scale, out, ws,
                                 gc.status)
            else:
                kvc.kvc_decode_attn(gc.desc, q, gc.k, gc.v, gc.seq_lens, gc.table, gc.scale, out,
                                    ws, gc.status)
            outs.append(out)
        assert gc.dev_status() == 0
        assert bool(torch.isfinite(outs[1]).all()), P
        assert torch.equal(outs[0], outs[1]), P


@pytest.mark.parametrize("B,n_q,lo,hi,bs", [(300, 1, 1, 40, 16), (1, 5, 5000, 5000, 0),
                                            (40, 5, 5, 2000, 32)])
def test_stream_k_split(ref, B, n_q, lo, hi, bs):
    """The matrix-core path's default (stream-K) split: workers whose runs
    cross many short segments (300 sequences of 1-40 keys: about 150 workers
    of 8 tiles, each spanning several sequences), one long sequence shared by
    many workers, and a mixed verify batch; every row against the oracle."""
    w = synth.custom(name="sk", seed=900 + B + n_q, B=B, Hq=8, Hkv=2, D=128, dtype="bf16",
                     block_size=bs, n_q=n_q, len_lo=lo, len_hi=hi)
    lengths = synth.final_lengths(w)
    gc = GpuCache(w, block_size=bs if bs else None)
    assert kvc.kvc_attn_partition_tokens(gc.desc, n_q) == 0
    gc.prefill(lengths - n_q)
    gc.step_rows(0)
    out = gc.attend(queries_dev(w), n_q)
    assert gc.dev_status() == 0
    want = oracle_outputs(ref, w, range(B), lengths - n_q)
    got = out.cpu().numpy()
    for b in range(B):
        assert_close(got[b], want[b], "sk B=%d b=%d L=%d" % (B, b, lengths[b]))


# (dtype, D, Hq, Hkv, n_q, len_lo, len_hi, B, block_size): paged batches whose
# fixed partitions would need more than one round of work items
VALU_SK = [
    ("bf16", 128, 16, 16, 1, 1, 2000, 70, 16),   # two 64-sequence chunks of the scans
    ("f32", 64, 8, 4, 3, 3, 2000, 40, 32),       # grouped fp32 heads, verify rows
    ("bf16", 64, 12, 12, 1, 1, 40, 400, 16),     # workers spanning many short segments
]


@pytest.mark.parametrize("case", VALU_SK, ids=["-".join(map(str, c)) for c in VALU_SK])
def test_valu_stream_k_split(ref, case):
    """The vector-ALU kernel's stream-K split (paged bf16 / fp32 caches too
    large for one round of work items): lengths of 1, 15, 16, 17, 31 and 32
    keys among random ones, rows of a KV head in (query row, head) order,
    every row against the oracle."""
    dtype, D, Hq, Hkv, n_q, lo, hi, B, bs = case
    w = synth.custom(name="vsk", seed=950 + B, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     block_size=bs, n_q=n_q, len_lo=lo, len_hi=hi)
    cached = synth.final_lengths(w) - n_q
    edge = np.array([1, 15, 16, 17, 31, 32]) - n_q
    cached[:len(edge)] = np.maximum(edge, 0)
    gc = GpuCache(w, block_size=bs)
    assert kvc.kvc_attn_partition_tokens(gc.desc, n_q) == 0
    gc.prefill(cached)
    gc.step_rows(0)
    out = gc.attend(queries_dev(w), n_q)
    assert gc.dev_status() == 0
    want = oracle_outputs(ref, w, range(B), cached)
    got = out.cpu().numpy()
    for b in range(B):
        assert_close(got[b], want[b], "vsk %s b=%d L=%d" % (dtype, b, cached[b] + n_q))


def test_valu_stream_k_bad_block_reports_and_does_not_fault():
    dtype, D, Hq, Hkv, n_q, lo, hi, B, bs = VALU_SK[0]
    w = synth.custom(name="vskbad", seed=960, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     block_size=bs, n_q=n_q, len_lo=lo, len_hi=hi)
    cached = synth.final_lengths(w) - n_q
    cached[3] = 100
    gc = GpuCache(w, block_size=bs)
    assert kvc.kvc_attn_partition_tokens(gc.desc, n_q) == 0
    gc.prefill(cached)
    gc.step_rows(0)
    gc.table[3, 2] = gc.N + 5  # outside the pool
    out = gc.attend(queries_dev(w), n_q)
    assert gc.dev_status() == -8
    assert bool(torch.isfinite(out).all())
