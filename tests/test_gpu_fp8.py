"""GPU parity of the FP8 cache: codes and scales written by the append equal
the oracle's quantization of the same bf16 rows bit for bit; attention over
the FP8 cache matches the oracle's attention over the exactly dequantized rows
(same tolerance as bf16 caches); block copies carry the scales."""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_cached_decode_kvc_amd import kvc, synth
from gpu_harness import (GpuCache, assert_close, i32, logical_rows, oracle_outputs, queries_dev,
                         to_dev)

pytestmark = pytest.mark.gpu


def gpu_rows(gc, which, b, L):
    """Sequence b's first L rows of the FP8 cache: (codes [Hkv, L, D], scales [Hkv, L])."""
    codes, scales = gc.fp8_rows(which)
    if gc.bs == 0:
        return codes[b, :, :L], scales[b, :, :L]
    table = gc.table.cpu().numpy()
    pos = np.arange(L)
    blk = table[b, pos // gc.bs]
    return (codes[blk, :, pos % gc.bs].transpose(1, 0, 2),
            scales[blk, :, pos % gc.bs].transpose(1, 0))


APPEND_CASES = [  # (fmt, D, block_size, B, len_hi)
    ("e4m3", 128, 0, 4, 90),
    ("e5m2", 128, 16, 5, 120),
    ("e4m3", 64, 32, 3, 200),
    ("e5m2", 64, 0, 3, 70),
]


@pytest.mark.parametrize("fmt,D,bs,B,hi", APPEND_CASES)
def test_append_codes_and_scales_bit_exact(ref, fmt, D, bs, B, hi):
    w = synth.custom(name="q", seed=40 + D + bs, B=B, Hq=4, Hkv=2, D=D, dtype="bf16",
                     block_size=bs, n_q=2, len_lo=2, len_hi=hi, kv=fmt)
    lengths = synth.final_lengths(w)
    cached = lengths - w.n_q
    gc = GpuCache(w, block_size=bs if bs else None)
    gc.prefill(cached)
    gc.step_rows(0)
    assert gc.dev_status() == 0
    for b in range(B):
        for which in ("k", "v"):
            rows = logical_rows(w, b, which, int(cached[b]))
            want_c, want_s = ref.quantize_rows(rows, fmt)
            got_c, got_s = gpu_rows(gc, which, b, int(lengths[b]))
            assert np.array_equal(got_s, want_s), (fmt, b, which)
            assert np.array_equal(got_c, want_c), (fmt, b, which)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_append_edge_rows(ref, fmt):
    """Rows that reach every corner of the encoding: a zero row, magnitudes
    spread over 2^-30 .. 1 (subnormal codes and values that round to zero),
    exact midpoints between neighbouring codes (ties to the even code), and a
    row whose largest element fixes a power-of-two scale."""
    D, Hkv = 128, 1
    rng = np.random.default_rng(90)
    top = ref.fp8_max(fmt)
    vals = ref.fp8_decode(np.arange(256, dtype=np.uint8), fmt)
    finite = [c for c in range(0x80) if np.isfinite(vals[c])]
    rows = [np.zeros(D)]
    for _ in range(6):
        rows.append(rng.standard_normal(D) * np.exp2(rng.uniform(-30, 0, D)))
    for k in range(3):  # midpoints times a power-of-two scale, amax = top * scale
        mids = [(vals[c] + vals[c + 1]) / 2 for c in finite[:-1]]
        r = np.resize(np.array(mids) * rng.choice([-1, 1], len(mids)), D)
        r[0] = top
        rows.append(r * 2.0 ** (-6 - k))
    x = np.array(rows, dtype=np.float64)
    bits = ref.round_bf16(x).reshape(len(rows), Hkv, D)
    w = synth.custom(name="edge", seed=91, B=1, Hq=1, Hkv=Hkv, D=D, dtype="bf16", block_size=0,
                     n_q=1, len_lo=len(rows), len_hi=len(rows), kv=fmt)
    gc = GpuCache(w, capacity=len(rows) + 5)
    gc.add_tokens(bits, bits, [len(rows)])
    assert gc.dev_status() == 0
    want_c, want_s = ref.quantize_rows(bits.transpose(1, 0, 2).copy(), fmt)
    got_c, got_s = gpu_rows(gc, "k", 0, len(rows))
    assert np.array_equal(got_s, want_s)
    assert np.array_equal(got_c, want_c)


# (name, fmt, D, Hq, Hkv, block_size, n_q, len_lo, len_hi, B, partition_tokens, capacity)
ATTN_CASES = [
    ("mha-e4m3-d128-contig", "e4m3", 128, 4, 4, 0, 1, 1, 700, 5, 0, None),
    ("mha-e5m2-d64-contig-cap301", "e5m2", 64, 3, 3, 0, 1, 1, 300, 4, 0, 301),
    ("mha-e4m3-d128-paged", "e4m3", 128, 4, 4, 16, 1, 1, 900, 6, 0, None),
    ("mha-e4m3-d64-paged-P32", "e4m3", 64, 2, 2, 16, 1, 1, 400, 4, 32, None),
    ("gqa4-e4m3-d128-paged", "e4m3", 128, 8, 2, 16, 1, 1, 900, 5, 0, None),
    ("gqa4-e5m2-d128-contig-cap301", "e5m2", 128, 8, 2, 0, 1, 1, 300, 4, 0, 301),
    ("gqa8-e4m3-d64-contig", "e4m3", 64, 8, 1, 0, 1, 1, 700, 3, 0, None),
    ("verify5-gqa4-e4m3-d128-paged", "e4m3", 128, 8, 2, 16, 5, 5, 900, 5, 0, None),
    ("verify5-gqa4-e5m2-d64-paged-P16", "e5m2", 64, 8, 2, 16, 5, 5, 300, 4, 16, None),
    ("verify3-mha-e4m3-d128-contig-cap301", "e4m3", 128, 2, 2, 0, 3, 3, 300, 3, 0, 301),
    # enough sequences that the launch-time partition length lands strictly
    # between its bounds (planned 256 keys, about 208 chosen from these lengths)
    ("verify5-gqa4-e4m3-d128-paged-B40", "e4m3", 128, 32, 8, 16, 5, 5, 2000, 40, 0, None),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_fp8_attention_parity(ref, case):
    name, fmt, D, Hq, Hkv, bs, n_q, lo, hi, B, P, cap = case
    w = synth.custom(name=name, seed=2000 + D + Hq, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16",
                     block_size=bs, n_q=n_q, len_lo=lo, len_hi=hi, kv=fmt)
    lengths = synth.final_lengths(w)
    cached = lengths - n_q
    gc = GpuCache(w, partition_tokens=P, block_size=bs if bs else None, capacity=cap)
    gc.prefill(cached)
    gc.step_rows(0)
    out = gc.attend(queries_dev(w), n_q)
    assert gc.dev_status() == 0
    want = oracle_outputs(ref, w, range(B), cached)
    got = out.cpu().numpy()
    for b in range(B):
        assert_close(got[b], want[b], "%s b=%d L=%d" % (name, b, int(lengths[b])))


def test_fp8_nan_poison_outside_lengths(ref):
    """Codes past every length and in unused blocks hold NaN patterns (and
    their scales NaN): outputs are unchanged."""
    w = synth.custom(name="p", seed=77, B=4, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=16,
                     n_q=1, len_lo=1, len_hi=300, kv="e4m3")
    lengths = synth.final_lengths(w)
    outs = []
    for poison in (False, True):
        gc = GpuCache(w, block_size=16, poison_nan=poison)
        if poison:
            for which in ("k", "v"):
                gc.fp8_parts(which)[1].fill_(float("nan"))
        gc.prefill(lengths - 1)
        gc.step_rows(0)
        outs.append(gc.attend(queries_dev(w), 1))
        assert gc.dev_status() == 0
    assert torch.equal(outs[0], outs[1])


def test_fp8_copy_blocks_carry_scales():
    w = synth.custom(name="c", seed=5, B=1, Hq=8, Hkv=8, D=128, dtype="bf16", block_size=32,
                     n_q=1, kv="e5m2")
    gc = GpuCache(w, block_size=32, capacity=32, pool_blocks=64)
    g = torch.Generator(device="cpu").manual_seed(5)
    gc.k.copy_(torch.randint(0, 256, gc.k.shape, generator=g, dtype=torch.uint8))
    gc.v.copy_(torch.randint(0, 256, gc.v.shape, generator=g, dtype=torch.uint8))
    src = torch.arange(0, 20, dtype=torch.int32)
    dst = torch.arange(40, 60, dtype=torch.int32)
    src[7] = -1
    before = {x: [t.clone() for t in gc.fp8_parts(x)] for x in ("k", "v")}
    kvc.kvc_copy_blocks(gc.desc, src.cuda(), dst.cuda(), 20, gc.k, gc.v, gc.status)
    assert gc.dev_status() == 0
    for x in ("k", "v"):
        codes, scales = gc.fp8_parts(x)
        c0, s0 = before[x]
        wc, ws = c0.clone(), s0.clone()
        for s_, d_ in zip(src.tolist(), dst.tolist()):
            if s_ >= 0:
                wc[d_], ws[d_] = c0[s_], s0[s_]
        assert torch.equal(codes, wc)
        assert torch.equal(scales.view(torch.int32), ws.view(torch.int32))


def test_fp8_parallel_samples_copy_on_write(ref):
    """Sharing on an FP8 pool: prompts forked into samples that then append
    different tokens; copy-on-write copies codes and scales, and every sample's
    attention matches the oracle's attention over its own quantized rows
    (prompt rows, then its new token)."""
    bs, B, fmt = 16, 6, "e4m3"
    w = synth.custom(name="s", seed=88, B=B, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=bs,
                     n_q=1, len_lo=1, len_hi=200, kv=fmt)
    gc = GpuCache(w, block_size=bs, capacity=256, pool_blocks=120)
    refs = torch.zeros(gc.N, dtype=torch.int32, device="cuda")
    prompt = [150, 77, 0, 0, 0, 0]
    gc.prefill(prompt)
    kvc.kvc_fork(gc.desc, i32([0, 0, 1, 1]), i32([2, 3, 4, 5]), 4, gc.seq_lens, gc.table, refs,
                 gc.status)
    rows_k = synth.normal(w, (B, w.Hkv, w.D), synth.S_KNEW, 7)
    rows_v = synth.normal(w, (B, w.Hkv, w.D), synth.S_VNEW, 7)
    src = torch.empty(B, dtype=torch.int32, device="cuda")
    dst = torch.empty(B, dtype=torch.int32, device="cuda")
    kvc.kvc_cow(gc.desc, gc.seq_lens, i32(synth.cu_from_counts([1] * B)), gc.table, gc.free_list,
                gc.head, gc.head, refs, gc.k, gc.v, src, dst, gc.status)
    gc.add_tokens(rows_k, rows_v, [1] * B)
    assert gc.dev_status() == 0
    assert int((src >= 0).sum().item()) == B  # every sharer copied its partly filled block
    q = synth.normal(w, (B, 1, w.Hq, w.D), synth.S_Q, 7)
    got = gc.attend(to_dev(q, "bf16"), 1).cpu().numpy()
    parent = [0, 1, 0, 0, 1, 1]
    for b in range(B):
        pb = parent[b]
        k = np.concatenate([synth.cache_rows(w, "k", pb, prompt[pb]), rows_k[b:b + 1]])
        v = np.concatenate([synth.cache_rows(w, "v", pb, prompt[pb]), rows_v[b:b + 1]])
        kd = ref.dequantize_rows(*ref.quantize_rows(k.transpose(1, 0, 2).copy(), fmt), fmt)
        vd = ref.dequantize_rows(*ref.quantize_rows(v.transpose(1, 0, 2).copy(), fmt), fmt)
        want = ref.attention(oracle.widen(q[b], "bf16"), kd, vd, 1 / math.sqrt(w.D), "f64")
        assert_close(got[b], want, "fp8 sample %d" % b)
