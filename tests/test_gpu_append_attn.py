"""kvc_append_attn (append and attention in one call on a contiguous cache)
against kvc_append followed by kvc_verify_attn: outputs bit for bit, cache
bytes and lengths; the fused partition launch (one query row per KV row, bf16
and fp32) and the append-first path (grouped rows, FP8); a refused append."""
import math

import numpy as np
import pytest
import torch

from kv_cached_decode_kvc_amd import kvc, synth
from gpu_harness import GpuCache, assert_close, i32, oracle_outputs, queries_dev, to_dev

pytestmark = pytest.mark.gpu

# (name, dtype, kv, D, Hq, Hkv, B, n_q, new_lo, new_hi, len_hi)
CASES = [
    ("gptlite-f32-decode", "f32", "", 64, 4, 4, 2, 1, 1, 1, 300),
    ("mha-bf16-decode", "bf16", "", 128, 4, 4, 6, 1, 1, 1, 900),
    ("mha-bf16-verify5", "bf16", "", 128, 3, 3, 5, 5, 5, 5, 700),
    ("mha-bf16-d64-chunks", "bf16", "", 64, 2, 2, 4, 3, 3, 40, 500),
    ("gqa-bf16-verify", "bf16", "", 128, 8, 2, 4, 5, 5, 5, 600),
    ("mha-fp8-decode", "bf16", "e4m3", 128, 4, 4, 4, 1, 1, 1, 600),
]


def _caches(case, seed=0):
    name, dtype, kv, D, Hq, Hkv, B, n_q, nlo, nhi, hi = case
    rng = np.random.default_rng(7000 + seed + len(name))
    w = synth.custom(name=name, seed=7100 + seed, B=B, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     block_size=0, n_q=n_q, len_lo=1, len_hi=hi, kv=kv)
    cached = rng.integers(1, hi + 1, size=B)
    new = rng.integers(nlo, nhi + 1, size=B)
    cap = int((cached + new).max()) + 5
    gcs = [GpuCache(w, capacity=cap) for _ in range(2)]
    for gc in gcs:
        gc.prefill(cached)
    total = int(new.sum())
    kr = synth.normal(w, (total, Hkv, D), synth.S_KNEW, 88, seed)
    vr = synth.normal(w, (total, Hkv, D), synth.S_VNEW, 88, seed)
    q = synth.normal(w, (B, n_q, Hq, D), synth.S_Q, 88, seed)
    return w, gcs, cached, new, kr, vr, q


def _bytes(t):
    return t.reshape(-1).view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_append_attn_equals_two_calls(ref, case):
    w, (ga, gb), cached, new, kr, vr, q = _caches(case)
    print("append+attn", w.name, flush=True)
    n_q = w.n_q
    cu = i32(synth.cu_from_counts(new))
    total, mx = int(new.sum()), int(new.max())
    k_d, v_d, q_d = to_dev(kr, w.dtype), to_dev(vr, w.dtype), to_dev(q, w.dtype)
    scale = 1.0 / math.sqrt(w.D)
    out_a = torch.full((w.B, n_q, w.Hq, w.D), float("nan"), device="cuda")
    out_b = out_a.clone()
    lens_a, lens_b = torch.empty_like(ga.seq_lens), torch.empty_like(gb.seq_lens)
    kvc.kvc_append(ga.desc, k_d, v_d, ga.seq_lens, cu, total, mx, None, ga.k, ga.v, lens_a,
                   ga.status)
    kvc.kvc_verify_attn(ga.desc, q_d, n_q, ga.k, ga.v, lens_a, None, scale, out_a,
                        ga.workspace(n_q), ga.status)
    kvc.kvc_append_attn(gb.desc, k_d, v_d, gb.seq_lens, cu, total, mx, gb.k, gb.v, lens_b, q_d,
                        n_q, scale, out_b, gb.workspace(n_q), gb.status)
    assert ga.dev_status() == 0 and gb.dev_status() == 0
    assert torch.equal(lens_a, lens_b)
    assert torch.equal(out_a, out_b)
    assert np.array_equal(_bytes(ga.k), _bytes(gb.k))
    assert np.array_equal(_bytes(ga.v), _bytes(gb.v))
    if not w.kv:  # the fused outputs against the oracle too
        got = out_b.cpu().numpy()
        cu_h = synth.cu_from_counts(new)
        for b in range(w.B):
            k = np.concatenate([synth.cache_rows(w, "k", b, int(cached[b])),
                                kr[cu_h[b]:cu_h[b + 1]]]).transpose(1, 0, 2).copy()
            v = np.concatenate([synth.cache_rows(w, "v", b, int(cached[b])),
                                vr[cu_h[b]:cu_h[b + 1]]]).transpose(1, 0, 2).copy()
            want = ref.attention(q[b], k, v, scale, w.dtype)
            assert_close(got[b], want, "%s b=%d" % (w.name, b))


def test_append_attn_refused_append_keeps_length():
    case = CASES[1]
    w, (ga, gb), cached, new, kr, vr, q = _caches(case, seed=1)
    cu = i32(synth.cu_from_counts(new))
    total = int(new.sum())
    k_d, v_d, q_d = to_dev(kr, w.dtype), to_dev(vr, w.dtype), to_dev(q, w.dtype)
    cap = gb.cap
    lens0 = gb.seq_lens.clone()
    lens0[2] = cap  # full: its new row would pass the capacity
    out = torch.zeros((w.B, 1, w.Hq, w.D), device="cuda")
    lens1 = torch.empty_like(lens0)
    kvc.kvc_append_attn(gb.desc, k_d, v_d, lens0, cu, total, 1, gb.k, gb.v, lens1, q_d, 1, 0.1,
                        out, gb.workspace(1), gb.status)
    assert gb.dev_status() == -5  # KVC_ERR_CAPACITY
    assert int(lens1[2].item()) == cap
    want = (lens0 + i32(new)).cpu().numpy()
    got = lens1.cpu().numpy()
    for b in range(w.B):
        if b != 2:
            assert got[b] == want[b]
