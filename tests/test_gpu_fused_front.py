"""kvc_block_table_append (block table and append in one launch) against
kvc_block_table followed by kvc_append: block table, free-list head, slots,
cache bytes and lengths bit for bit, for decode-, verify- and prefill-sized
appends into bf16, fp32, FP8 and key-only (MLA latent) pools, and the
all-or-nothing allocation errors."""
import numpy as np
import pytest
import torch

from kv_cached_decode_kvc_amd import kvc, synth
from gpu_harness import GpuCache, i32, to_dev

pytestmark = pytest.mark.gpu

# (name, dtype, kv, D, Hkv, bs, B, cached_hi, new_lo, new_hi, dv)
CASES = [
    ("decode-bf16", "bf16", "", 128, 8, 16, 40, 700, 1, 1, 0),
    ("verify-bf16-bs32", "bf16", "", 128, 2, 32, 9, 300, 5, 5, 0),
    ("prefill-bf16", "bf16", "", 64, 4, 16, 5, 200, 0, 300, 0),
    ("mixed-f32", "f32", "", 64, 2, 16, 12, 100, 0, 20, 0),
    ("decode-fp8", "bf16", "e4m3", 128, 8, 16, 30, 500, 1, 1, 0),
    ("verify-fp8-e5m2", "bf16", "e5m2", 64, 2, 16, 10, 300, 5, 5, 0),
    ("mla-key-only", "bf16", "", 576, 1, 64, 7, 300, 1, 4, 512),
]


def _pair(case, seed=0):
    name, dtype, kv, D, Hkv, bs, B, chi, nlo, nhi, dv = case
    rng = np.random.default_rng(6000 + seed + len(name))
    w = synth.custom(name=name, seed=6100 + seed, B=B, Hq=Hkv, Hkv=Hkv, D=D, dtype=dtype,
                     block_size=bs, n_q=1, len_lo=1, len_hi=chi + nhi + 1, kv=kv, dv=dv)
    cached = rng.integers(0, chi + 1, size=B)
    new = rng.integers(nlo, nhi + 1, size=B)
    cap = int((cached + new).max()) + 2 * bs
    caches = [GpuCache(w, block_size=bs, capacity=cap) for _ in range(2)]
    for gc in caches:
        gc.prefill(cached)
    total = int(new.sum())
    kr = synth.normal(w, (max(total, 1), Hkv, D), synth.S_KNEW, 77, seed)[:total]
    vr = None if dv else synth.normal(w, (max(total, 1), Hkv, D), synth.S_VNEW, 77, seed)[:total]
    return w, caches, new, kr, vr


def _state(gc):
    """Table, free-list head and cache bytes (host copies of the raw bytes)."""
    torch.cuda.synchronize()
    ts = (gc.table, gc.head, gc.k) + ((gc.v,) if gc.v is not None else ())
    return [t.reshape(-1).view(torch.uint8).cpu().numpy().copy() for t in ts]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_equals_two_calls(case):
    w, (ga, gb), new, kr, vr = _pair(case)
    print("fused front", w.name, flush=True)
    cu = i32(synth.cu_from_counts(new))
    total = int(new.sum())
    k_d = to_dev(kr, w.dtype) if total else None
    v_d = to_dev(vr, w.dtype) if (total and vr is not None) else None
    slots_a = torch.full((max(total, 1),), -7, dtype=torch.int32, device="cuda")
    slots_b = slots_a.clone()
    out_a, out_b = torch.empty_like(ga.seq_lens), torch.empty_like(gb.seq_lens)
    mx = int(new.max())
    kvc.kvc_block_table(ga.desc, ga.seq_lens, cu, total, ga.table, ga.free_list, ga.head, ga.head,
                        slots_a, ga.status)
    kvc.kvc_append(ga.desc, k_d, v_d, ga.seq_lens, cu, total, mx, slots_a, ga.k, ga.v, out_a,
                   ga.status)
    kvc.kvc_block_table_append(gb.desc, k_d, v_d, gb.seq_lens, cu, total, mx, gb.table,
                               gb.free_list, gb.head, gb.head, slots_b, gb.k, gb.v, out_b,
                               gb.status)
    assert ga.dev_status() == 0 and gb.dev_status() == 0
    assert torch.equal(slots_a, slots_b)
    assert torch.equal(out_a, out_b)
    for x, y in zip(_state(ga), _state(gb)):
        assert np.array_equal(x, y)


def test_fused_allocation_errors_write_nothing():
    case = CASES[2]  # prefill-sized appends: many new blocks
    w, (ga, gb), new, kr, vr = _pair(case, seed=1)
    cu = i32(synth.cu_from_counts(new))
    total = int(new.sum())
    k_d, v_d = to_dev(kr, w.dtype), to_dev(vr, w.dtype)
    slots = torch.full((total,), -7, dtype=torch.int32, device="cuda")
    out = torch.full_like(gb.seq_lens, -9)
    before = _state(gb)
    # a free-list head near the end of the pool: too few blocks left
    head = i32([gb.N - 1])
    head_out = torch.full((1,), -3, dtype=torch.int32, device="cuda")
    mx = int(new.max())
    kvc.kvc_block_table_append(gb.desc, k_d, v_d, gb.seq_lens, cu, total, mx, gb.table,
                               gb.free_list, head, head_out, slots, gb.k, gb.v, out, gb.status)
    assert gb.dev_status() == -6  # KVC_ERR_NO_BLOCKS
    assert int(head_out.item()) == gb.N - 1
    assert torch.equal(out, gb.seq_lens)
    assert bool((slots == -7).all())
    for x, y in zip(before, _state(gb)):
        assert np.array_equal(x, y)
    # a negative length
    gb.status.zero_()
    bad = gb.seq_lens.clone()
    bad[3] = -1
    kvc.kvc_block_table_append(gb.desc, k_d, v_d, bad, cu, total, mx, gb.table, gb.free_list,
                               gb.head, head_out, slots, gb.k, gb.v, out, gb.status)
    assert gb.dev_status() == -8
    assert torch.equal(out, bad)
    for x, y in zip(before, _state(gb)):
        assert np.array_equal(x, y)
