"""GPU parity of the block lifecycle: fork, copy-on-write, truncate and block
copies must leave tables, reference counts, free list, head, lengths and pool
bytes equal to the oracle's bit for bit, after every operation; attention over
shared and copied blocks must match the oracle's attention."""
import numpy as np
import pytest
import torch

from kv_cached_decode_kvc_amd import kvc, synth
from gpu_harness import GpuCache, assert_close, i32, to_dev, to_host_bits

pytestmark = pytest.mark.gpu


class Twin:
    """One paged cache held twice: on the device (through the C ABI) and in the
    oracle (numpy), driven by the same operations."""

    def __init__(self, ref, w, capacity, pool_blocks):
        self.ref, self.w = ref, w
        self.gc = GpuCache(w, block_size=w.block_size, capacity=capacity, pool_blocks=pool_blocks)
        gc = self.gc
        self.refs = torch.zeros(gc.N, dtype=torch.int32, device="cuda")
        self.src = torch.empty(w.B, dtype=torch.int32, device="cuda")
        self.dst = torch.empty(w.B, dtype=torch.int32, device="cuda")
        nd = np.uint16 if w.dtype == "bf16" else np.float32
        self.o_k = np.zeros((gc.N, w.Hkv, gc.bs, w.D), nd)
        self.o_v = np.zeros_like(self.o_k)
        self.o_table = np.full((w.B, gc.max_blocks), -1, np.int32)
        self.o_free = gc.free_host.copy()
        self.o_head = 0
        self.o_refs = np.zeros(gc.N, np.int32)
        self.o_lens = np.zeros(w.B, np.int32)
        self.o_src = np.full(w.B, -1, np.int32)
        self.o_dst = np.full(w.B, -1, np.int32)
        self.n_rows = 0

    def append(self, counts, cow=True):
        """Copy-on-write (optional), block allocation and append of fresh rows."""
        w, gc, ref = self.w, self.gc, self.ref
        counts = np.asarray(counts, np.int64)
        cu = synth.cu_from_counts(counts)
        total = int(cu[-1])
        kr = synth.normal(w, (total, w.Hkv, w.D), synth.S_KNEW, 991, self.n_rows)
        vr = synth.normal(w, (total, w.Hkv, w.D), synth.S_VNEW, 991, self.n_rows)
        self.n_rows += 1
        st = 0
        if cow:
            kvc.kvc_cow(gc.desc, gc.seq_lens, i32(cu), gc.table, gc.free_list, gc.head, gc.head,
                        self.refs, gc.k, gc.v, self.src, self.dst, gc.status)
            st, self.o_table, self.o_free, self.o_head, self.o_refs, self.o_src, self.o_dst = \
                ref.cow(self.o_lens, cu, self.o_table, self.o_free, self.o_head, self.o_refs,
                        self.o_k, self.o_v, gc.bs)
            if st != 0:
                return st
        st, o_table, o_head, slots = ref.block_table(self.o_lens, cu, self.o_table, self.o_free,
                                                     self.o_head, gc.bs)
        if st != 0:  # the device refuses the same allocation; no append follows
            dummy = torch.empty(max(total, 1), dtype=torch.int32, device="cuda")
            kvc.kvc_block_table(gc.desc, gc.seq_lens, i32(cu), total, gc.table, gc.free_list,
                                gc.head, gc.head, dummy, gc.status)
            return st
        self.o_table, self.o_head = o_table, o_head
        gc.add_tokens(kr, vr, counts)
        st, self.o_lens = ref.append(kr, vr, self.o_lens, cu, self.o_k, self.o_v, bs=gc.bs,
                                     slots=slots)
        return st

    def fork(self, parents, children):
        gc = self.gc
        kvc.kvc_fork(gc.desc, i32(parents), i32(children), len(parents), gc.seq_lens, gc.table,
                     self.refs, gc.status)
        st, self.o_lens, self.o_table, self.o_refs = self.ref.fork(
            parents, children, self.o_lens, self.o_table, self.o_refs, gc.bs, gc.N)
        return st

    def truncate(self, new_lens, with_refs=True):
        gc = self.gc
        out = torch.empty_like(gc.seq_lens)
        kvc.kvc_truncate(gc.desc, gc.seq_lens, i32(new_lens), gc.table, gc.free_list, gc.head,
                         gc.head, self.refs if with_refs else None, out, gc.status)
        st, self.o_table, self.o_free, self.o_head, o_refs, o_lens = self.ref.truncate(
            self.o_lens, new_lens, self.o_table, self.o_free, self.o_head,
            self.o_refs if with_refs else None, gc.bs)
        if st == 0:
            gc.seq_lens = out
            self.o_lens = o_lens
            if with_refs:
                self.o_refs = o_refs
        return st

    def check(self, what, pools=True, cow_pairs=False):
        gc = self.gc
        torch.cuda.synchronize()
        assert gc.dev_status() == 0, what
        assert np.array_equal(gc.table.cpu().numpy(), self.o_table), what
        assert np.array_equal(self.refs.cpu().numpy(), self.o_refs), what
        assert np.array_equal(gc.free_list.cpu().numpy(), self.o_free), what
        assert int(gc.head.item()) == self.o_head, what
        assert np.array_equal(gc.seq_lens.cpu().numpy(), self.o_lens), what
        if cow_pairs:
            assert np.array_equal(self.src.cpu().numpy(), self.o_src), what
            assert np.array_equal(self.dst.cpu().numpy(), self.o_dst), what
        if pools:
            assert np.array_equal(to_host_bits(gc.k), self.o_k), what
            assert np.array_equal(to_host_bits(gc.v), self.o_v), what


@pytest.mark.parametrize("seed", range(4))
def test_lifecycle_random_ops(ref, seed):
    """Random appends (with copy-on-write), forks of several sequences at once
    and truncations, on a pool small enough to run near empty."""
    rng = np.random.default_rng(700 + seed)
    dtype = "bf16" if seed % 2 == 0 else "f32"
    bs = 16 if seed < 2 else 32
    w = synth.custom(seed=seed, B=7, Hq=4, Hkv=2, D=64 if seed % 3 else 128, dtype=dtype,
                     block_size=bs, n_q=1)
    cap = 6 * bs
    t = Twin(ref, w, capacity=cap, pool_blocks=30)
    assert t.append([int(x) for x in rng.integers(1, 2 * bs, size=3)] + [0] * 4) == 0
    t.check("prefill", cow_pairs=True)
    for step in range(30):
        op = int(rng.integers(0, 3))
        lens = t.o_lens
        if op == 0:
            counts = [int(rng.integers(0, bs + 3)) if lens[b] + bs + 3 <= cap and rng.random() < 0.7
                      else 0 for b in range(w.B)]
            st = t.append(counts)
            what = "append %s (status %d)" % (counts, st)
            if st != 0:  # pool exhausted: the device reports it, nothing changed
                assert st == -6
                torch.cuda.synchronize()
                assert t.gc.dev_status() == -6, what
                t.gc.status.zero_()
                t.check(what)
                continue
            t.check(what, cow_pairs=True)
        elif op == 1:
            empty = [b for b in range(w.B) if lens[b] == 0]
            full = [b for b in range(w.B) if lens[b] > 0]
            n = min(len(empty), int(rng.integers(1, 4)))
            if n == 0 or not full:
                continue
            children = [int(c) for c in rng.choice(empty, size=n, replace=False)]
            parents = [int(rng.choice(full)) for _ in range(n)]
            assert t.fork(parents, children) == 0
            t.check("fork %s <- %s" % (children, parents))
        else:
            new_lens = np.array([int(rng.integers(0, lens[b] + 1)) if rng.random() < 0.5
                                 else int(lens[b]) for b in range(w.B)], np.int32)
            assert t.truncate(new_lens) == 0
            t.check("truncate to %s" % list(new_lens))


def test_lifecycle_wide_batch(ref):
    """More sequences than one workgroup's threads: forks, copy-on-write and
    truncation cross the 1024-entry chunks of the device scans."""
    rng = np.random.default_rng(77)
    B, bs = 2600, 16
    w = synth.custom(seed=9, B=B, Hq=2, Hkv=1, D=64, dtype="bf16", block_size=bs, n_q=1)
    t = Twin(ref, w, capacity=4 * bs, pool_blocks=4 * B)
    half = B // 2
    counts = [int(rng.integers(1, 2 * bs)) for _ in range(half)] + [0] * (B - half)
    assert t.append(counts) == 0
    t.check("prefill")
    parents = [int(x) for x in rng.integers(0, half, size=B - half)]
    children = [int(x) for x in rng.permutation(np.arange(half, B))]
    assert t.fork(parents, children) == 0
    t.check("fork")
    assert t.append([1] * B) == 0  # shared partly filled blocks are copied first
    t.check("append with copy-on-write", cow_pairs=True)
    new_lens = np.array([int(rng.integers(0, x + 1)) for x in t.o_lens], np.int32)
    assert t.truncate(new_lens) == 0
    t.check("truncate")


def test_truncate_without_refs(ref):
    rng = np.random.default_rng(3)
    w = synth.custom(seed=3, B=40, Hq=4, Hkv=4, D=64, dtype="f32", block_size=16, n_q=1)
    t = Twin(ref, w, capacity=128, pool_blocks=400)
    assert t.append([int(x) for x in rng.integers(0, 120, size=w.B)], cow=False) == 0
    new_lens = np.array([int(rng.integers(0, x + 1)) for x in t.o_lens], np.int32)
    assert t.truncate(new_lens, with_refs=False) == 0
    t.check("truncate, no reference counts")


def test_lifecycle_errors_change_nothing(ref):
    w = synth.custom(seed=4, B=4, Hq=2, Hkv=2, D=64, dtype="bf16", block_size=16, n_q=1)
    t = Twin(ref, w, capacity=64, pool_blocks=5)
    assert t.append([20, 10, 0, 0]) == 0
    t.check("prefill")
    gc = t.gc
    table0, head0 = gc.table.clone(), int(gc.head.item())
    head_out = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    out = torch.full((w.B,), -3, dtype=torch.int32, device="cuda")
    kvc.kvc_truncate(gc.desc, gc.seq_lens, i32([21, 0, 0, 0]), gc.table, gc.free_list, gc.head,
                     head_out, t.refs, out, gc.status)
    assert gc.dev_status() == -8
    assert torch.equal(gc.table, table0) and int(head_out.item()) == head0
    assert torch.all(out == -3)
    gc.status.zero_()
    for parents, children in (([0], [0]), ([0], [1]), ([0, 1], [2, 2]), ([0, 2], [2, 3]),
                              ([0], [7])):
        kvc.kvc_fork(gc.desc, i32(parents), i32(children), len(parents), gc.seq_lens, gc.table,
                     t.refs, gc.status)
        assert gc.dev_status() == -8, (parents, children)
        gc.status.zero_()
        st, *_ = ref.fork(parents, children, t.o_lens, t.o_table, t.o_refs, gc.bs, gc.N)
        assert st == -8, (parents, children)
    t.check("refused forks")
    # three sequences share sequence 0's partly filled last block: each needs a
    # copy and only 5 - 3 = 2 blocks are free
    assert t.fork([0, 0], [2, 3]) == 0
    t.check("fork")
    st = t.append([1, 0, 1, 1])
    assert st == -6
    torch.cuda.synchronize()
    assert gc.dev_status() == -6
    gc.status.zero_()
    t.check("copy-on-write refused")
    # a bad block id in a copy list is reported and skipped
    src, dst = i32([0, 7]), i32([4, 3])
    k0 = gc.k.clone()
    kvc.kvc_copy_blocks(gc.desc, src, dst, 2, gc.k, gc.v, gc.status)
    assert gc.dev_status() == -8
    assert torch.equal(gc.k[4], k0[0]) and torch.equal(gc.k[3], k0[3])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_copy_blocks_bytes(dtype):
    w = synth.custom(seed=5, B=1, Hq=8, Hkv=8, D=128, dtype=dtype, block_size=32, n_q=1)
    gc = GpuCache(w, block_size=32, capacity=32, pool_blocks=64)
    g = torch.Generator(device="cpu").manual_seed(5)
    gc.k.copy_(torch.randn(gc.k.shape, generator=g).to(gc.k.dtype))
    gc.v.copy_(torch.randn(gc.v.shape, generator=g).to(gc.v.dtype))
    src = torch.arange(0, 20, dtype=torch.int32)
    dst = torch.arange(40, 60, dtype=torch.int32)
    src[5] = -1
    k0, v0 = gc.k.clone(), gc.v.clone()
    kvc.kvc_copy_blocks(gc.desc, src.cuda(), dst.cuda(), 20, gc.k, gc.v, gc.status)
    assert gc.dev_status() == 0
    want_k, want_v = k0.clone(), v0.clone()
    for s, d in zip(src.tolist(), dst.tolist()):
        if s >= 0:
            want_k[d], want_v[d] = k0[s], v0[s]
    assert torch.equal(gc.k, want_k) and torch.equal(gc.v, want_v)


def test_parallel_samples_attention(ref):
    """Parallel sampling: a prompt forked into several samples that then decode
    different tokens; every sample's attention over its shared and copied
    blocks matches the oracle's attention over the oracle's cache."""
    bs, B = 16, 8
    w = synth.custom(seed=11, B=B, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=bs, n_q=1)
    t = Twin(ref, w, capacity=256, pool_blocks=200)
    assert t.append([150, 70] + [0] * 6) == 0
    assert t.fork([0, 0, 0, 1, 1, 1], [2, 3, 4, 5, 6, 7]) == 0
    for step in range(3):
        assert t.append([1] * B) == 0
        t.check("sample step %d" % step, cow_pairs=True)
    gc = t.gc
    q = synth.normal(w, (B, 1, w.Hq, w.D), synth.S_Q, 555)
    got = gc.attend(to_dev(q, w.dtype), 1).cpu().numpy()
    st, want = ref.cache_attention(q, t.o_k, t.o_v, t.o_lens, gc.scale, w.dtype, bs=bs,
                                   table=t.o_table)
    assert st == 0
    assert_close(got, want, "parallel samples")


def test_speculative_rollback_loop(ref):
    """Draft k tokens, verify them with causal attention, keep an accepted
    prefix and truncate the rest; the cache state stays equal to the oracle's and
    each verify output matches the oracle's."""
    rng = np.random.default_rng(12)
    bs, B, k = 16, 6, 5
    w = synth.custom(seed=12, B=B, Hq=8, Hkv=2, D=128, dtype="bf16", block_size=bs, n_q=k)
    t = Twin(ref, w, capacity=512, pool_blocks=B * 32)
    assert t.append([int(x) for x in rng.integers(1, 300, size=B)]) == 0
    gc = t.gc
    for rnd in range(6):
        base = t.o_lens.copy()
        assert t.append([k] * B) == 0
        t.check("drafts %d" % rnd, cow_pairs=True)
        q = synth.normal(w, (B, k, w.Hq, w.D), synth.S_Q, 600 + rnd)
        got = gc.attend(to_dev(q, w.dtype), k).cpu().numpy()
        st, want = ref.cache_attention(q, t.o_k, t.o_v, t.o_lens, gc.scale, w.dtype, bs=bs,
                                       table=t.o_table)
        assert st == 0
        assert_close(got, want, "verify %d" % rnd)
        accepted = rng.integers(0, k + 1, size=B)  # + 1 target token would follow
        assert t.truncate((base + accepted).astype(np.int32)) == 0
        t.check("rollback %d" % rnd)
