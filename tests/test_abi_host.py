"""The C-ABI library on the host: it loads, exports every symbol its header
declares, and refuses bad arguments before any launch (no GPU needed: each
call here returns during argument checking)."""
import ctypes
import os
import re
import subprocess

import pytest

from kv_cached_decode_kvc_amd import kvc, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its checks first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvc.LIB_PATH):
        from kv_cached_decode_kvc_amd import build
        build.build(verbose=False)
    return kvc.lib()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \t\*]*?\b(kvc_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared()
    for n in ("kvc_block_table", "kvc_append", "kvc_decode_attn", "kvc_verify_attn"):
        assert n in names
    assert set(names) == set(kvc.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", kvc.LIB_PATH], text=True)
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in declared():
        assert n in exported, n
        assert hasattr(lib, n)


def desc(**kw):
    base = dict(batch=16, num_q_heads=40, num_kv_heads=40, head_dim=128, dtype=0, block_size=0,
                max_seq_len=2048, max_blocks_per_seq=0, num_blocks=0, partition_tokens=0)
    base.update(kw)
    return kvc.kvc_cache_desc(*[base[f] for f, _ in kvc.kvc_cache_desc._fields_])


def decode(lib, d, q=FAKE, k=FAKE, v=FAKE, sl=FAKE, table=None, scale=0.1, out=FAKE, out_dtype=1,
           ws=FAKE, ws_bytes=1 << 40):
    return lib.kvc_decode_attn(ctypes.byref(d) if d is not None else None, q, k, v, sl, table,
                               scale, out, out_dtype, ws, ws_bytes, None, None)


def test_attention_argument_errors(lib):
    assert decode(lib, None) == -1
    assert decode(lib, desc(head_dim=96)) == -3
    assert decode(lib, desc(num_kv_heads=7)) == -2
    assert decode(lib, desc(dtype=7)) == -3
    assert decode(lib, desc(block_size=24, max_blocks_per_seq=4, num_blocks=8), table=FAKE) == -3
    assert decode(lib, desc(block_size=48, max_blocks_per_seq=4, num_blocks=8), table=FAKE) == -3
    assert decode(lib, desc(partition_tokens=24)) == -3
    assert decode(lib, desc(), q=None) == -1
    assert decode(lib, desc(), table=FAKE) == -1  # contiguous cache with a table
    assert decode(lib, desc(block_size=16, max_blocks_per_seq=4, num_blocks=8)) == -1  # no table
    assert decode(lib, desc(), ws_bytes=100) == -4
    assert decode(lib, desc(), ws=ctypes.c_void_p(0x1004)) == -1  # misaligned workspace
    assert decode(lib, desc(), scale=float("nan")) == -1
    assert decode(lib, desc(), out_dtype=5) == -3
    assert decode(lib, desc(max_seq_len=0)) == -2
    d = desc()
    for n_q in (0, 17):
        assert lib.kvc_verify_attn(ctypes.byref(d), FAKE, n_q, FAKE, FAKE, FAKE, None, 0.1, FAKE, 1,
                                   FAKE, 1 << 40, None, None) == -3
    # an empty batch is a no-op: nothing to check, nothing launched
    assert decode(lib, desc(batch=0), q=None, k=None, v=None, sl=None, out=None, ws=None) == 0


def test_paging_argument_errors(lib):
    paged = desc(block_size=16, max_blocks_per_seq=8, num_blocks=64)
    contig = desc()
    assert lib.kvc_block_table(ctypes.byref(contig), FAKE, FAKE, 1, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None) == -1
    assert lib.kvc_block_table(ctypes.byref(paged), FAKE, FAKE, -1, FAKE, FAKE, FAKE, FAKE, FAKE,
                               None, None) == -1
    assert lib.kvc_block_table(ctypes.byref(paged), FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, None,
                               None, None) == -1
    same = FAKE
    assert lib.kvc_append(ctypes.byref(contig), FAKE, FAKE, same, FAKE, 1, 1, None, FAKE, FAKE,
                          same, None, None) == -1  # seq_lens_out aliases seq_lens
    assert lib.kvc_append(ctypes.byref(contig), FAKE, FAKE, FAKE, FAKE, 1, 1, FAKE, FAKE, FAKE,
                          ctypes.c_void_p(0x2000), None, None) == -1  # slots on a contiguous cache
    assert lib.kvc_append(ctypes.byref(paged), FAKE, FAKE, FAKE, FAKE, 1, 1, None, FAKE, FAKE,
                          ctypes.c_void_p(0x2000), None, None) == -1  # paged without slots
    assert lib.kvc_append(ctypes.byref(contig), None, FAKE, FAKE, FAKE, 1, 1, None, FAKE, FAKE,
                          ctypes.c_void_p(0x2000), None, None) == -1


def test_attention_launch_count(lib):
    """One launch when the vector-ALU partition kernel combines its own
    partials (one query row per KV row, a grid of at most 4096 items), else
    two (a reduce launch follows)."""
    c1 = desc(batch=2, num_q_heads=4, num_kv_heads=4, head_dim=64, max_seq_len=288, dtype=1)
    assert kvc.kvc_attn_launches(c1, 1) == 1
    assert kvc.kvc_attn_launches(desc(), 1) == 1  # 16 x 40 heads, 2 partitions: 1280 items
    assert kvc.kvc_attn_launches(desc(batch=64), 1) == 2  # 5120 items: more than one round
    assert kvc.kvc_attn_launches(desc(num_kv_heads=8), 1) == 2  # grouped rows: matrix cores
    assert kvc.kvc_attn_launches(desc(), 5) == 2  # verify rows share a KV row: matrix cores
    assert kvc.kvc_attn_launches(desc(head_dim=80), 1) == -3
    assert kvc.kvc_attn_launches(desc(), 17) == -3


def test_workspace_and_partition_sizes(lib):
    d = desc()  # 16 x 40 heads, contiguous, 2048 tokens
    assert kvc.kvc_attn_partition_tokens(d, 1) == 1024  # contiguous: long runs
    rows, parts = 16 * 40, 2048 // 1024
    o = rows * parts * 128 * 4
    assert kvc.kvc_attn_workspace_bytes(d, 1) == CNT + ((o + 255) // 256) * 256 + rows * parts * 2 * 4
    small = desc(batch=2, num_q_heads=4, num_kv_heads=4, head_dim=64, max_seq_len=288, dtype=1)
    assert kvc.kvc_attn_partition_tokens(small, 1) == 64  # halved while fewer than 1024 items
    assert kvc.kvc_attn_partition_tokens(desc(partition_tokens=48), 1) == 48
    assert kvc.kvc_attn_workspace_bytes(desc(head_dim=80), 1) == 0
    assert kvc.kvc_attn_partition_tokens(desc(head_dim=80), 1) == -3
    # grouped rows (GQA decode, verify) and a paged MHA batch too large for one
    # round of work items use the stream-K split: no length (0)
    for name, want in (("C2", 1024), ("C3", 0), ("C4", 0), ("C5", 0)):
        w = synth.get(name)
        dd = desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                  block_size=w.block_size, max_seq_len=synth.capacity_tokens(w),
                  max_blocks_per_seq=synth.max_blocks_per_seq(w) if w.block_size else 0,
                  num_blocks=synth.pool_blocks(w) if w.block_size else 0)
        P = kvc.kvc_attn_partition_tokens(dd, w.n_q)
        assert P == want, (name, P)
        assert kvc.kvc_attn_workspace_bytes(dd, w.n_q) > 0


# every attention workspace starts with 256 KiB of combine counters (zero
# between calls); the partials follow
CNT = 256 << 10


def _ws_bytes(rows, parts, d):
    o = rows * parts * d * 4
    return CNT + ((o + 255) // 256) * 256 + rows * parts * 2 * 4


def _sk_bytes(pieces, rows, d, segs):
    o = pieces * rows * d * 4
    ml = ((o + 255) // 256) * 256 + pieces * rows * 2 * 4
    return CNT + ((ml + 255) // 256) * 256 + segs * 2 * 4


def test_stream_k_workspace(lib):
    # grouped rows by default: one partial per row of every piece, at most
    # segments + workers pieces; workers (1024 SIMDs when no device is
    # visible): one per SIMD for bf16, for FP8 one round of resident
    # wavefronts (2 per SIMD with 32-row blocks, 3 with 16-row blocks); an
    # explicit partition length keeps fixed partitions
    w = synth.get("C5")
    cap = synth.capacity_tokens(w)
    for dtype, workers in (("bf16", 1024), ("fp8_e4m3", 2048)):
        dd = desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                  dtype=kvc.DTYPE_CODES[dtype], block_size=w.block_size, max_seq_len=cap,
                  max_blocks_per_seq=synth.max_blocks_per_seq(w),
                  num_blocks=synth.pool_blocks(w))
        assert kvc.kvc_attn_partition_tokens(dd, w.n_q) == 0
        segs = w.B * w.Hkv  # 20 rows per KV head: one 32-row block
        assert kvc.kvc_attn_workspace_bytes(dd, w.n_q) == _sk_bytes(segs + workers, 20, w.D,
                                                                    segs)
    w = synth.get("C4")  # 4 rows per KV head: 16-row blocks
    dd = desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
              block_size=w.block_size, max_seq_len=synth.capacity_tokens(w),
              max_blocks_per_seq=synth.max_blocks_per_seq(w), num_blocks=synth.pool_blocks(w))
    segs = w.B * w.Hkv
    assert kvc.kvc_attn_workspace_bytes(dd, 1) == _sk_bytes(segs + 1024, 4, w.D, segs)
    dd.dtype = kvc.DTYPE_CODES["fp8_e4m3"]
    assert kvc.kvc_attn_workspace_bytes(dd, 1) == _sk_bytes(segs + 3072, 4, w.D, segs)
    w = synth.get("C5")
    dd = desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
              dtype=kvc.DTYPE_CODES["fp8_e4m3"], block_size=w.block_size, max_seq_len=cap,
              max_blocks_per_seq=synth.max_blocks_per_seq(w), num_blocks=synth.pool_blocks(w),
              partition_tokens=512)
    assert kvc.kvc_attn_partition_tokens(dd, w.n_q) == 512
    rows = w.B * w.Hq * w.n_q
    assert kvc.kvc_attn_workspace_bytes(dd, w.n_q) == _ws_bytes(rows, -(-cap // 512), w.D)


def test_valu_stream_k_plan(lib):
    # paged MHA: a batch whose fixed partitions (the power of two nearest an
    # eighth of the capacity) fit one round of resident work items combines
    # inside its partition launch; a larger one (C3: 64 x 40 rows, 512-key
    # partitions) takes the vector-ALU stream-K split, 2 workers per SIMD,
    # one partial row per piece and a record per segment (query row)
    w = synth.get("C3")
    cap = synth.capacity_tokens(w)

    def paged(batch, dtype="bf16", **kw):
        return desc(batch=batch, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                    dtype=kvc.DTYPE_CODES[dtype], block_size=w.block_size, max_seq_len=cap,
                    max_blocks_per_seq=synth.max_blocks_per_seq(w), num_blocks=synth.pool_blocks(w),
                    **kw)
    small = paged(8)  # 8 x 40 rows x 9 partitions: 2880 items, one round
    assert kvc.kvc_attn_partition_tokens(small, 1) == 512
    assert kvc.kvc_attn_launches(small, 1) == 1
    for dtype in ("bf16", "f32"):
        dd = paged(w.B, dtype)
        assert kvc.kvc_attn_partition_tokens(dd, 1) == 0
        assert kvc.kvc_attn_launches(dd, 1) == 2
        segs = w.B * w.Hq
        assert kvc.kvc_attn_workspace_bytes(dd, 1) == _sk_bytes(segs + 2048, 1, w.D, segs)
    # FP8 caches and an explicit partition length keep fixed partitions
    assert kvc.kvc_attn_partition_tokens(paged(w.B, "fp8_e4m3"), 1) == 512
    assert kvc.kvc_attn_partition_tokens(paged(w.B, partition_tokens=256), 1) == 256


def test_mla_workspace_covers_launch_time_partitions(lib):
    # MLA whose full-capacity batch fits one round of resident workgroups:
    # launches may use partitions down to half the planned length, so the
    # workspace holds twice the partitions; an explicit length keeps the count.
    # 16 rows (M2) use these partitions by default; more rows (M1, given an
    # explicit length here) are checked for the explicit case only.
    for alias, planned, explicits in (("M1", 1024, ((1024, 1),)),
                                      ("M2", 2048, ((0, 2), (2048, 1)))):
        w = synth.get(alias)
        cap = synth.capacity_tokens(w)
        rows = w.B * w.Hq * w.n_q
        for explicit, factor in explicits:
            dd = desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                      dtype=kvc.DTYPE_CODES[w.dtype], block_size=w.block_size, max_seq_len=cap,
                      max_blocks_per_seq=synth.max_blocks_per_seq(w),
                      num_blocks=synth.pool_blocks(w), partition_tokens=explicit)
            P = kvc.kvc_mla_partition_tokens(dd, w.n_q, w.dv)
            assert P == planned, (alias, P)
            parts = -(-cap // (P // factor))
            assert kvc.kvc_mla_workspace_bytes(dd, w.n_q, w.dv) == _ws_bytes(rows, parts, w.dv), alias


def test_mla_stream_k_plan(lib):
    # more than 16 rows by default: the stream-K split, one round of 256
    # workgroups shared by the row groups (128 heads: two 64-row groups, 128
    # workers), one partial per row of every (sequence, worker) piece (at
    # most sequences + workers pieces) and one worker record per sequence
    w = synth.get("M1")
    cap = synth.capacity_tokens(w)
    rows = w.Hq * w.n_q
    for n_q, workers in ((1, 128), (2, 64)):  # 256 rows: four row groups
        dd = desc(batch=w.B, num_q_heads=w.Hq, num_kv_heads=w.Hkv, head_dim=w.D,
                  dtype=kvc.DTYPE_CODES[w.dtype], block_size=w.block_size, max_seq_len=cap,
                  max_blocks_per_seq=synth.max_blocks_per_seq(w), num_blocks=synth.pool_blocks(w))
        assert kvc.kvc_mla_partition_tokens(dd, n_q, w.dv) == 0
        assert kvc.kvc_mla_workspace_bytes(dd, n_q, w.dv) == _sk_bytes(
            w.B + workers, rows * n_q, w.dv, w.B)
    # a sequence too long for one worker's run in the kernel's block-id
    # staging (128 workers of 16384 keys at most): fixed partitions
    big = desc(batch=4096, num_q_heads=128, num_kv_heads=1, head_dim=576,
               dtype=kvc.DTYPE_CODES["bf16"], block_size=64, max_seq_len=8192,
               max_blocks_per_seq=128, num_blocks=4096 * 128)
    assert kvc.kvc_mla_partition_tokens(big, 1, 512) > 0


def test_status_strings(lib):
    for code, name in kvc.STATUS_NAMES.items():
        s = kvc.kvc_status_string(code)
        assert s and s != "unknown status", name
    assert kvc.kvc_status_string(-99) == "unknown status"


def test_binding_refuses_host_tensors():
    import torch
    d = desc(batch=1, num_q_heads=1, num_kv_heads=1, head_dim=64, max_seq_len=16)
    t = torch.zeros(16)
    with pytest.raises(ValueError):
        kvc.kvc_decode_attn(d, t, t, t, t.int(), None, 0.1, t, t)


def test_noalloc_refusals_before_any_device_call(lib):
    """The allocation-free attention call refuses on the host: a batch whose
    partials exceed the static scratch, bad row counts, a missing output."""
    big = desc(batch=1024, num_q_heads=32, num_kv_heads=8, dtype=0, block_size=16,
               max_seq_len=0, max_blocks_per_seq=4096, num_blocks=600000)
    need = lib.kvc_attn_workspace_bytes(ctypes.byref(big), 16)
    assert need > kvc.NOALLOC_SCRATCH_BYTES
    call = lambda d, n_q=1, out=FAKE: lib.kvc_verify_attn_noalloc(
        ctypes.byref(d), FAKE, n_q, FAKE, FAKE, FAKE, FAKE if d.block_size else None, 0.1, out,
        1, None, None)
    assert call(big, 16) == -4  # KVC_ERR_WORKSPACE
    assert call(desc(), 0) == -3
    assert call(desc(), 17) == -3
    assert call(desc(), 1, None) == -1
    assert lib.kvc_verify_attn_noalloc(ctypes.byref(desc()), FAKE, 1, FAKE, FAKE, FAKE, None,
                                       0.1, FAKE, 5, None, None) == -3  # output type
    assert lib.kvc_verify_attn_noalloc(ctypes.byref(desc(batch=0)), None, 1, None, None, None,
                                       None, 0.1, None, 1, None, None) == 0


def test_block_table_append_refusals(lib):
    paged = desc(block_size=16, max_seq_len=0, max_blocks_per_seq=8, num_blocks=64)
    call = lambda d, sl=FAKE, out=ctypes.c_void_p(0x2000), total=1: lib.kvc_block_table_append(
        ctypes.byref(d), FAKE, FAKE, sl, FAKE, total, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
        out, None, None)
    assert call(desc()) == -1  # a contiguous cache has no table: kvc_append
    assert call(paged, total=-1) == -1
    assert call(paged, out=FAKE) == -1  # seq_lens_out aliases seq_lens
    assert call(paged, out=None) == -1
    assert call(desc(batch=9000, block_size=16, max_seq_len=0, max_blocks_per_seq=8,
                     num_blocks=64)) == -3  # every workgroup reads the batch: <= 8192
    assert lib.kvc_block_table_append(ctypes.byref(desc(batch=0, block_size=16, max_seq_len=0,
                                                        max_blocks_per_seq=8, num_blocks=64)),
                                      None, None, None, None, 0, 0, None, None, None, None, None,
                                      None, None, None, None, None) == 0
