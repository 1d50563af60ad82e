"""Builds caches and runs decode steps through the HIP library, for the GPU tests.

The oracle side is built separately from the same synthetic rows (``synth``),
never from anything the GPU produced.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

from kv_cached_decode_kvc_amd import kvc, synth

ATOL, RTOL = 2e-3, 1e-2  # tolerance fixed for attention outputs (bf16 in, fp32 accumulate)


from kv_cached_decode_kvc_amd.runner import LayerCache as GpuCache, i32, to_dev, torch_dtype  # noqa: E402,F401


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def queries_dev(w, step=0, dev="cuda"):
    return to_dev(synth.packed_queries(w, step), w.dtype, dev)


def logical_rows(w, b, which, cached_len, steps=1):
    """Sequence b's logical rows [Hkv, L, D] straight from the generator:
    its cached rows followed by the new rows of each step."""
    parts = [synth.cache_rows(w, which, b, cached_len)]
    parts += [synth.new_rows(w, which, b, s) for s in range(steps)]
    return np.ascontiguousarray(np.concatenate(parts, axis=0).transpose(1, 0, 2))


def oracle_attention(ref, w, q, k, v, scale):
    """The oracle's attention over generator rows; an FP8 cache holds the
    oracle's own quantization of those rows (dequantized exactly)."""
    if w.dv:  # MLA: one latent head whose rows are keys; values = their first dv dims
        return ref.mla_attention(q, k[0], scale, w.dv)
    if not w.kv:
        return ref.attention(q, k, v, scale, w.dtype)
    kd = ref.dequantize_rows(*ref.quantize_rows(k, w.kv), w.kv)
    vd = ref.dequantize_rows(*ref.quantize_rows(v, w.kv), w.kv)
    return ref.attention(oracle.widen(q, "bf16"), kd, vd, scale, "f64")


def oracle_outputs(ref, w, b_list, cached, steps=1, step_q=None, scale=None):
    """Oracle attention (float64) of the given sequences at the last step, from
    generator rows only: {b: [n_q, Hq, out_dim]}."""
    scale = 1.0 / math.sqrt(w.D) if scale is None else scale
    s = steps - 1 if step_q is None else step_q
    out = {}
    for b in b_list:
        k = logical_rows(w, b, "k", int(cached[b]), steps)
        v = None if w.dv else logical_rows(w, b, "v", int(cached[b]), steps)
        out[b] = oracle_attention(ref, w, synth.queries(w, b, s), k, v, scale)
    return out


def oracle_outputs_all(ref, w, cached, chunk: int = 16, threads: int = 16):
    """Oracle attention (float64) of every sequence of a workload at its first
    step, from generator rows only: {b: [n_q, Hq, out_dim]}.  Rows are drawn
    (and, for an FP8 cache, quantized by the oracle) in host threads, and the
    definition runs on all host cores through the oracle's many-sequence
    function, `chunk` sequences at a time to bound host memory."""
    scale = 1.0 / math.sqrt(w.D)

    def rows(b):
        k = logical_rows(w, b, "k", int(cached[b]))
        if w.dv:
            return k[0], None
        v = logical_rows(w, b, "v", int(cached[b]))
        if w.kv:
            k = ref.dequantize_rows(*ref.quantize_rows(k, w.kv), w.kv)
            v = ref.dequantize_rows(*ref.quantize_rows(v, w.kv), w.kv)
        return k, v

    dt = "f64" if w.kv else w.dtype
    out = {}
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for b0 in range(0, w.B, chunk):
            bs = list(range(b0, min(w.B, b0 + chunk)))
            kv = list(ex.map(rows, bs))
            qs = [synth.queries(w, b) for b in bs]
            if w.kv:
                qs = [oracle.widen(q, "bf16") for q in qs]
            res, _ = ref.attention_many(qs, [x[0] for x in kv],
                                        None if w.dv else [x[1] for x in kv], scale, dt, dv=w.dv)
            out.update(zip(bs, res))
    return out


def tolerance(want: np.ndarray, bf16_out: bool = False) -> np.ndarray:
    """Per-element bound: an element passes when it is within the absolute
    bound (max-abs 2e-3) or within the relative one (max-rel 1e-2) of the
    oracle, whichever is larger.  A bf16 output also gets the half-ulp of its
    own rounding (2^-8 relative), since the oracle is exact."""
    want = np.abs(np.asarray(want, dtype=np.float64))
    tol = np.maximum(ATOL, RTOL * want)
    return tol + want * 2.0 ** -8 if bf16_out else tol


def assert_close(got: np.ndarray, want: np.ndarray, what="", bf16_out: bool = False):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    bad = err > tolerance(want, bf16_out)
    big = np.abs(want) >= 1e-3
    max_rel = float((err[big] / np.abs(want[big])).max()) if big.any() else 0.0
    assert not bad.any(), "%s: %d elements out of tolerance, max abs err %.3e, max rel err %.3e" % (
        what, int(bad.sum()), float(err.max()), max_rel)
    return float(err.max())
