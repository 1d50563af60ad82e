"""Full-size workloads in the launch configuration the benchmark times: sampled
sequences (every head and row) against the oracle, evaluated on the
generator's rows of those sequences only."""
import numpy as np
import pytest
import torch

from kv_cached_decode_kvc_amd import runner, synth
from gpu_harness import assert_close, oracle_outputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5", "C2F8", "C3F8", "C4F8", "C5F8"])
def test_full_size_sampled(ref, name):
    w = synth.get(name)
    print("full-size workload", w.name, flush=True)
    lc = runner.build(w)
    out1 = lc.step().clone()
    out2 = lc.step().clone()  # replaying the prepared step changes nothing
    assert lc.dev_status() == 0
    assert torch.equal(out1, out2)
    lens = synth.final_lengths(w)
    assert np.array_equal(lc.s_len1.cpu().numpy(), lens)
    cached = synth.cached_lengths(w)
    sample = sorted({0, w.B // 2, w.B - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    want = oracle_outputs(ref, w, sample, cached)
    got = out1.cpu().numpy()
    for b in sample:
        assert_close(got[b], want[b], "%s b=%d L=%d" % (name, b, lens[b]))
    del lc
    torch.cuda.empty_cache()
