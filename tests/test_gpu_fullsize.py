"""Full-size workloads in the launch configuration the benchmark times: every
sequence, head and row against the oracle, evaluated on the generator's rows
(the oracle's own quantization for an FP8 cache), never on anything the GPU
wrote."""
import numpy as np
import pytest
import torch

from kv_cached_decode_kvc_amd import runner, synth
from gpu_harness import assert_close, oracle_outputs_all

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5", "C2F8", "C3F8", "C4F8", "C5F8",
                                  "M1", "M2"])
def test_full_size_every_sequence(ref, name):
    w = synth.get(name)
    print("full-size workload", w.name, flush=True)
    lc = runner.build(w)
    out1 = lc.step().clone()
    out2 = lc.step().clone()  # replaying the prepared step changes nothing
    assert lc.dev_status() == 0
    assert torch.equal(out1, out2)
    lens = synth.final_lengths(w)
    assert np.array_equal(lc.s_len1.cpu().numpy(), lens)
    got = out1.cpu().numpy()
    del lc
    torch.cuda.empty_cache()
    want = oracle_outputs_all(ref, w, synth.cached_lengths(w))
    assert sorted(want) == list(range(w.B))
    worst = 0.0
    for b in range(w.B):
        worst = max(worst, assert_close(got[b], want[b], "%s b=%d L=%d" % (name, b, lens[b])))
    print("%s: %d sequences, max abs err %.3e" % (name, w.B, worst), flush=True)
