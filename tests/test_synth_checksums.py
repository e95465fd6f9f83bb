"""The seeded synthetic workloads are the ones whose fingerprints were committed
(tests/golden/synth_checksums.json, written by tests/golden/write_synth_checksums.py):
head (0, 0) of every workload drawn on the CPU (byte checksums), and the whole
tensors drawn on the GPU, as the GPU tests and bench.py draw them (fp64 sums within
a relative 1e-6, or 1e-4 sqrt(elements) for sums near zero: a few last-bit
differences pass, another seed or recipe does not)."""
import json
import math
import os

import pytest

from block_sparse_quantized_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "synth_checksums.json")))


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_cpu_inputs_match_committed_checksums(name):
    want = GOLD["cpu"][name]
    wl = synth.workload(name, B=1, H=1)
    q, k, v = synth.make_qkv(wl, device="cpu")
    assert list(q.shape) == want["shape"]
    assert (synth.checksum(q), synth.checksum(k), synth.checksum(v)) == (want["q"], want["k"], want["v"])
    if wl.api == "block_sparse":
        assert synth.checksum(synth.make_block_mask(wl, device="cpu")) == want["mask"]


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_gpu_inputs_match_committed_checksums(dev, name):
    want = GOLD["cuda"][name]
    wl = synth.WORKLOADS[name]
    q, k, v = synth.make_qkv(wl, device=dev)
    assert list(q.shape) == want["shape"]
    got = {"q": synth.fingerprint(q), "k": synth.fingerprint(k), "v": synth.fingerprint(v)}
    if wl.api == "block_sparse":
        got["mask"] = synth.fingerprint(synth.make_block_mask(wl, device=dev))
    for key, vals in got.items():
        for a, b in zip(vals, want[key]):
            assert math.isclose(a, b, rel_tol=1e-6, abs_tol=1e-4 * math.sqrt(q.numel())), (key, vals, want[key])
