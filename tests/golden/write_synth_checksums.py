"""Writes tests/golden/synth_checksums.json: fingerprints of the seeded synthetic
inputs (block_sparse_quantized_amd/synth.py), so that a change of generator, seed
layout or torch RNG shows up as a failing test rather than as silently different
workloads.

    python tests/golden/write_synth_checksums.py cpu    # head (0, 0) of every workload
    python tests/golden/write_synth_checksums.py cuda   # whole tensors, drawn on the GPU
    python tests/golden/write_synth_checksums.py cuda OUT.json   # write elsewhere

The CPU entries are SHA-256 prefixes of head (0, 0) of every workload (every head
has its own generator stream, so head (0, 0) of a one-head workload is head (0, 0)
of the full one).  The GPU entries are fp64 fingerprints (synth.fingerprint) of the
whole tensors that the GPU tests and bench.py draw on the device, compared with a
relative tolerance: a device's own reductions may move a last bit, a different seed
or recipe moves them completely.  Each run updates only its own section.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
OUT = os.path.join(HERE, "synth_checksums.json")


def digests(device):
    from block_sparse_quantized_amd import synth
    res = {}
    for name, wl in synth.WORKLOADS.items():
        if device == "cpu":
            wl = synth.workload(name, B=1, H=1)
        q, k, v = synth.make_qkv(wl, device=device)
        digest = synth.checksum if device == "cpu" else synth.fingerprint
        d = {"shape": list(q.shape), "q": digest(q), "k": digest(k), "v": digest(v)}
        if wl.api == "block_sparse":
            d["mask"] = digest(synth.make_block_mask(wl, device=device))
        res[name] = d
        del q, k, v
    return res


def main():
    device = sys.argv[1] if len(sys.argv) > 1 else "cpu"
    out = sys.argv[2] if len(sys.argv) > 2 else OUT
    cur = json.load(open(OUT)) if os.path.exists(OUT) else {}
    cur[device] = digests(device)
    with open(out, "w") as f:
        json.dump(cur, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(cur[device], indent=1))


if __name__ == "__main__":
    main()
