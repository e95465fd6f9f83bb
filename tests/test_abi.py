"""The C-ABI library on the CPU: loads without a GPU, exports every symbol that
include/sparge.h declares, matches the header's struct layouts, rejects bad
arguments before any device work, and computes the host Hilbert order."""

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

from block_sparse_quantized_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparge.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.lib_path()):
        pytest.fail("libsparge.so is not built (python -m block_sparse_quantized_amd.build)")
    return L.lib()


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", src)) - {"if", "sizeof"})


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert "sparge_topk_attn" in names and "block_sparse_attn" in names
    out = subprocess.run(["nm", "-D", "--defined-only", L.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT\s+(\S+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    assert set(names) == set(L.PROTOTYPES), "binding prototypes must cover exactly the header"
    assert lib.sparge_abi_version() == 3


def test_every_symbol_resolves_at_load():
    """Binding every symbol when the library loads (RTLD_NOW) fails on any undefined
    one, e.g. a kernel's host launch stub that the host pass did not emit, which a
    lazily bound load would only report at the first launch."""
    ctypes.CDLL(L.lib_path(), mode=os.RTLD_NOW | os.RTLD_LOCAL)
    out = subprocess.run(["nm", "-D", "--undefined-only", L.lib_path()], capture_output=True, text=True).stdout
    assert "device_stub" not in out


def test_struct_layout_matches_c_compiler():
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "sparge.h"
int main(void) {
  printf("%zu %zu %zu\n", sizeof(sparge_tensor), sizeof(sparge_opts), sizeof(sparge_stats));
  printf("%zu %zu %zu %zu\n", offsetof(sparge_tensor, B), offsetof(sparge_tensor, sN),
         offsetof(sparge_opts, mask_out), offsetof(sparge_opts, stats));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = list(map(int, out))
    want = [ctypes.sizeof(L.SpargeTensor), ctypes.sizeof(L.SpargeOpts), ctypes.sizeof(L.SpargeStats),
            L.SpargeTensor.B.offset, L.SpargeTensor.sN.offset, L.SpargeOpts.mask_out.offset,
            L.SpargeOpts.stats.offset]
    assert got == want


FAKE = 0x7f0000000000  # aligned, never dereferenced: every case fails validation first


def T(dtype=L.SPARGE_BF16, B=1, H=2, N=256, D=64, data=FAKE, sN=None):
    sN = D if sN is None else sN
    return L.SpargeTensor(data, dtype, 0, B, H, N, D, H * N * sN, N * sN, sN)


def call_topk(lib, q, k, v, o, topk=0.5, ws=FAKE, wsb=1 << 40, opts=None):
    return lib.sparge_topk_attn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o),
                                topk, 0, opts, ws, wsb, None)


def test_validation_errors_topk(lib):
    q, k, v = T(data=FAKE), T(data=FAKE + 4096), T(data=FAKE + 8192)
    o = T(data=FAKE + 12288)
    assert call_topk(lib, T(data=0), k, v, o) == -1                       # null data
    assert call_topk(lib, T(D=96), T(D=96, data=FAKE + 4096), v, o) == -2  # D not in {64,128}
    assert call_topk(lib, T(N=0), k, v, o) == -2
    assert call_topk(lib, q, T(N=128, data=FAKE + 4096), v, o) == -2       # shape mismatch
    assert call_topk(lib, q, T(dtype=L.SPARGE_F16, data=FAKE + 4096), v, o) == -3
    assert call_topk(lib, T(dtype=7), k, v, o) == -3
    assert call_topk(lib, q, k, v, o, topk=0.0) == -4
    assert call_topk(lib, q, k, v, o, topk=1.5) == -4
    assert call_topk(lib, q, k, v, o, topk=float("nan")) == -4
    assert call_topk(lib, q, k, v, T(data=FAKE)) == -4                     # out aliases q
    assert call_topk(lib, T(data=FAKE + 2), k, v, o) == -5                 # misaligned
    assert call_topk(lib, T(sN=65), k, v, o) == -5                         # row stride not 16B
    assert call_topk(lib, q, T(sN=1 << 25, data=FAKE + 4096), v, o) == -5  # row stride of 64 MiB
    assert call_topk(lib, q, k, v, o, ws=None) == -6
    assert call_topk(lib, q, k, v, o, wsb=1024) == -6
    bad = L.SpargeOpts()
    lib.sparge_default_opts(ctypes.byref(bad))
    bad.filter_lambda = 1.0
    assert call_topk(lib, q, k, v, o, opts=ctypes.byref(bad)) == -4
    bad.filter_lambda = -10.0
    bad.scale = -1.0
    assert call_topk(lib, q, k, v, o, opts=ctypes.byref(bad)) == -4
    bad.scale = 0.0
    bad.pv_fp8, bad.pv_fp16 = 1, 1                                         # two P.V types
    assert call_topk(lib, q, k, v, o, opts=ctypes.byref(bad)) == -4
    bad.pv_fp16 = 0                                                         # fp8 P.V, fp32 inputs
    f32 = [T(dtype=L.SPARGE_F32, data=FAKE + 16384 * i) for i in range(4)]
    assert call_topk(lib, *f32, opts=ctypes.byref(bad)) == -5
    r = lib.block_sparse_attn(*(ctypes.byref(t) for t in f32[:3]), None, ctypes.byref(f32[3]),
                              ctypes.byref(bad), FAKE, 1 << 40, None)
    assert r == -5


def call_cdf(lib, q, k, v, o, tau=0.9, opts=None):
    return lib.sparge_cdf_attn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o),
                               tau, 0, opts, FAKE, 1 << 40, None)


def test_validation_errors_cdf_and_per_head_knobs(lib):
    q, k, v, o = T(), T(data=FAKE + 4096), T(data=FAKE + 8192), T(data=FAKE + 12288)
    for tau in (0.0, -0.5, 1.5, float("nan")):
        assert call_cdf(lib, q, k, v, o, tau) == -4
    H = q.H
    dbl = ctypes.POINTER(ctypes.c_double)

    def opts_with(**arrays):
        op = L.SpargeOpts()
        lib.sparge_default_opts(ctypes.byref(op))
        keep = []
        for name, vals in arrays.items():
            a = (ctypes.c_double * H)(*vals)
            keep.append(a)
            setattr(op, name, ctypes.cast(a, dbl))
        return op, keep
    # every check happens on the host before anything touches the (fake) device memory
    for name, vals in (("head_select", [0.5, 0.0]), ("head_select", [1.2, 0.5]),
                       ("head_sim_threshold", [0.1, float("nan")]),
                       ("head_filter_lambda", [-10.0, 0.5]), ("head_filter_lambda", [float("nan"), -1.0])):
        op, keep = opts_with(**{name: vals})
        assert call_topk(lib, q, k, v, o, opts=ctypes.byref(op)) == -4, (name, vals)
        assert call_cdf(lib, q, k, v, o, 0.9, opts=ctypes.byref(op)) == -4, (name, vals)
    op, keep = opts_with(head_filter_lambda=[-10.0, 0.5])
    r = lib.block_sparse_attn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, ctypes.byref(o),
                              ctypes.byref(op), FAKE, 1 << 40, None)
    assert r == -4
    op, keep = opts_with(head_select=[0.5, 2.0])
    r = lib.sparge_predict_mask(ctypes.byref(q), ctypes.byref(k), 0.5, 1, ctypes.byref(op), FAKE,
                                FAKE, 1 << 40, None)
    assert r == -4


def test_validation_errors_other_entry_points(lib):
    q, k, v, o = T(), T(data=FAKE + 4096), T(data=FAKE + 8192), T(data=FAKE + 12288)
    r = lib.block_sparse_attn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, ctypes.byref(o),
                              None, FAKE, 16, None)
    assert r == -6
    r = lib.sparge_predict_mask(ctypes.byref(q), ctypes.byref(k), 0.5, 1, None, None, FAKE, 1 << 40, None)
    assert r == -1
    r = lib.sparge_quantize_qk(ctypes.byref(q), ctypes.byref(k), None, FAKE, FAKE, FAKE, FAKE, FAKE,
                               1 << 40, None)
    assert r == -1
    r = lib.sparge_reorder(ctypes.byref(q), ctypes.byref(o), FAKE, 10, 300, 0, None)
    assert r == -4                                                          # offset+count > N
    r = lib.sparge_reorder(ctypes.byref(q), ctypes.byref(q), FAKE, 0, 10, 0, None)
    assert r == -4                                                          # aliasing
    assert lib.sparge_hilbert_perm3d(0, 2, 2, FAKE) == -2
    assert lib.sparge_hilbert_perm3d(2, 2, 2, None) == -1
    for s in range(-7, 1):
        assert lib.sparge_status_str(s)


def test_workspace_bytes(lib):
    a = lib.sparge_workspace_bytes(1, 32, 8192, 128, L.SPARGE_BF16, None)
    b = lib.sparge_workspace_bytes(1, 32, 16384, 128, L.SPARGE_BF16, None)
    c = lib.sparge_workspace_bytes(1, 32, 8192, 128, L.SPARGE_F32, None)
    assert 0 < a < b and c >= a
    assert lib.sparge_workspace_bytes(1, 32, 8192, 96, L.SPARGE_BF16, None) == 0
    assert lib.sparge_workspace_bytes(1, 32, 0, 128, L.SPARGE_BF16, None) == 0
    assert lib.sparge_workspace_bytes(1, 32, 8192, 128, 5, None) == 0


def test_default_opts(lib):
    o = L.SpargeOpts()
    lib.sparge_default_opts(ctypes.byref(o))
    assert (o.scale, o.sim_threshold, o.filter_lambda) == (0.0, 0.1, -10.0)
    assert (o.filter_on, o.qk_int8, o.pv_fp16, o.pv_fp8) == (1, 0, 0, 0)
    assert not o.mask_out and not o.stats


@pytest.mark.parametrize("shape", [(13, 30, 45), (1, 1, 1), (2, 3, 5), (8, 8, 8), (3, 64, 64), (64, 1, 7)])
def test_host_hilbert_matches_oracle_inverse_map(lib, shape):
    from oracle.hilbert_ref import hilbert_cell_order
    n = int(np.prod(shape))
    buf = (ctypes.c_int32 * n)()
    assert lib.sparge_hilbert_perm3d(*shape, buf) == 0
    got = np.frombuffer(buf, dtype=np.int32).astype(np.int64)
    assert np.array_equal(got, hilbert_cell_order(*shape))
