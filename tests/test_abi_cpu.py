"""CPU checks of the C-ABI library: it loads, exports every function that
include/bsa.h declares, and rejects bad arguments on the host with the
documented status codes (no GPU work is enqueued on any of these paths).
Also a host build of the library's per-index Gilbert descent against the
oracle's recursive enumeration."""

import ctypes
import itertools
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from oracle.gilbert import gilbert_order

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

bsa = pytest.importorskip("block_sparse_attention_gilbert_amd")
lib = bsa.library()

FAKE = ctypes.c_void_p(0x10000)   # aligned, never dereferenced on these paths
FAKE2 = ctypes.c_void_p(0x20000000)


def test_exports_match_header():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", text))
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), name
    assert set(bsa.EXPORTED) == declared


def test_version_and_strerror():
    assert lib.bsa_version() >= 100
    for code in range(5):
        assert lib.bsa_strerror(code)
    assert lib.bsa_strerror(99) == b"unknown status"


def _code_and_detail(code):
    return code, lib.bsa_last_error_detail().decode()


def test_gilbert_index_rejects():
    assert _code_and_detail(lib.bsa_gilbert_index(0, 3, 3, FAKE, None, None))[0] == bsa.BSA_EINVAL
    assert lib.bsa_gilbert_index(3, 30, 52, None, None, None) == bsa.BSA_EINVAL
    assert lib.bsa_gilbert_index(2048, 2048, 2048, FAKE, None, None) == bsa.BSA_EINVAL
    assert "exceeds" in lib.bsa_last_error_detail().decode()


def test_gilbert_perm_rejects():
    f = lib.bsa_gilbert_perm
    assert f(None, FAKE2, FAKE, 4680, 40, 128, 128, 5120, 4736 * 128, 0, 0, None) == bsa.BSA_EINVAL
    assert f(FAKE, FAKE2, FAKE, 4680, 40, 96, 128, 5120, 4736 * 128, 0, 0, None) == bsa.BSA_EUNSUPPORTED
    assert f(FAKE, FAKE2, FAKE, 4680, 40, 128, 32, 5120, 4736 * 128, 0, 0, None) == bsa.BSA_EUNSUPPORTED
    assert f(FAKE, FAKE2, FAKE, 4680, 40, 128, 128, 5120, 4736 * 128, 0, 7, None) == bsa.BSA_EUNSUPPORTED
    assert f(FAKE, FAKE2, FAKE, 4680, 40, 128, 128, 100, 4736 * 128, 0, 0, None) == bsa.BSA_EINVAL
    assert f(FAKE, FAKE2, FAKE, 4680, 40, 128, 128, 5120, 4680 * 128, 0, 0, None) == bsa.BSA_EINVAL
    assert f(FAKE, FAKE2, FAKE, 4680, 40, 128, 128, 5120, 4736 * 128, 2, 0, None) == bsa.BSA_EINVAL
    # overlapping src/dst
    assert f(FAKE, ctypes.c_void_p(0x10000 + 256), FAKE, 4680, 40, 128, 128, 5120, 4736 * 128, 0, 0, None) \
        == bsa.BSA_EINVAL
    assert "overlap" in lib.bsa_last_error_detail().decode()
    # misaligned pointer
    assert f(ctypes.c_void_p(0x10008), FAKE2, FAKE, 4680, 40, 128, 128, 5120, 4736 * 128, 0, 0, None) \
        == bsa.BSA_EINVAL


def _attn(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, dtype=0, heads=40, d=128, block=128, nqb=37, nkb=1776,
             qhs=37 * 128 * 128, khs=1776 * 128 * 128, vhs=1776 * 128 * 128, ohs=37 * 128 * 128, ql=None,
             kl=None, rp=FAKE, ci=FAKE, cl=1480 * 50, scale=0.088)
    a.update(over)
    return lib.bsa_block_sparse_attn(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dtype"], a["heads"], a["d"],
                                     a["block"], a["nqb"], a["nkb"], a["qhs"], a["khs"], a["vhs"], a["ohs"],
                                     a["ql"], a["kl"], a["rp"], a["ci"], a["cl"], a["scale"], None)


def test_attention_rejects():
    assert _attn(q=None) == bsa.BSA_EINVAL
    assert _attn(rp=None) == bsa.BSA_EINVAL
    assert _attn(d=80) == bsa.BSA_EUNSUPPORTED
    assert _attn(block=256) == bsa.BSA_EUNSUPPORTED
    assert _attn(dtype=3) == bsa.BSA_EUNSUPPORTED
    assert _attn(nqb=0) == bsa.BSA_EINVAL
    assert _attn(khs=100) == bsa.BSA_EINVAL
    assert _attn(ohs=37 * 128 * 128 - 8) == bsa.BSA_EINVAL
    assert _attn(qhs=37 * 128 * 128 + 3) == bsa.BSA_EINVAL   # breaks 16-byte row alignment
    assert _attn(scale=0.0) == bsa.BSA_EINVAL
    assert _attn(scale=-1.0) == bsa.BSA_EINVAL
    assert _attn(cl=-1) == bsa.BSA_EINVAL
    d = lib.bsa_dense_attn(FAKE, FAKE, FAKE, FAKE, None, 0, 40, 128, 128, 37, 1776, 37 * 128 * 128, 10, 10,
                           37 * 128 * 128, None, None, ctypes.c_float(0.088), None)
    assert d == bsa.BSA_EINVAL


def _route_args(**over):
    a = bsa.RouteArgs()
    a.struct_size = ctypes.sizeof(bsa.RouteArgs)
    a.q, a.k, a.dtype = 0x10000, 0x20000000, 0
    a.heads, a.d, a.block, a.nqb, a.nkb = 40, 128, 128, 37, 1776
    a.q_head_stride, a.k_head_stride = 37 * 128 * 128, 1776 * 128 * 128
    a.scale = 0.088
    a.lam, a.g_ref, a.tau = 2.0, 0.2, 0.1
    a.k_fixed, a.k_max = 50, 50
    a.row_ptr, a.col_idx, a.col_capacity = 0x30000, 0x40000, 1480 * 50
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_route_rejects_and_sizes():
    a = _route_args()
    need = lib.bsa_route_workspace_size(ctypes.byref(a))
    # qbar + kbar + keys + keff + flags, each 256-byte aligned
    assert need >= 8 * (40 * 37 * 128 + 40 * 1776 * 128 + 40 * 37 * 1776)
    assert lib.bsa_route_topk(ctypes.byref(a), None, 0, None) == bsa.BSA_EWORKSPACE
    assert lib.bsa_route_topk(ctypes.byref(a), FAKE, need - 1, None) == bsa.BSA_EWORKSPACE
    assert lib.bsa_route_topk(ctypes.byref(a), ctypes.c_void_p(0x10010), need, None) == bsa.BSA_EWORKSPACE
    bad = _route_args(struct_size=8)
    assert lib.bsa_route_topk(ctypes.byref(bad), FAKE, need, None) == bsa.BSA_EINVAL
    assert lib.bsa_route_workspace_size(ctypes.byref(bad)) == 0
    assert lib.bsa_route_topk(ctypes.byref(_route_args(col_capacity=1480 * 50 - 1)), FAKE, need, None) \
        == bsa.BSA_EINVAL
    assert lib.bsa_route_topk(ctypes.byref(_route_args(nkb=5000)), FAKE, need, None) == bsa.BSA_EUNSUPPORTED
    assert lib.bsa_route_topk(ctypes.byref(_route_args(n_dense_tail_blocks=2000)), FAKE, need, None) \
        == bsa.BSA_EINVAL
    assert lib.bsa_route_topk(ctypes.byref(_route_args(overlap=0x50000, overlap_row_stride=10)), FAKE, need,
                              None) == bsa.BSA_EINVAL
    assert lib.bsa_route_topk(ctypes.byref(_route_args(overlap=0x50000, overlap_row_stride=1776, g_ref=0.0)),
                              FAKE, need, None) == bsa.BSA_EINVAL
    assert lib.bsa_route_topk(ctypes.byref(_route_args(kpool=0x60000, kpool_valid_blocks=1777)), FAKE, need,
                              None) == bsa.BSA_EINVAL
    assert lib.bsa_route_topk(ctypes.byref(_route_args(kpool=0x60000, kpool_head_blocks=1775)), FAKE, need,
                              None) == bsa.BSA_EINVAL
    assert lib.bsa_route_topk(ctypes.byref(_route_args(k_per_row=0x70000, k_max=-1)), FAKE, need, None) \
        == bsa.BSA_EINVAL
    # kpool and sel_keys shrink the workspace
    small = lib.bsa_route_workspace_size(ctypes.byref(_route_args(kpool=0x60000, sel_keys=0x80000)))
    assert 0 < small < need


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_host_descent_matches_oracle(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = str(tmp_path / "gdesc")
    src = os.path.join(ROOT, "tests", "native", "gilbert_descent_host.cpp")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-I" + os.path.join(ROOT, "block_sparse_attention_gilbert_amd", "csrc"),
                    "-I" + os.path.join(ROOT, "include"), src, "-o", exe], check=True, capture_output=True)
    shapes = list(itertools.product(range(1, 7), repeat=3)) + [(3, 30, 52), (1, 30, 52), (21, 30, 52)]
    for s in shapes:
        out = subprocess.run([exe, *map(str, s)], capture_output=True, text=True, check=True).stdout.split()
        ref, _ = gilbert_order(*s)
        assert np.array_equal(np.array(out, dtype=np.int64), ref), s
