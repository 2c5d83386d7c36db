"""CPU checks of the C ABI: the library loads, exports every declared entry
point, and rejects bad arguments before touching the GPU.

No compute call is made here (there is no GPU): every call below fails a
host-side check before any HIP call, or is host-only.
"""

from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seer.h")


@pytest.fixture(scope="module")
def S():
    import block_sparse_attention_seer_amd as S
    if not os.path.exists(S.LIB_PATH):
        pytest.fail("libseer.so is not built (run __graft_entry__.build())")
    S.lib()
    return S


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(seer_[a-z_]+)\s*\(", text)))


def test_header_declares_the_pipeline():
    names = declared_functions()
    for want in ["seer_kcomp_update", "seer_gate_scores", "seer_select_blocks",
                 "seer_sparse_decode", "seer_dense_decode"]:
        assert want in names


def test_library_exports_every_declared_symbol(S):
    names = declared_functions()
    handle = ctypes.CDLL(S.LIB_PATH)
    missing = [n for n in names if not hasattr(handle, n)]
    assert not missing, missing
    assert set(names) == set(S.EXPORTED_SYMBOLS)
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", S.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r" T (seer_[a-z_]+)$", out, flags=re.M))
        assert exported == set(names)


def test_status_strings_and_version(S):
    assert S.seer_status_string(0) == "SEER_OK"
    for code in (1, 2, 3, 4):
        assert S.seer_status_string(code).startswith("SEER_ERR_")
    assert "gfx950" in S.seer_version()


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_error_paths_without_gpu(S):
    L = S.lib()
    d = S.make_dims(16, 40, 8, 128, 128, 64, 32768)
    A = _fake(0x10000)  # aligned, never dereferenced: every call fails first
    # null pointers
    rc = L.seer_sparse_decode(ctypes.byref(d), None, A, A, A, A, A, 53, 0.1, 4, A, 10 ** 9, A,
                              None, None)
    assert rc == 1 and "q is NULL" in S.seer_last_error_message()
    # misaligned K
    rc = L.seer_dense_decode(ctypes.byref(d), A, _fake(0x10002), A, A, 0.1, 4, A, 10 ** 9, A,
                             None, None)
    assert rc == 1 and "aligned" in S.seer_last_error_message()
    # unsupported head_dim
    bad = S.make_dims(16, 40, 8, 96, 128, 64, 32768)
    rc = L.seer_dense_decode(ctypes.byref(bad), A, A, A, A, 0.1, 4, A, 10 ** 9, A, None, None)
    assert rc == 2
    # workspace too small (explicit split count, so no device query)
    rc = L.seer_sparse_decode(ctypes.byref(d), A, A, A, A, A, A, 53, 0.1, 4, A, 16, A, None, None)
    assert rc == 3
    # num_split out of range (above 128, or below SEER_SPLIT_BALANCED = -1)
    for bad_split in (999, -2):
        rc = L.seer_sparse_decode(ctypes.byref(d), A, A, A, A, A, A, 53, 0.1, bad_split, A,
                                  10 ** 9, A, None, None)
        assert rc == 1
    # select: capacity too small for top-k, bad mode, bad threshold
    rc = L.seer_select_blocks(ctypes.byref(d), A, A, A, 1, 52, 0.0, 52, A, A, None)
    assert rc == 1
    rc = L.seer_select_blocks(ctypes.byref(d), A, A, A, 7, 52, 0.0, 53, A, A, None)
    assert rc == 1
    rc = L.seer_select_blocks(ctypes.byref(d), A, A, A, 2, 0, 1.5, 512, A, A, None)
    assert rc == 1
    rc = L.seer_select_blocks(ctypes.byref(d), A, A, A, 2, 0, 0.01, 511, A, A, None)
    assert rc == 1
    big = S.make_dims(1, 8, 8, 128, 128, 64, 1 << 20)
    rc = L.seer_select_blocks(ctypes.byref(big), A, A, A, 1, 4, 0.0, 5, A, A, None)
    assert rc == 2
    # kcomp / gate argument checks
    rc = L.seer_kcomp_update(ctypes.byref(d), A, A, A, A, A, 0, 10000.0, None)
    assert rc == 1
    rc = L.seer_kcomp_update(ctypes.byref(d), A, A, A, A, A, 1, -1.0, None)
    assert rc == 1
    rc = L.seer_gate_scores(ctypes.byref(d), A, A, A, A, A, 10000.0, A, 8, A, None)
    assert rc == 3
    # dims.reserved must be zero
    d2 = S.make_dims(16, 40, 8, 128, 128, 64, 32768)
    d2.reserved = 3
    rc = L.seer_gate_scores(ctypes.byref(d2), A, A, A, A, A, 10000.0, A, 10 ** 9, A, None)
    assert rc == 1


def test_host_only_sizes(S):
    d = S.make_dims(16, 40, 8, 128, 128, 64, 32768)
    assert S.seer_gate_workspace_bytes(d) == 16 * 8 * 128 * 4
    assert S.seer_decode_workspace_bytes(d, 53, 1) == 0
    assert S.seer_decode_workspace_bytes(d, 53, 4) == 512 + 10240 + 128 * 4 * 5 * 128 * 4
    assert S.seer_workspace_bytes(d, 53, 4) == S.seer_decode_workspace_bytes(d, 53, 4)


def test_checks_build_and_pass_under_host_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "abi_host_check"
    src = [os.path.join(ROOT, "tests", "abi_host_check.cpp"),
           os.path.join(ROOT, "block_sparse_attention_seer_amd", "csrc", "seer_checks.cpp")]
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), *src, "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout + run.stderr
