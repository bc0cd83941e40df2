"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and its host-only functions agree with the oracle.  No GPU call."""

import ctypes
import os
import re
import subprocess

import pytest

import oracle
from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ar.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ar_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for must in ("ar_create", "ar_allreduce", "ar_reduce_scatter", "ar_allgather", "ar_destroy"):
        assert must in names


def test_library_exports_every_declared_symbol():
    import ring_allreduce_rs_amd as ar
    lib = ctypes.CDLL(ar.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert sorted(ar.EXPORTS) == _declared()
    out = subprocess.run(["nm", "-D", "--defined-only", ar.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared()) <= exported
    # nothing but the ABI is exported as a C function of ours
    ours = {s for s in exported if s.startswith("ar_")}
    assert ours == set(_declared())


def test_built_for_gfx950():
    # the embedded offload bundle names its target
    import ring_allreduce_rs_amd as ar
    blob = open(ar.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 8, 16, 64])
def test_chunk_range_matches_oracle_layout(n):
    import ring_allreduce_rs_amd as ar
    for count in (0, 1, n - 1, n, n + 1, 1000, 6_553_600, 268_435_459, 1 << 30, (1 << 40) + 3):
        lay = oracle.chunk_layout(count, n)
        for c in range(n):
            assert ar.chunk_range(count, n, c) == lay[c]


@pytest.mark.parametrize("n", [2, 3, 63, 64])
def test_chunk_range_near_size_max(n):
    """Counts near 2^64 - 1: the ceiling split must hold exactly (no wrap in
    c*L or lo + L); the oracle's layout uses Python integers."""
    import ring_allreduce_rs_amd as ar
    top = (1 << 64) - 1
    for count in (top, top - 1, top - n, (1 << 63) + 1):
        lay = oracle.chunk_layout(count, n)
        got = [ar.chunk_range(count, n, c) for c in range(n)]
        assert got == lay
        assert sum(ln for _, ln in got) == count
    # the case that once wrapped: 2 ranks, chunk 1 of 2^64 - 1 elements
    assert ar.chunk_range(top, 2, 1) == (1 << 63, (1 << 63) - 1)


def test_chunk_range_rejects_bad_arguments():
    import ring_allreduce_rs_amd as ar
    for count, n, c in ((10, 0, 0), (10, 65, 0), (10, 4, 4), (10, 4, -1)):
        with pytest.raises(ar.ArError) as e:
            ar.chunk_range(count, n, c)
        assert e.value.status == 1


def test_status_strings_and_null_handles():
    import ring_allreduce_rs_amd as ar
    lib = ar.lib
    names = [lib.ar_status_string(s).decode() for s in range(5)]
    assert names == ["AR_OK", "AR_ERR_INVALID_ARG", "AR_ERR_UNSUPPORTED", "AR_ERR_RUNTIME",
                     "AR_ERR_NO_MEMORY"]
    assert lib.ar_status_string(99).decode() == "AR_ERR_UNKNOWN"
    assert lib.ar_destroy(None) == 0
    assert lib.ar_last_error(None) is not None
    # NULL context is rejected before anything touches a GPU
    arr = (ctypes.c_void_p * 2)(0, 0)
    assert lib.ar_allreduce(None, arr, 2, 4, 1, 0, 1) == 1
    assert lib.ar_reduce_scatter(None, arr, 2, 4, 1, 0, 1) == 1
    assert lib.ar_allgather(None, arr, 2, 4, 1, 1) == 1
    assert lib.ar_ring_rs_step(None, arr, 2, 4, 1, 0, 0) == 1
    assert lib.ar_ring_ag_step(None, arr, 2, 4, 1, 0) == 1
    assert lib.ar_tree_step(None, arr, 2, 4, 1, 0, 0) == 1
    assert lib.ar_copy(None, None, None, 16) == 1
    assert lib.ar_set_stream(None, None) == 1
    assert lib.ar_set_graphs(None, 1) == 1
    assert lib.ar_set_residency_caps(None, 0) == 1
    assert lib.ar_create(None, 0, None) == 1


def test_package_fails_loudly_without_the_library(tmp_path):
    # importing the binding from a copy without libar.so must raise, not fall back
    import shutil
    import sys
    pkg = tmp_path / "ring_allreduce_rs_amd"
    shutil.copytree(os.path.join(ROOT, "ring_allreduce_rs_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n import ring_allreduce_rs_amd\nexcept ImportError as e:\n print('RAISED', e)\n"
            % str(tmp_path))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert "RAISED" in out.stdout and "not built" in out.stdout
