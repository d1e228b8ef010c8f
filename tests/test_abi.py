"""The C ABI library loads, exports every declared symbol and validates its
arguments on the host (CPU only: nothing here launches a kernel)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashkm.h")
LIB = os.path.join(ROOT, "exact_means_clustering_amd", "libflashkm.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from exact_means_clustering_amd.build import build
        build()
    return ctypes.CDLL(LIB)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"KM_API\s+[\w\s\*]+?\b(kmeans_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    assert set(declared_symbols()) == {
        "kmeans_workspace_bytes", "kmeans_assign", "kmeans_update", "kmeans_fit", "kmeans_fit_streamed",
        "kmeans_last_error"}


def test_every_declared_symbol_is_exported(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


def _sig(lib):
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kmeans_workspace_bytes.argtypes = [i64, i32, i32, i32, i32]
    lib.kmeans_workspace_bytes.restype = sz
    lib.kmeans_assign.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P, sz, P]
    lib.kmeans_update.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P, sz, P]
    lib.kmeans_fit.argtypes = [P, i32, i64, i32, i32, P, i32, i32, P, P, P, P, P, sz, P]
    lib.kmeans_fit_streamed.argtypes = [P, i32, i64, i32, P, i32, i32, sz, P, P, P, P, P]
    lib.kmeans_last_error.restype = ctypes.c_char_p
    return lib


def test_workspace_bytes(lib):
    lib = _sig(lib)
    assert lib.kmeans_workspace_bytes(10, 128, 20, 1, 2) == 0          # K > N
    assert lib.kmeans_workspace_bytes(100, 100, 20, 1, 2) == 0         # unsupported D
    assert lib.kmeans_workspace_bytes(100, 128, 20, 1, 7) == 0         # bad dtype
    assert lib.kmeans_workspace_bytes(100, 128, 0, 1, 2) == 0          # K < 1
    assert lib.kmeans_workspace_bytes(100, 128, 20, 0, 2) == 0         # B < 1
    assert lib.kmeans_workspace_bytes(1 << 30, 128, 20, 2, 2) == 0     # B*N >= 2^31
    a = lib.kmeans_workspace_bytes(1 << 20, 128, 1024, 1, 1)
    b = lib.kmeans_workspace_bytes(1 << 21, 128, 1024, 1, 1)
    assert 0 < a < b and a % 256 == 0
    # the workspace holds no O(N*K) buffer: it grows linearly in N and K
    big = lib.kmeans_workspace_bytes(1 << 23, 128, 65536, 1, 2)
    assert big < 64 * (1 << 23) + 1024 * 65536


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first


def test_validation_codes(lib):
    lib = _sig(lib)
    # (status, message fragment) for calls that must fail before touching the device
    assert lib.kmeans_assign(FAKE, 2, 10, 128, 1, FAKE, 20, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert b"N >= K" in lib.kmeans_last_error()
    assert lib.kmeans_assign(FAKE, 2, 100, 96, 1, FAKE, 20, FAKE, None, None, FAKE, 1 << 30, None) == 2
    assert lib.kmeans_assign(FAKE, 5, 100, 128, 1, FAKE, 20, FAKE, None, None, FAKE, 1 << 30, None) == 2
    assert lib.kmeans_assign(None, 2, 100, 128, 1, FAKE, 20, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_assign(ctypes.c_void_p((1 << 20) + 8), 2, 100, 128, 1, FAKE, 20, FAKE, None, None, FAKE,
                             1 << 30, None) == 1                              # X not 16-byte aligned
    assert lib.kmeans_assign(FAKE, 2, 100, 128, 1, FAKE, 20, FAKE, None, None, FAKE, 16, None) == 3
    assert b"workspace too small" in lib.kmeans_last_error()
    assert lib.kmeans_update(FAKE, 1, 100, 128, 1, None, 20, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_update(FAKE, 1, 100, 128, 1, FAKE, 20, FAKE, FAKE, None, FAKE, 0, None) == 3
    assert lib.kmeans_update(FAKE, 1, 100, 128, 1, FAKE, 20, ctypes.c_void_p((1 << 20) + 4), FAKE, None, FAKE,
                             1 << 30, None) == 1                              # C_prev not 16-byte aligned
    assert lib.kmeans_fit(FAKE, 0, 100, 32, 1, FAKE, 20, 3, FAKE, ctypes.c_void_p((1 << 20) + 8), FAKE, None, FAKE,
                          1 << 30, None) == 1                                 # C_out not 16-byte aligned
    assert lib.kmeans_fit(FAKE, 0, 100, 32, 1, FAKE, 20, 0, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert b"iters" in lib.kmeans_last_error()
    assert lib.kmeans_fit(FAKE, 0, 100, 32, 1, FAKE, 20, 3, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_fit(FAKE, 0, 100, 32, 1, FAKE, 20, 3, FAKE, FAKE, FAKE, None, ctypes.c_void_p((1 << 20) + 64),
                          1 << 30, None) == 1                                 # workspace not 256-aligned
    assert lib.kmeans_fit_streamed(None, 1, 100, 128, FAKE, 20, 2, 1 << 30, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.kmeans_fit_streamed(FAKE, 1, 100, 128, FAKE, 20, 0, 1 << 30, FAKE, FAKE, FAKE, None, None) == 1
    assert lib.kmeans_fit_streamed(FAKE, 1, 100, 120, FAKE, 20, 2, 1 << 30, FAKE, FAKE, FAKE, None, None) == 2


def test_binding_has_no_cpu_fallback():
    """The binding loads the HIP library and exposes only ABI wrappers."""
    import exact_means_clustering_amd as km
    assert km.lib_path() == LIB
    src = open(os.path.join(ROOT, "exact_means_clustering_amd", "__init__.py")).read()
    assert "oracle" not in src and "numpy" not in src
