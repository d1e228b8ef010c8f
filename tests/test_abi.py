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
        import __graft_entry__
        __graft_entry__.build()
    return ctypes.CDLL(LIB)


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"KM_API\s+[\w\s\*]+?\b(kmeans_\w+)\s*\(", text)


def test_header_declares_the_entry_points():
    assert set(declared_symbols()) == {
        "kmeans_workspace_bytes", "kmeans_assign", "kmeans_update", "kmeans_fit", "kmeans_fit_streamed",
        "kmeans_assign_top2", "kmeans_assign_soft", "kmeans_gauss_sum", "kmeans_seed", "kmeans_tune", "kmeans_tune_save",
        "kmeans_tune_load", "kmeans_assign_configs", "kmeans_assign_noalloc", "kmeans_stream_timeline",
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
    lib.kmeans_tune.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, sz, P, P, P, P]
    lib.kmeans_assign_top2.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, sz, P]
    lib.kmeans_assign_soft.argtypes = [P, i32, i64, i32, i32, P, i32, P, ctypes.c_float, P, P, P, P, sz, P]
    lib.kmeans_gauss_sum.argtypes = [P, i32, i64, i32, i32, P, i32, P, ctypes.c_float, P, P, P, sz, P]
    lib.kmeans_seed.argtypes = [P, i32, i64, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    lib.kmeans_tune_save.argtypes = [ctypes.c_char_p]
    lib.kmeans_tune_load.argtypes = [ctypes.c_char_p]
    lib.kmeans_assign_configs.argtypes = [i32, i32, P, P, i32, P]
    lib.kmeans_assign_noalloc.argtypes = [P, i32, i64, i32, i32, P, i32, P, P, P, P]
    lib.kmeans_last_error.restype = ctypes.c_char_p
    return lib


def test_assign_configs_query(lib):
    """The compiled configurations per row size: (1, 4) everywhere; deeper
    blocking only where the point fragments fit the registers (rows of at most
    256 bytes for (2, 8), (4, 4) and the 16-bit (3, 8); 128 bytes for fp32 at
    (3, 8); 512 bytes for (2, 4) and (1, 8))."""
    lib = _sig(lib)

    def q(dt, d):
        pb, w, n = (ctypes.c_int32 * 8)(), (ctypes.c_int32 * 8)(), ctypes.c_int32(-1)
        assert lib.kmeans_assign_configs(dt, d, pb, w, 8, ctypes.byref(n)) == 0
        return {(pb[i], w[i]) for i in range(n.value)}

    every = {(4, 4), (3, 8), (2, 8), (2, 4), (1, 8), (1, 4)}
    assert q(2, 128) == every                      # bf16, 256-byte rows
    assert q(1, 64) == every                       # fp16, 128-byte rows
    assert q(0, 32) == every                       # fp32, 128-byte rows
    assert q(0, 64) == every - {(3, 8)}            # fp32, 256-byte rows
    assert q(1, 256) == {(2, 4), (1, 8), (1, 4)}   # 512-byte rows
    assert q(0, 256) == {(1, 4)}                   # 1 KB rows
    n = ctypes.c_int32(-1)
    assert lib.kmeans_assign_configs(2, 128, None, None, 0, ctypes.byref(n)) == 0 and n.value == 6
    assert lib.kmeans_assign_configs(2, 100, None, None, 0, ctypes.byref(n)) == 2     # unsupported D
    assert lib.kmeans_assign_configs(9, 128, None, None, 0, ctypes.byref(n)) == 2     # bad dtype
    assert lib.kmeans_assign_configs(2, 128, None, None, 4, ctypes.byref(n)) == 1     # cap > 0, null arrays
    assert lib.kmeans_assign_configs(2, 128, None, None, 0, None) == 1                # null count


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
    # a million one-row instances: the sort histogram grows with the keys, not
    # with the instance count (no per-instance sort tile).  The two bias /
    # weight arrays are padded to a 256-centroid tile per instance
    # (2 * B * 256 * 4 bytes); everything else stays in the hundreds of MB.
    B = 1 << 20
    tiny = lib.kmeans_workspace_bytes(1, 32, 1, B, 0)
    assert 0 < tiny - 2 * B * 256 * 4 < 400 * (1 << 20)


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
    assert lib.kmeans_tune(FAKE, 2, 10, 128, 1, FAKE, 20, FAKE, FAKE, 1 << 30, None, None, None, None) == 1
    assert lib.kmeans_tune(FAKE, 2, 100, 128, 1, FAKE, 20, FAKE, FAKE, 16, None, None, None, None) == 3
    assert lib.kmeans_assign_top2(FAKE, 2, 100, 128, 1, FAKE, 1, FAKE, None, FAKE, 1 << 30, None) == 1   # K < 2
    assert b"K >= 2" in lib.kmeans_last_error()
    assert lib.kmeans_assign_top2(FAKE, 2, 100, 128, 1, FAKE, 5, None, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_assign_top2(FAKE, 2, 100, 128, 1, FAKE, 5, FAKE, None, FAKE, 16, None) == 3
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.kmeans_assign_soft(FAKE, 2, 100, 128, 1, FAKE, 5, None, bad, FAKE, FAKE, None, FAKE, 1 << 30,
                                      None) == 1
        assert b"sigma2" in lib.kmeans_last_error()
    assert lib.kmeans_assign_soft(FAKE, 2, 100, 128, 1, FAKE, 5, None, 1.0, FAKE, None, None, FAKE, 1 << 30,
                                  None) == 1
    assert lib.kmeans_assign_soft(FAKE, 2, 100, 128, 1, FAKE, 5, ctypes.c_void_p((1 << 20) + 2), 1.0, FAKE, FAKE,
                                  None, FAKE, 1 << 30, None) == 1           # log_w misaligned
    assert lib.kmeans_gauss_sum(FAKE, 2, 100, 128, 1, FAKE, 5, None, 1.0, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_gauss_sum(FAKE, 2, 100, 128, 1, FAKE, 5, FAKE, -2.0, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_gauss_sum(FAKE, 2, 100, 128, 1, FAKE, 5, FAKE, 1.0, FAKE, None, FAKE, 16, None) == 3
    assert lib.kmeans_seed(FAKE, 2, 100, 128, 1, 5, 2, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1  # method
    assert b"method" in lib.kmeans_last_error()
    assert lib.kmeans_seed(FAKE, 2, 100, 128, 1, 5, 1, None, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert lib.kmeans_seed(FAKE, 2, 100, 128, 1, 5, 1, ctypes.c_void_p((1 << 20) + 4), FAKE, FAKE, None, FAKE,
                           1 << 30, None) == 1                                 # u not 8-byte aligned
    assert lib.kmeans_seed(FAKE, 2, 4, 128, 1, 5, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1   # K > N


def _table(lib, path):
    assert lib.kmeans_tune_save(str(path).encode()) == 0, lib.kmeans_last_error()
    return [" ".join(l.split()) for l in path.read_text().splitlines() if l.strip() and not l.startswith("#")]


def test_tuning_table_files(lib, tmp_path):
    """The tuning table's text format: round trip, comments, all-or-nothing
    loading, and rejection (naming the line) of malformed lines, unsupported
    shapes and configurations not compiled for the row size."""
    lib = _sig(lib)
    good = tmp_path / "good.txt"
    good.write_text("# a comment\n2 128 8388608 1 65536 2 8\n\n1 32 1000 3 7 1 4   # trailing comment\n")
    assert lib.kmeans_tune_load(str(good).encode()) == 0, lib.kmeans_last_error()
    rows = _table(lib, tmp_path / "out1.txt")
    assert "2 128 8388608 1 65536 2 8" in rows and "1 32 1000 3 7 1 4" in rows
    # a later entry for the same shape replaces the earlier one
    (tmp_path / "repl.txt").write_text("1 32 1000 3 7 1 8\n")
    assert lib.kmeans_tune_load(str(tmp_path / "repl.txt").encode()) == 0
    rows = _table(lib, tmp_path / "out2.txt")
    assert "1 32 1000 3 7 1 8" in rows and "1 32 1000 3 7 1 4" not in rows
    cases = [
        ("2 64 500 1 10 2 8\n2 64 500 1\n", b":2:"),          # too few fields (line 1 must not be added)
        ("2 64 500 1 10 2 8 9\n", b":1:"),                     # too many fields
        ("2 96 500 1 10 1 4\n", b"unsupported shape"),          # D not supported
        ("2 64 5 1 10 1 4\n", b"unsupported shape"),            # N < K
        ("0 256 500 1 10 2 8\n", b"not compiled"),              # fp32 D=256 rows are 1 KB: pb=2 x 8 waves not built
        ("2 64 500 1 10 3 4\n", b"not compiled"),              # no (3 blocks, 4 waves) configuration
        ("0 64 500 1 10 3 8\n", b"not compiled"),              # fp32 rows of 256 B: 3 blocks would spill
    ]
    for i, (text, msg) in enumerate(cases):
        f = tmp_path / f"bad{i}.txt"
        f.write_text(text)
        assert lib.kmeans_tune_load(str(f).encode()) == 1, text
        assert msg in lib.kmeans_last_error(), (text, lib.kmeans_last_error())
    assert "2 64 500 1 10 2 8" not in _table(lib, tmp_path / "out3.txt")
    assert lib.kmeans_tune_load(str(tmp_path / "missing.txt").encode()) == 1
    assert lib.kmeans_tune_load(None) == 1 and lib.kmeans_tune_save(None) == 1


def test_binding_has_no_cpu_fallback():
    """The binding loads the HIP library and exposes only ABI wrappers."""
    import exact_means_clustering_amd as km
    assert km.lib_path() == LIB
    src = open(os.path.join(ROOT, "exact_means_clustering_amd", "__init__.py")).read()
    assert "oracle" not in src and "numpy" not in src


def test_assign_noalloc_rejects_shapes_beyond_its_scratch(lib):
    """The allocation-free assignment validates on the host before any GPU
    call: a shape whose rounded centroids alone exceed the 32 MiB static
    scratch fails with KM_EWORKSPACE, one that fits passes the size check."""
    lib = _sig(lib)
    fake = ctypes.c_void_p(1 << 20)    # never dereferenced: rejected before any launch
    # K = 65,537 bf16 rows of D = 256: 33.6 MB of rounded centroids > 32 MiB
    rc = lib.kmeans_assign_noalloc(fake, 2, 70000, 256, 1, fake, 65537, fake, None, None, None)
    assert rc == 3, rc
    assert b"32" in lib.kmeans_last_error() or b"scratch" in lib.kmeans_last_error()
    # invalid shapes and pointers keep their usual codes
    assert lib.kmeans_assign_noalloc(fake, 2, 10, 128, 1, fake, 20, fake, None, None, None) == 1       # K > N
    assert lib.kmeans_assign_noalloc(fake, 2, 100, 100, 1, fake, 20, fake, None, None, None) == 2      # bad D
    assert lib.kmeans_assign_noalloc(None, 2, 100, 128, 1, fake, 20, fake, None, None, None) == 1      # null X


def test_stream_timeline_empty_before_any_streamed_fit(lib):
    lib.kmeans_stream_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    n = ctypes.c_int32(-1)
    assert lib.kmeans_stream_timeline(None, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.kmeans_stream_timeline(None, 4, ctypes.byref(n)) == 1           # cap > 0 without a buffer
    assert lib.kmeans_stream_timeline(None, 0, None) == 1                      # null count
