"""CPU-side checks of the C ABI: the library loads, exports every entry point
the header declares, and rejects invalid arguments on the host before any
device work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "staple.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(staple_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from token_indexed_ffn_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libstaple.so is not built (run `python -m token_indexed_ffn_amd.build`)")
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("staple_ffn_fwd", "staple_ffn_bwd_table_grad", "staple_cache_build",
                 "staple_cache_lookup", "staple_dedup"):
        assert must in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    from token_indexed_ffn_amd import _lib
    assert sorted(_lib.EXPORTED) == declared_functions()


def test_status_strings(lib):
    assert lib.staple_status_string(0) == b"ok"
    for st in range(-7, 0):
        assert lib.staple_status_string(st) not in (b"ok", b"unknown status")
    assert b"gfx950" in lib.staple_version()


def test_workspace_queries(lib):
    # radix sort: two buffers of 8-byte (key, value) pairs, digit histograms
    # (256 bins x 64 workgroups) and 64 per-workgroup run counts; up to 4096
    # positions the whole dedup runs in one workgroup's LDS
    pairs = lambda n: (n * 8 + 255) // 256 * 256
    radix = lambda n: 2 * pairs(n) + 256 * 64 * 4 + 64 * 4
    assert lib.staple_dedup_workspace_bytes(64) == 0
    assert lib.staple_dedup_workspace_bytes(4096) == 0
    assert lib.staple_dedup_workspace_bytes(32768) == radix(32768)
    assert lib.staple_dedup_workspace_bytes(4097) == radix(4097)
    # the prefill chunk rows: the dedup's workspace
    assert lib.staple_prefill_rows_workspace_bytes(4096) == 0
    assert lib.staple_prefill_rows_workspace_bytes(8192) == radix(8192)
    dgu = ((100 * 256 * 2 + 255) // 256) * 256          # [dg | du] in bf16
    aux = ((100 * 128 * 4 + 255) // 256) * 256           # fp32 du, then a recomputed h
    partials = 2 * ((100 + 31) // 32) * 128 * 4            # segment-sum chunk partials
    # bf16: K-major copies W_down^T [f x d], [W_gate^T | W_up^T] [d x 2f], dy^T [d x 128]
    kt = 128 * 64 * 2 + 64 * 256 * 2 + 64 * 128 * 2
    assert lib.staple_ffn_bwd_workspace_bytes(100, 64, 128, 1) == dgu + aux + partials + kt
    assert lib.staple_ffn_bwd_workspace_bytes(100, 64, 128, 0) == 2 * dgu + aux + partials
    assert lib.staple_ffn_fwd_workspace_bytes(100, 64, 100, 1) == 0   # d_ff not a multiple of 64
    assert lib.staple_cache_build_workspace_bytes(100352) == radix(100352)
    # decode forward: [h][split-K partials, 8 splits of n x d_model fp32]
    h = 64 * 8192 * 2
    down = 8 * 64 * 2048 * 4
    assert lib.staple_ffn_down_workspace_bytes(64, 2048, 8192, 1) == down
    assert lib.staple_ffn_fwd_workspace_bytes(64, 2048, 8192, 1) == h + down
    assert lib.staple_ffn_down_workspace_bytes(65, 2048, 8192, 1) == 0   # tiled GEMM, no partials
    # decode step driver: [dedup (none at 64 tokens)][row sources, n int32 in 256 B][h][partials]
    assert lib.staple_decode_step_workspace_bytes(64, 2048, 8192) == 256 + h + down
    assert lib.staple_decode_step_workspace_bytes(65, 2048, 8192) == 0   # past a decode batch


def test_invalid_arguments_are_rejected_before_device_work(lib):
    null = None
    # negative token count
    assert lib.staple_dedup(null, -1, 10, null, null, null, null, null, null, 0, null) == -1
    # missing outputs
    assert lib.staple_dedup(null, 0, 10, null, null, null, null, null, null, 0, null) == -1
    # unsupported dtype / shape
    assert lib.staple_ffn_fwd(4, 64, 128, 7, 0, *([null] * 5), 1, null, null, null, null, null,
                              null, 0, null) == -2
    assert lib.staple_ffn_fwd(4, 60, 128, 1, 1, *([null] * 5), 1, null, null, null, null, null,
                              null, 0, null) == -2
    # capacity beyond the vocabulary
    assert lib.staple_cache_build(null, 10, 11, null, null, null, 0, null) == -1
    # host-side check of miss IDs: an out-of-range ID is refused, nothing copied
    import numpy as np
    table = np.zeros((4, 8), dtype=np.float32)
    ids = np.array([1, 9], dtype=np.int32)
    stage = np.zeros((2, 8), dtype=np.float32)
    st = lib.staple_stage_misses(table.ctypes.data, 4, 8, 0, ids.ctypes.data, 2,
                                 stage.ctypes.data, 1, null)
    assert st == -6
    assert np.all(stage == 0)


def test_stage_misses_dma_rejects_before_any_copy(lib):
    import numpy as np
    table = np.zeros((4, 8), dtype=np.float32)
    ids = np.array([1, 9], dtype=np.int32)
    stage = np.zeros((2, 8), dtype=np.float32)
    tabs = (ctypes.c_void_p * 1)(table.ctypes.data)
    dst = (ctypes.c_void_p * 1)(16)   # never dereferenced: every case fails (or ends) first

    def call(n_layers=1, stride=0, vocab=4, d_ff=8, dtype=0, n_miss=2, t=tabs, d=dst):
        return lib.staple_stage_misses_dma(n_layers, ctypes.cast(t, ctypes.c_void_p) if t else None,
                                           stride, vocab, d_ff, dtype, ids.ctypes.data, n_miss,
                                           stage.ctypes.data,
                                           ctypes.cast(d, ctypes.c_void_p) if d else None)
    assert call(n_layers=0) == -1   # no layers
    assert call(stride=4) == -1     # a row stride shorter than a row
    assert call(dtype=7) == -1      # dtype
    assert call(t=None) == -1       # no tables
    assert call(d=None) == -1       # no destinations
    assert call(n_miss=0) == 0      # nothing to copy
    assert call() == -6             # ID 9 outside the vocabulary of 4: refused on the host
    assert np.all(stage == 0)


def test_prefill_rows_rejects_bad_arguments_before_device_work(lib):
    null, p = None, 16   # any non-null address: nothing is dereferenced before the checks
    outs = [p] * 8

    def call(n_layers, layers, n, d_ff, dtype=0, vocab=100, cap=0, wgs=0, ws_bytes=0, lookup=1):
        return lib.staple_prefill_rows_cached(n_layers, layers, n, d_ff, dtype, p, vocab, p, cap,
                                              lookup, wgs, *outs, null, ws_bytes, null)
    assert call(1, p, 0, 256) == -1            # no tokens
    assert call(0, p, 64, 256) == -1           # no layers
    assert call(1, null, 64, 256) == -1        # no descriptors
    assert call(1, p, 64, 256, dtype=7) == -1  # dtype
    assert call(1, p, 64, 4, dtype=1) == -1    # a bf16 row that is not whole 16-byte vectors
    assert call(1, p, 64, 256, wgs=-1) == -1   # workgroup cap
    assert call(1, p, 64, 256, cap=-1) == -1   # capacity
    assert call(1, p, 64, 256, lookup=2) == -1 # lookup is 0 or 1
    assert call(1, p, 8192, 256) == -3         # no workspace for the multi-workgroup dedup


def test_header_compiles_as_c99_and_cpp(tmp_path):
    """The boundary is a C ABI: the header alone compiles as strict C99 and as C++."""
    import shutil
    import subprocess
    inc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
    src = tmp_path / "use.c"
    src.write_text('#include "staple.h"\n'
                   "int main(void) { staple_row_source_t r = {0}; (void)r;\n"
                   "  return (int)staple_dedup_workspace_bytes(0); }\n")
    for cc, args in (("gcc", ["-std=c99", "-pedantic", "-Werror"]),
                     ("g++", ["-std=c++17", "-Werror", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not found")
        r = subprocess.run([cc, *args, "-Wall", "-I", inc, "-fsyntax-only", str(src)],
                           capture_output=True, text=True, timeout=60)
        assert r.returncode == 0, r.stderr
