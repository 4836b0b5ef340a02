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
    for st in range(-6, 0):
        assert lib.staple_status_string(st) not in (b"ok", b"unknown status")
    assert b"gfx950" in lib.staple_version()


def test_workspace_queries(lib):
    assert lib.staple_dedup_workspace_bytes(64) == 0
    assert lib.staple_dedup_workspace_bytes(32768) == 32768 * 8
    assert lib.staple_dedup_workspace_bytes(4097) == 8192 * 8
    dgu = ((100 * 256 * 2 + 255) // 256) * 256          # [dg | du] in bf16
    partials = 2 * ((100 + 31) // 32) * 128 * 4            # segment-sum chunk partials
    assert lib.staple_ffn_bwd_workspace_bytes(100, 64, 128, 1) == dgu + partials
    assert lib.staple_ffn_fwd_workspace_bytes(100, 64, 100, 1) == 0   # d_ff not a multiple of 64
    assert lib.staple_cache_build_workspace_bytes(100352) == 131072 * 8
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
