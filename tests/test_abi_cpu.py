"""The C-ABI library loads and exports every entry point include/dsa.h declares (CPU only).

Only host-side helpers are called here (version and workspace-size queries); no entry
point that launches work is called without a GPU.
"""
import ctypes
import os

import pytest

from dsa_sparse_attention_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libdsa.so not built (run __graft_entry__.build())")


def test_header_declares_the_four_calls_and_helpers():
    names = set(_lib.header_symbols())
    for n in ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_decode", "greedy_accept",
              "dsa_quantize_fp8", "dsa_verify_cache_write", "dsa_abi_version",
              "dsa_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    missing = [n for n in _lib.header_symbols() if not hasattr(lib, n)]
    assert not missing, f"declared but not exported: {missing}"
    assert set(_lib.SIGNATURES) == set(_lib.header_symbols())


def test_version_and_workspace_queries():
    lib = _lib.load()
    assert lib.dsa_abi_version() == 7
    assert lib.dsa_last_error() in (b"", None)
    assert lib.dsa_topk_workspace_size(32, 192, 65536, 2048, 0) == 0
    # the refine keeps one key-scale maximum per 2048 positions of every request
    assert lib.dsa_topk_workspace_size(32, 192, 65536, 2048, 1) == 32 * 32 * 4
    # 262144-position rows: 4 chunks of 2048 indices, then compact scores and positions
    assert lib.dsa_topk_workspace_size(4, 24, 262144, 2048, 0) == (24 * 4 * 2048 + 24 * 8192) * 4
    # with the refine: the scale maxima, then per row the long-row refine's record (48
    # bytes), band positions and exact band scores (4096 x (4 + 8) bytes) and the bitmap of
    # the keys kept above the band (2^18 bits)
    assert lib.dsa_topk_workspace_size(4, 24, 262144, 2048, 1) == (
        (24 * 4 * 2048 + 24 * 8192) * 4 + 4 * 128 * 4 + 24 * (48 + 4096 * 12 + 32768))
    assert lib.dsa_topk_workspace_size(3, 5, 100, 8, 1) == 16  # padded to 16 bytes
    # split-K partials: per (row, split, head) 512 bf16 outputs and a float32 (max, sum),
    # or none when one split suffices
    per = 512 * 2 + 2 * 4
    ws = lib.dsa_sparse_mla_workspace_size(192, 64, 2048)
    assert ws == 0 or ws % (192 * 64 * per) == 0
    # a split holds at most 2048 top-k entries: k = 2048 over many rows needs no partials,
    # k = 4096 needs two splits; few rows are split further (>= 256 entries per split)
    assert lib.dsa_sparse_mla_workspace_size(1024, 64, 2048) == 0
    assert lib.dsa_sparse_mla_workspace_size(1024, 64, 4096) == 1024 * 2 * 64 * per
    assert lib.dsa_sparse_mla_workspace_size(16, 128, 2048) == 16 * 8 * 128 * per
    # greedy accept: one (max, index) pair per 4096-entry vocabulary slice per row
    assert lib.greedy_accept_workspace_size(32, 5, 151552) == 32 * 6 * 37 * 8
    assert lib.greedy_accept_workspace_size(0, 5, 10) == 0


def test_key_scale_table_argument_checks_before_launch():
    # rejected on the host, before any HIP call (so this runs without a GPU)
    lib = _lib.load()
    assert lib.dsa_key_scale_max(None, 100, 10, 101, None, None) == 1  # row_end > N
    assert lib.dsa_key_scale_max(None, 100, 20, 10, None, None) == 1   # row_begin > row_end
    assert lib.dsa_key_scale_max(None, 100, 5, 5, None, None) == 0     # empty range: nothing
    assert lib.dsa_key_scale_max(None, 100, 0, 100, None, None) == 1   # null pointers
    assert b"null" in lib.dsa_last_error()
    # a refine with a table needs its length
    rf = _lib.TopkRefine(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 8, 64, 0.0, None,
                         1 << 20, 0)
    st = lib.dsa_topk(1 << 20, 64, 1 << 20, 1 << 20, 1, 2, 2, 64, 8, ctypes.byref(rf), 1 << 20,
                      None, 0, None)
    assert st == 1 and b"k_scale_max_len" in lib.dsa_last_error()
