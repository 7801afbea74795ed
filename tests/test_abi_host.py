"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before touching the device (no kernels are launched)."""
import ctypes
import os
import re

import pytest

from long_context_sparse_index_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = 0x100000  # a 16-byte aligned address that is never dereferenced here


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.library_path()):
        pytest.fail("libdsa.so not built (run python -m long_context_sparse_index_amd.build)")
    return dsa.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert set(names) == set(dsa.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.dsa_abi_version() == 4
    for s in range(9):
        assert L.dsa_status_string(s)
    assert L.dsa_status_string(99) == b"unknown status"


def _batch(T=4, B=1, max_ctx=100):
    return dsa._CBatch(T, B, max_ctx, 0, FAKE, FAKE, FAKE)


def test_index_scores_validation(L):
    b = _batch()
    f = L.dsa_index_scores
    assert f(None, FAKE, FAKE, FAKE, FAKE, 100, None) == 1
    assert f(ctypes.byref(b), None, FAKE, FAKE, FAKE, 100, None) == 1
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 96, None) == 2      # ld < max_ctx
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 102, None) == 3     # ld % 4
    assert f(ctypes.byref(b), FAKE + 2, FAKE, FAKE, FAKE, 100, None) == 3  # misaligned bf16
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE + 4, 100, None) == 3  # misaligned scores
    bad = _batch(T=-1)
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 100, None) == 2
    bad = _batch(B=0)
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 100, None) == 2
    bad = dsa._CBatch(4, 1, 100, 0, FAKE, FAKE, FAKE, None, 0, 3)  # unknown kv_format
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 100, None) == 5
    bad = dsa._CBatch(4, 1, 100, 0, None, FAKE, FAKE)
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, 100, None) == 1
    empty = _batch(T=0)
    assert f(ctypes.byref(empty), FAKE, FAKE, FAKE, FAKE, 100, None) == 0  # empty call: no-op


def test_topk_validation(L):
    b = _batch()
    f = L.dsa_topk
    assert f(ctypes.byref(b), FAKE, 100, 0, FAKE, None, 0, None) == 2
    assert f(ctypes.byref(b), FAKE, 100, 8193, FAKE, None, 0, None) == 2
    assert f(ctypes.byref(b), FAKE, 100, 16, None, None, 0, None) == 1
    assert f(ctypes.byref(b), None, 100, 16, FAKE, None, 0, None) == 1
    assert f(ctypes.byref(_batch(T=0)), FAKE, 100, 16, FAKE, None, 0, None) == 0


def test_sparse_mla_validation(L):
    b = _batch()
    f = L.dsa_sparse_mla_attn
    args = [FAKE] * 6
    need = L.dsa_workspace_bytes(dsa.OP_SPARSE_MLA, 4, 100, 2048)
    assert need > 0
    assert f(ctypes.byref(b), *args, 2048, 0.0625, FAKE, 0, FAKE, need - 1, None) == 4   # workspace
    assert f(ctypes.byref(b), *args, 2048, 0.0625, FAKE, 5, FAKE, need, None) == 5       # out dtype
    assert f(ctypes.byref(b), *args, 2048, -1.0, FAKE, 0, FAKE, need, None) == 2         # scale
    assert f(ctypes.byref(b), *args, 8193, 0.0625, FAKE, 0, FAKE, need, None) == 2       # k
    assert f(ctypes.byref(b), *args, 2048, 0.0625, FAKE, 0, None, need, None) == 1       # ws NULL
    assert f(ctypes.byref(b), *args, 2048, 0.0625, FAKE, 0, FAKE + 8, need, None) == 3   # ws align


def test_forward_validation(L):
    b = _batch()
    f = L.dsa_forward
    args = [FAKE] * 8
    one = L.dsa_workspace_bytes(dsa.OP_FORWARD, 1, 100, 2048)
    assert 0 < one <= L.dsa_workspace_bytes(dsa.OP_FORWARD, 4, 100, 2048)
    assert f(ctypes.byref(b), *args, 2048, 0.0625, FAKE, 0, None, FAKE, one - 1, None) == 4
    assert f(ctypes.byref(b), *args, 0, 0.0625, FAKE, 0, None, FAKE, one, None) == 2
    assert f(ctypes.byref(b), *args[:-1], None, 2048, 0.0625, FAKE, 0, None, FAKE, one, None) == 1


def test_workspace_bytes(L):
    assert L.dsa_workspace_bytes(dsa.OP_INDEX_SCORES, 8, 1000, 2048) == 0
    assert L.dsa_workspace_bytes(dsa.OP_TOPK, 8, 1000, 2048) > 0        # few rows: split path
    assert L.dsa_workspace_bytes(dsa.OP_TOPK, 4096, 1000, 2048) == 0     # many rows: one workgroup each
    assert L.dsa_workspace_bytes(dsa.OP_SPARSE_MLA, 8, 1000, 0) == 0        # invalid k
    assert L.dsa_workspace_bytes(99, 8, 1000, 16) == 0
    # decode (8 queries): q_lat + o_lat (64 KB each per query) + split partials
    mla8 = L.dsa_workspace_bytes(dsa.OP_SPARSE_MLA, 8, 204800, 2048)
    assert mla8 >= 8 * 2 * 64 * 512 * 2
    fwd = L.dsa_workspace_bytes(dsa.OP_FORWARD, 8, 204800, 2048)
    assert fwd >= mla8 + 8 * 204800 * 4 + 8 * 2048 * 4


def test_valid_call_without_gpu_reports_device_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the no-device path")
    b = _batch()
    assert L.dsa_index_scores(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 100, None) == 7


def test_index_share_schedule_matches_oracle(L):
    """Host-only call: the library's IndexShare schedule equals the oracle's
    for the page's configuration and a sweep of others; bad sizes are rejected."""
    from oracle import dsa_oracle as O
    for layers, dense, freq in [(78, 3, 4)] + [(n, d, f) for n in (1, 2, 5, 17, 40) for d in (1, 2, 3)
                                               for f in (1, 2, 3, 4, 8) if d <= n]:
        assert dsa.dsa_index_share_schedule(layers, dense, freq) == O.index_share_schedule(layers, dense, freq)
    src = (ctypes.c_int32 * 4)(-7, -7, -7, -7)
    assert L.dsa_index_share_schedule(4, 1, 2, None) == 1
    assert L.dsa_index_share_schedule(0, 1, 2, src) == 2
    assert L.dsa_index_share_schedule(4, 0, 2, src) == 2
    assert L.dsa_index_share_schedule(4, 5, 2, src) == 2
    assert L.dsa_index_share_schedule(4, 1, 0, src) == 2
    assert list(src) == [-7] * 4  # nothing written on error


def test_paged_batch_validation(L):
    """Paged layout: page size a power of two in 16 .. 2^20, a block table with
    enough pages per sequence; seq_row0 may then be NULL."""
    f = L.dsa_index_scores

    def call(page_size, table, max_pages, seq_row0=None, kv_format=0):
        b = dsa._CBatch(4, 2, 100, page_size, FAKE, FAKE, seq_row0, table, max_pages, kv_format)
        return f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 100, None)

    if not _gpu():  # valid layouts pass every check; without a GPU the device check answers
        assert call(16, FAKE, 7) == 7         # 7 * 16 >= 100
        assert call(64, FAKE, 2) == 7
    assert call(16, FAKE, 6) == 2             # 96 < 100 tokens
    assert call(48, FAKE, 4) == 2             # not a power of two
    assert call(8, FAKE, 16) == 2             # below 16
    assert call(1 << 21, FAKE, 1) == 2        # above 2^20
    assert call(-16, FAKE, 7) == 2
    assert call(16, None, 7) == 1             # block table required
    assert call(16, FAKE, 7, kv_format=2) == 5
    b = dsa._CBatch(4, 2, 100, 0, FAKE, FAKE, None, FAKE, 7, 0)  # contiguous needs seq_row0
    assert f(ctypes.byref(b), FAKE, FAKE, FAKE, FAKE, 100, None) == 1


def _gpu():
    import torch
    return torch.cuda.is_available()


def test_quantize_kv_int4_validation(L):
    f = L.dsa_quantize_kv_int4
    assert f(FAKE, 0, FAKE, None) == 0          # empty: nothing enqueued
    assert f(FAKE, -1, FAKE, None) == 2
    assert f(FAKE, (1 << 40) + 1, FAKE, None) == 2
    assert f(None, 4, FAKE, None) == 1
    assert f(FAKE, 4, None, None) == 1
    assert f(FAKE + 8, 4, FAKE, None) == 3
    assert f(FAKE, 4, FAKE + 4, None) == 3


def test_forward_noalloc_validation(L):
    """The no-allocation forward checks its arguments like dsa_forward (no workspace
    argument: its workspace is the library's static per-device scratch)."""
    b = _batch()
    f = L.dsa_forward_noalloc
    args = [FAKE] * 8
    assert f(None, *args, 2048, 0.0625, FAKE, 0, None, None) == 1
    assert f(ctypes.byref(b), *args, 0, 0.0625, FAKE, 0, None, None) == 2
    assert f(ctypes.byref(b), *args, 8193, 0.0625, FAKE, 0, None, None) == 2
    assert f(ctypes.byref(_batch(T=0)), *args, 2048, 0.0625, FAKE, 0, None, None) == 0
    # the largest single-query workspace fits the 64 MiB scratch
    assert L.dsa_workspace_bytes(dsa.OP_FORWARD, 1, 1 << 21, 8192) <= 64 << 20
    if not _gpu():
        assert f(ctypes.byref(b), *args, 2048, 0.0625, FAKE, 0, None, None) == 7


def test_check_device_args_validation(L):
    b = _batch()
    f = L.dsa_check_device_args
    assert f(None, None, 0, 0, FAKE, None) == 1
    assert f(ctypes.byref(b), None, 0, 0, None, None) == 1          # flags NULL
    assert f(ctypes.byref(b), None, 0, 0, FAKE + 2, None) == 3      # flags misaligned
    assert f(ctypes.byref(b), FAKE, 0, 0, FAKE, None) == 2          # idx given, k 0
    assert f(ctypes.byref(b), FAKE, 8193, 0, FAKE, None) == 2
    assert f(ctypes.byref(b), None, 0, -1, FAKE, None) == 2         # cache_rows < 0
    if not _gpu():
        assert f(ctypes.byref(b), FAKE, 16, 1000, FAKE, None) == 7
    assert L.dsa_last_device_arg_flags() == 0
    assert L.dsa_status_string(8).startswith(b"a device-side argument")
