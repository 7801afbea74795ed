"""Device-side argument check (dsa_check_device_args, and the DSA_CHECK_DEVICE_ARGS=1
debug mode of the ops).  The check kernel reads only q_seq, q_pos, seq_row0 /
block_table and idx; the out-of-range values below are never used to address
the caches."""
import os

import numpy as np
import pytest
import torch

from long_context_sparse_index_amd import dsa, synth
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


def _batch(q_seq, q_pos, seq_row0, max_ctx, table=None, page=0):
    c = lambda x, dt: torch.tensor(x, dtype=dt, device="cuda")
    if page:
        return dsa.Batch(c(q_seq, torch.int32), c(q_pos, torch.int32), None, max_ctx,
                         block_table=c(table, torch.int32), page_size=page)
    return dsa.Batch(c(q_seq, torch.int32), c(q_pos, torch.int32), c(seq_row0, torch.int64), max_ctx)


def _flags(b, idx=None, rows=0):
    f = dsa.dsa_check_device_args(b, None if idx is None else torch.tensor(idx, dtype=torch.int32, device="cuda"),
                                  rows)
    torch.cuda.synchronize()
    return int(f.item())


def test_check_finds_each_violation():
    print("[argcheck] contiguous caches", flush=True)
    # two sequences of 100 and 50 rows in a 150-row cache
    ok = _batch([0, 1], [99, 49], [0, 100], 100)
    assert _flags(ok) == 0
    assert _flags(ok, [[0, 99, -1], [49, -1, 3]], rows=150) == 0
    assert _flags(_batch([0, 2], [99, 49], [0, 100], 100)) == dsa.ARG_Q_SEQ
    assert _flags(_batch([-1, 1], [99, 49], [0, 100], 100)) == dsa.ARG_Q_SEQ
    assert _flags(_batch([0, 1], [100, 49], [0, 100], 100)) == dsa.ARG_Q_POS
    assert _flags(_batch([0, 1], [-3, 49], [0, 100], 100)) == dsa.ARG_Q_POS
    assert _flags(_batch([0, 1], [99, 50], [0, 100], 100), rows=150) == dsa.ARG_CACHE_ROW
    assert _flags(_batch([0, 1], [99, 49], [0, -1], 100)) == dsa.ARG_CACHE_ROW
    assert _flags(_batch([0, 1], [99, 50], [0, 100], 100), rows=0) == 0   # upper bound unchecked
    assert _flags(ok, [[0, 100, -1], [0, 1, 2]]) == dsa.ARG_IDX            # beyond q_pos
    assert _flags(ok, [[0, 1, 2], [-2, 1, 2]]) == dsa.ARG_IDX              # negative, not -1
    assert _flags(_batch([0, 3], [100, 49], [0, 100], 100), [[0, 1, 2], [60, 1, 2]]) == \
        dsa.ARG_Q_SEQ | dsa.ARG_Q_POS | dsa.ARG_IDX


def test_check_paged_block_table():
    print("[argcheck] paged caches", flush=True)
    # 16-token pages, a pool of 8 pages; sequence 0 uses pages 0..3, sequence 1 pages 0..1
    table = [[5, 2, 7, 0], [3, 6, -1, 99]]
    b = _batch([0, 1], [63, 31], None, 64, table, 16)
    assert _flags(b, rows=8 * 16) == 0                 # entries past a query's pages are not read
    assert _flags(_batch([0, 1], [63, 32], None, 64, table, 16), rows=128) == dsa.ARG_CACHE_ROW  # -1
    bad = [[5, 2, 8, 0], [3, 6, 0, 0]]                 # page 8 is outside the 8-page pool
    assert _flags(_batch([0, 1], [63, 31], None, 64, bad, 16), rows=128) == dsa.ARG_CACHE_ROW
    assert _flags(_batch([0, 1], [63, 31], None, 64, bad, 16), rows=0) == 0


def test_check_of_many_queries_and_empty_batch():
    T = 70000  # more queries than the check's grid: it strides over them
    q_pos = np.full(T, 5, np.int32)
    q_pos[T - 1] = 6
    b = dsa.Batch(torch.zeros(T, dtype=torch.int32, device="cuda"), torch.from_numpy(q_pos).cuda(),
                  torch.zeros(1, dtype=torch.int64, device="cuda"), 6)
    f = dsa.dsa_check_device_args(b)
    torch.cuda.synchronize()
    assert int(f.item()) == dsa.ARG_Q_POS
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    e = dsa.Batch(z, z, torch.zeros(1, dtype=torch.int64, device="cuda"), 1)
    f = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    dsa.dsa_check_device_args(e, flags=f)
    torch.cuda.synchronize()
    assert int(f.item()) == 0


def test_debug_mode_rejects_bad_idx_before_launching():
    """With DSA_CHECK_DEVICE_ARGS=1 a sparse-MLA call whose idx holds a position
    after its query's own (still a row inside the cache) returns
    DSA_ERR_DEVICE_ARGS and leaves the output untouched; valid calls give the
    same results as without the check."""
    print("[argcheck] debug mode", flush=True)
    inp = synth.custom([300, 200], [(0, 299), (1, 150)], seed=81)
    d = to_device(inp)
    good = torch.from_numpy(np.tile(np.arange(64, dtype=np.int32), (2, 1))).cuda()
    bad = good.clone()
    bad[1, 5] = 180  # > q_pos 150, < the sequence's 200 rows
    ref = dsa.dsa_sparse_mla_attn(d.batch, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv, good)
    ref_f, ref_i = dsa.dsa_forward(d.batch, d.q_idx, d.w, d.k_idx, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv, k=64)
    os.environ["DSA_CHECK_DEVICE_ARGS"] = "1"
    try:
        out = torch.full((2, 64, 256), 5.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(dsa.DsaError) as ei:
            dsa.dsa_sparse_mla_attn(d.batch, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv, bad, out=out)
        assert ei.value.status == dsa.ERR_DEVICE_ARGS and ei.value.arg_flags == dsa.ARG_IDX
        torch.cuda.synchronize()
        assert bool((out == 5.0).all())
        got = dsa.dsa_sparse_mla_attn(d.batch, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv, good)
        got_f, got_i = dsa.dsa_forward(d.batch, d.q_idx, d.w, d.k_idx, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv,
                                       k=64)
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(got_f, ref_f) and torch.equal(got_i, ref_i)
    finally:
        del os.environ["DSA_CHECK_DEVICE_ARGS"]
