"""Paged caches on the GPU: the same batch with its caches scattered over a
page pool (NaN in unused pool rows) gives bit-identical scores, selections and
outputs to the contiguous layout, and matches the oracle."""
import types

import numpy as np
import pytest
import torch

from long_context_sparse_index_amd import dsa, synth
from oracle import dsa_oracle as O
from tests.gpu_util import OUT_MAX_ABS, OUT_REL_L2, bf16_dev, check_selection, out_errors, run_forward, to_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def to_device_paged(inp, pc, d_contig):
    d = types.SimpleNamespace(**vars(d_contig))
    d.k_idx = bf16_dev(pc.k_idx)
    d.kv = bf16_dev(pc.kv)
    d.batch = dsa.Batch(d_contig.q_seq, d_contig.q_pos, None, d_contig.batch.max_ctx,
                        block_table=torch.from_numpy(pc.block_table).cuda(), page_size=pc.page_size)
    return d


def _oracle_check(inp, t, idx_row, out_row, k):
    b, p = int(inp.q_seq[t]), int(inp.q_pos[t])
    r0 = int(inp.seq_row0[b])
    s = O.indexer_scores(inp.q_idx[t], inp.w[t], inp.k_idx[r0: r0 + p + 1], p)
    check_selection(idx_row, s, O.topk_select(s, k), k)
    kept = idx_row[idx_row >= 0].astype(np.int64)
    ref = O.mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[r0 + kept], inp.w_uk, inp.w_uv)
    mx, rel = out_errors(out_row, ref)
    assert mx <= OUT_MAX_ABS and rel <= OUT_REL_L2, (t, mx, rel)


CASES = {
    # per-query key scan + split top-k; the 70,000-token row takes the sampled window
    "decode": ([3000, 9000, 70000, 200], [(0, 2999), (1, 8999), (2, 69999), (3, 199), (1, 4000)]),
    # indexer GEMM over blocks of consecutive queries, two sequences, one top-k workgroup per row
    "prefill": ([12000, 5000], [(0, 11960 + i) for i in range(24)] + [(1, 4990 + i) for i in range(10)]),
}


@pytest.mark.parametrize("page_size", [16, 64, 256, 65536])
@pytest.mark.parametrize("case", list(CASES))
def test_paged_forward_equals_contiguous(case, page_size):
    lens, qs = CASES[case]
    _say(f"[paged] {case} page_size={page_size}")
    inp = synth.custom(lens, qs, seed=51)
    pc = synth.to_paged(inp, page_size, seed=page_size)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    sc_c = dsa.dsa_index_scores(dc.batch, dc.q_idx, dc.w, dc.k_idx)
    sc_p = dsa.dsa_index_scores(dp.batch, dp.q_idx, dp.w, dp.k_idx)
    for t, (_, p) in enumerate(qs):  # entries past q_pos are not written
        assert torch.equal(sc_c[t, : p + 1], sc_p[t, : p + 1]), t
    oc, ic = run_forward(dc)
    op, ip = run_forward(dp)
    assert torch.equal(ic, ip)
    assert torch.equal(oc, op)
    mla_p = dsa.dsa_sparse_mla_attn(dp.batch, dp.q_nope, dp.q_rope, dp.kv, dp.w_uk, dp.w_uv, ic,
                                    out_dtype=torch.float32)
    mla_c = dsa.dsa_sparse_mla_attn(dc.batch, dc.q_nope, dc.q_rope, dc.kv, dc.w_uk, dc.w_uv, ic,
                                    out_dtype=torch.float32)
    assert torch.equal(mla_c, mla_p)
    torch.cuda.synchronize()
    out, idx = op.cpu().numpy(), ip.cpu().numpy()
    for t in ([0, 2, 4] if case == "decode" else [0, 23, 24, 33]):
        _oracle_check(inp, t, idx[t], out[t], 2048)


def test_paged_absent_entries_read_finite_rows():
    """-1 entries fetch the row of position 0 (not pool row 0, which holds NaN
    here) and are masked."""
    inp = synth.custom([500, 300], [(0, 499), (1, 299)], seed=52)

    def page0_spare(pc):
        return all(0 not in pc.block_table[b, : (n + 15) // 16] for b, n in enumerate(inp.wl.seq_lens))

    pc = next(pc for pc in (synth.to_paged(inp, 16, seed=s) for s in range(100)) if page0_spare(pc))
    assert np.all(pc.kv[:16] == synth.BF16_NAN)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    idx = np.full((2, 96), -1, np.int32)
    idx[0, 10:50] = np.arange(100, 140)
    idx[1, 60:70] = np.arange(5, 15)
    ti = torch.from_numpy(idx).cuda()
    oc = dsa.dsa_sparse_mla_attn(dc.batch, dc.q_nope, dc.q_rope, dc.kv, dc.w_uk, dc.w_uv, ti, out_dtype=torch.float32)
    op = dsa.dsa_sparse_mla_attn(dp.batch, dp.q_nope, dp.q_rope, dp.kv, dp.w_uk, dp.w_uv, ti, out_dtype=torch.float32)
    assert torch.isfinite(op).all()
    assert torch.equal(oc, op)


@pytest.mark.parametrize("T,k", [(12, 2048), (12, 8192), (8, 4096), (32, 2048)])
def test_paged_decode_core_ring_equals_contiguous(T, k):
    """The decode core's ring of 4-step rounds (more than 8 queries at k 2048,
    or k 4096 / 8192), and the key-split core above 16 queries, on 16-token pages: index rows with -1 entries (one row
    unsorted) give the same bytes as the contiguous layout, and sampled
    queries match the oracle."""
    _say(f"[paged decode ring] T={T} k={k}")
    rng = np.random.default_rng(700 + T + k)
    lens = [int(x) for x in rng.integers(k + 60, k + 3000, size=T)]
    inp = synth.custom(lens, [(b, lens[b] - 1) for b in range(T)], seed=710 + T + k)
    pc = synth.to_paged(inp, 16, seed=16)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        m = int(rng.integers(k // 2, k + 1))
        row = np.concatenate([np.sort(rng.choice(lens[t], m, replace=False)).astype(np.int32),
                              np.full(k - m, -1, np.int32)])
        idx[t] = rng.permutation(row) if t == 1 else row
    it = torch.from_numpy(idx).cuda()
    mla_c = dsa.dsa_sparse_mla_attn(dc.batch, dc.q_nope, dc.q_rope, dc.kv, dc.w_uk, dc.w_uv, it,
                                    out_dtype=torch.float32)
    mla_p = dsa.dsa_sparse_mla_attn(dp.batch, dp.q_nope, dp.q_rope, dp.kv, dp.w_uk, dp.w_uv, it,
                                    out_dtype=torch.float32)
    assert torch.equal(mla_c, mla_p)
    out = mla_p.cpu().numpy()
    for t in (0, 1, T - 1):
        b = int(inp.q_seq[t])
        r0 = int(inp.seq_row0[b])
        kept = idx[t][idx[t] >= 0].astype(np.int64)
        ref = O.mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[r0 + kept], inp.w_uk, inp.w_uv)
        mx, rel = out_errors(out[t], ref)
        assert mx <= OUT_MAX_ABS and rel <= OUT_REL_L2, (t, mx, rel)


def test_paged_full_size_decode_sampled():
    """decode_b8_ctx204k with 64-token pages: identical to the contiguous layout,
    sampled queries against the oracle."""
    _say("[paged full] decode_b8_ctx204k: generating inputs")
    inp = synth.make_inputs(synth.workload("decode_b8_ctx204k"))
    pc = synth.to_paged(inp, 64, seed=64)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    oc, ic = run_forward(dc)
    op, ip = run_forward(dp)
    assert torch.equal(ic, ip) and torch.equal(oc, op)
    torch.cuda.synchronize()
    out, idx = op.cpu().numpy(), ip.cpu().numpy()
    for t in (0, 5):
        _oracle_check(inp, t, idx[t], out[t], 2048)


@pytest.mark.parametrize("page_size", [16, 128])
def test_paged_one_split_equals_contiguous(page_size):
    """Batches with one key split per query (the warp-specialised core) on paged
    caches: index rows turned into pool rows, ragged k, -1 entries anywhere (the
    row of position 0, never the NaN spare rows), bit-identical to the
    contiguous layout; the forward too."""
    lens, qs = [2600, 1800], [(i % 2, 1500 + i) for i in range(260)]
    _say(f"[paged one split] page_size={page_size}")
    inp = synth.custom(lens, qs, seed=53)
    pc = synth.to_paged(inp, page_size, seed=page_size + 1)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    rng = np.random.default_rng(3)
    k = 100
    T = len(qs)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = int(inp.q_pos[t]) + 1
        m = int(rng.integers(1, k + 1))
        row = np.concatenate([rng.choice(n, m, replace=False).astype(np.int32), np.full(k - m, -1, np.int32)])
        idx[t] = rng.permutation(row)
    ti = torch.from_numpy(idx).cuda()
    oc = dsa.dsa_sparse_mla_attn(dc.batch, dc.q_nope, dc.q_rope, dc.kv, dc.w_uk, dc.w_uv, ti, out_dtype=torch.float32)
    op = dsa.dsa_sparse_mla_attn(dp.batch, dp.q_nope, dp.q_rope, dp.kv, dp.w_uk, dp.w_uv, ti, out_dtype=torch.float32)
    assert torch.isfinite(op).all()
    assert torch.equal(oc, op)
    out = op.cpu().numpy()
    for t in (0, 1, T // 2, T - 1):
        b = int(inp.q_seq[t])
        r0 = int(inp.seq_row0[b])
        kept = idx[t][idx[t] >= 0].astype(np.int64)
        ref = O.mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[r0 + kept], inp.w_uk, inp.w_uv)
        mx, rel = out_errors(out[t], ref)
        assert mx <= OUT_MAX_ABS and rel <= OUT_REL_L2, (t, mx, rel)
    fc, ic = run_forward(dc)
    fp, ip = run_forward(dp)
    assert torch.equal(ic, ip) and torch.equal(fc, fp)


def test_paged_one_split_at_index_topk_8192():
    """The warp-specialised core on 16-token pages at k 8192 (the largest index
    row, its entries and the row past k filling most of each query's entries
    area): ragged rows with -1 entries, bit-identical to the contiguous layout,
    and the oracle on four queries."""
    lens, qs = [12000, 9500], [(i % 2, 9000 + i) for i in range(260)]
    _say("[paged one split] k=8192 page_size=16")
    inp = synth.custom(lens, qs, seed=59)
    pc = synth.to_paged(inp, 16, seed=61)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    rng = np.random.default_rng(7)
    k = 8192
    T = len(qs)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = int(inp.q_pos[t]) + 1
        m = int(rng.integers(k - 300, k + 1)) if t % 3 else int(rng.integers(1, k + 1))
        row = np.concatenate([rng.choice(n, m, replace=False).astype(np.int32), np.full(k - m, -1, np.int32)])
        idx[t] = np.sort(row) if t % 2 else rng.permutation(row)
    ti = torch.from_numpy(idx).cuda()
    oc = dsa.dsa_sparse_mla_attn(dc.batch, dc.q_nope, dc.q_rope, dc.kv, dc.w_uk, dc.w_uv, ti, out_dtype=torch.float32)
    op = dsa.dsa_sparse_mla_attn(dp.batch, dp.q_nope, dp.q_rope, dp.kv, dp.w_uk, dp.w_uv, ti, out_dtype=torch.float32)
    assert torch.isfinite(op).all()
    assert torch.equal(oc, op)
    out = op.cpu().numpy()
    for t in (0, 1, T // 2, T - 1):
        b = int(inp.q_seq[t])
        r0 = int(inp.seq_row0[b])
        kept = idx[t][idx[t] >= 0].astype(np.int64)
        ref = O.mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[r0 + kept], inp.w_uk, inp.w_uv)
        mx, rel = out_errors(out[t], ref)
        assert mx <= OUT_MAX_ABS and rel <= OUT_REL_L2, (t, mx, rel)


@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_candidate_path_equals_contiguous(page_size):
    """A chunk whose query blocks fill the chip takes the candidate path (sampled
    scores read through the block table one page per sampled key, thresholds,
    candidate GEMM, candidate top-k) on paged caches too: bit-identical to the
    contiguous layout."""
    _say(f"[paged candidates] page_size={page_size}")
    inp = synth.custom([6000], [(0, 1904 + i) for i in range(4096)], seed=54)
    pc = synth.to_paged(inp, page_size, seed=page_size + 2)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    oc, ic = run_forward(dc)
    op, ip = run_forward(dp)
    assert torch.equal(ic, ip)
    assert torch.equal(oc, op)
    assert torch.isfinite(op).all()
    torch.cuda.synchronize()
    out, idx = op.cpu().numpy(), ip.cpu().numpy()
    for t in (0, 2047, 4095):
        _oracle_check(inp, t, idx[t], out[t], 2048)


def test_paged_full_size_prefill_sampled():
    """prefill_chunk4096_ctx204k with 64-token pages (the benchmark's paged
    prefill): identical to the contiguous layout, sampled queries against the
    oracle."""
    _say("[paged full] prefill_chunk4096_ctx204k: generating inputs")
    inp = synth.make_inputs(synth.workload("prefill_chunk4096_ctx204k"))
    pc = synth.to_paged(inp, 64, seed=65)
    dc = to_device(inp)
    dp = to_device_paged(inp, pc, dc)
    oc, ic = run_forward(dc)
    op, ip = run_forward(dp)
    assert torch.equal(ic, ip) and torch.equal(oc, op)
    torch.cuda.synchronize()
    out, idx = op.cpu().numpy(), ip.cpu().numpy()
    for t in (0, 4095):
        _oracle_check(inp, t, idx[t], out[t], 2048)
