"""The prefill forward's candidate path (chunks of >= 4,096 queries on contiguous
caches): the indexer GEMM keeps only scores at or above a threshold taken from a
1/128 sample of each row, and the top-k is selected among those candidates.  The
selection must equal the top-k of the full score row; rows where the threshold
misses (too few or too many candidates, or more ties at the threshold than fit)
take the full path.  These cases force each of those, and check the selection
bit-exactly against the top-k rule applied to the scores the GPU computes
(dsa_index_scores, the same GEMM), and against the oracle's scores within the
score error."""
import numpy as np
import pytest
import torch

from long_context_sparse_index_amd import dsa, synth
from oracle import dsa_oracle as O
from tests.gpu_util import (OUT_MAX_ABS, OUT_REL_L2, check_selection_vs_scores, out_errors, run_forward,
                            to_device)

pytestmark = pytest.mark.gpu

L = 30000          # context of the sequence
T = 4096           # queries: one GEMM workgroup per 16-query block over the whole context
STRIDE = 128       # the sample's stride (every 128th position is sampled)


def _inputs(seed, keys=None):
    inp = synth.custom([L], [(0, L - T + i) for i in range(T)], seed=seed)
    if keys is not None:
        inp.k_idx = keys(inp.k_idx.copy())
    return inp


def _scale_sampled(factor):
    def f(k):
        x = synth.bf16_to_f32(k)
        x[::STRIDE] *= np.float32(factor)
        return synth.bf16_rne(x)
    return f


def _check(inp, k=2048, sample=(0, 1, 777, 2048, 3000, 4095), outputs=(0, 4095)):
    print(f"  running k={k}", flush=True)
    d = to_device(inp)
    out, idx = run_forward(d, k=k)
    sc = dsa.dsa_index_scores(d.batch, d.q_idx, d.w, d.k_idx)
    torch.cuda.synchronize()
    out, idx, sc = out.cpu().numpy(), idx.cpu().numpy(), sc.cpu().numpy()
    worst = 0.0
    for t in sample:
        p = int(inp.q_pos[t])
        o_s = O.indexer_scores(inp.q_idx[t], inp.w[t], inp.k_idx[: p + 1], p)
        nd, eps = check_selection_vs_scores(idx[t], sc[t], o_s, O.topk_select(o_s, k), k)
        worst = max(worst, eps)
    # every row: the selection is the top-k of the GPU's own score row
    for t in range(0, T, 97):
        p = int(inp.q_pos[t])
        assert np.array_equal(idx[t], O.topk_select(sc[t, : p + 1], k)), f"row {t}"
    for t in outputs:
        kept = idx[t][idx[t] >= 0].astype(np.int64)
        mx, rel = out_errors(out[t], O.mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[kept], inp.w_uk, inp.w_uv))
        assert mx <= OUT_MAX_ABS and rel <= OUT_REL_L2
    print(f"  max |score err| {worst:.2e}", flush=True)
    return idx, sc


def test_candidates_random_rows():
    print("[candidates] random rows (threshold path)", flush=True)
    _check(_inputs(91))


def test_candidates_k8192():
    print("[candidates] k 8192", flush=True)
    _check(_inputs(92), k=8192)


def test_candidates_sample_too_high_falls_back():
    """Sampled keys scaled up: the sampled scores sit far above the row's, so
    the threshold keeps fewer than k scores and every row takes the full path."""
    print("[candidates] sample above the row", flush=True)
    _check(_inputs(93, _scale_sampled(4.0)))


def test_candidates_sample_too_low_falls_back():
    """Sampled keys scaled down: the threshold keeps nearly the whole row (more
    than the list holds), and every row takes the full path."""
    print("[candidates] sample below the row", flush=True)
    _check(_inputs(94, _scale_sampled(0.05)))


def test_candidates_heavy_ties():
    """Indexer keys k_s = beta_s e_0 with beta_s in {1..5} and queries along e_0
    (positive powers of two): exact scores with five distinct values.  About
    6,000 scores tie at the threshold value, more than the threshold bin's LDS
    capacity: those rows take the full path.  Positions of equal scores are
    kept from the lowest position, exactly as the oracle's stable sort."""
    print("[candidates] heavy ties", flush=True)
    inp = _inputs(95)
    rng = np.random.default_rng(5)
    beta = rng.integers(1, 6, size=L).astype(np.float32)
    k = np.zeros((L, 128), np.float32)
    k[:, 0] = beta
    inp.k_idx = synth.bf16_rne(k)
    q = np.zeros((T, 32, 128), np.float32)
    q[:, :, 0] = np.float32(0.5)
    inp.q_idx = synth.bf16_rne(q)
    inp.w = synth.bf16_rne(np.full((T, 32), 0.25, np.float32))
    idx, sc = _check(inp, sample=(0, 4095), outputs=(7,))
    for t in (0, 1000, 4095):
        p = int(inp.q_pos[t])
        s = O.indexer_scores(inp.q_idx[t], inp.w[t], inp.k_idx[: p + 1], p)
        assert np.array_equal(sc[t, : p + 1], s)             # exact scores
        assert np.array_equal(idx[t], O.topk_select(s, 2048))  # and the oracle's own selection


def test_candidates_dense_threshold_bin():
    """Exact scores 4*beta_s with beta_s = bf16(1 + u/10): every score of a row
    lies in one top-digit bin (more than its LDS capacity of candidates), which
    the candidate path refines by the next 12 key bits (about 2,300 ties per
    value) instead of falling back; ties keep the lowest positions."""
    print("[candidates] dense threshold bin", flush=True)
    inp = _inputs(96)
    rng = np.random.default_rng(6)
    beta = (1.0 + rng.random(L) / 10).astype(np.float32)
    k = np.zeros((L, 128), np.float32)
    k[:, 0] = beta
    inp.k_idx = synth.bf16_rne(k)
    q = np.zeros((T, 32, 128), np.float32)
    q[:, :, 0] = np.float32(0.5)
    inp.q_idx = synth.bf16_rne(q)
    inp.w = synth.bf16_rne(np.full((T, 32), 0.25, np.float32))
    idx, sc = _check(inp, sample=(0, 4095), outputs=(9,))
    for t in (0, 2222, 4095):
        p = int(inp.q_pos[t])
        s = O.indexer_scores(inp.q_idx[t], inp.w[t], inp.k_idx[: p + 1], p)
        assert np.array_equal(sc[t, : p + 1], s)
        assert np.array_equal(idx[t], O.topk_select(s, 2048))
