"""Helpers for GPU tests: move synthetic inputs to the device, compare results."""
import types

import numpy as np
import torch

from long_context_sparse_index_amd import dsa, synth


def bf16_dev(x: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device)


def to_device(inp: synth.Inputs, device="cuda", max_ctx=None):
    d = types.SimpleNamespace()
    d.q_seq = torch.from_numpy(inp.q_seq).to(device)
    d.q_pos = torch.from_numpy(inp.q_pos).to(device)
    d.seq_row0 = torch.from_numpy(inp.seq_row0).to(device)
    d.batch = dsa.Batch(d.q_seq, d.q_pos, d.seq_row0,
                        max_ctx if max_ctx is not None else int(inp.q_pos.max()) + 1)
    for f in ("k_idx", "kv", "q_idx", "w", "q_nope", "q_rope", "w_uk", "w_uv"):
        setattr(d, f, bf16_dev(getattr(inp, f), device))
    return d


def run_forward(d, k=2048, out_dtype=torch.float32, ws=None):
    return dsa.dsa_forward(d.batch, d.q_idx, d.w, d.k_idx, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv,
                           k=k, out_dtype=out_dtype, ws=ws)


def out_errors(got: np.ndarray, ref: np.ndarray):
    diff = got.astype(np.float64) - ref
    return float(np.abs(diff).max()), float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30))


# Output tolerance: max-abs 2e-2 (bf16 in, fp32 accumulate) and relative L2 1e-2.
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 1e-2
# Scores: max-abs 2e-2 is the contract; the fp32 path is expected far inside 1e-4.
SCORE_MAX_ABS = 1e-4


def check_selection(got_idx: np.ndarray, oracle_scores: np.ndarray, oracle_idx: np.ndarray, k: int,
                    tol: float = 1e-4, atol: float = None):
    """The GPU selection may differ from the oracle's only at near-ties of the k-th score:
    within tol * max(1, |theta|) of it, or within atol when that is given.

    Returns the number of differing positions; asserts validity of the rest."""
    n = oracle_scores.shape[0]
    g = got_idx[got_idx >= 0]
    o = oracle_idx[oracle_idx >= 0]
    assert len(g) == min(n, k)
    assert np.all(np.diff(g) > 0), "GPU indices must be strictly ascending"
    assert g.min() >= 0 and g.max() < n
    assert np.all(got_idx[len(g):] == -1)
    if n <= k:
        assert np.array_equal(g, np.arange(n))
        return 0
    theta = np.sort(oracle_scores.astype(np.float64))[::-1][k - 1]
    sym = np.setxor1d(g, o)
    if len(sym):
        lim = atol if atol is not None else tol * max(1.0, abs(theta))
        assert np.all(np.abs(oracle_scores[sym].astype(np.float64) - theta) <= lim), \
            f"selection differs away from the threshold: {sym[:10]}"
    return len(sym)


def check_selection_vs_scores(got_idx: np.ndarray, gpu_scores: np.ndarray, oracle_scores: np.ndarray,
                              oracle_idx: np.ndarray, k: int):
    """End-to-end selection of one query, checked exactly.

    * the GPU's scores of the query's row agree with the oracle's within SCORE_MAX_ABS;
    * the GPU's selection is bit-exactly the oracle's top-k rule applied to the GPU's
      own scores (so the selector adds no error of its own);
    * where it differs from the oracle's selection, the oracle score of every
      differing position lies within 2*eps of the oracle's k-th score, eps being the
      row's largest score error: scores moved by at most eps can only swap such
      positions (the k-th largest value moves by at most eps too).

    Returns (number of differing positions, eps)."""
    n = oracle_scores.shape[0]
    g = np.asarray(gpu_scores[:n], dtype=np.float32)
    eps = float(np.abs(g.astype(np.float64) - oracle_scores.astype(np.float64)).max())
    assert eps <= SCORE_MAX_ABS, f"score error {eps:.3e}"
    assert np.array_equal(got_idx, oracle_topk_of(g, k)), "selection is not the top-k of the GPU's own scores"
    nd = check_selection(got_idx, oracle_scores, oracle_idx, k, atol=2.0 * eps + 1e-12)
    return nd, eps


def oracle_topk_of(scores_f32: np.ndarray, k: int) -> np.ndarray:
    from oracle import dsa_oracle as O
    return O.topk_select(scores_f32, k)
