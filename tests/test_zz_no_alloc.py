"""dsa_forward_noalloc (workspace in the library's static per-device scratch)
against dsa_forward (caller workspace), through the C ABI: two calls in a row,
the second on a smaller batch, then a batch whose workspace exceeds the scratch
(run in query chunks)."""
import numpy as np
import pytest
import torch

from long_context_sparse_index_amd import dsa, synth
from tests.gpu_util import OUT_MAX_ABS, OUT_REL_L2, out_errors, run_forward, to_device

pytestmark = pytest.mark.gpu


def _noalloc(d, k, out_dtype):
    out = torch.full((d.batch.T, 64, 256), 3.0, dtype=out_dtype, device="cuda")
    idx = torch.full((d.batch.T, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_forward_noalloc(d.batch, d.q_idx, d.w, d.k_idx, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv,
                            out=out, idx=idx, k=k)
    return out, idx


def test_noalloc_matches_forward_on_consecutive_calls():
    cases = [
        # (sequence lengths, queries, k): the second is smaller than the first
        ([20000, 9000, 30000, 5000], [(0, 19999), (1, 8999), (2, 29999), (3, 4999)], 2048),
        ([3000, 700], [(0, 2999), (1, 699)], 512),
    ]
    for i, (lens, qs, k) in enumerate(cases):
        print(f"[noalloc] call {i}: T={len(qs)} k={k}", flush=True)
        d = to_device(synth.custom(lens, qs, seed=71 + i))
        need = dsa.dsa_workspace_bytes(dsa.OP_FORWARD, len(qs), d.batch.max_ctx, k)
        assert need <= 64 << 20  # one chunk in both calls: identical kernels and plans
        ref_out, ref_idx = run_forward(d, k=k, out_dtype=torch.float32)
        out, idx = _noalloc(d, k, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx)
        assert torch.equal(out, ref_out)
        outb, idxb = _noalloc(d, k, torch.bfloat16)
        ref_b, _ = run_forward(d, k=k, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(idxb, ref_idx) and torch.equal(outb, ref_b)


def test_noalloc_chunks_batches_beyond_the_scratch():
    qs = [(0, 131072 - 64 + i) for i in range(64)]
    print("[noalloc] 64 queries at 131,072 positions (workspace above the scratch)", flush=True)
    d = to_device(synth.custom([131072], qs, seed=73))
    assert dsa.dsa_workspace_bytes(dsa.OP_FORWARD, 64, d.batch.max_ctx, 2048) > 64 << 20
    ref_out, ref_idx = run_forward(d, k=2048, out_dtype=torch.float32)
    out, idx = _noalloc(d, 2048, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    mx, rel = out_errors(out.cpu().numpy(), ref_out.cpu().numpy().astype(np.float64))
    print(f"  chunked vs one chunk: max-abs {mx:.2e} rel-L2 {rel:.2e}", flush=True)
    assert mx <= OUT_MAX_ABS and rel <= OUT_REL_L2
