"""The Python binding checks every caller-supplied tensor before the library is
called: a wrong output dtype or shape, an index array of the wrong shape or
type, a score matrix too small or on the host, or a workspace too small raises
ValueError and nothing is launched (the caller's buffers keep their contents)."""
import numpy as np
import pytest
import torch

from long_context_sparse_index_amd import dsa, synth
from tests.gpu_util import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    print("[binding checks]", flush=True)
    inp = synth.custom([300, 200], [(0, 299), (1, 150), (0, 40)], seed=61)
    return to_device(inp)


def _sentinel(shape, dtype):
    return torch.full(shape, 7, dtype=dtype, device="cuda")


def test_forward_rejects_bad_outputs(dev):
    d, T = dev, 3
    args = (d.batch, d.q_idx, d.w, d.k_idx, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv)
    bad_outs = [
        (_sentinel((T, 64, 256), torch.bfloat16), torch.float32),   # bf16 buffer, fp32 requested
        (_sentinel((T, 64, 256), torch.float32), torch.bfloat16),   # fp32 buffer, bf16 requested
        (_sentinel((T, 64, 128), torch.bfloat16), torch.bfloat16),  # wrong shape
        (_sentinel((T + 1, 64, 256), torch.bfloat16), torch.bfloat16),
        (_sentinel((T, 64, 512), torch.bfloat16)[:, :, :256], torch.bfloat16),  # not contiguous
    ]
    for out, od in bad_outs:
        before = out.clone()
        with pytest.raises(ValueError):
            dsa.dsa_forward(*args, k=64, out_dtype=od, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, before)
    with pytest.raises(ValueError):
        dsa.dsa_forward(*args, k=64, out_dtype=torch.float16)
    for idx in (_sentinel((T, 32), torch.int32), _sentinel((T, 64), torch.int64),
                _sentinel((T, 64), torch.int32).cpu()):
        with pytest.raises(ValueError):
            dsa.dsa_forward(*args, k=64, idx=idx)
    for k in (0, 8193):
        with pytest.raises(ValueError):
            dsa.dsa_forward(*args, k=k)
    tiny = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        dsa.dsa_forward(*args, k=64, ws=tiny)
    with pytest.raises(ValueError):
        dsa.dsa_forward(*args, k=64, ws=torch.empty(1 << 20, dtype=torch.uint8))  # host memory


def test_index_scores_and_topk_reject_bad_buffers(dev):
    d, T = dev, 3
    for sc in (torch.empty((T - 1, 304), device="cuda"), torch.empty((T, 200), device="cuda"),
               torch.empty((T, 304)), torch.empty((T, 304), dtype=torch.float64, device="cuda")):
        with pytest.raises(ValueError):
            dsa.dsa_index_scores(d.batch, d.q_idx, d.w, d.k_idx, scores=sc)
        with pytest.raises(ValueError):
            dsa.dsa_topk(d.batch, sc, 16)
    sc = dsa.dsa_index_scores(d.batch, d.q_idx, d.w, d.k_idx)
    for idx in (_sentinel((T, 15), torch.int32), _sentinel((T, 16), torch.int64)):
        before = idx.clone()
        with pytest.raises(ValueError):
            dsa.dsa_topk(d.batch, sc, 16, idx=idx)
        assert torch.equal(idx, before)
    with pytest.raises(ValueError):
        dsa.dsa_topk(d.batch, sc, 16, ws=torch.empty(8, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        dsa.dsa_index_scores(d.batch, d.q_idx, d.w, d.k_idx[:, :64].contiguous())


def test_sparse_mla_rejects_bad_buffers(dev):
    d, T = dev, 3
    idx = torch.from_numpy(np.tile(np.arange(32, dtype=np.int32), (T, 1))).cuda()
    args = (d.batch, d.q_nope, d.q_rope, d.kv, d.w_uk, d.w_uv)
    out = _sentinel((T, 64, 256), torch.bfloat16)
    with pytest.raises(ValueError):
        dsa.dsa_sparse_mla_attn(*args, idx, out_dtype=torch.float32, out=out)
    with pytest.raises(ValueError):
        dsa.dsa_sparse_mla_attn(*args, idx[:2].contiguous())
    with pytest.raises(ValueError):
        dsa.dsa_sparse_mla_attn(*args, idx.to(torch.int64))
    with pytest.raises(ValueError):
        dsa.dsa_sparse_mla_attn(*args, idx, ws=torch.empty(64, dtype=torch.uint8, device="cuda"))
    with pytest.raises(ValueError):
        dsa.dsa_sparse_mla_attn(d.batch, d.q_nope, d.q_rope, d.kv[:, :512].contiguous(), d.w_uk, d.w_uv, idx)
    # a correct call still works and writes the caller's buffer
    got = dsa.dsa_sparse_mla_attn(*args, idx, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr() and not torch.equal(out, _sentinel((T, 64, 256), torch.bfloat16))
