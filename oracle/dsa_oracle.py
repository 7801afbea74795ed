"""CPU oracle for the DSA hot path: indexer -> top-k -> sparse MLA.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the HIP path never does, and this module
imports nothing from it.  It is plain numpy in float64, deliberately slow and
unblocked, so that it can be checked against the pages by eye.

Sources (the pages have no code; every step below is restated from prose):
  [CFG] page "2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解"
        §2.1 (parameter table: index_n_heads 32, index_head_dim 128,
        index_topk 2048, 64 heads, qk_nope 192, qk_rope 64, v_head 256,
        kv_lora_rank 512) and §2.2 (the indexer scores every query against all
        history and only ranks; the selector keeps the index_topk best keys,
        which alone take part in attention; DSA filters on top of MLA).
  [N2]  page "（五）一万亿次点积砍到两千次：DSA 怎么破 N²", sections on the indexer
        (low-dimensional 32x128 dot products over every token), the full DSA
        flow (indexer top-2048, then full Q.K.V, softmax, weighted V over those
        only) and the cache division of labour (skipped K/V stay cached); its
        IndexShare section (one indexer per 4 layers, the group figure, the
        21 full / 57 shared count) and the config fields listed at its end
        (index_topk_freq 4, num_hidden_layers 78, 3 dense + 75 sparse).
  [G5]  page "GLM-5 7440亿参数，202K长上下文突破极限", section 六 (deployment advice:
        paged KV caches for batched serving).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * score(t,s) = sum_h w[t,h] * ReLU(q_idx[t,h] . k_idx[s]); one 128-d key per
    cached token shared by the 32 indexer heads; no scale, no bias.
  * causal: s <= t (a token sees itself); sequence-local positions.
  * scores are rounded once to fp32; selection compares fp32 values (so -0.0
    equals +0.0), ties go to the lower position; the kept positions are
    returned ascending and padded with -1 to length k; with n <= k all n are kept.
  * IndexShare: a shared layer runs no indexer and reuses the selection of
    the nearest earlier full layer (a forward pass cannot use a later one);
    the group figure, which pairs layers 3-5 with layer 6, is read with each
    full layer feeding the three layers after it.
  * paged caches: token s of a sequence sits in page s // P of that
    sequence's page list, at offset s % P (page-table indirection is storage
    only; every computation above reads the same rows).
  * INT4 latent cache ([G5] section six recommends INT4 KV-cache quantisation
    and a saving above 60%, no format): per cache row, the 512 latent values
    in 8 groups of 64, each with scale s = bf16(absmax / 7) and codes
    q = clamp(rint(x / s), -7, 7) (each division correctly rounded in fp32,
    rint ties to even: the format fixes its arithmetic in fp32, so a code is a
    well-defined integer); the 64 rope values stay bf16.  400 bytes per
    row: 256 bytes of codes (element 2i in the low nibble of byte i, two's
    complement), 8 bf16 scales, 64 bf16 rope.  Dequantised latent = q * s.
  * MLA over the kept rows with explicit per-head up-projection
    K_nope = c @ W_UK[h], V = c @ W_UV[h]; logits (q_nope.K_nope + q_rope.r)
    times softmax_scale (1/sqrt(192+64) = 1/16 by default); softmax in full.

Parity pins: the functions here are pinned by tests/test_oracle_pins.py
(dense-attention equivalence, planted index sets, absorbed == explicit, brute
force, softmax special cases).  Nothing here is "parity unpinned".
"""
from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

# [CFG] §2.1 parameter table.
INDEX_N_HEADS = 32
INDEX_HEAD_DIM = 128
INDEX_TOPK = 2048
NUM_HEADS = 64
QK_NOPE_HEAD_DIM = 192
QK_ROPE_HEAD_DIM = 64
QK_HEAD_DIM = QK_NOPE_HEAD_DIM + QK_ROPE_HEAD_DIM
V_HEAD_DIM = 256
KV_LORA_RANK = 512
DEFAULT_SCALE = 1.0 / np.sqrt(QK_HEAD_DIM)  # = 1/16


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact conversion of bf16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- O1 indexer
def indexer_scores(q_idx_t, w_t, k_idx_seq, pos: int) -> np.ndarray:
    """Lightning-indexer scores of one query against its history, fp32.

    [CFG] §2.2 and [N2] (indexer section): one cheap relevance score per
    (query, earlier token) from 32 heads of 128-d dot products; the score only
    ranks keys.  Reading: score = sum over heads of w_h * ReLU(q_h . k_s) for
    s = 0..pos, evaluated in float64 and rounded once to fp32.

    q_idx_t [32,128] bf16, w_t [32] bf16, k_idx_seq [>=pos+1,128] bf16.
    Returns float32 [pos+1].
    """
    q = bf16_bits_to_f64(q_idx_t)                    # [32,128]
    w = bf16_bits_to_f64(w_t)                        # [32]
    k = bf16_bits_to_f64(k_idx_seq[: pos + 1])       # [n,128]
    per_head = k @ q.T                               # [n,32]  q_h . k_s
    relu = np.maximum(per_head, 0.0)                 # ReLU per head, before weighting
    score = relu @ w                                 # sum_h w_h * ReLU(.)
    return score.astype(np.float32)                  # one RNE rounding to fp32


# ---------------------------------------------------------------- O2 top-k
def topk_select(scores_f32, k: int = INDEX_TOPK) -> np.ndarray:
    """Top-k selector by a full stable sort.

    [CFG] §2.2 / [N2] (the 2048 best-scoring history positions are kept).
    Order: fp32 score descending, then position ascending.  Returns int32 [k]:
    the kept positions ascending, then -1 padding.  If n <= k all n are kept.
    """
    s = np.asarray(scores_f32, dtype=np.float32)
    n = int(s.shape[0])
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n, dtype=np.int32)
        return out
    key = s.astype(np.float64) + 0.0                 # -0.0 -> +0.0
    order = np.argsort(-key, kind="stable")          # equal scores keep position order
    kept = np.sort(order[:k])
    out[:] = kept.astype(np.int32)
    return out


# ---------------------------------------------------------------- O3 MLA
def mla_explicit(q_nope_t, q_rope_t, kv_rows, w_uk, w_uv,
                 scale: float = DEFAULT_SCALE) -> np.ndarray:
    """Full MLA attention of one query over the given latent-cache rows.

    [N2] (DSA flow: full Q.K.V over the kept tokens, softmax, weighted sum of
    V) with the MLA shapes of [CFG] §2.1.  Explicit form: every head
    up-projects the kept latent rows to its own keys and values.

    q_nope_t [64,192], q_rope_t [64,64], kv_rows [n,576] (512 latent | 64 rope,
    rope key shared by all heads), w_uk [64,512,192], w_uv [64,512,256]; all
    bf16 bit patterns.  Returns float64 [64,256].
    """
    qn = bf16_bits_to_f64(q_nope_t)
    qr = bf16_bits_to_f64(q_rope_t)
    rows = bf16_bits_to_f64(kv_rows)
    c = rows[:, :KV_LORA_RANK]
    r = rows[:, KV_LORA_RANK:]
    wuk = bf16_bits_to_f64(w_uk)
    wuv = bf16_bits_to_f64(w_uv)
    out = np.empty((NUM_HEADS, V_HEAD_DIM))
    for h in range(NUM_HEADS):
        k_nope = c @ wuk[h]                          # [n,192]
        v = c @ wuv[h]                               # [n,256]
        z = (k_nope @ qn[h] + r @ qr[h]) * scale     # [n]
        e = np.exp(z - z.max())
        p = e / e.sum()
        out[h] = p @ v
    return out


def mla_explicit_f64(q_nope_t, q_rope_t, rows, w_uk, w_uv, scale: float = DEFAULT_SCALE) -> np.ndarray:
    """``mla_explicit`` over cache rows already given as float64 [n,576] (e.g.
    dequantised INT4 rows); queries and weights are bf16 bit patterns.

    Pinned on its own: equal to ``mla_explicit`` on rows that are bf16 values,
    equal to torch's SDPA in fp64 (K/V up-projected explicitly) on dequantised
    INT4 rows, and the zero-query / single-row softmax special cases."""
    qn = bf16_bits_to_f64(q_nope_t)
    qr = bf16_bits_to_f64(q_rope_t)
    c = rows[:, :KV_LORA_RANK]
    r = rows[:, KV_LORA_RANK:]
    wuk = bf16_bits_to_f64(w_uk)
    wuv = bf16_bits_to_f64(w_uv)
    out = np.empty((NUM_HEADS, V_HEAD_DIM))
    for h in range(NUM_HEADS):
        z = (c @ wuk[h] @ qn[h] + r @ qr[h]) * scale
        e = np.exp(z - z.max())
        out[h] = (e / e.sum()) @ (c @ wuv[h])
    return out


def mla_absorbed(q_nope_t, q_rope_t, kv_rows, w_uk, w_uv,
                 scale: float = DEFAULT_SCALE) -> np.ndarray:
    """Same attention in weight-absorbed form (used only to cross-check O3).

    q_lat = W_UK[h] q_nope scores directly against the 512-d latent; the
    latent-weighted sum is up-projected by W_UV[h] afterwards.
    """
    qn = bf16_bits_to_f64(q_nope_t)
    qr = bf16_bits_to_f64(q_rope_t)
    rows = bf16_bits_to_f64(kv_rows)
    c = rows[:, :KV_LORA_RANK]
    r = rows[:, KV_LORA_RANK:]
    wuk = bf16_bits_to_f64(w_uk)
    wuv = bf16_bits_to_f64(w_uv)
    out = np.empty((NUM_HEADS, V_HEAD_DIM))
    for h in range(NUM_HEADS):
        q_lat = wuk[h] @ qn[h]                       # [512]
        z = (c @ q_lat + r @ qr[h]) * scale
        e = np.exp(z - z.max())
        p = e / e.sum()
        out[h] = (p @ c) @ wuv[h]
    return out


def softmax_weights(q_nope_t, q_rope_t, kv_rows, w_uk, h: int,
                    scale: float = DEFAULT_SCALE) -> np.ndarray:
    """The attention weights of head h (explicit form); rows of P sum to 1."""
    qn = bf16_bits_to_f64(q_nope_t)[h]
    qr = bf16_bits_to_f64(q_rope_t)[h]
    rows = bf16_bits_to_f64(kv_rows)
    z = (rows[:, :KV_LORA_RANK] @ bf16_bits_to_f64(w_uk)[h] @ qn
         + rows[:, KV_LORA_RANK:] @ qr) * scale
    e = np.exp(z - z.max())
    return e / e.sum()


# ---------------------------------------------------------------- whole path
def query_forward(inp, t: int, k: int = INDEX_TOPK, scale: float = DEFAULT_SCALE,
                  with_output: bool = True) -> Tuple[np.ndarray, np.ndarray, Optional[np.ndarray]]:
    """Indexer -> top-k -> sparse MLA for query t of an input batch.

    ``inp`` carries q_seq, q_pos, seq_row0, k_idx, kv, q_idx, w, q_nope, q_rope,
    w_uk, w_uv (numpy; bf16 as uint16).  Rows of sequence b start at
    seq_row0[b]; positions are sequence-local.  Returns (scores fp32 [p+1],
    idx int32 [k], out float64 [64,256] or None).
    """
    b = int(inp.q_seq[t])
    p = int(inp.q_pos[t])
    r0 = int(inp.seq_row0[b])
    scores = indexer_scores(inp.q_idx[t], inp.w[t], inp.k_idx[r0: r0 + p + 1], p)
    idx = topk_select(scores, k)
    out = None
    if with_output:
        kept = idx[idx >= 0].astype(np.int64)
        out = mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[r0 + kept],
                           inp.w_uk, inp.w_uv, scale)
    return scores, idx, out


def forward(inp, queries: Optional[Iterable[int]] = None, k: int = INDEX_TOPK,
            scale: float = DEFAULT_SCALE, with_output: bool = True):
    """query_forward over a set of queries (all by default); lists in query order."""
    qs = range(len(inp.q_seq)) if queries is None else list(queries)
    res = [query_forward(inp, t, k, scale, with_output) for t in qs]
    return [r[0] for r in res], [r[1] for r in res], [r[2] for r in res]


# ---------------------------------------------------------------- IndexShare
def index_share_schedule(num_layers: int = 78, num_dense: int = 3, freq: int = 4):
    """For every layer, the layer whose indexer selection it attends with.

    [N2] IndexShare section: every group of 4 adjacent layers runs the indexer
    once ("full") and the other 3 reuse it ("shared"); the first dense layers
    keep their own indexer and join no group; config: 78 layers, 3 dense,
    index_topk_freq 4, 21 full and 57 shared.  Walking the layers in forward
    order: a dense layer is full; a sparse layer is full when it completes a
    run of ``freq`` sparse layers, otherwise it reuses the last full layer seen.
    Returns a list: entry l is l for a full layer, else its source (< l).
    """
    source = []
    last_full = None
    sparse_seen = 0
    for layer in range(num_layers):
        if layer < num_dense:
            full = True
        else:
            sparse_seen += 1
            full = sparse_seen % freq == 0
        if full:
            last_full = layer
            source.append(layer)
        else:
            if last_full is None:
                raise ValueError("a shared layer has no earlier full layer")
            source.append(last_full)
    return source


def layer_stack_forward(layers, schedule, queries: Optional[Iterable[int]] = None,
                        k: int = INDEX_TOPK, scale: float = DEFAULT_SCALE):
    """DSA with IndexShare over a stack of layers.

    ``layers[l]`` holds layer l's inputs (as for ``query_forward``: the same
    batch geometry in every layer; a shared layer's indexer arrays are unused).
    A full layer selects with its own indexer; a shared layer attends over its
    own latent cache at the positions its source layer selected ([N2]
    IndexShare: the shared members take the representative's indices and do
    not compute their own).  Returns (idx, out): per layer, lists over the
    queries of int32 [k] and float64 [64,256].
    """
    qs = range(len(layers[0].q_seq)) if queries is None else list(queries)
    idx_of = {}
    out_all = []
    idx_all = []
    for layer, inp in enumerate(layers):
        src = schedule[layer]
        if src == layer:
            idx_of[layer] = [query_forward(inp, t, k, scale, with_output=False)[1] for t in qs]
        sel = idx_of[src]
        outs = []
        for j, t in enumerate(qs):
            b = int(inp.q_seq[t])
            r0 = int(inp.seq_row0[b])
            kept = sel[j][sel[j] >= 0].astype(np.int64)
            outs.append(mla_explicit(inp.q_nope[t], inp.q_rope[t], inp.kv[r0 + kept],
                                     inp.w_uk, inp.w_uv, scale))
        idx_all.append(sel)
        out_all.append(outs)
    return idx_all, out_all


# ---------------------------------------------------------------- paged caches
def paged_row(page_list, page_size: int, s: int) -> int:
    """Pool row of token s of a sequence whose cache lives in pages.

    [G5] section six recommends paged caches for batched serving; the pages do
    not fix a layout.  Reading: the sequence's tokens fill fixed-size pages in
    order, page j holding tokens j*P .. j*P+P-1, and ``page_list[j]`` names
    the pool page (rows page*P .. page*P+P-1) that holds them.
    """
    page, offset = divmod(int(s), int(page_size))
    return int(page_list[page]) * int(page_size) + offset


# ---------------------------------------------------------------- INT4 latent cache
INT4_GROUP = 64
INT4_ROW_BYTES = KV_LORA_RANK // 2 + 2 * (KV_LORA_RANK // INT4_GROUP) + 2 * QK_ROPE_HEAD_DIM  # 400


def _f32_to_bf16_bits(x):
    """fp32 -> bf16 bits, round to nearest even (finite values)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def quantize_kv_int4(kv_rows) -> np.ndarray:
    """bf16 cache rows [n,576] -> INT4 rows [n,400] uint8 (format above).

    Per group of 64 latent values: absmax in fp32 (exact for bf16 inputs), the
    scale is that divided by 7 in fp32 and rounded to bf16; each code is the
    value divided by the (bf16) scale in fp32, rounded half to even and clamped
    to [-7, 7]; a zero scale gives zero codes.
    """
    rows = np.asarray(kv_rows, dtype=np.uint16)
    n = rows.shape[0]
    x = bf16_bits_to_f64(rows[:, :KV_LORA_RANK]).astype(np.float32).reshape(n, -1, INT4_GROUP)
    absmax = np.abs(x).max(axis=2)                                   # [n, 8] fp32
    scale_bits = _f32_to_bf16_bits(absmax / np.float32(7.0))         # fp32 division, then bf16
    scale = bf16_bits_to_f64(scale_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(scale[:, :, None] > 0, np.rint(x / scale[:, :, None]), np.float32(0))
    q = np.clip(q, -7, 7).astype(np.int8).reshape(n, KV_LORA_RANK)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    out = np.empty((n, INT4_ROW_BYTES), dtype=np.uint8)
    out[:, : KV_LORA_RANK // 2] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    out[:, KV_LORA_RANK // 2: KV_LORA_RANK // 2 + 16] = scale_bits.astype("<u2").view(np.uint8).reshape(n, 16)
    out[:, KV_LORA_RANK // 2 + 16:] = rows[:, KV_LORA_RANK:].astype("<u2").view(np.uint8).reshape(n, 128)
    return out


def dequantize_kv_int4(q_rows) -> np.ndarray:
    """INT4 rows [n,400] -> float64 [n,576]: latent q * scale (exact), rope as stored."""
    b = np.asarray(q_rows, dtype=np.uint8)
    n = b.shape[0]
    codes = b[:, : KV_LORA_RANK // 2]
    lo = (codes & 0xF).astype(np.int16)
    hi = (codes >> 4).astype(np.int16)
    q = np.empty((n, KV_LORA_RANK), dtype=np.int16)
    q[:, 0::2] = np.where(lo > 7, lo - 16, lo)
    q[:, 1::2] = np.where(hi > 7, hi - 16, hi)
    scales = bf16_bits_to_f64(b[:, 256:272].copy().view("<u2").reshape(n, 8))
    rope = bf16_bits_to_f64(b[:, 272:400].copy().view("<u2").reshape(n, 64))
    lat = q.reshape(n, 8, INT4_GROUP).astype(np.float64) * scales[:, :, None]
    return np.concatenate([lat.reshape(n, KV_LORA_RANK), rope], axis=1)
