"""Seeded synthetic inputs for the DSA hot path (indexer -> top-k -> sparse MLA).

This module only *draws* inputs: random numbers, their rounding to bf16, and the
batch geometry. It contains none of the method's arithmetic, so both the CPU
oracle (``oracle/``) and the HIP path may be fed from it.

Shapes follow the dimension table of the page titled
"2026大模型架构概览（二）：GLM 5 DSV3.2 的 DSA 与 MoE 配置拆解" (§2.1): indexer 32 heads x 128
dims, 64 attention heads, qk 192 (nope) + 64 (rope), v 256, latent 512.

Distributions (the pages give none; these are the stated synthetic recipe):
  * indexer keys / queries: N(0,1)/sqrt(128), rounded to bf16 (round-to-nearest-even)
  * indexer head weights w: U(0,1)
  * latent cache (512) and rope key (64): N(0,1)
  * MLA queries q_nope, q_rope: N(0,1)
  * absorption weights W_UK [64,512,192], W_UV [64,512,256]: N(0,1)/sqrt(512)
  * planted variant: a set of 128-aligned key blocks gets +3.0 added to every
    N(0,1) draw of its indexer keys before the 1/sqrt(128) scale.

Draw order from one ``numpy.random.default_rng(seed)``:
  per sequence: [planted block ids], k_idx (L,128), latent (L,512), rope (L,64);
  per call:     q_idx (T,32,128), w (T,32), q_nope (T,64,192), q_rope (T,64,64),
                W_UK (64,512,192), W_UV (64,512,256).

Everything bf16 is returned as raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

IDX_HEADS = 32
IDX_DIM = 128
HEADS = 64
D_NOPE = 192
D_ROPE = 64
D_V = 256
D_LAT = 512
D_KV = D_LAT + D_ROPE  # one latent-cache row: 512 latent | 64 rope
PLANT_BLOCK = 128
PLANT_SHIFT = 3.0


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round-to-nearest-even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + r) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Workload:
    """Batch geometry of one call: sequences with their cache lengths and queries."""

    name: str
    seq_lens: List[int]
    queries: List[Tuple[int, int]]  # (sequence, position) per query, in call order
    seed: int
    planted_blocks: int = 0  # number of planted 128-key blocks per sequence (0 = none)

    @property
    def num_queries(self) -> int:
        return len(self.queries)

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def max_ctx(self) -> int:
        return max(p for _, p in self.queries) + 1 if self.queries else 1


def _decode(name: str, b: int, l: int, seed: int) -> Workload:
    return Workload(name, [l] * b, [(i, l - 1) for i in range(b)], seed)


def _chunk(name: str, l: int, t: int, seed: int, planted: int = 0) -> Workload:
    return Workload(name, [l], [(0, l - t + i) for i in range(t)], seed, planted)


# The workloads, by what they are.  Sizes follow the page-4 dimension table and
# the long-context windows the pages discuss (202K-204.8K positions).
WORKLOADS = {
    "tiny_ref_4k": lambda: Workload("tiny_ref_4k", [4096], [(0, 4080 + i) for i in range(16)], 0),
    "decode_b32_ctx32k": lambda: _decode("decode_b32_ctx32k", 32, 32768, 1),
    "prefill_chunk4096_ctx131k": lambda: _chunk("prefill_chunk4096_ctx131k", 131072, 4096, 2),
    "prefill_chunk4096_ctx204k": lambda: _chunk("prefill_chunk4096_ctx204k", 204800, 4096, 2),
    "decode_b8_ctx204k": lambda: _decode("decode_b8_ctx204k", 8, 204800, 3),
    "causal_prefill_65k_planted": lambda: Workload(
        "causal_prefill_65k_planted", [65536], [(0, i) for i in range(65536)], 4,
        planted_blocks=round(0.1 * 65536 / PLANT_BLOCK)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]()


@dataclasses.dataclass
class Inputs:
    """All arrays of one call (numpy, host).  bf16 arrays are uint16 bit patterns."""

    wl: Workload
    q_seq: np.ndarray      # [T] int32
    q_pos: np.ndarray      # [T] int32
    seq_row0: np.ndarray   # [B] int64, first row of each sequence in the flat caches
    k_idx: np.ndarray      # [rows,128] bf16
    kv: np.ndarray         # [rows,576] bf16 (512 latent | 64 rope)
    q_idx: np.ndarray      # [T,32,128] bf16
    w: np.ndarray          # [T,32] bf16
    q_nope: np.ndarray     # [T,64,192] bf16
    q_rope: np.ndarray     # [T,64,64] bf16
    w_uk: np.ndarray       # [64,512,192] bf16
    w_uv: np.ndarray       # [64,512,256] bf16
    planted: Dict[int, np.ndarray] = dataclasses.field(default_factory=dict)  # seq -> block ids

    @property
    def rows(self) -> int:
        return int(self.k_idx.shape[0])


def _normal_bf16(rng: np.random.Generator, shape, scale: float = 1.0,
                 shift_rows: Optional[np.ndarray] = None) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if shift_rows is not None:
        x[shift_rows] += np.float32(PLANT_SHIFT)
    if scale != 1.0:
        x *= np.float32(scale)
    return bf16_rne(x)


def make_inputs(wl: Workload, with_queries: bool = True) -> Inputs:
    """Draw every input of ``wl`` from ``default_rng(wl.seed)`` in the documented order."""
    rng = np.random.default_rng(wl.seed)
    rows = int(sum(wl.seq_lens))
    seq_row0 = np.zeros(len(wl.seq_lens), dtype=np.int64)
    if len(wl.seq_lens) > 1:
        seq_row0[1:] = np.cumsum(np.asarray(wl.seq_lens[:-1], dtype=np.int64))
    k_idx = np.empty((rows, IDX_DIM), dtype=np.uint16)
    kv = np.empty((rows, D_KV), dtype=np.uint16)
    planted = {}
    inv_sqrt_idx = float(1.0 / np.sqrt(np.float32(IDX_DIM)))
    for b, length in enumerate(wl.seq_lens):
        r0 = int(seq_row0[b])
        shift = None
        if wl.planted_blocks:
            nblk = length // PLANT_BLOCK
            blocks = np.sort(rng.choice(nblk, wl.planted_blocks, replace=False))
            planted[b] = blocks
            shift = (blocks[:, None] * PLANT_BLOCK + np.arange(PLANT_BLOCK)[None, :]).ravel()
        k_idx[r0:r0 + length] = _normal_bf16(rng, (length, IDX_DIM), inv_sqrt_idx, shift)
        kv[r0:r0 + length, :D_LAT] = _normal_bf16(rng, (length, D_LAT))
        kv[r0:r0 + length, D_LAT:] = _normal_bf16(rng, (length, D_ROPE))
    t = wl.num_queries
    q_seq = np.asarray([s for s, _ in wl.queries], dtype=np.int32).reshape(t)
    q_pos = np.asarray([p for _, p in wl.queries], dtype=np.int32).reshape(t)
    for s, p in wl.queries:
        if not (0 <= s < len(wl.seq_lens) and 0 <= p < wl.seq_lens[s]):
            raise ValueError(f"query ({s},{p}) outside its sequence")
    q_idx = _normal_bf16(rng, (t, IDX_HEADS, IDX_DIM), inv_sqrt_idx)
    w = bf16_rne(rng.random((t, IDX_HEADS), dtype=np.float32))
    q_nope = _normal_bf16(rng, (t, HEADS, D_NOPE))
    q_rope = _normal_bf16(rng, (t, HEADS, D_ROPE))
    inv_sqrt_lat = float(1.0 / np.sqrt(np.float32(D_LAT)))
    w_uk = _normal_bf16(rng, (HEADS, D_LAT, D_NOPE), inv_sqrt_lat)
    w_uv = _normal_bf16(rng, (HEADS, D_LAT, D_V), inv_sqrt_lat)
    return Inputs(wl, q_seq, q_pos, seq_row0, k_idx, kv, q_idx, w, q_nope, q_rope,
                  w_uk, w_uv, planted)


def make_layer_stack(wl: Workload, num_layers: int) -> List[Inputs]:
    """Inputs of ``num_layers`` layers over one batch geometry: layer l draws
    everything of ``make_inputs`` from ``default_rng(wl.seed + 7919 * l)``
    (own caches, queries and weights per layer)."""
    return [make_inputs(dataclasses.replace(wl, seed=wl.seed + 7919 * l)) for l in range(num_layers)]


@dataclasses.dataclass
class PagedCaches:
    """The caches of an ``Inputs`` moved into a pool of pages: token s of
    sequence b is pool row block_table[b, s // page_size] * page_size +
    s % page_size.  Pool pages no sequence uses hold bf16 NaN."""

    page_size: int
    block_table: np.ndarray  # [B, max_pages] int32
    k_idx: np.ndarray        # [pages * page_size, 128] bf16
    kv: np.ndarray           # [pages * page_size, 576] bf16


BF16_NAN = np.uint16(0x7FC0)


def to_paged(inp: Inputs, page_size: int, seed: int, spare_pages: int = 3) -> PagedCaches:
    """Scatter each sequence's cache rows, one page at a time, to pool pages in
    an order drawn from ``default_rng(seed)`` (a permutation of all pool
    pages, ``spare_pages`` of them left unused).  Row layout only: the rows
    themselves are copied unchanged."""
    rng = np.random.default_rng(seed)
    lens = list(inp.wl.seq_lens)
    pages_of = [(n + page_size - 1) // page_size for n in lens]
    max_pages = max(pages_of)
    total = sum(pages_of) + spare_pages
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((len(lens), max_pages), dtype=np.int32)
    k_pool = np.full((total * page_size, IDX_DIM), BF16_NAN, dtype=np.uint16)
    kv_pool = np.full((total * page_size, D_KV), BF16_NAN, dtype=np.uint16)
    nxt = 0
    for b, n in enumerate(lens):
        r0 = int(inp.seq_row0[b])
        for j in range(pages_of[b]):
            page = int(perm[nxt])
            nxt += 1
            table[b, j] = page
            m = min(page_size, n - j * page_size)
            k_pool[page * page_size: page * page_size + m] = inp.k_idx[r0 + j * page_size: r0 + j * page_size + m]
            kv_pool[page * page_size: page * page_size + m] = inp.kv[r0 + j * page_size: r0 + j * page_size + m]
    return PagedCaches(page_size, table, k_pool, kv_pool)


def derive_layer(inp: Inputs, seed: int) -> Inputs:
    """Another layer over the same batch, cheap to draw at full size: fresh
    q_nope, q_rope, W_UK, W_UV (distributions as above, drawn in that order
    from ``default_rng(seed)``), the latent cache of ``inp`` moved down one row
    (row r holds row r-1 of ``inp``, row 0 the last row), and the indexer
    arrays of ``inp`` (a layer that reuses another's selection reads none)."""
    rng = np.random.default_rng(seed)
    t = inp.q_nope.shape[0]
    inv_sqrt_lat = float(1.0 / np.sqrt(np.float32(D_LAT)))
    q_nope = _normal_bf16(rng, (t, HEADS, D_NOPE))
    q_rope = _normal_bf16(rng, (t, HEADS, D_ROPE))
    w_uk = _normal_bf16(rng, (HEADS, D_LAT, D_NOPE), inv_sqrt_lat)
    w_uv = _normal_bf16(rng, (HEADS, D_LAT, D_V), inv_sqrt_lat)
    return dataclasses.replace(inp, kv=np.roll(inp.kv, 1, axis=0), q_nope=q_nope, q_rope=q_rope,
                               w_uk=w_uk, w_uv=w_uv)


def custom(seq_lens: Sequence[int], queries: Sequence[Tuple[int, int]], seed: int,
           planted_blocks: int = 0, name: str = "custom") -> Inputs:
    return make_inputs(Workload(name, list(seq_lens), list(queries), seed, planted_blocks))


def random_scores(rng: np.random.Generator, t: int, n: int, kind: str = "normal") -> np.ndarray:
    """fp32 score rows for exercising selection alone (not produced by the indexer)."""
    if kind == "normal":
        return rng.standard_normal((t, n), dtype=np.float32) * np.float32(0.19) + np.float32(0.6)
    if kind == "few_values":  # heavy ties
        return rng.integers(0, 7, size=(t, n)).astype(np.float32) * np.float32(0.25)
    if kind == "signed":
        return rng.standard_normal((t, n), dtype=np.float32)
    raise ValueError(kind)
