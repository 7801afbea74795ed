"""Benchmark of the DSA hot path (indexer -> top-2048 -> sparse MLA) on one MI355X.

A step is one dsa_forward call (every stage of the path) over one batch of
seeded synthetic inputs that are already resident in HBM:
  * headline: long decode, 8 sequences x 204,800 cached tokens, one query each
    (value = decode queries/s);
  * also reported: a prefill chunk of 4,096 queries at positions
    200,704..204,799 of one 204,800-token sequence (query-tokens/s), and an
    IndexShare group of 4 decode layers (one selects, three reuse), index_topk
    4096/8192 on the same inputs, and both workloads with 64-token cache pages
    and with the INT4 latent cache.
Prints one JSON line.  Run `python bench.py --help` for options.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from long_context_sparse_index_amd import dsa, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
DECODE = "decode_b8_ctx204k"
PREFILL = "prefill_chunk4096_ctx204k"
TOPK = 2048
PAGE = 64  # tokens per cache page for the paged-cache measurement


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_device(inp):
    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    d = {f: bf(getattr(inp, f)) for f in ("k_idx", "kv", "q_idx", "w", "q_nope", "q_rope", "w_uk", "w_uv")}
    batch = dsa.Batch(torch.from_numpy(inp.q_seq).cuda(), torch.from_numpy(inp.q_pos).cuda(),
                      torch.from_numpy(inp.seq_row0).cuda(), int(inp.q_pos.max()) + 1)
    return batch, d


def algorithmic(inp):
    """Work the method must do (not counting score materialisation or extra
    selection passes).  Bytes: indexer keys 256 B per scanned (query, token)
    pair, 1152 B per gathered row, per-query q/w/q_nope/q_rope in and bf16
    out, and both absorption weights once.  Flops: 8192 per (query, token)
    pair (32x128 MACs), 139,264 per kept row (64 heads x (576 + 512) MACs),
    2 x 64 x 512 x (192 + 256) per query for absorption and up-projection."""
    n_scan = int((inp.q_pos.astype(np.int64) + 1).sum())
    n_kept = int(np.minimum(inp.q_pos.astype(np.int64) + 1, TOPK).sum())
    T = len(inp.q_pos)
    per_query_io = 32 * 128 * 2 + 32 * 2 + 64 * 192 * 2 + 64 * 64 * 2 + 64 * 256 * 2
    weights = 64 * 512 * (192 + 256) * 2
    return {
        "scan_bytes": 256 * n_scan,
        "gather_bytes": 1152 * n_kept,
        "bytes": 256 * n_scan + 1152 * n_kept + per_query_io * T + weights,
        "index_flops": 8192 * n_scan,
        "attn_flops": 139264 * n_kept,
        "flops": 8192 * n_scan + 139264 * n_kept + 2 * 64 * 512 * (192 + 256) * T,
    }


def recorded_traffic(name):
    """HBM bytes per launch recorded with rocprofv3 counters under profiles/
    (FETCH_SIZE and WRITE_SIZE, scaled by a copy-kernel calibration), or None
    when the kernel's sources have changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def attn_op_roofline(alg, T, op_ms):
    """The sparse-MLA op (dsa_sparse_mla_attn: absorption, core, split merge if
    any, up-projection) against both peaks: algorithmic bytes (gathered rows,
    both absorption weights, per-query q_nope/q_rope in and bf16 out) per HBM
    peak, and algorithmic flops (the core's 139,264 per kept row plus the
    absorption and up-projection) per bf16 MFMA peak."""
    t = op_ms * 1e-3
    nbytes = alg["gather_bytes"] + 64 * 512 * (192 + 256) * 2 + T * (64 * 192 * 2 + 64 * 64 * 2 + 64 * 256 * 2)
    flops = alg["attn_flops"] + 2 * 64 * 512 * (192 + 256) * T
    return {"launch": "dsa_sparse_mla_attn (absorption, core, split merge, up-projection)", "ms": op_ms,
            "algorithmic_bytes": nbytes, "hbm_gbs": nbytes / t / 1e9, "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS,
            "gather_gbs": alg["gather_bytes"] / t / 1e9,
            "algorithmic_flops": flops, "tflops": flops / t / 1e12,
            "mfma_frac": flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS}


def time_calls(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms


def time_each(fn, steps, warmup, flush=None):
    """Per-step HIP-event times (ms) on the current stream: median, p10, p90.
    With `flush` (a device tensor of 512 MB or more), it is overwritten before
    every step, outside the timed region, so that no input stays in the 256 MB
    MALL or in L2 from the previous step."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        if flush is not None:
            flush.fill_(1.0)
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.sort(np.asarray([a.elapsed_time(b) for a, b in ev]))
    return {"median": float(np.median(t)), "p10": float(np.percentile(t, 10)), "p90": float(np.percentile(t, 90))}


def paged_copy(inp, d, page_size, seed=4096):
    """The workload's caches scattered over a device page pool (seeded page
    permutation, 3 spare pages): every sequence length must be a multiple of
    page_size.  Returns (block_table [B, pages] int32, k_idx pool, kv pool)."""
    lens = list(inp.wl.seq_lens)
    assert all(n % page_size == 0 for n in lens)
    npg = sum(n // page_size for n in lens)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    perm = torch.randperm(npg + 3, generator=g, device="cuda")[:npg]
    pools = []
    for x, width in ((d["k_idx"], 128), (d["kv"], 576)):
        pool = torch.zeros(((npg + 3) * page_size, width), dtype=x.dtype, device="cuda")
        pool.view(npg + 3, page_size, width)[perm] = x.view(npg, page_size, width)
        pools.append(pool)
    table = torch.zeros((len(lens), max(lens) // page_size), dtype=torch.int32, device="cuda")
    j = 0
    for b, n in enumerate(lens):
        table[b, : n // page_size] = perm[j: j + n // page_size].to(torch.int32)
        j += n // page_size
    return table, pools[0], pools[1]


def run_workload(name, steps, warmup, with_ops=True, extra_k=(), page_size=0, dist=False):
    log(f"[bench] {name}: generating inputs")
    t0 = time.time()
    inp = synth.make_inputs(synth.workload(name))
    log(f"[bench] {name}: generated in {time.time() - t0:.1f}s; uploading")
    batch, d = to_device(inp)
    T = batch.T
    out = torch.empty((T, 64, 256), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, TOPK), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.OP_FORWARD, T, batch.max_ctx, TOPK), dtype=torch.uint8,
                     device="cuda")

    def step():
        dsa.dsa_forward(batch, d["q_idx"], d["w"], d["k_idx"], d["q_nope"], d["q_rope"], d["kv"], d["w_uk"],
                        d["w_uv"], k=TOPK, out=out, idx=idx, ws=ws)

    log(f"[bench] {name}: timing {steps} steps after {warmup} warmup")
    torch.cuda.synchronize()
    ms = time_calls(step, steps, warmup)
    by_k = {}
    if dist:
        # per-step distribution, inputs resident; then with a 512 MB write before
        # every step (nothing of the previous step left in the MALL)
        by_k["dist"] = time_each(step, steps, 2)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        by_k["flushed"] = time_each(step, steps, 2, flush=flush)
        del flush
        log(f"[bench] {name}: per step median {by_k['dist']['median']:.3f} ms; with a 512 MB MALL flush "
            f"between steps {by_k['flushed']['median']:.3f} ms")
    # index_topk as a runtime parameter: the same resident inputs with larger k
    for k in extra_k:
        idx_k = torch.empty((T, k), dtype=torch.int32, device="cuda")
        ws_k = torch.empty(dsa.dsa_workspace_bytes(dsa.OP_FORWARD, T, batch.max_ctx, k), dtype=torch.uint8,
                           device="cuda")

        def step_k():
            dsa.dsa_forward(batch, d["q_idx"], d["w"], d["k_idx"], d["q_nope"], d["q_rope"], d["kv"], d["w_uk"],
                            d["w_uv"], k=k, out=out, idx=idx_k, ws=ws_k)

        by_k[k] = time_calls(step_k, steps, warmup)
        log(f"[bench] {name}: k={k} {by_k[k]:.3f} ms/step")
        del idx_k, ws_k
    if page_size:
        # paged caches: the same rows behind a block table
        table, k_pool, kv_pool = paged_copy(inp, d, page_size)
        pb = dsa.Batch(batch.q_seq, batch.q_pos, None, batch.max_ctx, block_table=table, page_size=page_size)

        def step_p():
            dsa.dsa_forward(pb, d["q_idx"], d["w"], k_pool, d["q_nope"], d["q_rope"], kv_pool, d["w_uk"],
                            d["w_uv"], k=TOPK, out=out, idx=idx, ws=ws)

        by_k["paged"] = time_calls(step_p, steps, warmup)
        log(f"[bench] {name}: paged ({page_size}-token pages) {by_k['paged']:.3f} ms/step")
        del table, k_pool, kv_pool
        torch.cuda.empty_cache()
        # INT4 latent cache: the same rows quantised (400 B per row instead of 1152)
        kv_q = dsa.dsa_quantize_kv_int4(d["kv"])
        qb = dsa.Batch(batch.q_seq, batch.q_pos, batch.seq_row0, batch.max_ctx, kv_format=dsa.KV_INT4)

        def step_q():
            dsa.dsa_forward(qb, d["q_idx"], d["w"], d["k_idx"], d["q_nope"], d["q_rope"], kv_q, d["w_uk"],
                            d["w_uv"], k=TOPK, out=out, idx=idx, ws=ws)

        by_k["int4"] = time_calls(step_q, steps, warmup)
        log(f"[bench] {name}: INT4 latent cache {by_k['int4']:.3f} ms/step")
        del kv_q
        torch.cuda.empty_cache()
    if not with_ops:
        log(f"[bench] {name}: {ms:.3f} ms/step")
        del ws, out, idx
        torch.cuda.empty_cache()
        return inp, ms, {}, by_k
    # per-op breakdown: each ABI call below launches that op's kernels only
    scores = torch.empty((T, dsa.score_ld(batch.max_ctx)), dtype=torch.float32, device="cuda")
    mla_ws = torch.empty(max(dsa.dsa_workspace_bytes(dsa.OP_SPARSE_MLA, T, batch.max_ctx, TOPK), 256),
                         dtype=torch.uint8, device="cuda")
    ops = {
        "index_scores": time_calls(lambda: dsa.dsa_index_scores(batch, d["q_idx"], d["w"], d["k_idx"], scores),
                                   steps, warmup),
        "topk": time_calls(lambda: dsa.dsa_topk(batch, scores, TOPK, idx), steps, warmup),
        "sparse_mla": time_calls(lambda: dsa.dsa_sparse_mla_attn(batch, d["q_nope"], d["q_rope"], d["kv"],
                                                                 d["w_uk"], d["w_uv"], idx, out=out, ws=mla_ws),
                                 steps, warmup),
    }
    log(f"[bench] {name}: {ms:.3f} ms/step; ops(ms) " + ", ".join(f"{k}={v:.3f}" for k, v in ops.items()))
    return inp, ms, ops, by_k


def index_share_group(inp, steps, warmup, freq=4):
    """IndexShare on the decode workload: one group of `freq` layers, the first
    running the whole path and keeping its selection, the other freq-1 running
    sparse MLA alone on their own caches at those positions.  The shared
    layers' caches, queries and weights are drawn on the device from a seeded
    generator (same distributions as the synthetic recipe)."""
    batch, d = to_device(inp)
    T = batch.T
    g = torch.Generator(device="cuda")
    g.manual_seed(4099)
    rows = d["kv"].shape[0]

    def normal_bf16(shape, scale=1.0):
        return (torch.randn(shape, generator=g, device="cuda") * scale).to(torch.bfloat16)

    shared = []
    for _ in range(freq - 1):
        shared.append({"kv": normal_bf16((rows, 576)), "q_nope": normal_bf16((T, 64, 192)),
                       "q_rope": normal_bf16((T, 64, 64)), "w_uk": normal_bf16((64, 512, 192), 512 ** -0.5),
                       "w_uv": normal_bf16((64, 512, 256), 512 ** -0.5),
                       "out": torch.empty((T, 64, 256), dtype=torch.bfloat16, device="cuda")})
    out = torch.empty((T, 64, 256), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, TOPK), dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.dsa_workspace_bytes(dsa.OP_FORWARD, T, batch.max_ctx, TOPK), dtype=torch.uint8,
                     device="cuda")
    mla_ws = torch.empty(max(dsa.dsa_workspace_bytes(dsa.OP_SPARSE_MLA, T, batch.max_ctx, TOPK), 256),
                         dtype=torch.uint8, device="cuda")

    def group():
        dsa.dsa_forward(batch, d["q_idx"], d["w"], d["k_idx"], d["q_nope"], d["q_rope"], d["kv"], d["w_uk"],
                        d["w_uv"], k=TOPK, out=out, idx=idx, ws=ws)
        for L in shared:
            dsa.dsa_sparse_mla_attn(batch, L["q_nope"], L["q_rope"], L["kv"], L["w_uk"], L["w_uv"], idx,
                                    out=L["out"], ws=mla_ws)

    log(f"[bench] index share: timing {steps} groups of {freq} layers")
    ms = time_calls(group, steps, warmup)
    alg = algorithmic(inp)
    n_kept = int(np.minimum(inp.q_pos.astype(np.int64) + 1, TOPK).sum())
    shared_bytes = 1152 * n_kept + (64 * 192 * 2 + 64 * 64 * 2 + 64 * 256 * 2) * T + 64 * 512 * (192 + 256) * 2
    group_bytes = alg["bytes"] + (freq - 1) * shared_bytes
    log(f"[bench] index share: {ms:.3f} ms per group")
    return {"workload": DECODE, "layers_per_group": freq,
            "schedule": f"1 full layer (indexer + top-k + sparse MLA) + {freq - 1} shared (sparse MLA on the "
                        "full layer's selection)",
            "value": T * freq / (ms * 1e-3), "unit": "decode query-layers/s", "ms_per_group": ms,
            "ms_per_layer": ms / freq, "algorithmic_bytes_per_group": group_bytes,
            "hbm_frac": group_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def cpu_baseline(inp, budget_s):
    """The oracle as it stands (numpy fp64), on a bounded sample of queries."""
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    T = len(inp.q_pos)
    done = 0
    t0 = time.time()
    while done < 2 or time.time() - t0 < budget_s:  # cycles over the workload's queries
        O.query_forward(inp, done % T, k=TOPK)
        done += 1
        if done % T == 0:
            log(f"[bench] cpu oracle: {done} queries in {time.time() - t0:.1f}s")
    el = time.time() - t0
    return {"value": done / el, "unit": "decode queries/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} query evaluations cycling over the {T} queries of {DECODE} (full indexer scan, "
                      f"full-sort top-2048, explicit MLA), {el:.1f}s wall"}


def cpu_baseline_prefill(inp, budget_s):
    """The oracle on a bounded sample of the prefill chunk's queries (each: indexer
    over its whole history, full-sort top-2048, explicit MLA), in query-tokens/s."""
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    T = len(inp.q_pos)
    done = 0
    t0 = time.time()
    while done < 2 or time.time() - t0 < budget_s:  # queries spread over the chunk
        O.query_forward(inp, (done * 997) % T, k=TOPK)
        done += 1
    el = time.time() - t0
    log(f"[bench] cpu oracle (prefill): {done} queries in {el:.1f}s")
    return {"value": done / el, "unit": "query-tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of the 4,096 queries of {PREFILL} (every 997th, cyclic; each: indexer over "
                      f"its 200K+ history, full-sort top-2048, explicit MLA), {el:.1f}s wall"}


OTHER_CONFIGS = (
    # (workload, kind): the other configurations of the benchmark table, each one dsa_forward per step
    ("decode_b32_ctx32k", "decode"),
    ("prefill_chunk4096_ctx131k", "prefill"),
    ("causal_prefill_65k_planted", "prefill"),
)


def other_config(name, kind, steps, warmup):
    inp, ms, _, _ = run_workload(name, steps, warmup, with_ops=False)
    alg = algorithmic(inp)
    T = len(inp.q_pos)
    r = {"workload": name, "queries": T, "ctx": int(max(inp.wl.seq_lens)), "ms_per_step": ms,
         "value": T / (ms * 1e-3), "unit": "decode queries/s" if kind == "decode" else "query-tokens/s"}
    if kind == "decode":
        r["hbm_frac"] = alg["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
        r["algorithmic_bytes"] = alg["bytes"]
    else:
        r["mfma_frac"] = alg["flops"] / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS
        r["algorithmic_flops"] = alg["flops"]
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk measurement")
    ap.add_argument("--no-index-share", action="store_true", help="skip the IndexShare layer-group measurement")
    ap.add_argument("--no-topk-variants", action="store_true",
                    help="skip the index_topk 4096/8192 measurements (decode) and 8192 (prefill)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="profiling aid: run only the prefill chunk (prints no result line)")
    ap.add_argument("--no-ops", action="store_true", help="profiling aid: skip the per-op timing loops")
    ap.add_argument("--only", default="",
                    help="profiling aid: comma-separated workloads whose forward alone is run (prints no result "
                         "line), e.g. decode_b32_ctx32k,prefill_chunk4096_ctx204k")
    ap.add_argument("--decode-only", action="store_true",
                    help="profiling aid: run only the decode workload (prints no result line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="profiling aid: run a plain 1 GiB device-to-device copy 3 times and exit "
                         "(reference for HBM byte counters)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of CPU oracle work per workload, decode and prefill (0 = skip)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the 32K decode batch, the 131K prefill chunk and the full 65K causal prefill")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for {args.gpus}); the multi-GPU sharding "
              "is a design, not an implementation", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 1 GiB 3 times")
        return
    dsa.lib()
    if args.only:
        for name in args.only.split(","):
            run_workload(name, args.steps, args.warmup, not args.no_ops)
            torch.cuda.empty_cache()
        return
    extra_k = () if args.no_topk_variants else (4096, 8192)
    if args.decode_only:
        run_workload(DECODE, args.steps, args.warmup, not args.no_ops, extra_k)
        return
    if args.prefill_only:
        run_workload(PREFILL, args.steps, args.warmup, not args.no_ops, extra_k[-1:])
        return

    inp, ms, ops, dec_k = run_workload(DECODE, args.steps, args.warmup, extra_k=extra_k, page_size=PAGE,
                                       dist=True)
    dec_paged = dec_k.pop("paged")
    dec_int4 = dec_k.pop("int4")
    dec_dist = dec_k.pop("dist")
    dec_flushed = dec_k.pop("flushed")
    alg = algorithmic(inp)
    T = len(inp.q_pos)
    scan_ms = ops["index_scores"]
    achieved = alg["scan_bytes"] / (scan_ms * 1e-3) / 1e9
    result = {
        "metric": "decode queries/s + prefill query-tokens/s at 204.8K ctx; % HBM / MFMA peak",
        "value": T / (ms * 1e-3),
        "unit": "decode queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": DECODE, "sequences": 8, "ctx": 204800, "queries": T, "index_topk": TOPK},
        "roofline": {"bound": "hbm", "kernel": "idx_scan_kernel",
                     "launch": "dsa_index_scores: the forward's key scan without the slice lists, same grid",
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": recorded_traffic("idx_scan_kernel_hbm_traffic_decode_b8_ctx204k.json"),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                     "algorithmic_bytes": alg["scan_bytes"]},
        "whole_step": {"algorithmic_bytes": alg["bytes"],
                       "hbm_frac": alg["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "step_ms": {"resident": dec_dist,
                    "mall_flushed": dict(dec_flushed, note="512 MB written before every step, outside the "
                                                           "timed region"),
                    "flushed_value": T / (dec_flushed["median"] * 1e-3)},
        "ops_ms": ops,
        "attention_op": attn_op_roofline(alg, T, ops["sparse_mla"]),
        "index_topk_variants": {str(k): {"ms_per_step": v, "value": T / (v * 1e-3), "unit": "decode queries/s"}
                                for k, v in dec_k.items()},
        "paged": {"page_size": PAGE, "ms_per_step": dec_paged, "value": T / (dec_paged * 1e-3),
                  "unit": "decode queries/s", "vs_contiguous": ms / dec_paged},
        "kv_int4": {"ms_per_step": dec_int4, "value": T / (dec_int4 * 1e-3), "unit": "decode queries/s",
                    "vs_bf16_cache": ms / dec_int4, "row_bytes": 400},
    }
    if not args.no_index_share:
        result["index_share"] = index_share_group(inp, args.steps, args.warmup)
        torch.cuda.empty_cache()
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    del inp
    if not args.no_prefill:
        pre_steps, pre_warmup = max(10, min(args.steps // 2, 25)), max(3, min(args.warmup, 5))
        pinp, pms, pops, pre_k = run_workload(PREFILL, pre_steps, pre_warmup,
                                              extra_k=extra_k[-1:], page_size=PAGE)
        pre_paged = pre_k.pop("paged")
        pre_int4 = pre_k.pop("int4")
        palg = algorithmic(pinp)
        pach = palg["index_flops"] / (pops["index_scores"] * 1e-3) / 1e12
        result["prefill"] = {
            "workload": PREFILL, "value": len(pinp.q_pos) / (pms * 1e-3), "unit": "query-tokens/s",
            "ms_per_step": pms, "steps": pre_steps, "warmup": pre_warmup, "ops_ms": pops,
            "attention_op": attn_op_roofline(palg, len(pinp.q_pos), pops["sparse_mla"]),
            "index_topk_variants": {str(k): {"ms_per_step": v, "value": len(pinp.q_pos) / (v * 1e-3),
                                             "unit": "query-tokens/s"} for k, v in pre_k.items()},
            "paged": {"page_size": PAGE, "ms_per_step": pre_paged, "value": len(pinp.q_pos) / (pre_paged * 1e-3),
                      "unit": "query-tokens/s", "vs_contiguous": pms / pre_paged},
            "kv_int4": {"ms_per_step": pre_int4, "value": len(pinp.q_pos) / (pre_int4 * 1e-3),
                        "unit": "query-tokens/s", "vs_bf16_cache": pms / pre_int4, "row_bytes": 400},
            "mfma_frac_whole_step": palg["flops"] / (pms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "idx_gemm_kernel",
                         "launch": "dsa_index_scores: the indexer GEMM writing the score matrix (the forward runs "
                                   "the same tile loop keeping candidates instead)",
                         "achieved": pach,
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": pach / MFMA_BF16_PEAK_TFLOPS,
                         "traffic": recorded_traffic("idx_gemm_kernel_hbm_traffic_prefill_chunk4096_ctx204k.json"),
                         "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                         "algorithmic_flops": palg["index_flops"]},
        }
        if args.cpu_budget > 0:
            result["prefill"]["cpu_baseline"] = cpu_baseline_prefill(pinp, args.cpu_budget)
        del pinp
    if not args.no_other_configs:
        result["other_configs"] = [other_config(n, kind, max(5, min(args.steps // 4, 12)), 2) for n, kind in OTHER_CONFIGS]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
