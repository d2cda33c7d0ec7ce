"""Benchmark: routed block-sparse attention over a growing KV history at chunk
48 on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk C]
                    [--no-cpu-baseline] [--no-dense] [--tiles] [--sweep FILE] [--rollout FILE]

Workload: the 14B-like growing-context layer -- 40 heads, head dim 128, a
3 x 30 x 52 latent chunk (4680 tokens, 37 blocks of 128), a KV history of C
chunks (default 48: 224,640 tokens, 1776 blocks), fixed top-K 50, bf16.
Inputs are seeded synthetic tensors (``workloads.c4``), resident in HBM
before timing starts.

One step is one attention call of the chunked model, the whole hot path:
(the Gilbert index of the chunk grid is computed once per grid shape and
kept; it is timed alone in the breakdown) permutation of the current chunk's raster
Q, K, V into Gilbert head-major blocks (K, V into the store's newest slot);
routing (mean-pool Q and the K blocks appended since the previous call --
the pooled history keys are cached across calls, as the store only grows by
appending -- then score, top-K, CSR); block-sparse attention; inverse
permutation of O.  The step time with every history block re-pooled is
reported beside it (``step_full_k_pool_ms``), and so is the same step
replayed from a HIP graph (``step_hip_graph_ms``: identical kernels, no
launch gaps; every replay is checked bitwise against the eager step), and
each stage timed alone with its algorithmic bytes and GB/s, and the
attention launch with L2 and MALL flushed before each call
(``breakdown``), the bf16 matrix rate a register-only MFMA probe gets at
the current clock (``mfma_probe``), dense attention through the same kernel
(``dense``), the shader/memory clocks at start and end (``clocks``), the
ragged structured configuration C5 at chunk 48 (``c5``), the attention of
the Wan-1.3B-like layer C2 with its matrix-core roofline (``c2``), and
the step with the materialised route instead of the top-K
(``materialized``: coverage-gated budgets, previous-chunk reservation,
cumulative-mass prefix and the local window), its overlap and coverage
produced from frustum slabs on the GPU (``geometry``: camera-facing boxes,
separating-axis test, grid IoU; once per chunk, shared by all layers).

Printed: one JSON line.  ``value`` = effective TFLOP/s of the step (valid
selected (query, key) pairs x 4 d FLOP, divided by the step time).  The
attention kernel alone is timed with events on its stream inside the timed
region; ``roofline`` prices it against HBM bandwidth with its algorithmic
bytes (each distinct selected K/V block once, plus Q, O and the lists).
``cpu_baseline`` times the float64 oracle on a bounded sample on the host.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "block-sparse attn effective TFLOP/s + ms/call at chunk 48; % bf16 MFMA peak"
SETTLE_MS = 400.0              # steady GPU load run before the warm-up steps (clock ramp after set-up)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_c4_chunk48_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_attention_gilbert_amd", "csrc", "attn.hip")


def attn_source_hash() -> str:
    with open(ATTN_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def setup_c4(chunk: int = 48, heads=None, device="cuda:0"):
    """C4 at history length ``chunk``: the store holds chunks 0..chunk-1 in
    Gilbert block layout; the current chunk (index chunk-1) is also given in
    raster layout, obtained with the library's inverse permutation, so the
    step's forward permutation rewrites the slot with identical bits."""
    import torch

    import workloads
    from block_sparse_attention_gilbert_amd import gilbert_perm
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention

    w = workloads.c4(c=chunk, heads=heads)
    k_store = w.k.contiguous().to(device)
    v_store = w.v.contiguous().to(device)
    ra = RoutedAttention((3, 30, 52), w.heads, w.d, w.bs, chunk, device=device, k_cap=50,
                         k_store=k_store, v_store=v_store)
    cur = chunk - 1
    ks, vs = ra.slot(cur)
    # the step reads Q in raster order; the dense and sweep timings read the
    # permuted copy, which stays as set here
    ra.q_blk.copy_(w.q.to(device))
    q_raster = gilbert_perm(w.q.to(device), ra.perm, block=w.bs, inverse=True)
    k_raster = gilbert_perm(ks, ra.perm, block=w.bs, inverse=True)
    v_raster = gilbert_perm(vs, ra.perm, block=w.bs, inverse=True)
    torch.cuda.synchronize()
    return dict(w=w, ra=ra, q_raster=q_raster, k_raster=k_raster, v_raster=v_raster, cur=cur)


def run_step(st, attn_events=None):
    return st["ra"].step(st["q_raster"], st["k_raster"], st["v_raster"], st["cur"], attn_events=attn_events)


def work_counts(row_ptr, col_idx, q_len, k_len, heads, nqb, bs, d):
    """Exact effective FLOP, tile FLOP, distinct (head, block) pairs and the
    algorithmic bytes of one attention launch, from the CSR lists."""
    import numpy as np
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    k_len = np.asarray(k_len, dtype=np.int64)
    q_len = np.asarray(q_len, dtype=np.int64)
    eff = 0
    pairs = 0
    uniq_rows = 0
    for h in range(heads):
        seg = ci[rp[h * nqb]:rp[(h + 1) * nqb]]
        for i in range(nqb):
            lst = ci[rp[h * nqb + i]:rp[h * nqb + i + 1]]
            eff += int(q_len[i]) * int(k_len[lst].sum())
            pairs += len(lst)
        u = np.unique(seg)
        uniq_rows += int(k_len[u].sum())
    flop = 4 * d * eff
    tile_flop = 4 * d * bs * bs * pairs
    kv_bytes = 2 * uniq_rows * d * 2                   # K and V rows of the distinct selected blocks
    qo_bytes = 2 * heads * int(q_len.sum()) * d * 2    # Q in, O out
    list_bytes = 4 * (len(rp) + int(rp[-1]))
    return dict(flop=flop, tile_flop=tile_flop, pairs=pairs, uniq_rows=uniq_rows,
                alg_bytes=kv_bytes + qo_bytes + list_bytes, visits=pairs)


def step_graph_ms(st, reps: int):
    """The same step captured once into a HIP graph and replayed (the
    kernels are unchanged; the launch gaps between them go).  Every replay's
    output must equal the eager step's bitwise; returns ms per replay."""
    import torch
    ra = st["ra"]
    o_eager, _ = run_step(st)
    o_eager = o_eager.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run_step(st)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run_step(st)
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ra.o_raster, o_eager), "graph replay differs from the eager step"
        run_step(st)  # eager work between replays
        torch.cuda.synchronize()
    # untimed replays first: the capture and the checks allocate, which
    # slows the next few dozen steps
    for _ in range(30):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(ra.o_raster, o_eager), "graph replay differs from the eager step"
    return e0.elapsed_time(e1) / reps


def _time_ms(fn, reps: int, warm: int = 10, between=None):
    """Median ms of ``fn`` over ``reps`` back-to-back calls, each bracketed
    by events on the current stream (no host synchronisation in between, so
    the GPU does not idle and drop its clock); ``between`` runs, untimed,
    before each call."""
    import statistics

    import torch
    for _ in range(warm):
        if between:
            between()
        fn()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        if between:
            between()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in evs)


def breakdown(st, reps: int):
    """Each stage of the step alone (median of ``reps`` calls), with its
    algorithmic bytes and the GB/s that gives: the Gilbert index, the
    forward passes (K with its block means and V into the store slot, the
    block means of Q), the router over the pooled blocks, the attention
    launch (reading Q and writing O in raster order, so neither is
    permuted by a pass of its own)."""
    import torch
    w, ra = st["w"], st["ra"]
    cur = st["cur"]
    L, heads, d = 4680, w.heads, w.d
    raster = L * heads * d * 2
    blocked = ra.rows_c * heads * d * 2

    def fwd():                                 # as in the step: K and V permuted, Q only pooled
        ra.permute_inputs(st["q_raster"], st["k_raster"], st["v_raster"], cur, q_blocks=False)

    def route():                               # as in the step: every block's mean is already pooled
        return ra.route(cur, qpool=ra.qbar)

    nkb = w.nkb
    k_hist, v_hist = ra.k_store[:, : nkb * w.bs], ra.v_store[:, : nkb * w.bs]
    r = route()
    torch.cuda.synchronize()
    wc = work_counts(r["row_ptr"], r["col_idx"], w.q_len, w.k_len, w.heads, w.nqb, w.bs, w.d)
    n_cand = nkb
    pooled = heads * w.nqb * d * 8                         # one chunk's block means (float64)
    route_bytes = (pooled                                  # pooled queries read
                   + heads * n_cand * d * 8                # pooled keys (float64) read
                   + 2 * heads * w.nqb * n_cand * 8        # selection keys written and read
                   + 4 * (heads * w.nqb + 1 + int(r["row_ptr"][-1])))
    stages = {
        "gilbert_index": (lambda: ra._index(), 4 * 2 * L),
        "forward_permutes": (fwd, 3 * raster + 2 * blocked + 2 * pooled),
        "route": (route, route_bytes),
        "attention": (lambda: ra._attend(r, nkb, k_hist, v_hist, None, None, True, st["q_raster"]),
                      wc["alg_bytes"]),
    }
    out = {}
    for name, (fn, nbytes) in stages.items():
        ms = _time_ms(fn, reps)
        out[name] = {"ms": round(ms, 4), "alg_bytes": int(nbytes), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    # the same attention launch with L2 and the 256 MB MALL flushed before
    # each call (a 512 MB write, untimed, right before it)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=ra.device)
    ms = _time_ms(lambda: ra._attend(r, nkb, k_hist, v_hist, None, None, True, st["q_raster"]), reps,
                  between=lambda: scrub.fill_(1))
    del scrub
    out["attention_cold_ms"] = round(ms, 4)
    return out


def mfma_probe(reps: int = 10):
    """The bf16 matrix rate this GPU delivers right now: register-only
    v_mfma_f32_32x32x16_bf16 chains on every CU.  ``implied_sclk_mhz`` is
    the clock at which that rate would be the full matrix rate (256 CUs x 4
    SIMDs x 1024 FLOP per cycle)."""
    import torch

    import block_sparse_attention_gilbert_amd as bsa
    best = None
    for wgs in (512, 768, 1024):          # 2, 3 or 4 workgroups per CU
        iters = 256
        sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
        fn = lambda: bsa._check(bsa._lib.bsa_diag_mfma_bf16(wgs, iters, bsa._ptr(sink), bsa._stream(None)))
        ms = _time_ms(fn, reps)
        tf = wgs * 4 * 4 * iters * 32768 / (ms * 1e-3) / 1e12
        if best is None or tf > best["tflops"]:
            best = {"tflops": round(tf, 1), "ms": round(ms, 4), "workgroups_per_cu": wgs // 256}
    best["what"] = "register-only bf16 MFMA chains (4 per wave), best of 2-4 workgroups per CU"
    best["implied_sclk_mhz"] = round(best["tflops"] * 1e12 / (256 * 4 * 1024) / 1e6)
    return best


def clocks():
    """Current shader and memory clocks from rocm-smi (None if unavailable)."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20).stdout
    except Exception:  # pragma: no cover
        return None
    out = {}
    for key in ("sclk", "mclk", "fclk"):
        m = re.search(r"%s clock level: \d+: \((\d+)Mhz\)" % key, txt)
        if m:
            out[key + "_mhz"] = int(m.group(1))
    return out or None


def tiles(chunk: int, reps: int, device: str, tile=(1, 8, 16)):
    """The step with fixed 3-D tile blocks (a tile of 1 x 8 x 16 = 128 tokens;
    48 tiles per chunk, the edge tiles partly empty) instead of 128-token
    runs of the curve, at the same chunk, top-K 50: the same draws of C4 laid
    out in tiles (``workloads.c4`` with the tile lengths)."""
    import numpy as np
    import torch

    import workloads
    from block_sparse_attention_gilbert_amd import gilbert_tile_index
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention

    _, block_len, _ = gilbert_tile_index(3, 30, 52, tile, device=device)
    lens = block_len.cpu().numpy()
    w = workloads.c4(c=chunk, chunk_lens=lens)
    ra = RoutedAttention((3, 30, 52), w.heads, w.d, w.bs, chunk, device=device, k_cap=50,
                         k_store=w.k.contiguous().to(device), v_store=w.v.contiguous().to(device), tile=tile)
    cur = chunk - 1
    ks, vs = ra.slot(cur)
    q_r = ra.to_raster(w.q.to(device), torch.empty((4680, w.heads, w.d), dtype=w.dtype, device=device))
    k_r = ra.to_raster(ks, torch.empty((4680, w.heads, w.d), dtype=w.dtype, device=device))
    v_r = ra.to_raster(vs, torch.empty((4680, w.heads, w.d), dtype=w.dtype, device=device))
    before = ks.clone()
    for _ in range(3):
        ra.step(q_r, k_r, v_r, cur)
    torch.cuda.synchronize()
    assert torch.equal(before, ra.slot(cur)[0]), "tile permutation did not reproduce the store slot"
    del before
    for _ in range(30):  # allocations slow the next few dozen steps
        ra.step(q_r, k_r, v_r, cur)
    torch.cuda.synchronize()
    events = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        _, r = ra.step(q_r, k_r, v_r, cur, attn_events=events)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / reps
    attn_ms = sum(a.elapsed_time(b) for a, b in events) / len(events)
    wc = work_counts(r["row_ptr"], r["col_idx"], w.q_len, w.k_len, w.heads, w.nqb, w.bs, w.d)
    out = {"tile": list(tile), "blocks_per_chunk": int(w.nqb), "kv_blocks": int(w.nkb),
           "mean_valid_per_block": round(float(np.mean(lens)), 2),
           "ms_per_step": round(ms_step, 4), "attn_ms": round(attn_ms, 4),
           "step_effective_tflops": round(wc["flop"] / (ms_step * 1e-3) / 1e12, 2),
           "attn_effective_tflops": round(wc["flop"] / (attn_ms * 1e-3) / 1e12, 2),
           "attn_tile_tflops": round(wc["tile_flop"] / (attn_ms * 1e-3) / 1e12, 2),
           "effective_flop": wc["flop"]}
    del ra, w, ks, vs, q_r, k_r, v_r
    torch.cuda.empty_cache()
    return out


def setup_c5(device: str):
    """C5 at chunk 48 (ragged budgets K ~ U{8..143} over 47 history chunks of
    74 blocks of 64, the current chunk's 74 blocks attended densely, a
    structured field): the pipeline with the history appended chunk by
    chunk, and the current chunk's inputs on the device."""
    import torch

    import workloads
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention

    w = workloads.c5()
    n_chunks = 48
    ra = RoutedAttention(w.grid, w.heads, w.d, w.bs, n_chunks, device=device, k_cap=143, n_dense_tail_chunks=1)
    for c in range(n_chunks - 1):
        ra.append(w.k_raster[c].to(device), w.v_raster[c].to(device), c)
    kpr = torch.from_numpy(w.k_per_row).to(device)
    q_r, k_r, v_r = w.q_raster.to(device), w.k_raster[-1].to(device), w.v_raster[-1].to(device)
    return ra, kpr, q_r, k_r, v_r, n_chunks


def c5_config(reps: int, device: str):
    """C5 at chunk 48: the whole step and the attention launch (HIP events
    on the step's stream)."""
    import torch

    ra, kpr, q_r, k_r, v_r, n_chunks = setup_c5(device)
    for _ in range(30):
        _, r = ra.step(q_r, k_r, v_r, n_chunks - 1, k_per_row=kpr)
    torch.cuda.synchronize()
    events = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        _, r = ra.step(q_r, k_r, v_r, n_chunks - 1, k_per_row=kpr, attn_events=events)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / reps
    attn_ms = sum(a.elapsed_time(b) for a, b in events) / len(events)
    q_len = ra.q_len.cpu().numpy()
    k_len = ra.kv_len.cpu().numpy()
    wc = work_counts(r["row_ptr"], r["col_idx"], q_len, k_len, ra.heads, ra.nbc, ra.block, ra.d)
    out = {"workload": "C5 ragged structured, chunk 48, blocks of 64", "ms_per_step": round(ms_step, 4),
           "attn_ms": round(attn_ms, 4), "listed_blocks": wc["pairs"], "effective_flop": wc["flop"],
           "attn_effective_tflops": round(wc["flop"] / (attn_ms * 1e-3) / 1e12, 2),
           "attn_alg_gbs": round(wc["alg_bytes"] / (attn_ms * 1e-3) / 1e9, 1),
           "step_effective_tflops": round(wc["flop"] / (ms_step * 1e-3) / 1e12, 2)}
    del ra, q_r, k_r, v_r
    torch.cuda.empty_cache()
    return out


def c2_config(reps: int, device: str):
    """C2 (the Wan-1.3B-like layer: 12 heads, 37 query blocks of 128, 143
    history blocks, top-K 50, bf16): routed once, then the attention launch
    timed alone (median of ``reps``), its effective TFLOP/s and its
    roofline.  Every query block of a head reuses the same 143 history
    blocks (112 MB of K and V for the 12 heads), about 1300 FLOP per
    algorithmic byte: the launch is bound by the matrix cores, not HBM."""
    import statistics

    import numpy as np
    import torch

    import workloads
    from block_sparse_attention_gilbert_amd import block_sparse_attn, route_topk

    w = workloads.c2()
    q, k, v = w.q.to(device), w.k.to(device), w.v.to(device)
    ql = torch.from_numpy(w.q_len.astype(np.int32)).to(device)
    kl = torch.from_numpy(w.k_len.astype(np.int32)).to(device)
    r = route_topk(q, k, block=w.bs, nqb=w.nqb, nkb=w.nkb, scale=w.scale, q_block_len=ql, kv_block_len=kl,
                   k_fixed=50)
    out_t = torch.empty_like(q)

    def call():
        block_sparse_attn(q, k, v, r["row_ptr"], r["col_idx"], block=w.bs, scale=w.scale, q_block_len=ql,
                          kv_block_len=kl, out=out_t)

    for _ in range(max(20, reps)):
        call()
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    wc = work_counts(r["row_ptr"], r["col_idx"], w.q_len, w.k_len, w.heads, w.nqb, w.bs, w.d)
    tflops = wc["flop"] / (ms * 1e-3) / 1e12
    intensity = wc["flop"] / wc["alg_bytes"]
    out = {"workload": "C2 Wan-1.3B-like layer (12 heads, 143 history blocks, top-K 50)", "attn_ms": round(ms, 4),
           "effective_flop": wc["flop"], "attn_effective_tflops": round(tflops, 2),
           "pct_bf16_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
           "roofline": {"bound": "mfma" if intensity * PEAK_HBM_GBS / 1e3 > PEAK_BF16_TFLOPS else "hbm",
                        "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                        "intensity_flop_per_byte": round(intensity, 1), "alg_bytes_per_launch": wc["alg_bytes"]}}
    del q, k, v, out_t, r
    torch.cuda.empty_cache()
    return out


def geometry(st, reps: int):
    """Overlap and coverage of the current chunk's query blocks from frustum
    slabs (``workloads.geometry_inputs``: a camera path through a ray-cast
    corridor, slabs of every historical block, query depth), timed on the
    GPU; computed once per chunk and shared by every layer of the model."""
    import numpy as np
    import torch

    import block_sparse_attention_gilbert_amd as bsa
    import workloads

    w, ra = st["w"], st["ra"]
    dev = ra.device
    g = workloads.geometry_inputs(st["cur"], w.nqb)
    d = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) if isinstance(v, np.ndarray) else v
         for k, v in g.items()}
    ov = torch.empty((w.nqb, w.nkb), dtype=torch.float32, device=dev)
    cov = torch.empty(w.nqb, dtype=torch.float32, device=dev)

    def overlap():
        bsa.slab_overlap(d["cams"], d["q_ptr"], d["q_cam"], d["q_geom"], d["h_ptr"], d["h_cam"], d["h_geom"], out=ov)

    def coverage():
        bsa.slab_coverage(d["cams"], ra.perm, g["grid"], d["frame_cam"], d["depth"], d["h_cam"], d["h_geom"],
                          block=w.bs, out=cov)

    times = {}
    for name, fn in (("overlap", overlap), ("coverage", coverage)):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        times[name] = e0.elapsed_time(e1) / reps
    nq = np.diff(g["q_ptr"])
    nh = np.diff(g["h_ptr"])
    ovh = ov.cpu().numpy()
    covh = cov.cpu().numpy()
    summary = {"overlap_ms": round(times["overlap"], 4), "coverage_ms": round(times["coverage"], 4),
               "query_slabs": int(nq.sum()), "historical_slabs": int(nh.sum()),
               "slab_pairs": int(nq.sum()) * int(nh.sum()), "positive_block_pairs": int((ovh > 0).sum()),
               "median_positive_overlap": round(float(np.median(ovh[ovh > 0])), 4) if (ovh > 0).any() else 0.0,
               "covered_query_blocks": int((covh >= 0.9).sum()), "grid_n": 8}
    return summary, ov, cov


def materialized(st, reps: int, overlap, coverage):
    """The step with the materialised route instead of the fixed top-K, at
    the same chunk: coverage-gated budgets (eta_cov 0.9, K_cov 80, K_unc
    150, mass 0.9), the previous chunk reserved, the chunk's local window
    rebuilt on the GPU, no reference blocks, with the overlap and coverage
    the slab geometry produced.  Times the whole step, the routing part
    (window + materialisation) and the attention launch."""
    import numpy as np
    import torch

    w, ra = st["w"], st["ra"]
    mat = dict(coverage=coverage, k_cov=80, k_unc=150, mass=0.9)

    def one(events=None):
        return ra.step(st["q_raster"], st["k_raster"], st["v_raster"], st["cur"], overlap=overlap,
                       materialize=mat, attn_events=events)

    for _ in range(30):  # the first call allocates its lists and workspace
        one()
    torch.cuda.synchronize()
    events = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        _, r = one(events)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / reps
    attn_ms = sum(a.elapsed_time(b) for a, b in events) / len(events)
    # the routing part alone (the pooled keys are cached, as in the step)
    e0.record()
    for _ in range(reps):
        ra.route_materialized(st["cur"], overlap=overlap, **mat)
    e1.record()
    torch.cuda.synchronize()
    route_ms = e0.elapsed_time(e1) / reps
    wc = work_counts(r["row_ptr"], r["col_idx"], w.q_len, w.k_len, w.heads, w.nqb, w.bs, w.d)
    lens = np.diff(r["row_ptr"].cpu().numpy())
    return {"ms_per_step": round(ms_step, 4), "route_ms": round(route_ms, 4), "attn_ms": round(attn_ms, 4),
            "step_effective_tflops": round(wc["flop"] / (ms_step * 1e-3) / 1e12, 2),
            "attn_effective_tflops": round(wc["flop"] / (attn_ms * 1e-3) / 1e12, 2),
            "attn_achieved_gbs": round(wc["alg_bytes"] / (attn_ms * 1e-3) / 1e9, 1),
            "list_len_mean": round(float(lens.mean()), 2), "list_len_min": int(lens.min()),
            "list_len_max": int(lens.max()),
            "covered_query_blocks": int((coverage.cpu().numpy() >= 0.9).sum()), "query_blocks": int(w.nqb),
            "params": "eta_cov 0.9, K_cov 80, K_unc 150, mass 0.9, window on, no reference blocks; overlap and "
                      "coverage from the slab geometry"}


def cpu_baseline(st, n_heads=2):
    """Time the float64 oracle (route + attention) on ``n_heads`` heads of the
    same workload; report effective TFLOP/s on that sample."""
    import numpy as np

    from oracle import attention as oatt
    from oracle import route as oroute
    from oracle.numerics import bf16_bits_to_f64
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    w = st["w"]
    flop = 0
    t_route = t_attn = 0.0
    t0 = time.perf_counter()
    for h in range(n_heads):
        q = bf16_bits_to_f64(w.q[h].contiguous().view(__import__("torch").int16).numpy())
        k = bf16_bits_to_f64(w.k[h].contiguous().view(__import__("torch").int16).numpy())
        v = bf16_bits_to_f64(w.v[h].contiguous().view(__import__("torch").int16).numpy())
        ta = time.perf_counter()
        r = oroute.route_head(q, k, w.q_len, w.k_len, w.bs, scale=w.scale, k_per_row=w.k_per_row[:w.nqb])
        tb = time.perf_counter()
        oatt.block_sparse_head(q, k, v, w.q_len, w.k_len, w.bs, r["lists"], w.scale)
        tc = time.perf_counter()
        t_route += tb - ta
        t_attn += tc - tb
        for i, lst in enumerate(r["lists"]):
            flop += 4 * w.d * int(w.q_len[i]) * int(np.asarray(w.k_len)[lst].sum())
    dt = time.perf_counter() - t0
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "float64 oracle route + attention for %d of %d heads at chunk %d (%.1f s, %.3g FLOP)"
                      % (n_heads, w.heads, w.nkb // 37, dt, flop),
            "route_s": round(t_route, 2), "attention_s": round(t_attn, 2)}


def read_traffic(per_launch_bytes):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attn_source_sha256_16") != attn_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


COPY_BYTES = 1 << 30  # calibration copy: 1 GiB read + 1 GiB written


def profile_attention(launches: int, expect_out=None, chunk: int = 48):
    """Counter-collection mode: set up C4 at chunk 48, route once (over the
    first ``chunk`` chunks of the store when ``chunk`` < 48: the chunk sweep's
    workload at that history length), then run ``launches`` block-sparse
    attention launches, two dense ones over the same history, and one plain
    1 GiB device copy (the calibration kernel for the byte counters).  Prints
    nothing but a summary line; meant to run under rocprofv3 --pmc."""
    import torch
    st = setup_c4(48, device="cuda:0")
    ra = st["ra"]
    run_step(st)
    torch.cuda.synchronize()
    if not 1 <= chunk <= ra.store_chunks:
        raise ValueError("chunk must be 1..%d" % ra.store_chunks)
    # attention only, on the routed lists of the step above (or of a route
    # over the first `chunk` chunks, with the same queries)
    nkb = chunk * ra.nbc
    r = ra.route_out if chunk == ra.store_chunks else ra.route(chunk - 1, qpool=ra.qbar)
    k_hist, v_hist = ra.k_store[:, : nkb * ra.block], ra.v_store[:, : nkb * ra.block]
    for _ in range(launches):       # as in the step: Q read and O written in raster order
        ra._attend(r, nkb, k_hist, v_hist, None, None, out_raster=True, q_raster=st["q_raster"])
    for _ in range(2):  # dense attention over the same history, for comparison counters
        ra.dense(chunk - 1)
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    if expect_out:
        # what the launches must issue: every listed block is block / 32
        # sub-tiles of 32 keys (a partly valid block is masked, not cut), each
        # 8 MFMAs for S and 8 for P V in every wave whose 32 query rows are not
        # all padding (the others skip the math); an unlisted block costs
        # nothing
        import numpy as np
        rp = r["row_ptr"].cpu().numpy().astype(np.int64)
        ql = ra.q_len.cpu().numpy().astype(np.int64)
        nqb = len(ql)
        waves_q = -(-np.clip(ql, 0, ra.block) // 32)          # active waves per query block
        listed = rp[1:] - rp[:-1]                              # per (head, query block) row
        active = np.tile(waves_q, len(listed) // nqb)
        subs = ra.block // 32
        with open(expect_out, "w") as f:
            json.dump({"listed_blocks": int(rp[-1]), "rows": int(len(rp) - 1), "subtiles_per_block": subs,
                       "active_wave_rows": int(active.sum()),
                       "mfma_sparse_listed": int((active * listed).sum()) * subs * 16,
                       "mfma_dense_listed": int(active.sum()) * nkb * subs * 16}, f, indent=1)
    print("profile-attention done: %d attention launches, one %d-byte copy" % (launches, COPY_BYTES), flush=True)


def profile_c5(launches: int):
    """Counter-collection mode for C5 at chunk 48: one step (it routes the
    chunk), a settle phase, then ``launches`` attention launches on its lists
    exactly as the step makes them (Q read and O written in raster order),
    then one plain 1 GiB device copy (the calibration kernel for the byte
    counters).
    Prints a one-line summary of the lists; meant to run under rocprofv3
    --pmc."""
    import torch

    ra, kpr, q_r, k_r, v_r, n_chunks = setup_c5("cuda:0")
    _, r = ra.step(q_r, k_r, v_r, n_chunks - 1, k_per_row=kpr)
    torch.cuda.synchronize()
    nkb = n_chunks * ra.nbc
    k_hist, v_hist = ra.k_store[:, : nkb * ra.block], ra.v_store[:, : nkb * ra.block]
    # settle: the same launches for SETTLE_MS of GPU time first (the clock
    # ramps after set-up), so the counted ones run at the steady clock
    settle_ms, settle_n = 0.0, 0
    while settle_ms < SETTLE_MS and settle_n < 2000:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            ra._attend(r, nkb, k_hist, v_hist, None, None, out_raster=True, q_raster=q_r)
        e1.record()
        torch.cuda.synchronize()
        settle_ms += e0.elapsed_time(e1)
        settle_n += 20
    for _ in range(launches):
        ra._attend(r, nkb, k_hist, v_hist, None, None, out_raster=True, q_raster=q_r)
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    rp = r["row_ptr"].cpu()
    lens = (rp[1:] - rp[:-1]).float()
    print("profile-c5 done: %d settle + %d attention launches on %d listed blocks (per row: mean %.1f, min %d, "
          "max %d), one %d-byte copy" % (settle_n, launches, int(rp[-1]), float(lens.mean()), int(lens.min()),
                                         int(lens.max()), COPY_BYTES), flush=True)


def summarize_launch_counters(csvs, kernel: str, launches: int, workload: str, out_path: str):
    """Per-launch counters of the last ``launches`` dispatches of ``kernel``
    (a substring of its name) in rocprofv3 --pmc CSVs, with the byte
    counters (FETCH_SIZE, WRITE_SIZE; KiB) scaled by what they read for the
    1 GiB copy, and the derived rates: matrix cores busy, vector issue busy,
    L2 hit rate, resident waves per SIMD.  Counters of the SQ block are
    per-SIMD aggregates (the VALU, wave and wait ones in units of 4 cycles);
    GRBM_GUI_ACTIVE is summed over the 8 XCDs."""
    import csv

    per = {}      # counter -> dispatch -> value (summed over the CSV's rows of that dispatch)
    copy = {}
    for path in csvs:
        with open(path) as f:
            for row in csv.DictReader(f):
                name, cn = row["Kernel_Name"], row["Counter_Name"]
                disp = int(row.get("Dispatch_Id") or row.get("Correlation_Id") or 0)
                v = float(row["Counter_Value"])
                if kernel in name:
                    per.setdefault(cn, {}).setdefault(disp, 0.0)
                    per[cn][disp] += v
                elif "copy" in name.lower():
                    copy.setdefault(cn, {}).setdefault(disp, 0.0)
                    copy[cn][disp] += v
    avg = {}
    for cn, d in per.items():
        last = sorted(d)[-launches:]
        avg[cn] = sum(d[k] for k in last) / len(last)
    out = {"kernel": kernel, "workload": workload, "attn_source_sha256_16": attn_source_hash(),
           "launches": launches, "counters_per_launch": avg}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        if cn in avg and cn in copy:
            scale = COPY_BYTES / (max(copy[cn].values()) * 1024.0)
            out[cn.lower() + "_bytes_per_launch"] = avg[cn] * 1024.0 * scale
            out[cn.lower() + "_copy_scale"] = scale
    cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
    simds = 1024
    if cyc:
        out["gpu_cycles"] = cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            out["mfma_busy"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cyc
        if "SQ_ACTIVE_INST_VALU" in avg:
            out["valu_issue_busy"] = 4.0 * avg["SQ_ACTIVE_INST_VALU"] / simds / cyc
        if "SQ_WAVE_CYCLES" in avg:     # quad-cycles, like the VALU counter
            out["waves_per_simd"] = 4.0 * avg["SQ_WAVE_CYCLES"] / simds / cyc
    if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
        out["l2_hit_rate"] = avg["TCC_HIT_sum"] / max(1.0, avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"])
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def coloured_visit_order(row_ptr, col_idx, heads: int, nqb: int):
    """Measurement experiment (host side, not part of the path): the same
    lists, each row visited in a co-scheduled order.  Per head, every
    selected block gets one slot (blocks with more selectors first, each
    the smallest slot free in all its selectors), and each row visits its
    blocks by slot, so the query blocks that share a block reach it at the
    same list position.  Returns the reordered col_idx (row_ptr unchanged)."""
    import numpy as np
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy().astype(np.int64)
    out = ci.copy()
    for h in range(heads):
        rows = [ci[rp[h * nqb + i]:rp[h * nqb + i + 1]] for i in range(nqb)]
        sel = {}
        for i, row in enumerate(rows):
            for b in row.tolist():
                sel.setdefault(b, []).append(i)
        used = [0] * nqb
        slot = {}
        for b in sorted(sel, key=lambda x: (-len(sel[x]), x)):
            busy = 0
            for i in sel[b]:
                busy |= used[i]
            sl = 0
            while busy >> sl & 1:
                sl += 1
            slot[b] = sl
            for i in sel[b]:
                used[i] |= 1 << sl
        for i, row in enumerate(rows):
            r0 = rp[h * nqb + i]
            out[r0:r0 + len(row)] = sorted(row.tolist(), key=lambda x: (slot[x], x))
    return torch_int32(out)


def torch_int32(a):
    import torch
    return torch.from_numpy(a.astype("int32"))


def visit_order_experiment(order: str, launches: int, timing: bool):
    """C4 at chunk 48: the step's lists visited in ascending order (as the
    router writes them) or in the co-scheduled order of
    ``coloured_visit_order``; ``launches`` attention launches (for counter
    runs), or with ``timing`` both orders timed in alternation (median of
    their launch times) and the largest output difference between them."""
    import statistics

    import torch
    st = setup_c4(48, device="cuda:0")
    ra = st["ra"]
    for _ in range(20):
        run_step(st)
    torch.cuda.synchronize()
    nkb = ra.store_chunks * ra.nbc
    r = ra.route_out
    k_hist, v_hist = ra.k_store[:, : nkb * ra.block], ra.v_store[:, : nkb * ra.block]
    n = int(r["row_ptr"][-1].item())
    cols = {"ascending": r["col_idx"][:n].clone(),
            "coloured": coloured_visit_order(r["row_ptr"], r["col_idx"][:n], ra.heads, ra.nbc).to("cuda:0")}

    def launch(name, out):
        from block_sparse_attention_gilbert_amd import block_sparse_attn
        block_sparse_attn(ra.q_blk, k_hist, v_hist, r["row_ptr"], cols[name], block=ra.block, scale=ra.scale,
                          q_block_len=ra.q_len, kv_block_len=ra.kv_len[:nkb], out=out, lse=ra.lse)

    if not timing:
        for _ in range(launches):
            launch(order, ra.o_blk)
        torch.cuda.synchronize()
        print("visit-order %s: %d launches" % (order, launches), flush=True)
        return
    outs = {k: torch.empty_like(ra.o_blk) for k in cols}
    times = {k: [] for k in cols}
    for _ in range(8):
        for k in cols:
            for _ in range(3):
                launch(k, outs[k])
            evs = []
            for _ in range(15):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                launch(k, outs[k])
                e1.record()
                evs.append((e0, e1))
            torch.cuda.synchronize()
            times[k] += [a.elapsed_time(b) for a, b in evs]
    diff = float((outs["coloured"].float() - outs["ascending"].float()).abs().max())
    print(json.dumps({k: round(statistics.median(v), 4) for k, v in times.items()} | {"max_abs_diff": diff}),
          flush=True)


def summarize_mfma(counter_csv: str, expect_json: str, out_path: str):
    """Per-launch matrix-core counters of the attention launches (sparse and
    dense) from one rocprofv3 --pmc CSV, against the MFMA count the lists
    imply: a skipped block must cost no matrix work."""
    import csv
    per = {}
    with open(counter_csv) as f:
        for row in csv.DictReader(f):
            name = row["Kernel_Name"]
            kind = "sparse" if "attn_bf16_kernel<128, 128, false>" in name else (
                "dense" if "attn_bf16_kernel<128, 128, true>" in name else None)
            if kind is None:
                continue
            key = (kind, row["Dispatch_Id"])
            per.setdefault(key, {}).setdefault(row["Counter_Name"], 0.0)
            per[key][row["Counter_Name"]] += float(row["Counter_Value"])
    exp = json.load(open(expect_json))
    out = {"kernel": "attn_bf16_kernel<128,128,*>", "workload": "C4 chunk 48", "expected": exp,
           "attn_source_sha256_16": attn_source_hash()}
    for kind in ("sparse", "dense"):
        ds = [v for (k, _), v in per.items() if k == kind]
        if not ds:
            continue
        avg = {c: sum(d.get(c, 0.0) for d in ds) / len(ds) for c in ds[0]}
        out[kind] = {"launches": len(ds), "per_launch": avg}
        if "SQ_INSTS_MFMA" in avg:
            want = exp["mfma_%s_listed" % kind]
            out[kind]["mfma_over_expected"] = avg["SQ_INSTS_MFMA"] / want
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg and avg["GRBM_GUI_ACTIVE"] > 0:
            # busy cycles summed over the 1024 SIMDs, against the launch's
            # GPU-busy cycles (summed over the 8 XCDs)
            out[kind]["mfma_busy_fraction"] = (avg["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024) / (avg["GRBM_GUI_ACTIVE"] / 8)
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def profile_step(steps: int):
    """Counter-collection mode for the whole step: set up C4 at chunk 48, run
    ``steps`` steps, then one plain 1 GiB device copy (the calibration kernel
    for the byte counters).  Meant to run under rocprofv3."""
    import torch
    st = setup_c4(48, device="cuda:0")
    for _ in range(steps):
        run_step(st)
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print("profiled %d steps" % steps)


def step_kernel_alg_bytes():
    """Algorithmic bytes of each kernel of the C4 chunk-48 step (L = 4680
    tokens, 40 heads, d 128, 37 query blocks, 1776 candidates, top-K 50):
    what the kernel must read and write at least once."""
    L, heads, d, nqb, n_cand, K = 4680, 40, 128, 37, 1776, 50
    raster = L * heads * d * 2
    blocked = nqb * 128 * heads * d * 2
    pooled = heads * nqb * d * 8
    keys = heads * nqb * n_cand * 8
    lists = 4 * (heads * nqb + 1 + heads * nqb * K)
    return {
        "gilbert_index_kernel": (2 * 4 * L, "perm and inverse written"),
        "gilbert_perm_pool_kernel": (raster + (blocked + 2 * pooled) // 2,
                                     "mean of Q (raster read, block means written) and K (raster read, "
                                     "blocked written, block means written)"),
        "gilbert_perm_kernel<false>": (raster + blocked, "raster read, blocked written"),
        "gilbert_perm_pool_batch_kernel": (3 * raster + 2 * blocked + 2 * pooled,
                                           "Q, K and V raster read; K and V blocked written; block means "
                                           "of Q and K written"),
        "score_kernel": (heads * n_cand * d * 8 + pooled + keys,
                         "pooled keys and queries read, selection keys written"),
        "topk_kernel": (keys + lists, "selection keys read, lists written"),
    }


def summarize_step_traffic(fetch_csv: str, write_csv: str, stats_csv: str, out_md: str):
    """Per kernel of the step: HBM bytes from the FETCH_SIZE and WRITE_SIZE
    counter runs (KiB per dispatch, each scaled by what it reads for the
    plain 1 GiB copy), the kernel's mean duration from the kernel-trace
    statistics of the same program, and the GB/s both give, beside the
    kernel's algorithmic bytes."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name", counter) == counter:
                    vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    dur = {}
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            dur[row["Name"]] = float(row["AverageNs"])
    cf = [v for k, vs in fetch.items() if "copy" in k for v in vs]
    cw = [v for k, vs in write.items() if "copy" in k for v in vs]
    f_factor = COPY_BYTES / (max(cf) * 1024.0)
    w_factor = COPY_BYTES / (max(cw) * 1024.0)

    def short(name):
        tag = "(anonymous namespace)::"
        n = name[name.index(tag) + len(tag):] if tag in name else name
        return n[:n.index("(")] if "(" in n else n

    alg = step_kernel_alg_bytes()
    lines = ["| kernel | dispatches | mean duration (us) | HBM read (MB) | HBM written (MB) | HBM GB/s | "
             "algorithmic MB | algorithmic GB/s | algorithmic bytes |", "|---|---|---|---|---|---|---|---|---|"]
    for name in sorted(fetch, key=lambda n: -dur.get(n, 0.0)):
        if "bsa::" not in name:
            continue
        sn = short(name)
        fb = sum(fetch[name]) / len(fetch[name]) * 1024.0 * f_factor
        wb = sum(write.get(name, [0.0])) / max(1, len(write.get(name, []))) * 1024.0 * w_factor
        us = dur.get(name, 0.0) / 1e3
        key = next((k for k in alg if sn.startswith(k)), None)
        a, what = alg[key] if key else (None, "")
        if sn.startswith("attn_bf16_kernel"):
            what = "3.03 GB per launch (distinct selected K/V blocks once, Q, O, lists)"
        elif sn.startswith("pool_kernel"):
            what = "first step only: the full pool of the history (the cache starts empty)"
        elif sn.startswith("gilbert_perm_kernel<true>"):
            what = "set-up only: the raster inputs made from the blocked workload"
        lines.append("| `%s` | %d | %.1f | %.1f | %.1f | %.0f | %s | %s | %s |" % (
            sn, len(fetch[name]), us, fb / 1e6, wb / 1e6, (fb + wb) / (us * 1e3) if us else 0.0,
            "%.1f" % (a / 1e6) if a else "-", "%.0f" % (a / (us * 1e3)) if a and us else "-", what))
    text = "\n".join(lines) + "\n\nCounter scale factors (copy kernel): fetch %.3f, write %.3f.\n" % (f_factor, w_factor)
    with open(out_md, "w") as f:
        f.write(text)
    print(text)


def summarize_counters(fetch_csv: str, write_csv: str, out_path: str):
    """Turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, then WRITE_SIZE; KiB
    per dispatch) into HBM bytes per attention launch, each counter scaled by
    what it reads for the plain copy kernel of known size."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name", counter) != counter:
                    continue
                name = row["Kernel_Name"]
                vals.setdefault(name, []).append(float(row["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")

    def pick(vals, key):
        ks = [k for k in vals if key in k]
        return [v for k in ks for v in vals[k]]

    attn_f = pick(fetch, "attn_bf16_kernel<128, 128, false>")
    attn_w = pick(write, "attn_bf16_kernel<128, 128, false>")
    copy_f = pick(fetch, "copy")
    copy_w = pick(write, "copy")
    f_factor = COPY_BYTES / (max(copy_f) * 1024.0)
    w_factor = COPY_BYTES / (max(copy_w) * 1024.0)
    fetch_b = sum(attn_f) / len(attn_f) * 1024.0 * f_factor
    write_b = sum(attn_w) / len(attn_w) * 1024.0 * w_factor
    out = {"kernel": "attn_bf16_kernel<128,128,sparse>", "workload": "C4 chunk 48",
           "attn_source_sha256_16": attn_source_hash(),
           "fetch_kib_per_launch": sum(attn_f) / len(attn_f), "write_kib_per_launch": sum(attn_w) / len(attn_w),
           "copy_bytes": COPY_BYTES, "copy_fetch_kib": max(copy_f), "copy_write_kib": max(copy_w),
           "fetch_scale": f_factor, "write_scale": w_factor,
           "hbm_bytes_per_launch": fetch_b + write_b, "fetch_bytes_per_launch": fetch_b,
           "write_bytes_per_launch": write_b}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def summarize_pipe(csvs, out_path: str, chunk: int = 48):
    """Per-launch averages of the pipeline counters of the attention launches
    (block-sparse and dense) from rocprofv3 --pmc CSVs of bench.py
    --profile-attention, with the derived rates: matrix cores busy, vector
    issue busy, LDS busy and bank-conflict share, L2 hit rate.  Counters of
    the SQ block are per-SIMD aggregates (the VALU and wait ones in units of
    4 cycles); GRBM_GUI_ACTIVE is summed over the 8 XCDs."""
    import csv

    vals = {}
    for path in csvs:
        with open(path) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"]
                kind = ("sparse" if "attn_bf16_kernel<128, 128, false>" in name else
                        "dense" if "attn_bf16_kernel<128, 128, true>" in name else None)
                if kind is None:
                    continue
                vals.setdefault(kind, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    simds, cus = 1024, 256
    out = {"kernel": "attn_bf16_kernel<128,128>", "workload": "C4 chunk %d" % chunk,
           "attn_source_sha256_16": attn_source_hash()}
    for kind, c in vals.items():
        avg = {k: sum(v) / len(v) for k, v in c.items()}
        d = {"counters_per_launch": avg}
        cyc = avg.get("GRBM_GUI_ACTIVE", 0.0) / 8.0     # per XCD: the launch's GPU cycles
        if cyc:
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                d["mfma_busy"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cyc
            if "SQ_ACTIVE_INST_VALU" in avg:
                d["valu_issue_busy"] = 4.0 * avg["SQ_ACTIVE_INST_VALU"] / simds / cyc
            if "SQ_LDS_IDX_ACTIVE" in avg:
                d["lds_busy"] = avg["SQ_LDS_IDX_ACTIVE"] / cus / cyc
        if avg.get("SQ_LDS_IDX_ACTIVE"):
            d["lds_bank_conflict_share"] = avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / avg["SQ_LDS_IDX_ACTIVE"]
        if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
            d["l2_hit_rate"] = avg["TCC_HIT_sum"] / max(1.0, avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"])
        out[kind] = d
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--chunk", type=int, default=48,
                    help="C4 history length in chunks (1..48); with --profile-attention and --summarize-pipe: "
                         "the 48-chunk store routed over its first C chunks (the chunk sweep's workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=40)
    ap.add_argument("--no-dense", action="store_true", help="skip timing dense attention at the same chunk")
    ap.add_argument("--no-c5", action="store_true", help="skip timing the C5 (ragged, structured) configuration")
    ap.add_argument("--no-c2", action="store_true", help="skip timing the C2 (Wan-1.3B-like layer) attention")
    ap.add_argument("--oracle-table", default=None, metavar="FILE",
                    help="write the float64 oracle's host times beside the GPU's, config by config, to this JSONL file")
    ap.add_argument("--tiles", action="store_true",
                    help="also time the step with fixed 1 x 8 x 16 tile blocks at the same chunk")
    ap.add_argument("--no-materialized", action="store_true",
                    help="skip timing the slab geometry and the step with the materialised route")
    ap.add_argument("--sweep", default=None, help="write a chunk 1..C sparse/dense sweep to this JSONL file")
    ap.add_argument("--rollout", default=None,
                    help="write a 1..C chunk rollout (append, route with the pooled-key cache, attend) "
                         "to this JSONL file")
    ap.add_argument("--profile-attention", type=int, default=0, metavar="N",
                    help="counter mode: N attention launches + a 1 GiB copy, no JSON line")
    ap.add_argument("--expect-out", default=None, metavar="JSON",
                    help="counter mode: write the MFMA counts the launches must issue to this file")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("COUNTER_CSV", "EXPECT_JSON", "OUT_JSON"),
                    help="compare the MFMA instruction counters of the attention launches with the listed tiles")
    ap.add_argument("--visit-order", default=None, choices=["ascending", "coloured", "ab"],
                    help="experiment: the attention launch on the step's lists in ascending or co-scheduled "
                         "visit order (N launches, --visit-order-launches), or both timed in alternation (ab)")
    ap.add_argument("--visit-order-launches", type=int, default=5)
    ap.add_argument("--profile-c5", type=int, default=0, metavar="N",
                    help="counter mode: C5 at chunk 48, one step, N attention launches + a 1 GiB copy, no JSON line")
    ap.add_argument("--summarize-launch-counters", nargs="+", metavar="ARG",
                    help="KERNEL LAUNCHES WORKLOAD CSV... OUT_JSON: per-launch counters of the last LAUNCHES "
                         "dispatches of KERNEL in rocprofv3 --pmc CSVs")
    ap.add_argument("--profile-step", type=int, default=0, metavar="N",
                    help="counter mode: N whole steps + a 1 GiB copy, no JSON line")
    ap.add_argument("--summarize-step-traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "STATS_CSV", "OUT_MD"),
                    help="per-kernel HBM bytes and GB/s of the step from counter and kernel-trace runs")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_JSON"),
                    help="write HBM bytes per attention launch from two rocprofv3 --pmc CSVs")
    ap.add_argument("--summarize-pipe", nargs="+", metavar="CSV",
                    help="pipeline counters of the attention launches (matrix, vector, LDS, L2) from rocprofv3 "
                         "--pmc CSVs of --profile-attention; the last argument is the output JSON")
    args = ap.parse_args()
    if args.summarize_launch_counters:
        a = args.summarize_launch_counters
        summarize_launch_counters(a[3:-1], a[0], int(a[1]), a[2], a[-1])
        return
    if args.summarize_pipe:
        summarize_pipe(args.summarize_pipe[:-1], args.summarize_pipe[-1], args.chunk)
        return
    if args.summarize_step_traffic:
        summarize_step_traffic(*args.summarize_step_traffic)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (see the sharding notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_gilbert_amd as bsa  # fails loudly if libbsa.so is missing

    if args.profile_step:
        profile_step(args.profile_step)
        return
    if args.profile_attention:
        profile_attention(args.profile_attention, args.expect_out, args.chunk)
        return
    if args.profile_c5:
        profile_c5(args.profile_c5)
        return
    if args.visit_order:
        visit_order_experiment(args.visit_order, args.visit_order_launches, args.visit_order == "ab")
        return

    dev = "cuda:0"
    clocks_start = clocks()
    t_setup = time.perf_counter()
    st = setup_c4(args.chunk, device=dev)
    w, ra = st["w"], st["ra"]
    print("setup %.1f s (generate + upload + raster inputs)" % (time.perf_counter() - t_setup), file=sys.stderr,
          flush=True)

    # correctness guard of the step: the slot rewritten by the forward
    # permutation must equal the generated store bits.  It runs before the
    # warm-up: the allocations around the check disturb the next few dozen
    # steps (they run ~10 % slower), so the warm-up also covers that.
    ks_before = ra.slot(st["cur"])[0].clone()
    for _ in range(2):
        run_step(st)
    torch.cuda.synchronize()
    assert torch.equal(ks_before, ra.slot(st["cur"])[0]), "forward permutation did not reproduce the store slot"
    del ks_before
    # settle: after set-up (uploads, allocations, host work) the GPU's clock
    # takes a few hundred milliseconds of steady load to come back up, which
    # a short warm-up would leave inside the timed region; a fixed settle
    # phase of steps runs first, so the steady state does not depend on
    # --warmup
    settle_ms, settle_steps = 0.0, 0
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    while settle_ms < SETTLE_MS and settle_steps < 5000:
        s0.record()
        for _ in range(50):
            run_step(st)
        s1.record()
        torch.cuda.synchronize()
        settle_ms += s0.elapsed_time(s1)
        settle_steps += 50
    for _ in range(args.warmup):
        run_step(st)
    torch.cuda.synchronize()

    events = []
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        _, r = run_step(st, attn_events=events)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps
    attn_all = sorted(a.elapsed_time(b) for a, b in events)
    attn_ms = sum(attn_all) / len(attn_all)

    # the same step with the pooled-key cache dropped before each call
    n_full = max(1, min(args.steps, 5))
    torch.cuda.synchronize()
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record()
    for _ in range(n_full):
        ra.invalidate_kpool()
        run_step(st)
    f1.record()
    torch.cuda.synchronize()
    ms_full_pool = f0.elapsed_time(f1) / n_full

    ms_graph = step_graph_ms(st, n_full)

    wc = work_counts(r["row_ptr"], r["col_idx"], w.q_len, w.k_len, w.heads, w.nqb, w.bs, w.d)
    value = wc["flop"] / (ms_step * 1e-3) / 1e12
    attn_tflops = wc["flop"] / (attn_ms * 1e-3) / 1e12
    achieved_gbs = wc["alg_bytes"] / (attn_ms * 1e-3) / 1e9
    traffic = read_traffic(wc["alg_bytes"])
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_full_k_pool_ms": round(ms_full_pool, 4),
        "step_hip_graph_ms": None if ms_graph is None else round(ms_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) + per-block offsets; no dataset, no weights)",
        "config": {"workload": "C4 growing-context 14B-like layer at chunk %d" % args.chunk,
                   "heads": w.heads, "head_dim": w.d, "block": w.bs, "query_tokens": 4680,
                   "kv_tokens": 4680 * args.chunk, "kv_blocks": w.nkb, "top_k": 50,
                   "step": "one launch permuting K and V into the store (K with its block means, Q block "
                           "means only) + route (cached history pools; score all 1776 candidates; top-K) + "
                           "block-sparse attention reading Q and writing O in raster order; the Gilbert index "
                           "is computed once per grid shape (timed alone in breakdown)",
                   "parallelism": "single GPU"},
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1)},
        "pct_bf16_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "attn": {"ms_per_call": round(attn_ms, 4),
                 "ms_median": round(attn_all[len(attn_all) // 2], 4),
                 "ms_p10": round(attn_all[len(attn_all) // 10], 4),
                 "ms_p90": round(attn_all[(9 * len(attn_all)) // 10], 4),
                 "effective_tflops": round(attn_tflops, 2),
                 "pct_bf16_mfma_peak": round(100.0 * attn_tflops / PEAK_BF16_TFLOPS, 2),
                 "tile_tflops": round(wc["tile_flop"] / (attn_ms * 1e-3) / 1e12, 2),
                 "effective_flop": wc["flop"], "listed_blocks": wc["pairs"],
                 "distinct_kv_rows": wc["uniq_rows"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": "attn_bf16_kernel<128,128,sparse>",
                     "alg_bytes_per_launch": wc["alg_bytes"]},
    }
    if not args.no_dense:
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        for _ in range(2):
            ra.dense(st["cur"])
        torch.cuda.synchronize()
        ev[0].record()
        n_dense = max(1, min(args.steps, 5))
        for _ in range(n_dense):
            ra.dense(st["cur"])
        ev[1].record()
        torch.cuda.synchronize()
        dms = ev[0].elapsed_time(ev[1]) / n_dense
        dflop = 4 * w.d * int(w.q_len.sum()) * int(w.k_len.sum()) * w.heads
        out["dense"] = {"ms_per_call": round(dms, 3), "effective_tflops": round(dflop / (dms * 1e-3) / 1e12, 2),
                        "speedup_sparse_vs_dense": round(dms / attn_ms, 2)}
    # stages alone and the attention with cold caches, then the matrix-rate
    # probe (after dense: the scrub buffer's allocation slows the next steps)
    out["breakdown"] = breakdown(st, max(5, min(args.steps, 20)))
    mp = mfma_probe()
    out["mfma_probe"] = dict(mp, attn_frac_of_probe=round(attn_tflops / mp["tflops"], 4),
                             dense_frac_of_probe=round(out["dense"]["effective_tflops"] / mp["tflops"], 4)
                             if "dense" in out else None)
    if not args.no_materialized:
        geo, ov, cov = geometry(st, max(1, min(args.steps, 10)))
        out["geometry"] = geo
        out["materialized"] = materialized(st, max(1, min(args.steps, 10)), ov, cov)
    if args.tiles:
        out["tiles"] = tiles(args.chunk, max(1, min(args.steps, 10)), dev)
    if not args.no_c5:
        out["c5"] = c5_config(max(1, min(args.steps, 10)), dev)
    if not args.no_c2:
        out["c2"] = c2_config(max(10, min(args.steps, 50)), dev)
    if args.sweep:
        sweep(st, args.sweep)
    if args.rollout:
        rollout(st, args.rollout)
    if args.oracle_table:
        oracle_table(st, args.oracle_table)
    out["clocks"] = {"start": clocks_start, "end": clocks()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(st, args.cpu_heads)
    print(json.dumps(out), flush=True)


def sweep(st, path):
    """History-length sweep (chunk 1..C) of the routed call (route + sparse
    attention) and of dense attention, on the resident store; the queries
    stay those of the last chunk.  All sparse timings come first (each chunk
    warmed, then timed back to back), then all dense ones, so the heat of
    the long dense launches does not lower the clock under the sparse ones."""
    import statistics

    import torch
    ra = st["ra"]
    sparse = {}
    for c in range(1, ra.store_chunks + 1):
        cur = c - 1
        for _ in range(10):
            ra.route_and_attend(cur)
        ev = []
        for _ in range(10):
            ra.route_and_attend(cur, attn_events=ev)
        torch.cuda.synchronize()
        sparse[c] = statistics.median(a.elapsed_time(b) for a, b in ev)
        print("sweep sparse chunk %d done" % c, file=sys.stderr, flush=True)
    with open(path, "w") as f:
        for c in range(1, ra.store_chunks + 1):
            cur = c - 1
            ra.dense(cur)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                ra.dense(cur)
            e1.record()
            torch.cuda.synchronize()
            f.write(json.dumps({"chunk": c, "sparse_attn_ms": round(sparse[c], 4),
                                "dense_attn_ms": round(e0.elapsed_time(e1) / 3, 4)}) + "\n")
            f.flush()
            print("sweep dense chunk %d done" % c, file=sys.stderr, flush=True)


def oracle_table(st, path):
    """The float64 oracle timed on the host beside the GPU path, config by
    config: C1, C2, C3 in full, C4 sparse at chunk 1, 2, 12, 24, 48 (two heads
    timed, scaled to 40) and dense at chunk 1, 2, 12 (one head, scaled); the
    GPU route + attention time of the same call beside each, and the ratio."""
    import statistics

    import numpy as np
    import torch

    import block_sparse_attention_gilbert_amd as bsa
    import workloads
    from oracle import attention as oatt
    from oracle import route as oroute
    from oracle.numerics import bf16_bits_to_f64

    def f64(t):
        t = t.contiguous()
        return bf16_bits_to_f64(t.view(torch.int16).numpy()) if t.dtype == torch.bfloat16 else \
            t.numpy().astype(np.float64)

    def gpu_ms(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def oracle_s(w, heads, kpr, overlap=None, dense=False, nkb=None):
        nkb = w.nkb if nkb is None else nkb
        rows_k = nkb * w.bs
        k_len = np.asarray(w.k_len)[:nkb]
        tr = ta = 0.0
        for h in heads:
            q, k, v = f64(w.q[h]), f64(w.k[h][:rows_k]), f64(w.v[h][:rows_k])
            t0 = time.perf_counter()
            if dense:
                oatt.dense_head(q, k, v, w.q_len, k_len, w.bs, w.scale)
                ta += time.perf_counter() - t0
                continue
            r = oroute.route_head(q, k, w.q_len, k_len, w.bs, scale=w.scale, k_per_row=kpr, overlap=overlap,
                                  lam=w.lam, tau=w.tau, g_ref=w.g_ref)
            t1 = time.perf_counter()
            oatt.block_sparse_head(q, k, v, w.q_len, k_len, w.bs, r["lists"], w.scale)
            tr += t1 - t0
            ta += time.perf_counter() - t1
        return tr, ta

    def gpu_call(w, dev_t, nkb, kf, overlap=None, dense=False):
        q, k, v, ql, kl = dev_t
        rows = nkb * w.bs
        kh, vh, klh = k[:, :rows], v[:, :rows], kl[:nkb]
        ov = None if overlap is None else torch.from_numpy(overlap).to(q.device)
        if dense:
            return lambda: bsa.dense_attn(q, kh, vh, block=w.bs, scale=w.scale, q_block_len=ql, kv_block_len=klh)
        out = {}

        def fn():
            r = bsa.route_topk(q, kh, block=w.bs, nqb=w.nqb, nkb=nkb, scale=w.scale, q_block_len=ql,
                               kv_block_len=klh, overlap=ov, lam=w.lam, g_ref=w.g_ref, tau=w.tau, k_fixed=kf,
                               out=out.get("r"), workspace=(out.get("r") or {}).get("workspace"))
            out["r"] = r
            bsa.block_sparse_attn(q, kh, vh, r["row_ptr"], r["col_idx"], block=w.bs, scale=w.scale,
                                  q_block_len=ql, kv_block_len=klh)
        return fn

    rows = []

    def add(config, w, heads_timed, nkb, kf, overlap=None, dense=False, reps=1, dev_t=None):
        dev = "cuda:0"
        if dev_t is None:
            dev_t = (w.q.to(dev), w.k.to(dev), w.v.to(dev),
                     torch.from_numpy(np.asarray(w.q_len, dtype=np.int32)).to(dev),
                     torch.from_numpy(np.asarray(w.k_len, dtype=np.int32)).to(dev))
        g = gpu_ms(gpu_call(w, dev_t, nkb, kf, overlap, dense))
        kpr = np.full(w.nqb, min(kf, nkb))
        ts = [oracle_s(w, heads_timed, kpr, overlap, dense, nkb) for _ in range(reps)]
        tr = statistics.median(t[0] for t in ts)
        ta = statistics.median(t[1] for t in ts)
        scale = w.heads / len(heads_timed)
        total = (tr + ta) * scale
        row = {"config": config, "kind": "dense" if dense else "route + block-sparse",
               "heads_timed": len(heads_timed), "heads": w.heads, "oracle_route_s": round(tr, 3),
               "oracle_attention_s": round(ta, 3), "oracle_total_s_all_heads": round(total, 3),
               "scaled_from_heads": scale != 1, "gpu_ms": round(g, 4), "oracle_over_gpu": round(total * 1e3 / g, 1)}
        rows.append(row)
        print("oracle table:", json.dumps(row), file=sys.stderr, flush=True)

    w1 = workloads.c1()
    add("C1 tiny fp32", w1, [0], w1.nkb, 4, reps=5)
    w2 = workloads.c2()
    add("C2 Wan-1.3B-like", w2, list(range(w2.heads)), w2.nkb, 50)
    w3 = workloads.c3()
    add("C3 geometric bias", w3, list(range(w3.heads)), w3.nkb, 50, overlap=w3.overlap)
    w4, ra = st["w"], st["ra"]
    resident = (ra.q_blk, ra.k_store, ra.v_store, ra.q_len, ra.kv_len)   # Q permuted in q_blk at set-up
    for c in (1, 2, 12, 24, 48):
        add("C4 chunk %d" % c, w4, [0, 39], 37 * c, 50, dev_t=resident)
    for c in (1, 2, 12):
        add("C4 chunk %d" % c, w4, [0], 37 * c, 50, dense=True, dev_t=resident)
    with open(path, "w") as f:
        for row in rows:
            f.write(json.dumps(row) + "\n")


def rollout(st, path, reps: int = 5):
    """A chunked rollout on a fresh KV store: for chunk c = 0..C-1 one call
    appends chunk c's K and V (Gilbert permutation into slot c), permutes the
    queries, routes over chunks 0..c (pooling only chunk c's keys; the
    history's pooled keys come from the cache) and attends.  Each chunk's
    call is timed ``reps`` times (each repeat rewrites slot c with the same
    bits), whole call and attention alone, with events on the stream."""
    import torch
    from block_sparse_attention_gilbert_amd import gilbert_perm
    from block_sparse_attention_gilbert_amd.pipeline import RoutedAttention
    w, src = st["w"], st["ra"]
    chunks = src.store_chunks
    ra = RoutedAttention(src.grid, w.heads, w.d, w.bs, chunks, device=src.device, k_cap=50)
    q_raster = st["q_raster"]
    with open(path, "w") as f:
        for c in range(chunks):
            ks, vs = src.slot(c)
            k_r = gilbert_perm(ks, src.perm, block=w.bs, inverse=True)
            v_r = gilbert_perm(vs, src.perm, block=w.bs, inverse=True)
            ra.step(q_raster, k_r, v_r, c)
            torch.cuda.synchronize()
            steps, attn = [], []
            for _ in range(reps):
                ev = []
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                ra.step(q_raster, k_r, v_r, c, attn_events=ev)
                e1.record()
                torch.cuda.synchronize()
                steps.append(e0.elapsed_time(e1))
                attn.append(ev[0][0].elapsed_time(ev[0][1]))
            assert torch.equal(ra.slot(c)[0], ks), "rollout store slot differs from the generated chunk"
            steps.sort()
            attn.sort()
            f.write(json.dumps({"chunk": c + 1, "kv_tokens": (c + 1) * 4680, "step_ms": round(steps[reps // 2], 4),
                                "attn_ms": round(attn[reps // 2], 4)}) + "\n")
            f.flush()
            print("rollout chunk %d done" % (c + 1), file=sys.stderr, flush=True)


if __name__ == "__main__":
    main()
