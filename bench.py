"""Benchmark: one attention layer's chunked sparse prefill on one MI355X.

A step is the whole chunk loop over the prompt (per 32K chunk: keys rotated
into the KV cache at their DCA positions, V copied, vertical-slash pattern
estimated from the chunk's last 64 queries, sparse attention of the chunk),
inputs resident in HBM.  Default workload: the 7B-shaped layer (28 query /
4 KV heads, head_dim 128, bf16) at 1,048,576 tokens with DCA (C = 262,144,
W = 32,768), YaRN s = 4, budgets 1000 verticals + 6096 slashes.

Prints one JSON line (see the keys below).  --gpus above 1 is refused: the
benchmark runs on one GPU.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import long_context_sparse_rope_amd as L  # noqa: E402
import synth  # noqa: E402
from synth.configs import CONFIGS  # noqa: E402

METRIC = ("ms + effective TFLOP/s per 1M-token sparse prefill (one layer); "
          "% bf16 MFMA peak")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
CSRC = os.path.join(ROOT, "long_context_sparse_rope_amd", "csrc")
# sources of the kernels one vs_sparse_attn_prefill call launches, and the
# build script that holds their compiler flags
ATTN_SOURCES = ("attn.hip", "rope.hip", "lcsr_internal.h")


def attn_source_digest():
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(os.path.dirname(CSRC), "build.py"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(workload):
    """HBM bytes per attention call from the committed rocprofv3 counter
    summary, or None when it was taken on other sources or another workload
    (the counters cannot be read live)."""
    path = os.path.join(ROOT, "profiles", f"vs_sparse_attn_prefill_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    dig = re.search(r"attention source digest: `([0-9a-f]+)`", text)
    val = re.search(r"HBM bytes per call \(scaled\): ([0-9.eE+]+)", text)
    if not dig or not val or dig.group(1) != attn_source_digest():
        return None
    return float(val.group(1))


def make_layer(cfg, dev):
    rope = L.RopeConfig(base=cfg.rope_base, yarn_factor=cfg.yarn_factor,
                        orig_max_pos=cfg.yarn_orig_max_pos)
    dca = L.DcaConfig(cfg.dca_chunk, cfg.dca_local)
    sm = L.softmax_scale(cfg.head_dim, rope)
    return L.ChunkedSparsePrefill(cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.seq_len, rope,
                                  dca, sm, cfg.n_vert, cfg.n_slash, cfg.last_q, dev)


class StageTimer:
    """HIP events on the current stream around each stage of each chunk."""

    def __init__(self):
        self.marks = []

    def mark(self, name):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        self.marks.append((name, ev))

    def totals(self):
        out = {}
        for (name, a), (_, b) in zip(self.marks[:-1], self.marks[1:]):
            if name.startswith("end"):
                continue
            out.setdefault(name, []).append(a.elapsed_time(b))
        return out


def run_step(layer, cfg, q, k, v, out, stats, timer=None):
    for c in range(cfg.n_chunks):
        c0, lc = cfg.chunk_bounds(c)
        c1 = c0 + lc
        if timer:
            timer.mark("kv_append")
        layer.append_kv(k[:, c0:c1], v[:, c0:c1], c0)
        if timer:
            timer.mark("estimate")
        layer.estimate(q[:, c0:c1], c0)
        if timer:
            timer.mark("attention")
        layer.attend(q[:, c0:c1], c0, out=out[:, c0:c1], stats=stats)
        if timer:
            timer.mark("end")


def dense_baseline(cfg, layer, q, k, v, contexts):
    """Full causal attention (every key, same DCA logits) of one 32K chunk
    ending at each context length: the dense denominator of the sparse
    speedup.  The KV cache already holds the whole prompt (from the timed
    steps), so each point times one lcsr_vs_sparse_attn_prefill call with
    LCSR_ATTN_DENSE on the chunk's own rows."""
    out = {}
    for c1 in contexts:
        c1 = int(min(c1, cfg.seq_len)) // cfg.prefill_chunk * cfg.prefill_chunk
        c0 = c1 - cfg.prefill_chunk
        o = torch.empty((cfg.n_heads, cfg.prefill_chunk, cfg.head_dim), dtype=torch.bfloat16,
                        device=q.device)
        stats = torch.zeros(2, dtype=torch.int64, device=q.device)
        layer.attend(q[:, c0:c1], c0, out=o, dense=True)          # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        layer.attend(q[:, c0:c1], c0, out=o, stats=stats, dense=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        pairs = stats.cpu().tolist()[1]
        out[str(c1)] = {"ms": round(ms, 3), "pairs": pairs,
                        "tflops": round(4.0 * cfg.head_dim * pairs / (ms * 1e-3) / 1e12, 2)}
    return out


def a_shape_point(cfg, layer, q, n_sink=16, n_local=2048, reps=5):
    """The last chunk's attention with every head on the A-shape pattern
    (sink + recent window), in pattern buffers of its own: median call time
    with HIP events, exact pair count, algorithmic TFLOP/s."""
    c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
    c1 = c0 + lc
    pat = L.Pattern(cfg.n_heads, n_sink, n_local, q.device)
    L.pattern_fill_a_shape(pat, n_sink, n_local, c1)
    o = torch.empty((cfg.n_heads, lc, cfg.head_dim), dtype=torch.bfloat16, device=q.device)
    stats = torch.zeros(2, dtype=torch.int64, device=q.device)
    call = lambda st=None: L.vs_sparse_attn_prefill(  # noqa: E731
        q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0, layer.rope, layer.dca,
        layer.sm_scale, pat, out=o, stats=st)
    call(stats)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    pairs = stats.cpu().tolist()[1]
    return {"n_sink": n_sink, "n_local": n_local, "chunk": [c0, c1], "ms": round(ms, 3),
            "pairs": pairs,
            "tflops": round(4.0 * cfg.head_dim * pairs / (ms * 1e-3) / 1e12, 2)}


def block_sparse_point(cfg, layer, q, n_blocks=100, reps=5):
    """The last chunk with every head block-sparse (n_blocks kept 64-key
    blocks per 64-query block, 6,400 keys: about the vertical-slash
    budget): median times of the estimate (pooling, scores, selection) and
    of the attention, exact pair count, algorithmic TFLOP/s of the
    attention."""
    c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
    c1 = c0 + lc
    H = cfg.n_heads
    pat = L.BlockPattern(H, -(-lc // 64), n_blocks, q.device)
    o = torch.empty((H, lc, cfg.head_dim), dtype=torch.bfloat16, device=q.device)
    stats = torch.zeros(2, dtype=torch.int64, device=q.device)
    est = lambda: L.block_sparse_estimate(  # noqa: E731
        q[:, c0:c1], layer.k_cache[:, :c1], c0, layer.rope, layer.dca, layer.sm_scale,
        [n_blocks] * H, pat)
    att = lambda st=None: L.block_sparse_attn_prefill(  # noqa: E731
        q[:, c0:c1], layer.k_cache[:, :c1], layer.v_cache[:, :c1], c0, layer.rope, layer.dca,
        layer.sm_scale, pat, out=o, stats=st)
    est()
    att(stats)
    torch.cuda.synchronize()

    def timed(fn):
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    ms_e, ms_a = timed(est), timed(att)
    pairs = stats.cpu().tolist()[1]
    return {"n_blocks": n_blocks, "chunk": [c0, c1], "estimate_ms": round(ms_e, 3),
            "attention_ms": round(ms_a, 3), "pairs": pairs,
            "tflops": round(4.0 * cfg.head_dim * pairs / (ms_a * 1e-3) / 1e12, 2)}


def decode_points(cfg, layer, q, row_counts, reps=20):
    """Decode step over the full KV cache (left by the timed steps): the last
    n rows of the prompt against every key up to each, one lcsr_attn_decode
    call (the query rotations, the split-K kernel and the combine), median of
    `reps` calls timed with HIP events on the current stream.  The K and V
    caches are read once per call: 2 x H_kv x N x D two-byte elements."""
    res = {}
    n_ctx = cfg.seq_len
    kv_bytes = 2 * cfg.n_kv_heads * n_ctx * cfg.head_dim * 2
    for n in row_counts:
        p0 = n_ctx - n
        qs = q[:, p0:n_ctx]
        o = torch.empty((cfg.n_heads, n, cfg.head_dim), dtype=torch.float32, device=q.device)
        ws = torch.empty(L.workspace_bytes(L._capi.LCSR_WS_DECODE, qs, layer.k_cache, p0, layer.rope, layer.dca),
                         dtype=torch.uint8, device=q.device)
        call = lambda: L.attn_decode(qs, layer.k_cache, layer.v_cache, p0, layer.rope, layer.dca,
                                     layer.sm_scale, out=o, workspace=ws)
        call()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        gbs = kv_bytes / (ms * 1e-3) / 1e9
        res[str(n)] = {"ms": round(ms, 4), "kv_bytes": kv_bytes, "GB/s": round(gbs, 1),
                       "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    return res


def cpu_baseline(cfg, layer, q, k, v, budget_s=20.0, step_pairs=None):
    """Time the fp64 oracle on a bounded sample of the same workload: sparse
    attention rows of the last chunk (first query head, the GPU's own
    pattern), as many as fit in about `budget_s` seconds.  With the step's
    selected pair count, the time of the whole layer's sparse attention on
    the oracle is extrapolated from the measured seconds per pair (labelled
    as extrapolated; it is not run)."""
    import oracle
    from threadpoolctl import threadpool_info
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max(blas) if blas else 1
    c0, lc = cfg.chunk_bounds(cfg.n_chunks - 1)
    c1 = c0 + lc
    h, g = 0, 0
    verts, slashes = layer.pattern.lists()
    vh, sh = verts[h].numpy(), slashes[h].numpy()
    t_setup = time.perf_counter()
    K = k[g, :c1].float().cpu().numpy().astype(np.float64)
    V = v[g, :c1].float().cpu().numpy().astype(np.float64)
    th = oracle.rope_inv_freq(cfg.head_dim, cfg.rope_base)
    ctx = oracle.KeyContext(K, V, th, cfg.dca_chunk, cfg.dca_local)
    ctx.k_dca()
    setup_s = time.perf_counter() - t_setup
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(np.arange(c0, c1), size=min(16384, c1 - c0), replace=False))
    qh = q[h, rows].float().cpu().numpy().astype(np.float64)
    sm = layer.sm_scale
    done, pairs = 0, 0
    t0 = time.perf_counter()
    while done < rows.size and time.perf_counter() - t0 < budget_s:
        blk = slice(done, min(rows.size, done + 64))
        _, _, sizes = oracle.sparse_rows(qh[blk], rows[blk], ctx, vh, sh, sm)
        pairs += int(sizes.sum())
        done = blk.stop
    el = time.perf_counter() - t0
    flops = 4.0 * cfg.head_dim * pairs
    extra = {}
    if step_pairs:
        extra["extrapolated_layer_s"] = round(el / max(pairs, 1) * step_pairs, 1)
    return {**extra, "value": flops / el / 1e12, "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "host_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "sample": (f"fp64 sparse attention of {done} sampled rows of the last 32K chunk "
                       f"(query head 0, GPU pattern), {el:.1f} s after {setup_s:.1f} s of "
                       f"key rotation; {pairs} critical pairs"),
            "seconds": el, "rows": done}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="7b_1m_dca")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--dense-ctx", default="196608,589824,1048576",
                    help="context lengths of the dense one-chunk points ('' for none)")
    ap.add_argument("--no-a-shape", action="store_true",
                    help="skip the last-chunk A-shape (sink 16 + window 2048) point")
    ap.add_argument("--no-block-sparse", action="store_true",
                    help="skip the last-chunk block-sparse (100 blocks) point")
    ap.add_argument("--decode-rows", default="1,4",
                    help="rows per decode-step point over the full cache ('' for none)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU (one KV-head shard per GPU is the multi-GPU layout); --gpus must be 1"}))
        sys.exit(2)

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    q, k, v = synth.generate(cfg, dev)
    layer = make_layer(cfg, dev)
    out = torch.empty((cfg.n_heads, cfg.seq_len, cfg.head_dim), dtype=torch.bfloat16, device=dev)
    stats = torch.zeros(2, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        run_step(layer, cfg, q, k, v, out, stats)
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} done", file=sys.stderr, flush=True)
    stats.zero_()
    timer = StageTimer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(layer, cfg, q, k, v, out, stats, timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] {args.steps} timed steps in {wall:.3f} s", file=sys.stderr, flush=True)

    ms_step = wall * 1e3 / args.steps
    st = stats.cpu().tolist()
    sel_pairs = st[1] / args.steps
    exe_pairs = st[0] / args.steps
    alg_flops = 4.0 * cfg.head_dim * sel_pairs            # per step
    exe_flops = 4.0 * cfg.head_dim * exe_pairs
    totals = timer.totals()
    stages = {k_: sum(v_) / args.steps for k_, v_ in totals.items()}
    # attention ms of each chunk (mean over the timed steps): the cost grows
    # as the selected slashes spread over a longer context
    att = totals.get("attention", [])
    att_chunks = [round(sum(att[c::cfg.n_chunks]) / args.steps, 3) for c in range(cfg.n_chunks)] \
        if len(att) == cfg.n_chunks * args.steps else []
    attn_calls = cfg.n_chunks
    attn_ms_call = stages["attention"] / attn_calls
    achieved = alg_flops / attn_calls / (attn_ms_call * 1e-3) / 1e12
    exec_rate = exe_flops / attn_calls / (attn_ms_call * 1e-3) / 1e12
    eff = alg_flops / (ms_step * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "vs_sparse_attn_prefill (pattern aux + attention)",
                "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": counted_traffic(cfg.name), "traffic_unit": "bytes per call",
                "executed_tflops": round(exec_rate, 2),
                "executed_frac": round(exec_rate / PEAK_BF16_TFLOPS, 4),
                "avg_call_ms": round(attn_ms_call, 4)}
    rec = {
        "metric": METRIC, "value": round(eff, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16/fp16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "n_heads": cfg.n_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "seq_len": cfg.seq_len,
                   "prefill_chunk": cfg.prefill_chunk, "dca_chunk": cfg.dca_chunk,
                   "dca_local": cfg.dca_local, "yarn_factor": cfg.yarn_factor,
                   "n_vert": cfg.n_vert, "n_slash": cfg.n_slash, "out_dtype": "bf16",
                   "qk_operands": "fp16", "pv_operands": "bf16", "qk_noise": cfg.qk_noise},
        "stage_ms": {k_: round(v_, 3) for k_, v_ in stages.items()},
        "attention_ms_per_chunk": att_chunks,
        "algorithmic_tflop_per_step": round(alg_flops / 1e12, 3),
        "executed_tflop_per_step": round(exe_flops / 1e12, 3),
        "waste_ratio": round(exe_pairs / max(sel_pairs, 1), 3),
        "roofline": roofline,
        "attn_source_digest": attn_source_digest(),
    }
    if args.dense_ctx:
        print("[bench] dense one-chunk points", file=sys.stderr, flush=True)
        dense = dense_baseline(cfg, layer, q, k, v, [int(x) for x in args.dense_ctx.split(",")])
        # one-layer attention time, dense over sparse, of the chunk that ends
        # at each context (context for the pages' Figure 11, which compares
        # whole-model prefill, not one layer)
        for c1_s, pt in dense.items():
            ci = int(c1_s) // cfg.prefill_chunk - 1
            if att_chunks and 0 <= ci < len(att_chunks) and att_chunks[ci] > 0:
                pt["sparse_ms"] = att_chunks[ci]
                pt["dense_over_sparse"] = round(pt["ms"] / att_chunks[ci], 2)
        rec["dense_chunk"] = dense
    if not args.no_a_shape:
        print("[bench] a-shape chunk point", file=sys.stderr, flush=True)
        rec["a_shape_chunk"] = a_shape_point(cfg, layer, q)
    if not args.no_block_sparse:
        print("[bench] block-sparse chunk point", file=sys.stderr, flush=True)
        rec["block_sparse_chunk"] = block_sparse_point(cfg, layer, q)
    if args.decode_rows:
        print("[bench] decode-step points", file=sys.stderr, flush=True)
        rec["decode"] = decode_points(cfg, layer, q,
                                      [int(x) for x in args.decode_rows.split(",")])
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(cfg, layer, q, k, v, args.cpu_seconds, sel_pairs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
