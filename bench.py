#!/usr/bin/env python3
"""Decode benchmark of the compressed sparse attention path on one MI355X.

Workload (default): batched CSA decode, 32 sequences at 131,072 raw tokens
(32,768 entries of m = 4), indexer 32 heads x 128 channels (FP4 keys), top-512,
64 query heads, window 128.  One step is one decode step of one layer for
the 32 sequences (one new query token each):
  csa_compress     the newest 4-token block of every sequence -> entry N-1
  csa_index_scores indexer scores of all 32,768 entries per sequence
  csa_topk         top-512 per sequence
  csa_sparse_attn  attention over the 512 entries + 128 window rows (bf16 out)
Layer caches are rotated over --layers copies so that consecutive steps
touch different memory (the working set of the rotation is far above the
256 MB Infinity Cache), as the layers of a model would.  The timed region
replays HIP graphs of these launches; inputs are resident in HBM.

Prints one JSON line (see the keys below); everything else goes to stderr.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

ROPE_BASE = 10000.0  # rotary base of the fused-epilogue leg (the original rotary embedding's)
HIDDEN_D_MODEL = 4096  # hidden size of the compress-from-hidden-states leg (a stand-in)
METRIC = "CSA decode query-tokens/s + achieved HBM GB/s at 128K ctx (1 MI355X)"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counter_sources_sha() -> str:
    """SHA-256 of the sources the dominant kernel is built from (the counter
    file holds the value it was measured with)."""
    h = hashlib.sha256()
    for f in ("index.hip", "csa_device.hpp"):
        with open(os.path.join(ROOT, "compressed_sparse_attention_compressor_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def step_bytes(w) -> dict:
    """Algorithmic (compulsory) HBM bytes of one decode step, per stage."""
    B, N, dI = w.B, w.N, w.d_idx
    key = dI // 2 + dI // 32
    entry = 256 + 16 + 128
    per_q = {
        "index": N * key + w.H_I * (dI + 4),
        "attn": w.k * entry + 2 * w.n_win * 576 + 2 * (2 * w.H * 576),
        "compress": w.m * 576 * 2 * 2 + entry + key,
    }
    shared = {"compress": w.m * 4 + 576 * dI * 2}
    out = {s: B * v + shared.get(s, 0) for s, v in per_q.items()}
    out["topk_io"] = B * (w.k * 4)
    out["step"] = out["index"] + out["attn"] + out["compress"]
    return out


class Layer:
    pass


def build_layers(w, L, dev, log_every=8):
    import torch

    import compressed_sparse_attention_compressor_amd as csa
    from synth.workloads import params, queries, raw_rows

    bias, wik = params(w, device=dev)
    cache0 = csa.Cache(w.B, w.N, w.m, w.d_idx, device=dev)
    chunk = 4096
    t_start = time.time()
    for i, t0 in enumerate(range(0, w.T, chunk)):
        x, z = raw_rows(w, t0, t0 + chunk, device=dev)
        csa.compress(cache0, x, z, bias, wik, tok_begin=t0)
        if t0 + chunk == w.T:
            x_last, z_last = x[:, -max(w.n_win, w.m):].contiguous(), z[:, -w.m:].contiguous()
        if i % log_every == 0:
            torch.cuda.synchronize()
            log(f"[bench] cache build: {t0 + chunk}/{w.T} tokens ({time.time() - t_start:.1f}s)")
    cache0.n_entries.fill_(w.N)
    torch.cuda.synchronize()
    layers = []
    for l in range(L):
        ly = Layer()
        if l == 0:
            ly.cache = cache0
        else:
            ly.cache = csa.Cache(w.B, w.N, w.m, w.d_idx, device=dev, planes=dict(
                nope=cache0.nope.clone(), nscale=cache0.nscale.clone(), rope=cache0.rope.clone(),
                ikey=cache0.ikey.clone(), iscale=cache0.iscale.clone(), n_entries=cache0.n_entries.clone()))
        wl = dataclasses.replace(w, cfg=w.cfg + 100 * l)
        qs = queries(wl, device=dev)
        ly.q, ly.qI, ly.w, ly.q_pos = qs["q"], qs["qI"], qs["w"], qs["q_pos"].to(dev)
        ly.x_blk = x_last[:, -w.m:].clone()
        ly.z_blk = z_last.clone()
        ly.swa = x_last[:, -w.n_win:].clone()
        ly.swa8 = csa.swa_encode(ly.swa)     # the same rows as FP8 window planes
        ly.swa_pos0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=dev)
        ly.idx = torch.empty(w.B, 1, w.k, dtype=torch.int32, device=dev)
        ly.out = torch.empty(w.B, 1, w.H, 576, dtype=torch.bfloat16, device=dev)
        ly.lse = torch.empty(w.B, 1, w.H, dtype=torch.float32, device=dev)
        layers.append(ly)
        torch.cuda.synchronize()
    log(f"[bench] {L} layer caches ready ({time.time() - t_start:.1f}s)")
    return layers, bias, wik


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--kernel-reps", type=int, default=64)
    ap.add_argument("--cpu-sample", type=int, default=32, help="sequences the oracle baseline runs (0 = skip)")
    ap.add_argument("--only-index", action="store_true", help="run only the fused append + indexer launches (for counter passes)")
    ap.add_argument("--only", choices=["index", "topk", "attn", "front"], default=None,
                    help="run only this stage of the decode step (for counter passes; the step's inputs are "
                         "prepared once by one eager step)")
    ap.add_argument("--prefill-reps", type=int, default=3, help="timed passes of the 64K prefill chunk (0 = skip)")
    ap.add_argument("--hca-steps", type=int, default=256, help="graph-timed HCA 1M decode steps (0 = skip)")
    ap.add_argument("--csa2-steps", type=int, default=64, help="graph-timed CSA2 two-layer 1M decode steps (0 = skip)")
    ap.add_argument("--hier-steps", type=int, default=64,
                    help="graph-timed two-layer 1M decode steps with the hierarchical pool (0 = skip)")
    ap.add_argument("--stack-steps", type=int, default=64,
                    help="graph-timed four-layer CSA2 stack steps at 1M context (0 = skip)")
    ap.add_argument("--replays", type=int, default=20, help="individually timed graph replays (>= 20)")
    ap.add_argument("--copy-calibration", action="store_true", help="run a plain device copy of known size")
    args = ap.parse_args()
    if args.only_index:
        args.only = "index"

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): sequences are independent, so "
              "N GPUs would each run this same single-GPU step on B/N sequences; no multi-GPU path is "
              "implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import compressed_sparse_attention_compressor_amd as csa
    from synth.workloads import BATCHED_DECODE as w

    dev = "cuda"
    torch.cuda.set_device(0)
    csa.lib()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {n} bytes read and written per copy")
        return

    L = args.layers
    layers, bias, wik = build_layers(w, L, dev)
    scores_ws = torch.empty(w.B, 1, w.N, dtype=torch.float32, device=dev)
    topk_ws_bytes = csa.workspace_bytes(csa.WS_TOPK, w.B, 1, w.k, w.N)
    topk_ws = torch.empty(max(topk_ws_bytes, 16), dtype=torch.uint8, device=dev)
    attn_ws_bytes = csa.workspace_bytes(csa.WS_SPARSE_ATTN, w.B, 1, w.H, w.k, w.n_win)
    attn_ws = torch.empty(max(attn_ws_bytes, 16), dtype=torch.uint8, device=dev)
    # the front half's workspace (scores, then the top-k count hint, which
    # every call leaves zero for the next)
    front_ws = torch.zeros(csa.workspace_bytes(csa.WS_INDEX_TOPK, w.B, 1, w.k, w.N, 0), dtype=torch.uint8, device=dev)

    def st_compress(ly):
        csa.compress(ly.cache, ly.x_blk, ly.z_blk, bias, wik, tok_begin=w.T - w.m)

    def st_index(ly):
        csa.index_scores(ly.cache, ly.qI, ly.w, ly.q_pos, scores=scores_ws)

    def st_append(ly):
        # the decode append and the indexer in one launch (identical results)
        csa.compress_index_scores(ly.cache, ly.x_blk, ly.z_blk, bias, wik, w.T - w.m, ly.qI, ly.w, ly.q_pos,
                                  scores=scores_ws)

    def st_topk(ly):
        csa.topk(ly.cache, scores_ws, ly.q_pos, w.k, out=ly.idx, ws=topk_ws if topk_ws_bytes else None)

    def st_front(ly):
        # decode append + indexer (one launch, counting the scores for the
        # top-k), then the hinted top-k (compaction, final selection)
        csa.compress_index_topk(ly.cache, ly.x_blk, ly.z_blk, bias, wik, w.T - w.m, ly.qI, ly.w, ly.q_pos, w.k,
                                ws=front_ws, out=ly.idx)

    def st_attn_w8(ly):
        csa.sparse_attn_w8(ly.cache, ly.q, ly.q_pos, ly.idx, ly.swa8, ly.swa_pos0, w.n_win, w.softmax_scale,
                           out_dtype=torch.bfloat16, ws=attn_ws, out=ly.out, lse=ly.lse)

    def st_attn(ly):
        csa.sparse_attn(ly.cache, ly.q, ly.q_pos, ly.idx, ly.swa, ly.swa_pos0, w.n_win, w.softmax_scale,
                        out_dtype=torch.bfloat16, ws=attn_ws, out=ly.out, lse=ly.lse)

    stages = [st_front, st_attn]
    if args.only:
        # one eager step per layer prepares the scores and selections the
        # stage reads
        for l in range(L):
            for f in [st_append, st_topk, st_attn]:
                f(layers[l])
        torch.cuda.synchronize()
        stages = [{"index": st_append, "topk": st_topk, "attn": st_attn, "front": st_front}[args.only]]

    def step(l):
        for f in stages:
            f(layers[l])

    # warmup (eager)
    for i in range(args.warmup):
        step(i % L)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    g_all = capture(lambda: [step(l) for l in range(L)])
    g_one = [capture(lambda l=l: step(l)) for l in range(L)]
    K = args.steps
    for _ in range(2):
        g_all.replay()
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(K // L):
        g_all.replay()
    for j in range(K % L):
        g_one[j].replay()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    gpu_ms = e0.elapsed_time(e1)
    ms = max(gpu_ms, 0.0) / K
    log(f"[bench] timed {K} steps: {gpu_ms:.3f} ms (GPU events), {wall_ms:.3f} ms wall")

    # Spread: each replay of the L-layer graph timed on its own (>= 20).
    per_replay = []
    for _ in range(max(20, args.replays)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g_all.replay()
        b.record()
        torch.cuda.synchronize()
        per_replay.append(a.elapsed_time(b) / L)
    per_replay.sort()
    spread = {"median": round(per_replay[len(per_replay) // 2], 6), "min": round(per_replay[0], 6),
              "max": round(per_replay[-1], 6), "replays": len(per_replay), "steps_per_replay": L}
    # Cache-warm: the same layer L times in a row (its 491 MB mostly served
    # from the Infinity Cache), reported apart from the rotating figure.
    g_warm = capture(lambda: [step(0) for _ in range(L)])
    g_warm.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(max(1, K // L)):
        g_warm.replay()
    b.record()
    torch.cuda.synchronize()
    warm_ms = a.elapsed_time(b) / (max(1, K // L) * L)
    del g_warm
    log(f"[bench] per-replay ms/step median {spread['median']:.4f} min {spread['min']:.4f}; "
        f"cache-warm (one layer) {warm_ms:.4f}")

    # Per-stage average launch durations: graphs of back-to-back launches of
    # one stage over the rotating layers, timed with events on the stream
    # the kernels run on.
    R = args.kernel_reps
    stage_us = {}
    names = {st_front: "compress+index_topk", st_append: "compress+index_scores", st_compress: "compress",
             st_index: "index_scores", st_topk: "topk_two_stage", st_attn: "sparse_attn"}
    timed = stages if args.only else [st_front, st_append, st_compress, st_index, st_topk, st_attn]
    for f in timed:
        g = capture(lambda f=f: [f(layers[i % L]) for i in range(R)])
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        stage_us[names[f]] = a.elapsed_time(b) * 1e3 / (reps * R)
    log(f"[bench] stage averages (us): {stage_us}")

    # The same step with the window rows as FP8 planes (the window KV format
    # the pages state), and that step with the fused rotary epilogue as well
    # (rotary base 10,000); reported beside the headline, which keeps bf16
    # rows and no rotation.
    def st_attn_w8_rope(ly):
        csa.sparse_attn_w8(ly.cache, ly.q, ly.q_pos, ly.idx, ly.swa8, ly.swa_pos0, w.n_win, w.softmax_scale,
                           out_dtype=torch.bfloat16, ws=attn_ws, out=ly.out, lse=ly.lse, rope_base=ROPE_BASE)

    def time_variant(st_a):
        g8 = capture(lambda: [(st_front(layers[l]), st_a(layers[l])) for l in range(L)])
        g8.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(max(1, K // L)):
            g8.replay()
        b.record()
        torch.cuda.synchronize()
        ms8 = a.elapsed_time(b) / (max(1, K // L) * L)
        del g8
        ga = capture(lambda: [st_a(layers[i % L]) for i in range(R)])
        ga.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(5):
            ga.replay()
        b.record()
        torch.cuda.synchronize()
        attn8_us = a.elapsed_time(b) * 1e3 / (5 * R)
        del ga
        return ms8, attn8_us

    w8 = w8r = None
    if not args.only:
        by8 = step_bytes(w)
        win16 = w.B * 2 * w.n_win * 576
        win8 = w.B * w.n_win * (512 + 16 + 128)
        step8 = by8["step"] - win16 + win8
        ms8, attn8_us = time_variant(st_attn_w8)
        w8 = {"window": "MXFP8 content channels + bf16 positional channels (656 B per row)",
              "ms_per_step": round(ms8, 6), "q_tokens_per_s": round(w.B / (ms8 * 1e-3), 1), "step_bytes": step8,
              "achieved_GBps": round(step8 / (ms8 * 1e-3) / 1e9, 1), "sparse_attn_us": round(attn8_us, 3)}
        log(f"[bench] FP8 window step {ms8 * 1e3:.2f} us, attention {attn8_us:.2f} us")
        msr, attnr_us = time_variant(st_attn_w8_rope)
        w8r = {"window": "MXFP8 window rows", "rope_base": ROPE_BASE,
               "epilogue": "q rotated by its position, entries at (j+1)m-1 and window rows at their positions "
                           "rotated in the decode, output rotated back by -p, then cast to bf16",
               "ms_per_step": round(msr, 6), "q_tokens_per_s": round(w.B / (msr * 1e-3), 1), "step_bytes": step8,
               "achieved_GBps": round(step8 / (msr * 1e-3) / 1e9, 1), "sparse_attn_us": round(attnr_us, 3)}
        log(f"[bench] FP8 window + rotary epilogue step {msr * 1e3:.2f} us, attention {attnr_us:.2f} us")

    by = step_bytes(w)
    # the dominant kernel: the fused append + indexer launch
    idx_us = stage_us.get("compress+index_scores", float("nan"))
    dom_bytes = by["index"] + by["compress"]
    achieved = dom_bytes / (idx_us * 1e-6) / 1e9
    traffic = None
    prof = os.path.join(ROOT, "profiles", "append_index_counters.json")
    if os.path.exists(prof):
        with open(prof) as fh:
            pc = json.load(fh)
        if pc.get("sources_sha256") == counter_sources_sha():
            traffic = pc.get("traffic_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(w.B / (ms * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "context": w.T, "m": w.m, "entries": w.N, "top_k": w.k,
                   "heads": w.H, "index_heads": w.H_I, "d_idx": w.d_idx, "n_win": w.n_win, "layers_rotated": L,
                   "stages": [names[f] for f in stages]},
        "achieved_GBps": round(by["step"] / (ms * 1e-3) / 1e9, 1),
        "step_bytes": by["step"],
        "stage_us": {k: round(v, 3) for k, v in stage_us.items()},
        "ms_per_step_spread": spread,
        "fp8_window": w8,
        "fp8_window_rope": w8r,
        "warm_one_layer": {"ms_per_step": round(warm_ms, 6), "q_tokens_per_s": round(w.B / (warm_ms * 1e-3), 1),
                           "note": "one layer's cache replayed L times in a row (warm); not the headline"},
        "roofline": {"bound": "hbm", "kernel": "append_index_kernel (decode append + indexer)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "bytes_per_launch": dom_bytes,
                     "avg_launch_us": round(idx_us, 3)},
    }
    if args.only:
        result["value"] = None

    if args.prefill_reps > 0 and not args.only:
        del layers, scores_ws, topk_ws, attn_ws
        torch.cuda.empty_cache()
        result["prefill"] = prefill_leg(args.prefill_reps, oracle=args.cpu_sample > 0)

    if args.hca_steps > 0 and not args.only:
        torch.cuda.empty_cache()
        result["hca"] = hca_leg(K=args.hca_steps)
    if args.csa2_steps > 0 and not args.only:
        torch.cuda.empty_cache()
        result["csa2"] = csa2_leg(K=args.csa2_steps)
    if args.hier_steps > 0 and not args.only:
        torch.cuda.empty_cache()
        result["csa2_hier"] = hier_leg(K=args.hier_steps)
    if args.stack_steps > 0 and not args.only:
        torch.cuda.empty_cache()
        result["csa2_stack"] = stack_leg(K=args.stack_steps)

    if args.cpu_sample > 0 and not args.only:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_sample)

    print(json.dumps(result), flush=True)


def prefill_flops(w) -> float:
    """Useful indexer multiply-adds (x2) of a causal prefill chunk: query t
    sees the entries completed by token t, min(N, (t+1) // m) of them."""
    import numpy as np

    t = np.arange(w.Q, dtype=np.int64)
    vis = np.minimum(w.N, (t + 1) // w.m)
    return float(vis.sum()) * w.H_I * w.d_idx * 2.0 * w.B


def prefill_leg(reps, oracle=True):
    """One 65,536-token causal prefill chunk of one layer: compress all 16,384
    entries, indexer scores (FP8 queries x FP4 keys on the scaled MFMA),
    top-1024 per query, sparse attention with the window.  Each stage is
    timed alone with HIP events on the stream it runs on (eager launches:
    every stage runs for milliseconds)."""
    import torch

    import compressed_sparse_attention_compressor_amd as csa
    from synth.workloads import PREFILL as w, hidden_inputs, params, queries, raw_rows

    dev = "cuda"
    t_start = time.time()
    bias, wik = params(w, device=dev)
    cache = csa.Cache(w.B, w.N, w.m, w.d_idx, device=dev)
    x, z = raw_rows(w, 0, w.T, device=dev)
    qs = queries(w, device=dev)
    q_pos = qs["q_pos"].to(dev)
    s0 = torch.zeros(w.B, dtype=torch.int32, device=dev)
    scores = torch.empty(w.B, w.Q, w.N, dtype=torch.float32, device=dev)
    tws_bytes = csa.workspace_bytes(csa.WS_TOPK, w.B, w.Q, w.k, w.N)
    tws = torch.empty(max(tws_bytes, 16), dtype=torch.uint8, device=dev)
    idx = torch.empty(w.B, w.Q, w.k, dtype=torch.int32, device=dev)
    out = torch.empty(w.B, w.Q, w.H, 576, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.Q, w.H, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] prefill inputs ready ({time.time() - t_start:.1f}s)")

    def st_compress():
        csa.compress(cache, x, z, bias, wik, tok_begin=0)
        cache.n_entries.fill_(w.N)

    def st_index():
        csa.index_scores(cache, qs["qI"], qs["w"], q_pos, scores=scores)

    def st_topk():
        csa.topk(cache, scores, q_pos, w.k, out=idx, ws=tws if tws_bytes else None)

    def st_attn():
        csa.sparse_attn(cache, qs["q"], q_pos, idx, x, s0, w.n_win, w.softmax_scale, out_dtype=torch.bfloat16,
                        out=out, lse=lse)

    stages = {"compress": st_compress, "index_scores": st_index, "topk": st_topk, "sparse_attn": st_attn}
    ms = {}
    for name, f in stages.items():
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        ms[name] = a.elapsed_time(b) / reps
        log(f"[bench] prefill {name}: {ms[name]:.3f} ms")
    total = sum(ms.values())
    flops = prefill_flops(w)
    tflops = flops / (ms["index_scores"] * 1e-3) / 1e12
    res = {"workload": w.name, "q_tokens": w.B * w.Q, "entries": w.N, "top_k": w.k, "index_heads": w.H_I,
            "d_idx": w.d_idx, "stage_ms": {k: round(v, 4) for k, v in ms.items()}, "ms": round(total, 4),
            "q_tokens_per_s": round(w.B * w.Q / (total * 1e-3), 1),
            "indexer_mfma": {"achieved": round(tflops, 2), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tflops / FP8_PEAK_TFLOPS, 4), "useful_flops": flops,
                             "note": "causal useful work only; E4M3 x E2M1 scaled MFMA issues at the FP8 rate"}}
    del scores, out, x, z
    torch.cuda.empty_cache()
    # The same chunk's compressor fed from hidden states (x = h W^KV and
    # z = h W^Z formed and pooled inside csa_compress_hidden), d_model a
    # stand-in: the pages give no hidden size.
    h, wkv, wz = hidden_inputs(w, HIDDEN_D_MODEL, device=dev)
    hws = torch.empty(max(16, csa.lib().csa_compress_hidden_ws_bytes(w.B, w.T, w.m, 1)), dtype=torch.uint8,
                      device=dev)
    csa.compress_hidden(cache, h, wkv, wz, bias, wik, ws=hws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        csa.compress_hidden(cache, h, wkv, wz, bias, wik, ws=hws)
    b.record()
    torch.cuda.synchronize()
    hms = a.elapsed_time(b) / reps
    hflops = 2.0 * w.B * w.T * HIDDEN_D_MODEL * (576 + 576)
    htf = hflops / (hms * 1e-3) / 1e12
    log(f"[bench] prefill compress from hidden states (d_model {HIDDEN_D_MODEL}): {hms:.3f} ms, {htf:.1f} TFLOP/s")
    res["compress_hidden"] = {"d_model": HIDDEN_D_MODEL, "G": 576, "ms": round(hms, 4),
                              "projection_flops": hflops,
                              "mfma": {"achieved": round(htf, 2), "peak": 2500.0, "unit": "TFLOP/s",
                                       "frac": round(htf / 2500.0, 4)},
                              "note": "x = h W^KV, z = h W^Z (bf16 MFMA, fp32 sums) pooled on chip; d_model is a "
                                      "stand-in, the pages give no hidden size"}
    del h, wkv, wz, hws, cache
    torch.cuda.empty_cache()
    if oracle:
        res["cpu_oracle"] = prefill_oracle(w)
    return res


def prefill_oracle(w, nq=8):
    """The float64 oracle on the same chunk: the whole compressor, then the
    index, top-k and attention of `nq` queries at evenly spread positions
    (the mean of their costs stands for the chunk's mean query, whose
    visible entries grow linearly with the position)."""
    import oracle as O
    from synth.workloads import as_u16, params, queries, raw_rows

    bias, wik = params(w)
    x, z = raw_rows(w, 0, w.T)
    xu = as_u16(x[0])
    t0 = time.perf_counter()
    c = O.compress(xu, as_u16(z[0]), bias.numpy(), as_u16(wik), w.m)
    t_comp = time.perf_counter() - t0
    del z
    t_q = 0.0
    for i in range(nq):
        p = int((i + 0.5) * w.Q / nq)
        qs = queries(w, q0=p, nq=1)
        t1 = time.perf_counter()
        idx, _, _, _ = O.index_topk(c["ikey"], c["iscale"], qs["qI"][0, 0].numpy(), qs["w"][0, 0].numpy(), p, w.m,
                                    w.N, w.k)
        O.sparse_attention(as_u16(qs["q"][0, 0]), c["nope"], c["nscale"], c["rope"], idx, xu, 0, p, w.n_win,
                           w.softmax_scale, w.m, w.N)
        t_q += time.perf_counter() - t1
    est = t_comp + t_q / nq * w.Q
    log(f"[bench] prefill oracle: compress {t_comp:.2f} s, {nq} queries {t_q:.2f} s, chunk estimate {est:.0f} s")
    return {"value": round(w.Q / est, 3), "unit": "query-tokens/s", "cores": _oracle_threads(), "kind": "oracle",
            "stage_s": {"compress_all": round(t_comp, 3), "per_query_mean": round(t_q / nq, 4)},
            "sample": f"compressor over all {w.T} tokens ({t_comp:.2f} s) + index/top-{w.k}/attention of {nq} "
                      f"queries at evenly spread positions ({t_q:.2f} s); chunk time estimated as compress + "
                      f"{w.Q} x the mean query"}


def _capture(fn):
    """A HIP graph of fn's launches (after one eager run on the capture stream)."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _graph_ms(fn, units, reps=5):
    """Milliseconds per unit of a graph of fn (which launches `units` units)."""
    import torch

    g = _capture(fn)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * units)


def _layer_caches(w, planes, L, dev):
    import torch

    import compressed_sparse_attention_compressor_amd as csa

    n_ent = torch.full((w.B,), w.N, dtype=torch.int32, device=dev)
    out = []
    for l in range(L):
        pl = {k: (v if l == 0 else v.clone()) for k, v in planes.items()}
        out.append(csa.Cache(w.B, w.N, w.m, w.d_idx, device=dev, planes=dict(
            nope=pl["nope"], nscale=pl["nscale"], rope=pl["rope"], ikey=pl.get("ikey"), iscale=pl.get("iscale"),
            n_entries=n_ent.clone())))
    return out


def _oracle_threads():
    try:
        import threadpoolctl
        return int(max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return 1


def _host_cpus() -> str:
    """The host the oracle ran on: affinity cores, os.cpu_count() and the
    BLAS thread count (the oracle runs its sequences one after another, so
    only the BLAS calls inside it use more than one core)."""
    return (f"host: {len(os.sched_getaffinity(0))} cores in the affinity mask, os.cpu_count() = {os.cpu_count()}, "
            f"BLAS threads = {_oracle_threads()}")


def hca_leg(L=16, K=256):
    """HCA dense decode: 8 sequences at 1,048,576 raw tokens (m = 128, 8,192
    entries), every head attending to every entry plus the window; one step
    = one decode query per sequence.  Layer caches rotate over L copies
    (16 x 26 MB).  The compressor runs once per 128 tokens and is timed on
    its own (one block per sequence).  The oracle times one sequence."""
    import dataclasses

    import torch

    import compressed_sparse_attention_compressor_amd as csa
    import oracle as O
    from synth.workloads import HCA_DECODE as w, as_u16, params, queries, raw_rows, synthetic_cache

    dev = "cuda"
    planes = synthetic_cache(w, device=dev)
    caches = _layer_caches(w, planes, L, dev)
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=dev)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=dev)
    qs = [queries(dataclasses.replace(w, cfg=w.cfg + 100 * l), device=dev) for l in range(L)]
    outs = [torch.empty(w.B, 1, w.H, 576, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    lses = [torch.empty(w.B, 1, w.H, dtype=torch.float32, device=dev) for _ in range(L)]
    wsb = csa.workspace_bytes(csa.WS_DENSE_ATTN, w.B, 1, w.H, w.N, w.n_win)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

    def steps():
        for i in range(K):
            l = i % L
            csa.hca_dense_attn(caches[l], qs[l]["q"], qs[l]["q_pos"], x_win, s0, w.n_win, w.softmax_scale,
                               out_dtype=torch.bfloat16, ws=ws, out=outs[l], lse=lses[l])

    ms = _graph_ms(steps, K)
    bias, _ = params(w, device=dev)
    xb, zb = raw_rows(w, w.T - w.m, w.T, device=dev)

    def blocks():
        for _ in range(16):
            csa.compress(caches[0], xb, zb, bias, None, tok_begin=w.T - w.m)

    comp_ms = _graph_ms(blocks, 16)
    per_q = w.N * 400 + 2 * w.n_win * 576 + 2 * 2 * w.H * 576
    step_bytes = w.B * per_q
    flops = w.B * 4.0 * w.H * 576 * (w.N + w.n_win)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    log(f"[bench] hca step {ms * 1e3:.2f} us, {gbps:.0f} GB/s, {tfs:.1f} TFLOP/s; compress block {comp_ms * 1e3:.2f} us")

    # oracle, one sequence of the same step
    pc = {k: v[0].cpu() for k, v in planes.items()}
    t0 = time.perf_counter()
    O.dense_attention(as_u16(qs[0]["q"][0, 0]), pc["nope"].numpy(), pc["nscale"].numpy(), as_u16(pc["rope"]),
                      as_u16(x_win[0]), w.T - w.n_win, w.T - 1, w.n_win, w.softmax_scale, w.m, w.N)
    dt = time.perf_counter() - t0
    return {"workload": w.name, "B": w.B, "context": w.T, "m": w.m, "entries": w.N, "heads": w.H, "n_win": w.n_win,
            "layers_rotated": L, "steps": K, "ms_per_step": round(ms, 6),
            "q_tokens_per_s": round(w.B / (ms * 1e-3), 1), "step_bytes": step_bytes,
            "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "step_flops": flops, "achieved_TFLOPs_bf16": round(tfs, 2), "mfma_frac_bf16": round(tfs / 2500.0, 4),
            "compress_block_us": round(comp_ms * 1e3, 3),
            "cpu_oracle": {"value": round(1.0 / dt, 3), "unit": "query-tokens/s", "cores": _oracle_threads(),
                           "sample": f"one sequence's decode query over {w.N} entries + {w.n_win} window rows: "
                                     f"{dt:.2f} s"}}


def csa2_leg(L=8, K=64):
    """CSA2 two-layer decode: 4 sequences at 1,048,576 raw tokens (262,144
    entries); layer A scores every entry and keeps its top-2,048 and attends
    to them; layer B rescores A's 2,048 with its own indexer queries, keeps
    512 and attends over A's cache with its own window.  One step = both
    layers for one query per sequence.  L rotating cache copies (8 x 491 MB).
    The oracle times layer A's indexer and both attentions for one sequence."""
    import dataclasses

    import torch

    import compressed_sparse_attention_compressor_amd as csa
    import oracle as O
    from synth.workloads import CSA2_DECODE as w, as_u16, queries, raw_rows, second_layer_window, synthetic_cache

    dev = "cuda"
    planes = synthetic_cache(w, device=dev)
    caches = _layer_caches(w, planes, L, dev)
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=dev)
    xb_win = second_layer_window(w, w.T - w.n_win, w.T, device=dev)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=dev)
    wl = [dataclasses.replace(w, cfg=w.cfg + 100 * l) for l in range(L)]
    qa = [queries(x, device=dev) for x in wl]
    qb = [queries(x, device=dev, second=True) for x in wl]
    ia = [torch.empty(w.B, 1, w.k, dtype=torch.int32, device=dev) for _ in range(L)]
    ib = [torch.empty(w.B, 1, w.k_b, dtype=torch.int32, device=dev) for _ in range(L)]
    oa = [torch.empty(w.B, 1, w.H, 576, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    ob = [torch.empty(w.B, 1, w.H, 576, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    la = [torch.empty(w.B, 1, w.H, dtype=torch.float32, device=dev) for _ in range(L)]
    lb = [torch.empty(w.B, 1, w.H, dtype=torch.float32, device=dev) for _ in range(L)]
    sc_a = torch.empty(w.B, 1, w.N, dtype=torch.float32, device=dev)
    sc_b = torch.empty(w.B, 1, w.k, dtype=torch.float32, device=dev)
    tws_b = csa.workspace_bytes(csa.WS_TOPK, w.B, 1, w.k, w.N)
    tws = torch.empty(max(tws_b, 16), dtype=torch.uint8, device=dev)
    # the fused scores + top-k call (its indexer launch also clears the radix
    # selection's histograms, one launch fewer than the two calls)
    itws = torch.zeros(max(csa.workspace_bytes(csa.WS_INDEX_TOPK, w.B, 1, w.k, w.N, 0), 16), dtype=torch.uint8,
                       device=dev)
    aws = torch.empty(max(csa.workspace_bytes(csa.WS_SPARSE_ATTN, w.B, 1, w.H, w.k, w.n_win), 16), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(max(csa.workspace_bytes(csa.WS_SPARSE_ATTN, w.B, 1, w.H, w.k_b, w.n_win), 16),
                      dtype=torch.uint8, device=dev)

    def layer_a(l):
        c = caches[l]
        csa.index_topk(c, qa[l]["qI"], qa[l]["w"], qa[l]["q_pos"], w.k, ws=itws, out=ia[l])
        csa.sparse_attn(c, qa[l]["q"], qa[l]["q_pos"], ia[l], x_win, s0, w.n_win, w.softmax_scale,
                        out_dtype=torch.bfloat16, ws=aws, out=oa[l], lse=la[l])

    def layer_b(l):
        c = caches[l]
        csa.index_scores(c, qb[l]["qI"], qb[l]["w"], qb[l]["q_pos"], cand=ia[l], scores=sc_b)
        csa.topk(c, sc_b, qb[l]["q_pos"], w.k_b, cand=ia[l], out=ib[l])
        csa.sparse_attn(c, qb[l]["q"], qb[l]["q_pos"], ib[l], xb_win, s0, w.n_win, w.softmax_scale,
                        out_dtype=torch.bfloat16, ws=bws, out=ob[l], lse=lb[l])

    ms = _graph_ms(lambda: [(layer_a(i % L), layer_b(i % L)) for i in range(K)], K)
    ms_a = _graph_ms(lambda: [layer_a(i % L) for i in range(K)], K)
    ms_b = ms - ms_a
    # stage by stage (each a graph of K launches over the rotating layers)
    stage_us = {
        "a_index_topk": _graph_ms(lambda: [csa.index_topk(caches[i % L], qa[i % L]["qI"], qa[i % L]["w"],
                                                          qa[i % L]["q_pos"], w.k, ws=itws, out=ia[i % L])
                                           for i in range(K)], K),
        "a_index_scores": _graph_ms(lambda: [csa.index_scores(caches[i % L], qa[i % L]["qI"], qa[i % L]["w"],
                                                              qa[i % L]["q_pos"], scores=sc_a) for i in range(K)], K),
        "a_topk": _graph_ms(lambda: [csa.topk(caches[i % L], sc_a, qa[i % L]["q_pos"], w.k, out=ia[i % L],
                                              ws=tws if tws_b else None) for i in range(K)], K),
        "a_sparse_attn": _graph_ms(lambda: [csa.sparse_attn(caches[i % L], qa[i % L]["q"], qa[i % L]["q_pos"], ia[i % L],
                                                            x_win, s0, w.n_win, w.softmax_scale, out_dtype=torch.bfloat16,
                                                            ws=aws, out=oa[i % L], lse=la[i % L]) for i in range(K)], K),
        "b_index_scores": _graph_ms(lambda: [csa.index_scores(caches[i % L], qb[i % L]["qI"], qb[i % L]["w"],
                                                              qb[i % L]["q_pos"], cand=ia[i % L], scores=sc_b)
                                             for i in range(K)], K),
        "b_topk": _graph_ms(lambda: [csa.topk(caches[i % L], sc_b, qb[i % L]["q_pos"], w.k_b, cand=ia[i % L],
                                              out=ib[i % L]) for i in range(K)], K),
        "b_sparse_attn": _graph_ms(lambda: [csa.sparse_attn(caches[i % L], qb[i % L]["q"], qb[i % L]["q_pos"], ib[i % L],
                                                            xb_win, s0, w.n_win, w.softmax_scale, out_dtype=torch.bfloat16,
                                                            ws=bws, out=ob[i % L], lse=lb[i % L]) for i in range(K)], K),
    }
    stage_us = {k: round(v * 1e3, 3) for k, v in stage_us.items()}
    log(f"[bench] csa2 stages (us): {stage_us}")
    per_a = w.N * 68 + w.H_I * (w.d_idx + 4) + w.k * 400 + 2 * w.n_win * 576 + 2 * 2 * w.H * 576
    per_b = w.k * 68 + w.H_I * (w.d_idx + 4) + w.k_b * 400 + 2 * w.n_win * 576 + 2 * 2 * w.H * 576
    step_bytes = w.B * (per_a + per_b)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] csa2 step {ms * 1e3:.2f} us (layer A {ms_a * 1e3:.2f}), {gbps:.0f} GB/s")

    pc = {k: v[0].cpu().numpy() if k != "rope" else as_u16(v[0]) for k, v in planes.items()}
    t0 = time.perf_counter()
    idx, _, _, _ = O.index_topk(pc["ikey"], pc["iscale"], qa[0]["qI"][0, 0].cpu().numpy(),
                                qa[0]["w"][0, 0].cpu().numpy(), w.T - 1, w.m, w.N, w.k)
    O.sparse_attention(as_u16(qa[0]["q"][0, 0]), pc["nope"], pc["nscale"], pc["rope"], idx, as_u16(x_win[0]),
                       w.T - w.n_win, w.T - 1, w.n_win, w.softmax_scale, w.m, w.N)
    dt = time.perf_counter() - t0
    return {"workload": w.name, "B": w.B, "context": w.T, "entries": w.N, "top_k_a": w.k, "top_k_b": w.k_b,
            "heads": w.H, "index_heads": w.H_I, "d_idx": w.d_idx, "n_win": w.n_win, "layers_rotated": L, "steps": K,
            "ms_per_step": round(ms, 6), "layer_a_ms": round(ms_a, 6), "layer_b_ms": round(ms_b, 6),
            "stage_us": stage_us,
            "q_tokens_per_s": round(w.B / (ms * 1e-3), 1), "step_bytes": step_bytes,
            "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "cpu_oracle": {"value": round(1.0 / dt, 3), "unit": "layer-A query-tokens/s", "cores": _oracle_threads(),
                           "sample": f"one sequence's layer-A step (scores of {w.N} entries, top-{w.k}, "
                                     f"attention): {dt:.2f} s"}}


def hier_leg(L=8, K=64):
    """CSA2 two-layer 1M decode with the hierarchical sparse indexer pool:
    4 sequences at 1,048,576 raw tokens (262,144 entries).  The Full layer
    scores every entry, keeps its own top-512, attends to it and builds the
    pool of its 2,048 best blocks of 8 entries (16,384 candidates); the
    Reindex layer rescores the pool, keeps 512 and attends over the shared
    cache with its own window.  One step = both layers for one query per
    sequence; L rotating cache copies (8 x 491 MB).  The oracle times both
    layers of one sequence."""
    import dataclasses

    import torch

    import compressed_sparse_attention_compressor_amd as csa
    import oracle as O
    from synth.workloads import (CSA2_HIER_DECODE as w, as_u16, queries, raw_rows, second_layer_window,
                                 synthetic_cache)

    dev = "cuda"
    C = w.pool_block * w.pool_blocks
    planes = synthetic_cache(w, device=dev)
    caches = _layer_caches(w, planes, L, dev)
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=dev)
    xb_win = second_layer_window(w, w.T - w.n_win, w.T, device=dev)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=dev)
    wl = [dataclasses.replace(w, cfg=w.cfg + 100 * l) for l in range(L)]
    qa = [queries(x, device=dev) for x in wl]
    qb = [queries(x, device=dev, second=True) for x in wl]

    def buf(*shape, dt=torch.int32):
        return [torch.empty(*shape, dtype=dt, device=dev) for _ in range(L)]

    ia, ib, pools = buf(w.B, 1, w.k), buf(w.B, 1, w.k_b), buf(w.B, 1, C)
    oa, ob = buf(w.B, 1, w.H, 576, dt=torch.bfloat16), buf(w.B, 1, w.H, 576, dt=torch.bfloat16)
    la, lb = buf(w.B, 1, w.H, dt=torch.float32), buf(w.B, 1, w.H, dt=torch.float32)
    sc_a = torch.empty(w.B, 1, w.N, dtype=torch.float32, device=dev)
    sc_b = torch.empty(w.B, 1, C, dtype=torch.float32, device=dev)
    tws_b = csa.workspace_bytes(csa.WS_TOPK, w.B, 1, w.k, w.N)
    tws = torch.empty(max(tws_b, 16), dtype=torch.uint8, device=dev)
    pws = torch.empty(max(csa.workspace_bytes(csa.WS_INDEX_POOL, w.B, 1, w.pool_blocks, w.N, w.pool_block), 16),
                      dtype=torch.uint8, device=dev)
    aws = torch.empty(max(csa.workspace_bytes(csa.WS_SPARSE_ATTN, w.B, 1, w.H, w.k, w.n_win), 16), dtype=torch.uint8,
                      device=dev)
    bws = torch.empty(max(csa.workspace_bytes(csa.WS_SPARSE_ATTN, w.B, 1, w.H, w.k_b, w.n_win), 16),
                      dtype=torch.uint8, device=dev)

    def a_index(l):
        csa.index_scores(caches[l], qa[l]["qI"], qa[l]["w"], qa[l]["q_pos"], scores=sc_a)

    def a_topk(l):
        csa.topk(caches[l], sc_a, qa[l]["q_pos"], w.k, out=ia[l], ws=tws if tws_b else None)

    def a_pool(l):
        csa.index_pool(caches[l], sc_a, qa[l]["q_pos"], w.pool_block, w.pool_blocks, out=pools[l], ws=pws)

    def a_attn(l):
        csa.sparse_attn(caches[l], qa[l]["q"], qa[l]["q_pos"], ia[l], x_win, s0, w.n_win, w.softmax_scale,
                        out_dtype=torch.bfloat16, ws=aws, out=oa[l], lse=la[l])

    def b_index(l):
        csa.index_scores(caches[l], qb[l]["qI"], qb[l]["w"], qb[l]["q_pos"], cand=pools[l], scores=sc_b)

    def b_topk(l):
        csa.topk(caches[l], sc_b, qb[l]["q_pos"], w.k_b, cand=pools[l], out=ib[l])

    def b_attn(l):
        csa.sparse_attn(caches[l], qb[l]["q"], qb[l]["q_pos"], ib[l], xb_win, s0, w.n_win, w.softmax_scale,
                        out_dtype=torch.bfloat16, ws=bws, out=ob[l], lse=lb[l])

    stages_a = [a_index, a_topk, a_pool, a_attn]
    stages_b = [b_index, b_topk, b_attn]
    ms = _graph_ms(lambda: [f(i % L) for i in range(K) for f in stages_a + stages_b], K)
    ms_a = _graph_ms(lambda: [f(i % L) for i in range(K) for f in stages_a], K)
    stage_us = {}
    for f in stages_a + stages_b:
        stage_us[f.__name__] = round(_graph_ms(lambda f=f: [f(i % L) for i in range(K)], K) * 1e3, 3)
    log(f"[bench] hier stages (us): {stage_us}")
    per_a = w.N * 68 + w.H_I * (w.d_idx + 4) + w.k * 400 + 2 * w.n_win * 576 + 2 * 2 * w.H * 576
    per_b = C * 68 + w.H_I * (w.d_idx + 4) + w.k_b * 400 + 2 * w.n_win * 576 + 2 * 2 * w.H * 576
    step_bytes = w.B * (per_a + per_b)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] hier step {ms * 1e3:.2f} us (Full layer {ms_a * 1e3:.2f}), {gbps:.0f} GB/s")

    pc = {k: v[0].cpu().numpy() if k != "rope" else as_u16(v[0]) for k, v in planes.items()}
    lay = [dict(qI=q["qI"][0, 0].cpu().numpy(), w=q["w"][0, 0].cpu().numpy(), q=as_u16(q["q"][0, 0]),
                swa=as_u16(win[0]), swa_pos0=w.T - w.n_win) for q, win in ((qa[0], x_win), (qb[0], xb_win))]
    t0 = time.perf_counter()
    O.hier_pair(pc, lay[0], lay[1], w.T - 1, w.m, w.N, w.n_win, w.softmax_scale, w.k, w.k_b, w.pool_block,
                w.pool_blocks)
    dt = time.perf_counter() - t0
    return {"workload": w.name, "B": w.B, "context": w.T, "entries": w.N, "top_k_full": w.k, "top_k_reindex": w.k_b,
            "pool": {"block": w.pool_block, "blocks": w.pool_blocks, "candidates": C}, "heads": w.H,
            "index_heads": w.H_I, "d_idx": w.d_idx, "n_win": w.n_win, "layers_rotated": L, "steps": K,
            "ms_per_step": round(ms, 6), "full_layer_ms": round(ms_a, 6), "reindex_layer_ms": round(ms - ms_a, 6),
            "stage_us": stage_us, "q_tokens_per_s": round(w.B / (ms * 1e-3), 1), "step_bytes": step_bytes,
            "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "cpu_oracle": {"value": round(1.0 / dt, 3), "unit": "two-layer query-tokens/s", "cores": _oracle_threads(),
                           "sample": f"one sequence's Full layer (scores of {w.N} entries, top-{w.k}, pool, "
                                     f"attention) and Reindex layer ({C} candidates): {dt:.2f} s"}}


def stack_leg(L=8, K=64):
    """A four-layer CSA2 stack at 1M context ([V4.1] Fig. 4 modes, Fig. 5
    pool) through csa2_layer_stack: Full (top-512 and a pool of 2,048 blocks
    x 8), Reuse, Reindex over the pool (top-512), Reuse.  4 sequences,
    262,144 entries; one step = the four layers for one query per sequence;
    L rotating caches.  The oracle times the stack for one sequence."""
    import dataclasses

    import torch

    import compressed_sparse_attention_compressor_amd as csa
    import oracle as O
    from synth.workloads import CSA2_HIER_DECODE as w, as_u16, queries, raw_rows, synthetic_cache

    dev = "cuda"
    C = w.pool_block * w.pool_blocks
    planes = synthetic_cache(w, device=dev)
    caches = _layer_caches(w, planes, L, dev)
    x_win, _ = raw_rows(w, w.T - w.n_win, w.T, device=dev)
    s0 = torch.full((w.B,), w.T - w.n_win, dtype=torch.int32, device=dev)
    modes = [csa.CSA2_FULL, csa.CSA2_REUSE, csa.CSA2_REINDEX, csa.CSA2_REUSE]
    names = ["full+pool", "reuse", "reindex(pool)", "reuse"]
    qs = [queries(dataclasses.replace(w, cfg=w.cfg + 100 * (i + 1)), device=dev) for i in range(len(modes))]
    pos = qs[0]["q_pos"]

    def layers_for(l, upto=None):
        out = []
        for i, md in enumerate(modes[:upto]):
            d = dict(mode=md, q=qs[i]["q"], swa=x_win, swa_pos0=s0, n_win=w.n_win, scale=w.softmax_scale,
                     out=bufs[l]["out"][i], lse=bufs[l]["lse"][i])
            if md != csa.CSA2_REUSE:
                d.update(qI=qs[i]["qI"], w=qs[i]["w"], k=w.k, idx_out=bufs[l]["idx"][i])
            if md == csa.CSA2_FULL:
                d.update(cache=caches[l], pool_block=w.pool_block, pool_blocks=w.pool_blocks, pool_out=bufs[l]["pool"])
            if md == csa.CSA2_REINDEX:
                d["cand"] = csa.CAND_POOL
            out.append(d)
        return out

    bufs = []
    for _ in range(L):
        bufs.append(dict(out=[torch.empty(w.B, 1, w.H, 576, dtype=torch.bfloat16, device=dev) for _ in modes],
                         lse=[torch.empty(w.B, 1, w.H, dtype=torch.float32, device=dev) for _ in modes],
                         idx=[torch.empty(w.B, 1, w.k, dtype=torch.int32, device=dev) for _ in modes],
                         pool=torch.empty(w.B, 1, C, dtype=torch.int32, device=dev)))
    stacks = [layers_for(l) for l in range(L)]
    fulls = [layers_for(l, 1) for l in range(L)]
    ws = torch.empty(1 << 28, dtype=torch.uint8, device=dev)
    ms = _graph_ms(lambda: [csa.layer_stack(stacks[i % L], pos, ws=ws) for i in range(K)], K)
    ms_full = _graph_ms(lambda: [csa.layer_stack(fulls[i % L], pos, ws=ws) for i in range(K)], K)
    per_q = 2 * w.n_win * 576 + 2 * 2 * w.H * 576
    by = {"full+pool": w.N * 68 + w.H_I * (w.d_idx + 4) + w.k * 400 + per_q, "reuse": w.k * 400 + per_q,
          "reindex(pool)": C * 68 + w.H_I * (w.d_idx + 4) + w.k * 400 + per_q}
    step_bytes = w.B * sum(by[n] for n in names)
    gbps = step_bytes / (ms * 1e-3) / 1e9
    log(f"[bench] stack step {ms * 1e3:.2f} us (Full layer {ms_full * 1e3:.2f}), {gbps:.0f} GB/s")

    pc = {k: v[0].cpu().numpy() if k != "rope" else as_u16(v[0]) for k, v in planes.items()}
    pc["n_entries"] = w.N
    ol = []
    for i, md in enumerate(modes):
        d = dict(mode=md, q=as_u16(qs[i]["q"][0, 0]), swa=as_u16(x_win[0]), swa_pos0=w.T - w.n_win,
                 scale=w.softmax_scale)
        if md != csa.CSA2_REUSE:
            d.update(qI=qs[i]["qI"][0, 0].cpu().numpy(), w=qs[i]["w"][0, 0].cpu().numpy(), k=w.k)
        if md == csa.CSA2_FULL:
            d.update(cache=pc, pool_block=w.pool_block, pool_blocks=w.pool_blocks)
        if md == csa.CSA2_REINDEX:
            d["cand"] = O.CAND_POOL
        ol.append(d)
    t0 = time.perf_counter()
    O.csa2_stack(ol, w.T - 1, w.m, w.n_win)
    dt = time.perf_counter() - t0
    return {"workload": "csa2-stack4-decode-b4-1m", "B": w.B, "context": w.T, "entries": w.N, "layers": names,
            "top_k": w.k, "pool": {"block": w.pool_block, "blocks": w.pool_blocks, "candidates": C}, "heads": w.H,
            "index_heads": w.H_I, "d_idx": w.d_idx, "n_win": w.n_win, "layers_rotated": L, "steps": K,
            "ms_per_step": round(ms, 6), "full_layer_ms": round(ms_full, 6),
            "q_tokens_per_s": round(w.B / (ms * 1e-3), 1), "step_bytes": step_bytes,
            "achieved_GBps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
            "cpu_oracle": {"value": round(1.0 / dt, 3), "unit": "four-layer query-tokens/s", "cores": _oracle_threads(),
                           "sample": f"one sequence's four-layer stack: {dt:.2f} s"}}


def cpu_baseline(w, nseq, min_seconds=10.0):
    """The float64 oracle on `nseq` sequences of the same decode step (host cores)."""
    import numpy as np

    import oracle as O
    from synth.workloads import as_u16, params, queries, raw_rows, synthetic_cache

    threads = _oracle_threads()
    bias, wik = params(w)
    qs = queries(w)
    planes = synthetic_cache(w, nseq=nseq)
    x, z = raw_rows(w, w.T - max(w.n_win, w.m), w.T, nseq=nseq)
    p = w.T - 1
    done, passes = 0, 0
    t0 = time.perf_counter()
    # whole passes over the sample until about min_seconds of CPU work
    while passes == 0 or time.perf_counter() - t0 < min_seconds:
        for b in range(nseq):
            O.compress(as_u16(x[b, -w.m:]), as_u16(z[b, -w.m:]), bias.numpy(), as_u16(wik), w.m)
            ik, isc = planes["ikey"][b].numpy(), planes["iscale"][b].numpy()
            idx, _, _, _ = O.index_topk(ik, isc, qs["qI"][b, 0].numpy(), qs["w"][b, 0].numpy(), p, w.m, w.N, w.k)
            O.sparse_attention(as_u16(qs["q"][b, 0]), planes["nope"][b].numpy(), planes["nscale"][b].numpy(),
                               as_u16(planes["rope"][b]), idx, as_u16(x[b, -w.n_win:]), w.T - w.n_win, p, w.n_win,
                               w.softmax_scale, w.m, w.N)
            done += 1
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(done / dt, 3), "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} passes over {nseq} of {w.B} sequences of one decode step (compress block, index "
                      f"{w.N} entries, top-{w.k}, attention): {done} query tokens in {dt:.2f} s; "
                      f"{_host_cpus()}"}


if __name__ == "__main__":
    main()
