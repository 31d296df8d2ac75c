#!/usr/bin/env python3
"""Benchmark of the semantic-ID beam-decode step on one MI355X.

A bench "step" is one full beam decode of the whole request batch: every
request is rewound to its root beam, then n_levels gr_beam_step calls run over
all requests (context attention, BeamKV gather + merge, codebook logits,
trie-masked log-softmax, top-K and BeamPath update per level), then
gr_beams_get returns every surviving beam of every request.  The ContextKV is
resident in HBM before the timed region (it stands in for prefill, which is
not part of the step).

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "beam-decode req/s + step µs at ctx 5000, beam 256; % MFMA peak, HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector

# HBM bytes per layer of the context-attention kernels on this workload, from rocprofv3
# --pmc FETCH_SIZE and WRITE_SIZE runs of this benchmark (one counter per run), scaled by what
# the same counters read for a 1 GiB device copy (FETCH_SIZE x 2.000, WRITE_SIZE x 1.000); one
# dispatch covers one layer in the headline's launch sequence;
# profiles/hbm_traffic_ctx5k_beam256_r8.md.  They belong to the kernel code they were taken on
# (source_digest of gr_kernels.hip: comments excluded); with any other code, or a variant not
# measured (the several-layers-per-launch variant), the traffic is reported as null.
MEASURED_TRAFFIC = {
    "workload": "ctx5k_beam256_r8",
    "source_sha256": "ac741b57f9f3e38438b441a907e6a5bf045b9564788febaecedcb087398301a7",
    "per_layer": {"k_ctx_attn_wide": {"read": 168466022, "written": 34079130},
                  "k_ctx_attn_wide_level0": {"read": 166437478, "written": 270336}},
}


# per-layer launch sequences: the timed region's context-attention events sit on every seventh
# layer's launch, four per level (each carrying dispatch costs the stream a few us: on one box
# 1,028 req/s with events on every layer, 1,052-1,058 on every fourth, 1,061-1,063 on the first
# only)
PROF_STRIDE = 7


def source_digest(path):
    """SHA-256 of a C/HIP source with its // comments and blank lines removed (a comment edit
    does not change the code the counters ran)."""
    import hashlib
    import re
    lines = []
    with open(path, encoding="utf-8") as f:
        for line in f:
            line = re.sub(r"\s*//.*$", "", line.rstrip("\n")).rstrip()
            if line:
                lines.append(line)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(cfg, kernel, variant):
    src = os.path.join(ROOT, "semantic_id_beam_amd", "csrc", "gr_kernels.hip")
    if cfg.name != MEASURED_TRAFFIC["workload"] or source_digest(src) != MEASURED_TRAFFIC["source_sha256"]:
        return None
    t = MEASURED_TRAFFIC.get(variant, {}).get(kernel)
    return None if t is None else t["read"] + t["written"]


def ctx_load_bytes(cfg, n):
    """HBM bytes of one copy load of an n-token context: the caller's K and V read, native K and
    V^T written (padded to a multiple of 64 tokens); for bf16 models with head_dim 128 also the
    native V^T read again and its float16 copy written."""
    el = 2 if cfg.dtype == "bf16" else 4
    np_ = (n + 63) // 64 * 64
    row = cfg.n_layers * cfg.n_kv_heads * cfg.head_dim
    b = 2 * row * el * (n + np_)
    if cfg.dtype == "bf16" and cfg.head_dim == 128:
        b += 2 * row * 2 * np_
    return b


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def workload_text(cfg, shapes):
    ns = sorted({n for n, _ in shapes})
    ws = sorted({w for _, w in shapes})
    return (f"{cfg.name}: {cfg.n_requests} requests x {cfg.n_layers} layers, ctx "
            f"{ns[0] if len(ns) == 1 else f'{ns[0]}..{ns[-1]}'}, beam {ws[0] if len(ws) == 1 else ws}, "
            f"{cfg.n_levels} levels x {cfg.codebook} codes, {cfg.n_items} items ({cfg.item_dist}), "
            f"{cfg.n_q_heads} q / {cfg.n_kv_heads} kv heads, head_dim {cfg.head_dim}, {cfg.dtype}")


def scoring_leg(cfg, args, per_layer=True):
    """Candidate scoring on the same contexts: 500 given items per request per call (the pages'
    scoring workload), items of the set drawn with repeats; every request of the workload in
    one call, calls timed end to end (each call synchronises): by the item log-likelihood
    (gr_score_items_batch), and by two label tokens read after each candidate
    (gr_score_items_labels: the same steps plus the label step)."""
    import numpy as np
    import torch

    import synth
    from semantic_id_beam_amd.workloads import make_engine, request_tensors
    n_cand, n_calls = 500, max(4, args.steps // 2)
    R = cfg.n_requests
    eng = make_engine(cfg, max_requests=R, max_beam_width=512, per_layer=per_layer, n_labels=2)
    for r in range(R):
        k, v, q = request_tensors(cfg, r)
        eng.load(r, k, v, q, synth.request_shapes(cfg)[r][1])
        del k, v, q
    items = synth.items(cfg)
    rng = np.random.default_rng(11)
    cands = np.stack([items[rng.integers(0, items.shape[0], size=n_cand)] for _ in range(R)]).astype(np.int32)
    rids = list(range(R))

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n_calls):
            out = fn()
        return time.perf_counter() - t0, out

    dt, sc = timed(lambda: eng.score_items_batch(rids, cands))
    dl, (_, lab) = timed(lambda: eng.score_items_labels(rids, cands))
    eng.close()
    log(f"scoring: {n_calls} calls of {R} x {n_cand} candidates in {dt:.3f} s; with labels {dl:.3f} s")
    assert np.all(np.isfinite(sc)) and np.all(np.isfinite(lab))
    # shared-context attention flops of one call (QK^T and PV, 4 d flops per query row and
    # context token): every candidate's query rows at levels 1..levels-1 (level 0 has one
    # beam), plus the label step's; the whole call's time (every kernel) against the bf16
    # matrix peak
    N = sum(n for n, _ in synth.request_shapes(cfg))
    per_level = 4.0 * cfg.n_layers * n_cand * cfg.n_q_heads * cfg.head_dim * N
    f_items = per_level * (cfg.n_levels - 1 + 1.0 / n_cand)
    f_labels = f_items + per_level

    def roof(flops, sec):
        ach = flops * n_calls / sec / 1e12
        return {"bound": "mfma", "achieved": round(ach, 2), "peak": 2500.0, "unit": "TFLOP/s",
                "frac": round(ach / 2500.0, 4), "scope": "whole call (every kernel), context-attention flops"}

    return {"requests_per_call": R, "candidates_per_request": n_cand, "calls": n_calls,
            "ms_per_call": round(1e3 * dt / n_calls, 3),
            "candidates_per_s": round(R * n_cand * n_calls / dt, 1), "roofline": roof(f_items, dt),
            "labels": {"n_labels": 2, "ms_per_call": round(1e3 * dl / n_calls, 3),
                       "candidates_per_s": round(R * n_cand * n_calls / dl, 1), "roofline": roof(f_labels, dl)}}


def prefill_leg(cfg, args, vocab: int = 32768, user_dim: int = 256, embed_dim: int = 2048, reps: int = 5):
    """Prefill (gr_ctx_prefill) of the workload's requests from context token ids: per-layer
    token tables of a 32,768-token vocabulary, a soft token at position 0 (a 256-float user
    vector through one linear layer to a 2048-float embedding, Qwen3-1.7B's hidden size, then
    projected to q/k/v per layer with float32 weights).  Each pass prefills every request into
    the engine's pool (HIP events around the pass on the stream it runs on), then releases
    them."""
    import numpy as np
    import torch

    import synth
    from semantic_id_beam_amd import _lib as G
    from semantic_id_beam_amd.workloads import make_engine
    R, L, Hq, Hkv, d = cfg.n_requests, cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    shapes = synth.request_shapes(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed * 1000 + 17)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    tabs = [torch.randn((L, vocab, h, d), generator=g, device="cuda", dtype=dt) for h in (Hq, Hkv, Hkv)]
    proj = torch.randn((user_dim, embed_dim), generator=g, device="cuda") * (1.0 / user_dim) ** 0.5
    ws = [torch.randn((L, embed_dim, h * d), generator=g, device="cuda") * (1.0 / embed_dim) ** 0.5
          for h in (Hq, Hkv, Hkv)]
    users = torch.randn((R, user_dim), generator=g, device="cuda")
    toks = [synth.prefill_tokens(cfg, r, vocab) for r in range(R)]
    eng = make_engine(cfg, max_requests=R)
    eng.set_prefill(*tabs, proj, *ws)
    res = {}
    for soft in (0, -1):
        ms = []
        for rep in range(reps + 1):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for r in range(R):
                eng.prefill(r, toks[r], shapes[r][1], soft_pos=soft, user_vec=users[r] if soft >= 0 else None)
            e1.record()
            torch.cuda.synchronize()
            if rep:
                ms.append(e0.elapsed_time(e1))
            for r in range(R):
                eng.release(r)
        res[soft] = float(np.median(ms)) / R
    eng.close()
    el = 2 if cfg.dtype == "bf16" else 4
    ctx_b = sum(L * Hkv * d * 2 * el * (n + G.gr_ctx_padded_len(n)) for n, _ in shapes) / R
    soft_b = 4 * (L * embed_dim * (Hq + 2 * Hkv) * d + user_dim * embed_dim)
    log(f"prefill: {res[0]:.3f} ms per request with the soft token, {res[-1]:.3f} without")
    return {"vocab": vocab, "user_dim": user_dim, "embed_dim": embed_dim, "soft_pos": 0,
            "ms_per_request": round(res[0], 3), "ms_per_request_no_soft": round(res[-1], 3),
            "algorithmic_MB_per_request": round((ctx_b + soft_b) / 1e6, 1),
            "context_MB_per_request": round(ctx_b / 1e6, 1), "soft_weights_MB": round(soft_b / 1e6, 1),
            "achieved_GBs": round((ctx_b + soft_b) / (res[0] * 1e-3) / 1e9, 1),
            "achieved_GBs_no_soft": round(ctx_b / (res[-1] * 1e-3) / 1e9, 1)}


def workload_leg(name: str, reps: int = 3, per_layer: bool = True):
    """Another workload of the decode step, its requests admitted as the workload prescribes
    (all at once, or in admission waves interleaved with the earlier waves' steps).  The first
    pass loads the contexts (loads timed apart with events); the timed passes replay the same
    schedule with the contexts resident, a wave's admission being the reset of its requests
    to the root beam.  Requests per second of decode wall time, every beam set fetched."""
    import numpy as np
    import torch

    import synth
    from semantic_id_beam_amd.workloads import make_engine, request_tensors
    cfg = synth.get_config(name)
    shapes = synth.request_shapes(cfg)
    R, lv = cfg.n_requests, cfg.n_levels
    waves = getattr(cfg, "waves", 0) or 1
    per = R // waves
    schedule = [list(range(w * per, (w + 1) * per)) for w in range(waves)]
    eng = make_engine(cfg, max_requests=R, per_layer=per_layer)
    load_ms = [0.0]
    batch_sizes = []

    def run(first):
        level, active = {}, []
        for k in range(waves + lv - 1):
            if k < waves:
                wave = schedule[k]
                if first:
                    tens = [request_tensors(cfg, r) for r in wave]
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for r, (kk, vv, qq) in zip(wave, tens):
                        eng.load(r, kk, vv, qq, shapes[r][1])
                    e1.record()
                    torch.cuda.synchronize()
                    load_ms[0] += e0.elapsed_time(e1)
                    del tens
                else:
                    eng.reset_batch(wave)
                for r in wave:
                    level[r] = 0
                active += wave
            step = [r for r in active if level[r] < lv]
            if first:
                batch_sizes.append(len(step))
            eng.step(step)
            fin = []
            for r in step:
                level[r] += 1
                if level[r] == lv:
                    fin.append(r)
            if fin:
                eng.beams_batch(fin)

    run(True)
    torch.cuda.empty_cache()
    run(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run(False)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    eng.close()
    load_bytes = sum(ctx_load_bytes(cfg, n) for n, _ in shapes)
    log(f"{name}: {reps} schedules in {dt:.3f} s")
    return {"workload": workload_text(cfg, shapes), "req_per_s": round(R * reps / dt, 1),
            "ms_per_schedule": round(1e3 * dt / reps, 3), "batched_steps": batch_sizes,
            "ctx_load_ms_per_request": round(load_ms[0] / R, 3),
            "ctx_load_GBs": round(load_bytes / (load_ms[0] * 1e-3) / 1e9, 1)}


def serving_leg(name: str = "ctx2k_beam30_r64", rates=(500, 1000, 2000, 3000, 4000, 5000, 6000),
                n_req: int = 1000, max_active: int = 64, seed: int = 0, per_layer: bool = True, graph: bool = False):
    """Latency against offered load through the continuous-batching scheduler (gr_sched_*):
    Poisson arrivals at each offered rate, n_req requests per rate, at most max_active decoding
    at once, the way the paper-daily TensorRT-LLM summary reads its beam-search chart
    ("Performance": where latency turns sharply upward; "Limitations": 1,000 requests per rate
    point, a concurrency cap of 64).  Each request is admitted when it arrives, decoded in the
    shared batched steps and timed until the host holds its beams.  Its context is already in
    the native layout, as a prefill would leave it (GR_LOAD_ADOPT: the load only takes the
    key-norm and value-scale bounds); the workload's 64 seeded contexts serve the requests
    round-robin."""
    import numpy as np
    import torch

    import semantic_id_beam_amd as sib
    import synth
    from semantic_id_beam_amd.workloads import make_engine, native_layout, request_tensors
    cfg = synth.get_config(name)
    shapes = synth.request_shapes(cfg)
    tens = []
    for r in range(cfg.n_requests):
        k, v, q = request_tensors(cfg, r)
        kn, vn, _ = native_layout(k, v)
        del k, v
        tens.append((kn, vn, q))
    eng = make_engine(cfg, max_requests=max_active + 2, max_ctx_tokens=0, per_layer=per_layer, graph=graph)
    torch.cuda.synchronize()
    points, base = [], 0
    for lam in rates:
        sched = sib.Scheduler(eng, max_active)
        arrival = np.cumsum(np.random.default_rng(seed + lam).exponential(1.0 / lam, n_req))
        done = np.full(n_req, np.nan)
        sizes = []
        i = n_done = 0
        t0 = time.perf_counter()
        while n_done < n_req:
            now = time.perf_counter() - t0
            while i < n_req and arrival[i] <= now:
                r = i % cfg.n_requests
                sched.submit(base + i, *tens[r], shapes[r][1], ctx_len=shapes[r][0], adopt=True)
                i += 1
            c = sched.counts()
            if c["queued"] + c["active"] == 0 and i - n_done - c["done"] == 0:
                continue                                   # idle until the next arrival
            sizes.append(c["active"] + min(c["queued"], max_active - c["active"]))
            sched.advance()
            for rid in sched.completed():
                sched.result(int(rid))
                done[int(rid) - base] = time.perf_counter() - t0
                n_done += 1
        sched.close()
        lat = (done - arrival) * 1e3
        span = float(np.max(done) - arrival[0])
        points.append({"offered_rps": lam, "achieved_rps": round(n_req / span, 1),
                       "p50_ms": round(float(np.percentile(lat, 50)), 2),
                       "p90_ms": round(float(np.percentile(lat, 90)), 2),
                       "p99_ms": round(float(np.percentile(lat, 99)), 2),
                       "mean_batch": round(float(np.mean(sizes)), 1)})
        log(f"serving {lam} req/s offered: {points[-1]}")
        base += n_req
    eng.close()
    del tens
    torch.cuda.empty_cache()
    return {"workload": workload_text(cfg, shapes[:1] * 1).replace(f"{cfg.n_requests} requests", "requests"),
            "requests_per_rate": n_req, "max_active": max_active, "contexts": cfg.n_requests,
            "points": points}


def chain_leg(args, name: str = "chain_ctx5k_beam256_r8", reps: int = 5):
    """The decode with a real layer chain (28 Qwen3-1.7B-shaped pre-norm decoder layers: q/k/v/o
    projections, RMSNorm, SwiGLU MLP of 6144) on the headline's requests: one launch per kernel
    and layer.  HIP events carried by the dispatches time every kernel; the projections'
    algorithmic work is 2 x live beams x (weights per layer) flops."""
    import numpy as np
    import torch

    import synth
    from semantic_id_beam_amd import _lib as G
    from semantic_id_beam_amd.workloads import make_engine, request_tensors
    cfg = synth.get_config(name)
    shapes = synth.request_shapes(cfg)
    R, lv, L = cfg.n_requests, cfg.n_levels, cfg.n_layers
    t = time.time()
    eng = make_engine(cfg, max_requests=R)
    log(f"chain engine ready ({time.time() - t:.1f} s)")
    for r in range(R):
        k, v, x = request_tensors(cfg, r)
        eng.load(r, k, v, x, shapes[r][1])
        del k, v, x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    rids = list(range(R))
    n_live = np.zeros((R, lv), dtype=np.int64)
    n_live[:, 0] = 1
    for s_ in range(lv):
        eng.step(rids)
        if s_ + 1 < lv:
            for r in rids:
                n_live[r, s_ + 1] = eng.state(r)["n"]
    eng.beams_batch(rids)

    def decode_all():
        eng.reset_batch(rids)
        for _ in range(lv):
            eng.step(rids)
        return eng.beams_batch(rids)

    decode_all()
    torch.cuda.synchronize()
    G.gr_engine_profile_reset(eng.eng)
    G.gr_engine_set_profiling(eng.eng, True)
    t0 = time.perf_counter()
    for _ in range(reps):
        decode_all()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    G.gr_engine_set_profiling(eng.eng, False)
    prof = {k: {s_: G.gr_engine_profile_read(eng.eng, kind, s_) for s_ in range(lv)}
            for kind, k in [(G.GR_PROF_GEMM, "gemm"), (G.GR_PROF_CTX_ATTN, "attn"), (G.GR_PROF_BEAM_MERGE, "finish"),
                            (G.GR_PROF_NORM, "norm"), (G.GR_PROF_LOGITS, "logits"), (G.GR_PROF_TOPK, "topk")]}
    eng.close()
    del eng
    torch.cuda.empty_cache()
    D, I = cfg.n_q_heads * cfg.head_dim, cfg.intermediate
    Dkv = cfg.n_kv_heads * cfg.head_dim
    w_layer = D * (D + 2 * Dkv) + D * D + 2 * D * I + I * D       # weights per layer
    N = np.array([n for n, _ in shapes], dtype=np.float64)
    out = {"workload": workload_text(cfg, shapes) + f", layer chain (MLP {I})", "reps": reps,
           "req_per_s": round(R * reps / dt, 1), "ms_per_decode": round(1e3 * dt / reps, 3), "levels": {}}
    for s_ in range(lv):
        rows = float(n_live[:, s_].sum())
        g_ms, g_n = prof["gemm"][s_]
        a_ms, a_n = prof["attn"][s_]
        gemm_flops = 2 * rows * w_layer * L * reps
        attn_flops = float(np.sum(cfg.n_kv_heads * n_live[:, s_] * cfg.group * N * cfg.head_dim * 4)) * L * reps
        out["levels"][f"level{s_}"] = {
            "rows": int(rows),
            "gemm_ms": round(g_ms / reps, 3), "gemm_TFLOPs": round(gemm_flops / (g_ms * 1e-3) / 1e12, 1),
            "gemm_frac_bf16_peak": round(gemm_flops / (g_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "gemm_weight_GBs": round(2 * w_layer * L * reps / (g_ms * 1e-3) / 1e9, 1),
            "attn_ms": round(a_ms / reps, 3), "attn_us_per_layer": round(1e3 * a_ms / max(a_n, 1), 2),
            "attn_TFLOPs": round(attn_flops / (a_ms * 1e-3) / 1e12, 1),
            "finish_ms": round(prof["finish"][s_][0] / reps, 3), "norm_ms": round(prof["norm"][s_][0] / reps, 3),
            "logits_topk_ms": round((prof["logits"][s_][0] + prof["topk"][s_][0]) / reps, 3)}
    out["library_reference"] = gemm_library_reference(int(n_live[:, -1].sum()), D, Dkv, I)
    log(f"chain: {out['req_per_s']} req/s, {out['ms_per_decode']} ms per decode")
    return out


def gemm_library_reference(rows, D, Dkv, I, reps: int = 50):
    """Context for the chain's projections, not part of the path: torch.matmul (hipBLASLt) on the
    same bf16 shapes (rows x out x in), each timed back to back with warm caches."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    out = {"note": "torch.matmul (hipBLASLt) on the projection shapes, back to back; context only"}
    for name, n, k in (("qkv", D + 2 * Dkv, D), ("o", D, D), ("gate_up", 2 * I, D), ("down", D, I)):
        a = torch.randn(rows, k, device="cuda", dtype=torch.bfloat16, generator=g)
        w = torch.randn(n, k, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(5):
            c = a @ w.t()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            c = a @ w.t()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tf = 2.0 * rows * n * k / (us * 1e-6) / 1e12
        out[name] = {"shape": [rows, n, k], "us": round(us, 2), "TFLOPs": round(tf, 1),
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del a, w, c
    torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, n_beams: int):
    """The oracle, timed on the host cores on a bounded sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from oracle.inputs import model_for, prefixes_for, request_for

    model, ps = model_for(cfg), prefixes_for(cfg)
    req = request_for(cfg, 0)
    for l in range(cfg.n_layers):          # regenerate + decode the context before timing
        req.ctx(l)
    root = ps.valid_codes(())
    beams = [((int(c),), 0.0) for c in root[:n_beams]]
    t0 = time.perf_counter()
    oracle.step_candidates(req, model, ps, beams, "valid")
    dt = time.perf_counter() - t0
    per_beam = dt / len(beams)
    # beam evaluations of one full decode of one request: 1 at level 0, then n_s per level
    W = cfg.beam_width if isinstance(cfg.beam_width, int) else max(cfg.beam_width)
    evals, n = 1, 1
    for s in range(1, cfg.n_levels):
        n = min(W, len(ps.levels[s]), n * cfg.codebook)
        evals += n
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {
        "value": 1.0 / (evals * per_beam),
        "unit": "req/s",
        "cores": int(threads),
        "cpu": cpu,
        "kind": "oracle",
        "sample": (f"request 0, level 1, {len(beams)} beams, each recomputed as an independent "
                   f"{cfg.n_layers}-layer sequence of ctx+1 tokens with logits, log-softmax and candidates "
                   f"({dt:.1f} s); extrapolated to {evals} beam evaluations per request decode"),
        "seconds": dt,
    }


def graph_leg(cfg, args):
    """The headline decode (one launch per layer) launched directly and as replayed graphs
    (GR_ENGINE_GRAPH): the same engine options, no profiling, contexts resident, each decode
    (every level of every request, beam sets fetched) timed by HIP events on the stream."""
    import torch

    import synth
    from semantic_id_beam_amd import _lib as G
    from semantic_id_beam_amd.workloads import make_engine, request_tensors
    shapes = synth.request_shapes(cfg)
    R, lv = cfg.n_requests, cfg.n_levels
    out = {}
    for graph in (False, True):
        eng = make_engine(cfg, max_requests=R, per_layer=True, graph=graph)
        for r in range(R):
            k, v, q = request_tensors(cfg, r)
            eng.load(r, k, v, q, shapes[r][1])
            del k, v, q
        rids = list(range(R))

        def decode():
            eng.reset_batch(rids)
            for _ in range(lv):
                eng.step(rids)
            eng.beams_batch(rids)

        for _ in range(max(1, args.warmup)):
            decode()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            decode()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / args.steps
        key = "graph" if graph else "direct"
        out[key] = {"ms_per_decode": round(ms, 3), "req_per_s": round(R / (ms * 1e-3), 1)}
        if graph:
            out[key]["captures"], out[key]["replays"] = G.gr_engine_graph_stats(eng.eng)
        eng.close()
    log(f"graph replay: direct {out['direct']['req_per_s']} req/s, graphs {out['graph']['req_per_s']} req/s")
    return out


def decode_leg(cfg, args, per_layer: bool):
    """The timed decode of the workload's requests (contexts resident), with per-kernel times
    from HIP events carried by the dispatches on the decode stream."""
    import numpy as np
    import torch

    import synth
    from semantic_id_beam_amd import _lib as G
    from semantic_id_beam_amd.workloads import make_engine, request_tensors

    shapes = synth.request_shapes(cfg)
    R, lv = cfg.n_requests, cfg.n_levels
    t = time.time()
    eng = make_engine(cfg, max_requests=R, per_layer=per_layer)
    log(f"engine ready ({'one layer per launch' if per_layer else 'several layers per launch'}, "
        f"{eng.ws_bytes / 2**30:.2f} GiB workspace, {time.time() - t:.1f} s)")
    rids = list(range(R))
    t = time.time()
    # contexts are generated in HBM eight at a time; the loads (re-layout, key-norm bounds,
    # value scales) of each batch are timed with events on the load stream
    load_ms = 0.0
    k, v, q = request_tensors(cfg, 0)      # first launches of the loading kernels, untimed
    eng.load(0, k, v, q, shapes[0][1])
    torch.cuda.synchronize()
    eng.release(0)
    del k, v, q
    for r0 in range(0, R, 8):
        batch = [request_tensors(cfg, r) for r in range(r0, min(R, r0 + 8))]
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i, (k, v, q) in enumerate(batch):
            eng.load(r0 + i, k, v, q, shapes[r0 + i][1])
        e1.record()
        torch.cuda.synchronize()
        load_ms += e0.elapsed_time(e1)
        del batch
        log(f"loaded {min(R, r0 + 8)}/{R} contexts ({time.time() - t:.1f} s)")
    torch.cuda.empty_cache()
    load_bytes = sum(ctx_load_bytes(cfg, n) for n, _ in shapes)

    # live beams per level, measured once
    n_live = np.zeros((R, lv), dtype=np.int64)
    for r in rids:
        eng.reset(r)
    n_live[:, 0] = 1
    for s in range(lv):
        eng.step(rids)
        if s + 1 < lv:
            for r in rids:
                n_live[r, s + 1] = eng.state(r)["n"]
    for r in rids:
        eng.beams(r)

    def decode_all():
        eng.reset_batch(rids)
        for _ in range(lv):
            eng.step(rids)
        return eng.beams_batch(rids)

    for i in range(args.warmup):
        decode_all()
    torch.cuda.synchronize()
    # the timed region: the context-attention launches of every PROF_STRIDE-th layer carry HIP
    # events (the roofline's durations: the same kernel on the same work at every layer), the
    # other launches none
    G.gr_engine_profile_reset(eng.eng)
    G.gr_engine_set_profiling_kinds(eng.eng, 1 << G.GR_PROF_CTX_ATTN)
    G.gr_engine_set_profiling_stride(eng.eng, PROF_STRIDE)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        decode_all()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    decode_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    G.gr_engine_set_profiling(eng.eng, False)
    G.gr_engine_set_profiling_stride(eng.eng, 1)
    elapsed = t1 - t0
    log(f"timed {args.steps} decodes in {elapsed:.3f} s")

    # ---- per-kernel times (HIP events carried by the dispatches on the decode stream): context
    # attention from the timed region; the other kernels and whole steps from a second pass of as
    # many decodes with every launch carrying events (outside the timed region)
    prof = {"ctx_attn": {s: G.gr_engine_profile_read(eng.eng, G.GR_PROF_CTX_ATTN, s) for s in range(lv)}}
    ctx_disp = {s: G.gr_engine_profile_dispatches(eng.eng, G.GR_PROF_CTX_ATTN, s) for s in range(lv)}
    G.gr_engine_profile_reset(eng.eng)
    G.gr_engine_set_profiling(eng.eng, True)
    for i in range(args.steps):
        decode_all()
    torch.cuda.synchronize()
    G.gr_engine_set_profiling(eng.eng, False)
    for kind, name in [(G.GR_PROF_BEAM_MERGE, "beam_merge"), (G.GR_PROF_LOGITS, "logits"),
                       (G.GR_PROF_TOPK, "topk"), (G.GR_PROF_STEP, "step")]:
        prof[name] = {s: G.gr_engine_profile_read(eng.eng, kind, s) for s in range(lv)}

    d, g, Hkv = cfg.head_dim, cfg.group, cfg.n_kv_heads
    N = np.array([n for n, _ in shapes], dtype=np.float64)
    el = 2 if cfg.dtype == "bf16" else 4

    def ctx_flops(s):      # one layer, all requests
        return float(np.sum(Hkv * n_live[:, s] * g * N * d * 4))

    def ctx_bytes(s):      # K and V read once, queries read, one fp32 output row per (beam, head)
        return float(np.sum(Hkv * N * d * 2 * el + Hkv * n_live[:, s] * g * d * (el + 4)))

    levels_mfma = [s for s in range(lv) if np.all(n_live[:, s] * g >= 64)]
    ms_m = sum(prof["ctx_attn"][s][0] for s in levels_mfma)
    n_m = sum(prof["ctx_attn"][s][1] for s in levels_mfma)
    fl_m = sum(ctx_flops(s) * prof["ctx_attn"][s][1] for s in levels_mfma)
    achieved_tf = fl_m / (ms_m * 1e-3) / 1e12 if ms_m > 0 else 0.0
    ms_0, n_0 = prof["ctx_attn"][0]
    achieved_gbs0 = ctx_bytes(0) * n_0 / (ms_0 * 1e-3) / 1e9 if ms_0 > 0 else 0.0
    step_us = {f"level{s}": 1e3 * prof["step"][s][0] / max(prof["step"][s][1], 1) for s in range(lv)}

    # the unit is one layer of one step over every request: a dispatch covers one layer (the
    # headline's launch sequence) or several (the multi-layer variant, whose kernel also merges
    # the beam's own tokens and stores the layer's hidden partial: that time is in its
    # denominator, those bytes are not in the algorithmic count)
    wide = cfg.dtype == "bf16" and cfg.head_dim == 128
    d_m = sum(ctx_disp[s] for s in levels_mfma)
    d_0 = ctx_disp[0]
    variant = "per_layer" if per_layer else "fused"
    roofline = {
        "bound": "mfma", "achieved": round(achieved_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved_tf / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(cfg, "k_ctx_attn_wide", variant) if wide else None,
        "traffic_unit": "HBM bytes per layer (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
        "kernel": ("k_ctx_attn_wide" if wide else "k_ctx_attn") + " (levels %s)" % levels_mfma,
        "layers": int(n_m),
        "avg_us_per_layer": round(1e3 * ms_m / max(n_m, 1), 2),
        "dispatches": int(d_m),
        "avg_us_per_dispatch": round(1e3 * ms_m / max(d_m, 1), 2),
        "algorithmic_per_layer": f"{ctx_flops(levels_mfma[-1]) / 1e9:.2f} GFLOP" if levels_mfma else None,
        "timed_launches": (f"every {PROF_STRIDE}th layer's launch of the timed decodes" if per_layer
                           else "every launch of the timed decodes"),
    }
    kernels = {
        # the first level of the one-layer-per-launch sequence runs on the 8-wave kernel (4 token
        # ranges); several layers per launch, on the streaming kernel
        "ctx_attn_level0": {"kernel": ("k_ctx_attn_wide" if per_layer else "k_ctx_attn_stream") if wide else "k_ctx_attn",
                            "bound": "hbm", "achieved_GBs": round(achieved_gbs0, 1), "peak_GBs": PEAK_HBM_GBS,
                            "frac": round(achieved_gbs0 / PEAK_HBM_GBS, 4),
                            "avg_us_per_layer": round(1e3 * ms_0 / max(n_0, 1), 2),
                            "avg_us_per_dispatch": round(1e3 * ms_0 / max(d_0, 1), 2),
                            "dispatches": int(d_0),
                            "algorithmic_MB_per_layer": round(ctx_bytes(0) / 1e6, 2),
                            "traffic": measured_traffic(cfg, "k_ctx_attn_wide_level0", variant) if wide else None},
    }
    for name in ("beam_merge", "logits", "topk"):
        tot = sum(prof[name][s][0] for s in range(lv))
        n = sum(prof[name][s][1] for s in range(lv))
        kernels[name] = {"avg_launch_us": round(1e3 * tot / max(n, 1), 2), "ms_per_decode": round(tot / args.steps, 3)}
    # per-layer launches: the timed (sampled) launches' average duration times the layers of a
    # decode; otherwise every launch was timed
    if per_layer:
        ctx_ms = sum(prof["ctx_attn"][s][0] / max(prof["ctx_attn"][s][1], 1) * cfg.n_layers for s in range(lv))
    else:
        ctx_ms = sum(prof["ctx_attn"][s][0] for s in range(lv)) / args.steps
    kernels["ctx_attn"] = {"ms_per_decode": round(ctx_ms, 3)}
    # context loading (gr_ctx_kv_load), outside the timed decodes: caller K/V read, native
    # K/V^T written (padding included); the key norms and value scales add no traffic
    kernels["ctx_load"] = {"kernel": "k_load_ctx", "bound": "hbm", "ms_per_request": round(load_ms / R, 3),
                           "algorithmic_MB_per_request": round(load_bytes / R / 1e6, 1),
                           "achieved_GBs": round(load_bytes / (load_ms * 1e-3) / 1e9, 1),
                           "frac": round(load_bytes / (load_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    eng.close()
    del eng
    torch.cuda.empty_cache()
    return {
        "value": round(R * args.steps / elapsed, 2),
        "ms_per_step": round(1e3 * elapsed / args.steps, 3),
        "live_beams_per_level": n_live[0].tolist(),
        "step_us": {k: round(v, 1) for k, v in step_us.items()},
        "decode_ms": {"p10": round(float(np.percentile(decode_ms, 10)), 3),
                      "p50": round(float(np.percentile(decode_ms, 50)), 3),
                      "p90": round(float(np.percentile(decode_ms, 90)), 3)},
        "roofline": roofline,
        "kernels": kernels,
    }


def rate_probe_leg(timeout: int = 120):
    """Measured ceilings next to the published peaks: the package's rate probe (a child process,
    started before this process touches the GPU) times dense bf16 and f16 MFMA with no memory
    traffic, and the fp32 FMA and exp2 issue rates, on the whole chip."""
    import subprocess
    probe = os.path.join(os.path.dirname(os.path.abspath(__file__)), "semantic_id_beam_amd", "rate_probe")
    if not os.path.exists(probe):
        raise RuntimeError(f"{probe} is missing: build the package first (semantic_id_beam_amd/build.py)")
    res = subprocess.run([probe], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=timeout)
    if res.returncode != 0:
        raise RuntimeError(f"rate probe failed ({res.returncode}): {res.stderr.strip()}")
    r = json.loads(res.stdout.strip().splitlines()[-1])
    r["mfma_bf16_frac_of_peak"] = round(r["mfma_bf16_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
    r["mfma_f16_frac_of_peak"] = round(r["mfma_f16_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
    r["fma_f32_frac_of_peak"] = round(r["fma_f32_TFLOPs"] / PEAK_FP32_TFLOPS, 4)
    r["exp2_per_fma"] = round(r["exp2_f32_wave_instr_per_ns"] / r["fma_f32_wave_instr_per_ns"], 3)
    r["hbm_read_164MiB_frac_of_peak"] = round(r["hbm_read_164MiB_TBs"] * 1e3 / PEAK_HBM_GBS, 4)
    r["hbm_read_1GiB_frac_of_peak"] = round(r["hbm_read_1GiB_TBs"] * 1e3 / PEAK_HBM_GBS, 4)
    r["mfma_bf16_lds_operand_frac_of_peak"] = round(r["mfma_bf16_lds_operand_TFLOPs"] / PEAK_BF16_TFLOPS, 4)
    r["note"] = ("register-only loops, 4 waves per SIMD on every compute unit; the MFMA figures are the "
                 "sustained dense rate under full matrix-core load (the chip clocks down), not a target; "
                 "HBM: one read pass (16-byte loads, 4096 workgroups) over 164 MiB and over 1 GiB; LDS: "
                 "8 waves per compute unit reading 1 KB per ds_read_b128, and bf16 MFMA taking one such "
                 "read as its A operand per instruction (the context-attention loop's operand path)")
    log(f"rate probe: bf16 MFMA {r['mfma_bf16_TFLOPs']} TFLOP/s ({r['mfma_bf16_frac_of_peak']:.2f} of peak), "
        f"fp32 FMA {r['fma_f32_TFLOPs']} TFLOP/s, exp2 at {r['exp2_per_fma']} of the FMA issue rate, "
        f"HBM read {r['hbm_read_164MiB_TBs']} TB/s (164 MiB) / {r['hbm_read_1GiB_TBs']} TB/s (1 GiB), "
        f"LDS read {r['lds_read_TBs']} TB/s, MFMA with LDS operands {r['mfma_bf16_lds_operand_TFLOPs']} TFLOP/s")
    return r


def wave_times_child(cfg, level: int = 1, layer: int = 13, decodes: int = 3):
    """Runs inside the wave-timeline build (GR_BEAM_LIB_VARIANT=timed): the headline decode with
    one context-attention launch per layer, recording the launch of (level, layer); returns the
    per-wave breakdown of that launch (prologue, token loop, epilogue, copy waits and barriers
    inside the loop, the spread between XCDs)."""
    import ctypes as C

    import numpy as np
    import torch

    import synth
    from semantic_id_beam_amd import _lib as G
    from semantic_id_beam_amd.workloads import make_engine, request_tensors

    if not G.LIB_PATH.endswith("libgr_beam_timed.so"):
        raise RuntimeError("the wave timeline needs the timed library (GR_BEAM_LIB_VARIANT=timed)")
    shapes = synth.request_shapes(cfg)
    R = cfg.n_requests
    eng = make_engine(cfg, max_requests=R, per_layer=True)
    for r in range(R):
        k, v, q = request_tensors(cfg, r)
        eng.load(r, k, v, q, shapes[r][1])
        del k, v, q
    torch.cuda.synchronize()
    L = G.lib()
    if L.gr_wave_times_select(level, layer) != 0:
        raise RuntimeError("gr_wave_times_select failed")
    rids = list(range(R))
    for _ in range(decodes):
        eng.reset_batch(rids)
        for _s in range(cfg.n_levels):
            eng.step(rids)
        eng.beams_batch(rids)
    torch.cuda.synchronize()
    n = 1024 * 8 * 8
    buf = np.zeros(n, dtype=np.int64)
    if L.gr_wave_times_read(buf.ctypes.data_as(C.POINTER(C.c_int64)), n) != 0:
        raise RuntimeError("gr_wave_times_read failed")
    t = buf.reshape(1024, 8, 8)
    rec = t[:, :, 0] != 0
    if not rec.any():
        raise RuntimeError("no wave recorded")
    entry, lstart, lend, done = (t[:, :, f][rec] for f in range(4))
    wait, barrier, loop, nbar = (t[:, :, f][rec].astype(float) for f in range(4, 8))
    us = lambda x: round(float(x) / 100.0, 2)  # 100 MHz stamps
    wg_end = np.where(rec, t[:, :, 3], 0).max(axis=1)
    wg_ids = np.nonzero(rec.any(axis=1))[0]
    xcd_end = [float(np.median(wg_end[[i for i in wg_ids if i % 8 == x]] - entry.min())) / 100.0
               for x in range(8) if any(i % 8 == x for i in wg_ids)]
    return {
        "launch": f"level {level}, layer {layer}, last of {decodes} decodes",
        "workgroups": int(len(wg_ids)), "waves": int(rec.sum()),
        "span_us": us(done.max() - entry.min()),
        "entry_spread_us": us(entry.max() - entry.min()),
        "prologue_us": {"median": us(np.median(lstart - entry)), "max": us((lstart - entry).max())},
        "loop_us": {"median": us(np.median(lend - lstart)), "min": us((lend - lstart).min()),
                    "max": us((lend - lstart).max())},
        "epilogue_us": {"median": us(np.median(done - lend)), "max": us((done - lend).max())},
        "xcd_median_end_us": [round(x, 2) for x in xcd_end],
        "xcd_spread_us": round(max(xcd_end) - min(xcd_end), 2),
        "loop_copy_wait_frac": round(float(wait.sum() / loop.sum()), 4),
        "loop_barrier_frac": round(float(barrier.sum() / loop.sum()), 4),
        "barriers_per_wave": float(np.median(nbar)),
        "memtime_ticks_per_ns": round(float(loop.sum() / ((lend - lstart).sum() * 10.0)), 3),
        "note": "s_memrealtime stamps (entry, token-loop start and end, partial stores done) and "
                "s_memtime cycles of the copy waits and barriers inside the token loop, per wave; "
                "a separate build of the library (libgr_beam_timed.so), the product kernel has none",
    }


def wave_times_leg(level: int = 1, timeout: int = 300):
    """The wave timeline of one headline context-attention launch (layer 13 of the given decode
    level), from a child process that loads the wave-timeline build of the library."""
    import subprocess
    env = dict(os.environ, GR_BEAM_LIB_VARIANT="timed")
    res = subprocess.run([sys.executable, os.path.abspath(__file__), "--wave-times-child", "--wave-level",
                          str(level)], env=env,
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=timeout)
    if res.returncode != 0:
        raise RuntimeError(f"wave timeline failed ({res.returncode}): {res.stderr.strip()[-2000:]}")
    return json.loads(res.stdout.strip().splitlines()[-1])


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default=None, help="workload name (default: the ctx-5000 beam-256 headline)")
    ap.add_argument("--cpu-beams", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other two workloads (64 x ctx 2000 beam 30; ragged 128 in four waves)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the headline decode (one layer per launch): no other legs")
    ap.add_argument("--chain-only", action="store_true", help="only the layer-chain leg (prints its JSON)")
    ap.add_argument("--graph-only", action="store_true",
                    help="only the headline decode launched directly and as replayed graphs (prints its JSON)")
    ap.add_argument("--rate-probe", action="store_true",
                    help="only the unit-rate probe (MFMA, FMA, exp2 ceilings; prints its JSON)")
    ap.add_argument("--no-rate-probe", action="store_true", help="skip the unit-rate probe")
    ap.add_argument("--wave-times", action="store_true",
                    help="only the wave timeline of one headline context-attention launch (a child process "
                         "with the wave-timeline build; prints its JSON)")
    ap.add_argument("--wave-times-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-wave-times", action="store_true", help="skip the wave timeline")
    ap.add_argument("--wave-level", type=int, default=1, help="decode level of the recorded launch (default 1)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run one device-to-device copy of MIB MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.wave_times_child:
        import synth
        from synth.configs import HEADLINE
        print(json.dumps(wave_times_child(synth.get_config(args.config or HEADLINE), level=args.wave_level)),
              flush=True)
        return
    if args.wave_times:
        print(json.dumps({"wave_times": wave_times_leg(args.wave_level)}), flush=True)
        return
    if args.rate_probe:
        print(json.dumps({"rate_probe": rate_probe_leg()}), flush=True)
        return
    # before this process touches the GPU: the probe runs as a child process
    ceilings = None if (args.no_rate_probe or args.decode_only or args.chain_only or args.graph_only
                        or args.copy_probe or args.gpus != 1) else rate_probe_leg()
    timeline = None if (args.no_wave_times or args.decode_only or args.chain_only or args.graph_only
                        or args.copy_probe or args.gpus != 1 or args.config is not None) else wave_times_leg()
    if args.copy_probe:
        import torch
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step shards by request with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from synth.configs import HEADLINE

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.chain_only:
        print(json.dumps({"chain": chain_leg(args)}), flush=True)
        return
    cfg = synth.get_config(args.config or HEADLINE)
    if args.graph_only:
        print(json.dumps({"graph_replay": graph_leg(cfg, args)}), flush=True)
        return
    shapes = synth.request_shapes(cfg)
    R, lv = cfg.n_requests, cfg.n_levels
    log("workload", workload_text(cfg, shapes))
    # the headline: one context-attention launch per layer at every level (the launch sequence
    # of a model whose layers depend on each other)
    head = decode_leg(cfg, args, per_layer=True)
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "req/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": workload_text(cfg, shapes), "requests": R, "layers": cfg.n_layers,
                   "ctx_len": cfg.ctx_len, "beam_width": cfg.beam_width, "levels": lv,
                   "codebook": cfg.codebook, "items": cfg.n_items,
                   "live_beams_per_level": head["live_beams_per_level"],
                   "launches": "one context-attention launch per layer at every level"},
        "step_us": head["step_us"],
        "decode_ms": head["decode_ms"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
    }
    if ceilings is not None:
        ceil_tf = min(ceilings["mfma_bf16_TFLOPs"], ceilings["mfma_f16_TFLOPs"])  # QK^T bf16, PV f16
        out["roofline"]["measured_ceiling"] = {
            "TFLOPs": ceil_tf, "frac": round(out["roofline"]["achieved"] / ceil_tf, 4),
            "note": "the rate probe's sustained dense MFMA rate on this box (the lower of bf16 and f16); context only"}
        out["rate_probe"] = ceilings
        lv0 = out["kernels"]["ctx_attn_level0"]
        lv0["measured_ceiling"] = {
            "GBs": round(ceilings["hbm_read_164MiB_TBs"] * 1e3, 1),
            "frac": round(lv0["achieved_GBs"] / (ceilings["hbm_read_164MiB_TBs"] * 1e3), 4),
            "note": "the rate probe's read pass over 164 MiB (one layer's K and V) on this box; context only"}
    if timeline is not None:
        out["wave_times"] = timeline
    if not args.decode_only:
        # labelled variant, not the headline: where every layer's query is an input (this model
        # stand-in), the first level runs all layers in one launch and wide levels several
        fused = decode_leg(cfg, args, per_layer=False)
        out["fused_layers_variant"] = {
            "note": ("several layers per context-attention launch (first level: all layers; wide levels: "
                     "a group of layers): valid only because this model stand-in's layers are independent; "
                     "not the headline"),
            **{k: fused[k] for k in ("value", "ms_per_step", "step_us", "decode_ms", "roofline", "kernels")}}
        out["graph_replay"] = graph_leg(cfg, args)
        out["chain"] = chain_leg(args)
        out["scoring"] = scoring_leg(cfg, args)
        out["prefill"] = prefill_leg(cfg, args)
        if not args.no_workloads:
            out["workloads"] = {w: workload_leg(w) for w in ("ctx2k_beam30_r64", "ragged_r128")}
            out["workloads_fused_layers_variant"] = {w: workload_leg(w, per_layer=False)["req_per_s"]
                                                     for w in ("ctx2k_beam30_r64", "ragged_r128")}
            out["serving"] = serving_leg()
            out["serving_graph"] = serving_leg(graph=True)
    if not args.no_cpu_baseline:
        log(f"timing the oracle on {args.cpu_beams} beams ...")
        cb = cpu_baseline(cfg, args.cpu_beams)
        log(f"oracle sample took {cb.pop('seconds'):.1f} s")
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
