#!/usr/bin/env python3
"""Benchmark of one DFlash speculative step on one GPU.

A step is the whole hot path over one batch: feature fusion + KV injection of the 16 most
recently accepted context positions of every request (rewriting positions T-16..T-1 with
the same features, so every step sees the same cache), one block-diffusion draft pass
(16-slot block, 15 drafted tokens per request) and greedy verification.  The step is
captured once in a HIP graph and replayed.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload qwen3_b1]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense MFMA, per dtype


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_b1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--latency-shape", action="store_true",
                    help="time one draft pass of the batch-1 Qwen3-8B-shaped drafter at 1, 2, "
                         "3, 5 and 8 layers, and 8 sequential passes of the 1-layer drafter")
    ap.add_argument("--loop", action="store_true",
                    help="time the closed decoding loop (draft, verify, advance, inject) "
                         "against a seeded synthetic target instead of the single step")
    ap.add_argument("--prefill", action="store_true",
                    help="time only the drafter prefill of 2048 positions, KV injection "
                         "against the input-fusion variant")
    ap.add_argument("--verify-sampled", action="store_true",
                    help="time only the temperature-1 verify (64 x 16 x 128256 logits)")
    ap.add_argument("--kernel-reps", type=int, default=30)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra measurements of the default run (the Qwen3-8B-shaped "
                         "step at batch 32, greedy verify alone, temperature-1 verify)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_hbm_traffic_qwen3-8b-b1.txt")
GEMM_SOURCE = os.path.join(ROOT, "block_diffusion_drafter_hidden_amd", "csrc", "gemm.hip")


def measured_traffic(workload):
    """HBM bytes per LM-head launch from the committed counter profile, or None when the
    profile is for another workload or the kernel source has changed since it was taken."""
    import hashlib
    try:
        kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE).read().splitlines()
                  if ":" in line and not line.startswith(" "))
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
        if kv["gemm_source_sha256"].strip() != src or kv["workload"].strip() != workload:
            return None
        return int(kv["hbm_bytes_per_launch"].strip())
    except Exception:
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_drafter_hidden_amd import Drafter, binding as B
    from workloads import WORKLOADS, synth

    wl = WORKLOADS[args.workload]
    if args.loop:
        return loop_bench(args, wl)
    if args.latency_shape:
        return latency_bench(args, wl)
    if args.prefill:
        return prefill_bench(args, wl)
    if args.verify_sampled:
        s = torch.cuda.Stream(device=torch.device("cuda:0"))
        out = verify_sampled_timing(torch.device("cuda:0"), s)
        print(json.dumps({"metric": "temperature-1 verify time", "value": out["us_per_call"],
                          "unit": "us per call", "n_gpus": 1, "higher_is_better": False,
                          "dtype": "f32 logits, f64 weights", "data": "synthetic",
                          "config": {"workload": "llama3.1-8b-shaped-batch64-verify"},
                          **out}), flush=True)
        return
    cfg = wl.cfg
    Bn = wl.batch
    ctx = synth.context_lengths(wl)
    n_new = cfg.block_size
    dev = torch.device("cuda:0")

    log(f"[bench] workload {wl.name}: generating weights")
    w = synth.drafter_weights(cfg, seed=wl.seed)
    wd = {k: v.to(dev) for k, v in w.items()}
    table, num_pages = synth.page_table(wl.name, ctx, cfg.page_size, wl.seed)
    dr = Drafter(cfg, wd, max_batch=Bn, max_ctx=table.shape[1] * cfg.page_size,
                 max_inject_rows=min(max(256, Bn * n_new), 1024), device=dev)
    embed = wd["embed"]
    del wd
    torch.cuda.empty_cache()
    cache = dr.new_cache(table, ctx, num_pages)

    # Cache contents: request 0's context is injected through the library from its target
    # features (the oracle leg recomputes it); with a batch, the other requests' caches hold
    # seeded synthetic K/V of the same scale (their values do not change the work done).
    if Bn > 1:
        gen = torch.Generator(device=dev).manual_seed(synth.stream_seed(wl.seed, "bench/fill"))
        for pool in (cache.k_pool, cache.v_pool):
            pool.normal_(0.0, 3.0, generator=gen)
    log("[bench] prefill: injecting request 0's context")
    feats0 = synth.target_features(cfg, int(ctx[0]), "bench/ctx/b0", seed=wl.seed)
    dr.inject(cache, feats0.to(dev), torch.zeros((int(ctx[0]),), dtype=torch.int32, device=dev),
              torch.arange(int(ctx[0]), dtype=torch.int32, device=dev))
    torch.cuda.synchronize()

    # Step inputs: the last n_new positions of every request, re-injected (request 0 from its
    # own features, the others from seeded features of the same distribution).
    tail = [feats0[int(ctx[0]) - n_new:]] + [
        synth.target_features(cfg, n_new, f"bench/tail/b{b}", seed=wl.seed)
        for b in range(1, Bn)]
    new_feats = torch.cat(tail).to(dev)
    new_seq = torch.as_tensor(np.repeat(np.arange(Bn), n_new).astype(np.int32)).to(dev)
    new_pos = torch.as_tensor(np.concatenate([np.arange(int(T) - n_new, int(T)) for T in ctx])
                              .astype(np.int32)).to(dev)
    anchors_h = synth.anchor_ids(cfg, Bn, wl.seed)
    anchors = torch.as_tensor(anchors_h).to(dev)
    draft_ids = torch.zeros((Bn, 15), dtype=torch.int32, device=dev)
    accept = torch.zeros(Bn, dtype=torch.int32, device=dev)
    bonus = torch.zeros(Bn, dtype=torch.int32, device=dev)

    # ---------------- CPU oracle leg (rank 0, bounded sample: request 0, one step) -------
    cpu = None
    orc = None
    if not args.no_cpu_baseline:
        import oracle.dflash_oracle as ref
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            cores = os.cpu_count()
        T0 = int(ctx[0])
        log("[bench] oracle: prefill of request 0 (untimed)")
        ks, vs = ref.prefill_context(cfg, w, feats0[:T0 - n_new])
        tgt_dummy = np.zeros(16, dtype=np.int32)
        log("[bench] oracle: timed steps (inject 16 + draft + verify), at least 10 s")
        n_rep, t0 = 0, time.perf_counter()
        while True:
            orc = ref.draft_step(cfg, w, ks, vs, feats0[T0 - n_new:], int(anchors_h[0]),
                                 tgt_dummy)
            n_rep += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or n_rep >= 200:
                break
        cpu = {"value": round(15.0 * n_rep / dt, 3), "unit": "drafted tokens/s",
               "cores": int(cores), "kind": "oracle",
               "sample": f"request 0 of the batch, {n_rep} repeats of one step: inject {n_new} "
                         f"positions, draft one block over context {T0}, greedy verify; "
                         f"float64 numpy; prefill untimed; {dt:.2f} s"}
        del ks, vs

    if orc is not None:
        tgt_rows = [synth.planted_targets(orc["ids"][None], cfg.vocab, f"bench/plant/{b}",
                                          wl.seed)[0][0] for b in range(Bn)]
    else:
        fake = synth.uniform_ints("bench/ref-drafts", (Bn, 15), 0, cfg.vocab - 1, wl.seed)
        tgt_rows = list(synth.planted_targets(fake, cfg.vocab, "bench/plant", wl.seed)[0])
    target = torch.as_tensor(np.stack(tgt_rows).astype(np.int32)).to(dev)
    del w

    def step():
        dr.inject(cache, new_feats, new_seq, new_pos)
        dr.draft(cache, anchors, draft_ids)
        B.verify_accept(draft_ids, target, accept, bonus)

    # ---------------- GPU timed region ----------------
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            step()
        torch.cuda.synchronize()
    run = graph.replay if graph is not None else step
    with torch.cuda.stream(s):
        for _ in range(args.warmup):
            run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(args.steps):
            run()
        e1.record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps

    # ---------------- dominant kernel: LM head + argmax, timed alone ----------------
    roofline = lm_head_roofline(dr, Bn * 15, s, args.kernel_reps, wl.name)

    if args.copy_mib > 0:   # a plain copy of known size, for scaling the HBM byte counters
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        with torch.cuda.stream(s):
            for _ in range(3):
                dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------- parity of the timed step's drafts (request 0) ----------------
    parity = None
    if orc is not None:
        import oracle.dflash_oracle as ref
        got = draft_ids.cpu().numpy()[0]
        tie = ref.near_tie(orc["gap"], orc["top1"], orc["top2"], cfg.dtype)
        parity = {"request": 0, "mismatches": int(((got != orc["ids"]) & ~tie).sum()),
                  "near_ties_excused": int(tie.sum()),
                  "accept_len_gpu": int(accept.cpu()[0]),
                  "accept_len_oracle": int(ref.verify_greedy(orc["ids"], tgt_rows[0])[0])}

    acc_ = step_accounting(cfg, Bn, ctx, n_new, ms)
    step_bytes, roof = acc_["step_bytes"], acc_["roof_us"]
    drafted = Bn * 15
    value = drafted / (ms * 1e-3)

    out = {
        "metric": "drafted tokens/s (DFlash b16 draft step: inject + draft + verify)",
        "value": round(value, 1),
        "unit": "drafted tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) target features, random ids)",
        "config": {"workload": wl.name, "batch": Bn, "context": int(ctx.max()),
                   "context_min": int(ctx.min()), "block": cfg.block_size,
                   "layers": cfg.n_layers, "hidden": cfg.hidden, "vocab": cfg.vocab,
                   "graph": graph is not None},
        "step_hbm_fraction": acc_["step_hbm_fraction"],
        "step_algorithmic_bytes": int(step_bytes),
        "step_roofline_us": acc_["step_roofline_us"],
        "step_roofline_fraction": acc_["step_roofline_fraction"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "wall_s_timed": round(t_wall, 3),
    }
    if wl.name == WORKLOADS["qwen3_b1"].name and not args.no_extra:
        out.update(extra_measurements(args, dr, s))
    print(json.dumps(out), flush=True)


def time_replays(fn, s, steps, warmup, graph=True):
    """Capture fn once in a HIP graph on stream s, replay it `warmup` times, then time
    `steps` replays between events on s.  Returns ms per replay."""
    import torch
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    run = fn
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize()
        run = g.replay
    with torch.cuda.stream(s):
        for _ in range(warmup):
            run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        e0.record(s)
        for _ in range(steps):
            run()
        e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def lm_head_roofline(dr, rows, s, reps, workload):
    """The dominant kernel, the shared LM head + argmax, timed alone through
    dflash_lm_head_argmax on `rows` seeded hidden rows, with HIP events on its stream.  It is
    HBM-bound while its rows are few (15 flop per weight byte at one request) and MFMA-bound
    past the ridge: the object takes whichever bound is the larger time."""
    import torch
    from block_diffusion_drafter_hidden_amd import binding as B
    cfg, dev = dr.cfg, dr.device
    y = torch.randn((rows, cfg.hidden), device=dev, dtype=torch.float32)
    ids_tmp = torch.empty(rows, dtype=torch.int32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    with torch.cuda.stream(s):
        for _ in range(3):
            B.lm_head_argmax(dr.ccfg, dr.packed, y, ids_tmp, dr.ws)
        for a, b in evs:
            a.record(s)
            B.lm_head_argmax(dr.ccfg, dr.packed, y, ids_tmp, dr.ws)
            b.record(s)
    torch.cuda.synchronize()
    lm_us = 1000.0 * sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    es = 2 if cfg.dtype == "bf16" else 4
    V, H = cfg.vocab, cfg.hidden
    lm_bytes = V * H * es + rows * H * 4 + rows * 4
    lm_flops = 2.0 * V * H * rows
    kern = ("gemm_stream<bf16,A_HILO,1,4,EPI_ARGMAX>" if rows <= 64 or cfg.dtype != "bf16"
            else "gemm_tall256<EPI_ARGMAX> (256-row blocks)")
    out = {"kernel": f"shared LM head + argmax alone ({rows} rows): {kern}; launch_us spans "
                     "the entry point's three launches (rows to fragment layout, LM-head "
                     "GEMM, argmax finalize)",
           "scope": "dominant kernel only; the whole step is step_hbm_fraction / "
                    "step_roofline_fraction",
           "launch_us": round(lm_us, 2), "bytes_per_launch": int(lm_bytes),
           "flops_per_launch": int(lm_flops)}
    mfma_peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    if lm_flops / (mfma_peak * 1e12) > lm_bytes / (HBM_PEAK_GBS * 1e9):
        tf = lm_flops / (lm_us * 1e-6) / 1e12
        out.update({"bound": "mfma", "achieved": round(tf, 1), "peak": mfma_peak,
                    "unit": "TFLOP/s", "frac": round(tf / mfma_peak, 4), "traffic": None})
    else:
        gbs = lm_bytes / (lm_us * 1e-6) / 1e9
        out.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(workload)})
    return out


def extra_measurements(args, dr, s):
    """The default run's other figures, as extra keys of its line: the Qwen3-8B-shaped step
    at batch 32 (ragged contexts U[512, 8192], paged), greedy verify alone, and the
    temperature-1 verify at 64 x 16 x 128256 fp32 logits."""
    import numpy as np
    import torch
    from block_diffusion_drafter_hidden_amd import binding as B
    from workloads import WORKLOADS, synth

    dev = dr.device
    extra = {}
    # ---------------- Qwen3-8B shape, batch 32, ragged contexts ----------------
    wl = WORKLOADS["qwen3_b32"]
    cfg, Bn, n_new = wl.cfg, wl.batch, wl.cfg.block_size
    ctx = synth.context_lengths(wl)
    log(f"[bench] {wl.name}: batch {Bn}, contexts {ctx.min()}..{ctx.max()}")
    table, num_pages = synth.page_table(wl.name + "/bench", ctx, cfg.page_size, wl.seed)
    d32 = dr.sibling(Bn, table.shape[1] * cfg.page_size, min(Bn * n_new, 1024))
    cache = d32.new_cache(table, ctx, num_pages)
    gen = torch.Generator(device=dev).manual_seed(synth.stream_seed(wl.seed, "bench/b32/fill"))
    for pool in (cache.k_pool, cache.v_pool):   # context K/V of the injected scale (seeded)
        pool.normal_(0.0, 3.0, generator=gen)
    feats = torch.cat([synth.target_features(cfg, n_new, f"bench/b32/tail/b{b}", seed=wl.seed)
                       for b in range(Bn)]).to(dev)
    seq = torch.as_tensor(np.repeat(np.arange(Bn), n_new).astype(np.int32)).to(dev)
    pos = torch.as_tensor(np.concatenate([np.arange(int(T) - n_new, int(T)) for T in ctx])
                          .astype(np.int32)).to(dev)
    anchors = torch.as_tensor(synth.anchor_ids(cfg, Bn, wl.seed)).to(dev)
    fake = synth.uniform_ints("bench/b32/drafts", (Bn, 15), 0, cfg.vocab - 1, wl.seed)
    target = torch.as_tensor(synth.planted_targets(fake, cfg.vocab, "bench/b32/plant",
                                                   wl.seed)[0]).to(dev)
    ids = torch.zeros((Bn, 15), dtype=torch.int32, device=dev)
    acc = torch.zeros(Bn, dtype=torch.int32, device=dev)
    bon = torch.zeros_like(acc)

    def step():
        d32.inject(cache, feats, seq, pos)
        d32.draft(cache, anchors, ids)
        B.verify_accept(ids, target, acc, bon)

    steps32 = max(5, args.steps // 2)
    ms = time_replays(step, s, steps32, max(2, args.warmup // 2))
    a32 = step_accounting(cfg, Bn, ctx, n_new, ms)
    extra["batch32"] = {
        "workload": wl.name, "batch": Bn, "context_min": int(ctx.min()),
        "context_max": int(ctx.max()), "steps": steps32, "ms_per_step": round(ms, 4),
        "drafted_tokens_per_s": round(Bn * 15 / (ms * 1e-3), 1),
        "step_hbm_fraction": a32["step_hbm_fraction"],
        "step_algorithmic_bytes": a32["step_bytes"],
        "step_roofline_us": a32["step_roofline_us"],
        "step_roofline_fraction": a32["step_roofline_fraction"],
        "roofline": lm_head_roofline(d32, Bn * 15, s, max(5, args.kernel_reps // 3), wl.name),
    }
    log(f"[bench] batch 32: {ms:.4f} ms per step")
    del cache, d32
    torch.cuda.empty_cache()

    # ---------------- greedy verify alone ----------------
    gv = {}
    for nb in (1, 32, 4096):
        dd = torch.as_tensor(synth.uniform_ints(f"bench/gv/{nb}", (nb, 15), 0, 151935)).to(dev)
        tt = torch.as_tensor(synth.planted_targets(dd.cpu().numpy(), 151936,
                                                   f"bench/gv/plant/{nb}")[0]).to(dev)
        aa = torch.zeros(nb, dtype=torch.int32, device=dev)
        bb = torch.zeros_like(aa)
        calls = 64   # per graph replay, so the replay's own launch cost is spread thin

        def many():
            for _ in range(calls):
                B.verify_accept(dd, tt, aa, bb)
        us = 1000.0 * time_replays(many, s, 20, 3) / calls
        gv[f"batch{nb}"] = {"us_per_call": round(us, 2),
                            "calls_per_s": round(1e6 / us, 1),
                            "requests_per_s": round(nb * 1e6 / us, 1),
                            "method": f"{calls} dependent calls per graph replay"}
    extra["verify_greedy"] = gv

    extra["verify_sampled"] = verify_sampled_timing(dev, s)

    extra["prefill_2048"] = prefill_comparison(args, dr, s)
    return extra


def verify_sampled_timing(dev, s):
    """Temperature-1 verify at 64 x 16 x 128256 fp32 logits (the LLaMA-shaped batch-64
    configuration), four dependent calls per graph replay."""
    import torch
    from block_diffusion_drafter_hidden_amd import binding as B
    from workloads import WORKLOADS, synth

    wl = WORKLOADS["llama_b64"]
    dl, tl, ud, ua, ur = synth.sampled_verify_inputs(wl)
    Bn, V = dl.shape[0], dl.shape[2]
    t = lambda x: torch.as_tensor(x).to(dev).contiguous()
    dl_d, tl_d, ud_d, ua_d, ur_d = t(dl), t(tl), t(ud), t(ua), t(ur)
    del dl, tl
    d_ids = torch.empty((Bn, 15), dtype=torch.int32, device=dev)
    acc = torch.empty(Bn, dtype=torch.int32, device=dev)
    emi = torch.empty((Bn, 16), dtype=torch.int32, device=dev)
    ws = torch.empty(B.verify_sampled_workspace_size(Bn, V), dtype=torch.uint8, device=dev)
    calls = 4   # back-to-back calls per graph replay, so the replay's own launch cost is
                # spread over them (the inputs, 1.02 GB, do not fit the memory-side cache)

    def run():
        for _ in range(calls):
            B.verify_accept_sampled(dl_d, tl_d, ud_d, ua_d, ur_d, d_ids, acc, emi, ws)
    # 30 warm-up replays (~25 ms): the first ~20 replays after an idle GPU run up to 25% slower
    # while the clocks ramp (measured 280 -> 225 us per call over the first 30 replays).
    us = 1000.0 * time_replays(run, s, 20, 30) / calls
    nbytes = (Bn * 15 + Bn * 16) * V * 4    # every logit read once
    gbs = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] temperature-1 verify: {us:.1f} us ({gbs:.0f} GB/s)")
    out = {"shape": f"{Bn} x (15 + 16) x {V} fp32 logits", "us_per_call": round(us, 1),
           "requests_per_s": round(Bn * 1e6 / us, 1), "algorithmic_bytes": int(nbytes),
           "achieved_GBs": round(gbs, 1), "hbm_fraction": round(gbs / HBM_PEAK_GBS, 4),
           "method": f"{calls} dependent calls per graph replay"}
    del dl_d, tl_d, ws
    torch.cuda.empty_cache()
    return out


def prefill_bench(args, wl):
    """--prefill: the prefill comparison alone, as its own JSON line."""
    import torch
    from block_diffusion_drafter_hidden_amd import Drafter
    from workloads import WORKLOADS, synth

    wl = WORKLOADS["qwen3_b1"]
    dev = torch.device("cuda:0")
    log(f"[prefill] {wl.name}: generating weights")
    w = synth.drafter_weights(wl.cfg, seed=wl.seed)
    wd = {k: v.to(dev) for k, v in w.items()}
    del w
    dr = Drafter(wl.cfg, wd, max_batch=1, max_ctx=2048, max_inject_rows=16, device=dev)
    del wd
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    out = prefill_comparison(args, dr, s)
    print(json.dumps({
        "metric": "drafter prefill time of a 2048-position context: KV injection vs input "
                  "fusion", "value": out["input_fusion_over_kv_injection"],
        "unit": "input-fusion time / KV-injection time", "n_gpus": 1, "steps": out["replays"],
        "warmup": 2, "higher_is_better": True, "dtype": wl.cfg.dtype,
        "data": "synthetic (seeded weights and target features)",
        "config": {"workload": f"{wl.cfg.name}-prefill-2048"}, **out}), flush=True)


def prefill_comparison(args, dr, s, T=2048):
    """Drafter prefill of a T-position context, KV injection against the input-fusion
    variant, on the Qwen3-8B-shaped drafter (one request, a fresh cache, each as one call
    replayed from a HIP graph).  KV injection: the fusion GEMM plus every layer's K|V
    projection.  Input fusion: the fusion GEMM, then the context rows through the layers
    (causal attention), the last layer only as far as its K|V."""
    import torch
    from workloads import WORKLOADS, synth

    wl = WORKLOADS["qwen3_b1"]
    cfg, dev = dr.cfg, dr.device
    table, num_pages = synth.page_table(wl.name + "/prefill", [T], cfg.page_size, wl.seed)
    d = dr.sibling(1, table.shape[1] * cfg.page_size, 1024)
    cache = d.new_cache(table, [0], num_pages)
    feats = synth.target_features(cfg, T, "bench/prefill", seed=wl.seed).to(dev)
    seq = torch.zeros(T, dtype=torch.int32, device=dev)
    pos = torch.arange(T, dtype=torch.int32, device=dev)
    d.prefill_input_fusion(cache, feats, 0)       # sizes its workspace outside the graph
    torch.cuda.synchronize()
    reps = max(5, args.steps // 5)
    inj_ms = time_replays(lambda: d.inject(cache, feats, seq, pos), s, reps, 2)
    fus_ms = time_replays(lambda: d.prefill_input_fusion(cache, feats, 0), s, reps, 2)
    H, F, L, I = cfg.hidden, cfg.feat_dim, cfg.n_layers, cfg.intermediate
    qkv = (cfg.n_q_heads + 2 * cfg.n_kv_heads) * cfg.head_dim
    kv = 2 * cfg.n_kv_heads * cfg.head_dim
    qd = cfg.n_q_heads * cfg.head_dim
    inj_flops = 2.0 * T * (F * H + L * kv * H)
    layer = H * qkv + qd * H + 3 * H * I
    attn = 2.0 * 2 * (T * (T + 1) / 2) * qd          # causal QK^T and PV
    fus_flops = 2.0 * T * (F * H + (L - 1) * layer + H * qkv) + (L - 1) * attn
    peak = MFMA_PEAK_TFLOPS[cfg.dtype]
    out = {"positions": T, "kv_injection_ms": round(inj_ms, 4),
           "input_fusion_ms": round(fus_ms, 4),
           "input_fusion_over_kv_injection": round(fus_ms / inj_ms, 2),
           "kv_injection_tflops": round(inj_flops / (inj_ms * 1e-3) / 1e12, 1),
           "input_fusion_tflops": round(fus_flops / (fus_ms * 1e-3) / 1e12, 1),
           "mfma_peak_tflops": peak, "algorithmic_flops": {"kv_injection": int(inj_flops),
                                                            "input_fusion": int(fus_flops)},
           "replays": reps}
    log(f"[bench] prefill {T}: KV injection {inj_ms:.3f} ms, input fusion {fus_ms:.3f} ms")
    del cache, d
    torch.cuda.empty_cache()
    return out


def step_accounting(cfg, Bn, ctx, n_new, ms):
    """Algorithmic bytes of one step (weights once, context KV once, features; activations
    are small) and its roofline time: every kernel at the larger of its HBM time (bytes /
    peak bandwidth) and its MFMA time (flops / dense peak of the dtype), summed.  At one
    request every kernel is HBM-bound (the roofline fraction equals the HBM fraction); with
    a batch the GEMMs cross the ridge and the sum grows by their MFMA time."""
    es = 2 if cfg.dtype == "bf16" else 4
    H, F, V, I = cfg.hidden, cfg.feat_dim, cfg.vocab, cfg.intermediate
    L, qd, kvd = cfg.n_layers, cfg.q_dim, cfg.kv_dim
    w_layer = (qd + 2 * kvd) * H + H * qd + 2 * I * H + H * I
    step_bytes = es * (H * F + L * 2 * kvd * H + L * w_layer + V * H)
    step_bytes += es * Bn * n_new * F                                   # features read
    step_bytes += es * int(sum(int(T) for T in ctx)) * L * 2 * kvd       # context K/V read
    peak_tf = MFMA_PEAK_TFLOPS[cfg.dtype]

    def roof_us(nbytes, flops):
        return max(nbytes / (HBM_PEAK_GBS * 1e3), flops / (peak_tf * 1e6))

    R, Rn = Bn * 16, Bn * n_new
    roof = roof_us(es * (H * F + Rn * F), 2.0 * Rn * H * F)                     # fusion
    roof += roof_us(es * L * 2 * kvd * H, 2.0 * Rn * L * 2 * kvd * H)          # K|V injection
    for n_out, k_in in (((qd + 2 * kvd), H), (H, qd), (2 * I, H), (H, I)):     # per layer
        roof += L * roof_us(es * n_out * k_in, 2.0 * R * n_out * k_in)
    keys = int(sum(int(T) + 16 for T in ctx))
    roof += L * roof_us(es * int(sum(int(T) for T in ctx)) * 2 * kvd,         # attention
                        4.0 * 16 * cfg.n_q_heads * cfg.head_dim * keys)
    roof += roof_us(es * V * H, 2.0 * Bn * 15 * V * H)                        # LM head
    return {"step_bytes": int(step_bytes), "roof_us": roof,
            "step_hbm_fraction": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_roofline_us": round(roof, 1),
            "step_roofline_fraction": round(roof / (ms * 1e3), 4)}


def loop_bench(args, wl):
    """The closed speculative loop, one iteration per timed step: draft a block, build the
    synthetic target's ids (planted k ~ U{0..15} matching drafts per request and
    iteration), greedy verify, advance (context += accept length, anchor = bonus) and inject the
    target features of the block's 16 slots.  The graph of one iteration is replayed, so the
    contexts grow as in decoding.  The synthetic target's own kernels (a few torch ops) are
    timed alone and reported; accepted tokens/s excludes them."""
    import numpy as np
    import torch

    from block_diffusion_drafter_hidden_amd import Drafter, binding as B
    from workloads import synth

    cfg, Bn = wl.cfg, wl.batch
    ctx = synth.context_lengths(wl)
    dev = torch.device("cuda:0")
    iters = args.warmup + args.steps + 2
    w = synth.drafter_weights(cfg, seed=wl.seed)
    wd = {k: v.to(dev) for k, v in w.items()}
    del w
    table, num_pages = synth.page_table(wl.name + "/loop", ctx + 16 * (iters + 1),
                                        cfg.page_size, wl.seed)
    dr = Drafter(cfg, wd, max_batch=Bn, max_ctx=table.shape[1] * cfg.page_size,
                 max_inject_rows=min(max(256, Bn * 16), 1024), device=dev)
    del wd
    torch.cuda.empty_cache()
    cache = dr.new_cache(table, ctx, num_pages)
    gen = torch.Generator(device=dev).manual_seed(synth.stream_seed(wl.seed, "bench/loop/fill"))
    for pool in (cache.k_pool, cache.v_pool):   # context K/V: seeded, of the injected scale
        pool.normal_(0.0, 3.0, generator=gen)
    feats = torch.cat([synth.target_features(cfg, 16, f"bench/loop/b{b}", seed=wl.seed)
                       for b in range(Bn)]).to(dev)
    # Planting draws per iteration (k ~ U{0..15} per request and iteration), indexed on the
    # device by an iteration counter that the captured iteration advances.
    draws = [synth.plant_draws(f"bench/loop/it{i}", Bn, cfg.vocab, wl.seed) for i in range(iters)]
    k_d, fill_d, r_d = (torch.from_numpy(np.stack([np.asarray(d[j]) for d in draws])).to(dev)
                        for j in range(3))
    counters = [torch.zeros(1, dtype=torch.long, device=dev) for _ in range(2)]
    anchors = torch.as_tensor(synth.anchor_ids(cfg, Bn, wl.seed)).to(dev)
    ids = torch.zeros((Bn, 15), dtype=torch.int32, device=dev)
    acc = torch.zeros(Bn, dtype=torch.int32, device=dev)
    bonus = torch.zeros_like(acc)
    inj_seq = torch.zeros(Bn * 16, dtype=torch.int32, device=dev)
    inj_pos = torch.zeros_like(inj_seq)
    tgt = torch.zeros((Bn, 16), dtype=torch.int32, device=dev)

    def target_stub(c=counters[1]):
        i = torch.remainder(c, iters)
        tgt.copy_(synth.plant_device(ids, k_d.index_select(0, i)[0], fill_d.index_select(0, i)[0],
                                     r_d.index_select(0, i)[0], cfg.vocab))
        c.add_(1)

    def iteration():
        dr.draft(cache, anchors, ids)
        target_stub(counters[0])
        B.verify_accept(ids, tgt, acc, bonus)
        dr.advance(cache, acc, bonus, anchors, inj_seq, inj_pos)
        dr.inject(cache, feats, inj_seq, inj_pos)

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    for fn in (iteration, target_stub):
        with torch.cuda.stream(s):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize()
        graphs.append(g)
    T_start = cache.ctx_lens.clone()
    times = []
    for g, n in ((graphs[0], args.steps), (graphs[1], args.steps)):
        with torch.cuda.stream(s):
            for _ in range(args.warmup if g is graphs[0] else 2):
                g.replay()
        torch.cuda.synchronize()
        if g is graphs[0]:
            T_start = cache.ctx_lens.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            for _ in range(n):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / n)
    grown = (cache.ctx_lens - T_start).cpu().numpy()
    acc_per_iter = float(grown.sum()) / args.steps          # accepted tokens per iteration
    ms, stub_ms = times
    timed = [(1 + args.warmup + j) % iters for j in range(args.steps)]
    planted = float(sum((np.asarray(draws[i][0]) + 1).sum() for i in timed)) / args.steps
    out = {
        "metric": "accepted tokens/s (closed DFlash loop: draft + greedy verify + advance + "
                  "inject, seeded synthetic target with planted acceptance)",
        "value": round(acc_per_iter / ((ms - stub_ms) * 1e-3), 1),
        "unit": "accepted tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "synthetic_target_ms": round(stub_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded weights, features and planted target ids)",
        "config": {"workload": wl.name + "+closed-loop", "batch": Bn,
                   "context_start": int(ctx.max()),
                   "context_end": int(cache.ctx_lens.max().item()),
                   "accepted_per_iteration": round(acc_per_iter, 2),
                   "accepted_per_iteration_planted": planted,
                   "graph": True},
        "drafted_tokens_per_s": round(Bn * 15 / (ms * 1e-3), 1),
    }
    assert abs(acc_per_iter - planted) < 1e-6, (acc_per_iter, planted)
    print(json.dumps(out), flush=True)


def latency_bench(args, wl):
    """Draft latency against drafter depth and block size: one block pass of the workload's
    drafter shape at batch 1 with 1, 2, 3, 5 and 8 layers and blocks of 8, 16 and 32 tokens
    (7, 15 and 31 drafted), and 8 sequential passes of the 1-layer drafter, each waiting for
    the previous one -- the cost shape of a 1-layer drafter that proposes one token per pass.
    Those passes are 16-row passes: at batch 1 a pass streams the layer and LM-head weights
    whatever its row count, which the LM head timed alone at 1 and at 16 rows shows.
    Context K/V are seeded values (their content does not change the work)."""
    import torch

    from block_diffusion_drafter_hidden_amd import Drafter
    from workloads import scaled, synth

    depths = [1, 2, 3, 5, 8]
    dev = torch.device("cuda:0")
    T = int(synth.context_lengths(wl).max())
    cfg_max = scaled(wl.cfg, n_layers=max(depths))
    log(f"[latency] generating a {max(depths)}-layer {wl.cfg.name} drafter")
    w_all = synth.drafter_weights(cfg_max, seed=wl.seed)
    table, num_pages = synth.page_table(wl.name + "/latency", [T + 16], wl.cfg.page_size, wl.seed)
    anchors = torch.as_tensor(synth.anchor_ids(wl.cfg, 1, wl.seed)).to(dev)
    ids = torch.zeros((1, 15), dtype=torch.int32, device=dev)
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())

    def timed(fn, reps):
        with torch.cuda.stream(s):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            for _ in range(max(args.warmup, 3)):
                g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            for _ in range(reps):
                g.replay()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    from block_diffusion_drafter_hidden_amd import binding as B

    rows, ar_ms, lm_rows = [], None, {}
    for L in depths:
        cfg = scaled(wl.cfg, n_layers=L)
        keep = set(cfg.weight_shapes())
        wd = {k: v.to(dev) for k, v in w_all.items() if k in keep}
        dr = Drafter(cfg, wd, max_batch=1, max_ctx=table.shape[1] * cfg.page_size,
                     max_inject_rows=256, device=dev)
        del wd
        cache = dr.new_cache(table, [T], num_pages)
        gen = torch.Generator(device=dev).manual_seed(synth.stream_seed(wl.seed, "latency/fill"))
        for pool in (cache.k_pool, cache.v_pool):
            pool.normal_(0.0, 3.0, generator=gen)
        for nb in (8, 16, 32):
            d = dr if nb == cfg.block_size else dr.sibling(
                1, table.shape[1] * cfg.page_size, 256, block_size=nb)
            ids_nb = torch.zeros((1, nb - 1), dtype=torch.int32, device=dev)
            ms = timed(lambda: d.draft(cache, anchors, ids_nb), args.steps)
            rows.append({"layers": L, "block": nb, "ms_per_block": round(ms, 4),
                         "drafted_tokens_per_ms": round((nb - 1) / ms, 2)})
            log(f"[latency] {L} layers, block {nb}: {ms:.4f} ms per pass")
        if L == 1:
            def ar8():
                for _ in range(8):
                    dr.draft(cache, anchors, ids)
            ar_ms = timed(ar8, max(args.steps // 4, 5))
            log(f"[latency] 1 layer, 8 sequential passes: {ar_ms:.4f} ms")
            for r in (1, 16):   # the LM head alone at 1 and 16 rows
                y = torch.randn((r, cfg.hidden), device=dev, dtype=torch.float32)
                o = torch.empty(r, dtype=torch.int32, device=dev)
                lm_rows[f"lm_head_{r}_rows_ms"] = round(
                    timed(lambda: B.lm_head_argmax(dr.ccfg, dr.packed, y, o, dr.ws),
                          args.steps), 4)
        del dr, cache
        torch.cuda.empty_cache()
    five = next(r["ms_per_block"] for r in rows if r["layers"] == 5 and r["block"] == 16)
    out = {
        "metric": "draft latency: one block pass by drafter depth and block size vs 8 "
                  "sequential 1-layer passes (batch 1)",
        "value": round(five, 4), "unit": "ms per block (5 layers, 16 tokens)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "dtype": wl.cfg.dtype, "data": "synthetic (seeded weights, seeded context K/V)",
        "config": {"workload": f"{wl.cfg.name}-batch1-ctx{T}-depth-block-sweep",
                   "context": T},
        "rows": rows,
        "one_layer_8_sequential_passes_ms": round(ar_ms, 4),
        "five_layer_block16_vs_8_sequential_1_layer": round(five / ar_ms, 3),
        **lm_rows,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
