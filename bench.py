"""Benchmark of the canvas denoising hot path on one MI355X.

Prints one JSON line. A step is one dg_canvas_step: the decoder over the
256-token canvas (every layer: norm, QKV, RoPE, joint canvas+prefix
attention, output projection, router, expert permutation, grouped SwiGLU
experts, combine), the tied 262144-way LM head with the fused tempered
statistics, and the EB sampler (selection, Philox draws, re-mask, stop).
Canvases run back to back: every canvas starts all-MASK and, once finished,
is run through the encoder and appended to the KV cache (inside the timed
region when it falls there). Each step is a replay of the step captured as a
HIP graph (dg_step_graph; captured once per canvas, inside the timed region);
the host reads the canvas's done flag every 4 steps. `value` = timed steps /
timed wall time (HIP-synchronised). committed tokens/s = the 256 tokens of
one complete canvas, timed on its own after the timed steps (steps until the
device finishes it, argmax fill included, then the encoder append) / its
time. The per-kernel timing passes run eager steps of a fresh canvas with no
append among them. With one canvas, `diverse_canvas` times steps at the
headline state of the one-layer workload (128 positions committed to uniform
random ids, 128 MASK) through the whole stack.

Workloads (synthetic, seeded; random-init weights ~N(0, 0.02)):
  stack30   30 layers, d=2816, 16 q / 8 kv heads of 256, 128 experts top-8 +
            1 shared (F=704), Zipf(1.1) router bias, 262144 vocab, bf16,
            25 local (window 1024) + 5 global layers, 8192-token prompt
            prefilled by the encoder, 4 canvases of 256 (default)
  one_layer the same widths with 1 layer, 4096-token prompt
  longctx   the 30-layer stack with e4m3 expert and attention weights, a
            131072-token prompt prefilled by the encoder (untimed), then
            canvases as in stack30
  sampler   EB sampler only on bf16 logits [256][262144]
  tiny      2 layers, d=256, fp32, vocab 4096, canvas 32, 128-token prompt
  prefill   encoder prefill of a 131072-token prompt (--prefill-tokens) into
            an empty cache through the 30-layer stack with e4m3 expert and
            attention weights (the long-context geometry); a step is one
            whole prefill, value = prompt tokens/s
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "denoise steps/s and committed tokens/s, 256-token canvas, batch 1; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
SEED = 0x5EED


def _cores():
    try:
        import threadpoolctl
        n = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
        return int(n)
    except Exception:
        return len(os.sched_getaffinity(0))


def _sync_ms(fn, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


# --------------------------------------------------------------------------
# model workloads
# --------------------------------------------------------------------------

POLL_EVERY = 4      # timed loop: the host reads the done flag every this many steps
KERNELS = (("expert_gate_up", "TIME_EXPERT_GATE_UP"), ("expert_down", "TIME_EXPERT_DOWN"),
           ("qkv_proj", "TIME_QKV"), ("attention", "TIME_ATTENTION"), ("o_proj", "TIME_O_PROJ"),
           ("lm_head", "TIME_LM_HEAD"))
DIVERSE_COMMITTED = 128   # the headline canvas state of the one-layer workload: 128 committed, 128 MASK


def _kernel_record(cfg, name, tot_ms, launches, rec, nb, lm8):
    nbytes, flops = _algorithmic(cfg, name, rec, nb, lm8)
    return {"launches": launches, "ms_total": tot_ms, "bytes": nbytes, "flops": flops,
            "algorithmic_bytes_per_launch": round(nbytes / max(launches, 1)),
            "us_per_launch": round(tot_ms / max(launches, 1) * 1e3, 2),
            "ms_per_step": round(tot_ms / max(len(rec), 1), 4),
            "achieved_gbs": round(nbytes / (tot_ms * 1e-3) / 1e9, 1),
            "achieved_tflops": round(flops / (tot_ms * 1e-3) / 1e12, 1),
            "mean_experts_hit": round(sum(sum(h) for _, h in rec) / max(len(rec), 1) / cfg.n_layers, 2)}


def _model_workload(args, torch, B, cfg, prompt_len, n_canvases_cap):
    from synth import workloads as wl
    dev = torch.device("cuda:0")
    nb = args.batch
    t0 = time.perf_counter()
    embed = wl.embedding(cfg, device=dev)
    fnorm = wl.final_norm(cfg, device=dev)
    layers = [wl.layer_weights(cfg, l, device=dev) for l in range(cfg.n_layers)]
    lm8 = wl.lm_head_e4m3(cfg, device=dev) if args.fp8_lm_head else (None, None)
    model = B.Model(cfg, embed, fnorm, layers, max_canvas=cfg.canvas * nb, lm_head_e4m3=lm8[0], lm_head_scale=lm8[1])
    torch.cuda.synchronize()
    t_weights = time.perf_counter() - t0
    n = cfg.canvas
    steps_per_canvas = 48
    # canvases the run may finish: warmup + timed steps, the canvas timed on
    # its own, and one spare
    n_canv = -(-(args.warmup + args.steps) // steps_per_canvas) + 3
    kvs = [B.KVCache(model, prompt_len + n * n_canv) for _ in range(nb)]
    kv = kvs[0]
    ws = model.workspace(max(4096 if prompt_len > 8192 else 1024, n * nb))
    prompts = [wl.prefix_tokens(cfg, prompt_len, stream=b).to(dev) for b in range(nb)]
    ms_prefill = _sync_ms(lambda: [B.prefill_append(model, k, p, ws) for k, p in zip(kvs, prompts)], torch)
    canvases = [B.Canvas(n, cfg.mask_id, b, dev) for b in range(nb)]
    canvas = canvases[0]
    stats = B.StepStats(n * nb, device=dev, vocab=cfg.vocab, logits_dtype=model.act_dtype, n_layers=cfg.n_layers,
                        n_canvases=nb)
    scfg = B.sampler_default()
    scfg.draw_mode = B.DG_DRAW_GUMBEL_MAX if args.gumbel else B.DG_DRAW_INVERSE_CDF
    sched = {"t": 0, "canvas": 0, "committed": 0, "graph": None, "canvas_steps": 0}

    def all_done():
        if nb > 1:
            return bool(torch.stack([c.state[B.ST_DONE] for c in canvases]).all().item())
        return bool(canvas.state[B.ST_DONE].item())

    def finish_canvas():
        # the device finished the canvas (stop, last step or all committed,
        # with the argmax fill): the encoder appends it, the next one starts
        sched["canvas_steps"] += sched["t"]
        for c, k in zip(canvases, kvs):
            B.prefill_append(model, k, c.tokens, ws)
        sched["graph"] = None
        sched["committed"] += n * nb
        sched["canvas"] += 1
        sched["t"] = 0

    def run(K):
        # Steps of canvases run back to back. One canvas: each step is a
        # replay of the step captured as a HIP graph (captured once per
        # canvas: the KV length is part of the capture). Several canvases
        # step in lockstep, eagerly. The host reads the done flag every
        # POLL_EVERY steps and after the last step a canvas can take.
        for _ in range(K):
            if sched["t"] == 0:
                for b, c in enumerate(canvases):
                    c.canvas_idx = sched["canvas"] * nb + b
                    c.reset()
            if nb > 1:
                B.canvas_step_batch(model, canvases, kvs, sched["t"], SEED, scfg, stats, ws)
            else:
                if sched["graph"] is None:
                    sched["graph"] = B.StepGraph(model, canvas, kv, scfg, SEED, stats, ws)
                sched["graph"].launch()
            sched["t"] += 1
            if sched["t"] == scfg.max_steps or (sched["t"] % POLL_EVERY == 0 and all_done()):
                finish_canvas()

    def run_canvas():
        # one complete canvas from all-MASK: steps until the device marks it
        # finished, then the append
        assert sched["t"] == 0
        run(1)
        while sched["t"] != 0:
            run(1)

    run(args.warmup)
    if sched["t"]:
        while sched["t"]:                 # start the timed region on a fresh canvas
            run(1)
    ms = _sync_ms(lambda: run(args.steps), torch)
    # the tail of a canvas left unfinished by the timed steps is completed
    # (untimed), then one whole canvas is timed with its append: committed
    # tokens per second of generation
    while sched["t"]:
        run(1)
    c0, s0 = sched["committed"], sched["canvas_steps"]
    ms_canvas = _sync_ms(run_canvas, torch)
    canvas_tokens = sched["committed"] - c0
    canvas_steps = sched["canvas_steps"] - s0
    eb_per_step = None
    # per-kernel timing: eager steps of a fresh canvas (no append inside), HIP
    # events bracketing every launch of one kernel on the stream it runs on
    kernels = {}
    tsteps = min(args.steps, 16)
    for name, tgt in KERNELS:
        rec = []
        for c in canvases:
            c.reset()
        B.timing_enable(getattr(B, tgt))
        for t in range(tsteps):
            P = kv.length
            if nb > 1:
                B.canvas_step_batch(model, canvases, kvs, t, SEED, scfg, stats, ws)
            else:
                B.canvas_step(model, canvas, kv, t, SEED, scfg, stats, ws)
            rec.append((P, stats.experts_hit.cpu().tolist()))
        torch.cuda.synchronize()
        tot_ms, launches = B.timing_read()
        B.timing_enable(B.TIME_OFF)
        kernels[name] = _kernel_record(cfg, name, tot_ms, launches, rec, nb, args.fp8_lm_head)
    if nb == 1:
        eb_per_step = round(float(canvas.state[B.ST_COMMITTED].item()) / tsteps, 3) if tsteps < 48 else None
    # counter evidence (same kernel sources only): measured HBM bytes per
    # launch against the algorithmic ones, MFMA busy percentage
    ctr = _counters(args.workload) if nb == 1 and not args.fp8_lm_head else {}
    for name, k in kernels.items():
        c = ctr.get(name)
        per_launch = k["bytes"] / max(k["launches"], 1)
        k["counter_hbm_bytes"] = round(c["hbm_bytes"]) if c else None
        k["counter_vs_algorithmic"] = round(c["hbm_bytes"] / per_launch, 3) if c else None
        k["mfma_busy_pct"] = c["mfma_busy_pct"] if c else None
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    kd = kernels[dom]
    # the bound is the roof the kernel's algorithmic work reaches first: HBM
    # bytes at 8 TB/s or flops at the bf16 MFMA peak
    hbm_bound = kd["bytes"] / (HBM_PEAK_GBS * 1e9) >= kd["flops"] / (BF16_PEAK_TFLOPS * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": kd["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kd["achieved_gbs"] / HBM_PEAK_GBS, 4), "traffic": kd["counter_hbm_bytes"]}
    else:
        roof = {"bound": "mfma", "achieved": kd["achieved_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kd["achieved_tflops"] / BF16_PEAK_TFLOPS, 4), "traffic": kd["counter_hbm_bytes"]}
    res = {
        "ms_per_step": ms / args.steps,
        "committed_tokens_per_s": round(canvas_tokens / (ms_canvas * 1e-3), 2),
        "roofline": dict(roof, kernel=dom, us_per_launch=kd["us_per_launch"],
                         algorithmic_bytes_per_launch=round(kd["bytes"] / max(kd["launches"], 1)),
                         algorithmic_flops_per_launch=round(kd["flops"] / max(kd["launches"], 1)),
                         hbm_gbs=kd["achieved_gbs"], hbm_frac=round(kd["achieved_gbs"] / HBM_PEAK_GBS, 4),
                         mfma_tflops=kd["achieved_tflops"],
                         mfma_frac=round(kd["achieved_tflops"] / BF16_PEAK_TFLOPS, 4)),
        "kernels": {k: {kk: vv for kk, vv in v.items() if kk not in ("ms_total", "bytes", "flops")}
                    for k, v in kernels.items()},
        "extra": {"prefill_tokens": prompt_len, "prefill_ms": round(ms_prefill, 2),
                  "prefill_tokens_per_s": round(prompt_len / ms_prefill * 1e3, 1),
                  "canvas_ms": round(ms_canvas, 2), "canvas_steps": canvas_steps,
                  "canvas_tokens": canvas_tokens,
                  "committed_rate_from": "one complete canvas after the timed steps: graph replays until the "
                                         "device finished it (argmax fill included), then the encoder append",
                  "eb_commits_per_step": eb_per_step,
                  "poll_every": POLL_EVERY,
                  "weights_setup_s": round(t_weights, 1), "kv_len_end": kv.length},
        "dtype": cfg.act_dtype,
    }
    if nb == 1 and cfg.n_layers > 1 and not args.no_diverse:
        res["diverse_canvas"] = _diverse_canvas(args, torch, B, cfg, model, kv, ws, stats, scfg)
    return res, (model, kv, ws, canvas, stats)


def _diverse_canvas(args, torch, B, cfg, model, kv, ws, stats, scfg):
    """Steps at the one-layer workload's headline canvas state, through the
    whole stack: 128 positions committed to uniform random ids and 128 MASK
    (rows route to many more experts than on an all-MASK canvas). The state
    is restored before every step, so each timed step sees it."""
    from synth import workloads as wl
    n = cfg.canvas
    toks, com = wl.committed_canvas(cfg, DIVERSE_COMMITTED, device="cuda:0")
    c = B.Canvas(n, cfg.mask_id, 99, "cuda:0")
    T_STEP = 5

    def restore():
        c.tokens.copy_(toks)
        c.committed.copy_(com)
        c.state.zero_()
        c.state[B.ST_STEP] = T_STEP

    restore()
    graph = B.StepGraph(model, c, kv, scfg, SEED, stats, ws)
    K = max(4, min(args.steps, 16))
    for _ in range(2):
        restore()
        graph.launch()
    torch.cuda.synchronize()
    times = []
    for _ in range(K):
        restore()
        times.append(_sync_ms(graph.launch, torch))
    del graph
    kernels = {}
    hits = None
    ctr = _counters(args.workload + "_diverse") if not args.fp8_lm_head else {}
    for name, tgt in KERNELS:
        rec = []
        B.timing_enable(getattr(B, tgt))
        for _ in range(4):
            restore()
            B.canvas_step(model, c, kv, T_STEP, SEED, scfg, stats, ws)
            rec.append((kv.length, stats.experts_hit.cpu().tolist()))
        torch.cuda.synchronize()
        tot_ms, launches = B.timing_read()
        B.timing_enable(B.TIME_OFF)
        r = _kernel_record(cfg, name, tot_ms, launches, rec, 1, args.fp8_lm_head)
        cr = ctr.get(name)
        r["counter_hbm_bytes"] = round(cr["hbm_bytes"]) if cr else None
        r["counter_vs_algorithmic"] = round(cr["hbm_bytes"] / r["algorithmic_bytes_per_launch"], 3) if cr else None
        r["mfma_busy_pct"] = cr["mfma_busy_pct"] if cr else None
        kernels[name] = {kk: vv for kk, vv in r.items() if kk not in ("ms_total", "bytes", "flops")}
        hits = rec[-1][1]
    d, F = cfg.d_model, cfg.ffn_hidden
    wb = 1 if cfg.weight_dtype == "fp8" else 2
    expert_bytes = sum((h + 1) * 3 * F * d * wb for h in hits)
    ms_step = sorted(times)[len(times) // 2]
    return {"state": f"{DIVERSE_COMMITTED} of {n} positions committed to uniform random ids, the rest MASK; "
                     f"step index {T_STEP}; restored before each step",
            "ms_per_step": round(ms_step, 4), "steps_per_s": round(1e3 / ms_step, 2), "timed_steps": K,
            "experts_hit_per_layer": hits,
            "mean_experts_hit": round(sum(hits) / len(hits), 2),
            "expert_weight_bytes_per_step": expert_bytes,
            "expert_weight_gbs": round(expert_bytes / (ms_step * 1e-3) / 1e9, 1),
            "kernels": kernels}


def _algorithmic(cfg, name, rec, nbat=1, lm8=False):
    """Algorithmic HBM bytes and flops of every launch of kernel ``name`` over
    the recorded steps [(prefix length P, experts hit per layer)] of nbat
    canvases in lockstep (each with a cache of P rows): each weight byte of
    the experts actually hit once per step, activations in and out once."""
    n, d, F, k = cfg.canvas * nbat, cfg.d_model, cfg.ffn_hidden, cfg.top_k
    Hq, Hkv, hd, V, L = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.vocab, cfg.n_layers
    wb = 1 if cfg.weight_dtype == "fp8" else (4 if cfg.weight_dtype == "f32" else 2)
    ab = 4 if cfg.act_dtype == "f32" else 2
    nb = fl = 0.0
    for P, hits in rec:
        for l in range(L):
            h = hits[l]
            if name == "expert_gate_up":
                nb += (h + 1) * 2 * F * d * wb + n * d * ab + n * (k + 1) * F * ab
                fl += 2.0 * n * (k + 1) * 2 * F * d
            elif name == "expert_down":
                nb += (h + 1) * d * F * wb + n * (k + 1) * F * ab + n * (k + 1) * d * 4
                fl += 2.0 * n * (k + 1) * F * d
            elif name == "qkv_proj":
                nb += (Hq + 2 * Hkv) * hd * d * wb + n * d * ab + n * (Hq + 2 * Hkv) * hd * ab
                fl += 2.0 * n * (Hq + 2 * Hkv) * hd * d
            elif name == "o_proj":
                nb += d * Hq * hd * wb + n * Hq * hd * ab + 2 * n * d * 4
                fl += 2.0 * n * d * Hq * hd
            elif name == "attention":
                glob = cfg.global_every > 0 and l % cfg.global_every == cfg.global_every - 1
                keys = (P if glob else min(P, cfg.window)) + cfg.canvas      # per canvas
                nb += nbat * keys * Hkv * hd * 2 * ab + 2 * n * Hq * hd * ab
                fl += 4.0 * n * Hq * keys * hd
        if name == "lm_head":
            nb += V * d * (1 if lm8 else ab) + n * d * ab + n * V * ab
            fl += 2.0 * n * V * d
    return nb, fl


COUNTERS_FILE = {"stack30": "stack30_decode_counters.txt", "stack30_diverse": "stack30_diverse_counters.txt"}


def _counters(workload):
    """Per-kernel rocprofv3 counters of the denoising steps (HBM bytes read +
    written per launch, scaled by a copy of known size; MFMA busy percentage)
    from the summary committed under profiles/, if it was taken on the kernel
    sources as they are now; {} otherwise."""
    import hashlib
    name = COUNTERS_FILE.get(workload)
    path = os.path.join(ROOT, "profiles", name) if name else ""
    if not path or not os.path.exists(path):
        return {}
    kv, rows = {}, {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        a, b = line.split(":", 1)
        a, b = a.strip(), b.strip()
        if "=" in b:
            rows[a] = dict(x.split("=", 1) for x in b.split())
        else:
            kv[a] = b
    srcs = [x for x in kv.get("kernel_source", "").split(",") if x]
    hashes = kv.get("kernel_source_sha256", "").split(",")
    if not srcs or len(srcs) != len(hashes):
        return {}
    for src, h in zip(srcs, hashes):
        f = os.path.join(ROOT, src)
        if not os.path.isfile(f) or hashlib.sha256(open(f, "rb").read()).hexdigest() != h:
            return {}
    return {k: {"hbm_bytes": float(v["hbm_bytes"]), "mfma_busy_pct": float(v["mfma_busy_pct"])}
            for k, v in rows.items() if "hbm_bytes" in v}


def bench_stack(args, torch, B, which):
    from synth import workloads as wl
    cfg = {"stack30": wl.STACK30, "one_layer": wl.FULL_LAYER, "tiny": wl.TINY, "longctx": wl.STACK30_FP8}[which]
    plen = {"stack30": 8192, "one_layer": 4096, "tiny": wl.TINY_PREFIX, "longctx": 131072}[which]
    res, handles = _model_workload(args, torch, B, cfg, plen, 8)
    wname = (f"{cfg.name}_canvas{cfg.canvas}_prompt{plen}" + (f"_batch{args.batch}" if args.batch > 1 else "")
             + ("_e4m3head" if args.fp8_lm_head else "") + ("_gumbel" if args.gumbel else ""))
    res["config"] = {"workload": wname, "layers": cfg.n_layers,
                     "d_model": cfg.d_model, "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}",
                     "experts": f"{cfg.n_experts} top-{cfg.top_k} + 1 shared, F={cfg.ffn_hidden}",
                     "vocab": cfg.vocab, "canvas": cfg.canvas, "batch": args.batch, "window": cfg.window,
                     "global_every": cfg.global_every, "prompt": plen, "weights": cfg.weight_dtype,
                     "lm_head": "e4m3" if args.fp8_lm_head else cfg.act_dtype,
                     "draw": "gumbel_max" if args.gumbel else "inverse_cdf"}
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_model_step(cfg, handles, torch, B, plen, args.batch)
    return res


def _host_info():
    """CPU model and the BLAS numpy calls, for the oracle's timing record."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        import threadpoolctl
        libs = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer', '')}, "
                f"{i.get('num_threads')} threads)" for i in threadpoolctl.threadpool_info()
                if i.get("user_api") == "blas"]
        if libs:
            blas = "; ".join(libs)
    except Exception:
        pass
    return model, blas


def cpu_model_step(cfg, handles, torch, B, plen, nb=1):
    """The oracle on one local and one global decoder layer plus the LM head
    and one sampler step (float64 numpy), on the canvas state and KV the GPU
    run left, extrapolated to the stack's local and global layers (and to nb
    canvases: a batched step is nb canvas steps for the oracle)."""
    import numpy as np
    from oracle import model as M
    from oracle import sampler as S
    model, kv, ws, canvas, stats = handles
    P = kv.length
    n = cfg.canvas
    W = M.Weights(cfg, model.embed.cpu(), model.final_norm.cpu(),
                  lambda l: {k: v.cpu() for k, v in model.layers[l].items()})
    toks = canvas.tokens.cpu().numpy()
    X = W.E[toks].copy()

    def layer_time(l):
        Kl = kv.k[l][:, :P].float().cpu().numpy().astype(np.float64)
        Vl = kv.v[l][:, :, :P].transpose(1, 2).float().cpu().numpy().astype(np.float64)
        W.layer(l)
        t0 = time.perf_counter()
        out = M.decoder_layer(X, W.layer(l), Kl, Vl, l, cfg)
        return time.perf_counter() - t0, out

    t_local, X1 = layer_time(0)
    glob = [l for l in range(cfg.n_layers) if cfg.global_every > 0 and l % cfg.global_every == cfg.global_every - 1]
    t_global = layer_time(glob[0])[0] if glob else 0.0
    t0 = time.perf_counter()
    L = M.lm_logits(X1, W.final_norm, W.E, cfg.norm_eps)
    ocfg = S.SamplerConfig(mask_id=cfg.mask_id)
    st = S.CanvasState.fresh(n, cfg.mask_id)
    S.sampler_step(st, L, 0, ocfg, SEED)
    t_head = time.perf_counter() - t0
    n_glob = len(glob)
    step_s = (t_local * (cfg.n_layers - n_glob) + t_global * n_glob + t_head) * nb
    cpu, blas = _host_info()
    return {"value": round(1.0 / step_s, 5), "unit": "denoise steps/s", "cores": _cores(), "kind": "oracle",
            "sample": (f"1 local decoder layer ({t_local:.2f} s)"
                       + (f", 1 global layer over {P}+{n} keys ({t_global:.2f} s)" if n_glob else "")
                       + f", LM head and sampler ({t_head:.2f} s), float64 numpy, extrapolated to "
                       f"{cfg.n_layers - n_glob} local + {n_glob} global layers"
                       + (f" and {nb} canvases" if nb > 1 else "") + f"; canvas {n}, KV {P} rows"),
            "cpu": cpu, "blas": blas}


# --------------------------------------------------------------------------
# long-prompt encoder prefill
# --------------------------------------------------------------------------

PREFILL_CHUNK = 4096


def _prefill_algorithmic(cfg, n, name):
    """Algorithmic flops and HBM bytes of all launches of kernel ``name`` in
    one causal prefill of n tokens in PREFILL_CHUNK-row chunks. Attention
    counts only the keys each query sees (p + 1 on a global layer, at most the
    window on a local one); the last layer computes only its projections."""
    d, F, k = cfg.d_model, cfg.ffn_hidden, cfg.top_k
    Hq, Hkv, hd, L = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.n_layers
    wb = 1 if cfg.weight_dtype == "fp8" else 2
    ab = 2
    n_glob = sum(1 for l in range(L - 1) if cfg.global_every > 0 and l % cfg.global_every == cfg.global_every - 1)
    n_loc = L - 1 - n_glob
    fl = nb = 0.0
    for P in range(0, n, PREFILL_CHUNK):
        cn = min(PREFILL_CHUNK, n - P)
        if name == "qkv_proj":
            fl += L * 2.0 * cn * (Hq + 2 * Hkv) * hd * d
            nb += L * ((Hq + 2 * Hkv) * hd * d * wb + cn * d * ab + cn * (Hq + 2 * Hkv) * hd * ab)
        elif name == "attention":
            keys_glob = (P + 1 + P + cn) * cn / 2.0                     # sum of p + 1 over the chunk
            w = cfg.window
            keys_loc = sum(min(p + 1, w) for p in range(P, P + cn))
            fl += 4.0 * Hq * hd * (n_glob * keys_glob + n_loc * keys_loc)
            span_loc = P + cn - max(0, P - w + 1)                      # keys a local chunk reads
            nb += (n_glob * (P + cn) + n_loc * span_loc) * Hkv * hd * 2 * ab + (L - 1) * 2 * cn * Hq * hd * ab
        elif name == "o_proj":
            fl += (L - 1) * 2.0 * cn * d * Hq * hd
            nb += (L - 1) * (d * Hq * hd * wb + cn * Hq * hd * ab + 2 * cn * d * 4)
        elif name == "expert_gate_up":
            fl += (L - 1) * 2.0 * cn * (k + 1) * 2 * F * d
            nb += (L - 1) * ((cfg.n_experts + 1) * 2 * F * d * wb + cn * d * ab + cn * (k + 1) * F * ab)
        elif name == "expert_down":
            fl += (L - 1) * 2.0 * cn * (k + 1) * F * d
            nb += (L - 1) * ((cfg.n_experts + 1) * d * F * wb + cn * (k + 1) * F * ab + cn * (k + 1) * d * 4)
    return nb, fl


def bench_prefill(args, torch, B):
    from synth import workloads as wl
    cfg = wl.STACK30_FP8
    n = args.prefill_tokens
    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    embed = wl.embedding(cfg, device=dev)
    fnorm = wl.final_norm(cfg, device=dev)
    layers = [wl.layer_weights(cfg, l, device=dev) for l in range(cfg.n_layers)]
    model = B.Model(cfg, embed, fnorm, layers)
    torch.cuda.synchronize()
    t_weights = time.perf_counter() - t0
    kv = B.KVCache(model, n)
    ws = model.workspace(PREFILL_CHUNK)
    toks = wl.prefix_tokens(cfg, n).to(dev)

    def run(K):
        for _ in range(K):
            kv.length = 0
            B.prefill_append(model, kv, toks, ws)
            print(f"# prefill of {n} tokens enqueued", file=sys.stderr, flush=True)

    run(args.warmup)
    ms = _sync_ms(lambda: run(args.steps), torch)
    kernels = {}
    for name, target in (("attention", B.TIME_ATTENTION), ("expert_gate_up", B.TIME_EXPERT_GATE_UP),
                         ("expert_down", B.TIME_EXPERT_DOWN), ("qkv_proj", B.TIME_QKV),
                         ("o_proj", B.TIME_O_PROJ)):
        B.timing_enable(target)
        run(1)
        torch.cuda.synchronize()
        tot_ms, launches = B.timing_read()
        B.timing_enable(B.TIME_OFF)
        nbytes, flops = _prefill_algorithmic(cfg, n, name)
        kernels[name] = {"launches": launches, "ms_per_prefill": round(tot_ms, 2),
                         "us_per_launch": round(tot_ms / max(launches, 1) * 1e3, 2),
                         "achieved_tflops": round(flops / (tot_ms * 1e-3) / 1e12, 1),
                         "achieved_gbs": round(nbytes / (tot_ms * 1e-3) / 1e9, 1),
                         "flops_per_prefill": flops}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_prefill"])
    kd = kernels[dom]
    res = {
        "ms_per_step": ms / args.steps,
        "tokens_per_step": n,
        "roofline": {"bound": "mfma", "achieved": kd["achieved_tflops"], "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(kd["achieved_tflops"] / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": dom, "us_per_launch": kd["us_per_launch"],
                     "algorithmic_flops_per_launch": round(kd["flops_per_prefill"] / max(kd["launches"], 1))},
        "kernels": {k: {kk: vv for kk, vv in v.items() if kk != "flops_per_prefill"} for k, v in kernels.items()},
        "extra": {"weights_setup_s": round(t_weights, 1), "kv_len_end": kv.length, "chunk_rows": PREFILL_CHUNK},
        "config": {"workload": f"{cfg.name}_prefill{n}", "layers": cfg.n_layers, "d_model": cfg.d_model,
                   "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim}",
                   "experts": f"{cfg.n_experts} top-{cfg.top_k} + 1 shared, F={cfg.ffn_hidden}",
                   "weights": "e4m3 experts and projections, bf16 scales; MFMA in bf16",
                   "window": cfg.window, "global_every": cfg.global_every, "prompt": n, "batch": 1},
        "dtype": "bf16",
        "metric": "encoder prefill tokens/s, long prompt, batch 1; % MFMA peak",
        "unit": "prefill tokens/s",
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_prefill(cfg, model, n)
    return res


def cpu_prefill(cfg, model, n):
    """The oracle's causal encoder on a 1024-token prompt: layer 0 (local)
    complete and layer 1's projections, float64 numpy, scaled to the stack's
    layers. It leaves out the long-context attention of the global layers,
    which would only lower the oracle's rate."""
    from oracle import model as M
    from synth import workloads as wl
    cfg2 = cfg.replace(n_layers=2)
    W = M.Weights(cfg2, model.embed.cpu(), model.final_norm.cpu(),
                  lambda l: {k: v.cpu() for k, v in model.layers[l].items()})
    W.layer(0)
    W.layer(1)
    m = 1024
    toks = wl.prefix_tokens(cfg, m).numpy()
    kv = M.KVCache.empty(cfg2)
    t0 = time.perf_counter()
    M.encoder_append(W, kv, toks)
    t = time.perf_counter() - t0
    per_token_s = t / m * (cfg.n_layers - 1)
    return {"value": round(1.0 / per_token_s, 3), "unit": "prefill tokens/s", "cores": _cores(), "kind": "oracle",
            "sample": (f"encoder over {m} tokens: layer 0 complete plus layer 1 projections ({t:.2f} s), "
                       f"float64 numpy, scaled by {cfg.n_layers - 1} layers; global-layer long-context "
                       f"attention not included")}


# --------------------------------------------------------------------------
# sampler-only workload
# --------------------------------------------------------------------------

def bench_sampler(args, torch, B):
    from synth import workloads as wl
    n, V = wl.SAMPLER_ONLY_SHAPE
    mask = V - 1
    dev = torch.device("cuda:0")
    bufs = [wl.sampler_logits(t, device=dev) for t in range(4)]
    canvas = B.Canvas(n, mask, 0, dev)
    stats = B.StepStats(n, dev)
    ws = torch.empty(B.sampler_workspace_bytes(n, V), dtype=torch.uint8, device=dev)
    cfg = B.sampler_default()
    cfg.draw_mode = B.DG_DRAW_GUMBEL_MAX if args.gumbel else B.DG_DRAW_INVERSE_CDF

    def run(k0, K):
        for k in range(k0, k0 + K):
            t = k % 48
            if t == 0:
                canvas.reset()
            B.sampler_step(cfg, bufs[k % 4], mask, canvas, t, SEED, stats, ws)

    run(0, args.warmup)
    ms = _sync_ms(lambda: run(args.warmup, args.steps), torch)
    B.timing_enable(B.TIME_LM_HEAD)
    run(args.warmup + args.steps, args.steps)
    torch.cuda.synchronize()
    tot_ms, launches = B.timing_read()
    B.timing_enable(B.TIME_OFF)

    def whole_canvas():
        # steps from all-MASK until the device marks the canvas finished
        canvas.reset()
        for t in range(48):
            B.sampler_step(cfg, bufs[t % 4], mask, canvas, t, SEED, stats, ws)
            if t % POLL_EVERY == POLL_EVERY - 1 and canvas.state[B.ST_DONE].item():
                break
    ms_canvas = _sync_ms(whole_canvas, torch)
    canvas_steps = int(canvas.state[B.ST_STEP].item())
    bytes_per_launch = n * V * 2
    kern_ms = tot_ms / max(launches, 1)
    achieved = bytes_per_launch / (kern_ms * 1e-3) / 1e9
    res = {
        "ms_per_step": ms / args.steps,
        "committed_tokens_per_s": round(n / (ms_canvas * 1e-3), 2),
        "extra": {"canvas_ms": round(ms_canvas, 3), "canvas_steps": canvas_steps,
                  "committed_rate_from": "one complete canvas from all-MASK until the device finished it",
                  "poll_every": POLL_EVERY},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "logit_stats_kernel", "kernel_ms": round(kern_ms, 5),
                     "algorithmic_bytes_per_launch": bytes_per_launch},
        "config": {"workload": "sampler_only_256x262144_bf16" + ("_gumbel" if args.gumbel else ""), "canvas": n,
                   "vocab": V, "batch": 1, "draw": "gumbel_max" if args.gumbel else "inverse_cdf",
                   "logit_buffers": 4},
        "dtype": "bf16",
    }
    if not args.no_cpu:
        import numpy as np
        from oracle import sampler as S
        ocfg = S.SamplerConfig(mask_id=mask, draw_mode="gumbel_max" if args.gumbel else "inverse_cdf")
        Ls = [b.float().cpu().numpy() for b in bufs[:2]]
        st = S.CanvasState.fresh(n, mask)
        times = []
        t_end = time.perf_counter() + 12.0
        t = 0
        while time.perf_counter() < t_end or len(times) < 2:
            t0 = time.perf_counter()
            S.sampler_step(st, Ls[t % 2], t, ocfg, SEED)
            times.append(time.perf_counter() - t0)
            t += 1
            if st.done:
                st = S.CanvasState.fresh(n, mask)
                t = 0
        res["cpu_baseline"] = {"value": round(1.0 / float(np.median(times)), 4), "unit": "denoise steps/s",
                               "cores": _cores(), "kind": "oracle",
                               "sample": f"{len(times)} sampler steps (float64 numpy) on the same logits; median"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 96; prefill: 2)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 4; prefill: 1)")
    ap.add_argument("--workload", default="stack30", choices=["stack30", "one_layer", "sampler", "tiny", "prefill",
                                                                 "longctx"])
    ap.add_argument("--prefill-tokens", type=int, default=131072)
    ap.add_argument("--fp8-lm-head", action="store_true",
                    help="the LM head reads an e4m3 copy of the tied matrix (model workloads)")
    ap.add_argument("--gumbel", action="store_true", help="Gumbel-max draws fused into the statistics pass")
    ap.add_argument("--batch", type=int, default=1,
                    help="canvases of different users stepped together (model workloads; 256 x batch <= 1024)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-diverse", action="store_true",
                    help="skip the steps at the 128-committed canvas state (model workloads)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="finish with device copies of BYTES bytes (scale for HBM traffic counters)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 2 if args.workload == "prefill" else 96
    if args.warmup is None:
        args.warmup = 1 if args.workload == "prefill" else 4
    if (args.batch != 1 or args.fp8_lm_head) and args.workload in ("sampler", "prefill", "tiny"):
        ap.error("--batch and --fp8-lm-head apply to the bf16 model workloads")
    if args.gumbel and (args.batch != 1 or args.workload in ("prefill", "tiny")):
        ap.error("--gumbel applies to single-canvas bf16 steps and the sampler workload")
    if args.gpus != 1:
        print("bench.py measures one GPU: the denoising step here is built for a single MI355X "
              "and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from discrete_text_diffusion_canvas_amd import binding as B
    if args.workload == "sampler":
        res = bench_sampler(args, torch, B)
    elif args.workload == "prefill":
        res = bench_prefill(args, torch, B)
    else:
        res = bench_stack(args, torch, B, args.workload)
    ms = res.pop("ms_per_step")
    committed_rate = res.pop("committed_tokens_per_s", None)
    per_step = res.pop("tokens_per_step", 1)
    out = {
        "metric": res.pop("metric", METRIC),
        "value": round(per_step * 1e3 / ms, 3),
        "unit": res.pop("unit", "denoise steps/s"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.pop("dtype"),
        "data": "synthetic",
        "config": res.pop("config"),
        "roofline": res.pop("roofline"),
    }
    if committed_rate is not None:
        out = dict(list(out.items())[:7] + [("committed_tokens_per_s", committed_rate)] + list(out.items())[7:])
    for k in ("cpu_baseline", "kernels", "diverse_canvas", "extra"):
        if k in res:
            out[k] = res.pop(k)
    if args.copy_calibration > 0:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["extra"] = dict(out.get("extra", {}), copy_calibration_bytes=args.copy_calibration)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
