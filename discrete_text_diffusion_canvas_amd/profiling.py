"""Summaries of rocprofv3 output for the measurement record (plain text).

    python -m discrete_text_diffusion_canvas_amd.profiling stats DIR --command "..."
        DIR holds a `rocprofv3 --kernel-trace --stats` run; prints the per-kernel
        table (calls, average and total duration) of its *_kernel_stats.csv.

    python -m discrete_text_diffusion_canvas_amd.profiling steps DB --command "..."
        DB is the rocpd database (*_results.db) of a `rocprofv3 --kernel-trace`
        run of bench.py; prints the kernels of the denoising steps (everything
        after the first canvas reset) per step: time, calls, average duration,
        and the attention / GEMM launches split by grid shape.

    python -m discrete_text_diffusion_canvas_amd.profiling traffic \\
        --fetch F.csv --write W.csv --kernels REGEX --label NAME \\
        --copy-bytes B --sources a.hip,b.hip --command "..."
        F/W are `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` counter
        collections of one run that also made a device copy of B bytes. The
        counters of the kernels matching REGEX are averaged per dispatch and
        summed over the kernels (one logical launch may be several dispatches);
        each counter is scaled by B / (the counter on the copy), which turns the
        KiB the counters report into bytes the copy is known to move. With
        --after REGEX, dispatches before the first one of a kernel matching
        REGEX are left out (the prompt prefill runs other shapes). The
        output records the SHA-256 of the kernel sources, so a reader can tell
        whether the kernel changed since.

    python -m discrete_text_diffusion_canvas_amd.profiling drive \
        [--workload stack30|longctx] [--steps K] [--committed C] [--copy-bytes B]
        A short GPU run for counter collection: builds the workload, prefills
        the prompt, then K denoising steps (graph replays) of one canvas from
        its first step (or from a canvas with C committed positions, restored
        before each step), no append; then a device copy of B bytes.

    python -m discrete_text_diffusion_canvas_amd.profiling counters \
        --fetch F.csv --write W.csv --mfma M.csv --copy-bytes B --command "..."
        F, W, M: `rocprofv3 --pmc FETCH_SIZE`, `--pmc WRITE_SIZE` and
        `--pmc MfmaUtil MfmaFlopsBF16` collections of the same `drive` run.
        Per hot kernel of the denoising steps (each a fixed set of dispatches
        per layer or per step), the HBM bytes read and written per launch
        (counters scaled by the calibration copy), the MFMA flops per launch
        and the MFMA-busy fraction (time-weighted over its dispatches). The
        output records the SHA-256 of every kernel source.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys


def _name(row: dict) -> str:
    n = row.get("Kernel_Name") or row.get("Kernel-Name") or row.get("Name") or ""
    return re.sub(r"\(.*", "", n).replace("void ", "").strip()


def stats(args) -> None:
    files = glob.glob(os.path.join(args.dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        sys.exit(f"no *kernel_stats.csv under {args.dir}")
    rows = [r for r in csv.DictReader(open(files[0])) if re.search(args.filter, _name(r))]
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    print(f"# rocprofv3 kernel statistics ({os.path.basename(files[0])})")
    print(f"# command: {args.command}")
    if args.filter:
        print(f"# kernels matching {args.filter!r} only")
    print(f"# total kernel time {total / 1e6:.2f} ms over {sum(int(r['Calls']) for r in rows)} dispatches")
    print(f"{'calls':>7} {'avg_us':>10} {'total_ms':>10} {'pct':>6}  kernel")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows[: args.top]:
        print(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['TotalDurationNs']) / 1e6:10.3f} "
              f"{100 * float(r['TotalDurationNs']) / total:6.2f}  {_name(r)[:90]}")


def steps(args) -> None:
    import collections
    import sqlite3
    db = sqlite3.connect(args.db)
    cols = [r[1] for r in db.execute("pragma table_info(kernels)")]
    gz = "grid_z" if "grid_z" in cols else "grid_x"
    rows = list(db.execute(f"select name, start, end, duration, grid_x, {gz} from kernels order by start"))
    i0 = next(i for i, r in enumerate(rows) if "canvas_reset_kernel" in r[0])
    dec = rows[i0 + 1:]
    nsteps = max(1, sum(1 for r in dec if "eb_select_kernel" in r[0]))  # one sampler selection per step
    agg = collections.OrderedDict()
    shp = collections.OrderedDict()
    for r in dec:
        n = _name({"Name": r[0]}).replace("dg::", "")
        a = agg.setdefault(n, [0, 0.0])
        a[0] += 1
        a[1] += r[3]
        if re.search(r"attn|gemm_kernel|lmhead|reduce", n):
            b = shp.setdefault((n, r[4], r[5]), [0, 0.0])
            b[0] += 1
            b[1] += r[3]
    tot = sum(a[1] for a in agg.values())
    wall = dec[-1][2] - dec[0][1]
    print("# kernels of the denoising steps (rocprofv3 kernel trace)")
    print(f"# command: {args.command}")
    print(f"# steps: {nsteps}; kernel time per step {tot / nsteps / 1e6:.3f} ms; wall per step {wall / nsteps / 1e6:.3f} ms; "
          f"launches per step {sum(a[0] for a in agg.values()) / nsteps:.0f}")
    print(f"{'ms/step':>8} {'pct':>6} {'calls/step':>10} {'avg_us':>9}  kernel")
    for n, (c, t) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"{t / nsteps / 1e6:8.3f} {100 * t / tot:6.1f} {c / nsteps:10.1f} {t / c / 1e3:9.1f}  {n[:80]}")
    print("# by grid shape (grid x in threads, z = KV splits for attention)")
    for (n, gx, gzv), (c, t) in sorted(shp.items(), key=lambda kv: -kv[1][1]):
        print(f"  {n[:46]:46s} grid=({gx},{gzv}) calls/step={c / nsteps:6.1f} avg={t / c / 1e3:8.1f} us")


def _per_dispatch(path: str, counter: str, regex: str, after: str = "") -> dict:
    rows = [r for r in csv.DictReader(open(path)) if r.get("Counter_Name") == counter]
    first = 0
    if after:  # only dispatches from the first one of a kernel matching `after` on
        ids = [int(r["Dispatch_Id"]) for r in rows if re.search(after, _name(r))]
        first = min(ids) if ids else 0
    vals: dict = {}
    for r in rows:
        n = _name(r)
        if re.search(regex, n) and int(r.get("Dispatch_Id", 0)) >= first:
            vals.setdefault(n, []).append(float(r["Counter_Value"]))
    return vals


def traffic(args) -> None:
    out = {}
    for which, path, counter in (("fetch", args.fetch, "FETCH_SIZE"), ("write", args.write, "WRITE_SIZE")):
        kern = _per_dispatch(path, counter, args.kernels, args.after)
        copy = _per_dispatch(path, counter, args.copy_kernel)
        if not kern or not copy:
            sys.exit(f"{which}: no dispatches matched ({args.kernels!r} / {args.copy_kernel!r})")
        # the copy: its largest dispatch is the calibration copy
        cal = max(max(v) for v in copy.values())
        scale = args.copy_bytes / cal
        # the last dispatches of a run are decode steps (the prompt prefill comes first)
        per = {n: statistics.median(v[-args.last:]) for n, v in kern.items()}
        out[which] = (per, cal, scale)
    print(f"# HBM traffic of one launch of {args.label} (rocprofv3 FETCH_SIZE / WRITE_SIZE, KiB per dispatch,")
    print("# median over the last decode-step dispatches, scaled by a device copy of known size)")
    print(f"# command: {args.command}")
    srcs = [s for s in args.sources.split(",") if s]
    print(f"kernel: {args.label}")
    print(f"kernel_source: {','.join(srcs)}")
    print("kernel_source_sha256: " + ",".join(hashlib.sha256(open(s, 'rb').read()).hexdigest() for s in srcs))
    total = 0.0
    for which in ("fetch", "write"):
        per, cal, scale = out[which]
        print(f"{which}_copy_counter_kib: {cal:.1f}  ({args.copy_bytes} bytes -> scale {scale:.2f} bytes per unit)")
        for n, v in sorted(per.items()):
            print(f"{which}_{n}: {v:.1f} units -> {v * scale / 1e6:.2f} MB")
        total += sum(per.values()) * scale
    print(f"hbm_bytes_per_launch: {total:.0f}")


# kernels of one decoder layer / one step, by dispatch name (template
# instance); the router and the small-group expert down product are the same
# instance and are told apart by the dispatch that follows (the router's top-k)
HOT_KERNELS = {
    "lm_head": [r"^dg::lmhead_kernel<"],
    "attention": [r"^dg::attn_t_kernel<", r"^dg::attn_merge_kernel<"],
    "qkv_proj": [r"^dg::tile_gemm_kernel<128, 1, "],
    "o_proj": [r"^dg::tile_gemm_kernel<128, 2, "],
    "expert_gate_up": [r"^dg::stream_gemm_kernel<unsigned short, 0, 3>", r"^dg::tile_gemm_kernel<128, 3, ",
                       r"^dg::tile_swiglu_reduce_kernel"],
    "expert_down": [r"^dg::stream_gemm_kernel<unsigned short, 0, 0>#down", r"^dg::tile_gemm_kernel<128, 0, "],
    "router": [r"^dg::stream_gemm_kernel<unsigned short, 0, 0>#router"],
}
SOURCES = ["discrete_text_diffusion_canvas_amd/csrc/" + f for f in
           ("lmhead.hip", "attention.hip", "gemm_tile.hip", "gemm_stream.hip", "layer.hip", "sampler.hip")]


def _decode_dispatches(path: str, counters) -> list:
    """[(dispatch id, name, {counter: value})] of the denoising steps (from
    the first canvas reset on), the router's stream GEMM tagged #router."""
    by_id: dict = {}
    for r in csv.DictReader(open(path)):
        d = by_id.setdefault(int(r["Dispatch_Id"]), [_name(r), {}])
        if r.get("Counter_Name") in counters:
            d[1][r["Counter_Name"]] = d[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    ids = sorted(by_id)
    i0 = next((i for i, k in enumerate(ids) if "canvas_reset_kernel" in by_id[k][0]), 0)
    out = []
    ids = ids[i0:]
    for j, k in enumerate(ids):
        n, vals = by_id[k]
        if n.startswith("dg::stream_gemm_kernel<unsigned short, 0, 0>"):
            nxt = by_id[ids[j + 1]][0] if j + 1 < len(ids) else ""
            n += "#router" if "router_topk" in nxt else "#down"
        out.append((k, n, vals))
    return out


def _copy_scale(path: str, counter: str, copy_regex: str, copy_bytes: float) -> float:
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if r.get("Counter_Name") == counter and re.search(copy_regex, _name(r))]
    if not vals:
        sys.exit(f"{path}: no calibration copy matched {copy_regex!r}")
    return copy_bytes / max(vals)


def counters(args) -> None:
    fetch = _decode_dispatches(args.fetch, ("FETCH_SIZE",))
    write = _decode_dispatches(args.write, ("WRITE_SIZE",))
    mfma = _decode_dispatches(args.mfma, ("MfmaUtil", "MfmaFlopsBF16"))
    fs = _copy_scale(args.fetch, "FETCH_SIZE", args.copy_kernel, args.copy_bytes)
    ws = _copy_scale(args.write, "WRITE_SIZE", args.copy_kernel, args.copy_bytes)
    steps = sum(1 for _, n, _ in mfma if n.startswith("dg::lmhead_kernel<"))
    layer_steps = sum(1 for _, n, _ in mfma if n.startswith("dg::attn_t_kernel<"))
    if not steps or not layer_steps:
        sys.exit("no LM-head / attention dispatches in the denoising steps")
    print("# rocprofv3 counters of the hot kernels, per launch (one launch = the dispatches of one layer,")
    print("# or of one step for the LM head), over the denoising steps of the run")
    print(f"# command: {args.command}")
    print(f"# steps: {steps}; layer launches: {layer_steps}")
    print("kernel_source: " + ",".join(SOURCES))
    print("kernel_source_sha256: " + ",".join(hashlib.sha256(open(x, 'rb').read()).hexdigest() for x in SOURCES))
    print(f"fetch_scale_bytes_per_unit: {fs:.2f}")
    print(f"write_scale_bytes_per_unit: {ws:.2f}")
    for label, pats in HOT_KERNELS.items():
        launches = steps if label == "lm_head" else layer_steps

        def pick(rows):
            return [(n, v) for _, n, v in rows if any(re.search(p, n) for p in pats)]
        f = sum(v.get("FETCH_SIZE", 0.0) for _, v in pick(fetch)) * fs / launches
        w = sum(v.get("WRITE_SIZE", 0.0) for _, v in pick(write)) * ws / launches
        m = pick(mfma)
        flops = sum(v.get("MfmaFlopsBF16", 0.0) for _, v in m) / launches
        # busy fraction weighted by dispatch count (each dispatch reports its own)
        util = statistics.fmean([v["MfmaUtil"] for _, v in m if "MfmaUtil" in v]) if m else 0.0
        print(f"{label}: fetch_bytes={f:.0f} write_bytes={w:.0f} hbm_bytes={f + w:.0f} "
              f"mfma_flops={flops:.4g} mfma_busy_pct={util:.2f} dispatches={len(m)}")


def drive(args) -> None:
    import time

    import torch

    from discrete_text_diffusion_canvas_amd import binding as B
    from synth import workloads as wl
    cfg = {"stack30": wl.STACK30, "longctx": wl.STACK30_FP8}[args.workload]
    plen = {"stack30": 8192, "longctx": 131072}[args.workload]
    dev = torch.device("cuda:0")
    layers = [wl.layer_weights(cfg, l, device=dev) for l in range(cfg.n_layers)]
    model = B.Model(cfg, wl.embedding(cfg, device=dev), wl.final_norm(cfg, device=dev), layers)
    kv = B.KVCache(model, plen + cfg.canvas)
    ws = model.workspace(4096 if plen > 8192 else 1024)
    B.prefill_append(model, kv, wl.prefix_tokens(cfg, plen).to(dev), ws)
    torch.cuda.synchronize()
    print(f"# prefill of {plen} tokens done", flush=True)
    canvas = B.Canvas(cfg.canvas, cfg.mask_id, 0, dev)
    stats = B.StepStats(cfg.canvas, device=dev, vocab=cfg.vocab, logits_dtype=model.act_dtype,
                        n_layers=cfg.n_layers)
    canvas.reset()
    toks = com = None
    if args.committed:
        toks, com = wl.committed_canvas(cfg, args.committed, device=dev)
    graph = None
    t0 = time.perf_counter()
    for t in range(args.steps):
        if toks is not None:
            canvas.tokens.copy_(toks)
            canvas.committed.copy_(com)
            canvas.state.zero_()
            canvas.state[B.ST_STEP] = 5
        if graph is None:
            graph = B.StepGraph(model, canvas, kv, B.sampler_default(), 0x5EED, stats, ws)
        graph.launch()
    torch.cuda.synchronize()
    print(f"# {args.steps} steps in {time.perf_counter() - t0:.2f} s; experts hit per layer "
          f"{stats.experts_hit.cpu().tolist()}", flush=True)
    if args.copy_bytes:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--top", type=int, default=30)
    a.add_argument("--command", default="")
    a.add_argument("--filter", default="", help="only kernels whose name matches this regex")
    c = sub.add_parser("steps")
    c.add_argument("db")
    c.add_argument("--command", default="")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernels", required=True)
    b.add_argument("--copy-kernel", default=r"copyBuffer|copy_kernel|CopyKernel|elementwise")
    b.add_argument("--copy-bytes", type=float, required=True)
    b.add_argument("--label", required=True)
    b.add_argument("--sources", default="")
    b.add_argument("--command", default="")
    b.add_argument("--last", type=int, default=30, help="dispatches per kernel at the end of the run to use")
    b.add_argument("--after", default="", help="ignore dispatches before the first of a kernel matching this regex "
                   "(e.g. one that only the decode steps launch, to leave out the prompt prefill)")
    d = sub.add_parser("counters")
    d.add_argument("--fetch", required=True)
    d.add_argument("--write", required=True)
    d.add_argument("--mfma", required=True)
    d.add_argument("--copy-kernel", default=r"copyBuffer|copy_kernel|CopyKernel|elementwise")
    d.add_argument("--copy-bytes", type=float, required=True)
    d.add_argument("--command", default="")
    e = sub.add_parser("drive")
    e.add_argument("--workload", default="stack30", choices=["stack30", "longctx"])
    e.add_argument("--steps", type=int, default=4)
    e.add_argument("--committed", type=int, default=0)
    e.add_argument("--copy-bytes", type=int, default=1 << 30)
    args = ap.parse_args(argv)
    {"stats": stats, "steps": steps, "traffic": traffic, "counters": counters, "drive": drive}[args.cmd](args)


if __name__ == "__main__":
    main()
