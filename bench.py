"""Throughput of the layer-streamed training step on one MI355X.

Workload (default): the 14B-shaped decoder -- 48 layers, d_model 5120, 40
query / 8 kv heads (head_dim 128), SwiGLU FFN 13824, vocab 152064 -- batch
1 x 4096 uniform-random token ids with next-token targets, weights N(0, 0.02)
(norm gains 1) from seed 0, bf16 matrix-core compute with fp32 master weights
and AdamW state in host memory, streamed through two device layer buffers.

A step is one full mt_train_step: forward, head, recompute + backward, every
gradient copied to the host and every AdamW update applied. Inputs (token ids)
are generated before the timed region; the timed region is K steps bracketed
by device synchronisation. Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2.5e15        # dense bf16 matrix-core FLOP/s (MI355X)
PEAK_FP32 = 157.3e12      # dense fp32 matrix-core FLOP/s
PEAK_HBM = 8.0e12         # bytes/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_context(w, dtype, seed, flags, host_threads=0, chunk_rows=0, ckpt_host=0, buffers=2, micro_batches=0):
    from host_memory_streamed_amd import mt, synth
    cfg = mt.make_config(w.n_layers, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_dim, w.vocab,
                         w.batch, w.seq, dtype=dtype, n_layer_buffers=buffers,
                         host_threads=host_threads,
                         flags=flags, chunk_rows=chunk_rows, ckpt_host=ckpt_host, micro_batches=micro_batches)
    t0 = time.perf_counter()
    ctx = mt.Context(cfg)
    log(f"context created in {time.perf_counter() - t0:.1f}s; device bytes {ctx.device_bytes() / 1e9:.2f} GB; "
        f"{ctx.layout_info()}")
    t0 = time.perf_counter()
    biggest = max(int(np.prod(s)) for _, s in ctx.table)
    buf = np.empty(biggest, dtype=np.float32)
    for i, (name, shape) in enumerate(ctx.table):
        n = int(np.prod(shape))
        view = buf[:n]
        synth.init_tensor(seed, i, (n,), name.endswith("norm"), out=view)
        ctx.set_param(i, view)
    log(f"parameters drawn and loaded in {time.perf_counter() - t0:.1f}s")
    return ctx


def recorded_traffic(kernel_class):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary, if it covers this kernel class and the kernel's
    source has not changed since the counters were taken; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemm_nt_bf16_14b_traffic.md")
    src = os.path.join(ROOT, "host_memory_streamed_amd", "csrc", "gemm.hip")
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith(("|", "#", "`")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if kv.get("kernel_class") == kernel_class and kv.get("gemm_source_sha256_16") == digest:
            return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        pass
    return None


def link_probe(mib=1024, reps=3):
    """Plain pinned-host <-> device copies of `mib` MiB, each direction alone
    (HIP events on a side stream): the host link's per-direction rate on this
    box, the bandwidth the step's link bound is priced at."""
    import torch
    n = mib << 18   # fp32 elements
    dev = torch.empty(n, device="cuda")
    host = torch.empty(n, pin_memory=True)
    s = torch.cuda.Stream()
    out = {}
    for name, dst, src in (("h2d", dev, host), ("d2h", host, dev)):
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s):
                e0.record(s)
                dst.copy_(src, non_blocking=True)
                e1.record(s)
            e1.synchronize()
            best = max(best, n * 4 / (e0.elapsed_time(e1) * 1e-3))
        out[name] = best
    del dev, host
    torch.cuda.synchronize()
    return out


def fit_layers(w, dtype, flags, share=0.85, device_free=None):
    """The most layers of w (at most its own count) whose host store, as the
    library sizes it, takes at most `share` of the memory available now.
    Residual checkpoints that would not fit in device memory are parked in
    host memory (one pageable slab each, plus two pinned bounce slabs): they
    count too, estimating that the layer workspace leaves 70% of the free
    device memory to checkpoint slots."""
    from host_memory_streamed_amd import mt
    avail = None
    with open("/proc/meminfo") as f:
        for line in f:
            if line.startswith("MemAvailable:"):
                avail = int(line.split()[1]) * 1024
    if avail is None:
        return w.n_layers
    best = 0
    for L in range(1, w.n_layers + 1):
        cfg = mt.make_config(L, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_dim, w.vocab,
                             w.batch, w.seq, dtype=dtype, flags=flags)
        hb = mt.host_bytes(cfg)
        parked = 0
        if device_free:
            # the library keeps as many checkpoint slots on the device as fit
            # next to its fixed part (1 GiB margin) and parks the rest, each
            # in a host slab, through two pinned bounce slabs
            plan = mt.device_plan(cfg)
            slot = plan["ckpt_slot"]
            fit = (device_free - (1 << 30) - plan["fixed"]) // slot
            if fit < L + 1:
                if L < 3 or fit < 2:
                    break
                parked = (L - fit + 2) * slot
        if hb["pinned"] + hb["pageable"] + parked > share * avail:
            break
        best = L
    return max(best, 1)


def host_probe(n=1 << 28, reps=3):
    """The library's own host AdamW (the step's pool size) over n parameters
    with a bf16 image, alone: the rate of host-memory traffic the box sustains
    for it, 30 bytes per parameter (read p, m, v, g; write p, m, v, image)."""
    from host_memory_streamed_amd import mt
    p, m, v, g = (np.full(n, x, np.float32) for x in (0.01, 0.0, 0.0, 1e-3))
    img = np.zeros(n, np.uint16)
    best = 0.0
    for t in range(1, reps + 1):
        t0 = time.perf_counter()
        mt.adamw_host(p, m, v, g, t, 1e-4, 0.9, 0.999, 1e-8, 0.01, bf16_out=img)
        best = max(best, 30.0 * n / (time.perf_counter() - t0))
    return best


def link_roofline(w, stats, step_s, bw, wbytes):
    """The step's host-link bound from the bytes the step moves in each phase.
    Forward phase: every unit image in, plus x0 and the targets. Backward
    phase: L-1 layer images in (layer L-1 is still resident at the turn)
    against every gradient, x0's gradient and the losses out. Phase-aware:
    the phases run one after the other (no gradient exists before the turn);
    duplex: both directions busy the whole step."""
    d, L, M = w.d_model, w.n_layers, w.batch * w.seq
    qkv = (w.n_heads + 2 * w.n_kv_heads) * w.head_dim
    layer_img = 2 * d * 4 + (qkv * d + d * w.n_heads * w.head_dim + 3 * d * w.ffn_dim) * wbytes
    h2d, d2h = stats["h2d_bytes"], stats["d2h_bytes"]
    b_in = (L - 1) * layer_img
    f = h2d - b_in
    t_phase = f / bw["h2d"] + max(b_in / bw["h2d"], d2h / bw["d2h"])
    t_dup = max(h2d / bw["h2d"], d2h / bw["d2h"])
    return {
        "bw_h2d_GBps": round(bw["h2d"] / 1e9, 2), "bw_d2h_GBps": round(bw["d2h"] / 1e9, 2),
        "fwd_h2d_bytes": f, "bwd_h2d_bytes": b_in, "d2h_bytes": d2h,
        "t_link_phase_s": round(t_phase, 4), "t_link_duplex_s": round(t_dup, 4),
        "tokens_s_phase": round(M / t_phase, 1),
        "frac_phase": round(t_phase / step_s, 4), "frac_duplex": round(t_dup / step_s, 4),
    }


def cpu_baseline(w, vocab_share=8):
    """The CPU oracle (plain float64 NumPy, as it stands) timed on a bounded
    sample of the same workload: one decoder layer of the real shape forward
    and backward on the workload's own 1 x T tokens, the head on the same
    tokens over 1/vocab_share of the vocabulary (its products and its
    cross-entropy are linear in the vocabulary size), and AdamW on 16M
    elements; composed into a full-depth step and reported as tokens/s."""
    import oracle as O
    from oracle.decoder import _Prec, _threads
    from host_memory_streamed_amd import synth

    Vs = max(2, w.vocab // vocab_share)
    cfg = O.Config(1, w.d_model, w.n_heads, w.n_kv_heads, w.head_dim, w.ffn_dim, Vs)
    table = O.tensor_table(cfg)
    params = [synth.init_tensor(0, i, s, g) for i, (_, s, g) in enumerate(table)]
    P = [p.astype(np.float64) for p in params]
    B, T = 1, w.seq
    tokens, targets = synth.token_batch(0, B, T, Vs)
    prec = _Prec("bf16")
    rope = O.rope_tables(T, cfg.head_dim, cfg.rope_base)
    W = {n: P[1 + i] for i, n in enumerate(O.LAYER_TENSORS)}
    x = P[0][tokens.reshape(-1)]
    t0 = time.perf_counter()
    y, cache = O.layer_fwd(x, W, cfg, prec, rope, B, T)
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    _, g, _, _ = O.head_fwd_bwd(y, P[-2], P[-1], targets.reshape(-1), cfg, prec)
    t_head = (time.perf_counter() - t0) * (w.vocab / Vs)
    t0 = time.perf_counter()
    O.layer_bwd(g, cache, W, cfg, prec, rope, B, T)
    t_bwd = time.perf_counter() - t0
    n = 1 << 24
    rng = np.random.default_rng(0)
    pa, ga = rng.standard_normal(n), rng.standard_normal(n)
    t0 = time.perf_counter()
    O.adamw(pa, ga, np.zeros(n), np.zeros(n), 1, cfg)
    t_adam = (time.perf_counter() - t0) / n
    layer_params = sum(int(np.prod(s)) for _, s, _ in table[1:10])
    total_params = w.n_layers * layer_params + 2 * w.vocab * w.d_model + w.d_model
    step = w.n_layers * (t_fwd + t_bwd) + t_head + total_params * t_adam
    blas = None
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info())
    except Exception:
        pass
    heads = _threads()
    return {
        "value": round(B * T / step, 4),
        "unit": "tokens/s",
        "cores": int(max(blas or 1, heads)),
        "kind": "oracle",
        "os_cpu_count": os.cpu_count(),
        "blas_threads": blas,
        "attention_threads": heads,
        "sample": (f"float64 NumPy oracle, bf16 cast emulation, on the {w.name} shape at its own "
                   f"{B}x{T} tokens: one decoder layer forward ({t_fwd:.2f}s) and backward ({t_bwd:.2f}s); "
                   f"the head forward+backward over {Vs} of the {w.vocab} vocabulary rows, scaled by "
                   f"{w.vocab / Vs:.2f} to {t_head:.2f}s; AdamW {t_adam * 1e9:.2f} ns/param on 16M params; "
                   f"composed as {w.n_layers} x (fwd + bwd) + head + AdamW over {total_params / 1e9:.2f}B "
                   f"params = {step:.1f}s per {B * T}-token step"),
    }


def summarize_kernel_trace(path, steps, skip, kernel_substr, flops_per_launch=None):
    """Per-dispatch durations of one kernel from a rocprofv3 kernel trace
    (its kernel_trace.csv): the dispatches of the last steps - skip steps
    (the kernel's launches split evenly over the traced steps, in start
    order), all of them and those that overlap no runtime copy kernel
    (under kernel tracing the runtime runs each device-to-host copy as a
    blit kernel, and a dispatch that overlaps one waits for compute units).
    Copies overlap some shapes more often than others, so the clean subset
    has another mix of shapes than the step: the per-launch estimate weights
    each grid size's clean mean by that grid size's share of all kept
    dispatches. Prints a markdown summary."""
    import csv
    rows = list(csv.DictReader(open(path)))
    for r in rows:
        r["t0"], r["t1"] = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
    copies = sorted((r["t0"], r["t1"]) for r in rows if "copyBuffer" in r["Kernel_Name"])
    mine = sorted((r for r in rows if kernel_substr in r["Kernel_Name"]), key=lambda r: r["t0"])
    per = len(mine) // steps
    kept = mine[skip * per:]
    starts = [c[0] for c in copies]

    import bisect

    def overlaps(r):
        i = bisect.bisect_left(starts, r["t1"])
        return any(copies[j][1] > r["t0"] for j in range(max(0, i - 64), i))
    clean = [r for r in kept if not overlaps(r)]
    avg = lambda rs: sum(r["t1"] - r["t0"] for r in rs) / max(1, len(rs)) / 1e3
    grid = lambda r: int(r.get("Grid_Size") or r.get("Grid_Size_X"))
    shapes = sorted({grid(r) for r in kept})
    by = {g: ([r for r in kept if grid(r) == g], [r for r in clean if grid(r) == g]) for g in shapes}
    weighted = sum(len(a) / len(kept) * avg(c) for a, c in by.values() if c)
    print(f"| dispatches | count | average us |\n|---|---:|---:|")
    print(f"| `{kernel_substr}`, {steps - skip} of {steps} traced steps | {len(kept)} | {avg(kept):.1f} |")
    print(f"| the same, overlapping no copy kernel | {len(clean)} | {avg(clean):.1f} |")
    print(f"| clean mean per grid size, weighted by the step's mix | {len(kept)} | {weighted:.1f} |")
    print(f"\n| grid size (threads) | dispatches | clean | average us, all | average us, clean |\n|---:|---:|---:|---:|---:|")
    for g, (a, c) in by.items():
        print(f"| {g} | {len(a)} | {len(c)} | {avg(a):.1f} | {avg(c):.1f} |")
    if flops_per_launch:
        for name, t in (("all", avg(kept)), ("no copy overlap", avg(clean)), ("shape-weighted, no copy overlap", weighted)):
            t *= 1e-6
            print(f"\n{name}: {flops_per_launch / t / 1e12:.1f} TFLOP/s, frac {flops_per_launch / t / PEAK_BF16:.4f} "
                  f"of {PEAK_BF16 / 1e12:.0f}")


def main():
    if "--summarize-trace" in sys.argv:
        sp = argparse.ArgumentParser()
        sp.add_argument("--summarize-trace", required=True, help="rocprofv3 kernel_trace.csv")
        sp.add_argument("--trace-steps", type=int, required=True, help="steps in the traced run (warmup included)")
        sp.add_argument("--trace-skip", type=int, default=1, help="leading steps to leave out")
        sp.add_argument("--kernel", default="gemm_big_kernelIDF16bLi0EE", help="substring of the kernel symbol")
        sp.add_argument("--flops-per-launch", type=float, default=None)
        a = sp.parse_args()
        summarize_kernel_trace(a.summarize_trace, a.trace_steps, a.trace_skip, a.kernel, a.flops_per_launch)
        return
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="14b",
                    help="tiny | 1.3b | 14b | 7b-512k | 7b-1m | 120b (120b and 7b-1m: cut to fit, or --layers)")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--batch", type=int, default=None,
                    help="override the batch (sequences per step): more tokens per streamed byte")
    ap.add_argument("--seq-len", type=int, default=None,
                    help="override the tokens per sequence (the workload's layer shape kept)")
    ap.add_argument("--host-threads", type=int, default=0,
                    help="host AdamW / gather worker threads (0 = online CPUs)")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace", default=None, help="write the last step's schedule as Chrome JSON")
    ap.add_argument("--chunk-rows", type=int, default=0, help="token rows per projection/MLP chunk (0 = auto)")
    ap.add_argument("--ckpt-host", type=int, default=0, help="checkpoints parked in host memory (0 = auto)")
    ap.add_argument("--resident", action="store_true",
                    help="device cache of every unit (one buffer per layer and the head) instead of streaming "
                         "through two buffers: same as --layer-buffers n_layers+1")
    ap.add_argument("--layer-buffers", type=int, default=2,
                    help="device layer buffers: 2 streams every unit; k > 2 keeps the head and the top k-3 "
                         "layers in a device cache, refreshed with each update as it lands")
    ap.add_argument("--sync-opt", action="store_true",
                    help="every AdamW update lands before its step returns (default: updates may finish "
                         "during the next step's forward, in the order it loads the units)")
    ap.add_argument("--no-refresh", action="store_true",
                    help="with a device cache, fetch cached units in the next forward instead of refreshing them "
                         "in the backward")
    ap.add_argument("--bf16-grads", action="store_true",
                    help="gradients cross the host link as bf16 (a measured variant; the default keeps them fp32)")
    ap.add_argument("--micro-batches", type=int, default=0,
                    help="run each streamed unit over the batch in this many micro-batches, summing the weight "
                         "gradients on the device (one weight stream per step)")
    ap.add_argument("--progress", action="store_true",
                    help="print a line as each layer of a step finishes (for steps that take minutes)")
    ap.add_argument("--no-link-probe", action="store_true",
                    help="skip the plain pinned-copy measurement of the host link after the run")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="after the run, one plain device copy of this many MiB (a known-size reference "
                         "dispatch for hardware byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the streamed step on one GPU: this build has no multi-GPU path "
              "(no collectives). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from host_memory_streamed_amd import mt, synth

    if not os.path.exists(mt.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    w = mt.WORKLOADS[args.workload]
    dtype = mt.MT_BF16 if args.dtype == "bf16" else mt.MT_FP32
    flags = mt.MT_KERNEL_TIMING | mt.MT_TRACE | (0 if args.sync_opt else mt.MT_OVERLAP_OPT) | \
        (mt.MT_PROGRESS if args.progress else 0) | (mt.MT_CACHE_NO_REFRESH if args.no_refresh else 0) | \
        (mt.MT_BF16_GRADS if args.bf16_grads else 0)
    layers_note = None
    if args.batch:
        w = mt.Workload(**{**w.__dict__, "batch": args.batch})
    if args.seq_len:
        w = mt.Workload(**{**w.__dict__, "seq": args.seq_len})
    if args.layers:
        w = mt.Workload(**{**w.__dict__, "n_layers": args.layers})
    elif args.workload in ("120b", "7b-1m"):
        # the 120B-shaped and the million-token workloads keep their layer
        # shape and are cut to the layers whose host store (and parked
        # checkpoints) fit in this machine's RAM
        L = fit_layers(w, dtype, flags, device_free=torch.cuda.mem_get_info()[0])
        if L < w.n_layers:
            layers_note = f"cut from {w.n_layers} to {L} layers to fit host RAM and device memory"
            log(layers_note)
            w = mt.Workload(**{**w.__dict__, "n_layers": L})
    buffers = w.n_layers + 1 if args.resident else min(max(2, args.layer_buffers), w.n_layers + 1)
    ctx = build_context(w, dtype, args.seed, flags, host_threads=args.host_threads, chunk_rows=args.chunk_rows,
                        ckpt_host=args.ckpt_host,
                        buffers=buffers, micro_batches=args.micro_batches)
    layout = ctx.layout_info()
    tokens, targets = synth.token_batch(args.seed, w.batch, w.seq, w.vocab)
    M = w.batch * w.seq

    losses = []
    for i in range(args.warmup):
        t0 = time.perf_counter()
        losses.append(ctx.train_step(tokens, targets))
        log(f"warmup step {i}: {time.perf_counter() - t0:.3f}s loss {losses[-1]:.4f}")
    # the timed region holds exactly the K steps' work: the warmup's updates
    # land before it starts, the last step's updates before it ends
    ctx.sync()
    torch.cuda.synchronize()
    stats = []
    kstats = {}
    t_start = time.perf_counter()
    for i in range(args.steps):
        losses.append(ctx.train_step(tokens, targets))
        s = ctx.stats()
        stats.append(s)
        for k in ctx.kernel_stats():
            acc = kstats.setdefault(k["name"], {"launches": 0, "ms": 0.0, "flops": 0.0, "bytes": 0.0})
            for f in ("launches", "ms", "flops", "bytes"):
                acc[f] += k[f]
        log(f"step {i}: {s['step_ms']:.1f} ms loss {losses[-1]:.4f} fwd {s['forward_ms']:.0f} ms "
            f"tail {s['tail_ms']:.0f} ms adamw(sum) {s['adamw_ms']:.0f} ms")
    ctx.sync()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    if args.trace:
        ctx.trace_dump(args.trace)
    sched = ctx.schedule()

    ms = elapsed / args.steps * 1e3
    tok_s = M * args.steps / elapsed
    mean = lambda key: float(np.mean([s[key] for s in stats]))
    peak = PEAK_BF16 if dtype == mt.MT_BF16 else PEAK_FP32
    mfu = mean("model_flops") / (ms * 1e-3) / peak
    h2d, d2h = mean("h2d_bytes"), mean("d2h_bytes")
    # copy engine rates over the last step's copies
    loads = [e for e in sched if e["phase"] in ("load", "refresh", "ckpt_in") and e["stream"] == 0]
    grads = [e for e in sched if e["phase"] in ("grad", "ckpt_out") and e["stream"] == 2]
    h2d_busy = sum(e["t1"] - e["t0"] for e in loads) * 1e-3
    d2h_busy = sum(e["t1"] - e["t0"] for e in grads) * 1e-3
    unit_bytes_h2d = stats[-1]["h2d_bytes"] - M * (w.d_model + 1) * 4
    unit_bytes_d2h = stats[-1]["d2h_bytes"] - M * (w.d_model + 1) * 4

    # dominant kernel class by time, its algorithmic rate against its peak
    dom_name, dom = max(kstats.items(), key=lambda kv: kv[1]["ms"])
    gemm = dom_name.startswith("gemm") or dom_name.startswith("attn")
    achieved = dom["flops"] / (dom["ms"] * 1e-3) if gemm else dom["bytes"] / (dom["ms"] * 1e-3)
    kpeak = peak if gemm else PEAK_HBM
    gpu_ms = sum(v["ms"] for v in kstats.values()) / args.steps
    out = {
        "metric": ("training tokens/sec, MFU and host-link GB/s for 14B-shaped streamed step" if w.name == "14b"
                   else f"training tokens/sec, MFU and host-link GB/s for {w.name}-shaped streamed step"),
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dtype == mt.MT_BF16 else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name + "-shaped decoder, " + (
                       "streamed through 2 layer buffers" if buffers == 2 else
                       ("every unit in a device cache, " + ("fetched in the forward" if args.no_refresh else
                                                            "refreshed by each update"))
                       if buffers == w.n_layers + 1 else
                       f"head and top {buffers - 3} layers in a device cache, the rest streamed through 2 buffers"),
                   "layer_buffers": buffers,
                   **({"layers_note": layers_note} if layers_note else {}),
                   "n_layers": w.n_layers, "d_model": w.d_model, "n_heads": w.n_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "ffn_dim": w.ffn_dim,
                   "vocab": w.vocab, "global_batch": w.batch, "seq_len": w.seq,
                   "master": "fp32 p/m/v in host memory", "parallelism": "none (1 GPU)",
                   "optimizer": ("host AdamW, each update landing before its step returns" if args.sync_opt else
                                 "host AdamW, updates finishing during the next step's forward in load order"),
                   "grad_transfer": "bf16" if args.bf16_grads else "fp32",
                   **({"micro_batches": args.micro_batches} if args.micro_batches > 1 else {}),
                   **({"host_threads": args.host_threads} if args.host_threads > 0 else {}),
                   **layout},
        "mfu": round(mfu, 4),
        "host_link": {
            "h2d_GBps_step": round(h2d / (ms * 1e-3) / 1e9, 2),
            "d2h_GBps_step": round(d2h / (ms * 1e-3) / 1e9, 2),
            "h2d_GBps_copies": round(unit_bytes_h2d / h2d_busy / 1e9, 2) if h2d_busy > 0 else None,
            "d2h_GBps_copies": round(unit_bytes_d2h / d2h_busy / 1e9, 2) if d2h_busy > 0 else None,
            "h2d_bytes_step": h2d, "d2h_bytes_step": d2h,
        },
        "host_adamw": {"thread_ms_step": round(mean("adamw_ms"), 1),
                       "bytes_step": mean("adamw_bytes"),
                       "tail_ms": round(mean("tail_ms"), 1)},
        "gpu_kernel_ms_step": round(gpu_ms, 1),
        "loss_first": round(losses[0], 4),
        "roofline": {
            "kernel": dom_name,
            "bound": "mfma" if gemm else "hbm",
            "achieved": round(achieved / (1e12 if gemm else 1e9), 2),
            "peak": round(kpeak / (1e12 if gemm else 1e9), 1),
            "unit": "TFLOP/s" if gemm else "GB/s",
            "frac": round(achieved / kpeak, 4),
            "traffic": (recorded_traffic(dom_name) if w.name == "14b" else None),
            "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "launches_per_step": dom["launches"] // args.steps,
            "avg_launch_us": round(dom["ms"] / dom["launches"] * 1e3, 2),
        },
        "kernels": {k: {"ms_step": round(v["ms"] / args.steps, 2), "launches_step": v["launches"] // args.steps,
                        "TFLOPs": round(v["flops"] / (v["ms"] * 1e-3) / 1e12, 1) if v["flops"] else None,
                        "GBps": round(v["bytes"] / (v["ms"] * 1e-3) / 1e9, 1)}
                    for k, v in sorted(kstats.items(), key=lambda kv: -kv[1]["ms"]) if v["launches"]},
        "cpu_baseline": None,
    }
    ctx.close()
    if not args.no_link_probe:
        bw = link_probe()
        log(f"link probe: H2D {bw['h2d'] / 1e9:.1f} GB/s, D2H {bw['d2h'] / 1e9:.1f} GB/s")
        if buffers == 2 and not layout["ckpt_host"]:
            out["link_roofline"] = link_roofline(w, stats[-1], ms * 1e-3, bw, 2 if dtype == mt.MT_BF16 else 4)
        else:
            # a device cache moves its refreshes into the backward: only the
            # duplex bound applies
            t_dup = max(h2d / bw["h2d"], d2h / bw["d2h"])
            out["link_roofline"] = {"bw_h2d_GBps": round(bw["h2d"] / 1e9, 2), "bw_d2h_GBps": round(bw["d2h"] / 1e9, 2),
                                    "t_link_duplex_s": round(t_dup, 4), "frac_duplex": round(t_dup / (ms * 1e-3), 4)}
    if not args.no_link_probe:
        # host-memory bound: every byte the step's AdamW moves plus every byte
        # the copies move, at the rate the AdamW alone sustains
        hbw = host_probe()
        log(f"host probe: AdamW {hbw / 30e9:.2f} Gparam/s, {hbw / 1e9:.1f} GB/s")
        hbytes = mean("adamw_bytes") + h2d + d2h
        out["host_roofline"] = {"adamw_GBps": round(hbw / 1e9, 1), "bytes_step": hbytes,
                                "t_host_s": round(hbytes / hbw, 4), "frac": round(hbytes / hbw / (ms * 1e-3), 4)}
    if args.copy_probe:
        n = args.copy_probe << 18   # fp32 elements
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {n * 4} bytes read, {n * 4} bytes written")
        del src, dst
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline in {time.perf_counter() - t0:.1f}s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
