#!/usr/bin/env python3
"""STCA forward throughput on one MI355X.

One step = one full STCA forward (every row of the hot path: planning, the
history gather + SwiGLU FFN + LN + W_K/W_V of every layer, the query chain,
the m-target multi-head cross attention with its split-L merge, W_O, the
fusion update and z) over the RLB long-history workload: 32 users with
10,240-item histories, 64 targets per user sharing the user's K/V, a
4,000,000 x 256 bf16 table with Zipf(1.1) ids, d = 256, 8 heads, SwiGLU
hidden 512, 4 stacked layers.  Inputs are synthetic, seeded, and resident in
HBM before the timed region.

Prints one JSON line.  ``value`` = history tokens per second per STCA layer
(sum of history lengths x layers / time per forward).  The roofline block
covers the dominant kernel (per-launch duration from HIP events recorded by
the library at stage boundaries on its own stream); the attention kernel's HBM
roofline is reported beside it.  ``cpu_baseline`` times the float64 oracle on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
NOMINAL_CLOCK_GHZ = 2.4        # the clock the bf16 peak is quoted at (256 CUs x 4 SIMDs x 1024 flop/clk)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_peaks():
    """Attainable rates on this GPU, quoted beside the nominal peaks the
    rooflines are priced against: dense bf16 MFMA from registers (the
    library's MFMA-only kernel, best of three launches, on fixed low-entropy
    operands and on operands that vary like real data), an HBM read stream
    (the library's streaming-read kernel over 2 GiB, best of four) and a
    1 GiB device copy (read + write bytes / time, best of five)."""
    import torch
    from recsys_ultra_long_amd import stca
    mfma, mfma_clk = stca.peak_mfma_bf16()
    mfma_mx, mfma_mx_clk = stca.peak_mfma_bf16(mixed=True)
    hbm_read = stca.peak_hbm_read()
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.copy_(a)
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        best = max(best, 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a, b
    return {"mfma_bf16_tflops": round(mfma, 1), "mfma_bf16_clock_ghz": round(mfma_clk, 3),
            "mfma_bf16_mixed_tflops": round(mfma_mx, 1), "mfma_bf16_mixed_clock_ghz": round(mfma_mx_clk, 3),
            "hbm_read_gbs": round(hbm_read, 1), "hbm_copy_gbs": round(best, 1)}


def attach_measured_peaks(res, skip=False):
    """Beside each roofline's nominal peak: the attainable rate measured in
    this run and the achieved fraction of it (context; `frac` stays the
    fraction of the nominal peak)."""
    if skip:
        res["measured_peaks"] = None
        return
    mp = measured_peaks()
    res["measured_peaks"] = mp
    log(f"measured peaks: {mp}")
    for k, roof in res.items():
        if k.startswith("roofline") and isinstance(roof, dict):
            # the attention reads K/V (one write per target): priced against the read stream
            pm = mp["mfma_bf16_tflops"] if roof["unit"] == "TFLOP/s" else mp["hbm_read_gbs"]
            roof["peak_measured"] = pm
            roof["frac_measured"] = round(roof["achieved"] / pm, 4)
            if roof["unit"] == "TFLOP/s":  # the same, for operands that switch like real data
                roof["peak_measured_mixed"] = mp["mfma_bf16_mixed_tflops"]
                roof["frac_measured_mixed"] = round(roof["achieved"] / mp["mfma_bf16_mixed_tflops"], 4)


def workload(name):
    from recsys_ultra_long_amd import inputs as I
    from dataclasses import replace
    if name.endswith("-relu"):
        # the same workload with ReLU-scored attention (and active counts)
        return replace(workload(name[:-len("-relu")]), score="relu")
    if name.endswith("-longer"):
        # the same workload with the LONGER-style sequence encoding: each
        # layer's history is the cross attention of the last 256 items over
        # all of them (the pages fix no short length; 256 << 8192)
        from dataclasses import replace
        return replace(workload(name[:-len("-longer")]), encoder="longer", l_short=256)
    if name == "rlb-long":
        return I.spec(3)
    if name == "single-target":
        return I.spec(2)
    if name == "ragged":
        return I.spec(4)
    if name == "rlb-train":
        return I.spec(6)
    if name in ("hyformer-feed", "hyformer-search"):
        # the HyFormer workload's sequence with generated, boosted queries
        return replace(I.spec(5)[name.split("-")[1]], qmode="hyformer", n_ns=8)
    if name in ("hyformer-feed-linear", "hyformer-search-linear", "hyformer-linear"):
        # the HyFormer-style workload as configured: N_q = 8 given queries per
        # sequence, the next layer's queries a fixed random linear map of the
        # cross output; "hyformer-linear" is both sequences (feed, then search)
        return I.spec(5)["search" if "search" in name else "feed"]
    raise SystemExit(f"unknown workload {name}")


def host_info():
    """What the CPU baseline ran on: CPU model, the cores this process may
    use, and the BLAS library numpy calls (with its thread count)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas, threads = "unknown", None
    try:
        import numpy  # noqa: F401  (loads the BLAS library threadpoolctl inspects)
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = (f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')}, "
                        f"{i.get('threading_layer')}; {os.path.basename(i.get('filepath', ''))})")
                threads = i.get("num_threads")
                break
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas": blas,
            "blas_threads": threads}


def cpu_baseline(p, seconds):
    """Float64 oracle on whole users of the same workload until `seconds`
    pass.  Its products run in the BLAS library on every core of the process's
    affinity set; its per-target and per-head loops are single-threaded
    Python, so `cores` is the affinity count (the threads it may use), with
    the host's CPU model and BLAS named beside it."""
    import numpy as np
    from oracle import stca_oracle as O
    hi = host_info()
    cores = hi["affinity_cores"]
    sp = p.spec
    layers, z, wz = O.weights_f64(p.layers, p.z, p.wz)
    cfg = dict(d=sp.d, H=sp.H, M=sp.M, score=sp.score, qmode=sp.qmode, kv_ln=sp.kv_ln,
               z_ln=sp.z_ln, encoder=sp.encoder, l_short=sp.l_short)
    rows = lambda ids: O.stored_to_f64(p.rows(ids))
    t0 = time.perf_counter()
    users, toks, tgts = 0, 0, 0
    q0 = O.stored_to_f64(p.q0) if p.q0 is not None else None
    hy = None
    if sp.qmode == "hyformer":
        hy = {"ns": O.stored_to_f64(p.extra["ns"]),
              "qgen": {k: O.stored_to_f64(v) for k, v in p.extra["qgen"].items()}}
    while users < sp.B:
        O.forward(cfg, p.hist_offsets, p.hist_ids, p.tgt_offsets, rows, layers, z, wz,
                  tgt_ids=p.tgt_ids, q0=q0, users=[users], hy=hy)
        toks += int(p.hist_offsets[users + 1] - p.hist_offsets[users])
        tgts += int(p.tgt_offsets[users + 1] - p.tgt_offsets[users])
        users += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": toks * sp.M / dt, "unit": "history tokens/s per STCA layer",
            "cores": int(cores), "kind": "oracle",
            "sample": f"{users} of {sp.B} users ({toks} history tokens, {tgts} targets, "
                      f"{sp.M} layers) in {dt:.1f} s, float64 numpy (BLAS products on "
                      f"{hi['blas_threads']} threads, per-target loops single-threaded)",
            "target_scores_per_s": tgts / dt, **hi}


def cpu_baseline_backward(p, dz, seconds):
    """Float64 backward oracle on whole users of the training workload until
    `seconds` pass."""
    from oracle import stca_grad as OG
    hi = host_info()
    cores = hi["affinity_cores"]
    sp = p.spec
    t0 = time.perf_counter()
    users, toks = 0, 0
    while users < sp.B:
        OG.backward_problem(p, dz, users=[users])
        toks += int(p.hist_offsets[users + 1] - p.hist_offsets[users])
        users += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": toks * sp.M / dt, "unit": "history tokens/s per STCA layer (backward)",
            "cores": int(cores), "kind": "oracle",
            "sample": f"{users} of {sp.B} users ({toks} history tokens, {sp.M} layers) in {dt:.1f} s, "
                      "float64 numpy backward (forward recompute included)", **hi}


def traffic_for(kernel_prefix, name):
    """Calibrated HBM bytes per launch of the kernel whose name starts with
    kernel_prefix, from profiles/traffic_<name>.md, or None when that summary
    is missing or was taken on other kernel sources."""
    from recsys_ultra_long_amd import profiling
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{name}.md"))
    if tr is None:
        return None
    hits = [v["hbm_bytes"] for k, v in tr["kernels"].items() if k.startswith(kernel_prefix)]
    return round(max(hits)) if hits else None


def bench_backward(args):
    """One training step = a forward (z for the loss head) + stca_backward
    (gradients of every weight and table row for a seeded dz).  The forward is
    stca_forward_for_backward, which leaves its activations in the backward's
    workspace so that the backward skips its recompute; with --recompute it is
    stca_forward on the fused path and the backward recomputes."""
    import numpy as np
    import torch
    from recsys_ultra_long_amd import inputs as I
    from recsys_ultra_long_amd import stca
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stca.load()
    sp = workload(args.workload)
    t = time.time()
    p = I.make_problem(sp, with_table=True, threads=min(16, os.cpu_count() or 8))
    log(f"workload generated in {time.time() - t:.1f}s: B={sp.B} n_hist={p.n_hist} n_tgt={p.n_tgt}")
    dz_np = I.upstream_grad(sp, p.n_tgt)
    dz = torch.from_numpy(dz_np).cuda()
    dp_b = stca.upload(p, dedup=args.dedup)
    M = sp.M
    nev = stca.n_backward_stage_events(M)
    evs = [stca.StageEvents(nev) for _ in range(args.steps)]
    bw = stca.Backward(dp_b, dz, outputs=("table",))
    log(f"backward workspace {bw.ws_bytes / 2**30:.2f} GiB")
    if args.recompute:  # forward on the fused path, the backward recomputes its activations
        dp_f = stca.upload(p, path="fused", table=dp_b.table)
        fwd = stca.Forward(dp_f, want=(), dumps=())

        def f():
            fwd()

        def b():
            bw()
    else:  # the forward keeps its activations in the backward's workspace
        z = torch.empty((p.n_tgt, sp.d), dtype=torch.float32, device="cuda")

        def f():
            bw.forward_for_backward(z)

        def b():
            bw(saved_forward=True)
    for _ in range(args.warmup):
        bw.zero()
        f()
        b()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        bw.zero()
        bw.g.stage_events = evs[k].ptr
        bw.g.n_stage_events = nev
        ev[k][0].record()
        f()
        ev[k][1].record()
        b()
        ev[k][2].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / args.steps
    ms_f = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    ms_b = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    if int(bw.status[0].item()) != 0 or (args.recompute and int(fwd.status[0].item()) != 0):
        raise SystemExit("device status flagged")

    def stage(i, j):
        return float(np.mean([e.elapsed(i, j) for e in evs]))
    recompute, zhead = stage(0, 1), stage(1, 2)
    attn_b, qside, hist_b, usum, hrows, hwgrad = [], [], [], [], [], []
    # j-th layer processed: layer M-1-j (five events per layer).  The history
    # side runs on the library's second stream from the attention backward's
    # end (event b) on, alongside the query side: its stages are timed from b.
    for j in range(M):
        b = 3 + 5 * j
        prev = 2 if j == 0 else b - 4  # the previous layer's query side
        attn_b.append(stage(prev, b))
        qside.append(stage(b, b + 1))
        hist_b.append(stage(b, b + 4))
        usum.append(stage(b, b + 2))
        hrows.append(stage(b + 2, b + 3))
        hwgrad.append(stage(b + 3, b + 4))
    table_t = stage(2 + 5 * M, 3 + 5 * M)
    for e in evs:
        e.close()
    d, h = sp.d, sp.hidden
    n_hist, T = p.n_hist, p.n_tgt
    n_unique = int(len(np.unique(p.hist_ids)))
    rows_h = n_unique if args.dedup else n_hist
    pairs = int(np.sum(np.diff(p.hist_offsets).astype(np.int64) * np.diff(p.tgt_offsets)))
    # backward proper, per layer: history 18 d h + 8 d^2 per row (recomputed
    # FFN 6dh, dXt 4d^2, dG 2dh, dX 4dh, weight gradients 6dh + 4d^2), over
    # the unique rows with dedup; attention 10 d per (item, target) pair
    flops_hist_layer = rows_h * (18 * d * h + 8 * d * d)
    flops_b = M * (flops_hist_layer + 10 * d * pairs)
    flops_f = M * (rows_h * (6 * d * h + 4 * d * d) + 4 * d * pairs)
    t_hist = float(np.mean(hist_b)) * 1e-3
    hist_tf = flops_hist_layer / t_hist / 1e12
    # attention backward: K, V rows read, dK | dV rows written (bf16), Q, dA read
    bytes_attn = n_hist * 8 * d + T * 4 * d
    t_attn = float(np.mean(attn_b)) * 1e-3
    attn_gbs = bytes_attn / t_attn / 1e9
    roof_hist = {"kernel": "history backward stage of one layer (per-unique-row dK | dV sums with dedup, "
                           "the row pass, five split-K weight-gradient GEMMs)", "bound": "mfma",
                 "achieved": round(hist_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(hist_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                 "launch_ms": round(t_hist * 1e3, 4),
                 "per_launch": f"{rows_h} {'unique rows' if args.dedup else 'history items'} x "
                               f"{18 * d * h + 8 * d * d} flop"}
    # the row pass alone: at d = 256 one launch (hist_bwd256_kernel): recomputed
    # FFN 6dh, dX~ 4d^2, dG 2dh, dX 4dh per row
    t_rows = float(np.mean(hrows)) * 1e-3
    row_flops = 12 * d * h + 4 * d * d
    rows_tf = rows_h * row_flops / t_rows / 1e12
    roof_rows = {"kernel": "hist_bwd256_kernel (history backward row pass of one layer: recomputed FFN + LN, "
                           "dX~, LN backward, dG, SwiGLU backward, dX)" if d == 256 and h % 128 == 0 else
                           "history backward row pass of one layer (strided GEMMs + row kernels)",
                 "bound": "mfma", "achieved": round(rows_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(rows_tf / PEAK_BF16_TFLOPS, 4),
                 "traffic": traffic_for("hist_bwd256_kernel<true>", "rlb-train_backward"
                                        + ("_dedup" if args.dedup else "")),
                 "launch_ms": round(t_rows * 1e3, 4),
                 "per_launch": f"{rows_h} {'unique rows' if args.dedup else 'history items'} x {row_flops} flop"}
    roof_attn = {"kernel": "attention backward of one layer (incl. W_O and the dQ fold)", "bound": "hbm",
                 "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(attn_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                 "launch_ms": round(t_attn * 1e3, 4),
                 "per_launch": f"{n_hist} items x {8 * d} B + {T} targets x {4 * d} B"}
    ms = ms_f + ms_b
    res = {
        "metric": "training step (forward + backward) history tokens/s per STCA layer",
        "value": round(n_hist * M / (ms * 1e-3), 1),
        "unit": "history tokens/s per STCA layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "ms_forward": round(ms_f, 4), "ms_backward": round(ms_b, 4),
        "ms_wall_per_step": round(wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{sp.name}: B={sp.B} users, L ~ max(16, ceil(10240 Beta({sp.beta_a},1))) "
                               f"(sum {n_hist}), m={sp.m} targets/user, table {sp.table_rows}x{d} bf16 "
                               f"Zipf({sp.zipf_s}) ids, d={d}, H={sp.H}, hidden={h}, M={M}, softmax; "
                               + ("forward on the fused path, backward recomputes on the staged path"
                                  if args.recompute else "forward on the staged path keeping its activations "
                                  "for the backward (stca_forward_for_backward)")
                               + (f", unique-id dedup of the history side ({n_unique} unique "
                                  f"of {n_hist})" if args.dedup else ""),
                   "global_batch": sp.B, "targets": T, "parallelism": "single GPU"},
        "roofline": roof_rows if sum(hrows) >= sum(attn_b) else roof_attn,
        "roofline_history_backward": roof_hist,
        "roofline_history_row_pass": roof_rows,
        "roofline_attention_backward": roof_attn,
        "backward_stages_ms": {"forward_recompute": round(recompute, 4), "z_head": round(zhead, 4),
                               "attention_backward": [round(x, 4) for x in attn_b],
                               "query_side": [round(x, 4) for x in qside],
                               "history_backward": [round(x, 4) for x in hist_b],
                               "history_unique_sums": [round(x, 4) for x in usum],
                               "history_row_pass": [round(x, 4) for x in hrows],
                               "history_weight_gradients": [round(x, 4) for x in hwgrad],
                               "table_scatter": round(table_t, 4)},
        "backward_tflops": round((flops_b + flops_f) / (ms_b * 1e-3) / 1e12, 2),
        "backward_flops": {"proper": flops_b, "recompute": flops_f},
    }
    attach_measured_peaks(res, args.no_measured_peaks)
    if not args.no_cpu_baseline:
        log(f"timing the float64 backward oracle for ~{args.cpu_seconds:.0f}s")
        res["cpu_baseline"] = cpu_baseline_backward(p, dz_np, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def bench_lsweep(args):
    """History length sweep at a fixed total: the RLB long model (d 256, H 8,
    M 4, m 64 targets per user) over sum(L) = 327,680 history tokens cut into
    B = sum(L) / L users of length L, for L = 1,024 .. 10,240.  The review's
    complexity table gives STCA O(L d_h) time per layer, so the history
    encoding and the attention -- the stages whose work is per history token
    (the attention's per (token, target) pair, with m fixed) -- should run at a
    flat rate in history tokens per second; the query side grows with the
    number of users (targets = B m) and is reported apart."""
    from dataclasses import replace
    import numpy as np
    import torch
    from recsys_ultra_long_amd import inputs as I
    from recsys_ultra_long_amd import stca
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stca.load()
    total = 327_680
    base = I.spec(3)
    table = None
    rows = []
    for L in (1024, 2048, 4096, 8192, 10240):
        sp = replace(base, L=L, B=total // L)
        p = I.make_problem(sp, with_table=table is None, threads=min(16, os.cpu_count() or 8))
        dp = stca.upload(p, path="staged", table=table)
        table = dp.table
        M = sp.M
        nev = stca.n_stage_events(M)
        evs = [stca.StageEvents(nev) for _ in range(args.steps)]
        f = stca.Forward(dp, want=(), dumps=())
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for k in range(args.steps):
            f.out.stage_events = evs[k].ptr
            f.out.n_stage_events = nev
            f()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / args.steps
        if int(f.status[0].item()) != 0:
            raise SystemExit("device status flagged")
        stage = lambda a, b: float(np.mean([e.elapsed(a, b) for e in evs]))
        hist = sum(stage(1 + i, 2 + i) for i in range(M))
        attn = [stage(2 + M + 4 * i, 3 + M + 4 * i) + stage(3 + M + 4 * i, 4 + M + 4 * i) for i in range(M)]
        rest = ms - hist - sum(attn)
        rows.append({"L": L, "B": sp.B, "targets": p.n_tgt, "ms_per_step": round(ms, 4),
                     "tokens_per_s_per_layer": round(total * M / (ms * 1e-3), 1),
                     "history_ms": round(hist, 4), "history_tokens_per_s_per_layer": round(total * M / (hist * 1e-3), 1),
                     "attention_ms_per_layer": round(float(np.mean(attn)), 4),
                     "attention_tokens_per_s": round(total / (float(np.mean(attn)) * 1e-3), 1),
                     "query_side_and_rest_ms": round(rest, 4)})
        log(f"L={L} B={sp.B}: {ms:.3f} ms/step, history {hist:.3f} ms, attention {np.mean(attn):.4f} ms/layer")
        for e in evs:
            e.close()
        del f, dp
        torch.cuda.synchronize()
    flat = lambda key: round(max(r[key] for r in rows) / min(r[key] for r in rows), 4)
    res = {"metric": "history tokens/s per STCA layer across L at fixed sum(L) (O(L) check)",
           "unit": "history tokens/s per STCA layer", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"rlb-long model (d 256, H 8, hidden 512, M 4, m 64), sum(L) = {total} "
                                  "history tokens in B = sum(L) / L users, staged path"},
           "sweep": rows,
           "max_over_min": {"history": flat("history_tokens_per_s_per_layer"),
                            "attention": flat("attention_tokens_per_s"),
                            "whole_forward": flat("tokens_per_s_per_layer")}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="rlb-long")
    ap.add_argument("--cross-mask", action="store_true",
                    help="Cross-Mask attention: heads 2 and 6 see a quarter of the items (seeded "
                         "per-item masks) and pairs of heads share one attention map (staged path)")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step (forward + stca_backward) on the training "
                         "workload (rlb-train unless --workload names another)")
    ap.add_argument("--recompute", action="store_true",
                    help="with --backward: the step's forward on the fused path and the backward "
                         "recomputing its activations (default: the forward keeps them)")
    ap.add_argument("--path", default="staged", choices=["staged", "fused"],
                    help="staged (default: K/V streamed through HBM, so the projection (MFMA) and "
                         "attention (HBM) stages are timed apart) or fused (no K/V in HBM)")
    ap.add_argument("--dedup", action="store_true",
                    help="staged path with unique-id dedup of the history encoding "
                         "(bit-identical results; valid because a row's encoding depends on its id alone)")
    ap.add_argument("--no-other-path", action="store_true",
                    help="skip timing the other path for comparison")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the MFMA-only and device-copy measurements (for profiler runs)")
    ap.add_argument("--lsweep", action="store_true",
                    help="history-length sweep at fixed sum(L) (one JSON line of its own)")
    ap.add_argument("--replicas", type=int, default=1,
                    help="the workload with this many times its users (same per-user shape): K/V "
                         "beyond the 256 MB Infinity Cache for the attention's HBM figure")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of 1 GiB (x5), to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.backward:
        if args.workload == "rlb-long":
            args.workload = "rlb-train"
        return bench_backward(args)
    if args.lsweep:
        return bench_lsweep(args)
    if args.copy_calibration:
        import torch
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the STCA forward "
              "shards by user with no exchange, so throughput at N GPUs is N times this "
              "figure by construction and is not measured here.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from recsys_ultra_long_amd import inputs as I
    from recsys_ultra_long_amd import stca

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stca.load()
    sp = workload(args.workload)
    if args.replicas > 1:
        from dataclasses import replace
        sp = replace(sp, B=sp.B * args.replicas)
    if args.dedup or args.cross_mask or sp.d == 512 or sp.qmode in ("hyformer", "linear"):
        args.path = "staged"  # the fused path serves d <= 256 and STCA (fusion) queries
    t = time.time()
    p = I.make_problem(sp, with_table=True, threads=min(16, os.cpu_count() or 8))
    log(f"workload generated in {time.time() - t:.1f}s: B={sp.B} n_hist={p.n_hist} "
        f"n_tgt={p.n_tgt} table={sp.table_rows}x{sp.d} {sp.dtype}")
    if args.cross_mask:
        p.extra["key_mask"] = I.cross_mask(sp, p.n_hist, (2, 6), keep=0.25)
        p.extra["head_map"] = [h - (h % 2) for h in range(sp.H)]
    dp = stca.upload(p, path=args.path, dedup=args.dedup)
    n_unique = int(len(np.unique(p.hist_ids))) if args.dedup else None
    # both sequences of the HyFormer-style workload: the search sequence's
    # forward follows the feed's in every step (each has its own table and
    # weights); stage figures are the feed's
    companion = None
    if args.workload == "hyformer-linear":
        sp2 = workload("hyformer-search-linear")
        p2 = I.make_problem(sp2, with_table=True, threads=min(16, os.cpu_count() or 8))
        companion = stca.Forward(stca.upload(p2, path="staged"), want=(), dumps=())
        log(f"search sequence: B={sp2.B} n_hist={p2.n_hist} n_tgt={p2.n_tgt}")
    torch.cuda.synchronize()
    log("uploaded")
    M = sp.M
    longer = sp.encoder == "longer"
    nev = stca.n_stage_events(M, longer)
    evs = [stca.StageEvents(nev) for _ in range(args.steps)]
    f = stca.Forward(dp, want=(), dumps=())
    for _ in range(args.warmup):
        f()
        if companion is not None:
            companion()
    torch.cuda.synchronize()
    log(f"warm-up done ({args.warmup} steps)")

    # shader clock during the history launch (staged bf16 path at d = 128, 256)
    clk = torch.zeros(8, 4, dtype=torch.int64, device="cuda")
    f.out.clock_probe = clk.data_ptr()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for k in range(args.steps):
        f.out.stage_events = evs[k].ptr
        f.out.n_stage_events = nev
        f()
        if companion is not None:
            companion()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    st = int(f.status[0].item()) | (int(companion.status[0].item()) if companion is not None else 0)
    if st != 0:
        raise SystemExit(f"device status flagged: {st}")
    log(f"timed {args.steps} steps: {ms:.3f} ms/step")

    # per-stage durations from the library's boundary events
    def stage(a, b):
        return float(np.mean([e.elapsed(a, b) for e in evs]))
    prep = stage(0, 1)
    hist = [stage(1 + i, 2 + i) for i in range(M)]
    query, part, merge, wo = [], [], [], []
    for i in range(M):
        prev = 1 + M if i == 0 else 5 + M + 4 * (i - 1)
        query.append(stage(prev, 2 + M + 4 * i))
        part.append(stage(2 + M + 4 * i, 3 + M + 4 * i))
        merge.append(stage(3 + M + 4 * i, 4 + M + 4 * i))
        wo.append(stage(4 + M + 4 * i, 5 + M + 4 * i))
    zt = stage(5 + M + 4 * (M - 1), 2 + 5 * M)

    d, h, H = sp.d, sp.hidden, sp.H
    n_hist, T = p.n_hist, p.n_tgt
    lens = np.diff(p.hist_offsets).astype(np.int64)
    # LONGER: the layers decode over each user's min(L_u, l_short) encoded rows
    dec_lens = np.minimum(lens, sp.l_short) if longer else lens
    n_dec = int(dec_lens.sum())
    enc_rows = n_unique if args.dedup else n_dec              # rows the history chain processes
    row_flops = 4 * d * d if longer else 6 * d * h + 4 * d * d
    flops_hist = enc_rows * row_flops                         # per layer
    # attention flops: 4 d per (history token, target of the same user) pair
    pairs = int(np.sum(dec_lens * np.diff(p.tgt_offsets)))
    flops_attn = 4 * d * pairs
    bytes_attn = n_dec * 4 * d + T * 2 * d                   # K,V bf16 read once + Q
    # bf16 at d <= 256 encodes every layer's history in one launch (its
    # duration lands in the first history stage): per-layer figures use
    # the total over layers
    t_hist = float(np.sum(hist)) / M * 1e-3
    multi = sp.dtype == "bf16" and d <= 256 and args.path == "staged"
    hist_layers_per_launch = M if multi else 1
    t_attn = float(np.mean(part)) * 1e-3
    hist_tf = flops_hist / t_hist / 1e12
    attn_gbs = bytes_attn / t_attn / 1e9
    roof_hist = {"kernel": "history chain (gather+W_K|W_V of the encoded short rows)" if longer
                 else "history chain (gather+SwiGLU+LN+W_K|W_V)", "bound": "mfma",
                 "achieved": round(hist_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(hist_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                 "launch_ms": round(t_hist * hist_layers_per_launch * 1e3, 4),
                 "per_launch": f"{enc_rows} {'unique rows' if args.dedup else 'tokens'} x "
                               f"{hist_layers_per_launch} layer(s) x {row_flops} flop"}
    roof_attn = {"kernel": "m-target cross attention (split-L partials)", "bound": "hbm",
                 "achieved": round(attn_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(attn_gbs / PEAK_HBM_GBS, 4), "traffic": None,
                 "launch_ms": round(t_attn * 1e3, 4),
                 "per_launch": f"{n_dec} tokens x {4 * d} B + {T} targets x {2 * d} B"}
    # HBM bytes per launch from the committed rocprofv3 --pmc summary, if it
    # was taken on the current kernel sources
    from recsys_ultra_long_amd import profiling
    roofs = {"history": roof_hist, "attention": roof_attn}
    times = {"history": float(np.sum(hist)), "attention": float(np.sum(part))}
    enc_stages = {}
    if longer:
        # the encoding pre-pass, per layer: S W'_K | S W'_V over the raw rows,
        # S_short W'_Q, the short rows' attention over the raw rows, W'_O
        e0 = 3 + 5 * M
        enc_kv = [stage(e0 + 4 * i, e0 + 1 + 4 * i) for i in range(M)]
        enc_q = [stage(e0 + 1 + 4 * i, e0 + 2 + 4 * i) for i in range(M)]
        enc_at = [stage(e0 + 2 + 4 * i, e0 + 3 + 4 * i) for i in range(M)]
        enc_wo = [stage(e0 + 3 + 4 * i, e0 + 4 + 4 * i) for i in range(M)]
        enc_stages = {"enc_setup": round(stage(0, e0), 4), "enc_kv": [round(x, 4) for x in enc_kv],
                      "enc_q": [round(x, 4) for x in enc_q], "enc_attention": [round(x, 4) for x in enc_at],
                      "enc_wo": [round(x, 4) for x in enc_wo], "prep_plan": round(stage(e0 + 4 * M, 1), 4)}
        t_ekv = float(np.mean(enc_kv)) * 1e-3
        ekv_tf = n_hist * 4 * d * d / t_ekv / 1e12
        roofs["encoder_kv"] = {"kernel": "encoder chain (gather+W'_K|W'_V, raw rows)", "bound": "mfma",
                               "achieved": round(ekv_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                               "frac": round(ekv_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                               "launch_ms": round(t_ekv * 1e3, 4),
                               "per_launch": f"{n_hist} tokens x {4 * d * d} flop"}
        pairs_enc = int(np.sum(dec_lens * lens))
        t_eat = float(np.mean(enc_at)) * 1e-3
        eat_tf = 4 * d * pairs_enc / t_eat / 1e12
        roofs["encoder_attention"] = {
            "kernel": "encoder attention (short rows over raw rows, partials + merge)", "bound": "mfma",
            "achieved": round(eat_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(eat_tf / PEAK_BF16_TFLOPS, 4), "traffic": None, "launch_ms": round(t_eat * 1e3, 4),
            "per_launch": f"{pairs_enc} (short row, raw row) pairs x {4 * d} flop"}
        times["encoder_kv"] = float(np.sum(enc_kv))
        times["encoder_attention"] = float(np.sum(enc_at))
    if args.path == "fused":
        # one kernel per layer: gather, history FFN + LN, W_K | W_V and the
        # attention; K/V never leave the chip, so it is bound by the MFMA
        fused_tf = (flops_hist + flops_attn) / t_attn / 1e12
        roofs = {"fused": {"kernel": "fused gather+SwiGLU+LN+W_K|W_V+attention", "bound": "mfma",
                           "achieved": round(fused_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(fused_tf / PEAK_BF16_TFLOPS, 4), "traffic": None,
                           "launch_ms": round(t_attn * 1e3, 4),
                           "per_launch": f"{n_hist} tokens x {6 * d * h + 4 * d * d} flop + "
                                         f"{pairs} (token, target) pairs x {4 * d} flop"}}
    ghz = stca.clock_ghz(clk.cpu().numpy())
    if args.path == "staged" and d in (128, 256) and sp.dtype == "bf16" and ghz == ghz:
        at_clk = PEAK_BF16_TFLOPS * ghz / NOMINAL_CLOCK_GHZ
        roof_hist.update({"shader_clock_ghz": round(ghz, 3), "peak_at_clock": round(at_clk, 1),
                          "frac_at_clock": round(hist_tf / at_clk, 4)})
        log(f"history launch: shader clock {ghz:.3f} GHz -> bf16 MFMA peak at that clock "
            f"{at_clk:.0f} TFLOP/s, achieved {hist_tf / at_clk:.1%}")
    # kernel names in the traffic summary (template arguments: <D, rows, input mode, FFN, LN, projection,
    # output> for the chain; the attention's last argument is its one-wave-per-group mode).  With the
    # LONGER encoding the short-row history chain and the encoder K/V chain are one kernel instance,
    # so a per-name average would mix them: neither gets a traffic figure.
    picks = {"history": lambda k: not longer and (
                 k.startswith("hist256_kernel<") or k.startswith("hist128_kernel<") or
                 (k.startswith(f"chain_kernel<{d},") and ", 0, true, " in k)),
             "attention": lambda k: k.startswith("attn_bf16_kernel<") and k.endswith("false>"),
             "encoder_attention": lambda k: k.startswith("attn_bf16_kernel<") and k.endswith("true>"),
             "encoder_kv": lambda k: False,
             "fused": lambda k: k.startswith("fused256_kernel<") or k.startswith(f"fused_kernel<{d},")}
    rep = f"-x{args.replicas}" if args.replicas > 1 else ""
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", f"traffic_{args.workload}{rep}_{args.path}"
                                                                 f"{'_dedup' if args.dedup else ''}.md"))
    if tr is not None:
        for name, roof in roofs.items():
            hits = [v["hbm_bytes"] for k, v in tr["kernels"].items() if picks[name](k)]
            if hits:
                roof["traffic"] = round(max(hits))
    if args.path == "fused":
        dominant = roofs["fused"]
    else:
        dominant = roofs[max(times, key=times.get)]

    n_hist_all, T_all = n_hist, T
    if companion is not None:
        n_hist_all += companion.dp.n_hist
        T_all += companion.dp.n_tgt
    value = n_hist_all * M / (ms * 1e-3)
    res = {
        "metric": "history tokens/s + target scores/s per STCA layer at L=10K; % of HBM/MFMA peak",
        "value": round(value, 1),
        "unit": "history tokens/s per STCA layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{sp.name}: B={sp.B} users, "
                               + (f"L={sp.L}" if sp.L else f"L = max({sp.L_min}, ceil({sp.L_max} Beta({sp.beta_a}, 1))) "
                                  f"(sum {n_hist})")
                               + f", m={sp.m} {'queries' if sp.qmode != 'fusion' else 'targets'}/user (RLB), "
                               f"table {sp.table_rows}x{d} bf16 Zipf({sp.zipf_s}) ids, d={d}, H={H}, "
                               f"hidden={h}, M={M} layers, {sp.score}, path={args.path}"
                               + (", queries N(0,1), next queries a fixed random linear map of the cross "
                                  "output, no history LN" if sp.qmode == "linear" else "")
                               + (f"; with the search sequence (B={companion.dp.cfg.B}, L=1024, its own "
                                  "2,000,000x512 table and weights) in the same step" if companion is not None else "")
                               + (f"; {args.replicas}x the workload's users (K/V beyond the 256 MB Infinity "
                                  "Cache)" if args.replicas > 1 else "")
                               + (", Cross-Mask: heads 2 and 6 see 25% of the items, heads 2k and 2k+1 "
                                  "share the map of head 2k" if args.cross_mask else "")
                               + (f", HyFormer queries: {sp.n_ns} non-sequence tokens, query FFN hidden "
                                  f"{sp.hy_hidden or d}, no history LN" if sp.qmode == "hyformer" else "")
                               + (f", unique-id dedup ({n_unique} unique of {n_hist})" if args.dedup else "")
                               + (f", LONGER-style encoding: each layer's history is the cross attention of the "
                                  f"last {sp.l_short} items over all items" if longer else ""),
                   "global_batch": sp.B, "seq_len": sp.L, "targets": T, "parallelism": "single GPU"},
        "target_scores_per_s_per_layer": round(T_all * M / (ms * 1e-3), 1),
        "target_scores_per_s": round(T_all / (ms * 1e-3), 1),
        "history_tokens_per_s": round(n_hist_all / (ms * 1e-3), 1),
        "roofline": dominant,
        **({"roofline_attention": roof_attn, "roofline_history": roof_hist}
           if args.path == "staged" else {}),
        **({"roofline_encoder_kv": roofs["encoder_kv"], "roofline_encoder_attention": roofs["encoder_attention"],
            "encoder_stages_ms": enc_stages} if longer else {}),
        "stages_ms": {"prep_plan": round(prep, 4),
                      **({"history": [round(x, 4) for x in hist]} if args.path == "staged" else {}),
                      "query": [round(x, 4) for x in query],
                      ("attn_partial" if args.path == "staged" else "fused"): [round(x, 4) for x in part],
                      "attn_merge": [round(x, 4) for x in merge], ("w_o+boost" if sp.qmode == "hyformer" else "w_o"): [round(x, 4) for x in wo],
                      "z": round(zt, 4)},
    }
    for e in evs:
        e.close()
    if not args.no_other_path and not args.dedup and not longer and companion is None:
        # the same inputs through the other path, and through the staged path
        # with unique-id dedup (bit-identical outputs, valid because a history
        # row here depends on its id alone)
        del f
        others = [("staged" if args.path == "fused" else "fused", False), ("staged", True)]
        if sp.d == 512 or sp.qmode in ("hyformer", "linear") or args.cross_mask:
            others = [("staged", True)]
        res["other_paths"] = []
        for other, dd in others:
            dpo = stca.upload(p, path=other, table=dp.table, dedup=dd)
            fo = stca.Forward(dpo, want=(), dumps=())
            for _ in range(args.warmup):
                fo()
            torch.cuda.synchronize()
            start.record()
            for _ in range(args.steps):
                fo()
            end.record()
            torch.cuda.synchronize()
            mso = start.elapsed_time(end) / args.steps
            if int(fo.status[0].item()) != 0:
                raise SystemExit(f"device status flagged on path {other}")
            res["other_paths"].append({"path": other + ("+dedup" if dd else ""), "ms_per_step": round(mso, 4),
                                       "value": round(n_hist * M / (mso * 1e-3), 1)})
            log(f"other path ({other}{'+dedup' if dd else ''}): {mso:.3f} ms/step")
            del fo, dpo
    attach_measured_peaks(res, args.no_measured_peaks)
    if not args.no_cpu_baseline:
        log(f"timing the float64 oracle for ~{args.cpu_seconds:.0f}s")
        res["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
