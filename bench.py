#!/usr/bin/env python3
"""Benchmark of the mixed-adapter LoRA linear on one MI355X (gfx950).

Workload: one Llama-3-8B decode step of q_proj. T = 64 tokens, 4096 -> 4096,
a 9-slot pool per layer (slots 1-8 rank 16, alpha 32; slot 0 the zero
adapter), 8 adapters x 8 tokens in shuffled order, over 32 layers, each with
its own seeded weights and pool (so a step streams ~1.1 GB, far beyond the
256 MB MALL). One step = the host plan (lora_plan) and its upload, then the
32 lora_linear calls, replayed from a HIP graph captured once.

value = T * layers / step time: tokens through one adapted linear per second
(T / mean lora_linear time).

After the timed region the same step runs eagerly with the library's
per-kernel HIP-event timing on (behind a long filler GEMM so the host stays
ahead of the GPU); those durations give the roofline figures. Then, each as
its own labelled figure: a warm call (one layer repeated, MALL-resident) and
the launch floor of a replayed graph; q/k/v in one lora_linear_multi call
against three calls; the prefill-shaped gate projection (T = 8192,
4096 -> 14336) for the base GEMM's matrix-core fraction; single cold calls
of the k/v mixed-rank and o/down workloads; and the fp64 CPU oracle on a
bounded sample of the decode workload.

Prints one JSON line. --gpus N > 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mixed-LoRA linear tokens/s + % MFMA/HBM roofline at Llama-3-8B shapes"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-slices", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--crossover", action="store_true",
                    help="also time the SGMV shrink against the BGMV shrink over ranks, adapters and tokens per adapter")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of a graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain 256 MiB device copies (reference for the FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


def stage_bytes(ids, ranks, d_in, d_out, r_max, es=2):
    """Algorithmic bytes per launch: the shrink kernel, and the base GEMM
    kernel whose epilogue applies the expand (base bytes plus B_s and the h
    read; y is written once, inside the base bytes)."""
    from rank_gemm_amd import accounting as acc
    seg = acc.segments(ids, ranks)
    T_a = sum(seg.values())
    shrink = es * T_a * d_in + sum(es * int(ranks[s]) * d_in for s in seg) + 4 * T_a * r_max
    expand = sum(es * int(ranks[s]) * d_out for s in seg) + 4 * T_a * r_max + 2 * es * T_a * d_out
    assert shrink + expand == acc.correction_bytes(ids, ranks, d_in, d_out, es, r_max)
    base = acc.base_bytes(len(ids), d_in, d_out, es)
    fused = base + sum(es * int(ranks[s]) * d_out for s in seg) + 4 * T_a * r_max
    return {"base": base, "shrink": shrink, "expand": expand, "fused": fused}


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy), or None when
    the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic_decode_q_proj.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    src = b"".join(open(os.path.join(ROOT, "rank_gemm_amd", "csrc", n), "rb").read()
                   for n in ("splitk.hip", "fuse.h", "shrink.h", "common.h", "kernels.h"))
    if t.get("kernel") != kernel or hashlib.sha256(src).hexdigest() != t.get("sources_sha256"):
        return None
    return int(t["bytes_per_launch"])


def us_of(stats, name):
    return stats[name]["mean_ms"] * 1e3 if name in stats else 0.0


def filler(torch, ms_target=60.0):
    """Queue ~ms_target of GPU work so the host can run ahead of the GPU."""
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    n = max(1, int(ms_target / 1.0))
    for _ in range(n):
        a = torch.matmul(a, a) * 1e-2
    return a


def shrink_crossover(torch, np, lora, K=4096):
    """SGMV (lora_shrink: 16-row items, plan given) against BGMV
    (lora_shrink_bgmv: token by token, no plan), both graph-replayed, warm."""
    rows = []
    g = np.random.default_rng(0)
    cases = [(r, na, tpa, "uniform") for r in (8, 16, 64) for na in (4, 16, 64) for tpa in (1, 2, 4, 8, 16, 64)
             if na * tpa <= 4096]
    cases += [(16, 32, T // 32, "zipf") for T in (64, 512, 4096)]
    for r, na, tpa, kind in cases:
        T, S = na * tpa, na + 1
        if kind == "uniform":
            ids = np.repeat(np.arange(1, S, dtype=np.int32), tpa)
            g.shuffle(ids)
        else:
            p = np.arange(1, S, dtype=np.float64) ** -1.1
            ids = (g.choice(S - 1, size=T, p=p / p.sum()) + 1).astype(np.int32)
        pool = lora.Pool(S, r, K, 64, "bf16")
        A = (torch.randn(r, K, device="cuda") * 0.01).to(torch.bfloat16)
        B = torch.zeros(64, r, device="cuda").to(torch.bfloat16)
        for s in range(1, S):
            pool.install(s, A, B, 2.0 * r)
        x = torch.randn(T, K, device="cuda").to(torch.bfloat16)
        plan = lora.plan(ids, S)
        ids_dev = torch.from_numpy(ids).cuda()
        ws = pool.workspace(T)
        h = torch.empty(T, r, device="cuda")

        def timed(fn, reps=20, calls=8):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(calls):
                    fn()
            gr.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * calls)

        sg = timed(lambda: lora.shrink(x, pool, plan, h=h))
        bg = timed(lambda: lora.shrink_bgmv(x, pool, ids_dev, h=h, workspace=ws))
        rows.append({"rank": r, "adapters": na, "tokens_per_adapter": tpa if kind == "uniform" else None,
                     "T": T, "slots": kind, "items": plan.info.n_items, "sgmv_us": round(sg, 2),
                     "bgmv_us": round(bg, 2), "faster": "sgmv" if sg < bg else "bgmv"})
        log(f"crossover {rows[-1]}")
        del pool, A, B, x, h, ws
    return rows


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported by this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from rank_gemm_amd import accounting as acc
    from rank_gemm_amd import lora
    from rank_gemm_amd.inputs import make_config, make_qkv_decode

    lora.lib()  # fail loudly if the library was not built
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    torch.cuda.set_device(0)
    L = args.layers

    t0 = time.perf_counter()
    with ThreadPoolExecutor(8) as ex:
        ws_host = list(ex.map(lambda l: make_config(2, layer=l), range(L)))
    log(f"generated {L} layers in {time.perf_counter() - t0:.1f}s")
    w0 = ws_host[0]
    T, S, r_max = w0.T, w0.S, w0.r_max
    ids = w0.slot_ids
    d_in, d_out = w0.projections[0].d_in, w0.projections[0].d_out
    ranks = w0.ranks

    pools, xs, Ws, ys = [], [], [], []
    for w in ws_host:
        pr = w.projections[0]
        pool = lora.Pool(S, r_max, d_in, d_out, "bf16")
        for s, a in sorted(pr.adapters.items()):
            pool.install(s, lora.to_device(a.A, "bf16"), lora.to_device(a.B, "bf16"), a.alpha)
        pools.append(pool)
        xs.append(lora.to_device(pr.x, "bf16"))
        Ws.append(lora.to_device(pr.W, "bf16"))
        ys.append(torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda"))
    ws = torch.empty(pools[0].workspace_bytes(T), dtype=torch.uint8, device="cuda")
    p = lora.plan(ids, S)
    info0 = (p.info.T, p.info.S, p.info.T_a, p.info.k, p.info.n_items, p.info.max_seg)
    torch.cuda.synchronize()

    def layers_once():
        for l in range(L):
            lora.linear(xs[l], Ws[l], pools[l], p, y=ys[l], workspace=ws)

    def step_plan():
        lora.plan_into(p, ids)
        assert (p.info.T, p.info.S, p.info.T_a, p.info.k, p.info.n_items, p.info.max_seg) == info0

    # ---- timed region: graph replay (default) or eager --------------------------
    graph = None
    if not args.eager:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                layers_once()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layers_once()
        torch.cuda.synchronize()

    def step():
        step_plan()
        if graph is not None:
            graph.replay()
        else:
            layers_once()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    value = T * L * args.steps / elapsed
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.4g} tokens/s")

    # ---- per-kernel durations (HIP events on the launch stream) -------------------
    def profile(plan_ids):
        lora.plan_into(p, plan_ids)
        f = filler(torch)
        lora.profile_begin(8 * L * args.profile_steps + 64)
        for _ in range(args.profile_steps):
            lora.plan_into(p, plan_ids)
            layers_once()
        stats = lora.profile_end()
        torch.cuda.synchronize()
        del f
        return stats

    stats = profile(ids)
    stats_base = profile(np.zeros_like(ids))
    lora.plan_into(p, ids)
    sb = stage_bytes(ids, ranks, d_in, d_out, r_max)
    # decode path: kernel 1 = split-K GEMM partials + shrink workgroups,
    # kernel 2 = split reduction + fused expand + bf16 store
    k1, k2 = "gemm_splitk", "gemm_splitk_epilogue"
    t1, t2 = us_of(stats, k1), us_of(stats, k2)
    t1b, t2b = us_of(stats_base, k1), us_of(stats_base, k2)
    # kernel 1 reads x once, W once and each active slot's A_s at true rank
    a_bytes = sum(2 * int(ranks[s]) * d_in for s in acc.segments(ids, ranks))
    k1_bytes = 2 * T * d_in + 2 * d_in * d_out + a_bytes
    k1_gbs = k1_bytes / (t1 * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(k1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(k1_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("splitk_gemm_kernel<8, false, false>"),
            "kernel": "splitk_gemm_kernel (base GEMM K-split partials + SGMV shrink workgroups)",
            "bytes_per_launch": k1_bytes, "mean_us": round(t1, 3)}
    call_bytes = sb["base"] + sb["shrink"] + sb["expand"]
    corr_us = max(t1 - t1b, 0.0) + max(t2 - t2b, 0.0)
    corr = {"bytes_per_call": sb["shrink"] + sb["expand"],
            "incremental_us": round(corr_us, 3),
            "kernel1_us": round(t1, 3), "kernel1_base_only_us": round(t1b, 3),
            "kernel2_us": round(t2, 3), "kernel2_base_only_us": round(t2b, 3),
            "call_us": round(t1 + t2, 3),
            "call_achieved_gbs": round(call_bytes / ((t1 + t2) * 1e-6) / 1e9, 1),
            "call_frac_hbm": round(call_bytes / ((t1 + t2) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    kernels = {k: {"mean_us": round(v["mean_ms"] * 1e3, 3), "median_us": round(v["median_ms"] * 1e3, 3),
                   "min_us": round(v["min_ms"] * 1e3, 3), "count": v["count"]} for k, v in stats.items()}
    log(f"kernels: {kernels}; base-only: {stats_base}")

    # ---- warm figure and launch floor -------------------------------------------
    # warm: layer 0 called 32 times (its 32 MB W stays in the 256 MB MALL);
    # floor: 32 one-element fill kernels, graph-replayed the same way
    def graph_us(fn, n_calls, reps=20):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * n_calls)

    def warm_calls():
        for _ in range(L):
            lora.linear(xs[0], Ws[0], pools[0], p, y=ys[0], workspace=ws)

    tiny = torch.zeros(1, device="cuda")

    def tiny_fills():
        for _ in range(L):
            tiny.fill_(1.0)

    warm_us = graph_us(warm_calls, L)
    floor_us = graph_us(tiny_fills, L)
    warm = {"call_us": round(warm_us, 3), "tokens_per_s": round(T / (warm_us * 1e-6), 1),
            "note": "one layer's weights called 32 times in a graph (MALL-resident)"}
    floor = {"kernel_us": round(floor_us, 3),
             "note": "one-element fill kernel, 32 per graph: launch-to-launch floor of a replayed step"}
    log(f"warm: {warm}; floor: {floor}")

    # ---- the same step with the plan built on the device --------------------------
    # plan_device + 32 lora_linear_device_plan in one graph: no host work per step
    ids_dev = torch.from_numpy(ids.copy()).cuda()
    dplan = lora.plan_device(ids_dev, S)

    def dev_step():
        lora.plan_device(ids_dev, S, out=dplan)
        for l in range(L):
            lora.linear(xs[l], Ws[l], pools[l], dplan, y=ys[l], workspace=ws)

    dstep_us = graph_us(dev_step, 1, reps=args.steps)

    def plans_only():
        for _ in range(L):
            lora.plan_device(ids_dev, S, out=dplan)

    plan_us = graph_us(plans_only, L)
    device_plan = {"ms_per_step": round(dstep_us * 1e-3, 4), "tokens_per_s": round(T * L / (dstep_us * 1e-6), 1),
                   "plan_kernel_us": round(plan_us, 3),
                   "note": "lora_plan_device + 32 lora_linear_device_plan captured in one graph"}
    log(f"device plan: {device_plan}")

    # ---- q/k/v in one call against three calls ----------------------------------
    slices = None
    if not args.no_slices:
        LQ = 8  # 8 layers of q/k/v weights (384 MiB) so the replays stream from HBM
        with ThreadPoolExecutor(8) as ex:
            qkv_host = list(ex.map(lambda l: make_qkv_decode(layer=l), range(LQ)))
        qkv = []
        for w in qkv_host:
            pls = []
            for pr in w.projections:
                pl = lora.Pool(w.S, w.r_max, pr.d_in, pr.d_out, "bf16")
                for s_, a in sorted(pr.adapters.items()):
                    pl.install(s_, lora.to_device(a.A, "bf16"), lora.to_device(a.B, "bf16"), a.alpha)
                pls.append(pl)
            qkv.append((lora.to_device(w.projections[0].x, "bf16"), [lora.to_device(pr.W, "bf16") for pr in w.projections],
                        pls, [torch.empty((w.T, pr.d_out), dtype=torch.bfloat16, device="cuda")
                              for pr in w.projections]))
        wq = qkv_host[0]
        pq = lora.plan(wq.slot_ids, wq.S)
        wsq = torch.empty(max(lora.workspace_bytes_multi(qkv[0][2], wq.T),
                              max(pl.workspace_bytes(wq.T) for pl in qkv[0][2])), dtype=torch.uint8, device="cuda")

        def merged():
            for x_, W_, pl_, y_ in qkv:
                lora.linear_multi(x_, W_, pl_, pq, ys=y_, workspace=wsq)

        def separate():
            for x_, W_, pl_, y_ in qkv:
                for i in range(3):
                    lora.linear(x_, W_[i], pl_[i], pq, y=y_[i], workspace=wsq)

        def time_graph(fn, reps=20):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / (reps * LQ)

        us_m, us_s = time_graph(merged), time_graph(separate)
        rq = wq.ranks
        outs = [pr.d_out for pr in wq.projections]
        a_q = sum(2 * int(rq[s_]) * d_in for s_ in acc.segments(wq.slot_ids, rq))
        b_q = sum(2 * int(rq[s_]) * n for s_ in acc.segments(wq.slot_ids, rq) for n in outs)
        lay_bytes = 2 * wq.T * d_in + sum(2 * d_in * n + 2 * wq.T * n for n in outs) + 3 * a_q + b_q
        slices = {"workload": f"llama3-8b q/k/v decode: T={wq.T}, {d_in}->{outs}, S={wq.S} rank 16, {LQ} layers",
                  "merged_us_per_layer": round(us_m, 3), "separate_us_per_layer": round(us_s, 3),
                  "speedup": round(us_s / us_m, 3), "bytes_per_layer": lay_bytes,
                  "merged_frac_hbm": round(lay_bytes / (us_m * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"slices: {slices}")
        del qkv, wsq

    # ---- prefill-shaped base GEMM (matrix-core fraction) --------------------------
    prefill = None
    if not args.no_prefill:
        del pools, xs, Ws, ys
        torch.cuda.empty_cache()
        w3 = make_config(3)
        pr = w3.projections[0]
        pool3 = lora.Pool(w3.S, w3.r_max, pr.d_in, pr.d_out, "bf16")
        for s, a in sorted(pr.adapters.items()):
            pool3.install(s, lora.to_device(a.A, "bf16"), lora.to_device(a.B, "bf16"), a.alpha)
        x3, W3 = lora.to_device(pr.x, "bf16"), lora.to_device(pr.W, "bf16")
        p3 = lora.plan(w3.slot_ids, w3.S)
        y3 = torch.empty((w3.T, pr.d_out), dtype=torch.bfloat16, device="cuda")
        # one untimed batch first: the first batch after the decode part runs
        # ~10% slower (clocks settling under the heavier load)
        for _ in range(10):
            lora.linear(x3, W3, pool3, p3, y=y3)
        torch.cuda.synchronize()
        n3 = 10
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(n3):
            lora.linear(x3, W3, pool3, p3, y=y3)
        ev1.record()
        torch.cuda.synchronize()
        call_ms = ev0.elapsed_time(ev1) / n3
        lora.profile_begin(8 * n3 + 64)
        for _ in range(n3):
            lora.linear(x3, W3, pool3, p3, y=y3)
        s3 = lora.profile_end()
        p3b = lora.plan(np.zeros_like(w3.slot_ids), w3.S)
        lora.profile_begin(8 * n3 + 64)
        for _ in range(n3):
            lora.linear(x3, W3, pool3, p3b, y=y3)
        s3b = lora.profile_end()
        # the same product through torch's linear (hipBLASLt), against the
        # base-only call, both timed with stream events, interleaved
        lib_us, own_us = [], []
        for _ in range(3):
            for which in ("lib", "own"):
                ev0.record()
                for _ in range(n3):
                    if which == "lib":
                        torch.nn.functional.linear(x3, W3, out=y3)
                    else:
                        lora.linear(x3, W3, pool3, p3b, y=y3)
                ev1.record()
                torch.cuda.synchronize()
                (lib_us if which == "lib" else own_us).append(ev0.elapsed_time(ev1) / n3 * 1e3)
        fl = acc.base_flops(w3.T, pr.d_in, pr.d_out)
        t_b = us_of(s3b, "gemm_bf16")
        t_f = us_of(s3, "gemm_bf16")
        tf = fl / (t_b * 1e-6) / 1e12
        tf_f = fl / (t_f * 1e-6) / 1e12
        prefill = {"workload": "llama3-8b gate_proj prefill T=8192 4096->14336, 16 seqs x 512, S=17 rank 16",
                   "base_gemm_us": round(t_b, 2), "base_tflops": round(tf, 1),
                   "base_frac_mfma": round(tf / BF16_PEAK_TFLOPS, 4),
                   "fused_gemm_us": round(t_f, 2), "fused_frac_mfma": round(tf_f / BF16_PEAK_TFLOPS, 4),
                   "shrink_us": round(us_of(s3, "sgmv_shrink"), 2),
                   "call_ms": round(call_ms, 4), "tokens_per_s": round(w3.T / (call_ms * 1e-3), 1),
                   "kernels": {k: round(v["mean_ms"] * 1e3, 2) for k, v in s3.items()},
                   "vs_library": {"torch_linear_us": round(min(lib_us), 2), "base_call_us": round(min(own_us), 2),
                                  "note": "torch.nn.functional.linear (hipBLASLt) on the same x and W against "
                                          "lora_linear with a base-only plan; stream events over 10 calls, "
                                          "best of 3 interleaved rounds"}}
        log(f"prefill: {prefill}")

    crossover = shrink_crossover(torch, np, lora) if args.crossover else None

    # ---- other configs, single cold calls ------------------------------------------
    others = None
    if not args.no_configs:
        torch.cuda.empty_cache()
        flush = torch.empty(512 * 2**20, dtype=torch.uint8, device="cuda")
        others = {}
        for cfg in (4, 5):
            wc = make_config(cfg)
            pc = lora.plan(wc.slot_ids, wc.S)
            for pr in wc.projections:
                pool_c = lora.Pool(wc.S, wc.r_max, pr.d_in, pr.d_out, "bf16")
                for s_, a in sorted(pr.adapters.items()):
                    pool_c.install(s_, lora.to_device(a.A, "bf16"), lora.to_device(a.B, "bf16"), a.alpha)
                xc, Wc = lora.to_device(pr.x, "bf16"), lora.to_device(pr.W, "bf16")
                yc = torch.empty((wc.T, pr.d_out), dtype=torch.bfloat16, device="cuda")
                lora.linear(xc, Wc, pool_c, pc, y=yc)
                torch.cuda.synchronize()
                n_c = 10
                lora.profile_begin(8 * n_c + 64)
                for _ in range(n_c):
                    flush.add_(1)  # evict the MALL and L2 before each call
                    lora.linear(xc, Wc, pool_c, pc, y=yc)
                sc = lora.profile_end()
                torch.cuda.synchronize()
                call_us = sum(v["median_ms"] for v in sc.values()) * 1e3
                entry = {"T": wc.T, "d_in": pr.d_in, "d_out": pr.d_out, "S": wc.S,
                         "call_us": round(call_us, 2), "tokens_per_s": round(wc.T / (call_us * 1e-6), 1),
                         "kernels_median_us": {k: round(v["median_ms"] * 1e3, 2) for k, v in sc.items()}}
                rk = wc.ranks
                if "gemm_splitk" in sc:
                    a_b = sum(2 * int(rk[s_]) * pr.d_in for s_ in acc.segments(wc.slot_ids, rk))
                    kb = 2 * wc.T * pr.d_in + 2 * pr.d_in * pr.d_out + a_b
                    gbs = kb / (sc["gemm_splitk"]["median_ms"] * 1e-3) / 1e9
                    entry["kernel1_frac_hbm"] = round(gbs / HBM_PEAK_GBS, 4)
                else:
                    # the tiled GEMM, and when it is split over K, the reduction of its partials
                    gemm_ms = sc["gemm_bf16"]["median_ms"] + (sc["gemm_splitk_epilogue"]["median_ms"]
                                                              if "gemm_splitk_epilogue" in sc else 0.0)
                    fl = acc.base_flops(wc.T, pr.d_in, pr.d_out)
                    tf = fl / (gemm_ms * 1e-3) / 1e12
                    entry["gemm_frac_mfma"] = round(tf / BF16_PEAK_TFLOPS, 4)
                others[f"config{cfg} {pr.name}"] = entry
                del pool_c, xc, Wc, yc
        del flush
        log(f"other configs: {others}")

    if args.copy_calibration:
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 5 x 256 MiB device copies")

    # ---- CPU oracle baseline (bounded sample of the same workload) ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        done, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            pr = ws_host[done % L].projections[0]
            oracle.lora_rows("bf16", pr.x, pr.W, S, pr.adapters, ids)
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(T * done / el, 2), "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"fp64 oracle, all {T} rows of {done} q_proj layer calls (cycling over the "
                         f"{L} layers of the decode workload), {el:.1f} s"}
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3-8b q_proj decode step: T={T}, {d_in}->{d_out}, S={S} (8 adapters x 8 "
                               f"tokens, rank 16, alpha 32), {L} layers, plan + {L} lora_linear per step",
                   "T": T, "d_in": d_in, "d_out": d_out, "S": S, "rank": 16, "layers": L,
                   "mode": "eager" if graph is None else "hip graph replay"},
        "roofline": roof, "cpu_baseline": cpu,
        "correction": corr, "kernels": kernels, "warm": warm, "launch_floor": floor, "device_plan": device_plan,
        "prefill": prefill,
        "slices": slices, "other_configs": others, "shrink_crossover": crossover,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
