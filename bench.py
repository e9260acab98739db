#!/usr/bin/env python3
"""Benchmark of the mixed-adapter LoRA linear on one MI355X (gfx950).

Headline workload: the prefill-shaped Llama-3-8B gate and up projections.
T = 8192 tokens in 16 sequences of 512, each sequence on one slot drawn
from {0..16}; d_in 4096 -> d_out 14336; a 17-slot pool per projection
(slots 1-16 rank 16, alpha 32; slot 0 the zero adapter). One step = the
host plan (lora_plan) and its upload, then one lora_linear_multi over the
gate and up slices with that plan (one SGMV shrink reading the x rows once
for both slices' A, then each slice's base GEMM with its expand as extra K
steps). Inputs, weights and pools are resident in HBM;
the step's working set (x 64 MiB, two W of 112 MiB, two y of 224 MiB) is
three times the 256 MiB MALL, so every call streams from HBM.

value = T * 2 / step time: tokens through one adapted linear per second
(T / mean lora_linear time), as for the decode figure.

The steps are timed twice. The first pass runs them as they are and gives
value. The second runs the same steps with the library's per-kernel
profiler on: each kernel launch carries a pair of HIP events on its own
stream that the runtime stamps with the kernel's start and end
(hipExtLaunchKernel). The value thus comes from launches without
instrumentation, and the durations from the same steps run again. The dominant kernel is the tiled base GEMM
(gemm_tile_kernel, matrix-core bound): achieved = its algorithmic FLOPs per
launch (2 T d_in d_out for the base product plus 2 T_a r d_out for the
expand it carries) / its mean duration over the second pass.

Side figures, each labelled: the same call with a base-only plan and
torch's linear (hipBLASLt) on the same product; the decode step (q_proj,
T = 64, 32 layers, HIP-graph replay) with its HBM figures; q/k/v in one
call; the device planner; single cold calls of the other workloads (tiny
fp32, k/v mixed ranks, o/down); and the fp64 CPU oracle: on a bounded
sample of the headline workload (cpu_baseline) and on every other workload,
on all threads and, for the three smaller ones, on one thread.

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
FP32_PEAK_TFLOPS = 157.3


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200,
                    help="timed steps (a step of the headline takes ~1.5 ms; many steps average out the "
                         "box's slower spells of some tens of milliseconds)")
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first: the clocks take a few tens of ms of this load to settle")
    ap.add_argument("--layers", type=int, default=32, help="layers of the decode-step figure")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time on the headline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-slices", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-library", action="store_true", help="skip the hipBLASLt comparison")
    ap.add_argument("--headline-only", action="store_true",
                    help="only the headline steps (for profiler passes: no side figures, no oracle)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-step figures (for profiler passes; the line's value is then null)")
    ap.add_argument("--no-crossover", action="store_true",
                    help="skip timing the SGMV correction against the BGMV correction over ranks, adapters and "
                         "tokens per adapter")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain 256 MiB device copies (reference for the FETCH_SIZE/WRITE_SIZE counters)")
    a = ap.parse_args()
    if a.headline_only:
        a.no_cpu_baseline = a.no_decode = a.no_slices = a.no_configs = a.no_library = a.no_crossover = True
    if a.decode_only:
        a.no_cpu_baseline = a.no_slices = a.no_configs = a.no_library = a.no_crossover = True
    return a


def measured_traffic(kernel, summary, sources):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 PMC summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy), or None when the
    kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    src = b"".join(open(os.path.join(ROOT, "rank_gemm_amd", "csrc", n), "rb").read() for n in sources)
    if t.get("kernel") != kernel or hashlib.sha256(src).hexdigest() != t.get("sources_sha256"):
        return None
    return int(t["bytes_per_launch"])


def us_of(stats, name, key="mean_ms"):
    return stats[name][key] * 1e3 if name in stats else 0.0


def kstats(stats):
    return {k: {"mean_us": round(v["mean_ms"] * 1e3, 3), "median_us": round(v["median_ms"] * 1e3, 3),
                "min_us": round(v["min_ms"] * 1e3, 3), "count": v["count"]} for k, v in stats.items()}


def filler(torch, ms_target=60.0):
    """Queue ~ms_target of GPU work so the host can run ahead of the GPU."""
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    n = max(1, int(ms_target / 1.0))
    for _ in range(n):
        a = torch.matmul(a, a) * 1e-2
    return a


def graph_us(torch, fn, n_calls, reps=20):
    """Mean time per call of `fn` (which makes n_calls calls), captured in a
    HIP graph and replayed `reps` times between stream events."""
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


def install_pool(lora, w, pr):
    pool = lora.Pool(w.S, w.r_max, pr.d_in, pr.d_out, w.dtype)
    for s, a in sorted(pr.adapters.items()):
        pool.install(s, lora.to_device(a.A, w.dtype), lora.to_device(a.B, w.dtype), a.alpha)
    return pool


# --------------------------------------------------------------------------- headline
def headline(args, torch, np, lora, acc, w3):
    """Config 3 gate + up. Two timed passes of the same steps: the first
    without instrumentation gives the value; the second, with per-kernel HIP
    events (hipExtLaunchKernel start/stop events), gives the kernels'
    durations for the roofline."""
    T, S = w3.T, w3.S
    ids = w3.slot_ids
    projs = w3.projections
    pools = [install_pool(lora, w3, pr) for pr in projs]
    x = lora.to_device(projs[0].x, "bf16")
    Ws = [lora.to_device(pr.W, "bf16") for pr in projs]
    ys = [torch.empty((T, pr.d_out), dtype=torch.bfloat16, device="cuda") for pr in projs]
    ws = torch.empty(max(lora.workspace_bytes_multi(pools, T), max(pl.workspace_bytes(T) for pl in pools)),
                     dtype=torch.uint8, device="cuda")
    # The plan is computed on the host and copied on the compute stream ahead
    # of the step's kernels. (Copying it on a side stream during the previous
    # step saved about 10 us per step, but stalled single GEMM launches for
    # several milliseconds now and then while both queues were busy.)
    p = lora.plan(ids, S)
    torch.cuda.synchronize()

    def step():
        lora.plan_into(p, ids)
        lora.linear_multi(x, Ws, pools, p, ys=ys, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = 2 * T * args.steps / elapsed
    lora.profile_begin(8 * args.steps + 64)
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_instr = (time.perf_counter() - t1) * 1e3 / args.steps
    stats = lora.profile_end()
    log(f"headline: {args.steps} steps, {ms_per_step:.4f} ms/step, {value:.5g} tokens/s; with per-kernel events "
        f"{ms_instr:.4f} ms/step, kernels {kstats(stats)}")

    d_in, d_out = projs[0].d_in, projs[0].d_out
    ranks = w3.ranks
    seg = acc.segments(ids, ranks)
    T_a = sum(seg.values())
    base_fl = acc.base_flops(T, d_in, d_out)
    expand_fl = sum(2 * n * int(ranks[s]) * d_out for s, n in seg.items())
    shrink_fl = sum(2 * n * int(ranks[s]) * d_in for s, n in seg.items())
    t_gemm = us_of(stats, "gemm_bf16")
    # one shrink launch per step serves both slices: half of it per projection
    n_shrink = stats.get("sgmv_shrink", {}).get("count", 0)
    n_gemm = stats.get("gemm_bf16", {}).get("count", 0)
    t_shrink = us_of(stats, "sgmv_shrink") * (n_shrink / n_gemm if n_gemm else 1.0)
    gemm_fl = base_fl + expand_fl
    ach = gemm_fl / (t_gemm * 1e-6) / 1e12
    roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic("gemm_tile_kernel<256, 256, 2, 2, 2, false, false, false, true>", "traffic_prefill_gate_up.json",
                                        ("gemm_bf16.hip", "fuse.h", "common.h", "kernels.h")),
            "traffic_note": "bytes per launch between the L2s and the memory fabric (MALL/HBM): FETCH_SIZE x 2.0 + "
                            "WRITE_SIZE x 1.0 (a plain 256 MiB copy reads those factors), against 416 MB of "
                            "algorithmic bytes; each XCD fetches its own copy of its tiles' x and W blocks",
            "kernel": "gemm_tile_kernel (tiled bf16 base GEMM, 256x256 tiles on 4 waves, expand as extra K steps)",
            "flops_per_launch": gemm_fl, "mean_us": round(t_gemm, 2),
            "median_us": round(us_of(stats, "gemm_bf16", "median_ms"), 2),
            "launches": stats.get("gemm_bf16", {}).get("count", 0),
            "timing": "per-kernel hipExtLaunchKernel events over a second timed pass of the same steps "
                      f"({ms_instr:.4f} ms per step with the events on)"}
    call_us = t_shrink + t_gemm
    call_fl = base_fl + expand_fl + shrink_fl
    call = {"T_a": T_a, "active_slots": len(seg), "shrink_us": round(t_shrink, 2), "gemm_us": round(t_gemm, 2),
            "shrink_note": "the step's one shrink launch (both slices) split evenly over the two projections",
            "kernels_us_per_call": round(call_us, 2),
            "call_tflops": round(call_fl / (call_us * 1e-6) / 1e12, 1),
            "call_frac_mfma": round(call_fl / (call_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "correction_flops": expand_fl + shrink_fl,
            "correction_share_of_base": round((expand_fl + shrink_fl) / base_fl, 5)}

    base = None
    if not args.no_library:
        # the same calls with a base-only plan, and torch's linear (hipBLASLt)
        # on the same product, interleaved, stream events over 10 calls each
        pb = lora.plan(np.zeros_like(ids), S)
        lora.profile_begin(8 * 10 + 64)
        for _ in range(10):
            lora.linear(x, Ws[0], pools[0], pb, y=ys[0], workspace=ws)
        sb = lora.profile_end()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lib_us, own_us = [], []
        for _ in range(3):
            for which in ("lib", "own"):
                ev0.record()
                for _ in range(10):
                    if which == "lib":
                        torch.nn.functional.linear(x, Ws[0], out=ys[0])
                    else:
                        lora.linear(x, Ws[0], pools[0], pb, y=ys[0], workspace=ws)
                ev1.record()
                torch.cuda.synchronize()
                (lib_us if which == "lib" else own_us).append(ev0.elapsed_time(ev1) / 10 * 1e3)
        tb = us_of(sb, "gemm_bf16")
        base = {"gemm_us": round(tb, 2), "frac_mfma": round(base_fl / (tb * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "torch_linear_us": round(min(lib_us), 2), "base_call_us": round(min(own_us), 2),
                "note": "gate projection with a base-only plan (no correction kernel); torch.nn.functional.linear "
                        "(hipBLASLt) on the same x and W; stream events over 10 calls, best of 3 interleaved rounds"}
        log(f"headline base-only / library: {base}")
    del pools, x, Ws, ys, ws, p
    torch.cuda.empty_cache()
    return value, ms_per_step, roof, call, base, stats


# --------------------------------------------------------------------------- decode step
def decode_step(args, torch, np, lora, acc, make_config, make_qkv_decode):
    L = args.layers
    t0 = time.perf_counter()
    with ThreadPoolExecutor(8) as ex:
        ws_host = list(ex.map(lambda l: make_config(2, layer=l), range(L)))
    log(f"decode: generated {L} layers in {time.perf_counter() - t0:.1f}s")
    w0 = ws_host[0]
    T, S, r_max = w0.T, w0.S, w0.r_max
    ids = w0.slot_ids
    d_in, d_out = w0.projections[0].d_in, w0.projections[0].d_out
    ranks = w0.ranks
    pools = [install_pool(lora, w, w.projections[0]) for w in ws_host]
    xs = [lora.to_device(w.projections[0].x, "bf16") for w in ws_host]
    Ws = [lora.to_device(w.projections[0].W, "bf16") for w in ws_host]
    ys = [torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda") for _ in ws_host]
    del ws_host
    ws = torch.empty(pools[0].workspace_bytes(T), dtype=torch.uint8, device="cuda")
    p = lora.plan(ids, S)
    info0 = (p.info.T, p.info.S, p.info.T_a, p.info.k, p.info.n_items, p.info.max_seg)
    torch.cuda.synchronize()

    def layers_once():
        for l in range(L):
            lora.linear(xs[l], Ws[l], pools[l], p, y=ys[l], workspace=ws)

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
        lora.plan_into(p, ids)
        assert (p.info.T, p.info.S, p.info.T_a, p.info.k, p.info.n_items, p.info.max_seg) == info0
        graph.replay()

    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.decode_steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / args.decode_steps

    def profile(plan_ids):
        # planned once: re-planning each step would make the host wait for the
        # plan upload two steps back and let the GPU idle between layers
        lora.plan_into(p, plan_ids)
        f = filler(torch)
        lora.profile_begin(8 * L * args.profile_steps + 64)
        for _ in range(args.profile_steps):
            layers_once()
        stats = lora.profile_end()
        torch.cuda.synchronize()
        del f
        return stats

    stats = profile(ids)
    stats_b = profile(np.zeros_like(ids))
    lora.plan_into(p, ids)
    seg = acc.segments(ids, ranks)
    T_a = sum(seg.values())
    a_bytes = sum(2 * int(ranks[s]) * d_in for s in seg)
    k1_bytes = 2 * T * d_in + 2 * d_in * d_out + a_bytes
    corr_bytes = acc.correction_bytes(ids, ranks, d_in, d_out, 2, r_max)
    call_bytes = acc.base_bytes(T, d_in, d_out, 2) + corr_bytes
    k1, k2 = "gemm_splitk", "gemm_splitk_epilogue"
    t1, t2 = us_of(stats, k1), us_of(stats, k2)
    t1b, t2b = us_of(stats_b, k1), us_of(stats_b, k2)
    dec = {
        "workload": f"llama3-8b q_proj decode step: T={T}, {d_in}->{d_out}, S={S} (8 adapters x 8 tokens, rank 16, "
                    f"alpha 32), {L} layers each with its own W and pool, plan + {L} lora_linear per step, "
                    f"HIP graph replay",
        "ms_per_step": round(ms_step, 4), "tokens_per_s": round(T * L / (ms_step * 1e-3), 1),
        "call_bytes": call_bytes, "correction_bytes": corr_bytes,
        "call_us": round(t1 + t2, 3),
        "call_frac_hbm": round(call_bytes / ((t1 + t2) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel1": {"kernel": "splitk_gemm_kernel (split-K base GEMM partials + SGMV shrink workgroups)",
                    "bytes_per_launch": k1_bytes, "mean_us": round(t1, 3),
                    "frac_hbm": round(k1_bytes / (t1 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "base_only_us": round(t1b, 3),
                    "traffic": measured_traffic("splitk_gemm_kernel<8, false, false>", "traffic_decode_q_proj.json",
                                                ("splitk.hip", "fuse.h", "shrink.h", "common.h", "kernels.h"))},
        "kernel2": {"kernel": "splitk_epilogue_kernel (split reduction + fused expand + bf16 store)",
                    "mean_us": round(t2, 3), "base_only_us": round(t2b, 3)},
        "correction_increment_us": round(max(t1 - t1b, 0.0) + max(t2 - t2b, 0.0), 3),
        "kernels": kstats(stats),
    }
    log(f"decode: {dec}")

    # warm call (one layer's weights, MALL-resident) and the launch floor
    def warm_calls():
        for _ in range(L):
            lora.linear(xs[0], Ws[0], pools[0], p, y=ys[0], workspace=ws)

    tiny = torch.zeros(1, device="cuda")

    def tiny_fills():
        for _ in range(L):
            tiny.fill_(1.0)

    warm_us = graph_us(torch, warm_calls, L)
    dec["warm_call_us"] = round(warm_us, 3)
    dec["launch_floor_us"] = round(graph_us(torch, tiny_fills, L), 3)

    # the same step with the plan built on the device (no host work per step)
    ids_dev = torch.from_numpy(ids.copy()).cuda()
    dplan = lora.plan_device(ids_dev, S)

    def dev_step():
        lora.plan_device(ids_dev, S, out=dplan)
        for l in range(L):
            lora.linear(xs[l], Ws[l], pools[l], dplan, y=ys[l], workspace=ws)

    dstep_us = graph_us(torch, dev_step, 1, reps=args.decode_steps)

    def plans_only():
        for _ in range(L):
            lora.plan_device(ids_dev, S, out=dplan)

    dec["device_plan"] = {"ms_per_step": round(dstep_us * 1e-3, 4), "plan_kernel_us": round(graph_us(torch, plans_only, L), 3),
                          "note": "lora_plan_device + 32 lora_linear_device_plan captured in one graph"}
    del pools, xs, Ws, ys, ws
    torch.cuda.empty_cache()

    if not args.no_slices:
        LQ = 8  # 8 layers of q/k/v weights (384 MiB) so the replays stream from HBM
        with ThreadPoolExecutor(8) as ex:
            qkv_host = list(ex.map(lambda l: make_qkv_decode(layer=l), range(LQ)))
        qkv = []
        for wq_ in qkv_host:
            pls = [install_pool(lora, wq_, pr) for pr in wq_.projections]
            qkv.append((lora.to_device(wq_.projections[0].x, "bf16"),
                        [lora.to_device(pr.W, "bf16") for pr in wq_.projections], pls,
                        [torch.empty((wq_.T, pr.d_out), dtype=torch.bfloat16, device="cuda")
                         for pr in wq_.projections]))
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

        us_m, us_s = graph_us(torch, merged, LQ), graph_us(torch, separate, LQ)
        rq = wq.ranks
        outs = [pr.d_out for pr in wq.projections]
        sq = acc.segments(wq.slot_ids, rq)
        a_q = sum(2 * int(rq[s_]) * d_in for s_ in sq)
        b_q = sum(2 * int(rq[s_]) * n for s_ in sq for n in outs)
        lay_bytes = 2 * wq.T * d_in + sum(2 * d_in * n + 2 * wq.T * n for n in outs) + 3 * a_q + b_q
        dec["slices"] = {"workload": f"llama3-8b q/k/v decode: T={wq.T}, {d_in}->{outs}, S={wq.S} rank 16, {LQ} layers",
                         "merged_us_per_layer": round(us_m, 3), "separate_us_per_layer": round(us_s, 3),
                         "speedup": round(us_s / us_m, 3), "bytes_per_layer": lay_bytes,
                         "merged_frac_hbm": round(lay_bytes / (us_m * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"slices: {dec['slices']}")
        del qkv, wsq
        torch.cuda.empty_cache()
    return dec


# --------------------------------------------------------------------------- other workloads
def other_configs(args, torch, np, lora, acc, make_config):
    """Single cold calls (MALL and L2 evicted before each) of configs 1, 2,
    4 and 5, each projection on its own."""
    flush = torch.empty(512 * 2**20, dtype=torch.uint8, device="cuda")
    out = {}
    for cfg in (1, 2, 4, 5):
        wc = make_config(cfg)
        pc = lora.plan(wc.slot_ids, wc.S)
        es = 2 if wc.dtype == "bf16" else 4
        for pr in wc.projections:
            pool_c = install_pool(lora, wc, pr)
            xc, Wc = lora.to_device(pr.x, wc.dtype), lora.to_device(pr.W, wc.dtype)
            yc = torch.empty((wc.T, pr.d_out), dtype=xc.dtype, device="cuda")
            wsc = pool_c.workspace(wc.T)
            lora.linear(xc, Wc, pool_c, pc, y=yc, workspace=wsc)
            torch.cuda.synchronize()
            n_c = 10
            lora.profile_begin(8 * n_c + 64)
            for _ in range(n_c):
                flush.add_(1)  # evict the MALL and L2 before each call
                lora.linear(xc, Wc, pool_c, pc, y=yc, workspace=wsc)
            sc = lora.profile_end()
            torch.cuda.synchronize()
            call_us = sum(v["median_ms"] for v in sc.values()) * 1e3
            rk = wc.ranks
            fl = acc.call_flops(wc.slot_ids, rk, pr.d_in, pr.d_out)
            by = acc.call_bytes(wc.slot_ids, rk, pr.d_in, pr.d_out, es, wc.r_max)
            entry = {"T": wc.T, "d_in": pr.d_in, "d_out": pr.d_out, "S": wc.S, "dtype": wc.dtype,
                     "call_us": round(call_us, 2), "tokens_per_s": round(wc.T / (call_us * 1e-6), 1),
                     "call_tflops": round(fl / (call_us * 1e-6) / 1e12, 3),
                     "call_frac_hbm": round(by / (call_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "kernels_median_us": {k: round(v["median_ms"] * 1e3, 2) for k, v in sc.items()}}
            if "gemm_splitk" in sc:
                a_b = sum(2 * int(rk[s_]) * pr.d_in for s_ in acc.segments(wc.slot_ids, rk))
                kb = 2 * wc.T * pr.d_in + 2 * pr.d_in * pr.d_out + a_b
                entry["kernel1_frac_hbm"] = round(kb / (sc["gemm_splitk"]["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            elif "gemm_bf16" in sc:
                # the tiled GEMM, and when it is split over K, the reduction of its partials
                gemm_ms = sc["gemm_bf16"]["median_ms"] + (sc["gemm_splitk_epilogue"]["median_ms"]
                                                          if "gemm_splitk_epilogue" in sc else 0.0)
                tf = acc.base_flops(wc.T, pr.d_in, pr.d_out) / (gemm_ms * 1e-3) / 1e12
                entry["gemm_frac_mfma"] = round(tf / BF16_PEAK_TFLOPS, 4)
            elif "gemm_generic" in sc:
                tf = acc.base_flops(wc.T, pr.d_in, pr.d_out) / (sc["gemm_generic"]["median_ms"] * 1e-3) / 1e12
                entry["gemm_frac_fp32"] = round(tf / FP32_PEAK_TFLOPS, 5)
            out[f"config{cfg} {pr.name}"] = entry
            del pool_c, xc, Wc, yc, wsc
        torch.cuda.empty_cache()
    del flush
    log(f"other configs: {out}")
    return out


# --------------------------------------------------------------------------- CPU oracle
def cpu_oracle(args, np, make_config, w3):
    """The fp64 oracle as it stands: on a bounded sample of the headline
    workload (rows spread over all 16 sequences, gate and up alternately) for
    about --cpu-seconds, and on every other workload once, all threads; the
    three smaller workloads also on one thread."""
    import oracle
    oracle.build(force=False)
    n_thr = oracle.threads()
    ids = w3.slot_ids
    order = np.random.default_rng(0).permutation(w3.T).astype(np.int32)
    done, chunk, t0 = 0, 128, time.perf_counter()
    while time.perf_counter() - t0 < args.cpu_seconds and done < w3.T * 2:
        pr = w3.projections[(done // chunk) % 2]
        rows = order[(done // 2) % w3.T:(done // 2) % w3.T + chunk]
        oracle.lora_rows("bf16", pr.x, pr.W, w3.S, pr.adapters, ids, rows=rows)
        done += len(rows)
    el = time.perf_counter() - t0
    head = {"value": round(done / el, 2), "unit": "tokens/s", "cores": n_thr, "kind": "oracle",
            "sample": f"fp64 oracle (plain C loops, OpenMP over rows), {done} rows of the T=8192 gate/up prefill "
                      f"workload ({chunk}-row batches of seeded random rows, gate and up alternately), {el:.1f} s; "
                      f"tokens through one adapted linear per second, as the GPU value"}
    log(f"cpu baseline: {head}")
    table = {}
    for cfg in (1, 2, 4, 5):
        wc = make_config(cfg)
        entry = {}
        for pr in wc.projections:
            t0 = time.perf_counter()
            oracle.lora_rows(wc.dtype, pr.x, pr.W, wc.S, pr.adapters, wc.slot_ids)
            e = {"tokens_per_s": round(wc.T / (time.perf_counter() - t0), 2), "threads": n_thr}
            if cfg in (1, 2, 4):
                oracle.set_threads(1)
                try:
                    t0 = time.perf_counter()
                    oracle.lora_rows(wc.dtype, pr.x, pr.W, wc.S, pr.adapters, wc.slot_ids)
                    e["tokens_per_s_1_thread"] = round(wc.T / (time.perf_counter() - t0), 2)
                finally:
                    oracle.set_threads(n_thr)
            entry[pr.name] = e
        table[f"config{cfg}"] = entry
    table["config3"] = {"gate_proj+up_proj": {"tokens_per_s": head["value"], "threads": n_thr,
                                              "sample_rows": done}}
    log(f"cpu oracle per workload: {table}")
    return head, table


# --------------------------------------------------------------------------- crossover
def correction_crossover(torch, np, lora, K=4096, N=4096):
    """The whole correction (shrink + expand into y) in SGMV form (plan,
    chunked items) against BGMV form (token by token, no plan), over ranks,
    adapters and tokens per adapter; graph-replayed, warm. See
    lora.correction / lora.correction_bgmv."""
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
        pool = lora.Pool(S, r, K, N, "bf16")
        A = (torch.randn(r, K, device="cuda") * 0.01).to(torch.bfloat16)
        B = (torch.randn(N, r, device="cuda") * 0.02).to(torch.bfloat16)
        for s in range(1, S):
            pool.install(s, A, B, 2.0 * r)
        x = torch.randn(T, K, device="cuda").to(torch.bfloat16)
        y = torch.zeros(T, N, device="cuda").to(torch.bfloat16)
        ids_dev = torch.from_numpy(ids).cuda()
        ws = pool.workspace(T)
        res = {"rank": r, "adapters": na, "tokens_per_adapter": tpa if kind == "uniform" else None, "T": T,
               "slots": kind}
        for chunk in (16, 32, 64, 128):
            pl = lora.plan(ids, S, chunk=chunk)
            res[f"sgmv{chunk}_us"] = round(graph_us(torch, lambda: lora.correction(x, pool, pl, y, workspace=ws), 8), 2)
        res["bgmv_us"] = round(graph_us(torch, lambda: lora.correction_bgmv(x, pool, ids_dev, y, workspace=ws), 8), 2)
        best = min((v, k) for k, v in res.items() if k.endswith("_us"))
        res["fastest"] = best[1][:-3]
        rows.append(res)
        log(f"crossover {res}")
        del pool, A, B, x, y, ws
    return rows


def ceilings(torch):
    """What library kernels reach on this machine, as reproducible reference
    points for the rooflines: a plain device-to-device copy of 1 GiB (read +
    write bytes per second) and hipBLASLt's bf16 GEMM at 8192 x 8192 x 8192 in
    the base product's layout, each timed with stream events, best of 3
    rounds."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_us(fn, n=10):
        fn()
        torch.cuda.synchronize()
        t = []
        for _ in range(3):
            ev0.record()
            for _ in range(n):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            t.append(ev0.elapsed_time(ev1) / n * 1e3)
        return min(t)

    src = torch.empty(2**30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    cp_us = best_us(lambda: dst.copy_(src))
    del src, dst
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    c = torch.empty(8192, 8192, device="cuda", dtype=torch.bfloat16)
    mm_us = best_us(lambda: torch.nn.functional.linear(a, b, out=c), 5)
    del a, b, c
    torch.cuda.empty_cache()
    out = {"hbm_copy": {"bytes": 2 * 2**30, "us": round(cp_us, 1), "tbps": round(2 * 2**30 / cp_us / 1e6, 3),
                        "frac_of_8tbps": round(2 * 2**30 / cp_us / 1e3 / HBM_PEAK_GBS, 4),
                        "note": "torch device-to-device copy of 1 GiB; read + write bytes"},
           "library_gemm": {"shape": "8192 x 8192 x 8192 bf16", "us": round(mm_us, 1),
                            "tflops": round(2 * 8192**3 / mm_us / 1e6, 1),
                            "frac_of_peak": round(2 * 8192**3 / mm_us / 1e6 / BF16_PEAK_TFLOPS, 4),
                            "note": "torch.nn.functional.linear (hipBLASLt), x [M, K] times W [N, K] transposed, "
                                    "the layout of the base product"}}
    log(f"ceilings {out}")
    return out


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

    t0 = time.perf_counter()
    w3 = make_config(3)
    log(f"generated the gate/up prefill workload in {time.perf_counter() - t0:.1f}s")
    value = ms_per_step = roof = call = base = None
    hstats = {}
    if not args.decode_only:
        value, ms_per_step, roof, call, base, hstats = headline(args, torch, np, lora, acc, w3)

    dec = None if args.no_decode else decode_step(args, torch, np, lora, acc, make_config, make_qkv_decode)
    others = None if args.no_configs else other_configs(args, torch, np, lora, acc, make_config)
    crossover = None if args.no_crossover else correction_crossover(torch, np, lora)
    ceil = None if (args.no_library or args.no_configs) else ceilings(torch)

    if args.copy_calibration:
        src = torch.empty(256 * 2**20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 5 x 256 MiB device copies")

    cpu, cpu_table = (None, None) if args.no_cpu_baseline else cpu_oracle(args, np, make_config, w3)

    pr = w3.projections[0]
    out = {
        "metric": METRIC, "value": None if value is None else round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": None if ms_per_step is None else round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"llama3-8b gate_proj + up_proj prefill: T={w3.T} (16 sequences x 512, each on one "
                               f"slot drawn from 0..16), {pr.d_in}->{pr.d_out}, S={w3.S} (rank 16, alpha 32), "
                               f"plan + lora_linear_multi(gate, up) per step (one shared shrink, two GEMMs)",
                   "T": w3.T, "d_in": pr.d_in, "d_out": pr.d_out, "S": w3.S, "rank": 16, "projections_per_step": 2,
                   "value_is": "tokens through one adapted linear per second = 2 T / step time",
                   "mode": "eager calls; plan computed on the host and copied ahead of the step's kernels; "
                           "no per-kernel events in this pass"},
        "roofline": roof, "cpu_baseline": cpu,
        "call": call, "kernels": kstats(hstats), "base_only": base,
        "decode": dec, "other_configs": others, "cpu_oracle": cpu_table, "correction_crossover": crossover,
        "ceilings": ceil,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
