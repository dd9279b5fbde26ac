"""Benchmark of the MoE layer share on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config tp_share]

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: route -> permute -> gate/up grouped GEMM with the
SiLU*up epilogue -> down grouped GEMM -> top-k weighted combine (moe_layer).
About 200 ms of untimed back-to-back steps (the clocks of the part move for
several milliseconds after work starts), then W untimed warmup steps, then
exactly K timed steps bracketed by device synchronizations.  Per-kernel durations come from HIP events recorded on the
launch stream around each step of the same path called entry point by entry
point (medians; a grouped GEMM entry point also builds its row-task plan),
and, for the short HBM-bound combine and row gather, from HIP graphs of
back-to-back calls over buffers that do not fit the Infinity Cache.  Also reported: per-step percentiles with the Infinity Cache warm and
flushed (a 512 MiB write before each step, outside the events), the
weighted-scatter variant of the combine (moe_layer_ex), and the part's
measured MFMA and HBM-read peaks next to the published ones.  Prints one
JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6   # dense bf16 / fp16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="untimed back-to-back steps for this long before the W warmup steps, "
                        "so the part's clocks have settled when the timed region starts")
    p.add_argument("--config", default="tp_share")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample (0 disables it)")
    p.add_argument("--cpu-seconds-other", type=float, default=4.0,
                   help="the same for each of the other workloads")
    p.add_argument("--others", default="dense,ep_skew,ep_skew_small,prefill",
                   help="other workloads measured in the same run (comma list; '' for none)")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="instead of the layer, run a plain device copy of MIB MiB a few times "
                        "(reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return p.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(collectives and sharding are out of scope); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from moe_expert_grouped_amd import synthetic as syn

    torch.cuda.set_device(0)
    if a.calibrate_copy:
        calibrate_copy(a.calibrate_copy)
        return
    meta = run_meta(torch)
    if syn.CONFIGS[a.config]["kind"] == "dense":
        rec = bench_dense(a, headline=True)
    else:
        rec = bench_moe(a, a.config, headline=True)
    others = [c for c in (a.others.split(",") if a.others else []) if c and c != a.config]
    if others:
        # every other workload, in the same run: layer (or GEMM) time, per-kernel
        # times, the roofline of its dominant kernel and the oracle beside it
        rec["configs"] = {}
        for name in others:
            print("[bench] %s" % name, file=sys.stderr, flush=True)
            if syn.CONFIGS[name]["kind"] == "dense":
                rec["configs"][name] = bench_dense(a, headline=False)
            else:
                rec["configs"][name] = bench_moe(a, name, headline=False)
            torch.cuda.empty_cache()
    meta["clocks_after"] = gpu_clocks(getattr(torch.cuda.get_device_properties(0), "pci_bus_id", None))
    rec["meta"] = meta
    print(json.dumps(rec), flush=True)


def bench_moe(a, name, headline):
    """One MoE layer share: the whole step (moe_layer) timed, its kernels one
    by one, the roofline of the gate/up GEMM and the oracle beside it.  The
    headline workload also times the weighted-scatter combine, the graph-
    replayed step, the plain weight layout and the short HBM-bound steps in
    graph-captured batches."""
    import torch
    import moe_expert_grouped_amd as moe
    from moe_expert_grouped_amd import synthetic as syn
    cfg = syn.CONFIGS[name]
    d = syn.make_config(name)
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    sha = input_sha256(d)
    dev16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    x, wg, wu, wd = dev16(d["x"]), dev16(d["wg"]), dev16(d["wu"]), dev16(d["wd"])
    given = "logits" not in d
    logits = None if given else torch.from_numpy(d["logits"]).cuda()
    tidx = torch.from_numpy(d["topk_idx"]).cuda() if given else None
    tw = torch.from_numpy(d["topk_w"]).cuda() if given else None
    ws = moe.layer_workspace(T, H, E, k, I, combine="scatter" if headline else "gather")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    # gate and up weights interleaved in 128-column blocks, once, before any
    # timing (a weight-load transform: the gate/up GEMM then streams each k row
    # of a weight tile as one 512-byte piece); the plain layout is timed too
    packed = I % 128 == 0
    # moe_layer's rule: weights loaded non-temporally when the experts
    # average at most two 128-row blocks (each weight tile read about once)
    stream_w = T * k <= 2 * 128 * E
    wgu = moe.pack_gate_up(wg, wu) if packed else wg
    wu_arg = None if packed else wu
    torch.cuda.synchronize()

    def step():
        moe.layer(x, wgu, wu_arg, wd, k, logits=logits, topk_idx=tidx, topk_w=tw, workspace=ws,
                  out=out)

    settle_steps = settle(step, a.settle_ms if headline else a.settle_ms / 2)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / a.steps
    stats = step_stats(step, a.steps)

    # ---- per-kernel durations: HIP events on the launch stream around each
    # kernel of the same path called step by step.  The GEMMs run on a plan
    # built once beforehand (plan_ready), as inside moe_layer, where the
    # permutation kernel writes it: each pair of events brackets one kernel.
    stream = torch.cuda.current_stream()
    names = ["route", "permute", "gate_up", "down", "combine"]
    R = T * k
    idx_t, w_t = (tidx, tw) if given else moe.route(logits, k)
    P = moe.permute(idx_t, E)
    gws = torch.empty(moe.load_library().grouped_gemm_workspace_size(P.cap), dtype=torch.uint8,
                      device="cuda")
    gu_kw = dict(N=I, K=H, cap=P.cap, a_src_row=P.row_to_pair, a_src_div=k, B2=wu_arg,
                 epilogue="silu_mul", b_layout="kn_gate_up" if packed else "kn", b_stream=stream_w,
                 workspace=gws)
    dn_kw = dict(N=H, K=I, cap=P.cap, row_pair=P.row_to_pair, b_stream=stream_w, workspace=gws)
    h = moe.grouped_gemm(x, wgu, P.block_expert, P.num_padded_rows, **gu_kw)  # builds the plan
    y = moe.grouped_gemm(h, wd, P.block_expert, P.num_padded_rows, plan_ready=True, **dn_kw)
    timed = []
    for it in range(a.warmup + a.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        e[0].record(stream)
        if not given:
            moe.route(logits, k)
        e[1].record(stream)
        moe.permute(idx_t, E)
        e[2].record(stream)
        moe.grouped_gemm(x, wgu, P.block_expert, P.num_padded_rows, out=h, plan_ready=True, **gu_kw)
        e[3].record(stream)
        moe.grouped_gemm(h, wd, P.block_expert, P.num_padded_rows, out=y, plan_ready=True, **dn_kw)
        e[4].record(stream)
        moe.combine(y, P.pair_to_row, w_t, out=out)
        e[5].record(stream)
        if it >= a.warmup:
            timed.append(e)
    torch.cuda.synchronize()
    per = {n: np.array([es[i].elapsed_time(es[i + 1]) for es in timed]) * 1e3
           for i, n in enumerate(names)}
    # medians (a stalled host iteration would otherwise move the mean) and means
    dur = {n: float(np.median(v)) for n, v in per.items()}
    mean = {n: float(np.mean(v)) for n, v in per.items()}
    m_pad = int(P.num_padded_rows.item())
    counts = P.counts.cpu().numpy()
    e_act = int((counts > 0).sum())

    # ---- algorithmic work
    gemm_flops = 6.0 * R * H * I
    gu_flops = 4.0 * R * H * I
    gu_bytes = 4.0 * e_act * H * I + 2.0 * T * H + 2.0 * R * I      # weights, x, h
    dn_bytes = 2.0 * e_act * I * H + 2.0 * R * I + 2.0 * R * H      # weights, h, y
    comb_bytes = 2.0 * R * H + 2.0 * T * H                          # y rows read, out written
    layer_s = ms * 1e-3
    gemm_s = (dur["gate_up"] + dur["down"]) * 1e-6
    # the roofline of the dominant kernel, the gate/up GEMM: HBM-bound where
    # its FLOPs per byte stay under the ridge (peak FLOP/s / peak bytes/s)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    # the GEMM kernel alone on its prebuilt plan: 100 ms of it untimed, then
    # launches back to back
    n_roof = max(a.steps, 100)
    gu_us = batch_us(lambda: moe.grouped_gemm(x, wgu, P.block_expert, P.num_padded_rows, out=h,
                                              plan_ready=True, **gu_kw), n_roof)
    if gu_flops / gu_bytes < ridge:
        roof = {"bound": "hbm", "achieved": round(gu_bytes / (gu_us * 1e-6) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "algorithmic_bytes": gu_bytes}
    else:
        roof = {"bound": "mfma", "achieved": round(gu_flops / (gu_us * 1e-6) / 1e12, 1),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "algorithmic_flops": gu_flops}
    roof = {"kernel": "grouped_gemm gate/up (SiLU*up epilogue), the GEMM kernel alone", **roof,
            "frac": round(roof["achieved"] / roof["peak"], 4),
            "duration_us": round(gu_us, 2), "launches": n_roof,
            "timing": "one HIP event pair around %d back-to-back launches, after 100 ms of the "
                      "same untimed" % n_roof,
            "traffic": recorded_traffic("grouped_gemm_gate_up_%s" % name)}

    rec = {
        "metric": "MoE layer us + grouped-GEMM TFLOP/s (% bf16 MFMA peak), T=2048 H=4096 E=64",
        "value": round(gemm_flops / layer_s / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup, "settle_steps": settle_steps,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s MoE layer share" % name, "T": T, "H": H, "E": E, "top_k": k,
                   "I": I, "routing": cfg.get("routing"), "m_pad": m_pad, "active_experts": e_act,
                   "gate_up_weights": ("interleaved in 128-column blocks (moe_pack_gate_up, once "
                                       "before timing)") if packed else "separate [E][H][I]",
                   "weight_loads": "non-temporal" if stream_w else "default"},
        "layer_us": round(ms * 1e3, 2),
        "gemm_tflops": round(gemm_flops / gemm_s / 1e12, 2),
        "gemm_mfma_peak_frac": round(gemm_flops / gemm_s / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernel_us": {n: round(v, 2) for n, v in dur.items()},
        "kernel_us_mean": {n: round(v, 2) for n, v in mean.items()},
        "layer_us_per_step": stats,
        "roofline": roof,
        "input_sha256": sha,
    }
    if name == "ep_skew_small":
        # the one workload with less than one wave of GEMM tasks: the layer
        # with split K (MOE_LAYER_SPLIT_K) against without, interleaved, and
        # a decode-sized share of the same experts
        rec["split_k_ab"] = split_k_ab(a, d, step, dict(wgu=wgu, wu_arg=wu_arg, wd=wd, ws=ws, out=out))
    hbm = [("gate_up", dur["gate_up"], gu_bytes), ("down", dur["down"], dn_bytes),
           ("combine", dur["combine"], comb_bytes)]
    if headline:
        rec.update(moe_headline_legs(a, d, locals()))
        hbm = [hbm[0], hbm[1], ("combine", rec["kernel_us_batched"]["combine"], comb_bytes),
               ("gather", rec["kernel_us_batched"]["gather"], 2.0 * T * H + 2.0 * m_pad * H),
               ("router", rec["kernel_us_batched"]["router"], 2.0 * T * H + 2.0 * E * H + 8.0 * T * k)]
    rec["hbm_gbs"] = {
        n: {"us": round(us, 2), "algorithmic_bytes": b, "gbs": round(b / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)} for n, us, b in hbm}
    wr_bits = rec.pop("_wr_bits", None)
    if a.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_baseline(d, a.cpu_seconds if headline else a.cpu_seconds_other)
        if wr_bits is not None:
            rec["cpu_baseline_router"] = cpu_router_baseline(d["x"], wr_bits, k)
    if not headline:
        for key in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline",
                    "data"):
            rec.pop(key)
    return rec


def split_k_ab(a, d, step, v):
    """Layer us per step, 5 interleaved rounds of back-to-back steps, without
    and with split K: on this workload's share, and on the first 16 of its
    tokens routed by the same recipe (a decode-sized batch, few row tasks)."""
    import torch
    import moe_expert_grouped_amd as moe
    from moe_expert_grouped_amd import synthetic as syn
    H, E, k, I = d["H"], d["E"], d["k"], d["I"]
    res = {}
    n = max(a.steps // 5, 20)
    for T in (d["T"], 16):
        s = d if T == d["T"] else syn.make_moe(T, H, E, k, I, routing="zipf", seed=0, with_weights=False)
        x = torch.from_numpy(s["x"].view(np.int16)).view(torch.bfloat16).cuda()
        kw = dict(topk_idx=torch.from_numpy(s["topk_idx"]).cuda(), topk_w=torch.from_numpy(s["topk_w"]).cuda())
        out = v["out"][:T]

        def run(split):
            moe.layer(x, v["wgu"], v["wu_arg"], v["wd"], k, workspace=v["ws"], out=out, split_k=split, **kw)

        r = {"unsplit": [], "split": [], "active_experts": int(np.unique(s["topk_idx"]).size)}
        settle(lambda: run(False), 50.0)
        for _ in range(5):
            r["unsplit"].append(round(batch_us(lambda: run(False), n, settle_ms=0.0), 2))
            r["split"].append(round(batch_us(lambda: run(True), n, settle_ms=0.0), 2))
        res["T%d" % T] = r
    return {"what": "layer us per step, 5 interleaved rounds of %d back-to-back steps, unsplit "
                    "against split K (MOE_LAYER_SPLIT_K); T16: the first Zipf draw of 16 tokens "
                    "over the same experts" % n, **res}


def moe_headline_legs(a, d, v):
    """The extra legs of the headline workload: the weighted-scatter combine,
    the graph-replayed step, the plain gate/up weight layout, and the combine,
    permutation, row gather and router front end in graph-captured batches."""
    import torch
    import moe_expert_grouped_amd as moe
    from moe_expert_grouped_amd import synthetic as syn
    T, H, E, k = d["T"], d["H"], d["E"], d["k"]
    x, wg, wu, wd, wgu, wu_arg = v["x"], v["wg"], v["wu"], v["wd"], v["wgu"], v["wu_arg"]
    logits, tidx, tw, ws, out, step = v["logits"], v["tidx"], v["tw"], v["ws"], v["out"], v["step"]
    P, h, y, idx_t, w_t, dn_kw = v["P"], v["h"], v["y"], v["idx_t"], v["w_t"], v["dn_kw"]
    stream = torch.cuda.current_stream()

    def step_scatter():
        moe.layer(x, wgu, wu_arg, wd, k, logits=logits, topk_idx=tidx, topk_w=tw, workspace=ws,
                  out=out, combine="scatter")

    for _ in range(a.warmup):
        step_scatter()
    stats_scatter = step_stats(step_scatter, a.steps, cold=False)

    # the same step captured once in a HIP graph and replayed (no host launch
    # cost per kernel; the layer launches kernels only, so it captures whole)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(a.warmup):
        graph.replay()
    # back-to-back replays between one event pair: an event pair around each
    # replay would also hold the host's graph-launch time before the first
    # kernel (the GPU is idle by then), not the step's
    graph_us = batch_us(graph.replay, max(a.steps, 50), settle_ms=50.0)
    del graph

    def step_unpacked():
        moe.layer(x, wg, wu, wd, k, logits=logits, topk_idx=tidx, topk_w=tw, workspace=ws, out=out)

    for _ in range(a.warmup):
        step_unpacked()
    stats_unpacked = step_stats(step_unpacked, a.steps, cold=False)

    # the permutation as its own launch instead of inside the gate/up GEMM's
    # prologue (the layer's default where the shape allows), interleaved
    # with the default so both see the same clocks
    def step_separate():
        moe.layer(x, wgu, wu_arg, wd, k, logits=logits, topk_idx=tidx, topk_w=tw, workspace=ws,
                  out=out, separate_permute=True)

    for _ in range(a.warmup):
        step_separate()
    ab = {"fused": [], "separate": []}
    for _ in range(5):
        ab["fused"].append(step_stats(step, max(a.steps // 5, 4), cold=False)["warm"]["median"])
        ab["separate"].append(step_stats(step_separate, max(a.steps // 5, 4), cold=False)["warm"]["median"])

    # the weighted-scatter down GEMM (alone, on the plan built before) and its finalize
    acc = torch.empty((T, H), dtype=torch.float32, device="cuda")
    sc = []
    for it in range(a.warmup + a.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        acc.zero_()
        e[1].record(stream)
        moe.grouped_gemm(h, wd, P.block_expert, P.num_padded_rows, epilogue="weighted_scatter",
                         pair_w=w_t, out=acc, plan_ready=True, **dn_kw)
        e[2].record(stream)
        moe.finalize(acc, out=out)
        e[3].record(stream)
        if it >= a.warmup:
            sc.append(e)
    torch.cuda.synchronize()
    dur_sc = {n: float(np.median([es[i].elapsed_time(es[i + 1]) for es in sc]))
              for i, n in enumerate(["zero", "down_scatter", "finalize"])}
    # the short HBM-bound entry points without event packets between kernels:
    # a.steps calls captured back to back in one HIP graph, replayed between
    # two HIP events.  The combine's y and the gather's x_perm rotate over
    # enough buffers (400 MB, 308 MB) that none is still in the 256 MB
    # Infinity Cache when it is read or rewritten, so the rates are HBM rates.
    out_b = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ys = [y.clone() for _ in range(4)]
    xps = [torch.empty((P.cap, H), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    rot = {"y": 0, "xp": 0}

    def next_buf(name, bufs):
        rot[name] = (rot[name] + 1) % len(bufs)
        return bufs[rot[name]]
    pws = torch.empty(max(moe.load_library().moe_permute_workspace_size(T, k, E), 256),
                      dtype=torch.uint8, device="cuda")
    batched = {
        "combine": graph_batch_us(
            lambda: moe.combine(next_buf("y", ys), P.pair_to_row, w_t, out=out_b), a.steps),
        "permute": graph_batch_us(lambda: moe.permute(idx_t, E, workspace=pws), a.steps),
        "permute_with_gather": graph_batch_us(
            lambda: moe.permute(idx_t, E, x=x, x_perm=next_buf("xp", xps), workspace=pws),
            a.steps),
    }
    # the router front end (moe_router: logits = x . W_r^T, then the routing)
    # on the same tokens, with seeded router weights [E][H]
    wr_bits = syn.bf16_bits((np.random.default_rng(7).standard_normal((E, H)) /
                             np.sqrt(H)).astype(np.float32))
    wr = torch.from_numpy(wr_bits.view(np.int16)).view(torch.bfloat16).cuda()
    rws = torch.empty(max(moe.load_library().moe_router_workspace_size(T, H, E), 256),
                      dtype=torch.uint8, device="cuda")
    # one launch: logits, top-k, softmax and the per-expert counts
    batched["router"] = graph_batch_us(lambda: moe.router(x, wr, k, workspace=rws, with_counts=True),
                                       a.steps)
    # the whole layer from x and W_r (moe_layer_router: the router front end,
    # then the permutation on its counts, the GEMMs and the combine)
    lws = torch.empty(moe.load_library().moe_layer_router_workspace_size(T, H, E, k, d["I"], 0),
                      dtype=torch.uint8, device="cuda")

    def step_router():
        moe.layer_router(x, wr, wgu, wu_arg, wd, k, workspace=lws, out=out)

    for _ in range(a.warmup):
        step_router()
    # interleaved with the layer from logits, so both see the same clocks;
    # back-to-back steps between one event pair per round
    n_r = max(a.steps // 5, 10)
    ab_router = {"from_logits": [], "from_router": []}
    for _ in range(5):
        ab_router["from_logits"].append(round(batch_us(step, n_r, settle_ms=0.0), 2))
        ab_router["from_router"].append(round(batch_us(step_router, n_r, settle_ms=0.0), 2))
    # the row gather alone: the permutation with it minus the permutation
    batched["gather"] = batched["permute_with_gather"] - batched["permute"]
    del ys, xps
    return {
        "kernel_us_batched": {n: round(t, 2) for n, t in batched.items()},
        "hip_graph": {"layer_us_per_step": round(graph_us, 2),
                      "timing": "one HIP event pair around %d back-to-back replays" % max(a.steps, 50)},
        "unpacked_gate_up_weights": {"layer_us_per_step": stats_unpacked},
        "front_end_ab": {"what": "layer step medians (us), 5 interleaved rounds: the reorder by route "
                                 "inside the gate/up GEMM prologue (fused, the default) against the "
                                 "permutation as its own launch (separate)",
                         "fused": ab["fused"], "separate": ab["separate"]},
        "layer_with_router_front_end": {
            "what": "layer us per step, 5 interleaved rounds of %d back-to-back steps: from the "
                    "router logits (route kernel) against from x and W_r (moe_layer_router)" % n_r,
            **ab_router},
        "scatter_combine": {"layer_us_per_step": stats_scatter,
                            "kernel_us": {n: round(t * 1e3, 2) for n, t in dur_sc.items()}},
        "measured_peaks": measured_peaks(),
        "_wr_bits": wr_bits,
    }


def bench_dense(a, headline):
    """The degenerate one-group case: D = A . B^T, fp16 4096^3 (B stored [N][K])."""
    import torch
    import moe_expert_grouped_amd as moe
    from moe_expert_grouped_amd import synthetic as syn
    d = syn.make_config("dense")
    M, N, K = d["M"], d["N"], d["K"]
    sha = input_sha256(d)
    dev16 = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.float16).cuda()
    A, B = dev16(d["A"]), dev16(d["B"])
    bg = torch.zeros(M // 128, dtype=torch.int32, device="cuda")
    nr = torch.tensor([M], dtype=torch.int32, device="cuda")
    D = torch.empty((M, N), dtype=torch.float16, device="cuda")
    ws = moe.gemm_workspace(M)

    def step():
        moe.grouped_gemm(A, B, bg, nr, N=N, K=K, cap=M, b_layout="nk", out=D, workspace=ws)

    settle_steps = settle(step, a.settle_ms if headline else a.settle_ms / 2)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(a.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / a.steps
    # the GEMM kernel alone (its plan built by the calls above), launches
    # back to back after 100 ms of the same: five batches, the mean of their
    # per-launch means
    n_batch = max(a.steps // 5, 20)
    us = np.array([batch_us(lambda: moe.grouped_gemm(A, B, bg, nr, N=N, K=K, cap=M, b_layout="nk",
                                                     out=D, workspace=ws, plan_ready=True), n_batch,
                            settle_ms=100.0 if i == 0 else 0.0)
                   for i in range(5)])
    kern_us = float(np.mean(us))
    flops = 2.0 * M * N * K
    tf = flops / (kern_us * 1e-6) / 1e12
    rec = {
        "metric": "dense fp16 GEMM D = A.B^T (one-group grouped_gemm)", "value": round(tf, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "settle_steps": settle_steps,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "config": {"workload": "dense fp16 GEMM M=N=K=4096, D = A.B^T, fp32 accumulate"},
        "step_us": round(ms * 1e3, 2),
        "kernel_us": round(kern_us, 2), "kernel_us_batches": [round(float(u), 2) for u in us],
        "roofline": {"kernel": "grouped_gemm (one group, B [N][K], fp16), the GEMM kernel alone",
                     "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "duration_us": round(kern_us, 2), "algorithmic_flops": flops, "launches": 5 * n_batch,
                     "timing": "five HIP event pairs, each around %d back-to-back launches" % n_batch,
                     "traffic": None},
        "input_sha256": sha,
    }
    if a.cpu_seconds > 0:
        rec["cpu_baseline"] = cpu_dense_baseline(d, a.cpu_seconds if headline else a.cpu_seconds_other)
    if not headline:
        for key in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline",
                    "data"):
            rec.pop(key)
    return rec


def input_sha256(d):
    """SHA-256 of every input array of a workload (numpy does not promise the
    same Generator streams across versions: the hashes name the bits)."""
    import hashlib
    out = {}
    for n, v in d.items():
        if isinstance(v, np.ndarray):
            out[n] = hashlib.sha256(memoryview(np.ascontiguousarray(v)).cast("B")).hexdigest()
    return out


def gpu_clocks(pci_bus=None):
    """Current shader and memory clock levels and the power figures of the
    GPU, read from the amdgpu driver's sysfs files (the clocks are recorded,
    not locked); None where they are not readable.  No tool is started, so
    this also works under a profiler that preloads itself into children."""
    import glob
    devs = sorted(os.path.dirname(f) for f in glob.glob("/sys/class/drm/card[0-9]*/device/pp_dpm_sclk"))
    if pci_bus is not None:
        same = [d for d in devs if os.path.basename(os.path.realpath(d)).split(":")[1:2] == ["%02x" % pci_bus]]
        devs = same or devs
    if not devs:
        return None
    dev = devs[0]

    def read(path):
        try:
            with open(path) as f:
                return f.read()
        except OSError:
            return None

    out = {"card": os.path.basename(os.path.dirname(dev)), "pci": os.path.basename(os.path.realpath(dev))}
    for key in ("sclk", "mclk"):
        txt = read(os.path.join(dev, "pp_dpm_%s" % key)) or ""
        cur = [ln.strip() for ln in txt.splitlines() if ln.rstrip().endswith("*")]
        out[key] = cur[0] if cur else None
    for hw in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
        for name in ("power1_cap", "power1_average", "power1_input"):
            v = read(os.path.join(hw, name))
            if v is not None and v.strip().isdigit():
                out[name + "_w"] = int(v) / 1e6
    return out


def run_meta(torch):
    import platform
    p = torch.cuda.get_device_properties(0)
    return {"numpy": np.__version__, "torch": torch.__version__, "hip": torch.version.hip,
            "device": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "host_cpu": platform.processor() or platform.machine(),
            "host_threads": len(os.sched_getaffinity(0)),
            "clocks_before": gpu_clocks(getattr(p, "pci_bus_id", None))}


CSRC = os.path.join(ROOT, "moe_expert_grouped_amd", "csrc")
GEMM_SRCS = [os.path.join(CSRC, f)
             for f in ("gg_kernel.h", "gg_inst.hip", "grouped_gemm.hip", "common.h")]
PROFILES = os.path.join(ROOT, "profiles")


def gemm_source_sha256():
    """SHA-256 of the grouped GEMM sources (kernel header, instantiation
    unit, dispatcher, shared device helpers), concatenated in that order, with // comments and
    blank lines dropped and runs of whitespace folded: comment edits do not
    change the code the counters were taken on."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in GEMM_SRCS:
        for line in open(f, encoding="utf-8"):
            code = re.sub(r"\s+", " ", re.sub(r"//.*", "", line)).strip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def _pcts(ms):
    us = np.asarray(ms) * 1e3
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2), "n": int(len(us))}


def graph_batch_us(fn, n):
    """Mean microseconds per call of `fn` over n calls captured back to back in
    one HIP graph, replayed between two HIP events (for entry points whose
    kernels are shorter than their host-side call)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            fn()
    graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) * 1e3 / n


def batch_us(fn, n, settle_ms=100.0, lead=4):
    """Mean duration of one call of `fn` (one kernel launch): `n` calls
    enqueued back to back between one pair of HIP events on the launch
    stream.  The same call runs untimed for `settle_ms` first (from idle the
    shader clock needs some tens of milliseconds of load to reach its
    steady level), then `lead` more so the host is ahead of the GPU and the
    queue never runs dry inside the timed region; one event pair per batch
    keeps the marker packets' own few microseconds out of the figure."""
    import torch
    settle(fn, settle_ms)
    stream = torch.cuda.current_stream()
    for _ in range(lead):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def settle(step, ms):
    """Run `step` back to back, untimed, for about `ms` milliseconds of wall
    time (at most 20000 steps); returns the number of steps run."""
    import torch
    if ms <= 0:
        return 0
    n, t0 = 0, time.perf_counter()
    while n < 20000:
        for _ in range(16):
            step()
        n += 16
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            break
    return n


def step_stats(step, n, cold=True):
    """Per-step layer time from HIP events on the launch stream: with the
    caches warm (steps back to back), and, if `cold`, with a 512 MiB write
    before every step (outside the events) to evict the 256 MB Infinity Cache."""
    import torch
    stream = torch.cuda.current_stream()
    res = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if cold else None
    for mode in (("warm", "cold") if cold else ("warm",)):
        ev = []
        for i in range(n):
            if mode == "cold":
                flush.fill_(i & 0xff)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        res[mode] = _pcts([a.elapsed_time(b) for a, b in ev])
    del flush
    return res


PEAK_LIB = os.path.join(ROOT, "moe_expert_grouped_amd", "libmoe_peak_gfx950.so")


def measured_peaks():
    """The part's MFMA-only bf16 throughput and read-only HBM bandwidth,
    measured with the kernels of libmoe_peak_gfx950.so (median of 5)."""
    import ctypes
    import torch
    if not os.path.exists(PEAK_LIB):
        return None
    lib = ctypes.CDLL(PEAK_LIB)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moe_peak_mfma_flops.argtypes, lib.moe_peak_mfma_flops.restype = [I, I], ctypes.c_longlong
    lib.moe_peak_mfma.argtypes, lib.moe_peak_mfma.restype = [I, I, P, P], I
    lib.moe_peak_read.argtypes, lib.moe_peak_read.restype = [P, Z, I, P, P], I
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def timed(launch, reps=5):
        launch()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if launch() != 0:
                raise RuntimeError("peak kernel launch failed")
            e1.record(stream)
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e-3

    wgs, iters = 2 * cus, 20000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    t = timed(lambda: lib.moe_peak_mfma(wgs, iters, ctypes.c_void_p(sink.data_ptr()), sp))
    mfma = lib.moe_peak_mfma_flops(wgs, iters) / t / 1e12
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    rwgs = 8 * cus
    rsink = torch.empty(rwgs, dtype=torch.int32, device="cuda")
    t = timed(lambda: lib.moe_peak_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rwgs,
                                        ctypes.c_void_p(rsink.data_ptr()), sp))
    hbm = nbytes / t / 1e9
    del buf
    return {"mfma_bf16_tflops": round(mfma, 1), "mfma_published": PEAK_BF16_TFLOPS,
            "hbm_read_gbs": round(hbm, 1), "hbm_published": PEAK_HBM_GBS,
            "how": "MFMA-only loop (8 independent 32x32x16 bf16 chains per wavefront, %d workgroups); "
                   "read-only stream of 2 GiB, 16-byte loads, 1 MiB contiguous per workgroup" % wgs}


def recorded_traffic(name):
    """HBM bytes per launch of a kernel from its committed rocprof counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy calibration),
    or None when there is none or the kernel source changed since."""
    import hashlib
    path = os.path.join(PROFILES, name + ".md")
    if not os.path.exists(path):
        return None
    want = gemm_source_sha256()
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith(("traffic_bytes_per_launch", "kernel_source_sha256")):
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != want:
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(d, target_s):
    """The oracle, untuned, on a bounded sample of tokens of the same workload."""
    import oracle
    T, H, E, k, I = d["T"], d["H"], d["E"], d["k"], d["I"]
    if "logits" in d:
        idx, w = oracle.route(d["logits"], k)
    else:
        idx, w = d["topk_idx"], d["topk_w"]
    n = 8
    rng = np.random.default_rng(0)
    while True:
        toks = np.sort(rng.choice(T, min(n, T), replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.moe_tokens(d["x"], idx, w, d["wg"], d["wu"], d["wd"], tokens=toks)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= T:
            break
        n = int(min(T, max(2 * n, n * target_s / max(dt, 1e-3) * 1.1)))
    flops = 6.0 * len(toks) * k * H * I
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "%d of %d tokens (all %d routed slots each), fp64 per-token loops" % (len(toks), T, k)}


def cpu_router_baseline(x_bits, wr_bits, k):
    """The oracle of the router front end (fp64 logits, then the routing) on
    all tokens of the workload, beside the router leg."""
    import oracle
    t0 = time.perf_counter()
    lg = oracle.router_logits(x_bits, wr_bits)
    oracle.route(lg.astype(np.float32), k)
    dt = time.perf_counter() - t0
    return {"value": round(dt * 1e6, 1), "unit": "us per call", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "all %d tokens: fp64 logits x . W_r^T, then the top-%d routing" % (x_bits.shape[0], k)}


def cpu_dense_baseline(d, target_s):
    """The oracle of the dense case on a bounded sample of output rows."""
    import oracle
    M, N, K = d["M"], d["N"], d["K"]
    B = d["B"].reshape(1, N, K)
    bg = np.zeros(M // 128, np.int32)
    n = 8
    rng = np.random.default_rng(0)
    while True:
        rows = np.sort(rng.choice(M, min(n, M), replace=False)).astype(np.int32)
        t0 = time.perf_counter()
        oracle.grouped_gemm(d["A"], B, bg, N=N, K=K, is_fp16=True, b_layout="nk", rows=rows)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= M:
            break
        n = int(min(M, max(2 * n, n * target_s / max(dt, 1e-3) * 1.1)))
    flops = 2.0 * len(rows) * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "%d of %d rows of D, fp64 dot products" % (len(rows), M)}


if __name__ == "__main__":
    main()
