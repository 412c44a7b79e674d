"""Benchmark of the MoE dispatch hot path on one MI355X.

One step is one pass of the whole path over one batch of the large skewed
prefill workload (32768 tokens, 256 experts with Zipf-skewed load, top-8,
hidden 7168):
    top-k gating -> token map (counts, offsets, positions) ->
    fused expand + per-128-channel e4m3 cast (262144 expert-grouped rows) ->
    SwiGLU + e4m3 cast over the batch's 262144 routed rows (I = 2048,
    U(0,1) routing weights).
Inputs are seeded synthetic data, resident in HBM before timing starts.

Output: one JSON line.  value = algorithmic HBM bytes of the step / step time
(GB/s); roofline = the dominant kernel's algorithmic GB/s from HIP events on
its stream vs MI355X's 8 TB/s; cpu_baseline = the CPU oracle timed on a
bounded sample of the same batch (1 host thread).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + tokens/s for top-k→expand→FP8 cast, 1 GPU"
HBM_PEAK_GBS = 8000.0
SWIGLU_INTER = 2048
EVENT_EVERY = 8  # timed steps per step that carries the per-stage events


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="large", choices=["large", "dsv3", "mid"])
    p.add_argument("--cpu-sample-tokens", type=int, default=24576,
                   help="tokens of the batch the CPU oracle runs on (0 = skip the CPU leg)")
    p.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    p.add_argument("--with-combine", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the combine (the reduce after the expert GEMMs) on the same batch")
    p.add_argument("--with-decode", action=argparse.BooleanOptionalAction, default=True,
                   help="also time moe_dispatch on decode-sized batches (single launch vs split)")
    p.add_argument("--with-formats", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the expand and SwiGLU in MXFP8 / MXFP4 on the same batch")
    p.add_argument("--with-configs", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the DeepSeek-V3 expand and the SwiGLU configuration, cache flushed per call")
    p.add_argument("--decode-only", action="store_true",
                   help="run only the decode-sized moe_dispatch timing (prints its JSON; for profiling)")
    p.add_argument("--configs-only", action="store_true",
                   help="run only the cache-flushed DeepSeek-V3 expand / SwiGLU-config timing (for profiling)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run torch's plain device copy of MIB MiB three times (the known-size "
                        "kernel that scales the FETCH_SIZE / WRITE_SIZE counters), then exit")
    return p.parse_args()


def copy_calibration(mib):
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))


def counted_traffic(path, workload, stage):
    """(kernel name, HBM bytes per launch) of `stage` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by the copy-kernel
    calibration); the bytes are None when there is no entry or the kernel's
    sources changed since the counters were taken."""
    import hashlib

    if not os.path.exists(path):
        return stage, None
    with open(path) as f:
        entry = json.load(f).get(workload, {}).get(stage)
    if entry is None:
        return stage, None
    h = hashlib.sha256()
    for src in entry.get("sources", []):
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != entry.get("source_sha256"):
        return entry.get("kernel", stage), None
    return entry.get("kernel", stage), entry.get("hbm_bytes_per_launch")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the dispatch path is built and timed on a single "
              "MI355X (multi-GPU sharding is design-only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.decode_only or args.configs_only:
        import numpy as np
        import torch

        import moe_routing_fp8_amd as moe
        import workloads as W

        torch.cuda.set_device(0)
        dev = torch.device("cuda:0")
        if args.decode_only:
            print(json.dumps({"decode_dispatch": time_decode(moe, torch, np, W, dev)}), flush=True)
        else:
            print(json.dumps({"configs": time_configs(moe, torch, np, W, dev)}), flush=True)
        return

    import numpy as np
    import torch

    import moe_routing_fp8_amd as moe
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = W.WORKLOADS[args.workload]
    T, E, K, H = w.num_tokens, w.num_experts, w.num_topk, w.hidden
    R, G, I = T * K, H // 128, SWIGLU_INTER
    t0 = time.time()
    scores = W.make_scores(w)
    x = W.make_x(w)
    gate_up = W.make_gate_up(w, rows=R, inter=I)
    row_w = W.make_row_weights(w, rows=R)
    log(f"inputs generated in {time.time() - t0:.1f}s: scores {scores.shape} x {x.shape} "
        f"gate_up {gate_up.shape}")
    # the same identifiers as tests/golden/input_sha256.txt (gate_up: its first 16384 rows)
    inputs_sha256 = {"scores": W.sha256_hex(scores), "x": W.sha256_hex(x),
                     "gate_up[:16384]": W.sha256_hex(gate_up[:16384])}

    s_d = torch.from_numpy(scores).to(dev)
    x_d = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    gu_d = torch.from_numpy(gate_up.view(np.int16)).to(dev).view(torch.bfloat16)
    rw_d = torch.from_numpy(row_w).to(dev)
    idx = torch.empty((T, K), dtype=torch.int64, device=dev)
    wts = torch.empty((T, K), dtype=torch.float32, device=dev) if w.renormalize else None
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((T, K), dtype=torch.int32, device=dev)
    ws = torch.empty(max(256, moe.moe_token_map_workspace_bytes(T, K, E)), dtype=torch.uint8, device=dev)
    q = torch.empty((R, H), dtype=torch.uint8, device=dev)
    sf = torch.empty((R, G), dtype=torch.float32, device=dev)
    ow = torch.empty(R, dtype=torch.float32, device=dev) if w.renormalize else None
    sq = torch.empty((R, I), dtype=torch.uint8, device=dev)
    ssf = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    stages = ["topk", "token_map", "expand", "swiglu"]

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        moe.moe_topk_gate(s_d, K, renormalize=w.renormalize, out=(idx, wts), stream=stream)
        if ev is not None:
            ev[1].record(stream)
        moe.moe_token_map(idx, E, with_row_token=False, workspace=ws,
                          out=(counts, offsets, pos, None), stream=stream)
        if ev is not None:
            ev[2].record(stream)
        moe.moe_expand_cast_fp8(x_d, pos, wts, out=(q, sf, ow), stream=stream)
        if ev is not None:
            ev[3].record(stream)
        moe.swiglu_cast_fp8(gu_d, rw_d, out=(sq, ssf), stream=stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Every EVENT_EVERY-th timed step carries the stage events; the rest run bare.  Recording an event
    # costs GPU time (about 16 us per step for the five stage events, large and DeepSeek-V3 batches
    # alike), which would otherwise be counted in every step.
    sampled = [i for i in range(args.steps) if i % EVENT_EVERY == 0]
    events = {i: [torch.cuda.Event(enable_timing=True) for _ in range(5)] for i in sampled}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start

    ms_per_step = wall * 1e3 / args.steps
    per_step = {s: [ev[j].elapsed_time(ev[j + 1]) for ev in events.values()] for j, s in enumerate(stages)}
    stage_ms = {s: sum(v) / len(v) for s, v in per_step.items()}

    ab = W.algorithmic_bytes(w)
    bytes_stage = {"topk": ab["topk"], "token_map": ab["map"], "expand": ab["expand"],
                   "swiglu": W.swiglu_bytes(R, I, True)}
    step_bytes = sum(bytes_stage.values())
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    stage_report = {s: {"us": round(stage_ms[s] * 1e3, 2),
                        "us_p10_p50_p90": [round(float(v) * 1e3, 2)
                                           for v in np.percentile(per_step[s], [10, 50, 90])],
                        "bytes": bytes_stage[s],
                        "GB/s": round(bytes_stage[s] / (stage_ms[s] * 1e-3) / 1e9, 1),
                        "frac_of_peak": round(bytes_stage[s] / (stage_ms[s] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                    for s in stages}
    dominant = max(("expand", "swiglu"), key=lambda s: stage_ms[s])
    achieved = bytes_stage[dominant] / (stage_ms[dominant] * 1e-3) / 1e9
    kernel_name, traffic = counted_traffic(args.traffic_file, args.workload, dominant)
    roofline = {"bound": "hbm", "kernel": kernel_name, "stage": dominant, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": bytes_stage[dominant]}
    log(f"step {ms_per_step * 1e3:.1f} us; " + "; ".join(
        f"{s} {stage_report[s]['us']} us {stage_report[s]['GB/s']} GB/s" for s in stages))

    next_stages = {}
    if args.with_combine:
        next_stages["combine"] = time_combine(moe, torch, T, K, H, R, pos, wts, dev, stream, args)

    if args.with_formats:
        next_stages["formats"] = time_formats(moe, torch, T, K, H, R, I, x_d, pos, wts, gu_d, rw_d, stream,
                                              args)
    if args.with_decode:
        next_stages["decode_dispatch"] = time_decode(moe, torch, np, W, dev)
    if args.with_configs:
        next_stages["configs"] = time_configs(moe, torch, np, W, dev)

    cpu = None
    if args.cpu_sample_tokens > 0:
        cpu = cpu_baseline(w, scores, x, gate_up, row_w, min(args.cpu_sample_tokens, T), I)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {T} tokens, {E} experts, top-{K}, hidden {H}, e4m3 "
                               f"groups of 128; SwiGLU over the {R} routed rows, I={I}",
                   "tokens": T, "experts": E, "topk": K, "hidden": H, "routed_rows": R,
                   "swiglu_inter": I, "group_size": 128, "seed": w.seed, "inputs_sha256": inputs_sha256},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(T / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "stages": stage_report,
        "stage_events": {"every": EVENT_EVERY, "steps_sampled": len(sampled),
                         "note": "stage times and roofline.achieved: event pairs on the launch stream in every "
                                 f"{EVENT_EVERY}th timed step; the other steps carry no events"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if next_stages:
        out["next_stages"] = next_stages
    print(json.dumps(out), flush=True)


def time_formats(moe, torch, T, K, H, R, I, x_d, pos, wts, gu_d, rw_d, stream, args):
    """The expand (routed, this batch's positions) and the SwiGLU (its routed
    rows) in the block-scaled formats with 32-channel groups and UE8M0 scales:
    MXFP8 (e4m3 codes) and MXFP4 (e2m1 codes, two per byte).  Timed like the
    combine: HIP events around each call on the launch stream, after warmup;
    not part of `value`."""
    res = {}
    w_in = wts if wts is not None else None
    for name, dt in (("mxfp8", "e4m3"), ("mxfp4", "e2m1")):
        fmt = dict(dtype=dt, group_size=32, round_sf=True, sf_ue8m0=True)
        code_b = H if dt == "e4m3" else H // 2
        icode_b = I if dt == "e4m3" else I // 2
        outs = moe.moe_expand_cast(x_d, pos, w_in, stream=stream, **fmt)
        souts = moe.swiglu_cast(gu_d, rw_d, stream=stream, **fmt)
        for stage, call, nbytes in (
                ("expand", lambda: moe.moe_expand_cast(x_d, pos, w_in, out=outs, stream=stream, **fmt),
                 T * H * 2 + T * K * 4 + (T * K * 8 if w_in is not None else 0) + R * code_b + R * (H // 32)),
                ("swiglu", lambda: moe.swiglu_cast(gu_d, rw_d, out=souts, stream=stream, **fmt),
                 R * 4 * I + R * 4 + R * icode_b + R * (I // 32))):
            for _ in range(args.warmup):
                call()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            for a, b in evs:
                a.record(stream)
                call()
                b.record(stream)
            torch.cuda.synchronize()
            us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
            kernel, traffic = counted_traffic(args.traffic_file, args.workload, f"{name}_{stage}")
            res[f"{name}_{stage}"] = {"us": round(us, 2), "bytes": nbytes,
                                      "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
                                      "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                      "kernel": kernel, "traffic": traffic}
            log(f"{name} {stage}: {res[f'{name}_{stage}']['us']} us {res[f'{name}_{stage}']['GB/s']} GB/s")
        del outs, souts
    res["note"] = ("groups of 32, power-of-two scales stored as UE8M0 bytes; MXFP4 codes are e2m1, two per byte; "
                   "same batch and positions as the step; not part of `value`")
    return res


def time_configs(moe, torch, np, W, dev, iters=50, warmup=5):
    """The smaller configurations, one call per timed iteration with a 1 GiB
    read in between (outside the event pair) so the 256 MB Infinity Cache
    holds none of the inputs -- a read, not a write, so no dirty lines are
    left to be written back during the timed call.  Gated kernels: the
    DeepSeek-V3 expand + cast (4096 tokens, top-8, hidden 7168, renormalised
    weights) and the SwiGLU configuration (8192 rows, I = 2048, row weights).
    Also the DeepSeek-V3 dispatch pipeline (top-k, map and expand in one
    event pair, with its tokens/s) and the mid configuration's expand and
    identity cast (1024 tokens, hidden 4096).  Median and p10 / p90 of the
    per-call times."""
    flush = torch.ones((1 << 30) // 8, dtype=torch.int64, device=dev)
    res = {}
    w = W.WORKLOADS["dsv3"]
    T, E, K, H = w.num_tokens, w.num_experts, w.num_topk, w.hidden
    s_d = torch.from_numpy(W.make_scores(w)).to(dev)
    x_d = torch.from_numpy(W.make_x(w).view(np.int16)).to(dev).view(torch.bfloat16)
    idx, wts = moe.moe_topk_gate(s_d, K, renormalize=True)
    _, _, pos, _ = moe.moe_token_map(idx, E)
    out = moe.moe_expand_cast_fp8(x_d, pos, wts)
    R = T * K
    ws = W.WORKLOADS["swiglu"]
    gu = torch.from_numpy(W.make_gate_up(ws).view(np.int16)).to(dev).view(torch.bfloat16)
    rw = torch.from_numpy(W.make_row_weights(ws)).to(dev)
    sout = moe.swiglu_cast_fp8(gu, rw)
    RS, I = ws.swiglu_rows, ws.swiglu_inter
    # the DeepSeek-V3 dispatch pipeline: top-k (renormalised) -> token map -> expand, one event pair
    idx_p, wts_p = torch.empty_like(idx), torch.empty_like(wts)
    counts_p = torch.empty(E, dtype=torch.int32, device=dev)
    offsets_p = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos_p = torch.empty_like(pos)
    ws_p = torch.empty(max(256, moe.moe_token_map_workspace_bytes(T, K, E)), dtype=torch.uint8, device=dev)
    out_p = (torch.empty_like(out[0].view(torch.uint8)), torch.empty_like(out[1]), torch.empty_like(out[2]))

    def dsv3_pipeline():
        moe.moe_topk_gate(s_d, K, renormalize=True, out=(idx_p, wts_p))
        moe.moe_token_map(idx_p, E, with_row_token=False, workspace=ws_p, out=(counts_p, offsets_p, pos_p, None))
        moe.moe_expand_cast_fp8(x_d, pos_p, wts_p, out=out_p)

    pipeline_bytes = (T * E * 4 + T * K * 12            # top-k: scores in; ids and weights out
                      + T * K * 8 + T * K * 4 + E * 4 + (E + 1) * 4  # map: ids in; pos, counts, offsets out
                      + T * H * 2 + T * K * 8 + R * H + R * (H // 128) * 4 + R * 4)  # expand
    # the mid configuration (reported, not gated): expand into 8192 rows, and the identity per-token cast
    wm = W.WORKLOADS["mid"]
    TM, EM, KM, HM = wm.num_tokens, wm.num_experts, wm.num_topk, wm.hidden
    xm = torch.from_numpy(W.make_x(wm).view(np.int16)).to(dev).view(torch.bfloat16)
    idx_m, _ = moe.moe_topk_gate(torch.from_numpy(W.make_scores(wm)).to(dev), KM)
    _, _, pos_m, _ = moe.moe_token_map(idx_m, EM)
    out_m = moe.moe_expand_cast_fp8(xm, pos_m)
    out_i = moe.moe_expand_cast_fp8(xm)
    RM, GM = TM * KM, HM // 128
    cases = (
        ("dsv3_expand", lambda: moe.moe_expand_cast_fp8(x_d, pos, wts, out=(out[0].view(torch.uint8), out[1], out[2])),
         T * H * 2 + T * K * 8 + R * H + R * (H // 128) * 4 + R * 4, None),
        ("dsv3_pipeline", dsv3_pipeline, pipeline_bytes, T),
        ("swiglu_config", lambda: moe.swiglu_cast_fp8(gu, rw, out=(sout[0].view(torch.uint8), sout[1])),
         RS * 4 * I + RS * 4 + RS * I + RS * (I // 128) * 4, None),
        ("mid_expand", lambda: moe.moe_expand_cast_fp8(xm, pos_m, out=(out_m[0].view(torch.uint8), out_m[1], None)),
         TM * HM * 2 + TM * KM * 4 + RM * HM + RM * GM * 4, None),
        ("mid_identity_cast", lambda: moe.moe_expand_cast_fp8(xm, out=(out_i[0].view(torch.uint8), out_i[1], None)),
         TM * HM * 2 + TM * HM + TM * GM * 4, None),
    )
    for name, call, nbytes, tokens in cases:
        times = []
        for i in range(warmup + iters):
            flush.sum()  # reads 1 GiB: the cache then holds none of the inputs and no dirty lines
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            call()
            b.record()
            b.synchronize()
            if i >= warmup:
                times.append(a.elapsed_time(b) * 1e3)
        p10, p50, p90 = (float(v) for v in np.percentile(times, [10, 50, 90]))
        res[name] = {"us_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)], "bytes": nbytes,
                     "GB/s": round(nbytes / (p50 * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(nbytes / (p50 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if tokens is not None:
            res[name]["tokens_per_s"] = round(tokens / (p50 * 1e-6), 1)
        log(f"{name}: median {p50:.2f} us {res[name]['GB/s']} GB/s")
    del flush
    res["note"] = ("one call per timed iteration, a 1 GiB read between calls to empty the Infinity Cache; "
                   "median GB/s; dsv3_pipeline is top-k + token map + expand in one event pair (tokens/s = "
                   "4096 tokens / its median); mid_* are reported, not gated; not part of `value`")
    return res


def time_decode(moe, torch, np, W, dev, token_counts=(1, 16, 64), calls=20, replays=10):
    """moe_dispatch (top-k -> map -> expand + cast) on the first T tokens of the
    DeepSeek-V3-shaped layer (256 experts, top-8, renormalised, hidden 7168):
    the single launch with a grid barrier against the split launches.  Each
    form is captured `calls` times into one HIP graph and replayed, so the time
    per call is the GPU's (launch gaps included, host overhead excluded)."""
    w = W.WORKLOADS["dsv3"]
    K, E = w.num_topk, w.num_experts
    res = {}
    for T in token_counts:
        s_d = torch.from_numpy(W.make_scores(w, T)).to(dev)
        x_d = torch.from_numpy(W.make_x(w, T).view(np.int16)).to(dev).view(torch.bfloat16)
        ws = torch.zeros(moe.moe_dispatch_workspace_bytes(T, K, E), dtype=torch.uint8, device=dev)
        per_mode = {}
        for name, mode in (("single_launch", moe.MOE_DISPATCH_SINGLE_LAUNCH), ("split", moe.MOE_DISPATCH_SPLIT)):
            out = moe.moe_dispatch(s_d, x_d, K, renormalize=True, mode=mode, workspace=ws)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                moe.moe_dispatch(s_d, x_d, K, renormalize=True, mode=mode, workspace=ws, out=out)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(calls):
                    moe.moe_dispatch(s_d, x_d, K, renormalize=True, mode=mode, workspace=ws, out=out)
            g.replay()
            torch.cuda.synchronize()
            best = float("inf")
            for _ in range(replays):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                b.synchronize()
                best = min(best, a.elapsed_time(b) * 1e3 / calls)
            per_mode[name] = round(best, 2)
            del g
        per_mode["speedup"] = round(per_mode["split"] / per_mode["single_launch"], 3)
        res[f"T={T}"] = per_mode
        log(f"decode dispatch T={T}: single launch {per_mode['single_launch']} us, "
            f"split {per_mode['split']} us")
    res["note"] = ("us per moe_dispatch call from HIP-graph replay; DeepSeek-V3 shape (E=256, top-8, "
                   "hidden 7168); not part of `value`")
    return res


def time_combine(moe, torch, T, K, H, R, pos, wts, dev, stream, args):
    """The combine after the expert GEMMs, on this batch: out[t] = sum_k w[t,k] *
    y_rows[pos[t,k]] with synthetic bf16 expert outputs y_rows [R, H] (not part
    of the step above; timed on its own, same stream, HIP events)."""
    gen = torch.Generator(device=dev).manual_seed(11)
    y_rows = torch.randn((R, H), device=dev, generator=gen).to(torch.bfloat16)
    w = wts if wts is not None else torch.rand((T, K), device=dev, generator=gen)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    for _ in range(args.warmup):
        moe.moe_combine(y_rows, pos, w, out=out, stream=stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        moe.moe_combine(y_rows, pos, w, out=out, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    us = sum(a.elapsed_time(b) for a, b in evs) / len(evs) * 1e3
    nbytes = R * H * 2 + T * K * 8 + T * H * 2  # rows, pos + weights, output
    del y_rows
    kernel, traffic = counted_traffic(args.traffic_file, args.workload, "combine")
    return {"us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel": kernel, "traffic": traffic,
            "note": "bf16 y_rows [R, H] synthetic (torch randn on the device); not part of `value`"}


def cpu_baseline(w, scores, x, gate_up, row_w, n_tok, inter):
    """The oracle (plain C, one host thread) on the first n_tok tokens of the
    batch: top-k -> map -> expand on those tokens, SwiGLU on their routed rows."""
    import numpy as np

    import oracle
    import workloads as W

    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    K, E = w.num_topk, w.num_experts
    rows = n_tok * K
    s, xs = np.ascontiguousarray(scores[:n_tok]), np.ascontiguousarray(x[:n_tok])
    gu, rw = np.ascontiguousarray(gate_up[:rows]), np.ascontiguousarray(row_w[:rows])
    log(f"cpu baseline: oracle on {n_tok} tokens / {rows} routed rows")
    t0 = time.perf_counter()
    idx, wt = oracle.topk_gate(s, K, renormalize=w.renormalize)
    t1 = time.perf_counter()
    _, _, pos, _ = oracle.token_map(idx, E)
    t2 = time.perf_counter()
    oracle.expand_cast_fp8(xs, pos, wt)
    t3 = time.perf_counter()
    oracle.swiglu_cast_fp8(gu, rw)
    t4 = time.perf_counter()
    dt = t4 - t0
    stage_s = {"topk": round(t1 - t0, 4), "token_map": round(t2 - t1, 4), "expand": round(t3 - t2, 4),
               "swiglu": round(t4 - t3, 4)}
    sub = W.Workload(w.name, w.seed, n_tok, E, K, w.hidden, renormalize=w.renormalize)
    ab = W.algorithmic_bytes(sub)
    nbytes = ab["pipeline"] + W.swiglu_bytes(rows, inter, True)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2), "stage_seconds": stage_s, "tokens_per_s": round(n_tok / dt, 1),
            "host_cpu": _host_cpu(), "host_cpu_count": os.cpu_count(),
            "sample": f"first {n_tok} of {w.num_tokens} tokens of the same batch: top-k, token map, "
                      f"expand+cast, and SwiGLU+cast over their {rows} routed rows "
                      f"({nbytes} algorithmic bytes); one run, pinned to one core"}


def _host_cpu():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
