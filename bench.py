"""Benchmark of the MoE dispatch hot path on one MI355X.

The metric: achieved HBM GB/s (and % of the 8 TB/s peak) plus tokens/s of
top-k gating -> token map -> fused expand + per-128-channel e4m3 cast, on the
large skewed prefill workload (32768 tokens, 256 experts with Zipf-skewed
load, top-8, hidden 7168, 262144 expert-grouped output rows), with the
SwiGLU + e4m3 cast (I = 2048, U(0,1) routing weights, over the batch's
262144 routed rows) measured as its own stage.

One step = one pass of the whole hot path over the batch: top-k, token map,
expand + cast, then SwiGLU + cast.  Inputs are seeded synthetic data,
resident in HBM before timing starts.

Timing:
  * W warmup steps, then exactly K bare steps between two device
    synchronisations, wall clock: ms_per_step.
  * metric pass, max(K, 50) steps: one HIP-event pair around top-k -> map ->
    expand and one around the SwiGLU in each step; value = algorithmic bytes
    of top-k -> map -> expand / the median pipeline time; tokens_per_s =
    tokens / the same median.
  * stage pass, max(K, 50) steps: events between the stages; per-stage
    medians, and the roofline of the expand (the pipeline's dominant kernel).
Output: one JSON line.  cpu_baseline = the CPU oracle on a bounded sample of
the same batch (1 host thread, 1 warm-up + 3 timed runs, medians).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) + tokens/s for top-k\u2192expand\u2192FP8 cast, 1 GPU"
HBM_PEAK_GBS = 8000.0
SWIGLU_INTER = 2048
MIN_EVENT_SAMPLES = 50  # event-timed medians come from at least this many samples


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="large", choices=["large", "dsv3", "mid"])
    p.add_argument("--cpu-sample-tokens", type=int, default=8192,
                   help="tokens of the batch the CPU oracle runs on (0 = skip the CPU leg)")
    p.add_argument("--traffic-file", default=os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    p.add_argument("--with-combine", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the combine (the reduce after the expert GEMMs) on the same batch")
    p.add_argument("--with-decode", action=argparse.BooleanOptionalAction, default=True,
                   help="also time moe_dispatch on decode-sized batches (single launch vs split)")
    p.add_argument("--with-padded", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the aligned map and padded expand (segments rounded up to 128 rows)")
    p.add_argument("--with-formats", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the expand and SwiGLU in MXFP8 / MXFP4 on the same batch")
    p.add_argument("--with-configs", action=argparse.BooleanOptionalAction, default=True,
                   help="also time the DeepSeek-V3 expand and pipeline and the SwiGLU configuration")
    p.add_argument("--decode-only", action="store_true",
                   help="run only the decode-sized moe_dispatch timing (prints its JSON; for profiling)")
    p.add_argument("--configs-only", action="store_true",
                   help="run only the DeepSeek-V3 / SwiGLU-configuration timing (for profiling)")
    p.add_argument("--configs-protocol", default="both", choices=["both", "flushed", "rotating"],
                   help="which timing protocol(s) the configurations use")
    p.add_argument("--config-cases", default="",
                   help="comma list of configuration cases to time (default: all of them)")
    p.add_argument("--event-samples", type=int, default=MIN_EVENT_SAMPLES,
                   help="event-timed samples per pass (at least the timed steps); lower only for profiling runs")
    p.add_argument("--traffic-from", default="", metavar="DIR",
                   help="CPU only: read the rocprofv3 FETCH_SIZE / WRITE_SIZE counter CSVs under DIR "
                        "(pmc_<COUNTER>/bench_ and copy_counter_collection.csv), write --traffic-file and print "
                        "the per-kernel table, then exit")
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


def algorithmic_bytes(T, E, K, H, weights, group=128):
    """Bytes each stage of top-k -> map -> expand must move: every input read
    once, every output written once (workspace and re-reads excluded)."""
    R, G = T * K, H // group
    wt = 4 if weights else 0
    d = {"topk": T * E * 4 + R * 8 + R * wt,                       # scores in; ids (+ weights) out
         "map": R * 8 + R * 4 + E * 4 + (E + 1) * 4,               # ids in; pos, counts, offsets out
         "expand": T * H * 2 + R * 4 + R * wt + R * H + R * G * 4 + R * wt}  # x, pos (+ w) in; codes, sf (+ w) out
    d["pipeline"] = d["topk"] + d["map"] + d["expand"]
    return d


def swiglu_bytes(rows, inter, weights, group=128):
    """SwiGLU + cast: read [R, 2I] bf16 (+ R weights), write [R, I] e4m3 + [R, I/group] fp32."""
    return rows * 2 * inter * 2 + (rows * 4 if weights else 0) + rows * inter + rows * (inter // group) * 4


def pctl(np, xs):
    p10, p50, p90 = (float(v) for v in np.percentile(xs, [10, 50, 90]))
    return p10, p50, p90


def gbs(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the dispatch path is built and timed on a single "
              "MI355X (multi-GPU sharding is design-only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.traffic_from:
        summarize_traffic(args.traffic_from, args.traffic_file)
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
    if args.decode_only:
        print(json.dumps({"decode_dispatch": time_decode(moe, torch, np, W, dev)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"configs": time_configs(moe, torch, np, W, dev, args.configs_protocol,
                                                  cases_wanted=args.config_cases)}), flush=True)
        return

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
    route_ws = torch.zeros(moe.moe_route_workspace_bytes(T, K, E), dtype=torch.uint8, device=dev)  # zeroed once
    route_out = {"topk_idx": idx, "topk_weights": wts, "counts": counts, "offsets": offsets, "pos": pos,
                 "row_token": None}
    q = torch.empty((R, H), dtype=torch.uint8, device=dev)
    sf = torch.empty((R, G), dtype=torch.float32, device=dev)
    ow = torch.empty(R, dtype=torch.float32, device=dev) if w.renormalize else None
    sq = torch.empty((R, I), dtype=torch.uint8, device=dev)
    ssf = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def topk():
        moe.moe_topk_gate(s_d, K, renormalize=w.renormalize, out=(idx, wts), stream=stream)

    def token_map():
        moe.moe_token_map(idx, E, with_row_token=False, workspace=ws, out=(counts, offsets, pos, None),
                          stream=stream)

    def route():
        # top-k -> map: the fused form where it is faster (grids of at most four workgroups per compute unit),
        # else the kernels of topk() and token_map() above
        moe.moe_route(s_d, K, renormalize=w.renormalize, with_weights=w.renormalize, with_row_token=False,
                      workspace=route_ws, out=route_out, stream=stream)

    def expand():
        moe.moe_expand_cast_fp8(x_d, pos, wts, out=(q, sf, ow), stream=stream)

    def swiglu():
        moe.swiglu_cast_fp8(gu_d, rw_d, out=(sq, ssf), stream=stream)

    stage_fns = (("topk", topk), ("token_map", token_map), ("expand", expand), ("swiglu", swiglu))

    def step():
        for _, fn in stage_fns:
            fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # 1. exactly K bare steps, wall clock
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps

    n_ev = max(args.steps, args.event_samples)

    def new_events(n):
        return [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    # 2. metric pass: one event pair around top-k -> map -> expand, one around the SwiGLU
    evs = [new_events(3) for _ in range(n_ev)]
    for ev in evs:
        ev[0].record(stream)
        route()
        expand()
        ev[1].record(stream)
        swiglu()
        ev[2].record(stream)
    torch.cuda.synchronize()
    pipe_us = [ev[0].elapsed_time(ev[1]) * 1e3 for ev in evs]
    swiglu_pair_us = [ev[1].elapsed_time(ev[2]) * 1e3 for ev in evs]

    # 3. stage pass: events between the stages
    evs = [new_events(len(stage_fns) + 1) for _ in range(n_ev)]
    for ev in evs:
        ev[0].record(stream)
        for j, (_, fn) in enumerate(stage_fns):
            fn()
            ev[j + 1].record(stream)
    torch.cuda.synchronize()
    stage_us = {name: [ev[j].elapsed_time(ev[j + 1]) * 1e3 for ev in evs] for j, (name, _) in enumerate(stage_fns)}

    ab = algorithmic_bytes(T, E, K, H, w.renormalize)
    bytes_stage = {"topk": ab["topk"], "token_map": ab["map"], "expand": ab["expand"],
                   "swiglu": swiglu_bytes(R, I, True)}
    pipe_p = pctl(np, pipe_us)
    value = gbs(ab["pipeline"], pipe_p[1])
    stage_report = {}
    for name, _ in stage_fns:
        p = pctl(np, stage_us[name])
        stage_report[name] = {"us_p50": round(p[1], 2), "us_p10_p50_p90": [round(v, 2) for v in p],
                              "bytes": bytes_stage[name], "GB/s": round(gbs(bytes_stage[name], p[1]), 1),
                              "frac_of_peak": round(gbs(bytes_stage[name], p[1]) / HBM_PEAK_GBS, 4)}
    sw_p = pctl(np, swiglu_pair_us)
    stage_report["swiglu"]["metric_pass_us_p10_p50_p90"] = [round(v, 2) for v in sw_p]
    stage_report["swiglu"]["rows_per_s"] = round(R / (stage_report["swiglu"]["us_p50"] * 1e-6), 1)
    exp_us = stage_report["expand"]["us_p50"]
    achieved = gbs(bytes_stage["expand"], exp_us)
    kernel_name, traffic = counted_traffic(args.traffic_file, args.workload, "expand")
    roofline = {"bound": "hbm", "kernel": kernel_name, "stage": "expand", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": bytes_stage["expand"],
                "launch_us_p50": exp_us, "samples": n_ev}
    sw_kernel, sw_traffic = counted_traffic(args.traffic_file, args.workload, "swiglu")
    swiglu_roofline = {"bound": "hbm", "kernel": sw_kernel, "stage": "swiglu",
                       "achieved": stage_report["swiglu"]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": stage_report["swiglu"]["frac_of_peak"], "traffic": sw_traffic,
                       "algorithmic_bytes_per_launch": bytes_stage["swiglu"],
                       "launch_us_p50": stage_report["swiglu"]["us_p50"], "samples": n_ev}
    step_bytes = ab["pipeline"] + bytes_stage["swiglu"]
    log(f"pipeline (top-k -> map -> expand) median {pipe_p[1]:.1f} us: {value:.1f} GB/s, "
        f"{T / (pipe_p[1] * 1e-6) / 1e6:.2f} M tokens/s; whole step (with SwiGLU) {ms_per_step * 1e3:.1f} us wall")
    log("stages: " + "; ".join(f"{s} {stage_report[s]['us_p50']} us {stage_report[s]['GB/s']} GB/s"
                               for s, _ in stage_fns))

    next_stages = {}
    if args.with_combine:
        next_stages["combine"] = time_combine(moe, torch, np, T, K, H, R, pos, wts, dev, stream, args, n_ev)
    if args.with_padded:
        next_stages["padded"] = time_padded(moe, torch, np, T, K, H, E, R, idx, x_d, stream, args, n_ev)
    if args.with_formats:
        next_stages["formats"] = time_formats(moe, torch, np, T, K, H, R, I, x_d, pos, wts, gu_d, rw_d, stream,
                                              args, n_ev)
    if args.with_decode:
        next_stages["decode_dispatch"] = time_decode(moe, torch, np, W, dev)
    if args.with_configs:
        next_stages["configs"] = time_configs(moe, torch, np, W, dev, args.configs_protocol,
                                              cases_wanted=args.config_cases)

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
        "config": {"workload": f"{w.name}: {T} tokens, {E} experts, top-{K}, hidden {H}, e4m3 groups of 128 "
                               f"(top-k -> token map -> expand + cast into {R} rows); SwiGLU + cast over the "
                               f"{R} routed rows, I={I}, as its own stage",
                   "tokens": T, "experts": E, "topk": K, "hidden": H, "routed_rows": R,
                   "swiglu_inter": I, "group_size": 128, "seed": w.seed, "inputs_sha256": inputs_sha256},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(T / (pipe_p[1] * 1e-6), 1),
        "pipeline": {"us_p10_p50_p90": [round(v, 2) for v in pipe_p], "bytes": ab["pipeline"], "samples": n_ev,
                     "note": "one HIP-event pair around top-k -> token map -> expand per step; value, "
                             "frac_of_hbm_peak and tokens_per_s come from its median"},
        "step": {"us_wall": round(ms_per_step * 1e3, 2), "bytes": step_bytes,
                 "GB/s_wall": round(gbs(step_bytes, ms_per_step * 1e3), 1),
                 "note": "K bare steps (top-k, map, expand, SwiGLU) between two synchronisations, wall clock"},
        "stages": stage_report,
        "stage_events": {"samples": n_ev, "note": "per-stage medians from a separate pass with events between "
                                                  "the stages"},
        "roofline": roofline,
        "swiglu_roofline": swiglu_roofline,
        "cpu_baseline": cpu,
    }
    if next_stages:
        out["next_stages"] = next_stages
    print(json.dumps(out), flush=True)


def time_calls(torch, np, call, stream, warmup, n):
    """(p10, p50, p90) in us of `call`, one HIP-event pair per call on `stream`, after `warmup` calls."""
    for _ in range(warmup):
        call()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return pctl(np, [a.elapsed_time(b) * 1e3 for a, b in evs])


def time_padded(moe, torch, np, T, K, H, E, R, idx, x_d, stream, args, n_ev):
    """Padded segments on the same batch: the aligned map over all experts with
    every segment rounded up to 128 rows (a grouped GEMM's tile), then the
    padded expand, whose grid writes the routed rows and zero-fills the
    padding rows.  One HIP-event pair per call on the launch stream, after
    warmup, medians; not part of `value`.  Expand bytes: x read once, pos and
    row_token read once, every row's codes and scales written."""
    align = 128
    rows = moe.moe_token_map_aligned_rows(T, K, E, align)
    ws = torch.empty(max(256, moe.moe_token_map_workspace_bytes(T, K, E)), dtype=torch.uint8, device=x_d.device)
    m = moe.moe_token_map_aligned(idx, 0, E, align, num_rows=rows, workspace=ws, stream=stream)
    outs = moe.moe_expand_cast_fp8_padded(x_d, m[2], m[3], stream=stream)
    G = H // 128
    exp_bytes = T * H * 2 + T * K * 4 + rows * 4 + rows * H + rows * G * 4
    res = {"align": align, "rows": rows, "padding_rows": rows - R}
    for stage, call, nbytes in (
            ("map", lambda: moe.moe_token_map_aligned(idx, 0, E, align, num_rows=rows, workspace=ws, out=m,
                                                      stream=stream), None),
            ("expand", lambda: moe.moe_expand_cast_fp8_padded(x_d, m[2], m[3], out=outs, stream=stream), exp_bytes)):
        p = time_calls(torch, np, call, stream, args.warmup, n_ev)
        res[stage] = {"us_p10_p50_p90": [round(v, 2) for v in p]}
        if nbytes is not None:
            res[stage].update({"bytes": nbytes, "GB/s": round(gbs(nbytes, p[1]), 1),
                               "frac_of_peak": round(gbs(nbytes, p[1]) / HBM_PEAK_GBS, 4)})
        log(f"padded {stage}: median {p[1]:.2f} us" + (f" {res[stage]['GB/s']} GB/s" if nbytes else ""))
    res["note"] = ("all experts, segments rounded up to 128 rows; the padded expand zero-fills the padding rows "
                   "in the same grid; event-pair medians; not part of `value`")
    del outs
    return res


def time_formats(moe, torch, np, T, K, H, R, I, x_d, pos, wts, gu_d, rw_d, stream, args, n_ev):
    """The expand (routed, this batch's positions) and the SwiGLU (its routed
    rows) in the block-scaled formats with 32-channel groups and UE8M0 scales:
    MXFP8 (e4m3 codes) and MXFP4 (e2m1 codes, two per byte).  One HIP-event
    pair per call on the launch stream, after warmup, medians; not part of
    `value`."""
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
            p = time_calls(torch, np, call, stream, args.warmup, n_ev)
            kernel, traffic = counted_traffic(args.traffic_file, args.workload, f"{name}_{stage}")
            res[f"{name}_{stage}"] = {"us_p10_p50_p90": [round(v, 2) for v in p], "bytes": nbytes,
                                      "GB/s": round(gbs(nbytes, p[1]), 1),
                                      "frac_of_peak": round(gbs(nbytes, p[1]) / HBM_PEAK_GBS, 4),
                                      "kernel": kernel, "traffic": traffic}
            log(f"{name} {stage}: median {p[1]:.2f} us {res[f'{name}_{stage}']['GB/s']} GB/s")
        del outs, souts
    res["note"] = ("groups of 32, power-of-two scales stored as UE8M0 bytes; MXFP4 codes are e2m1, two per byte; "
                   "same batch and positions as the step; event-pair medians; not part of `value`")
    return res


def time_configs(moe, torch, np, W, dev, protocol="both", iters=50, warmup=5, cases_wanted=""):
    """The smaller configurations under the two cache protocols:

    flushed   one call per event pair, a 1 GiB read before each call (outside
              the pair) so the 256 MB Infinity Cache holds none of the inputs --
              a read, not a write, so no dirty lines are left to be written back
              during the timed call;
    rotating  at least 4 buffer sets (distinct copies of every input and
              output) totalling more than 1 GiB, one call on each set back to
              back inside one event pair; per-call time = pair / sets.  A set is
              touched again only after the others (> 768 MB) have passed
              through the cache.  The round is enqueued behind a device-side
              spin, so the calls run back to back on the GPU rather than at the
              host's launch rate.
    Gated kernels: the DeepSeek-V3 expand + cast (4096 tokens, top-8, hidden
    7168, renormalised weights) and the SwiGLU configuration (8192 rows,
    I = 2048, row weights).  Also the DeepSeek-V3 dispatch pipeline (top-k,
    map and expand in one event pair, with its tokens/s) and the mid
    configuration's expand and identity cast (1024 tokens, hidden 4096).
    Median and p10 / p90 over `iters` samples."""
    res = {}
    w = W.WORKLOADS["dsv3"]
    T, E, K, H = w.num_tokens, w.num_experts, w.num_topk, w.hidden
    R = T * K
    s_h = torch.from_numpy(W.make_scores(w))
    x_h = torch.from_numpy(W.make_x(w).view(np.int16)).view(torch.bfloat16)
    ws_cfg = W.WORKLOADS["swiglu"]
    RS, I = ws_cfg.swiglu_rows, ws_cfg.swiglu_inter
    gu_h = torch.from_numpy(W.make_gate_up(ws_cfg).view(np.int16)).view(torch.bfloat16)
    rw_h = torch.from_numpy(W.make_row_weights(ws_cfg))
    wm = W.WORKLOADS["mid"]
    TM, EM, KM, HM = wm.num_tokens, wm.num_experts, wm.num_topk, wm.hidden
    RM, GM = TM * KM, HM // 128
    xm_h = torch.from_numpy(W.make_x(wm).view(np.int16)).view(torch.bfloat16)
    sm_h = torch.from_numpy(W.make_scores(wm))

    def dsv3_set():
        """One buffer set of the DeepSeek-V3 layer: inputs, map outputs, expand outputs."""
        b = {"s": s_h.to(dev), "x": x_h.to(dev)}
        b["idx"], b["w"] = moe.moe_topk_gate(b["s"], K, renormalize=True)
        b["counts"], b["offsets"], b["pos"], _ = moe.moe_token_map(b["idx"], E, with_row_token=False)
        b["ws"] = torch.zeros(moe.moe_route_workspace_bytes(T, K, E), dtype=torch.uint8, device=dev)  # zeroed once
        b["route"] = {"topk_idx": b["idx"], "topk_weights": b["w"], "counts": b["counts"], "offsets": b["offsets"],
                      "pos": b["pos"], "row_token": None}
        q, sf, ow = moe.moe_expand_cast_fp8(b["x"], b["pos"], b["w"])
        b["out"] = (q.view(torch.uint8), sf, ow)
        return b

    def dsv3_expand(b):
        moe.moe_expand_cast_fp8(b["x"], b["pos"], b["w"], out=b["out"])

    def dsv3_pipeline(b):
        # top-k -> map, fused (4096 tokens: one workgroup of 16 tokens per compute unit), then the expand
        moe.moe_route(b["s"], K, renormalize=True, with_row_token=False, workspace=b["ws"], out=b["route"])
        moe.moe_expand_cast_fp8(b["x"], b["pos"], b["w"], out=b["out"])

    def swiglu_set():
        b = {"gu": gu_h.to(dev), "rw": rw_h.to(dev)}
        q, sf = moe.swiglu_cast_fp8(b["gu"], b["rw"])
        b["out"] = (q.view(torch.uint8), sf)
        return b

    def swiglu_call(b):
        moe.swiglu_cast_fp8(b["gu"], b["rw"], out=b["out"])

    def mid_set():
        b = {"x": xm_h.to(dev)}
        idx, _ = moe.moe_topk_gate(sm_h.to(dev), KM)
        _, _, b["pos"], _ = moe.moe_token_map(idx, EM)
        q, sf, _ = moe.moe_expand_cast_fp8(b["x"], b["pos"])
        b["out"] = (q.view(torch.uint8), sf, None)
        qi, sfi, _ = moe.moe_expand_cast_fp8(b["x"])
        b["out_id"] = (qi.view(torch.uint8), sfi, None)
        return b

    pipeline_bytes = algorithmic_bytes(T, E, K, H, True)["pipeline"]
    expand_bytes = algorithmic_bytes(T, E, K, H, True)["expand"]
    cases = (
        # name, set factory, call, algorithmic bytes, tokens (for tokens/s) or None
        ("dsv3_expand", dsv3_set, dsv3_expand, expand_bytes, None),
        ("dsv3_pipeline", dsv3_set, dsv3_pipeline, pipeline_bytes, T),
        ("swiglu_config", swiglu_set, swiglu_call, swiglu_bytes(RS, I, True), None),
        ("mid_expand", mid_set, lambda b: moe.moe_expand_cast_fp8(b["x"], b["pos"], out=b["out"]),
         TM * HM * 2 + TM * KM * 4 + RM * HM + RM * GM * 4, None),
        ("mid_identity_cast", mid_set, lambda b: moe.moe_expand_cast_fp8(b["x"], out=b["out_id"]),
         TM * HM * 2 + TM * HM + TM * GM * 4, None),
    )
    if cases_wanted:
        keep = set(cases_wanted.split(","))
        cases = tuple(c for c in cases if c[0] in keep)
    protocols = ("flushed", "rotating") if protocol == "both" else (protocol,)
    flush = torch.ones((1 << 30) // 8, dtype=torch.int64, device=dev) if "flushed" in protocols else None
    for name, make_set, call, nbytes, tokens in cases:
        entry = {"bytes": nbytes}
        if "flushed" in protocols:
            b = make_set()
            times = []
            for i in range(warmup + iters):
                flush.sum()  # reads 1 GiB: the cache then holds none of the inputs and no dirty lines
                a = torch.cuda.Event(enable_timing=True)
                e = torch.cuda.Event(enable_timing=True)
                a.record()
                call(b)
                e.record()
                e.synchronize()
                if i >= warmup:
                    times.append(a.elapsed_time(e) * 1e3)
            p = pctl(np, times)
            entry["flushed"] = {"us_p10_p50_p90": [round(v, 2) for v in p], "GB/s": round(gbs(nbytes, p[1]), 1),
                                "frac_of_peak": round(gbs(nbytes, p[1]) / HBM_PEAK_GBS, 4)}
            if tokens is not None:
                entry["flushed"]["tokens_per_s"] = round(tokens / (p[1] * 1e-6), 1)
            del b
            log(f"{name} (flushed): median {p[1]:.2f} us {entry['flushed']['GB/s']} GB/s")
        if "rotating" in protocols:
            n_sets = max(4, -(-(1 << 30) // nbytes) + 1)  # at least 4 sets, more than 1 GiB together
            sets = [make_set() for _ in range(n_sets)]
            torch.cuda.synchronize()
            t_host = time.perf_counter()
            for _ in range(warmup):
                for b in sets:
                    call(b)
            t_host = (time.perf_counter() - t_host) / warmup  # host time to enqueue one round (upper bound)
            torch.cuda.synchronize()
            # the GPU waits in a spin kernel while the host enqueues the round, so the event pair sees the
            # calls back to back on the device (the binding's host time per call does not pace them)
            spin = int(min(5e8, max(2e6, 4 * t_host * 2.5e9)))
            times = []
            for _ in range(iters):
                a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(spin)
                a.record()
                for b in sets:
                    call(b)
                e.record()
                e.synchronize()
                times.append(a.elapsed_time(e) * 1e3 / n_sets)
            p = pctl(np, times)
            entry["rotating"] = {"us_p10_p50_p90": [round(v, 2) for v in p], "sets": n_sets,
                                 "set_bytes_total": n_sets * nbytes, "GB/s": round(gbs(nbytes, p[1]), 1),
                                 "frac_of_peak": round(gbs(nbytes, p[1]) / HBM_PEAK_GBS, 4)}
            if tokens is not None:
                entry["rotating"]["tokens_per_s"] = round(tokens / (p[1] * 1e-6), 1)
            del sets
            log(f"{name} (rotating, {n_sets} sets): median {p[1]:.2f} us per call {entry['rotating']['GB/s']} GB/s")
        res[name] = entry
    del flush
    res["note"] = ("flushed: one call per event pair after a 1 GiB read; rotating: one event pair around one call "
                   "on each of >= 4 buffer sets totalling > 1 GiB, enqueued behind a device spin so the calls run "
                   "back to back, per-call median; dsv3_pipeline is moe_route (fused: top-k with the counting, "
                   "then the slots) + expand (tokens/s = 4096 tokens / its median); mid_* are reported, not gated; not "
                   "part of `value`")
    return res


def time_decode(moe, torch, np, W, dev, token_counts=(1, 16, 64, 128, 256, 4096), calls=20, replays=10):
    """moe_dispatch (top-k -> map -> expand + cast) on the first T tokens of the
    DeepSeek-V3-shaped layer (256 experts, top-8, renormalised, hidden 7168):
    the single launch (local routing up to 32 tokens, a grid barrier above; up
    to 16384 routed copies), the top-k kernel then the single launch's map and
    copies (same limit), moe_route's fused routing (two launches) then the
    expand, the split launches, and AUTO.  Each form is captured `calls` times
    into one HIP graph and replayed, so the time per call is the GPU's (launch
    gaps included, host overhead excluded)."""
    w = W.WORKLOADS["dsv3"]
    K, E = w.num_topk, w.num_experts
    res = {}
    for T in token_counts:
        s_d = torch.from_numpy(W.make_scores(w, T)).to(dev)
        x_d = torch.from_numpy(W.make_x(w, T).view(np.int16)).to(dev).view(torch.bfloat16)
        ws = torch.zeros(moe.moe_dispatch_workspace_bytes(T, K, E), dtype=torch.uint8, device=dev)
        per_mode = {}
        forms = [("single_launch", moe.MOE_DISPATCH_SINGLE_LAUNCH),
                 ("topk_then_copy", moe.MOE_DISPATCH_TOPK_THEN_COPY)] if T * K <= 16384 else []
        forms += [("route_fused", moe.MOE_DISPATCH_ROUTE_FUSED), ("split", moe.MOE_DISPATCH_SPLIT),
                  ("auto", moe.MOE_DISPATCH_AUTO)]
        for name, mode in forms:
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
        best_form = min((n for n, _ in forms if n != "auto"), key=per_mode.get)
        per_mode["speedup_over_split"] = round(per_mode["split"] / per_mode[best_form], 3)
        per_mode["fastest"] = best_form
        res[f"T={T}"] = per_mode
        log(f"dispatch T={T}: " + ", ".join(f"{n} {per_mode[n]} us" for n, _ in forms))
    res["note"] = ("us per moe_dispatch call from HIP-graph replay; DeepSeek-V3 shape (E=256, top-8, "
                   "hidden 7168); single_launch and topk_then_copy only up to 16384 routed copies; auto is "
                   "the form MOE_DISPATCH_AUTO picks; not part of `value`")
    return res


def time_combine(moe, torch, np, T, K, H, R, pos, wts, dev, stream, args, n_ev):
    """The combine after the expert GEMMs, on this batch: out[t] = sum_k w[t,k] *
    y_rows[pos[t,k]] with synthetic bf16 expert outputs y_rows [R, H] (not part
    of the step; one event pair per call on the same stream, median)."""
    gen = torch.Generator(device=dev).manual_seed(11)
    y_rows = torch.randn((R, H), device=dev, generator=gen).to(torch.bfloat16)
    w = wts if wts is not None else torch.rand((T, K), device=dev, generator=gen)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    p = time_calls(torch, np, lambda: moe.moe_combine(y_rows, pos, w, out=out, stream=stream), stream,
                   args.warmup, n_ev)
    nbytes = R * H * 2 + T * K * 8 + T * H * 2  # rows, pos + weights, output
    del y_rows
    kernel, traffic = counted_traffic(args.traffic_file, args.workload, "combine")
    log(f"combine: median {p[1]:.2f} us {gbs(nbytes, p[1]):.1f} GB/s")
    return {"us_p10_p50_p90": [round(v, 2) for v in p], "bytes": nbytes, "GB/s": round(gbs(nbytes, p[1]), 1),
            "frac_of_peak": round(gbs(nbytes, p[1]) / HBM_PEAK_GBS, 4),
            "kernel": kernel, "traffic": traffic,
            "note": "bf16 y_rows [R, H] synthetic (torch randn on the device); not part of `value`"}


def cpu_baseline(w, scores, x, gate_up, row_w, n_tok, inter, runs=3):
    """The oracle (plain C, one host thread pinned to one core) on the first
    n_tok tokens of the batch: top-k -> map -> expand on those tokens, and the
    SwiGLU on their routed rows.  One warm-up run, then `runs` timed runs;
    per-stage medians (perf_counter around each oracle call)."""
    import numpy as np

    import oracle

    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    K, E = w.num_topk, w.num_experts
    rows = n_tok * K
    s, xs = np.ascontiguousarray(scores[:n_tok]), np.ascontiguousarray(x[:n_tok])
    gu, rw = np.ascontiguousarray(gate_up[:rows]), np.ascontiguousarray(row_w[:rows])
    log(f"cpu baseline: oracle on {n_tok} tokens / {rows} routed rows, 1 warm-up + {runs} timed runs")
    names = ("topk", "token_map", "expand", "swiglu")
    times = {n: [] for n in names}
    for run in range(runs + 1):
        t0 = time.perf_counter()
        idx, wt = oracle.topk_gate(s, K, renormalize=w.renormalize)
        t1 = time.perf_counter()
        _, _, pos, _ = oracle.token_map(idx, E)
        t2 = time.perf_counter()
        oracle.expand_cast_fp8(xs, pos, wt)
        t3 = time.perf_counter()
        oracle.swiglu_cast_fp8(gu, rw)
        t4 = time.perf_counter()
        if run > 0:
            for n, dt in zip(names, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
                times[n].append(dt)
    med = {n: float(np.median(v)) for n, v in times.items()}
    ab = algorithmic_bytes(n_tok, E, K, w.hidden, w.renormalize)
    nbytes = {"topk": ab["topk"], "token_map": ab["map"], "expand": ab["expand"],
              "swiglu": swiglu_bytes(rows, inter, True)}
    pipe_s = med["topk"] + med["token_map"] + med["expand"]
    return {"value": round(ab["pipeline"] / pipe_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_per_s": round(n_tok / pipe_s, 1),
            "pipeline_seconds": round(pipe_s, 4),
            "stages": {n: {"seconds_median": round(med[n], 4), "bytes": nbytes[n],
                           "GB/s": round(nbytes[n] / med[n] / 1e9, 4) if med[n] > 0 else None} for n in names},
            "host_cpu": _host_cpu(), "host_cpu_count": os.cpu_count(),
            "sample": f"first {n_tok} of {w.num_tokens} tokens of the same batch: top-k -> token map -> "
                      f"expand+cast ({ab['pipeline']} algorithmic bytes; `value` and tokens_per_s are this "
                      f"pipeline's), and SwiGLU+cast over their {rows} routed rows as its own stage; "
                      f"1 warm-up + {runs} timed runs, medians, pinned to one core"}


# Stages whose HBM traffic the counter runs record: (stage, kernel as rocprofv3 names it, sources, bytes)
# on the large workload (32768 tokens, top-8, hidden 7168; SwiGLU and MX formats over its 262144 rows).
def _traffic_stages():
    T, E, K, H, I = 32768, 256, 8, 7168, SWIGLU_INTER
    R = T * K
    ab = algorithmic_bytes(T, E, K, H, False)
    mx = ["moe_routing_fp8_amd/csrc/cast_mx.hip", "moe_routing_fp8_amd/csrc/device_utils.hpp",
          "moe_routing_fp8_amd/csrc/swiglu_math.hpp"]
    return [
        # the large batch's 470 MB input takes the streaming-load instance of the expand
        ("expand", "expand_cast_split_kernel<true>",
         ["moe_routing_fp8_amd/csrc/cast_fp8.hip", "moe_routing_fp8_amd/csrc/device_utils.hpp"], ab["expand"]),
        ("swiglu", "swiglu_mx_kernel<0, 128>", mx, swiglu_bytes(R, I, True)),
        ("combine", "combine_kernel<8, true>",
         ["moe_routing_fp8_amd/csrc/combine.hip", "moe_routing_fp8_amd/csrc/device_utils.hpp"],
         R * H * 2 + T * K * 8 + T * H * 2),
        ("mxfp8_expand", "expand_mx_split_kernel<0, 32>", mx, T * H * 2 + R * 4 + R * H + R * (H // 32)),
        ("mxfp4_expand", "expand_mx_split_kernel<1, 32>", mx, T * H * 2 + R * 4 + R * H // 2 + R * (H // 32)),
        ("mxfp8_swiglu", "swiglu_mx_kernel<0, 32>", mx, R * 4 * I + R * 4 + R * I + R * (I // 32)),
        ("mxfp4_swiglu", "swiglu_mx_kernel<1, 32>", mx, R * 4 * I + R * 4 + R * I // 2 + R * (I // 32)),
    ]


def _short_kernel(name):
    import re

    m = re.search(r"moe::\(anonymous namespace\)::([A-Za-z_0-9]+(?:<[^>]*>)?)", name)
    return m.group(1) if m else name.split("(")[0]


def _counter_per_kernel(path):
    """kernel -> [counter value per dispatch, in dispatch order] from a rocprofv3 counter CSV."""
    import csv

    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    out = {}
    for r in rows:
        out.setdefault(_short_kernel(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return out


def summarize_traffic(root, traffic_file):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled by what the counter
    reads for torch's plain copy of a known size (`--copy-calibration`), averaged over every dispatch of the
    kernel but the first; written to traffic_file with a hash of each kernel's sources."""
    import hashlib

    fetch = _counter_per_kernel(os.path.join(root, "pmc_FETCH_SIZE", "bench_counter_collection.csv"))
    write = _counter_per_kernel(os.path.join(root, "pmc_WRITE_SIZE", "bench_counter_collection.csv"))
    cf = _counter_per_kernel(os.path.join(root, "pmc_FETCH_SIZE", "copy_counter_collection.csv"))
    cw = _counter_per_kernel(os.path.join(root, "pmc_WRITE_SIZE", "copy_counter_collection.csv"))
    copy_kib = 1 << 20  # --copy-calibration 1024: 1 GiB read and 1 GiB written per copy
    copy_name = next(k for k in cf if "copyBuffer" in k)
    fs = copy_kib / (sum(cf[copy_name]) / len(cf[copy_name]))
    ws = copy_kib / (sum(cw[copy_name]) / len(cw[copy_name]))

    def avg(d, k):
        v = d[k][1:] if len(d[k]) > 1 else d[k]
        return sum(v) / len(v)

    out = {"large": {}, "calibration": {"fetch_scale": fs, "write_scale": ws, "copy_kernel": copy_name,
                                        "copy_bytes": copy_kib * 1024},
           "summary": "profiles/dispatch_large_hbm_counters.md"}
    print(f"scales: FETCH_SIZE x {fs:.5f}, WRITE_SIZE x {ws:.5f} (copy of 1 GiB: "
          f"FETCH {sum(cf[copy_name]) / len(cf[copy_name]):.1f} KiB, WRITE {sum(cw[copy_name]) / len(cw[copy_name]):.1f} KiB)")
    print("| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (scaled) | HBM write MB (scaled) | "
          "algorithmic MB | measured / algorithmic |")
    print("|---|---|---|---|---|---|---|")
    for stage, kernel, sources, alg in _traffic_stages():
        if kernel not in fetch or kernel not in write:
            continue
        rd = int(round(avg(fetch, kernel) * 1024 * fs))
        wr = int(round(avg(write, kernel) * 1024 * ws))
        h = hashlib.sha256()
        for src in sources:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        out["large"][stage] = {"hbm_read_bytes_per_launch": rd, "hbm_write_bytes_per_launch": wr,
                               "hbm_bytes_per_launch": rd + wr, "algorithmic_bytes_per_launch": alg,
                               "kernel": kernel, "source_sha256": h.hexdigest(), "sources": sources}
    for k in fetch:
        if k not in write or "copyBuffer" in k or k.startswith("__") or "at::" in k or "void " in k:
            continue
        rd, wr = avg(fetch, k) * 1024 * fs, avg(write, k) * 1024 * ws
        alg = next((a for _, kk, _, a in _traffic_stages() if kk == k), None)
        ratio = f"{(rd + wr) / alg:.3f}" if alg else ""
        print(f"| `{k}` | {avg(fetch, k):.1f} | {avg(write, k):.1f} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
              f"{alg / 1e6 if alg else 0:.1f} | {ratio} |")
    with open(traffic_file, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    # the configurations (bench.py --configs-only), if counted: DeepSeek-V3 expand and the SwiGLU configuration
    cfg_f = os.path.join(root, "pmc_FETCH_SIZE", "cfg_counter_collection.csv")
    cfg_w = os.path.join(root, "pmc_WRITE_SIZE", "cfg_counter_collection.csv")
    if os.path.exists(cfg_f) and os.path.exists(cfg_w):
        fetch, write = _counter_per_kernel(cfg_f), _counter_per_kernel(cfg_w)
        dsv3 = algorithmic_bytes(4096, 256, 8, 7168, True)
        known = {"expand_cast_split_kernel<false>": dsv3["expand"], "topk_gate_kernel<4, true>": dsv3["topk"]}
        print()
        print("| kernel (configurations) | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM MB (scaled) | "
              "algorithmic MB | measured / algorithmic |")
        print("|---|---|---|---|---|---|---|")
        for k in fetch:
            if k not in write or k.startswith("__") or "at::" in k or "void " in k:
                continue
            alg = known.get(k)
            if k.startswith("swiglu_mx_row_kernel<0, 128") or k.startswith("swiglu_mx_kernel<0, 128"):
                alg = swiglu_bytes(8192, SWIGLU_INTER, True)
            tot = avg(fetch, k) * 1024 * fs + avg(write, k) * 1024 * ws
            ratio = f"{tot / alg:.3f}" if alg else ""
            print(f"| `{k}` | {len(fetch[k])} | {avg(fetch, k):.1f} | {avg(write, k):.1f} | {tot / 1e6:.1f} | "
                  f"{alg / 1e6 if alg else 0:.1f} | {ratio} |")


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
