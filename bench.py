"""Decode benchmark: batch-1 greedy BF16 decode tok/s and the fraction of the HBM
bytes-per-token roofline, for the tile-scheduled persistent kernel on one MI355X.

A "step" is one cooperative launch that decodes a whole workload (64 tokens after
1023 cached positions for the Llama-3.2-1B-shaped model) from the same starting
KV state; inputs are seeded synthetic tensors already resident in HBM.

Prints ONE JSON line.  The CPU oracle is timed on the host cores on a bounded
sample of the same workload (``cpu_baseline``).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s at batch 1 and % of HBM roofline (weight+KV bytes/token)"
HBM_PEAK_GBS = 8000.0
KERNEL_NAME = "tiles_worker"


def _counter_traffic(workload_key: str, build_id: int):
    """HBM traffic per launch from a committed rocprofv3 counter summary of the same
    kernel build (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), else None."""
    path = os.path.join(ROOT, "profiles", f"{KERNEL_NAME}_{workload_key}_counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if int(d.get("build_id", "0"), 16) != build_id:
        return None
    return d.get("traffic_bytes_per_launch")


def cpu_baseline(setup_bits, m, wl, token, budget_s: float):
    """Time the CPU oracle (as it stands) on the host cores: free-running steps of the
    same workload from the same starting state, after one warm-up step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import OracleModel, convert_kv_int8, sample_token
    from tile_scheduled_persistent_amd import synth

    w_bits, kv_bits = setup_bits
    o = OracleModel(m, w_bits, np.float32, weight_format=wl.weights)
    if wl.kv == "int8":
        kv = convert_kv_int8(kv_bits, wl.n_cached)
    else:
        kv = {"k": kv_bits["k"].copy(), "v": kv_bits["v"].copy()}
    uniforms = synth.make_uniforms(m, wl.n_steps)

    def select(logits, i):
        return int(np.argmax(logits)) if wl.sampling is None else sample_token(logits, *wl.sampling, float(uniforms[i]))

    t_prep = time.perf_counter()
    logits, _ = o.step(kv, token, wl.n_cached)  # warm-up (also widens the weights once)
    prep = time.perf_counter() - t_prep
    tok = select(logits, 0)
    n = 0
    t0 = time.perf_counter()
    while True:
        logits, _ = o.step(kv, tok, wl.n_cached + 1 + n)
        tok = select(logits, n + 1)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= wl.n_steps - 1:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": n / el, "unit": "tok/s", "cores": int(threads), "kind": "oracle", "cpu_model": cpu_model,
            "sample": f"{n} free-running decode steps of the same workload after 1 warm-up step "
                      f"({el:.1f} s timed; warm-up incl. BF16->FP32 widening {prep:.1f} s), NumPy FP32"}


def _edge_floor(stream) -> dict:
    """Latency floor of one dependency edge on this GPU, same run: the library's ping-pong
    (tiles_edge_latency, the decode kernel's publish and poll forms) between workgroup 0 and a peer
    on the same XCD (8, 16) or on another (1, 2, 5); median round trip over 3 runs of 2000 each."""
    import numpy as np
    import torch

    from tile_scheduled_persistent_amd import tiles

    words = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    iters = 2000
    res = {}
    for name, peers in (("same_xcd", (8, 16)), ("cross_xcd", (1, 2, 5))):
        rt = []
        for peer in peers:
            for _ in range(3):
                words.zero_()
                out.zero_()
                torch.cuda.synchronize()
                tiles.edge_latency(words, peer, iters, out, stream=stream)
                stream.synchronize()
                ticks, gave_up_peer, gave_up_0 = (int(x) for x in out.cpu())
                if gave_up_peer or gave_up_0:
                    continue
                rt.append(ticks * 0.01 / iters)  # 100 MHz wall clock
        res["round_trip_us_" + name] = round(float(np.median(rt)), 3) if rt else None
    res["how"] = "one lane each of workgroup 0 and a peer pass a counter through two words, agent-scope stores and device-coherent polls"
    return res


def _read_ceiling(n_workers: int, stream) -> dict:
    """Measured stream-read ceiling of this GPU, same run: the library's stream-read kernel (the decode
    kernel's 16-byte non-temporal load form) over 2 GiB, one and two 512-thread workgroups per CU;
    the better median of 5 timed launches (HIP events on the launch stream)."""
    import numpy as np
    import torch

    from tile_scheduled_persistent_amd import tiles

    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best, how = 0.0, ""
    for per_cu in (1, 2):
        groups = n_workers * per_cu
        for _ in range(2):
            tiles.stream_read(buf, groups, sink, stream)
        ms = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            tiles.stream_read(buf, groups, sink, stream)
            b.record(stream)
            b.synchronize()
            ms.append(a.elapsed_time(b))
        gbs = buf.numel() / (float(np.median(ms)) * 1e-3) / 1e9
        if gbs > best:
            best, how = gbs, (f"tiles_stream_read over 2 GiB, {groups} workgroups x 512 threads, 16-byte "
                              f"non-temporal loads, median of 5 launches")
    del buf
    return {"gbs": best, "how": how}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama1b")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of timed oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--trace-report", default="", help="write a per-wave timing table (in-kernel trace) here")
    ap.add_argument("--verify-tokens", type=int, default=16,
                    help="also time greedy verify steps of this many tokens (added to the line as 'verify'; "
                         "greedy workloads; 0: none)")
    ap.add_argument("--trace-plan-tokens", type=int, default=0,
                    help="with --trace-report: trace a verify plan of this many positions per step (2 .. 4) running "
                         "the workload's greedy continuation as drafts, instead of the decode launch")
    ap.add_argument("--verify-plan-tokens", type=int, default=-1,
                    help="with --verify-tokens: time them with a verify plan taking this many positions per step "
                         "through every tile (2 .. 4, the positions timed rounded down to a multiple; -1: the most "
                         "the plan's LDS holds; 0 or 1: the decode plan, one position per step)")
    ap.add_argument("--kv-splits", type=int, default=0)
    ap.add_argument("--combine-mode", type=int, default=0)
    ap.add_argument("--attn-heads", type=int, default=0, help="query heads per attention tile (0: planner choice)")
    ap.add_argument("--o-placement", type=int, default=0,
                    help="o_proj workers: 0 planner choice, 1 all, 2 those without an attention tile")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed launches, run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the decode path has no multi-GPU component (it would shard "
                                   "per layer by KV head, with two all-reduces of the hidden state per layer)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    from tile_scheduled_persistent_amd import synth, tiles
    from tile_scheduled_persistent_amd.configs import WORKLOADS

    wl = WORKLOADS[args.workload]
    m = wl.model
    torch.cuda.set_device(0)
    dev = "cuda"
    w = synth.make_weights(m, device=dev)
    k0, v0 = synth.make_kv(m, wl.capacity, wl.n_cached, key_scale=wl.key_scale, device=dev)
    token = synth.make_tokens(m, 1)[0]
    stream = torch.cuda.current_stream()
    plan = tiles.Plan(m, w, wl.capacity, flags=0, kv_splits=args.kv_splits, combine_mode=args.combine_mode,
                      attn_heads=args.attn_heads, o_placement=args.o_placement, weight_format=wl.weights,
                      sampling=wl.sampling, kv_format=wl.kv,
                      stream=stream)
    info = plan.info()
    if wl.kv == "int8":  # the INT8 cache of the same prefix (setup: not timed)
        kv = tiles.KVCache.convert_int8(plan, k0, v0, wl.n_cached)
    else:
        kv = tiles.KVCache(k0.clone(), v0.clone(), wl.n_cached)
    n_tok = wl.n_steps
    out_t = torch.zeros(n_tok, dtype=torch.int32, device=dev)
    out_l = torch.zeros((n_tok, m.vocab), dtype=torch.float32, device=dev)

    uniforms = (torch.from_numpy(synth.make_uniforms(m, n_tok)).to(dev) if wl.sampling is not None else None)

    def launch():
        kv.length = wl.n_cached
        plan.decode(kv, token, n_tok, out_t, None, uniforms=uniforms)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    if plan.status() != tiles.TILES_OK:
        raise RuntimeError(tiles.last_error())

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if plan.status() != tiles.TILES_OK:
        raise RuntimeError(tiles.last_error())
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if args.calib_copy_mb:
        # a plain copy of known size: rocprofv3 FETCH_SIZE / WRITE_SIZE of this kernel calibrate the counters
        src = torch.empty(args.calib_copy_mb << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    avg_ms = float(np.mean(launch_ms))
    ceiling = _read_ceiling(info.n_workers, stream)
    edge = _edge_floor(stream)

    bpt = wl.bytes_per_token()
    tok_s = args.steps * n_tok / wall
    achieved = bpt * n_tok / (avg_ms * 1e-3) / 1e9
    traffic = _counter_traffic(args.workload, info.build_id)
    result = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if wl.weights == "bf16" and wl.kv == "bf16" else
                  f"{wl.weights} weights, {wl.kv} KV, fp32 activations"),
        "data": "synthetic",
        "config": {"workload": wl.description, "batch": 1, "cached_positions": wl.n_cached,
                   "tokens_per_step": n_tok, "parallelism": "single GPU, one workgroup per CU"},
        "pct_hbm_roofline": round(100.0 * tok_s * bpt / (HBM_PEAK_GBS * 1e9), 2),
        "bytes_per_token": int(bpt),
        "launch_ms": {"min": round(min(launch_ms), 4), "median": round(float(np.median(launch_ms)), 4),
                      "max": round(max(launch_ms), 4)},
        "plan": {"waves_per_token": info.waves_per_step, "kv_splits": info.kv_splits,
                 "sync": "tagged data (parity bit), no grid barrier",
                 "combine": "o_proj prologue" if info.combine_mode == 1 else "own wave",
                 "attn_heads_per_tile": info.attn_heads, "o_proj_workers": info.o_workers,
                 "workers": info.n_workers, "block_threads": info.block_threads},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "read_ceiling": {"gbs": round(ceiling["gbs"], 1), "frac": round(achieved / ceiling["gbs"], 4),
                         "how": ceiling["how"]},
        "edge_floor": edge,
    }

    if args.verify_tokens > 0 and wl.sampling is None:
        # (after the timed decode launches; a failure here is reported in the line, not raised)
        vplan = plan
        try:
            for T in ((4, 3, 2) if args.verify_plan_tokens < 0 else (args.verify_plan_tokens,)):
                if T < 2:
                    break
                try:
                    vplan = tiles.Plan(m, w, wl.capacity, flags=0, kv_splits=args.kv_splits, weight_format=wl.weights,
                                       kv_format=wl.kv, stream=stream, tokens_per_step=T)
                    break
                except tiles.TilesError:
                    if args.verify_plan_tokens >= 0 or T == 2:
                        raise
            result["verify"] = _verify_timing(vplan, kv, wl, token, out_t, args, stream)
            if vplan is not plan:
                vi = vplan.info()
                result["verify"]["plan"] = {"positions_per_step": vi.tokens_per_step,
                                            "waves_per_step": vi.waves_per_step,
                                            "combine": "o_proj prologue" if vi.combine_mode == 1 else "own wave"}
        except (tiles.TilesError, RuntimeError) as e:
            result["verify"] = {"error": str(e)}
        finally:
            if vplan is not plan:
                vplan.close()

    if args.trace_report:
        _trace_report(args.trace_report, m, wl, w, k0, v0, token, args, info, out_t)

    if not args.no_cpu_baseline:
        w_bits = synth.weights_as_bits(w)
        kv_bits = {"k": synth.bits(k0), "v": synth.bits(v0)}
        del w
        result["cpu_baseline"] = cpu_baseline((w_bits, kv_bits), m, wl, token, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    plan.close()
    print(json.dumps(result), flush=True)


def _verify_timing(plan, kv, wl, token, out_t, args, stream):
    """Greedy verify steps of M tokens (tiles_verify) from the same cached prefix: the drafts are the
    workload's own greedy continuation (all accepted), each launch timed with HIP events on the
    plan's stream (the draft copy into the plan's buffer included)."""
    import ctypes

    import numpy as np
    import torch

    from tile_scheduled_persistent_amd import tiles

    M = min(args.verify_tokens, wl.n_steps)
    T = plan.info().tokens_per_step
    M -= M % T  # a verify plan takes a multiple of its positions per step
    toks = [int(token)] + [int(t) for t in out_t[:M - 1].cpu().tolist()]
    buf = (ctypes.c_int32 * M)(*toks)
    out_a = torch.zeros(M, dtype=torch.int32, device="cuda")
    L = tiles.lib()

    def launch():
        kv.length = wl.n_cached
        c = kv.struct()
        rc = L.tiles_verify(plan._h, ctypes.byref(c), buf, M, ctypes.c_void_p(out_a.data_ptr()), None)
        if rc != tiles.TILES_OK:
            raise RuntimeError(tiles.last_error())

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for s0, e0 in ev:
        s0.record(stream)
        launch()
        e0.record(stream)
    torch.cuda.synchronize()
    if plan.status() != tiles.TILES_OK:
        raise RuntimeError(tiles.last_error())
    ms = float(np.median([s0.elapsed_time(e0) for s0, e0 in ev]))
    a = out_a.cpu().numpy()
    accepted = 0
    while accepted < M - 1 and int(a[accepted]) == toks[accepted + 1]:
        accepted += 1
    how = ("one weight stream per position" if T == 1 else
           f"a verify plan: {T} positions per kernel step, one weight stream per {T} positions")
    return {"tokens_per_step": M, "accepted": accepted, "ms_per_step": round(ms, 4),
            "positions_per_s": round(M / (ms * 1e-3), 1),
            "how": f"tiles_verify launches (m positions each, {how}), median of {args.steps}, HIP events on the "
                   "plan's stream"}


def _trace_report(path, m, wl, w, k0, v0, token, args, info, drafts):
    """Per-wave timing from the in-kernel trace (separate launch).  With --trace-plan-tokens T: a verify
    plan of T positions per step verifying the workload's greedy continuation (``drafts``); its times
    per kernel step then cover T positions."""
    import numpy as np
    import torch

    from tile_scheduled_persistent_amd import tiles

    T = args.trace_plan_tokens
    plan = tiles.Plan(m, w, wl.capacity, flags=tiles.TILES_TRACE, kv_splits=args.kv_splits, attn_heads=args.attn_heads,
                      combine_mode=args.combine_mode, o_placement=args.o_placement, weight_format=wl.weights,
                      sampling=wl.sampling, kv_format=wl.kv, tokens_per_step=T)
    if wl.kv == "int8":
        kv = tiles.KVCache.convert_int8(plan, k0, v0, wl.n_cached)
    else:
        kv = tiles.KVCache(k0.clone(), v0.clone(), wl.n_cached)
    out_t = torch.zeros(wl.n_steps, dtype=torch.int32, device="cuda")
    from tile_scheduled_persistent_amd import synth
    uniforms = torch.from_numpy(synth.make_uniforms(m, wl.n_steps)).cuda() if wl.sampling is not None else None
    if T > 1:
        n = wl.n_steps - wl.n_steps % T
        plan.verify(kv, [int(token)] + [int(t) for t in drafts[:n - 1].cpu().tolist()])
    else:
        plan.decode(kv, token, wl.n_steps, out_t, None, uniforms=uniforms)
    _, tr = plan.read_debug(hidden=False, trace=True)
    waves = plan.waves()
    plan.close()
    # [steps, waves, W, 12] 100 MHz ticks (see tiles_read_debug in include/tiles.h)
    tr = tr.astype(np.int64)
    steps, nw = tr.shape[0], tr.shape[1]
    names = tiles.WAVE_KINDS
    end = tr[:, :, :, 3].max(axis=2)                      # [steps, waves] last worker's publish
    prev_end = np.concatenate([np.concatenate([[tr[0, 0, :, 0].min()], end[:-1, -1]])[:, None], end[:, :-1]], axis=1)
    dur = (end - prev_end) * 0.01
    edge = (tr[:, :, :, 1].max(axis=2) - prev_end) * 0.01  # last producer's publish -> last consumer staged
    def phase(a, b):  # per (step, wave): max over workers of t_b - t_a, in us
        return (tr[:, :, :, b] - tr[:, :, :, a]).max(axis=2) * 0.01
    wait, cmp_, pub = phase(0, 1), phase(1, 2), phase(2, 3)
    pro = phase(1, 7)                                      # LDS prologue (control wave, P -> A)
    has = tr[:, :, :, 4] != 0
    cw = (np.where(has, tr[:, :, :, 4] - tr[:, :, :, 6], 0)).max(axis=2) * 0.01  # first compute wave, A -> done
    setup = (np.where(has, tr[:, :, :, 9] - tr[:, :, :, 6], 0)).max(axis=2) * 0.01  # A -> streaming loop entered
    first = (np.where(has, tr[:, :, :, 8] - tr[:, :, :, 9], 0)).max(axis=2) * 0.01  # entry -> first batch consumed
    hasl = tr[:, :, :, 11] != 0
    lastw = (np.where(hasl, tr[:, :, :, 11] - tr[:, :, :, 7], 0)).max(axis=2) * 0.01  # A -> last compute wave done
    hasb = tr[:, :, :, 10] != 0
    ctlb = (np.where(hasb, tr[:, :, :, 10] - tr[:, :, :, 7], 0)).max(axis=2) * 0.01  # A -> control ready for B
    lines = ["# per-wave timing from the in-kernel trace (wall clock 100 MHz).  dur = last publish of this wave",
             "# minus last publish of the previous one; edge = last worker's inputs staged minus the previous",
             "# wave's last publish; wait / compute / publish = max over workers of each phase (control wave);",
             "# prologue = LDS prologue (P -> A); cw1 = first compute wavefront's own work after A (max over workers);",
             "# setup = its A -> streaming loop entry; first = loop entry -> first batch consumed (max over workers);",
             "# lastw = A -> last compute wavefront done; ctlB = A -> control wavefront ready for B (attention)",
             f"# workload: {wl.description}; steps traced: {steps}; waves per step: {nw}" +
             (f"; a verify plan, {T} positions per step (times per step)" if T > 1 else ""),
             "wave\tkind\tlayer\tMB\tdur_us\tGB/s\tedge_us\twait_us\tcompute_us\tpublish_us\tprologue_us\tcw1_us\tsetup_us\tfirst_us\tlastw_us\tctlB_us"]
    sl = slice(1, None) if steps > 2 else slice(None)  # the first step includes the launch ramp
    tot = 0.0
    per_kind = {}
    for i, wv in enumerate(waves):
        d_us = float(np.median(dur[sl, i]))
        tot += d_us
        gbs = (wv.weight_bytes / 1e9) / (d_us * 1e-6) if d_us > 0 else 0.0
        k = names.get(wv.kind, str(wv.kind))
        ph = [float(np.median(x[sl, i])) for x in (edge, wait, cmp_, pub, pro, cw, setup, first, lastw, ctlb)]
        acc = per_kind.setdefault(k, [0.0] * 12)
        acc[0] += d_us
        acc[1] += wv.weight_bytes
        for j in range(10):
            acc[2 + j] += ph[j]
        lines.append(f"{i}\t{k}\t{wv.layer}\t{wv.weight_bytes / 1e6:.2f}\t{d_us:.2f}\t{gbs:.0f}\t" +
                     "\t".join(f"{x:.2f}" for x in ph))
    lines.append("# per kind (us per token): total | GB/s | edge | wait | compute | publish | prologue | cw1 | setup | first"
                 " | lastw | ctlB")
    for k, d in per_kind.items():
        lines.append(f"# {k}\t{d[0]:.1f}\t{d[1] / 1e9 / (d[0] * 1e-6) if d[0] else 0:.0f} GB/s\t"
                     f"{d[2]:.1f}\t{d[3]:.1f}\t{d[4]:.1f}\t{d[5]:.1f}\t{d[6]:.1f}\t{d[7]:.1f}\t{d[8]:.1f}\t{d[9]:.1f}\t"
                     f"{d[10]:.1f}\t{d[11]:.1f}")
    step_us = float(np.median(np.diff(end[:, -1]))) * 0.01 if steps > 1 else tot
    lines.append(f"# token time (median step-to-step) {step_us:.1f} us; sum of wave medians {tot:.1f} us")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
