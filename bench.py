#!/usr/bin/env python3
"""One speculative-decoding iteration of the QSpec hot path on one MI355X.

Workload: the Llama-3-8B-shaped INT4 linear stack (32 layers of fused q|k|v,
o, fused gate|up, down; group-128 INT4 weights, random init, shared by both
modes) plus the 4096 -> 128256 LM-head.  One step = one iteration at batch 1
with draft length 3:
  3 x [W4A4 draft pass at M = 1 -> draft Top-1]        (sequential draft phase)
  1 x  W4A16 verify pass at M = 4                      (target scores 4 positions)
  greedy accept + sampling accept over the 4 positions (V = 128256)
Each phase is captured once as a HIP graph and replayed; HIP events between
the phases time them.

Also measured (batched verify): the same stack at M = B (gamma + 1) rows for
B in {1, 4, 16} x gamma in {3, 5, 7}, both modes, with MFMA utilisation.

Printed JSON line: `value` = verify-pass weight GB/s (3,869,589,504 weight
bytes per pass / verify-pass time), plus draft-pass rates, accept positions/s,
the roofline of the dominant kernel (the persistent W4A4 pass kernel: the three
draft passes take most of a step) and of the W4A16 verify pass kernel, each
timed with HIP events around graph replays of one pass, and the CPU oracle
baseline.  Per-call distributions (mean, median, p10, p90) are given for 100
replays of the verify phase and for the accept kernels, warm (logits just read)
and cold (L2 and MALL flushed by a 1 GiB read before each call).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "verify-pass weight GB/s (% HBM peak) at M=4; accept positions/sec"


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "pass_kernels_llama8b_iteration.md")


def counted_traffic(key):
    """HBM bytes per launch of a pass kernel, from the rocprofv3 FETCH_SIZE / WRITE_SIZE runs recorded
    (copy-calibrated) in the committed profile summary; None if the summary is missing or the kernel
    sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            line = next(ln for ln in f if ln.startswith("traffic-json: "))
        rec = json.loads(line[len("traffic-json: "):])
        h = hashlib.sha256()
        for name in rec["files"]:
            with open(os.path.join(ROOT, name), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return rec[key]["fetch_bytes_per_launch"] + rec[key]["write_bytes_per_launch"]
    except (OSError, StopIteration, KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--eager", action="store_true", help="launch phases directly instead of replaying graphs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=10.0)
    ap.add_argument("--core-only", action="store_true",
                    help="time the iteration and the pass rooflines only (for counter runs under a profiler: no "
                         "accept, per-linear, batched or timing-model sections)")
    ap.add_argument("--pass-trace", action="store_true",
                    help="instead of the bench: time every stage boundary of the persistent passes from in-kernel "
                         "timestamps (qs_chain_forward_trace) and print the breakdown as one JSON line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the bench, copy this many MiB device to device twice (a plain copy kernel of known "
                         "size, to scale memory-traffic counters under a profiler)")
    return ap.parse_args()


def cpu_baseline(budget_s: float):
    """Time the CPU oracle (as it stands) on a bounded sample of the verify
    pass: W4A16 linears of one layer's shapes, then LM-head row blocks, at
    M = 4, until about budget_s seconds of work.  Rate in weight GB/s."""
    import numpy as np

    from oracle import qspec_oracle as O
    from quantized_speculative_decoding_int4_amd import workloads as W

    rng = W.rng_for(11)
    layer = [s for s in W.stack_shapes(1) if not s[0].startswith("lm")]
    head_block = ("lm_head_rows", 8192, W.HIDDEN)
    # the pass's own mix: per layer q|k|v, o, gate|up, down; LM-head row blocks in between
    shapes = (layer + [head_block]) * 1000
    done_bytes, t_used, items = 0, 0.0, []
    for name, n, k in shapes:
        q, s = W.int4_weights(rng, n, k)
        x, _ = W.activations(rng, 4, k)
        t0 = time.perf_counter()
        O.linear_w4a16(x, q, s)
        dt = time.perf_counter() - t0
        t_used += dt
        done_bytes += n * k // 2 + n * (k // 128) * 2
        items.append(name)
        if t_used >= budget_s:
            break
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    cores = len(os.sched_getaffinity(0))
    return {
        "value": done_bytes / t_used / 1e9,
        "unit": "GB/s",
        "cores": min(threads, cores),
        "kind": "oracle",
        "sample": (f"oracle W4A16 linears at M=4 on {len(items)} weight blocks "
                   f"({done_bytes / 1e9:.3f} GB of packed-equivalent weights: repeated q|k|v, o, gate|up, "
                   f"down and an 8192-row LM-head block) in {t_used:.1f} s; float64 NumPy, "
                   f"BLAS threads {threads}, affinity cores {cores}"),
    }


def pass_trace_report(qs, W, torch, chain, shapes):
    """Boundary breakdown of the persistent passes of the Llama-shaped stack from the timestamps of
    qs_chain_forward_trace: per workgroup and entry, t0 input staged, t1 stage done (partials parked),
    t2 outputs stored, t3 hand-over done.  Per boundary (entry e -> e + 1), medians over workgroups of
    epilogue = t2 - t1, hand-over = t3 - t2, staging = t0(e + 1) - t3 and the whole gap
    t0(e + 1) - t1, grouped by the linear the boundary feeds; per stage, the median streaming time
    t1 - t0.  Ticks are converted with the rate implied by a HIP-event-timed pass."""
    import numpy as np
    dev = "cuda"
    kinds = [name.split(".")[-1] if "." in name else name for name, _, _ in shapes]
    grid = torch.cuda.get_device_properties(0).multi_processor_count
    report = {"workload": "Llama-3-8B-shaped INT4 stack, 129 linears", "grid": grid, "passes": {}}
    rng = W.rng_for(5)
    for mode, m, label in ((qs.QS_W4A16, 4, "verify W4A16 M=4"), (qs.QS_W4A4, 1, "draft W4A4 M=1"),
                           (qs.QS_W4A16, 1, "target W4A16 M=1"), (qs.QS_W4A4, 4, "draft W4A4 M=4")):
        nbytes = chain.trace_bytes(mode, m)
        if nbytes == 0:
            continue
        x = torch.from_numpy(W.activations(rng, m, W.HIDDEN)[0]).to(dev)
        out = torch.empty((m, chain.out_features), dtype=torch.float32, device=dev)
        ws = torch.empty(chain.workspace_bytes(mode, m), dtype=torch.uint8, device=dev)
        tr = torch.zeros(nbytes // 8, dtype=torch.int64, device=dev)
        for _ in range(3):  # warm
            qs.qs_chain_forward_trace(mode, x, chain, tr, out=out, ws=ws)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        qs.qs_chain_forward_trace(mode, x, chain, tr, out=out, ws=ws)
        eb.record()
        torch.cuda.synchronize()
        ms = ea.elapsed_time(eb)
        t = tr.cpu().numpy().reshape(-1, grid, 4).astype(np.float64)
        span = t[:, :, 3].max() - t[:, :, 0].min()
        rate = span / (ms * 1e-3)  # ticks per second, the pass's own (launch overheads included)
        us = 1e6 / rate
        n_e = t.shape[0]
        if n_e != len(shapes):  # K-chunked entries: not broken down per linear here
            report["passes"][label] = {"entries": n_e, "pass_ms": ms}
            continue
        stream = np.median(t[:, :, 1] - t[:, :, 0], axis=1) * us
        epi = np.median(t[:-1, :, 2] - t[:-1, :, 1], axis=1) * us
        hand = np.median(t[:-1, :, 3] - t[:-1, :, 2], axis=1) * us
        stag = np.median(t[1:, :, 0] - t[:-1, :, 3], axis=1) * us
        gap = np.median(t[1:, :, 0] - t[:-1, :, 1], axis=1) * us
        by = {}
        for e in range(n_e - 1):
            k = kinds[e + 1]
            d = by.setdefault(k, {"n": 0, "epilogue_us": [], "handover_us": [], "staging_us": [], "gap_us": []})
            d["n"] += 1
            d["epilogue_us"].append(epi[e])
            d["handover_us"].append(hand[e])
            d["staging_us"].append(stag[e])
            d["gap_us"].append(gap[e])
        feeds = {k: {"boundaries": v["n"], **{f: float(np.median(v[f])) for f in
                                              ("epilogue_us", "handover_us", "staging_us", "gap_us")}}
                 for k, v in by.items()}
        streams = {}
        for e in range(n_e):
            streams.setdefault(kinds[e], []).append(stream[e])
        report["passes"][label] = {
            "pass_ms": ms, "ticks_per_s": rate, "entries": n_e,
            "sum_gap_ms": float(gap.sum()) / 1e3, "sum_stream_ms": float(stream.sum()) / 1e3,
            "boundary_into": feeds,
            "stage_stream_us": {k: float(np.median(v)) for k, v in streams.items()},
        }
        log(f"{label}: pass {ms:.3f} ms; per-workgroup gaps sum to {gap.sum() / 1e3:.3f} ms, streaming "
            f"{stream.sum() / 1e3:.3f} ms (medians over workgroups)")
        for k, v in feeds.items():
            log(f"  into {k:8s} x{v['boundaries']:3d}: epilogue {v['epilogue_us']:.2f}  hand-over "
                f"{v['handover_us']:.2f}  staging {v['staging_us']:.2f}  gap {v['gap_us']:.2f} us; stage "
                f"streams {report['passes'][label]['stage_stream_us'][k]:.2f} us")
        del x, out, ws, tr
    print(json.dumps(report), flush=True)


def linear_rates(qs, W, torch, E):
    """Configs 0-2 measured one linear at a time: each shape's packed weights are copied until the
    copies exceed 512 MiB (twice the 256 MiB MALL), and a HIP graph of one call per copy is replayed,
    so every call streams its weights from HBM and the host's launch latency is not timed.  Rate =
    packed weight bytes (0.515625 B per weight) / time per call; the fused LM-head Top-1 is timed
    the same way."""
    import numpy as np
    dev = "cuda"
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    rng = W.rng_for(17)
    shapes = [("cfg0 4096x4096", 4096, 4096)] + [(f"cfg1 {n_}", n, k) for n_, n, k in W.LAYER_LINEARS] + \
             [("cfg2 lm_head", W.VOCAB, W.HIDDEN)]
    out = {}
    for name, n, k in shapes:
        q, s_ = W.int4_weights_device(gen, n, k, device=dev)
        wp, sp = qs.qs_pack_weights(q, s_)
        del q, s_
        wbytes = n * k // 2 + n * (k // 128) * 2
        copies = max(2, -(-(512 << 20) // wbytes))
        ws_list = [(wp.clone(), sp.clone()) for _ in range(copies)]
        rec = {"N": n, "K": k, "weight_bytes": wbytes, "copies": copies}
        runs = [("w4a16_M4", qs.QS_W4A16, 4), ("w4a4_M1", qs.QS_W4A4, 1)]
        if name.startswith("cfg0"):
            runs.append(("w4a4_M4", qs.QS_W4A4, 4))
        for key, mode, m in runs:
            x = torch.from_numpy(W.activations(rng, m, k)[0]).to(dev)
            y = torch.empty((m, n), dtype=torch.float32, device=dev)
            lw = qs.linear_workspace_bytes(mode, m, n, k)
            wsp = torch.zeros(max(lw, 1), dtype=torch.uint8, device=dev)

            def call(wpk, spk, lg=None):
                if name.startswith("cfg2"):
                    qs.qs_lmhead(mode, x, wpk, spk, n, logits=y, ws=wsp if lw else None)
                elif mode == qs.QS_W4A16:
                    qs.qs_linear_w4a16(x, wpk, spk, n, y=y)
                else:
                    qs.qs_linear_w4a4(x, wpk, spk, n, y=y, ws=wsp if lw else None)
            for wpk, spk in ws_list[:2]:
                call(wpk, spk)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for wpk, spk in ws_list:
                    call(wpk, spk)
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                a, b = E(enable_timing=True), E(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e3 / copies)
            us = float(np.median(ts))
            rec[key] = {"us": us, "GBps": wbytes / (us * 1e-6) / 1e9, "hbm_frac": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
            del g, x, y, wsp
        if name.startswith("cfg2"):  # the LM-head with the fused Top-1 epilogue, same rotation
            for key, mode, m in (("top1_w4a16_M4", qs.QS_W4A16, 4), ("top1_w4a4_M1", qs.QS_W4A4, 1)):
                x = torch.from_numpy(W.activations(rng, m, k)[0]).to(dev)
                wst = torch.zeros(qs.lmhead_top1_workspace_bytes(mode, m, n, k), dtype=torch.uint8, device=dev)
                o = qs.qs_lmhead_top1(mode, x, ws_list[0][0], ws_list[0][1], n, want_logits=False, ws=wst)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for wpk, spk in ws_list:
                        qs.qs_lmhead_top1(mode, x, wpk, spk, n, want_logits=False, top1=o["top1"],
                                          top1_prob=o["top1_prob"], ws=wst)
                g.replay()
                torch.cuda.synchronize()
                a, b = E(enable_timing=True), E(enable_timing=True)
                a.record()
                g.replay()
                b.record()
                torch.cuda.synchronize()
                us = a.elapsed_time(b) * 1e3 / copies
                rec[key] = {"us": us, "GBps": wbytes / (us * 1e-6) / 1e9}
                del g, wst, o, x
        out[name] = rec
        del ws_list, wp, sp
        torch.cuda.empty_cache()
    return out


def cpu_per_config(budget_s: float):
    """The oracle (as it stands) per config, on bounded samples, in the GPU lines' units: weight GB/s
    of single linears (configs 0, 1), of the LM-head (config 2, one 8192-row block), positions/s of the
    accept step (configs 0, 2, 4), and config 3's iteration time extrapolated from layer 0."""
    import time as _t

    import numpy as np

    from oracle import qspec_oracle as O
    from quantized_speculative_decoding_int4_amd import workloads as W

    rng = W.rng_for(12)
    res = {}
    t_start = _t.perf_counter()

    def wrate(fn, n, k, m):
        q, s = W.int4_weights(rng, n, k)
        x, _ = W.activations(rng, m, k)
        t0 = _t.perf_counter()
        fn(x, q, s)
        dt = _t.perf_counter() - t0
        return {"s": dt, "GBps": (n * k // 2 + n * (k // 128) * 2) / dt / 1e9}

    w16 = lambda x, q, s: O.linear_w4a16(x, q, s)  # noqa: E731
    w4 = lambda x, q, s: O.linear_w4a4(x, q, s)    # noqa: E731
    wrate(w16, 4096, 4096, 4)  # untimed: the process's first large allocations
    res["cfg0"] = {"w4a16_M4": wrate(w16, 4096, 4096, 4), "w4a4_M4": wrate(w4, 4096, 4096, 4)}
    res["cfg1"] = {}
    layer_s = {"w4a16_M4": 0.0, "w4a4_M1": 0.0}
    for name, n, k in W.LAYER_LINEARS:
        a_, b_ = wrate(w16, n, k, 4), wrate(w4, n, k, 1)
        res["cfg1"][name] = {"w4a16_M4": a_, "w4a4_M1": b_}
        layer_s["w4a16_M4"] += a_["s"]
        layer_s["w4a4_M1"] += b_["s"]
    head_rows = 8192  # one block of the LM-head; the rate is per weight byte
    res["cfg2"] = {"lm_head_block_rows": head_rows, "w4a16_M4": wrate(w16, head_rows, W.HIDDEN, 4),
                   "w4a4_M1": wrate(w4, head_rows, W.HIDDEN, 1)}
    head_s = {k_: res["cfg2"][k_]["s"] * W.VOCAB / head_rows for k_ in ("w4a16_M4", "w4a4_M1")}

    def accept_rate(B, G, V, reps=1):
        tg = W.logits(rng, (B, G + 1, V), sigma=5.24)
        dr = W.perturb(rng, tg[:, :G])
        d = rng.integers(0, V, size=(B, G)).astype(np.int32)
        ua, uf = W.uniforms(rng, (B, G)), W.uniforms(rng, (B,))
        t0 = _t.perf_counter()
        for _ in range(reps):
            O.verify_greedy(tg, d)
        tgr = (_t.perf_counter() - t0) / reps
        t0 = _t.perf_counter()
        for _ in range(reps):
            O.verify_sample(tg, dr, d, ua, uf)
        tsm = (_t.perf_counter() - t0) / reps
        pos = B * (G + 1)
        return {"greedy_positions_per_s": pos / tgr, "sample_positions_per_s": pos / tsm}

    res["cfg0"]["accept_V32_gamma3"] = accept_rate(1, 3, 32, reps=200)
    res["cfg2"]["accept_B1_gamma3"] = accept_rate(1, 3, W.VOCAB)
    res["cfg4"] = {"accept_B16_gamma7": accept_rate(16, 7, W.VOCAB)}
    # config 3: 32 x layer 0 + the head, extrapolated (labelled so): 3 draft passes (W4A4, M = 1) + one verify
    # pass (W4A16, M = 4); accept costs are negligible next to them
    it = 3 * (32 * layer_s["w4a4_M1"] + head_s["w4a4_M1"]) + 32 * layer_s["w4a16_M4"] + head_s["w4a16_M4"]
    res["cfg3"] = {"iteration_s_extrapolated": it, "verify_pass_s_extrapolated": 32 * layer_s["w4a16_M4"] + head_s["w4a16_M4"]}
    res["wall_s"] = _t.perf_counter() - t_start
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from quantized_speculative_decoding_int4_amd import qspec as qs
    from quantized_speculative_decoding_int4_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = "cuda"
    V, H, GAMMA = W.VOCAB, W.HIDDEN, 3
    M_VERIFY = GAMMA + 1

    # ---------------- weights (random init, generated and packed on the GPU)
    t0 = time.perf_counter()
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    shapes = W.stack_shapes()
    layers, pass_bytes = [], 0
    for name, n, k in shapes:
        q, s = W.int4_weights_device(gen, n, k, device=dev)
        wp, sp = qs.qs_pack_weights(q, s)
        del q, s
        layers.append((wp, sp, n, k))
        pass_bytes += n * k // 2 + n * (k // 128) * 2
    torch.cuda.synchronize()
    chain = qs.Chain(layers)
    log(f"packed {len(shapes)} linears, {pass_bytes} weight bytes per pass, {time.perf_counter() - t0:.1f} s")
    if args.pass_trace:
        pass_trace_report(qs, W, torch, chain, shapes)
        return

    # ---------------- inputs and buffers
    rng = W.rng_for(3)
    x_np, _ = W.activations(rng, M_VERIFY, H)
    x_verify = torch.from_numpy(x_np).to(dev)
    x_draft = [x_verify[i:i + 1] for i in range(GAMMA)]
    logits_q = torch.empty((1, GAMMA, V), dtype=torch.float32, device=dev)
    logits_p = torch.empty((1, M_VERIFY, V), dtype=torch.float32, device=dev)
    d = torch.zeros((1, GAMMA), dtype=torch.int32, device=dev)
    u_acc = torch.from_numpy(W.uniforms(rng, (1, GAMMA))).to(dev)
    u_fin = torch.from_numpy(W.uniforms(rng, (1,))).to(dev)
    ws_draft = torch.empty(chain.top1_workspace_bytes(qs.QS_W4A4, 1), dtype=torch.uint8, device=dev)
    ws_verify = torch.empty(chain.top1_workspace_bytes(qs.QS_W4A16, M_VERIFY), dtype=torch.uint8, device=dev)
    ws_acc2 = torch.zeros(qs.verify_workspace_bytes(1, GAMMA, V), dtype=torch.uint8, device=dev)
    d_steps = torch.zeros((GAMMA, 1), dtype=torch.int32, device=dev)  # draft step i's token, row i
    t_verify = torch.empty((M_VERIFY,), dtype=torch.int32, device=dev)
    p_verify = torch.empty((M_VERIFY,), dtype=torch.float32, device=dev)
    greedy_out = {
        "n_accept": torch.empty((1,), dtype=torch.int32, device=dev),
        "out_tokens": torch.empty((1, M_VERIFY), dtype=torch.int32, device=dev),
    }
    sample_out = {
        "accept_prob": torch.empty((1, GAMMA), dtype=torch.float32, device=dev),
        "n_accept": torch.empty((1,), dtype=torch.int32, device=dev),
        "out_tokens": torch.empty((1, M_VERIFY), dtype=torch.int32, device=dev),
        "final_dist": None,
    }

    # The greedy path never re-reads logits: each draft pass and the verify pass reduce their LM-head
    # output to the Top-1 in the last stage's epilogue, and acceptance takes the Top-1 ids.  The logits
    # are still written, for the sampling acceptance the step also runs.
    def draft_phase():
        for i in range(GAMMA):
            qs.qs_chain_forward_top1(qs.QS_W4A4, x_draft[i], chain, out=logits_q[0, i:i + 1], top1=d_steps[i],
                                     want_prob=False, ws=ws_draft)
        d.copy_(d_steps.view(1, GAMMA))

    def verify_phase():
        qs.qs_chain_forward_top1(qs.QS_W4A16, x_verify, chain, out=logits_p[0], top1=t_verify, top1_prob=p_verify,
                                 ws=ws_verify)

    def accept_phase():
        qs.qs_accept_greedy(t_verify.view(1, M_VERIFY), d, out=greedy_out)
        qs.qs_verify_sample(logits_p, logits_q, d, u_acc, u_fin, out=sample_out, ws=ws_acc2)

    phases = [draft_phase, verify_phase, accept_phase]
    for f in phases:  # eager warm-up (caches device info / kernel attributes)
        f()
    torch.cuda.synchronize()
    if not args.eager:
        graphs = []
        for f in phases:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                f()
            graphs.append(g)
        torch.cuda.synchronize()
        runners = [g.replay for g in graphs]
    else:
        runners = phases
    log("graphs captured" if not args.eager else "eager mode")

    def step():
        for r in runners:
            r()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---------------- timed region: exactly `steps` iterations
    K = args.steps
    E = torch.cuda.Event
    ev = [[E(enable_timing=True) for _ in range(4)] for _ in range(K)]
    start, end = E(enable_timing=True), E(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        ev[i][0].record()
        runners[0]()
        ev[i][1].record()
        runners[1]()
        ev[i][2].record()
        runners[2]()
        ev[i][3].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(end) / K
    draft_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    verify_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    accept_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    verify_gbs = pass_bytes / (verify_ms * 1e-3) / 1e9
    draft_gbs = GAMMA * pass_bytes / (draft_ms * 1e-3) / 1e9
    log(f"step {ms_step:.3f} ms (wall {wall / K * 1e3:.3f}); draft {draft_ms:.3f} verify {verify_ms:.3f} "
        f"accept {accept_ms:.3f} ms; verify {verify_gbs:.0f} GB/s, draft {draft_gbs:.0f} GB/s")
    # a persistent pass whose wait timed out leaves NaN in its output and sets its workspace's time-out word:
    # such a run is not a measurement
    for mode, m, ws, name in ((qs.QS_W4A4, 1, ws_draft, "draft"), (qs.QS_W4A16, M_VERIFY, ws_verify, "verify")):
        if qs.qs_chain_pass_status(mode, m, chain, ws):
            log(f"the {name} pass reported a wait time-out: results invalid")
            sys.exit(3)
    n_acc = int(greedy_out["n_accept"].item())
    assert bool(torch.isfinite(logits_p).all()) and bool(torch.isfinite(logits_q).all()), "non-finite logits"
    agree = float((t_verify.view(1, M_VERIFY)[:, :GAMMA] == d).float().mean().item())

    # ---------------- accept throughput at the batched-verify scale (B=16, gamma=7)
    def time_calls(fn, reps=20):
        fn()
        torch.cuda.synchronize()
        a, b = E(enable_timing=True), E(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # Per-call HIP events: mean, median, p10 and p90 in us over `reps` calls.  `before` (untimed, on the
    # same stream) runs ahead of each call, e.g. a 1 GiB read that evicts the inputs from L2 and MALL.
    def time_dist(fn, reps=100, before=None):
        fn()
        torch.cuda.synchronize()
        evs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            if before is not None:
                before()
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        return {"reps": reps, "mean_us": float(t.mean()), "median_us": float(np.median(t)),
                "p10_us": float(np.percentile(t, 10)), "p90_us": float(np.percentile(t, 90))}

    verify_dist = time_dist(runners[1], reps=100)
    log(f"verify phase over 100 replays: median {verify_dist['median_us']:.1f} us, "
        f"p10 {verify_dist['p10_us']:.1f}, p90 {verify_dist['p90_us']:.1f}")
    draft_dist = time_dist(runners[0], reps=100)  # the draft phase: GAMMA passes back to back
    log(f"draft phase ({GAMMA} passes) over 100 replays: median {draft_dist['median_us']:.1f} us, "
        f"p10 {draft_dist['p10_us']:.1f}, p90 {draft_dist['p90_us']:.1f}")
    def optional_sections():
        """Accept throughput, per-linear rates, batched sweep and the timing model (skipped by --core-only)."""
        # "cold": a 1 GiB read before each call evicts the inputs from L2 and the 256 MiB MALL with clean
        # lines (a write would leave dirty lines whose write-back then competes with the call's reads)
        flush_buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev).view(torch.int64)
        flush = lambda: flush_buf.sum()  # noqa: E731
        # A spin kernel that touches no memory keeps the GPU busy while the host marshals the next call, so
        # a warm call's events bracket its kernels rather than the host's launch latency.
        spin = lambda: torch.cuda._sleep(200_000)  # noqa: E731
    
        accept = {}
        for (B, G) in ((1, GAMMA), (16, 7)):
            tg = torch.from_numpy(W.logits(rng, (B, G + 1, V), sigma=5.24)).to(dev)
            dr = torch.from_numpy(W.perturb(rng, tg[:, :G].cpu().numpy())).to(dev)
            dd = torch.from_numpy(rng.integers(0, V, size=(B, G)).astype(np.int32)).to(dev)
            ua = torch.from_numpy(W.uniforms(rng, (B, G))).to(dev)
            uf = torch.from_numpy(W.uniforms(rng, (B,))).to(dev)
            wsg = torch.zeros(qs.verify_workspace_bytes(B, G, V), dtype=torch.uint8, device=dev)
            go = qs.qs_verify_greedy(tg, dd, ws=wsg)
            so = qs.qs_verify_sample(tg, dr, dd, ua, uf, ws=wsg)
            tgms = time_calls(lambda: qs.qs_verify_greedy(tg, dd, out=go, ws=wsg))
            tsms = time_calls(lambda: qs.qs_verify_sample(tg, dr, dd, ua, uf, out=so, ws=wsg))
            pos = B * (G + 1)
            greedy_bytes = 4.0 * V * pos                                  # every logit read once
            sample_bytes = 4.0 * V * B * (2 * G + 1) + 8.0 * V * B         # plus the two drawn-from rows again
            accept[f"B{B}_gamma{G}"] = {
                "positions": pos,
                "greedy_bytes": greedy_bytes, "sample_bytes": sample_bytes,
                "greedy_us": tgms * 1e3, "greedy_positions_per_s": pos / (tgms * 1e-3),
                "sample_us": tsms * 1e3, "sample_positions_per_s": pos / (tsms * 1e-3),
                "greedy_GBps": 4.0 * V * pos / (tgms * 1e-3) / 1e9,
                # per-call distributions: warm (logits just read, as in the pipeline) and cold (L2 and
                # MALL flushed by a 1 GiB read before each call)
                "greedy_warm": time_dist(lambda: qs.qs_verify_greedy(tg, dd, out=go, ws=wsg), before=spin),
                "greedy_cold": time_dist(lambda: qs.qs_verify_greedy(tg, dd, out=go, ws=wsg), reps=30, before=flush),
                "sample_warm": time_dist(lambda: qs.qs_verify_sample(tg, dr, dd, ua, uf, out=so, ws=wsg), before=spin),
                "sample_cold": time_dist(lambda: qs.qs_verify_sample(tg, dr, dd, ua, uf, out=so, ws=wsg), reps=30,
                                         before=flush),
            }
            a_ = accept[f"B{B}_gamma{G}"]
            # achieved HBM (or MALL, when warm) rate of the median call against the 8 TB/s HBM peak
            a_["roofline"] = {k: {"GBps": byt / (a_[k]["median_us"] * 1e-6) / 1e9,
                                  "frac": byt / (a_[k]["median_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS}
                              for k, byt in (("greedy_warm", greedy_bytes), ("greedy_cold", greedy_bytes),
                                             ("sample_warm", sample_bytes), ("sample_cold", sample_bytes))}
            del tg, dr, wsg
        del flush_buf
    
        # tree-shaped greedy verify: 16 sequences x 8-node random trees (parent uniform over earlier
        # nodes; a node's token is its parent's Top-1 with probability 0.96), V = 128256
        Bt, Tt = 16, 8
        tgt_tree = torch.from_numpy(W.logits(rng, (Bt, Tt, V), sigma=5.24)).to(dev)
        par_np = np.zeros((Bt, Tt), np.int32)
        par_np[:, 0] = -1
        for i in range(1, Tt):
            par_np[:, i] = rng.integers(0, i, size=Bt)
        tok_np = rng.integers(0, V, size=(Bt, Tt)).astype(np.int32)
        tree_tok, tree_par = torch.from_numpy(tok_np).to(dev), torch.from_numpy(par_np).to(dev)
        wst = torch.zeros(qs.verify_workspace_bytes(Bt, Tt - 1, V), dtype=torch.uint8, device=dev)
        r0 = qs.qs_verify_tree_greedy(tgt_tree, tree_tok, tree_par, ws=wst)
        t1 = r0["tgt_top1"].cpu().numpy()
        agree_t = rng.random((Bt, Tt)) < 0.96
        for i in range(1, Tt):
            tok_np[:, i] = np.where(agree_t[:, i], t1[np.arange(Bt), par_np[:, i]], tok_np[:, i])
        tree_tok.copy_(torch.from_numpy(tok_np))
        tr = qs.qs_verify_tree_greedy(tgt_tree, tree_tok, tree_par, ws=wst)
        ttms = time_calls(lambda: qs.qs_verify_tree_greedy(tgt_tree, tree_tok, tree_par, out=tr, ws=wst))
        accept[f"tree_B{Bt}_T{Tt}"] = {
            "positions": Bt * Tt, "greedy_us": ttms * 1e3, "greedy_positions_per_s": Bt * Tt / (ttms * 1e-3),
            "mean_accepted": float(tr["n_accept"].float().mean().item()),
        }
        del tgt_tree, wst
    
        # LM-head with the fused Top-1 epilogue against LM-head + a separate Top-1 launch (the head of
        # the stack above; W4A4 at M = 1 as in a draft step, W4A16 at M = 4 as in the verify)
        head_wp, head_sp, head_n, head_k = layers[-1]
        lmtop = {}
        for mode, mname, mm in ((qs.QS_W4A4, "w4a4_M1", 1), (qs.QS_W4A16, "w4a16_M4", 4)):
            xh = x_verify[:mm].contiguous()
            lg = torch.empty((mm, V), dtype=torch.float32, device=dev)
            wsl = torch.empty(max(1, qs.linear_workspace_bytes(mode, mm, V, head_k)), dtype=torch.uint8, device=dev)
            wsg = torch.zeros(qs.verify_workspace_bytes(mm, 0, V), dtype=torch.uint8, device=dev)
            go = qs.qs_verify_greedy(lg.view(mm, 1, V), None, ws=wsg, want_prob=True)
            wst1 = torch.zeros(qs.lmhead_top1_workspace_bytes(mode, mm, V, head_k), dtype=torch.uint8, device=dev)
            fo = qs.qs_lmhead_top1(mode, xh, head_wp, head_sp, V, logits=lg, ws=wst1)
    
            def separate():
                qs.qs_lmhead(mode, xh, head_wp, head_sp, V, logits=lg, ws=wsl)
                qs.qs_verify_greedy(lg.view(mm, 1, V), None, out=go, ws=wsg)
    
            sep_ms = time_calls(separate)
            fused_ms = time_calls(lambda: qs.qs_lmhead_top1(mode, xh, head_wp, head_sp, V, logits=lg, top1=fo["top1"],
                                                            top1_prob=fo["top1_prob"], ws=wst1))
            nolog_ms = time_calls(lambda: qs.qs_lmhead_top1(mode, xh, head_wp, head_sp, V, want_logits=False,
                                                            top1=fo["top1"], top1_prob=fo["top1_prob"], ws=wst1))
            assert bool((fo["top1"] == go["tgt_top1"].view(-1)).all()), "fused Top-1 differs from the verify kernel's"
            lmtop[mname] = {"separate_us": sep_ms * 1e3, "fused_us": fused_ms * 1e3, "fused_no_logits_us": nolog_ms * 1e3}
            del wsl, wsg, wst1, lg
        accept["lmhead_top1"] = lmtop
    
        # Verify pass + greedy acceptance, graph-replayed: the pass writing logits then the greedy verify
        # kernel reading them, against the pass with the Top-1 fused into its LM-head stage then the prefix
        # rule on the Top-1 ids (B = 1, gamma = 3: the persistent pass; B = 16, gamma = 7: batched kernels).
        fused_top1 = {}
        for (B, G) in ((1, GAMMA), (16, 7)):
            mm = B * (G + 1)
            xb = torch.from_numpy(W.activations(W.rng_for(22), mm, H)[0]).to(dev)
            db = torch.from_numpy(rng.integers(0, V, size=(B, G)).astype(np.int32)).to(dev)
            lg = torch.empty((mm, V), dtype=torch.float32, device=dev)
            wsc = torch.empty(chain.top1_workspace_bytes(qs.QS_W4A16, mm), dtype=torch.uint8, device=dev)
            wsg = torch.zeros(qs.verify_workspace_bytes(B, G, V), dtype=torch.uint8, device=dev)
            t1b = torch.empty((mm,), dtype=torch.int32, device=dev)
            p1b = torch.empty((mm,), dtype=torch.float32, device=dev)
            go = qs.qs_verify_greedy(lg.view(B, G + 1, V), db, ws=wsg)
            ao = qs.qs_accept_greedy(t1b.view(B, G + 1), db)
    
            def separate():
                qs.qs_chain_forward(qs.QS_W4A16, xb, chain, out=lg, ws=wsc)
                qs.qs_verify_greedy(lg.view(B, G + 1, V), db, out=go, ws=wsg)
    
            def fused():
                qs.qs_chain_forward_top1(qs.QS_W4A16, xb, chain, out=None, want_logits=False, top1=t1b, top1_prob=p1b,
                                         ws=wsc)
                qs.qs_accept_greedy(t1b.view(B, G + 1), db, out=ao)
    
            graphs_ = {}
            for name, fn in (("separate", separate), ("fused", fused)):
                fn()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn()
                graphs_[name] = g
            # interleaved rounds, median of the per-round means (the pass itself varies by ~1% between replays)
            rounds = {"separate": [], "fused": []}
            for _ in range(5):
                for name in ("separate", "fused"):
                    rounds[name].append(time_calls(graphs_[name].replay, reps=8) * 1e3)
            res = {k: float(np.median(v)) for k, v in rounds.items()}
            assert bool((go["out_tokens"] == ao["out_tokens"]).all()), "fused and separate greedy paths disagree"
            fused_top1[f"B{B}_gamma{G}"] = {"M": mm, "separate_us": res["separate"], "fused_us": res["fused"],
                                            "saved_us": res["separate"] - res["fused"],
                                            "logit_bytes_not_reread": 4 * mm * V}
            log(f"verify + greedy, B={B} gamma={G}: pass then greedy kernel {res['separate']:.1f} us, fused Top-1 then "
                f"accept {res['fused']:.1f} us")
            del lg, wsc, wsg
    
        # ---------------- configs 0-2, one linear at a time (MALL-rotated weight copies)
        per_linear = linear_rates(qs, W, torch, E)
        log("per-linear W4A16 M=4 GB/s: " + ", ".join(f"{k}: {v['w4a16_M4']['GBps']:.0f}" for k, v in per_linear.items()))
    
        # ---------------- batched verify: B sequences x (gamma + 1) rows through the same stack
        # Sweep gamma in {3, 5, 7} x B in {1, 4, 16} (M = B (gamma + 1)) in all three modes (W4A8: the same
        # INT4 weights with 8-bit activations on the int8 MFMA); each point is one
        # graph-replayed pass, timed with HIP events.  MFMA utilisation = 2 M (weights) flop / time
        # against the dense peak of the mode's MFMA (fp16 2.5166 PFLOP/s, int8 5.0332 POP/s).
        n_weights = sum(n * k for (_, n, k) in shapes)
        peaks = {qs.QS_W4A16: 2.5166e15, qs.QS_W4A4: 5.0332e15, qs.QS_W4A8: 5.0332e15}
        batched = {"points": []}
        rng_b = W.rng_for(21)
        for (B, G) in ((1, 3), (1, 5), (1, 7), (4, 3), (4, 5), (4, 7), (16, 3), (16, 5), (16, 7)):
            m = B * (G + 1)
            xb = torch.from_numpy(W.activations(rng_b, m, W.HIDDEN)[0]).to(dev)
            ob = torch.empty((m, V), dtype=torch.float32, device=dev)
            for mode, mname in ((qs.QS_W4A16, "w4a16"), (qs.QS_W4A4, "w4a4"), (qs.QS_W4A8, "w4a8")):
                wsb = torch.empty(chain.workspace_bytes(mode, m), dtype=torch.uint8, device=dev)
                qs.qs_chain_forward(mode, xb, chain, out=ob, ws=wsb)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    qs.qs_chain_forward(mode, xb, chain, out=ob, ws=wsb)
                g.replay()
                torch.cuda.synchronize()
                ea, eb = E(enable_timing=True), E(enable_timing=True)
                ea.record()
                for _ in range(3):
                    g.replay()
                eb.record()
                torch.cuda.synchronize()
                ms = ea.elapsed_time(eb) / 3
                ops = 2.0 * m * n_weights
                batched["points"].append({
                    "B": B, "gamma": G, "M": m, "mode": mname, "pass_ms": ms,
                    "weight_GBps": pass_bytes / (ms * 1e-3) / 1e9,
                    "tflops": ops / (ms * 1e-3) / 1e12,
                    "mfma_util": ops / (ms * 1e-3) / peaks[mode],
                    "persistent_launches": chain.pass_launches(mode, m),
                })
                del g, wsb
            assert bool(torch.isfinite(ob).all()), "non-finite batched logits"
            del xb, ob
        for pt in batched["points"]:
            if pt["M"] == 128:
                batched[f"M128_{pt['mode']}"] = {k: pt[k] for k in ("pass_ms", "weight_GBps", "tflops", "mfma_util")}
        log("batched verify M=128: W4A16 %.3f ms (%.1f%% of fp16 MFMA), W4A4 %.3f ms (%.1f%% of int8 MFMA)" % (
            batched["M128_w4a16"]["pass_ms"], 100 * batched["M128_w4a16"]["mfma_util"],
            batched["M128_w4a4"]["pass_ms"], 100 * batched["M128_w4a4"]["mfma_util"]))
    
        # ---------------- speculative timing model and draft-length choice (host-side planner)
        # t_target: one plain decoding step = W4A16 pass at M = 1 (graph-replayed); t_draft: one draft
        # pass + draft Top-1 of the iteration above; t_verify: its verify pass; t_overhead: its accept
        # phase.  alpha = 0.96 (the pages' W4A4/W4A16 Top-1 agreement, rounded).
        from quantized_speculative_decoding_int4_amd import planner as PL
        ALPHA = 0.96
        x1 = x_verify[:1].contiguous()
        o1 = torch.empty((1, V), dtype=torch.float32, device=dev)
        ws1 = torch.empty(chain.workspace_bytes(qs.QS_W4A16, 1), dtype=torch.uint8, device=dev)
        qs.qs_chain_forward(qs.QS_W4A16, x1, chain, out=o1, ws=ws1)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            qs.qs_chain_forward(qs.QS_W4A16, x1, chain, out=o1, ws=ws1)
        target_ms = time_calls(g1.replay, reps=10)
        del g1, ws1
        # the same one-row pass in W4A8 (8-bit activation codes on the same int8 MFMA), as a draft
        ws8 = torch.empty(chain.workspace_bytes(qs.QS_W4A8, 1), dtype=torch.uint8, device=dev)
        qs.qs_chain_forward(qs.QS_W4A8, x1, chain, out=o1, ws=ws8)
        g8 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g8):
            qs.qs_chain_forward(qs.QS_W4A8, x1, chain, out=o1, ws=ws8)
        w4a8_draft_ms = time_calls(g8.replay, reps=10)
        del g8, ws8
        t_draft1 = draft_ms / GAMMA
        spec = {
            "alpha": ALPHA, "gamma": GAMMA,
            "expected_tokens": PL.expected_tokens(ALPHA, GAMMA),
            "t_target_ms": target_ms, "t_draft_ms": t_draft1, "t_verify_ms": verify_ms, "t_overhead_ms": accept_ms,
            "modelled_speedup": PL.modelled_speedup(ALPHA, GAMMA, target_ms, t_draft1, verify_ms, accept_ms),
            "itl_ms": PL.inter_token_latency(ALPHA, GAMMA, ms_step),
            "target_itl_ms": target_ms,
            "w4a8_draft_pass_ms": w4a8_draft_ms,
            "w4a8_draft_persistent_launches": chain.pass_launches(qs.QS_W4A8, 1),
        }
        # per batch: draft step = W4A4 pass at M = B (B = 1: the draft pass above), verify = W4A16 pass at
        # M = B (gamma + 1), both from the sweep; accept / Top-1 costs (tens of us) left out
        pts = {(p_["mode"], p_["M"]): p_["pass_ms"] for p_ in batched["points"]}
        choice = {}
        for B in (1, 4, 16):
            td = t_draft1 if B == 1 else pts.get(("w4a4", B))
            tv = {G: pts[("w4a16", B * (G + 1))] for G in (3, 5, 7) if ("w4a16", B * (G + 1)) in pts}
            if td is None or not tv:
                continue
            c = PL.choose_gamma(ALPHA, B, td, tv)
            choice[f"B{B}"] = {"best_gamma": c["best_gamma"], "t_draft_ms": td,
                               "tokens_per_s": {str(G): 1e3 * r["tokens_per_time"] for G, r in c["table"].items()}}
        spec["gamma_choice"] = choice
        log("speculative model: E[T] %.3f, t_target %.3f ms, speed-up %.3f, ITL %.3f ms (target alone %.3f); "
            "best gamma by batch %s" % (spec["expected_tokens"], target_ms, spec["modelled_speedup"], spec["itl_ms"],
                                        target_ms, {k: v["best_gamma"] for k, v in choice.items()}))
        return accept, fused_top1, per_linear, batched, spec

    if args.core_only:
        accept, fused_top1, per_linear, batched, spec = None, None, None, None, None
    else:
        accept, fused_top1, per_linear, batched, spec = optional_sections()

    # ---------------- rooflines of the pass kernels (HIP events on the launch stream)
    # Algorithmic bytes of one pass: packed weights (0.515625 B per weight) plus, per linear,
    # x = 2*M*K and y = 4*M*N bytes.  A pass runs as `launches` persistent launches, each
    # preceded by a one-workgroup control reset; bytes and time are averaged per launch.  The pass
    # is the one of the iteration: the LM-head's Top-1 fused into the last stage.
    stream = torch.cuda.current_stream()

    def pass_roofline(mode, m, x, out, top1, ws, name, traffic_key, reps=10):
        launches = chain.pass_launches(mode, m)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qs.qs_chain_forward_top1(mode, x, chain, out=out, top1=top1, want_prob=False, ws=ws)
        g.replay()
        torch.cuda.synchronize()
        evs = [(E(enable_timing=True), E(enable_timing=True)) for _ in range(reps)]
        for a, b in evs:
            a.record(stream)
            g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        pass_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        alg = pass_bytes + sum(2 * m * k + 4 * m * n for (_, n, k) in shapes)
        per = max(launches, 1)
        achieved = alg / (pass_ms * 1e-3) / 1e9
        log(f"{name}: {pass_ms * 1e3:.1f} us per pass, {launches} launches, {achieved:.0f} GB/s")
        return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": counted_traffic(traffic_key), "kernel": name,
                "bytes_per_launch": alg / per, "avg_launch_us": pass_ms * 1e3 / per,
                "launches_per_pass": launches, "passes_timed": reps}

    roof_draft = pass_roofline(qs.QS_W4A4, 1, x_draft[0], logits_q[0, 0:1], d_steps[0], ws_draft,
                               "pass_kernel<W4A4> (draft pass, M=1, int8 MFMA)", "w4a4")
    roof_verify = pass_roofline(qs.QS_W4A16, M_VERIFY, x_verify, logits_p[0], t_verify, ws_verify,
                                "pass_kernel<W4A16> (verify pass, M=4, fp16 MFMA)", "w4a16")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline(args.cpu_budget_s)
        cpu["per_config"] = cpu_per_config(args.cpu_budget_s)
        log(f"oracle per config: {cpu['per_config']['wall_s']:.1f} s")

    result = {
        "metric": METRIC,
        "value": verify_gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": ("Llama-3-8B-shaped INT4 (group-128, fp16 scales) 32-layer linear stack + 4096->128256 "
                         "LM-head; one speculative iteration at batch 1, gamma 3: 3 W4A4 draft passes (M=1, "
                         "int8 MFMA), 1 W4A16 verify pass (M=4, fp16 MFMA), each pass's Top-1 fused into its "
                         "LM-head stage, greedy accept on the Top-1 ids + sampling accept on the logits"),
            "verify_rows": M_VERIFY, "gamma": GAMMA, "batch": 1, "vocab": V,
            "weight_bytes_per_pass": pass_bytes, "graphs": not args.eager,
        },
        "hbm_frac": verify_gbs / HBM_PEAK_GBS,
        "verify_pass_ms": verify_ms,
        "verify_phase_dist": verify_dist,
        "draft_pass_ms": draft_ms / GAMMA,
        "draft_phase_dist": draft_dist,
        "draft_pass_GBps": draft_gbs,
        "accept_phase_ms": accept_ms,
        "iteration_accepted_tokens": n_acc + 1,
        "draft_verify_top1_agreement": agree,
        "accept_positions_per_s": accept,
        "verify_greedy_fused_top1": fused_top1,
        "batched_verify": batched,
        "per_linear": per_linear,
        "speculative_model": spec,
        "roofline": roof_draft,
        "roofline_verify": roof_verify,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_calibration_mib} MiB copied twice")


if __name__ == "__main__":
    main()
