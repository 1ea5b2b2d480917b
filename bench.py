"""Throughput of the predictor-gated sparse FFN decode stack on one MI355X.

Default workload: the OPT-175B-shaped FFN stack on one GPU (96 layers,
d_model 12288, d_ff 49152, INT4-g128 FFN weights quantised from N(0, 0.02),
ReLU at ~90% per-token sparsity, rank-1024 fp16 predictor per layer), batch 1,
decode steps of fresh x ~ N(0, I) through the RMS-normalised residual chain.
The weights of 4 distinct layers (3 GB, far beyond the 256 MB memory-side
cache) are cycled through the 96 layers.  One step = one sfnn_stack_decode
call: for every layer, predict -> compact -> sparse FFN, joined by the
residual + RMSNorm chain, in the look-ahead schedule (layer l+1's predictor
runs on layer l's input, two launches per layer); --per-layer-predictor times
the schedule that predicts each layer from its own input.  Weights are drawn
on the host from seeded streams and copied to HBM before timing; a step is
captured once in a HIP graph and replayed, the next token copied in between.

Prints one JSON line: metric/value/unit, ms_per_step (and the median and p90
of the per-step times), the roofline of one stack layer, the error of sampled
layers against the CPU oracle, the CPU-oracle baseline, and a breakdown under
"extra" (including the LLaMA-ReGLU-70B stack at batch 1).

--copy-probe only runs the 16-byte copy kernel over a known number of bytes
(the calibration run for the HBM traffic counters) and prints its size.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--config", default="c5", help="workload: c5 (default) | c2 | c3 | c4")
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--rho", type=float, default=None, help="override the mean fire probability")
    ap.add_argument("--per-layer-predictor", action="store_true",
                    help="time the schedule that predicts every layer from its own input "
                         "(default: the look-ahead schedule, layer l+1 predicted from layer l's input)")
    ap.add_argument("--heads", action="store_true",
                    help="head-gated Q/K/V and output projections over head density and batch (OPT-6.7B and "
                         "OPT-175B attention shapes)")
    ap.add_argument("--read-sizes", action="store_true",
                    help="time one read-probe launch per size (4 MB .. 512 MB), each on a region not read "
                         "for the last 32 launches, so neither L2 nor the memory-side cache serves it")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run the copy kernel over 1 GiB, 4 times (traffic-counter calibration)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-extra", action="store_true", help="skip per-kernel, dense and probe timings")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--distinct-layers", type=int, default=-1,
                    help="draw this many distinct layers and cycle them through the stack (0: all distinct; "
                         "default: all when the stack holds at most 10 GB of FFN weights, else 4)")
    ap.add_argument("--extra-config", default="c4",
                    help="a second stack at batch 1 reported under extra ('' to skip)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the stack: sparse vs dense FFN per layer over batch sizes and fire rates")
    ap.add_argument("--sweep-batches", default="1,2,4,8,16,32")
    ap.add_argument("--sweep-rhos", default="0.05,0.1,0.2")
    ap.add_argument("--hot-prefix", default="0",
                    help="dense hot prefix of power-law workloads: a neuron count (multiple of 64) or 'auto' "
                         "(chosen per layer from the profiled fire rates of the batch's union)")
    ap.add_argument("--dense-min-batch", default="0",
                    help="the predictor descriptors' dense switch: from this batch on a layer skips the predictor "
                         "and runs the dense FFN (0, the library default, or negative: never; 'auto': per layer "
                         "from fire counts profiled on the stack, the union law and the measured crossover)")
    ap.add_argument("--isg", action="store_true",
                    help="time the input-sparse GEMV (ReLU after the norm) over input densities and batches")
    ap.add_argument("--only", default="",
                    help="with --isg or --heads: one point, 'shape,batch,density' (e.g. 'up,1,0.5' or "
                         "'opt6.7b,1,1.0'), for profiling a single workload")
    return ap.parse_args()


HBM_PEAK_GBS = 8000.0
# Union share of d_ff from which the dense FFN beats predictor + sparse FFN,
# measured on MI355X: fp16 ReLU 0.45 (OPT-6.7B sweep: the layer wins on a 34%
# union, loses on 57%), INT4-g128 0.65 (OPT-175B sweep: wins at 56%, loses at
# 72%), fp16 ReGLU 0.85 (three matrices per neuron, so the predictor weighs
# less: the LLaMA-ReGLU-70B stack ran sparse on a 58% union at batch 16 in 266
# us against 317 dense, and on a 78% union at batch 32 in 350 against 372);
# fp32 takes the fp16 ReLU figure (not measured on its own).
def dense_crossover(spec):
    if spec.wtype == "i4g128":
        return 0.65
    return 0.85 if spec.act == "reglu" else 0.45
COPY_PROBE_BYTES = 1 << 30
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def _kernel_source_digest():
    """Digest of the kernel sources, to tell whether stored counter figures still apply."""
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "activation_sparse_gemv_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _stored_traffic(workload):
    """HBM bytes per stack layer from a committed counter summary under
    profiles/ (a `traffic-json:` line), if one was taken on this workload with
    the current kernel sources (else None)."""
    digest = _kernel_source_digest()
    try:
        names = sorted(os.listdir(PROFILES))
    except OSError:
        return None
    for name in names:
        if not name.endswith("_hbm_traffic.md"):
            continue
        with open(os.path.join(PROFILES, name)) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("source_digest") == digest and rec.get("workload") == workload:
                        return rec
    return None


def main():
    args = _parse()
    if args.gpus != 1:
        msg = ("bench.py measures one GPU only: the hot path has no inter-GPU step; "
               f"--gpus {args.gpus} is not supported")
        print(msg, file=sys.stderr)
        print(json.dumps({"error": msg, "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import synth
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import to_dev, upload_layer, workspace

    if args.read_sizes:
        _read_sizes(sg)
        return
    if args.copy_probe:
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            sg.sfnn_probe_copy(src, dst, COPY_PROBE_BYTES)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "launches": 4}), flush=True)
        return

    dev = "cuda"
    over = {}
    if args.rho is not None:
        over["rho"] = args.rho
    spec = synth.config(args.config, **over)
    if args.isg:
        _isg_sweep(args)
        return
    if args.heads:
        _heads_sweep(args)
        return
    if args.sweep:
        _sweep(args, spec)
        return
    res = _stack_run(args, spec, args.batch, headline=True)
    out = res.pop("out")
    extra = res.pop("extra")
    if args.extra_config and not args.no_extra and args.extra_config != args.config:
        # a second workload at batch 1, reported beside the headline
        spec2 = synth.config(args.extra_config)
        r2 = _stack_run(args, spec2, 1, headline=False)
        o2, e2 = r2["out"], r2["extra"]
        extra["other_workload"] = {"workload": o2["config"]["workload"], "batch": 1,
                                   "tokens_s": o2["value"], "ms_per_step": o2["ms_per_step"],
                                   "ms_per_step_median": o2["ms_per_step_median"],
                                   "roofline_frac": o2["roofline"]["frac"],
                                   "achieved_GBps": o2["roofline"]["achieved"],
                                   "active_fraction": e2["active_fraction"],
                                   "max_rel_err_vs_oracle": o2.get("max_rel_err_vs_oracle")}
    out["extra"] = extra
    print(json.dumps(out), flush=True)


def _stack_run(args, spec, B, headline):
    """Time sfnn_stack_decode over the workload's layers at batch B; returns
    the JSON line's fields ("out") and the breakdown ("extra")."""
    import torch
    import synth
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import to_dev, upload_layer, workspace
    dev = "cuda"
    L = spec.n_layers
    d, f, r = spec.d_model, spec.d_ff, spec.rank
    t0 = time.time()

    # ---- weights: drawn per layer on the host, resident in HBM -------------
    wb = {"f32": 4.0, "f16": 2.0, "i4g128": 0.5 + 2.0 / 128}[spec.wtype]
    layer_gb = spec.n_mat * f * d * wb / 1e9
    nd = args.distinct_layers
    if nd < 0:
        nd = L if L * layer_gb <= 10.0 else 4
    nd = L if nd == 0 else min(nd, L)
    distinct, hosts = [], []
    for l in range(nd):
        lay = synth.make_layer(spec, layer=l)
        distinct.append(upload_layer(lay, device=dev))
        if headline and len(hosts) < 4:
            hosts.append(lay)  # kept for the oracle check and the CPU baseline
        del lay
    layers = [distinct[l % nd] for l in range(L)]
    auto_switch = args.dense_min_batch == "auto"
    for pred, _ in distinct:
        pred.dense_min_batch = -1 if auto_switch else int(args.dense_min_batch)
    torch.cuda.synchronize()
    t_setup = time.time() - t0
    print(f"# {L} layers of {spec.name} ({nd} distinct) resident in HBM after {t_setup:.1f}s",
          file=sys.stderr, flush=True)

    # ---- hot-first relayout for power-law workloads -------------------------
    hots = [0] * nd
    if spec.profile == "zipf":
        hots = _hot_first(sg, distinct, spec, B, dev, args.hot_prefix)
        for k, lay in enumerate(hosts):
            # the host copies follow the device relayout (rows permuted the same way)
            hosts[k] = _host_relayout(lay, distinct[k])
    elif args.hot_prefix != "0":
        sys.exit("a dense hot prefix needs the hot-first relayout of a power-law workload (c3, c4)")
    hot_mean = float(np.mean([hots[l % nd] for l in range(L)]))

    # ---- dense switch per layer (past it: the dense FFN, no predictor) ------
    if auto_switch:
        _auto_dense_switch(sg, distinct, spec, dev, 0 if args.per_layer_predictor else sg.SFNN_STACK_LOOKAHEAD)
    thr = [pred.dense_min_batch for pred, _ in distinct]
    dense_l = [0 < thr[l % nd] <= B for l in range(L)]
    n_dense = int(sum(dense_l))
    dense = n_dense == L

    xdt = torch.float32 if spec.wtype == "f32" else torch.float16
    steps, warmup = (args.steps, args.warmup) if headline else (min(args.steps, 64), min(args.warmup, 8))
    ntok = steps + warmup
    tokens = to_dev(synth.make_tokens(spec, ntok * B, stream=7, dtype=np.float32)).view(ntok, B, d)
    stage = torch.empty((B, d), dtype=torch.float32, device=dev)
    rbuf = torch.empty((B, d), dtype=torch.float32, device=dev)
    counts = torch.zeros((L + 4,), dtype=torch.int32, device=dev)
    ws = workspace(layers[0][0], layers[0][1], B)
    stack = sg.Stack(layers)

    lookahead = not args.per_layer_predictor
    flags = sg.SFNN_STACK_LOOKAHEAD if lookahead else 0

    def make_step(fl):
        # one decode step: every layer's predict -> compact -> sparse FFN, joined
        # by the residual chain (r += y; x = RMSNorm(r)), all inside the library
        return lambda: sg.sfnn_stack_decode(stack, B, stage, rbuf, 1e-6, ws, flags=fl, count_cap=counts)

    def capture(fn):
        # eager warm-up on a side stream, then capture one step
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            stage.copy_(tokens[0])
            fn()
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def run(g, n, first):
        """n steps (token copy + graph replay); HIP events on the stream the
        kernels run on, one before each step and one after the last.
        Returns (total ms, per-step ms)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for t in range(n):
            stage.copy_(tokens[first + t])
            g.replay()
            ev[t + 1].record()
        torch.cuda.synchronize()
        per = [ev[t].elapsed_time(ev[t + 1]) for t in range(n)]
        return ev[0].elapsed_time(ev[n]), per

    graph = capture(make_step(flags))
    run(graph, warmup, 0)
    elapsed_ms, per_step = run(graph, steps, warmup)
    ms_per_step = elapsed_ms / steps
    tok_s = B * steps / (elapsed_ms / 1e3)
    cnt = counts[:L].cpu().numpy().astype(np.float64)
    mean_u = float(cnt.mean())
    # the other schedule, timed the same way (reported beside the main figure)
    other = capture(make_step(0 if lookahead else sg.SFNN_STACK_LOOKAHEAD))
    run(other, min(warmup, 8), 0)
    n_other = min(steps, 64)
    other_ms = run(other, n_other, warmup)[0] / n_other
    del other

    # the layer inputs, masks, ids and outputs of one more step, for the
    # oracle check and the per-call timings below
    xcap = torch.empty((L, B, d), dtype=xdt, device=dev)
    ycap = torch.empty((L, B, d), dtype=torch.float32, device=dev)
    masks = torch.zeros((L, B, f // 64), dtype=torch.uint64, device=dev)
    ids = torch.zeros((L, f), dtype=torch.int32, device=dev)
    stage.copy_(tokens[0])
    sg.sfnn_stack_decode(stack, B, stage, rbuf, 1e-6, ws, flags=flags, x_cap=xcap, y_cap=ycap, mask_cap=masks,
                         ids_cap=ids, count_cap=counts)
    torch.cuda.synchronize()

    # ---- algorithmic bytes ----------------------------------------------------
    row_bytes = d * wb
    xb = 4 if spec.wtype == "f32" else 2
    pb = 4 if spec.pred_dtype == "f32" else 2
    nmat = spec.n_mat
    ffn_bytes_u = lambda u: u * nmat * row_bytes + u * (nmat - 1) * xb          # noqa: E731
    pred_bytes = (d * r + r * (f - hot_mean)) * pb + 4 * (f - hot_mean)  # hot-prefix rows are not read
    pred_bytes *= (L - n_dense) / L  # dense layers run no predictor
    ffn_bytes = ffn_bytes_u(mean_u)
    cycled = "" if nd == L else f" (weights of {nd} distinct layers, {nd * layer_gb:.1f} GB, cycled)"
    workload = (f"{spec.name} FFN stack: {L} layers{cycled}, d_model {d}, d_ff {f}, rank-{r} predictor, "
                f"{spec.act}, {spec.wtype}, "
                f"{'zipf phi=%.2f ' % spec.phi if spec.profile == 'zipf' else ''}rho={spec.rho}, batch {B}"
                f"{', dense hot prefix %s' % args.hot_prefix if hot_mean else ''}"
                + (f", dense switch: every layer dense (thresholds {thr}), no predictor" if dense else
                   (", look-ahead predictor" if lookahead else ", per-layer predictor")
                   + (f", dense switch: {n_dense} of {L} layers dense (thresholds {thr})" if n_dense else "")))
    per_sorted = np.sort(np.asarray(per_step))
    out = {
        "metric": "sparse-FFN decode tokens/sec at batch 1 + effective HBM GB/s on active bytes",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(float(np.median(per_sorted)), 4),
        "ms_per_step_p90": round(float(per_sorted[min(len(per_sorted) - 1, int(np.ceil(0.9 * len(per_sorted))) - 1)]), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if spec.wtype == "f16" else ("f32" if spec.wtype == "f32" else "i4g128+f16"),
        "data": "synthetic (seeded N(0,0.02) weights, calibrated biases/thresholds, x~N(0,1))",
        "config": {"workload": workload, "global_batch": B, "decode_steps": steps, "layers": L,
                   "distinct_layers": nd,
                   "predictor": ("none: every layer past its dense switch") if dense else
                   ("look-ahead (layer l+1 from x_l)" if lookahead else "per layer (layer l from x_l)")},
    }
    extra = {"mean_active_neurons": round(mean_u, 1), "active_fraction": round(mean_u / f, 4),
             "expected_union_fraction": round(synth.union_density(synth.layer_probs(spec, 0), B), 4),
             "ffn_active_bytes_per_layer": int(ffn_bytes), "predictor_bytes_per_layer": int(pred_bytes),
             "setup_s": round(t_setup, 1), "dense_min_batch_per_distinct_layer": thr,
             "dense_switch": "auto" if auto_switch else args.dense_min_batch, "dense_layers": n_dense}
    if hot_mean:
        extra["hot_prefix_per_layer"] = hots
    extra["layer_GBps_stack"] = round(L * (ffn_bytes + pred_bytes) / (ms_per_step / 1e3) / 1e9, 1)
    key = "tokens_s_per_layer_predictor" if lookahead else "tokens_s_lookahead_predictor"
    extra[key] = round(B / (other_ms / 1e3), 2)

    # ---- the oracle on sampled layers of the captured step ------------------
    if headline:
        out.update(_oracle_check(spec, hosts, nd, L, B, xcap, ycap, masks, ids, counts, lookahead, dense_l))

    # ---- per-call timings: each call captured for all layers in one graph ----
    if headline and not args.no_extra:
        reps = 8
        y2 = torch.empty((B, d), dtype=torch.float32, device=dev)

        def timed(fn):
            """Average duration of one layer's call, us (HIP events around graph replays)."""
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                g.replay()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / (reps * L) * 1e3

        gate = (lambda l: masks[l]) if B > 1 else (lambda l: None)
        t_ffn = timed(lambda: [sg.sfnn_sparse_ffn(ffn, xcap[l], B, ids[l], counts[l:l + 1], gate(l), y2, ws)
                               for l, (_, ffn) in enumerate(layers)])
        t_pred = timed(lambda: [sg.sfnn_predict(pred, xcap[l], B, masks[l], None, ws)
                                for l, (pred, _) in enumerate(layers)])
        t_comp = timed(lambda: [sg.sfnn_compact(masks[l], B, f, ids[l], counts[l:l + 1]) for l in range(L)])
        t_dense = timed(lambda: [sg.sfnn_dense_ffn(ffn, xcap[l], B, y2, ws) for l, (_, ffn) in enumerate(layers)])
        t_layer = timed(lambda: [sg.sfnn_layer(pred, ffn, xcap[l], B, y2, masks[l], ids[l], counts[l:l + 1], ws)
                                 for l, (pred, ffn) in enumerate(layers)])
        dense_bytes = f * nmat * row_bytes + f * (nmat - 1) * xb
        extra.update({
            "us_sparse_ffn": round(t_ffn, 2), "us_predict": round(t_pred, 2), "us_compact": round(t_comp, 2),
            "us_layer": round(t_layer, 2), "us_dense_ffn": round(t_dense, 2),
            "GBps_ffn_active": round(ffn_bytes / t_ffn / 1e3, 1),
            "GBps_predict": round(pred_bytes / t_pred / 1e3, 1),
            "GBps_layer": round((ffn_bytes + pred_bytes) / t_layer / 1e3, 1),
            "GBps_dense_ffn": round(dense_bytes / t_dense / 1e3, 1),
            "speedup_sparse_vs_dense_ffn": round(t_dense / t_ffn, 2),
            "tokens_s_dense_ffn_stack_only": round(B / (L * t_dense * 1e-6), 1),
        })
        # read-bandwidth probe over 4 GiB (same 16-byte load width)
        buf = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
        sink = torch.zeros(4, dtype=torch.float32, device=dev)
        sg.sfnn_probe_read(buf, buf.numel(), sink)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            sg.sfnn_probe_read(buf, buf.numel(), sink)
        b.record()
        torch.cuda.synchronize()
        probe = 5 * buf.numel() / (a.elapsed_time(b) / 1e3) / 1e9
        extra["probe_read_GBps"] = round(probe, 1)
        del buf
        extra["sparse_ffn_call_roofline"] = {
            "kernels": "sfnn_sparse_ffn: k_up (listed rows of W_up) + k_down (column-tiled W_down^T rows)",
            "bytes_per_call": int(ffn_bytes), "us_per_call": round(t_ffn, 2),
            "achieved_GBps": round(ffn_bytes / t_ffn / 1e3, 1),
            "frac": round(ffn_bytes / t_ffn / 1e3 / HBM_PEAK_GBS, 4)}

    # ---- roofline of one stack layer (the timed step / layers) ---------------
    # algorithmic bytes of a layer: the active rows of the FFN plus the whole
    # predictor; its time: the step's HIP-event time divided by the layers
    us_layer_stack = ms_per_step * 1e3 / L
    layer_bytes = ffn_bytes + pred_bytes
    workload_key = (f"{spec.name}/b{B}/{'dense' if dense else ('lookahead' if lookahead else 'per-layer')}"
                    f"{'/mixed%d' % n_dense if n_dense and not dense else ''}"
                    f"{'/hot%s' % args.hot_prefix if hot_mean else ''}")
    tr = _stored_traffic(workload_key)
    out["roofline"] = {
        "bound": "hbm", "achieved": round(layer_bytes / us_layer_stack / 1e3, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(layer_bytes / us_layer_stack / 1e3 / HBM_PEAK_GBS, 4),
        "traffic": (int(tr["fetch_bytes_per_layer"] + tr["write_bytes_per_layer"]) if tr else None),
        "kernel": ("stack layer, dense switch: RMSNorm + the dense FFN" if dense else
                   ("stack layer, %d of %d layers dense (RMSNorm + the dense FFN), the others predictor-gated"
                    % (n_dense, L)) if n_dense else
                   ("stack layer, look-ahead: k_la_up_pred1 (FFN_l up rows + predictor stage 1 of l+1) "
                    "+ k_la_down_pred2 (FFN_l column-tiled down rows + predictor stage 2 of l+1)") if lookahead else
                   ("stack layer, per-layer predictor: k_pred1 + k_pred2 + k_up + k_down")),
        "bytes_per_launch": int(layer_bytes), "us_per_launch": round(us_layer_stack, 3),
        "launch": "one stack layer (two kernels in the look-ahead schedule)",
    }
    extra["us_per_layer_stack"] = round(us_layer_stack, 3)
    extra["traffic_workload_key"] = workload_key

    # ---- CPU oracle baseline (bounded sample) ---------------------------------
    if headline and not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(hosts, spec, B, L, args.cpu_seconds)
    return {"out": out, "extra": extra}


def _host_relayout(lay, dev_layer):
    """The host copy of a layer in the device's hot-first order: the device
    tensors were permuted in place by sfnn_gather_rows, so read them back."""
    import copy
    pred, ffn = dev_layer
    h = copy.copy(lay)
    for k in ("w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t", "b_up", "b_gate"):
        t = ffn.t.get(k)
        if t is not None:
            name = k if getattr(lay, k, None) is not None else k.replace("w_", "q_")
            setattr(h, name, t.cpu().numpy())
    h.w2_t = pred.w2_t.cpu().numpy()
    h.tau = pred.tau.cpu().numpy()
    return h


def _oracle_check(spec, hosts, nd, L, B, xcap, ycap, masks, ids, counts, lookahead, dense_l):
    """Layers 0 and L-1 of the captured step against the fp64 oracle on the
    same inputs: the ids and count of the mask the GPU used (bit-exact), the
    FFN output for that mask (normwise relative error), and for layer 0 the
    predicted mask (bit-exact outside the fp32 rounding band).  A layer past
    its dense switch (dense_l[l]) has the all-ones mask (no predictor ran),
    so its FFN check is the oracle's dense FFN, on token 0 only, and only
    where its float64 rows stay small (d_model * d_ff <= 2^27): over every
    row of a larger layer the host would need minutes per token."""
    import oracle
    f = spec.d_ff
    big = spec.d_model * f > (1 << 27)
    checked = [l for l in sorted({0, L - 1}) if not (dense_l[l] and big)]
    if not checked:
        return {"max_rel_err_vs_oracle": None,
                "oracle_check": {"skipped": "dense FFN of d_model %d x d_ff %d: the float64 oracle over every "
                                            "row takes minutes per token on the host; the dense switch's parity "
                                            "is in tests/test_gpu_dense_switch.py" % (spec.d_model, f)}}
    errs, ids_ok, flips = [], True, 0
    xs = xcap.float().cpu().numpy()
    ys = ycap.cpu().numpy()
    ms = masks.cpu().numpy()
    ids_h = ids.cpu().numpy()
    cnt_h = counts.cpu().numpy()
    for l in checked:
        dense = dense_l[l]
        lay = hosts[l % nd] if l % nd < len(hosts) else None
        if lay is None:
            continue
        x = xs[l].astype(spec.x_dtype)
        rid, rc, _ = oracle.compact(ms[l], B, f)
        ids_ok = ids_ok and rc == int(cnt_h[l]) and np.array_equal(rid, ids_h[l][:rc])
        nb = 1 if dense else B
        ref = oracle.masked_ffn(lay, x[:nb], oracle.unpack_mask(ms[l][:nb], f))
        errs.append(float(np.abs(ys[l][:nb] - ref).max() / max(np.abs(ref).max(), 1e-30)))
        if dense:
            ids_ok = ids_ok and bool((oracle.unpack_mask(ms[l], f)).all())
        elif l == 0 or not lookahead:
            lg, ob = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
            band = oracle.guard_band(lay.w1_t, lay.w2_t, x)
            gb = oracle.unpack_mask(ms[l], f)
            outside = np.abs(lg - lay.tau[None, :].astype(np.float64)) > band
            flips += int(((gb != ob) & outside).sum())
    return {"max_rel_err_vs_oracle": round(max(errs), 8) if errs else None,
            "oracle_check": {"layers": checked, "ids_count_bit_exact": bool(ids_ok),
                             "mask_bits_outside_rounding_band_differing": flips, "tolerance": 2e-3}}


def _sweep(args, spec):
    """Sparse vs dense FFN per layer over batch sizes and fire rates.  Each point
    cycles over enough distinct layers (>= 1 GB of weights) that the 256 MB
    Infinity Cache cannot serve them; each call is timed with HIP events around
    a graph of calls over those layers."""
    import torch
    import synth
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import to_dev, upload_layer, workspace
    dev = "cuda"
    d, f, r = spec.d_model, spec.d_ff, spec.rank
    wb = {"f32": 4.0, "f16": 2.0, "i4g128": 0.5 + 2.0 / 128}[spec.wtype]
    nmat = spec.n_mat
    layer_bytes = f * nmat * d * wb + (d * r + r * f) * (4 if spec.pred_dtype == "f32" else 2)
    nl = max(2, int(np.ceil(1.0e9 / layer_bytes)))
    batches = [int(b) for b in args.sweep_batches.split(",") if b]
    rhos = [float(x) for x in args.sweep_rhos.split(",") if x] if spec.profile == "uniform" else [spec.rho]
    xdt = np.float32 if spec.wtype == "f32" else np.float16
    points = []
    for rho in rhos:
        sp = synth.config(args.config, rho=rho)
        layers = [upload_layer(synth.make_layer(sp, layer=l), device=dev) for l in range(nl)]
        for pred, _ in layers:
            pred.dense_min_batch = -1  # the predictor's union at every batch (the switch is timed below)
        if sp.profile == "zipf":
            _hot_first(sg, layers, sp, 8, dev)
        auto_thr = _thresholds_from_predictor(sg, layers, sp, dev)
        for B in batches:
            ws = workspace(layers[0][0], layers[0][1], B)
            x = [to_dev(synth.make_tokens(sp, B, stream=500 + l).astype(xdt)) for l in range(nl)]
            y = torch.empty((B, d), dtype=torch.float32, device=dev)
            masks = torch.zeros((nl, B, f // 64), dtype=torch.uint64, device=dev)
            ids = torch.zeros((nl, f), dtype=torch.int32, device=dev)
            cnt = torch.zeros((nl,), dtype=torch.int32, device=dev)
            for l, (pred, ffn) in enumerate(layers):
                sg.sfnn_layer(pred, ffn, x[l], B, y, masks[l], ids[l], cnt[l:l + 1], ws)
            torch.cuda.synchronize()
            u = float(cnt.float().mean().item())
            gate = (lambda l: masks[l]) if B > 1 else (lambda l: None)

            def timed(fn, reps=8):
                fn()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn()
                g.replay()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(reps):
                    g.replay()
                b.record()
                torch.cuda.synchronize()
                return a.elapsed_time(b) / (reps * nl) * 1e3

            def t_sparse():
                return timed(lambda: [sg.sfnn_sparse_ffn(ffn, x[l], B, ids[l], cnt[l:l + 1], gate(l), y, ws)
                                      for l, (_, ffn) in enumerate(layers)])

            def t_dense():
                return timed(lambda: [sg.sfnn_dense_ffn(ffn, x[l], B, y, ws) for l, (_, ffn) in enumerate(layers)])

            # the default batch-aware dispatch
            t_sp, t_de = t_sparse(), t_dense()
            t_ly = timed(lambda: [sg.sfnn_layer(pred, ffn, x[l], B, y, masks[l], ids[l], cnt[l:l + 1], ws)
                                  for l, (pred, ffn) in enumerate(layers)])
            t_pr = timed(lambda: [sg.sfnn_predict(pred, x[l], B, masks[l], None, ws)
                                  for l, (pred, _) in enumerate(layers)])
            pbytes = (d * r + r * f) * (4 if spec.pred_dtype == "f32" else 2) + 4 * f
            act_bytes = u * nmat * d * wb
            pt = {"rho": rho, "batch": B, "union_frac": round(u / f, 4),
                  "us_sparse_ffn": round(t_sp, 2), "us_layer": round(t_ly, 2), "us_dense_ffn": round(t_de, 2),
                  "us_predict": round(t_pr, 2), "GBps_predict": round(pbytes / t_pr / 1e3, 1),
                  "speedup_ffn": round(t_de / t_sp, 2), "speedup_layer_vs_dense_ffn": round(t_de / t_ly, 2),
                  "GBps_sparse_ffn": round(act_bytes / t_sp / 1e3, 1),
                  "GBps_dense_ffn": round(f * nmat * d * wb / t_de / 1e3, 1)}
            if spec.wtype in ("f16", "i4g128"):
                # both FFN paths at every batch size: per-row kernels and matrix cores
                for name, thr in (("rows", -1), ("mfma", 1)):
                    for _, ffn in layers:
                        ffn.mfma_min_batch = thr
                    pt[f"us_sparse_ffn_{name}"] = round(t_sparse(), 2)
                    pt[f"us_dense_ffn_{name}"] = round(t_dense(), 2)
                for _, ffn in layers:
                    ffn.mfma_min_batch = 0
            # last (they overwrite the masks, ids and counts past the switch):
            # the layer call with the dense switch at batch 16, and at the
            # threshold profiled from fire counts (union law + crossover)
            for key, th in (("us_layer_switch_at_16", [16] * nl), ("us_layer_auto_switch", auto_thr)):
                for (pred, _), t in zip(layers, th):
                    pred.dense_min_batch = t
                pt[key] = round(
                    timed(lambda: [sg.sfnn_layer(pred, ffn, x[l], B, y, masks[l], ids[l], cnt[l:l + 1], ws)
                                   for l, (pred, ffn) in enumerate(layers)]), 2)
            pt["auto_dense_min_batch"] = auto_thr
            for pred, _ in layers:
                pred.dense_min_batch = -1
            points.append(pt)
            print(json.dumps(points[-1]), file=sys.stderr, flush=True)
        del layers
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": spec.name, "distinct_layers": nl, "points": points}), flush=True)


def _isg_sweep(args):
    """Input-sparse GEMV (relufication stage 2) at OPT-6.7B shapes: the up
    projection (4096 -> 16384) and the fused QKV projection (4096 -> 12288),
    over input densities (1.0 = every input nonzero: every row read) and
    batches.  Each point cycles over distinct weight copies holding at least
    1 GB; HIP events around replays of one graph of calls over the copies."""
    import torch
    import synth
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import to_dev
    points = []
    only = args.only.split(",") if args.only else None
    for name, n_in, n_out in (("up 4096->16384", 4096, 16384), ("qkv 4096->12288", 4096, 12288)):
        if only and not name.startswith(only[0]):
            continue
        nc = max(2, int(np.ceil(1.0e9 / (n_in * n_out * 2))))
        ops = []
        for c in range(nc):
            w_t, b = synth.make_isg_weights(n_in, n_out, "f16", seed=0, key=c)
            ops.append(sg.Isg(to_dev(w_t), to_dev(b)))
        for B in ((int(only[1]),) if only else (1, 4, 16)):
            ws = torch.empty(sg.sfnn_isg_workspace_bytes(ops[0], B), dtype=torch.uint8, device="cuda")
            y = torch.empty((B, n_out), dtype=torch.float32, device="cuda")
            cols = torch.empty((nc, n_in), dtype=torch.int32, device="cuda")
            cnt = torch.zeros((nc,), dtype=torch.int32, device="cuda")
            for dens in ((float(only[2]),) if only else (1.0, 0.5, 0.3, 0.1)):
                xs = [to_dev(synth.make_relu_inputs(n_in, B, dens, seed=0, stream=700 + c)) for c in range(nc)]

                def calls():
                    for c in range(nc):
                        sg.sfnn_input_sparse_gemv(ops[c], xs[c], B, y, ws, cols[c], cnt[c:c + 1])

                calls()
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    calls()
                g.replay()
                torch.cuda.synchronize()
                a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 8
                a.record()
                for _ in range(reps):
                    g.replay()
                e.record()
                torch.cuda.synchronize()
                us = a.elapsed_time(e) / (reps * nc) * 1e3
                rows = float(cnt.float().mean().item())
                pt = {"shape": name, "batch": B, "input_density": dens, "rows_read_frac": round(rows / n_in, 4),
                      "us": round(us, 2), "GBps_rows_read": round(rows * n_out * 2 / us / 1e3, 1)}
                points.append(pt)
                print(json.dumps(pt), file=sys.stderr, flush=True)
        del ops
        torch.cuda.empty_cache()
    for pt in points:
        dense = next((q for q in points if q["shape"] == pt["shape"] and q["batch"] == pt["batch"]
                      and q["input_density"] == 1.0), None)
        if dense is not None:
            pt["speedup_vs_all_rows"] = round(dense["us"] / pt["us"], 2)
    print(json.dumps({"isg_sweep": points}), flush=True)


def _heads_sweep(args):
    """Head-gated attention projections: sfnn_head_qkv and sfnn_head_out at the
    OPT-6.7B (d 4096, 32 heads of 128) and OPT-175B (d 12288, 96 heads of 128)
    attention shapes, over the fraction of heads each token uses (1.0 = every
    head, the dense projections) and batches.  Each point cycles over distinct
    weight copies holding at least 1 GB; HIP events around replays of one graph
    of calls over the copies."""
    import torch
    import synth
    import activation_sparse_gemv_amd as sg
    from activation_sparse_gemv_amd.device import to_dev
    points = []
    only = args.only.split(",") if args.only else None
    for name, d, H, hd in (("opt6.7b", 4096, 32, 128), ("opt175b", 12288, 96, 128)):
        if only and name != only[0]:
            continue
        n = H * hd
        nc = max(2, int(np.ceil(1.0e9 / (4 * n * d * 2))))
        ops = []
        for c in range(nc):
            w_qkv, b_qkv, w_o_t, b_o = synth.make_head_weights(d, H, hd, "f16", seed=c)
            ops.append(sg.Heads(to_dev(w_qkv), to_dev(w_o_t), hd, to_dev(b_qkv), to_dev(b_o)))
        for B in ((int(only[1]),) if only else (1, 8)):
            ws = torch.empty(sg.sfnn_heads_workspace_bytes(ops[0], B), dtype=torch.uint8, device="cuda")
            qkv = torch.empty((B, 3 * n), dtype=torch.float32, device="cuda")
            y = torch.empty((B, d), dtype=torch.float32, device="cuda")
            x = to_dev(synth.make_relu_inputs(d, B, 1.0, seed=1, stream=B))
            attn = to_dev(synth.make_relu_inputs(n, B, 1.0, seed=2, stream=B))
            for dens in ((float(only[2]),) if only else (1.0, 0.5, 0.2)):
                masks = []
                used = []
                for c in range(nc):
                    bits, words = synth.make_head_masks(B, H, dens, seed=800 + c)
                    masks.append(to_dev(words))
                    used.append(float(bits.any(axis=0).mean()))

                def timed(fn):
                    fn()
                    torch.cuda.synchronize()
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        fn()
                    g.replay()
                    torch.cuda.synchronize()
                    a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    for _ in range(8):
                        g.replay()
                    e.record()
                    torch.cuda.synchronize()
                    return a.elapsed_time(e) / (8 * nc) * 1e3

                t_qkv = timed(lambda: [sg.sfnn_head_qkv(ops[c], x, B, masks[c], qkv) for c in range(nc)])
                t_out = timed(lambda: [sg.sfnn_head_out(ops[c], attn, B, masks[c], y, ws) for c in range(nc)])
                u = float(np.mean(used))
                pt = {"shape": name, "batch": B, "head_density": dens, "heads_read_frac": round(u, 4),
                      "us_qkv": round(t_qkv, 2), "us_out": round(t_out, 2),
                      "GBps_qkv_rows_read": round(u * 3 * n * d * 2 / t_qkv / 1e3, 1),
                      "GBps_out_rows_read": round(u * n * d * 2 / t_out / 1e3, 1)}
                points.append(pt)
                print(json.dumps(pt), file=sys.stderr, flush=True)
        del ops
        torch.cuda.empty_cache()
    for pt in points:
        dense = next((q for q in points if q["shape"] == pt["shape"] and q["batch"] == pt["batch"]
                      and q["head_density"] == 1.0), None)
        if dense is not None:
            pt["speedup_qkv_vs_all_heads"] = round(dense["us_qkv"] / pt["us_qkv"], 2)
            pt["speedup_out_vs_all_heads"] = round(dense["us_out"] / pt["us_out"], 2)
    print(json.dumps({"heads_sweep": points}), flush=True)


def _read_sizes(sg):
    """Single-launch read rate against size: the ceiling for a kernel that
    streams S bytes in one launch (launch ramp and drain included)."""
    import torch
    total = 3 << 30
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    rows = []
    for mb in (4, 8, 16, 24, 34, 40, 64, 128, 512):
        size, n = mb << 20, 32
        views = [buf[o:o + size] for o in (((k * (size + (1 << 20))) % (total - size)) & ~0xFFF for k in range(n))]
        for v in views[:2]:
            sg.sfnn_probe_read(v, size, sink)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for v in views:
                sg.sfnn_probe_read(v, size, sink)
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(4):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / (4 * n)
        rows.append({"MB": mb, "us_per_launch": round(us, 2), "GBps": round(size / us / 1e3, 1)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"read_sizes": rows}), flush=True)


def _hot_first(sg, layers, spec, B, dev, hot_arg="0"):
    """Offline profile: fire counts of seeded tokens give the hot-first
    relayout of each distinct layer; then, for hot_arg 'auto', a few stack
    steps on other seeded tokens give each neuron's fire rate in the batch's
    union on the decode path itself, which sets the layer's dense hot prefix.
    Returns the prefix per distinct layer (``layers`` is cycled through the
    stack)."""
    import torch
    import synth
    from activation_sparse_gemv_amd.device import to_dev, workspace
    f, d, L, nd = spec.d_ff, spec.d_model, spec.n_layers, len(layers)
    W = f // 64
    nprof = 256
    xs = to_dev(synth.make_tokens(spec, nprof, stream=99))
    for pred, ffn in layers:
        ws = workspace(pred, None, 8)
        m = torch.zeros((nprof, W), dtype=torch.uint64, device=dev)
        for i in range(0, nprof, 8):
            sg.sfnn_predict(pred, xs[i:i + 8], 8, m[i:i + 8], None, ws)
        counts = torch.zeros(f, dtype=torch.int32, device=dev)
        sg.sfnn_fire_counts(m, nprof, f, counts)
        ch = counts.cpu().numpy().view(np.uint32).copy()
        perm = np.empty(f, dtype=np.int32)
        sg.sfnn_hot_first_perm(ch, f, perm)
        pd = to_dev(perm)
        for t in [ffn.t[k] for k in ("w_up", "w_gate", "w_down_t", "s_up", "s_gate", "s_down_t", "b_up",
                                     "b_gate")] + [pred.w2_t, pred.tau]:
            if t is None:
                continue
            src = t.clone()
            rb = t.numel() * t.element_size() // f
            sg.sfnn_gather_rows(src, pd, f, rb, t)
        torch.cuda.synchronize()
    if hot_arg != "auto":
        for pred, _ in layers:
            pred.hot_prefix = int(hot_arg)
        return [int(hot_arg)] * nd
    steps = max(8, 256 // B)
    st = sg.Stack([layers[l % nd] for l in range(L)])
    xr = to_dev(synth.make_tokens(spec, steps * B, stream=98, dtype=np.float32)).view(steps, B, d)
    rout = torch.empty((B, d), dtype=torch.float32, device=dev)
    ws = workspace(layers[0][0], layers[0][1], B)
    mc = torch.zeros((L, B, W), dtype=torch.uint64, device=dev)
    hits = np.zeros((nd, f))
    for t in range(steps):
        sg.sfnn_stack_decode(st, B, xr[t], rout, 1e-6, ws, mask_cap=mc)
        uw = np.bitwise_or.reduce(mc.cpu().numpy(), axis=1)                       # [L][W]
        bits = np.unpackbits(uw.view(np.uint8), axis=1, bitorder="little")[:, :f]  # [L][f]
        for l in range(L):
            hits[l % nd] += bits[l]
    n = np.array([steps * len(range(k, L, nd)) for k in range(nd)], dtype=np.float64)
    hots = []
    for k, (pred, _) in enumerate(layers):
        pred.hot_prefix = _auto_hot_prefix(spec, hits[k] / n[k])
        hots.append(pred.hot_prefix)
    return hots


def _switch_thresholds(sg, counts, n_prof, spec):
    """dense_min_batch per layer from its fire counts ([layers][d_ff] int32 on
    the device) over n_prof[k] tokens: the smallest batch whose expected union
    share reaches the weight type's crossover, -1 if none up to 64 does."""
    ch = counts.cpu().numpy().view(np.uint32)
    return [sg.sfnn_dense_min_batch(np.ascontiguousarray(c), n, spec.d_ff, dense_crossover(spec), 64)
            for c, n in zip(ch, n_prof)]


def _thresholds_from_predictor(sg, layers, spec, dev, nprof=256):
    """Dense switch of single layers: fire counts of the predictor's masks on
    seeded fresh tokens (the layer calls' own workload)."""
    import torch
    import synth
    from activation_sparse_gemv_amd.device import to_dev, workspace
    f, W = spec.d_ff, spec.d_ff // 64
    xs = to_dev(synth.make_tokens(spec, nprof, stream=97))
    counts = torch.zeros((len(layers), f), dtype=torch.int32, device=dev)
    m = torch.zeros((nprof, W), dtype=torch.uint64, device=dev)
    for k, (pred, _) in enumerate(layers):
        ws = workspace(pred, None, 8)
        for i in range(0, nprof, 8):
            sg.sfnn_predict(pred, xs[i:i + 8], 8, m[i:i + 8], None, ws)
        sg.sfnn_fire_counts(m, nprof, f, counts[k])
    torch.cuda.synchronize()
    return _switch_thresholds(sg, counts, [nprof] * len(layers), spec)


def _auto_dense_switch(sg, distinct, spec, dev, flags, steps=64):
    """Dense switch of a stack's layers: fire counts of the masks each
    distinct layer's predictor makes on the decode path itself (a batch-1
    stack over seeded tokens, every layer sparse), then the union law.
    Sets each Pred's dense_min_batch; a Stack built afterwards carries it."""
    import torch
    import synth
    from activation_sparse_gemv_amd.device import to_dev, workspace
    f, d, L, nd = spec.d_ff, spec.d_model, spec.n_layers, len(distinct)
    W = f // 64
    st = sg.Stack([distinct[l % nd] for l in range(L)])
    xr = to_dev(synth.make_tokens(spec, steps, stream=96, dtype=np.float32)).view(steps, 1, d)
    rout = torch.empty((1, d), dtype=torch.float32, device=dev)
    ws = workspace(distinct[0][0], distinct[0][1], 1)
    mc = torch.zeros((steps, L, W), dtype=torch.uint64, device=dev)
    for t in range(steps):
        sg.sfnn_stack_decode(st, 1, xr[t], rout, 1e-6, ws, flags=flags, mask_cap=mc[t])
    counts = torch.zeros((nd, f), dtype=torch.int32, device=dev)
    n_prof = []
    for k in range(nd):
        mk = mc[:, k::nd].reshape(-1, W).contiguous()  # every position of distinct layer k, every step
        sg.sfnn_fire_counts(mk, mk.shape[0], f, counts[k])
        n_prof.append(mk.shape[0])
    torch.cuda.synchronize()
    thr = _switch_thresholds(sg, counts, n_prof, spec)
    for (pred, _), t in zip(distinct, thr):
        pred.dense_min_batch = t
    print(f"# dense switch per distinct layer (auto, crossover {dense_crossover(spec)}): {thr}",
          file=sys.stderr, flush=True)
    return thr


def _auto_hot_prefix(spec, urate):
    """Leading mask words (hot-first order) worth running as a dense block: a
    word joins while computing its 64 neurons for every token reads fewer bytes
    than predicting them, i.e. while sum(1 - u_i) FFN rows < 64 predictor rows,
    where u_i is the neuron's fire rate in the batch's union."""
    d, r = spec.d_model, spec.rank
    wb = {"f32": 4.0, "f16": 2.0, "i4g128": 0.5 + 2.0 / 128}[spec.wtype]
    ffn_row = spec.n_mat * d * wb
    pred_row = r * (4 if spec.pred_dtype == "f32" else 2) + 4
    w = 0
    while w < spec.d_ff // 64 and (1.0 - urate[64 * w:64 * w + 64]).sum() * ffn_row < 64 * pred_row:
        w += 1
    return 64 * w


def _row_sample(lay, k):
    """The first k neurons of a layer as a layer of their own (the dense FFN is a
    sum over neurons, so its time scales with the neuron count)."""
    import copy
    import dataclasses
    sub = copy.copy(lay)
    sub.spec = dataclasses.replace(lay.spec, d_ff=k)
    for name in ("w_up", "w_gate", "w_down_t", "q_up", "q_gate", "q_down_t", "s_up", "s_gate", "s_down_t",
                 "b_up", "b_gate", "w2_t", "tau", "probs"):
        v = getattr(lay, name, None)
        if v is not None:
            setattr(sub, name, v[:k])
    return sub


def _cpu_baseline(hosts, spec, B, L, budget_s):
    """The float64 oracle (as it stands) on a bounded sample of the same
    workload: predict + compact + masked FFN per (token, layer) over up to four
    sampled layers, the median extrapolated to the stack; and the dense FFN on
    a sample of neurons, extrapolated to d_ff.  BLAS threads = the cores this
    process may run on."""
    import oracle
    import synth
    import contextlib
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limit = contextlib.nullcontext()
    with limit:
        nmax = 256
        xs = synth.make_tokens(spec, nmax * B, stream=123)
        times, n, t_start = [], 0, time.perf_counter()
        while n < nmax and (time.perf_counter() - t_start < 0.6 * budget_s or n < 2):
            lay = hosts[n % len(hosts)]
            x = xs[n * B:(n + 1) * B]
            t = time.perf_counter()
            _, m = oracle.predict(lay.w1_t, lay.w2_t, lay.tau, x)
            oracle.compact(oracle.pack_mask(m), B, spec.d_ff)
            oracle.masked_ffn(lay, x, m)
            times.append(time.perf_counter() - t)
            n += 1
        per_layer = float(np.median(times))
        # dense FFN: time 64 neurons, then a sample sized to ~30% of the budget
        x = xs[:B]
        k = 64
        t = time.perf_counter()
        oracle.dense_ffn(_row_sample(hosts[0], k), x)
        t64 = time.perf_counter() - t
        k = int(min(spec.d_ff, max(64, (0.3 * budget_s / max(t64, 1e-6)) * 64)) // 64 * 64)
        t = time.perf_counter()
        oracle.dense_ffn(_row_sample(hosts[0], k), x)
        t_dense = (time.perf_counter() - t) * spec.d_ff / k
    layers_used = min(len(hosts), n)
    return {"value": round(B / (per_layer * L), 4), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n} (token batch, layer) samples over {layers_used} distinct layers of the same stack, "
                      f"batch {B}, float64 NumPy predict + compact + masked_ffn, median per layer "
                      f"{per_layer * 1e3:.1f} ms, tokens/s extrapolated x{L} layers; dense_ffn timed on the first "
                      f"{k} of {spec.d_ff} neurons of layer 0 and scaled to d_ff",
            "median_ms_per_layer": round(per_layer * 1e3, 2),
            "dense_ffn_ms_per_layer": round(t_dense * 1e3, 1),
            "dense_ffn_tokens_s": round(B / (t_dense * L), 5)}


if __name__ == "__main__":
    main()
