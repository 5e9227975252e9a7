#!/usr/bin/env python3
"""Benchmark of the packed low-bit weight-only GEMV / verify GEMM on one MI355X.

A step is one decode pass of a 27B-class dense layer's linear set -- q, k, v, o
(5120x5120, 5120x1024 x2, 5120x5120), gate, up (5120x17408) and down
(17408x5120), K x N = in x out -- at M = 1 activation row, 3-bit codes with one
fp16 scale per 128 weights, fp16 activations, in decode order with the
siblings that read one input batched into one launch (qgemv_run_batch): q,k,v
| o | gate,up | down, four launches.  All inputs are seeded and synthetic and
already resident in HBM.  The weights
exist in R distinct copies (>= 1 GiB in total, four times the 256 MB Infinity
Cache) and consecutive steps use consecutive copies, so every step streams its
weights from HBM.  Steps are replayed from captured HIP graphs (no host launch
gaps between kernels): exactly --warmup untimed steps, then --trials timed
trials of exactly --steps steps each; the line reports the median trial.

Printed (one JSON line): effective weight GB/s of the step (value), per-shape
us/call at M = 1, 8, 16, 32 and the M=32 / M=1 ratio, each M = 1 call against
the measured streaming read of the same bytes, the fused MLP with mixed widths,
the trellis format, the roofline entry of the dominant kernel (the batched
M = 1 GEMV over the gate and up matrices, 2 x 5120x17408, one launch) and the
CPU oracle on bounded samples of every workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak of the MI355X


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--trials", type=int, default=5, help="timed trials of --steps steps each (median reported)")
    p.add_argument("--copies", type=int, default=0, help="weight copies (default: enough for >= 1 GiB)")
    p.add_argument("--quick", action="store_true", help="skip the verify/MLP/CPU sections")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only-layer", action="store_true", help="only the timed layer-set step (for profiling)")
    p.add_argument("--profile-gate", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the M=1 GEMV on the 5120x17408 shape over all "
                        "weight copies, then a 256 MiB device copy (the counter calibration), then exit")
    p.add_argument("--profile-gateup", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the step's dominant launch -- the M=1 GEMV over "
                        "the gate and up matrices batched into one launch -- over all weight copies, then a "
                        "256 MiB device copy (the counter calibration), then exit")
    p.add_argument("--profile-rows", type=int, default=1, choices=(1, 8, 16, 32), metavar="M",
                   help="rows of the profiled gate/up product (1 = the GEMV, more = the verify GEMM)")
    p.add_argument("--profile-mlp", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the fused mixed-width MLP at --profile-rows rows "
                        "(1, 8 or 32) over weight copies of >= 1 GiB, then exit")
    p.add_argument("--profile-prefill", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the prefill route (dequantise, then the fp16 "
                        "GEMM) on the 5120x17408 shape at --prefill-rows rows over all weight copies, then a "
                        "256 MiB device copy (the counter calibration), then exit")
    p.add_argument("--prefill-rows", type=int, default=256, choices=(256, 1024, 2048), metavar="M",
                   help="rows of the profiled prefill call")
    p.add_argument("--profile-trellis", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the trellis product on the 5120x17408 shape at "
                        "--profile-rows rows (1 or 8) over weight copies of >= 1 GiB, then exit")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# the sources the per-group M = 1 GEMV (the roofline entry's kernel) is built
# from, and the host code that plans its launch (quads per wave, waves, slices)
GEMV_SOURCES = ("k_m1q.hip", "qg_gemv.h", "qg_stage.h", "qg_decode.h", "qg_common.h", "qg_args.h", "qg_launch.h",
                "qgemv.hip")


def src_hash(files=None) -> str:
    """sha256 prefix over the library sources (all of them, or the named ones)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_weight_only_packed_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if not f.endswith((".h", ".hip")) or (files is not None and f not in files):
            continue
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def profile_other(args, torch, Q, S, dev, dw, df16, capture, time_graph):
    """Profiling modes for the fused MLP and the trellis product: one HIP graph
    over weight copies of at least 1 GiB (every launch reads its weights from
    HBM), replayed 2 + REPS times, then one JSON line."""
    M = args.profile_rows
    if args.profile_mlp:
        if M not in (1, 8, 32):
            sys.exit("--profile-mlp takes --profile-rows 1, 8 or 32")
        H, I = S.MLP["hidden"], S.MLP["inter"]
        cb_gu = S.column_bits(I, 0.2, 4, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK)
        cb_dn = S.column_bits(H, 0.2, 2, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK + 100)
        wg = S.mixed_code_words(cb_gu, H, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES)
        wu = S.mixed_code_words(cb_gu, H, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES + 10)
        wd = S.mixed_code_words(cb_dn, I, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES + 20)
        sg = S.scales(I, H, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE)
        su = S.scales(I, H, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE + 10)
        sd = S.scales(H, I, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE + 20)
        nbytes = wg.nbytes + wu.nbytes + wd.nbytes + sg.nbytes + su.nbytes + sd.nbytes
        R = int(np.ceil((1 << 30) / nbytes))
        dg, du, dd = (dw(wg), df16(sg)), (dw(wu), df16(su)), (dw(wd), df16(sd))
        mlps = [(Q.QLinear(dg[0], dg[1], H, I, col_bits=cb_gu, max_M=32),
                 Q.QLinear(du[0], du[1], H, I, col_bits=cb_gu, max_M=32),
                 Q.QLinear(dd[0], dd[1], I, H, col_bits=cb_dn, max_M=32)) for _ in range(R)]
        x = df16(S.activations(M, H, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + M))
        out = torch.empty((M, H), dtype=torch.float16, device=dev)

        def f():
            for (a, b, c) in mlps:
                Q.mlp(a, b, c, x, out=out)
        reps, what = args.profile_mlp, f"fused mlp M={M} 5120->17408->5120 mixed widths"
    else:
        if M not in (1, 8):
            sys.exit("--profile-trellis takes --profile-rows 1 or 8")
        K, N = 5120, 17408
        cbk = df16(S.codebook(cfg_id=S.CFG_TRELLIS))
        tw = S.trellis_words(N, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_TRELLIS + 40)
        ts = S.scales(N, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_SCALE + 40)
        nbytes = tw.nbytes + ts.nbytes
        R = int(np.ceil((1 << 30) / nbytes))
        dtw = torch.from_numpy(np.ascontiguousarray(tw).view(np.int16).copy()).to(dev)
        tl = [Q.QLinear(dtw, df16(ts), K, N, trellis=True, codebook=cbk, max_M=8) for _ in range(R)]
        x = df16(S.activations(M, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + M))
        out = torch.empty((M, N), dtype=torch.float16, device=dev)

        def f():
            for t in tl:
                t.run(x, out=out)
        reps, what = args.profile_trellis, f"trellis M={M} 5120x17408"
    torch.cuda.synchronize()
    g = capture(f)
    time_graph(g, 2)
    us = time_graph(g, reps) / (reps * R) * 1e6
    print(json.dumps({"profile": what, "launches": reps * R, "graph_us_per_launch": round(us, 3),
                      "weight_bytes": nbytes, "src_hash": src_hash()}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library runs on a single MI355X (--gpus {args.gpus} "
              f"was asked for; multi-GPU sharding is described in the design notes, not built).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_weight_only_packed_amd as Q
    import qg_synth as S

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dw(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32).copy()).to(dev)

    def df16(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16).copy()).to(dev)

    def capture(fn, reps=1):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(2):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        return g

    def time_graph(g, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3  # s

    if args.profile_mlp or args.profile_trellis:
        profile_other(args, torch, Q, S, dev, dw, df16, capture, time_graph)
        return

    # ---------------- weights: layer set, R copies ----------------
    shapes = S.LAYER_SET
    per_copy = 0
    canon = []
    for i, sh in enumerate(shapes):
        w = S.uniform_code_words(sh["N"], sh["K"], 3, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 10 * i)
        sc = S.scales(sh["N"], sh["K"], cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 10 * i)
        canon.append((dw(w), df16(sc)))
        per_copy += w.nbytes + sc.nbytes
    R = args.copies or int(np.ceil((1 << 30) / per_copy))
    log(f"layer set: {per_copy} weight bytes per copy, {R} copies")
    lins = []
    for r in range(R):
        row = []
        for i, sh in enumerate(shapes):
            row.append(Q.QLinear(canon[i][0], canon[i][1], sh["K"], sh["N"], bits=3, max_M=32))
        lins.append(row)
    del canon
    torch.cuda.synchronize()
    xs = {M: df16(S.activations(M, 17408, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + M)) for M in (1, 8, 16, 32)}
    ys = {M: torch.empty((M, 17408), dtype=torch.float16, device=dev) for M in (1, 8, 16, 32)}

    def xin(M, K):
        return xs[M][:, :K] if K == 17408 else xs[M].view(-1)[: M * K].view(M, K)

    # distinct x rows per K (contiguous [M][K] views)
    xk = {(M, K): xin(M, K).contiguous() for M in (1, 8, 16, 32) for K in (5120, 17408)}

    def layer_step_each(r, M=1):
        """the layer set, one launch per matrix"""
        for i, sh in enumerate(shapes):
            lins[r][i].run(xk[(M, sh["K"])], out=ys[M][:, : sh["N"]] if sh["N"] == 17408 else
                           ys[M].view(-1)[: M * sh["N"]].view(M, sh["N"]))

    # M = 1 outputs of the batched launches, one tensor per matrix
    yb = [torch.empty((1, sh["N"]), dtype=torch.float16, device=dev) for sh in shapes]

    def batch_siblings(r):
        """decode order, siblings that read one x batched: q,k,v | o | gate,up | down"""
        L, x5, x17 = lins[r], xk[(1, 5120)], xk[(1, 17408)]
        Q.run_batch([L[0], L[1], L[2]], [x5, x5, x5], yb[0:3])
        L[3].run(x5, out=yb[3])
        Q.run_batch([L[4], L[5]], [x5, x5], yb[4:6])
        L[6].run(x17, out=yb[6])

    def batch_gateup(r):
        L, x5 = lins[r], xk[(1, 5120)]
        Q.run_batch([L[4], L[5]], [x5, x5], yb[4:6])

    def layer_step(r, M=1):
        """the timed step: at M = 1 the batched decode order, else one launch per matrix"""
        if M == 1:
            batch_siblings(r)
        else:
            layer_step_each(r, M)

    def calibration_copies():
        n = 64 << 20
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        return 4 * n

    if args.profile_gateup:
        # the step's dominant launch alone, launched exactly as the timed step
        # launches it, then plain copies of known size for the HBM counter scale
        def gateup_all():
            for r in range(R):
                batch_gateup(r)
        g = capture(gateup_all)
        time_graph(g, 2)
        t = time_graph(g, args.profile_gateup)
        us = t / (args.profile_gateup * R) * 1e6
        cb = calibration_copies()
        print(json.dumps({"profile": "gemv batch M=1 gate,up 2 x 5120x17408 (one launch)",
                          "launches": args.profile_gateup * R, "graph_us_per_launch": round(us, 3),
                          "copy_bytes_each_way": cb, "src_hash": src_hash(),
                          "gemv_src_hash": src_hash(GEMV_SOURCES)}), flush=True)
        return

    if args.profile_gate:
        # the dominant kernel alone, launched exactly as the per-shape timing below
        # launches it, then a plain copy of known size for the HBM counter scale
        Mp = args.profile_rows
        out1 = ys[Mp][:, : shapes[4]["N"]]

        def gate_all():
            for r in range(R):
                lins[r][4].run(xk[(Mp, 5120)], out=out1)
        g = capture(gate_all)
        time_graph(g, 2)
        t = time_graph(g, args.profile_gate)
        us = t / (args.profile_gate * R) * 1e6
        cb = calibration_copies()
        print(json.dumps({"profile": f"{'gemv' if Mp == 1 else 'verify gemm'} M={Mp} 5120x17408",
                          "launches": args.profile_gate * R,
                          "graph_us_per_launch": round(us, 3), "copy_bytes_each_way": cb,
                          "src_hash": src_hash(), "gemv_src_hash": src_hash(GEMV_SOURCES)}), flush=True)
        return

    if args.profile_prefill:
        # the prefill route alone, launched as the prefill timing below launches it
        Mp = args.prefill_rows
        wsb = torch.empty(lins[0][4].prefill_workspace()[1], dtype=torch.uint8, device=dev)
        xp = df16(S.activations(Mp, 5120, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + 1000 + Mp))
        yp = torch.empty((Mp, shapes[4]["N"]), dtype=torch.float16, device=dev)

        def prefill_all():
            for r in range(R):
                lins[r][4].run_prefill(xp, out=yp, workspace=wsb)
        g = capture(prefill_all)
        time_graph(g, 2)
        t = time_graph(g, args.profile_prefill)
        us = t / (args.profile_prefill * R) * 1e6
        cb = calibration_copies()
        print(json.dumps({"profile": f"prefill route M={Mp} 5120x17408 (dequantise + fp16 GEMM)",
                          "calls": args.profile_prefill * R, "graph_us_per_call": round(us, 3),
                          "copy_bytes_each_way": cb, "src_hash": src_hash()}), flush=True)
        return

    # ---------------- the timed step: layer set at M = 1 ----------------
    def steps_graph(n, M=1, step=None):
        """One graph of n consecutive steps, on weight copies 0 .. n-1."""
        step = step or layer_step

        def f():
            for r in range(n):
                step(r, M)
        return capture(f)

    def run_steps(n, g_full, g_rem):
        for _ in range(n // R):
            g_full.replay()
        if g_rem is not None:
            g_rem.replay()

    K_steps, W_steps = max(1, args.steps), max(0, args.warmup)
    g_layer = steps_graph(R)
    g_krem = steps_graph(K_steps % R) if K_steps % R else None
    g_wrem = steps_graph(W_steps % R) if W_steps % R else None
    torch.cuda.synchronize()
    run_steps(W_steps, g_layer, g_wrem)
    trial_s = []
    for _ in range(max(1, args.trials)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        run_steps(K_steps, g_layer, g_krem)
        e1.record()
        torch.cuda.synchronize()
        trial_s.append(e0.elapsed_time(e1) / 1e3)
    t_s = float(np.median(trial_s))
    ms_per_step = t_s * 1e3 / K_steps
    value = per_copy / (t_s / K_steps) / 1e9
    log(f"layer set M=1: {ms_per_step * 1e3:.2f} us/step, {value:.0f} GB/s ({100 * value / HBM_PEAK_GBS:.1f} % of 8 TB/s); "
        f"trials {[round(t * 1e6 / K_steps, 2) for t in trial_s]} us/step")
    result = {
        "metric": "effective weight GB/s & % HBM roofline; us/call at M=1 and M=8/32 verify",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV, M=1, 27B-class layer set q,k,v,o,gate,up,down "
                               "(5120x5120 x2, 5120x1024 x2, 5120x17408 x2, 17408x5120), 3-bit codes, "
                               "fp16 scale per 128, fp16 x, decode order with siblings batched "
                               "(q,k,v | o | gate,up | down: 4 launches)", "M": 1,
                   "weight_bytes_per_step": per_copy, "weight_copies": R,
                   "pct_of_8TBs": round(100 * value / HBM_PEAK_GBS, 2)},
        "trials": {"n": len(trial_s), "us_per_step": [round(t * 1e6 / K_steps, 3) for t in trial_s]},
    }
    if args.only_layer:
        print(json.dumps(result), flush=True)
        return

    # ---------------- per shape, per M ----------------
    def graph_us(g, launches, reps=20, trials=5):
        """us per launch: median over trials of `reps` replays of graph g."""
        time_graph(g, 2)
        return float(np.median([time_graph(g, reps) / (reps * launches) * 1e6 for _ in range(trials)]))

    def shape_us(i, M, reps=20):
        sh = shapes[i]
        out = ys[M][:, : sh["N"]] if sh["N"] == 17408 else ys[M].view(-1)[: M * sh["N"]].view(M, sh["N"])

        def f():
            for r in range(R):
                lins[r][i].run(xk[(M, sh["K"])], out=out)
        return graph_us(capture(f), R, reps)

    def stream_us(nbytes, reps=20):
        """The measured read roofline: a plain streaming read of nbytes (buffer
        copies of >= 1 GiB in rotation, like the weights), us per launch."""
        nb = (nbytes + 15) // 16 * 16
        Rs = int(np.ceil((1 << 30) / nb))
        bufs = [torch.empty(nb // 4, dtype=torch.int32, device=dev) for _ in range(Rs)]

        def f():
            for b in bufs:
                Q.stream_read(b)
        us = graph_us(capture(f), Rs, reps)
        del bufs
        return us

    distinct = {"qo": 0, "kv": 1, "gateup": 4, "down": 6}
    per_shape = {}
    for name, i in distinct.items():
        sh = shapes[i]
        wb = lins[0][i].weight_bytes()
        row = {"K": sh["K"], "N": sh["N"], "weight_bytes": wb}
        for M in (1, 8, 16, 32):
            us = shape_us(i, M)
            row[f"us_M{M}"] = round(us, 3)
            if M == 1:
                row["GBs_M1"] = round(wb / us / 1e3, 1)
                row["pct_8TBs_M1"] = round(100 * wb / us / 1e3 / HBM_PEAK_GBS, 1)
        row["ratio_M32_M1"] = round(row["us_M32"] / row["us_M1"], 3)
        row["ratio_M8_M1"] = round(row["us_M8"] / row["us_M1"], 3)
        st = stream_us(wb)
        row["stream_read_us"] = round(st, 3)
        row["pct_of_stream_read_M1"] = round(100 * st / row["us_M1"], 1)
        per_shape[name] = row
        log(name, row)
    result["per_shape"] = per_shape
    ls_stream = stream_us(per_copy)
    result["stream_read_layer_set_us"] = round(ls_stream, 3)
    result["pct_of_stream_read"] = round(100 * ls_stream * R / (t_s * 1e6 / K_steps * R), 1)

    # the layer set with one launch per matrix at every row count (the verify
    # steps; at M = 1 beside the batched step above)
    layer_us = {}
    for M in (1, 8, 16, 32):
        layer_us[M] = graph_us(steps_graph(R, M, layer_step_each), R, reps=3)
    result["layer_set_each_us"] = {f"M{M}": round(v, 3) for M, v in layer_us.items()}
    result["layer_set_each_ratio_M32_M1"] = round(layer_us[32] / layer_us[1], 3)
    result["layer_set_each_ratio_M8_M1"] = round(layer_us[8] / layer_us[1], 3)
    result["layer_set_ratio_M32_vs_batched_M1"] = round(layer_us[32] / (t_s * 1e6 / K_steps), 3)
    log("layer set, one launch per matrix, us", result["layer_set_each_us"])

    # ---------------- the layer set in one qgemv_run_batch launch ----------------
    # all seven products in one launch (independent inputs): the floor of the
    # batched launch path, beside the 4-launch decode order of the timed step
    def batch_all(r):
        Q.run_batch(lins[r], [xk[(1, sh["K"])] for sh in shapes], yb)

    def f_all():
        for r in range(R):
            batch_all(r)
    us = graph_us(capture(f_all), R, reps=5)
    result["layer_set_one_launch"] = {"us_M1": round(us, 3), "GBs_M1": round(per_copy / us / 1e3, 1),
                                      "pct_8TBs_M1": round(100 * per_copy / us / 1e3 / HBM_PEAK_GBS, 2),
                                      "pct_of_stream_read": round(100 * ls_stream / us, 1), "launches": 1}
    log("layer_set_one_launch", result["layer_set_one_launch"])

    # ---------------- the same layer set with sibling projections fused ----------------
    # q|k|v and gate|up read the same input: each pair of siblings runs as one
    # launch over its rows stacked (N = 7168 and 34816) -- the same weights, bytes
    # and outputs in 4 launches instead of 7
    if not args.quick:
        groups = [(0, 1, 2), (3,), (4, 5), (6,)]
        cw = [(S.uniform_code_words(sh["N"], sh["K"], 3, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 10 * i),
               S.scales(sh["N"], sh["K"], cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 10 * i))
              for i, sh in enumerate(shapes)]
        fmats = []
        for grp in groups:
            w = np.concatenate([cw[i][0].reshape(shapes[i]["N"], -1) for i in grp], axis=0)
            sc = np.concatenate([cw[i][1] for i in grp], axis=0)
            fmats.append((dw(w), df16(sc), sum(shapes[i]["N"] for i in grp), shapes[grp[0]]["K"]))
        del cw
        flins = [[Q.QLinear(w, sc, K, N, bits=3, max_M=32) for (w, sc, N, K) in fmats] for _ in range(R)]
        del fmats
        fys = {M: [torch.empty((M, N), dtype=torch.float16, device=dev) for N in (7168, 5120, 34816, 5120)]
               for M in (1, 8, 16, 32)}
        fks = (5120, 5120, 5120, 17408)
        fused_us = {}
        for M in (1, 8, 16, 32):
            def fstep(M=M):
                for r in range(R):
                    for j in range(4):
                        flins[r][j].run(xk[(M, fks[j])], out=fys[M][j])
            fused_us[M] = graph_us(capture(fstep), R, reps=3)
        result["layer_set_fused"] = {
            "launches": 4, "note": "q|k|v and gate|up as one launch each over stacked rows",
            **{f"us_M{M}": round(v, 3) for M, v in fused_us.items()},
            "GBs_M1": round(per_copy / fused_us[1] / 1e3, 1),
            "pct_8TBs_M1": round(100 * per_copy / fused_us[1] / 1e3 / HBM_PEAK_GBS, 2),
            "ratio_M32_M1": round(fused_us[32] / fused_us[1], 3)}
        log("fused layer set", result["layer_set_fused"])
        for row in flins:
            for l in row:
                l.close()
        del flins

    # ---------------- roofline entry: the step's dominant launch ----------------
    # the batched M = 1 GEMV over gate and up (one launch, 2 x 5120x17408),
    # timed live like the step: a graph of its launches over every weight copy
    def f_gu():
        for r in range(R):
            batch_gateup(r)
    gu_us = graph_us(capture(f_gu), R, reps=20)
    gu_bytes = lins[0][4].weight_bytes() + lins[0][5].weight_bytes()
    achieved = gu_bytes / gu_us / 1e3
    gu_stream = stream_us(gu_bytes)
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_gemv_batch_gateup.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        if tj.get("gemv_src_hash") == src_hash(GEMV_SOURCES):
            traffic = tj.get("bytes_per_launch")
    result["roofline"] = {"bound": "hbm",
                          "kernel": "qg::k_gemv_batch<3, 3> (M=1 GEMV, gate and up 2 x 5120x17408 in one launch, 3-bit, 3 quads per wave)",
                          "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                          "algorithmic_bytes_per_launch": gu_bytes, "avg_launch_us": round(gu_us, 3),
                          "stream_read_us": round(gu_stream, 3),
                          "pct_of_stream_read": round(100 * gu_stream / gu_us, 1),
                          "src_hash": src_hash(), "gemv_src_hash": src_hash(GEMV_SOURCES)}
    log("roofline", result["roofline"])

    # ---------------- fused MLP, mixed widths ----------------
    if not args.quick:
        H, I = S.MLP["hidden"], S.MLP["inter"]
        cb_gu = S.column_bits(I, 0.2, 4, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK)
        cb_dn = S.column_bits(H, 0.2, 2, cfg_id=S.CFG_MLP, tensor_id=S.T_MASK + 100)
        wg = S.mixed_code_words(cb_gu, H, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES)
        wu = S.mixed_code_words(cb_gu, H, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES + 10)
        wd = S.mixed_code_words(cb_dn, I, cfg_id=S.CFG_MLP, tensor_id=S.T_CODES + 20)
        sg = S.scales(I, H, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE)
        su = S.scales(I, H, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE + 10)
        sd = S.scales(H, I, cfg_id=S.CFG_MLP, tensor_id=S.T_SCALE + 20)
        mlp_bytes = wg.nbytes + wu.nbytes + wd.nbytes + sg.nbytes + su.nbytes + sd.nbytes
        Rm = int(np.ceil((1 << 30) / mlp_bytes))
        dg, du, dd = (dw(wg), df16(sg)), (dw(wu), df16(su)), (dw(wd), df16(sd))
        mlps = [(Q.QLinear(dg[0], dg[1], H, I, col_bits=cb_gu, max_M=32),
                 Q.QLinear(du[0], du[1], H, I, col_bits=cb_gu, max_M=32),
                 Q.QLinear(dd[0], dd[1], I, H, col_bits=cb_dn, max_M=32)) for _ in range(Rm)]
        del dg, du, dd
        mres = {"weight_bytes": mlp_bytes, "bpw": round(mlp_bytes * 8 / (3 * H * I), 4), "copies": Rm}
        outm = {M: torch.empty((M, H), dtype=torch.float16, device=dev) for M in (1, 8, 32)}
        for M in (1, 8, 32):
            xm = xk[(M, 5120)]

            def f():
                for (a, b, c) in mlps:
                    Q.mlp(a, b, c, xm, out=outm[M])
            g = capture(f)
            time_graph(g, 2)
            us = time_graph(g, 20) / (20 * Rm) * 1e6
            mres[f"us_M{M}"] = round(us, 3)
            mres[f"GBs_M{M}"] = round(mlp_bytes / us / 1e3, 1)
        mres["ratio_M32_M1"] = round(mres["us_M32"] / mres["us_M1"], 3)
        result["mlp"] = mres
        log("mlp", mres)
        del mlps

    # ---------------- trellis-coded weights (27B-class shapes, M = 1 and 8) ----------------
    if not args.quick:
        cbk = df16(S.codebook(cfg_id=S.CFG_TRELLIS))
        tres = {}
        for name, i in distinct.items():
            sh = shapes[i]
            N, K = sh["N"], sh["K"]
            tw = S.trellis_words(N, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_TRELLIS + 10 * i)
            ts = S.scales(N, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_SCALE + 10 * i)
            dtw = torch.from_numpy(np.ascontiguousarray(tw).view(np.int16).copy()).to(dev)
            dts = df16(ts)
            wbt = tw.nbytes + ts.nbytes
            Rt = int(np.ceil((1 << 30) / wbt))
            tl = [Q.QLinear(dtw, dts, K, N, trellis=True, codebook=cbk, max_M=8) for _ in range(Rt)]
            del dtw
            row = {"K": K, "N": N, "weight_bytes": wbt, "codebook_bytes": 131072, "copies": Rt}
            for M in (1, 8):
                xt = xk[(M, K)]
                out = ys[M][:, :N] if N == 17408 else ys[M].view(-1)[: M * N].view(M, N)

                def f():
                    for t in tl:
                        t.run(xt, out=out)
                g = capture(f)
                time_graph(g, 2)
                us = time_graph(g, 10) / (10 * Rt) * 1e6
                row[f"us_M{M}"] = round(us, 3)
                row[f"GBs_M{M}"] = round(wbt / us / 1e3, 1)
            row["ratio_M8_M1"] = round(row["us_M8"] / row["us_M1"], 3)
            tres[name] = row
            log("trellis", name, row)
            for t in tl:
                t.close()
            del tl
        result["trellis"] = tres

    # ---------------- W4A16 at scale groups 128, 64 and 32 (gate/up shape) ----------------
    if not args.quick:
        N, K = shapes[4]["N"], shapes[4]["K"]
        w4 = S.uniform_code_words(N, K, 4, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 500)
        fres = {}
        for gs in (128, 64, 32):
            sc = S.scales(N, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 500 + gs, group=gs)
            wb = w4.nbytes + sc.nbytes
            Rf = int(np.ceil((1 << 30) / wb))
            dwf, dsf = dw(w4), df16(sc)
            fl = [Q.QLinear(dwf, dsf, K, N, bits=4, max_M=32, group_size=gs) for _ in range(Rf)]
            row = {"weight_bytes": wb, "copies": Rf}
            for M in (1, 8, 32):
                xf = xk[(M, K)]
                out = ys[M][:, :N]

                def f(fl=fl, xf=xf, out=out):
                    for l in fl:
                        l.run(xf, out=out)
                us = graph_us(capture(f), Rf, reps=10, trials=3)
                row[f"us_M{M}"] = round(us, 3)
                row[f"GBs_M{M}"] = round(wb / us / 1e3, 1)
            row["ratio_M32_M1"] = round(row["us_M32"] / row["us_M1"], 3)
            fres[f"g{gs}"] = row
            log("w4a16", gs, row)
            for l in fl:
                l.close()
            del fl, dwf, dsf
        # MXFP4 (E2M1 elements) and MXFP6 (E3M2 elements), one UE8M0 byte per 32, on the same shape
        e8 = S.mx_scales(N, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 600)
        w6 = S.uniform_code_words(N, K, 6, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 600)
        for name, wmx in (("mxfp4", w4), ("mxfp6", w6)):
            wb = wmx.nbytes + e8.nbytes
            Rf = int(np.ceil((1 << 30) / wb))
            dwf, def8 = dw(wmx), torch.from_numpy(e8.copy()).to(dev)
            fl = [Q.QLinear(dwf, def8, K, N, max_M=32, **{name: True}) for _ in range(Rf)]
            row = {"weight_bytes": wb, "copies": Rf}
            for M in (1, 8, 32):
                xf = xk[(M, K)]
                out = ys[M][:, :N]

                def f(fl=fl, xf=xf, out=out):
                    for l in fl:
                        l.run(xf, out=out)
                us = graph_us(capture(f), Rf, reps=10, trials=3)
                row[f"us_M{M}"] = round(us, 3)
                row[f"GBs_M{M}"] = round(wb / us / 1e3, 1)
            row["ratio_M32_M1"] = round(row["us_M32"] / row["us_M1"], 3)
            fres[name] = row
            log(name, row)
            for l in fl:
                l.close()
            del fl, dwf, def8
        result["w4a16_gateup"] = fres

    # ---------------- prefill route: dequantise to fp16, then a plain fp16 GEMM ----------------
    # gate/up shape; each call reads its codes from HBM (weight copies in
    # rotation); beside it the fp16 GEMM alone on the weights the last call
    # dequantised (what the route costs over a dense fp16 model)
    if not args.quick:
        ig = 4
        N, K = shapes[ig]["N"], shapes[ig]["K"]
        full = lins[0][ig].prefill_workspace()[1]
        wsb = torch.empty(full, dtype=torch.uint8, device=dev)
        wf = wsb[32 << 20:(32 << 20) + N * K * 2].view(torch.float16).view(N, K)
        pres = {"K": K, "N": N, "weight_bytes": lins[0][ig].weight_bytes(), "copies": R}
        for M in (64, 192, 256, 1024, 2048):
            xp = df16(S.activations(M, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + 1000 + M))
            yp = torch.empty((M, N), dtype=torch.float16, device=dev)

            def f(xp=xp, yp=yp):
                for r in range(R):
                    lins[r][ig].run_prefill(xp, out=yp, workspace=wsb)
            us = graph_us(capture(f), R, reps=3, trials=3)

            def fg(xp=xp, yp=yp):
                torch.mm(xp, wf.t(), out=yp)
            gus = graph_us(capture(fg), 1, reps=10, trials=3)
            tf = 2.0 * M * N * K / us / 1e6
            pres[f"M{M}"] = {"us": round(us, 3), "TFLOPs": round(tf, 1),
                             "pct_fp16_mfma_peak": round(100 * tf / MFMA_F16_PEAK_TFLOPS, 1),
                             "fp16_gemm_alone_us": round(gus, 3), "route_over_gemm": round(us / gus, 3)}
            log("prefill", M, pres[f"M{M}"])
        result["prefill_gateup"] = pres
        del wsb, wf

    # ---------------- CPU oracle on a bounded sample ----------------
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


def cpu_baseline():
    """The oracle (unpack, dequantise, fp64 matmul) timed on the host cores on a
    bounded sample of every workload: for each matrix shape a sample of output
    columns (the per-column work is the same for every column), the rest
    scaled by the column count; reported per workload and row count as us/call
    and weight GB/s, with the dequantisation and matmul phases apart, at the
    BLAS thread count of this process and at one thread."""
    import oracle as O
    import qg_synth as S
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threadpool_limits, cores = None, os.cpu_count()

    def timed(f):
        t0 = time.perf_counter()
        out = f()
        return out, time.perf_counter() - t0

    def uniform_case(N, K, Ms, ncols, bits=3, cfg=S.CFG_DECODE, tid=0):
        """us/call per M: dequant of the sampled columns, matmul of each M, scaled to N columns."""
        G = K // 128
        cols = np.arange(min(ncols, N))
        w = S.code_words(len(cols) * K * bits // 32, cfg_id=cfg, tensor_id=S.T_CODES + 10 * tid)
        sc = S.scales(len(cols), K, cfg_id=cfg, tensor_id=S.T_SCALE + 10 * tid)
        wd, t_dq = timed(lambda: O.dequant_uniform(O.unpack_uniform(w, len(cols), K, bits), sc, bits))
        scale = N / len(cols)
        res = {}
        for M in Ms:
            x = S.activations(M, K, cfg_id=cfg, tensor_id=S.T_X + M)
            _, t_mm = timed(lambda: O.matmul(x, wd))
            res[M] = (t_dq * scale * 1e6, t_mm * scale * 1e6)
        return res, (N * K * bits // 8 + N * G * 2)

    def trellis_case(N, K, Ms, nrows):
        nb = max(1, min(nrows, N) // 16)
        tw = S.trellis_words(16 * nb, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_TRELLIS)
        ts = S.scales(16 * nb, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_SCALE)
        cb = S.codebook(cfg_id=S.CFG_TRELLIS)
        wd, t_dq = timed(lambda: O.trellis_dequant(O.trellis_states(tw, 16 * nb, K), cb, ts))
        scale = N / (16 * nb)
        res = {}
        for M in Ms:
            x = S.activations(M, K, cfg_id=S.CFG_TRELLIS, tensor_id=S.T_X + M)
            _, t_mm = timed(lambda: O.matmul(O.rotate(x), wd))
            res[M] = (t_dq * scale * 1e6, t_mm * scale * 1e6)
        return res, (N * K * 3 // 8 + N * (K // 128) * 2)

    def fmt(res, nbytes):
        out = {}
        for M, (dq, mm) in res.items():
            out[f"M{M}"] = {"us": round(dq + mm, 1), "dequant_us": round(dq, 1), "matmul_us": round(mm, 1),
                            "weight_GBs": round(nbytes / (dq + mm) / 1e3, 4)}
        return out

    t_start = time.perf_counter()
    report = {}
    # tiny reference (all of it)
    r, nb = uniform_case(512, 512, (1,), 512, cfg=S.CFG_TINY)
    report["tiny_512x512"] = fmt(r, nb)
    # decode and verify: the four distinct layer shapes, 8192 sampled columns each
    ls_us = {M: 0.0 for M in (1, 8, 16, 32)}
    ls_bytes = 0
    for name, (K, N, mult) in {"qo": (5120, 5120, 2), "kv": (5120, 1024, 2), "gateup": (5120, 17408, 2),
                               "down": (17408, 5120, 1)}.items():
        r, nb = uniform_case(N, K, (1, 8, 16, 32), 8192)
        report[name] = fmt(r, nb)
        ls_bytes += mult * nb
        for M, (dq, mm) in r.items():
            ls_us[M] += mult * (dq + mm)
    report["layer_set"] = {f"M{M}": {"us": round(v, 1), "weight_GBs": round(ls_bytes / v / 1e3, 4)}
                           for M, v in ls_us.items()}
    # fused MLP (mixed widths counted at 3 bits: the oracle's work per weight is the same)
    gu, nbg = uniform_case(17408, 5120, (1, 8, 32), 4096, tid=1)
    dn, nbd = uniform_case(5120, 17408, (1, 8, 32), 4096, tid=2)
    report["mlp"] = {f"M{M}": {"us": round(2 * sum(gu[M]) + sum(dn[M]), 1)} for M in (1, 8, 32)}
    # trellis, gate/up shape
    r, nb = trellis_case(17408, 5120, (1, 8), 2048)
    report["trellis_gateup"] = fmt(r, nb)
    t_all = time.perf_counter() - t_start
    # one thread: the layer set at M = 1
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            us1 = 0.0
            for name, (K, N, mult) in {"qo": (5120, 5120, 2), "kv": (5120, 1024, 2), "gateup": (5120, 17408, 2),
                                       "down": (17408, 5120, 1)}.items():
                r, nb = uniform_case(N, K, (1,), 2048)
                us1 += mult * sum(r[1])
        one = {"us": round(us1, 1), "weight_GBs": round(ls_bytes / us1 / 1e3, 4)}
    v = ls_bytes / ls_us[1] / 1e3
    log(f"cpu oracle: layer set M=1 {ls_us[1]:.0f} us = {v:.3f} GB/s ({cores} threads), 1 thread "
        f"{one}; sampled in {t_all:.1f} s")
    return {"value": round(v, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "the first 8192 output columns of each distinct 27B-class layer shape (all 5120 or 1024 "
                      "where it has fewer; 2048 at one thread, 4096 for the MLP, 2048 rows of the trellis shape), scaled to whole matrices; the value is the "
                      "layer set q,k,v,o,gate,up,down at M=1",
            "seconds": round(t_all, 1), "one_thread_layer_set_M1": one, "per_workload": report}


if __name__ == "__main__":
    main()
