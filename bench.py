#!/usr/bin/env python3
"""Benchmark of the packed low-bit weight-only GEMV / verify GEMM on one MI355X.

A step is one decode pass of a 27B-class dense layer's linear set -- q, k, v, o
(5120x5120, 5120x1024 x2, 5120x5120), gate, up (5120x17408) and down
(17408x5120), K x N = in x out -- at M = 1 activation row, 3-bit codes with one
fp16 scale per 128 weights, fp16 activations.  All inputs are seeded and
synthetic and already resident in HBM.  The weights exist in R distinct copies
(>= 1 GiB in total, four times the 256 MB Infinity Cache) and consecutive steps
use consecutive copies, so every step streams its weights from HBM.  Steps are
replayed from a captured HIP graph (no host launch gaps between kernels).

Printed (one JSON line): effective weight GB/s of the step (value), per-shape
us/call at M = 1, 8, 16, 32 and the M=32 / M=1 ratio, the fused MLP with mixed
widths, the roofline entry of the dominant kernel (the M = 1 GEMV on the
5120x17408 gate/up shape) and the CPU oracle's rate on a bounded sample.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--copies", type=int, default=0, help="weight copies (default: enough for >= 1 GiB)")
    p.add_argument("--quick", action="store_true", help="skip the verify/MLP/CPU sections")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--only-layer", action="store_true", help="only the timed layer-set step (for profiling)")
    p.add_argument("--profile-gate", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the M=1 GEMV on the 5120x17408 shape over all "
                        "weight copies, then a 256 MiB device copy (the counter calibration), then exit")
    p.add_argument("--profile-rows", type=int, default=1, choices=(1, 8, 16, 32), metavar="M",
                   help="rows of the profiled gate/up product (1 = the GEMV, more = the verify GEMM)")
    p.add_argument("--profile-mlp", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the fused mixed-width MLP at --profile-rows rows "
                        "(1, 8 or 32) over weight copies of >= 1 GiB, then exit")
    p.add_argument("--profile-trellis", type=int, default=0, metavar="REPS",
                   help="profiling mode: REPS graph replays of the trellis product on the 5120x17408 shape at "
                        "--profile-rows rows (1 or 8) over weight copies of >= 1 GiB, then exit")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "bit_weight_only_packed_amd", "csrc")
    for f in sorted(os.listdir(d)):
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

    def layer_step(r, M=1):
        for i, sh in enumerate(shapes):
            lins[r][i].run(xk[(M, sh["K"])], out=ys[M][:, : sh["N"]] if sh["N"] == 17408 else
                           ys[M].view(-1)[: M * sh["N"]].view(M, sh["N"]))

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
        n = 64 << 20
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": f"{'gemv' if Mp == 1 else 'verify gemm'} M={Mp} 5120x17408",
                          "launches": args.profile_gate * R,
                          "graph_us_per_launch": round(us, 3), "copy_bytes_each_way": 4 * n,
                          "src_hash": src_hash()}), flush=True)
        return

    # ---------------- the timed step: layer set at M = 1 ----------------
    def all_copies(M=1):
        def f():
            for r in range(R):
                layer_step(r, M)
        return f

    g_layer = capture(all_copies(1))
    reps_w = max(1, args.warmup // R)
    reps_t = max(1, args.steps // R)
    time_graph(g_layer, reps_w)
    steps = reps_t * R
    t_s = time_graph(g_layer, reps_t)
    ms_per_step = t_s * 1e3 / steps
    value = per_copy / (t_s / steps) / 1e9
    log(f"layer set M=1: {ms_per_step * 1e3:.2f} us/step, {value:.0f} GB/s ({100 * value / HBM_PEAK_GBS:.1f} % of 8 TB/s)")
    result = {
        "metric": "effective weight GB/s & % HBM roofline; us/call at M=1 and M=8/32 verify",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": reps_w * R,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV, M=1, 27B-class layer set q,k,v,o,gate,up,down "
                               "(5120x5120 x2, 5120x1024 x2, 5120x17408 x2, 17408x5120), 3-bit codes, "
                               "fp16 scale per 128, fp16 x", "M": 1, "weight_bytes_per_step": per_copy,
                   "weight_copies": R, "pct_of_8TBs": round(100 * value / HBM_PEAK_GBS, 2)},
    }
    if args.only_layer:
        print(json.dumps(result), flush=True)
        return

    # ---------------- per shape, per M ----------------
    def shape_us(i, M, reps=20):
        sh = shapes[i]
        out = ys[M][:, : sh["N"]] if sh["N"] == 17408 else ys[M].view(-1)[: M * sh["N"]].view(M, sh["N"])

        def f():
            for r in range(R):
                lins[r][i].run(xk[(M, sh["K"])], out=out)
        g = capture(f)
        time_graph(g, 2)
        return time_graph(g, reps) / (reps * R) * 1e6

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
        per_shape[name] = row
        log(name, row)
    result["per_shape"] = per_shape

    layer_us = {}
    for M in (1, 8, 16, 32):
        g = capture(all_copies(M))
        time_graph(g, 1)
        layer_us[M] = time_graph(g, max(1, reps_t // 2)) / (max(1, reps_t // 2) * R) * 1e6
    result["layer_set_us"] = {f"M{M}": round(v, 3) for M, v in layer_us.items()}
    result["layer_set_ratio_M32_M1"] = round(layer_us[32] / layer_us[1], 3)
    result["layer_set_ratio_M8_M1"] = round(layer_us[8] / layer_us[1], 3)
    log("layer set us", result["layer_set_us"])

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
            g = capture(fstep)
            time_graph(g, 1)
            fused_us[M] = time_graph(g, max(1, reps_t // 2)) / (max(1, reps_t // 2) * R) * 1e6
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

    # ---------------- roofline entry: M=1 GEMV on the gate/up shape ----------------
    gate_us = per_shape["gateup"]["us_M1"]
    gate_bytes = per_shape["gateup"]["weight_bytes"]
    achieved = gate_bytes / gate_us / 1e3
    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_gemv_m1_gateup.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        if tj.get("src_hash") == src_hash():
            traffic = tj.get("bytes_per_launch")
    result["roofline"] = {"bound": "hbm", "kernel": "qg::k_gemv_q (M=1 GEMV, 5120x17408, 3-bit)",
                          "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                          "algorithmic_bytes_per_launch": gate_bytes, "avg_launch_us": gate_us,
                          "src_hash": src_hash()}

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

    # ---------------- CPU oracle on a bounded sample ----------------
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


def cpu_baseline():
    """The oracle (unpack, dequantise, fp64 matmul) on every 2nd output column of
    each layer-set matrix at M = 1; reported as weight GB/s of that sample."""
    import oracle as O
    import qg_synth as S
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    t_total, bytes_total = 0.0, 0
    for i, sh in enumerate(S.LAYER_SET):
        N, K = sh["N"], sh["K"]
        w = S.uniform_code_words(N, K, 3, cfg_id=S.CFG_DECODE, tensor_id=S.T_CODES + 10 * i)
        sc = S.scales(N, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_SCALE + 10 * i)
        x = S.activations(1, K, cfg_id=S.CFG_DECODE, tensor_id=S.T_X + 1)
        rows = np.arange(N)
        t0 = time.perf_counter()
        O.gemv_uniform_rows(x, w, sc, N, K, 3, rows)
        t_total += time.perf_counter() - t0
        bytes_total += len(rows) * (K * 3 // 8 + (K // 128) * 2)
    gbs = bytes_total / t_total / 1e9
    log(f"cpu oracle: {bytes_total} B in {t_total:.2f} s = {gbs:.3f} GB/s ({cores} threads)")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds": round(t_total, 2),
            "sample": "all output columns of q,k,v,o,gate,up,down at M=1 "
                      f"({bytes_total} weight bytes, one full layer set)"}


if __name__ == "__main__":
    main()
