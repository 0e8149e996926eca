#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one verify round over the whole batch, through every kernel of the
hot path, on inputs already in HBM:
  sv_softmax_warp(target logits) + sv_softmax_warp(draft logits)
  + sv_accept(p, q, tokens, uniforms) + sv_verify_greedy(target logits)
(probability workloads: the two verifies). Default workload: B = 512
sequences, K = 16 draft tokens, V = 256000, bf16 logits (target ~ N(0, 5^2)
with a Zipf(1.1) rank bias, draft = target + N(0, 1)), seeded synthetic data.

Every mode is timed twice with HIP events on the stream the kernels run on:
"hbm", cycling through n >= 4 copies of the inputs of more than 1 GiB
together, so that no call finds its inputs in the L2 caches or the MALL; and
"resident", calling on one copy over and over. ``value`` is the whole step's
hbm rounds/s. ``modes`` gives rounds/s per mode (greedy round, sampled round
through the warps, sampled round fused from logits -- also with the draft
rows' normalisers given -- the filtered warps and the penalty stage), each
with its bytes needed (what the method must move) and,
when rocprofv3 counters of these sources are on file, its bytes read, both as
GB/s and as fractions of MI355X's 8 TB/s; the greedy round is also timed at
look-ahead depths L = 1, 2 and K + 1 (rows read ahead of the decision), with
the bytes those depths load. ``roofline`` is the dominant
kernel (the warp) on algorithmic bytes. ``cpu_baseline`` times the fp64 CPU
oracle on a bounded sample of the same workload with every host thread and
with one (medians over repeats).

Prints ONE JSON line.
"""
import argparse
import json
import os
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0
COPY_BYTES = 1 << 31  # read and written once by the calibration copy


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="logits-bf16-b512-k16-v256000-zipf")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lookahead-sweep", action="store_true",
                    help="skip the greedy look-ahead depths (profiler runs: one launch shape, one depth)")
    ap.add_argument("--top-k", type=int, default=50, help="top-k of the filtered-warp leg")
    ap.add_argument("--top-p", type=float, default=0.9, help="top-p of the filtered-warp leg")
    ap.add_argument("--copy-calibrate", action="store_true",
                    help="also run a plain fp32 device copy of COPY_BYTES (counter calibration under rocprofv3)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a --copy-calibrate run "
                         "into the traffic file, then exit")
    ap.add_argument("--traffic", default=os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                                      "warp_traffic.json"),
                    help="measured HBM bytes per warp launch (from rocprofv3 counters), if present")
    return ap.parse_args()


class Rotation:
    """Copies of the batch's inputs in HBM: copy 0 is the batch itself, the rest
    clones, so that consecutive calls can read different copies. With n copies
    of more than 1 GiB together (and n >= 4) every call of a cycle reads inputs
    that the n - 1 calls before it have pushed out of the L2 caches and the
    256 MB MALL: the "hbm" timings. Timing copy 0 over and over gives the
    "resident" ones."""

    def __init__(self, batch, min_total=1 << 30, min_copies=4):
        import torch
        t, d = batch.target, batch.draft
        per = t.numel() * t.element_size() + d.numel() * d.element_size() + batch.tokens.numel() * 4 \
            + batch.uniforms.numel() * 4
        self.n = max(min_copies, -(-min_total // per) + 1)
        self.bytes_per_copy = per
        extra = self.n - 1

        def stack(x):
            if x is None:
                return [None] * self.n
            more = x.unsqueeze(0).expand((extra,) + tuple(x.shape)).clone() if extra else None
            return [x] + ([more[i] for i in range(extra)] if extra else [])
        self.target, self.draft = stack(t), stack(d)
        self.tokens, self.uniforms = stack(batch.tokens), stack(batch.uniforms)
        self.lens = stack(batch.lens)
        torch.cuda.synchronize()


def timed(fn, indices, stream):
    """Milliseconds per call of fn(i) over the indices, HIP events on `stream`."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in indices:
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / len(indices)


def main():
    args = parse()
    if args.traffic_from:
        traffic_from_counters(args.traffic_from[0], args.traffic_from[1], args.workload, args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              f"(sequences would shard across GPUs with no exchange between them)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_token_verification_amd as sv
    import synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    batch = synth.generate(args.workload, dev)
    B, K, V = batch.B, batch.K, batch.V
    T = batch.temperature
    elem = 2 if batch.dtype == "bf16" else 4
    logits = batch.kind == "logits"
    rot = Rotation(batch)
    stream = torch.cuda.current_stream(dev)

    p = torch.empty((B, K + 1, V), dtype=torch.float32, device=dev) if logits else None
    q = torch.empty((B, K, V), dtype=torch.float32, device=dev) if logits else None
    o = {m: (torch.empty(B, dtype=torch.int32, device=dev), torch.empty(B, dtype=torch.int32, device=dev))
         for m in ("greedy", "sampled", "fused", "fused_lse")}
    # each draft row's normaliser log sum_x exp(z_d / T): an input the draft model has when it
    # samples (the same for every copy of the inputs); fp64 in torch, rounded to fp32
    lse = None
    if logits and K > 0:
        lse = torch.empty((B, K), dtype=torch.float32, device=dev)
        for b0 in range(0, B, 32):
            lse[b0:b0 + 32] = torch.logsumexp(batch.draft[b0:b0 + 32].double() / T, -1).float()

    # the modes, each a function of the input copy it reads
    def greedy(c):
        sv.sv_verify_greedy(rot.target[c], rot.tokens[c], rot.lens[c], out=o["greedy"])

    def warp_t(c):
        sv.sv_softmax_warp(rot.target[c], T, rot.lens[c], 1, out=p)

    def warp_d(c):
        sv.sv_softmax_warp(rot.draft[c], T, rot.lens[c], 0, out=q)

    def accept(c):
        pp, qq = (p, q) if logits else (rot.target[c], rot.draft[c])
        sv.sv_accept(pp, qq, rot.tokens[c], rot.uniforms[c], rot.lens[c], out=o["sampled"])

    def sampled_warps(c):
        if logits:
            warp_t(c)
            warp_d(c)
        accept(c)

    def fused(c):
        sv.sv_accept_logits(rot.target[c], rot.draft[c], rot.tokens[c], rot.uniforms[c], T, rot.lens[c],
                            out=o["fused"])

    def fused_lse(c):
        sv.sv_accept_logits(rot.target[c], rot.draft[c], rot.tokens[c], rot.uniforms[c], T, rot.lens[c],
                            out=o["fused_lse"], draft_lse=lse)

    def step(c):  # one pass of the whole hot path: both warps, the sampled verify, the greedy verify
        sampled_warps(c)
        greedy(c)

    W, S, n = args.warmup, args.steps, rot.n
    hbm = [(W + i) % n for i in range(S)]      # each call a different copy from the last n - 1
    resident = [0] * S

    def measure(fn):
        for i in range(W):
            fn(i % n)
        h = timed(fn, hbm, stream)
        for _ in range(W):
            fn(0)
        r = timed(fn, resident, stream)
        return h, r

    modes = {"step": step, "greedy": greedy, "sampled_warps": sampled_warps}
    if logits:
        modes["sampled_fused"] = fused
    if lse is not None:
        modes["sampled_fused_lse"] = fused_lse
    ms = {m: measure(fn) for m, fn in modes.items()}

    # the step's kernels one by one (HBM copies): events between the launches
    per = np.zeros(4)
    for i in hbm:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        ev[0].record(stream)
        if logits:
            warp_t(i)
        ev[1].record(stream)
        if logits:
            warp_d(i)
        ev[2].record(stream)
        accept(i)
        ev[3].record(stream)
        greedy(i)
        ev[4].record(stream)
        torch.cuda.synchronize()
        per += [ev[j].elapsed_time(ev[j + 1]) for j in range(4)]
    per /= len(hbm)
    warp_t_ms, warp_d_ms, accept_ms, greedy_ms = per

    # algorithmic bytes of each kernel (what the method must move)
    kb = batch.lens.cpu().numpy() if batch.lens is not None else np.full(B, K)
    n_s = o["sampled"][0].cpu().numpy().astype(np.int64)
    n_g = o["greedy"][0].cpu().numpy().astype(np.int64)
    rows_t, rows_d = int((kb + 1).sum()), int(kb.sum())
    warp_bytes_t = rows_t * V * (elem + 4)
    warp_bytes_d = rows_d * V * (elem + 4)
    greedy_bytes = int(((n_g + 1) * V * elem).sum()) + 4 * B * K + 8 * B
    accept_bytes = int((8 * np.minimum(n_s + 1, kb) + np.where(n_s < kb, 2 * V * 4, V * 4)).sum()) \
        + 4 * B * (K + 1) + 8 * B
    gbs = lambda nbytes, t_ms: nbytes / (t_ms * 1e-3) / 1e9 if t_ms and t_ms > 0 else None
    frac = lambda x: None if x is None else round(x / HBM_PEAK_GBS, 4)
    r1 = lambda x, d=1: None if x is None else round(x, d)

    # bytes the kernels read (rocprofv3 FETCH_SIZE, scaled; from the traffic file when it matches these sources)
    traffic = {}
    if os.path.exists(args.traffic):
        with open(args.traffic) as f:
            tr = json.load(f)
        if tr.get("workload") == args.workload and tr.get("library_source_sha") == kernel_source_sha(True):
            traffic = tr

    def read_bytes(kernel, launches=1):
        """FETCH bytes of one call's launches of `kernel`: its recorded launch
        shapes, which must number `launches` (one per launch of the call)."""
        grids = traffic.get("kernels", {}).get(kernel, {})
        if len(grids) != launches:
            return None
        return sum(g["fetch"] for g in grids.values())

    def mode_record(name, t_hbm, t_res, needed=None, read=None, **extra):
        rec = {"hbm_ms": round(t_hbm, 4), "resident_ms": round(t_res, 4),
               "hbm_rounds_per_s": round(1000.0 / t_hbm, 3), "resident_rounds_per_s": round(1000.0 / t_res, 3)}
        if needed is not None:
            g = gbs(needed, t_hbm)
            rec.update({"needed_bytes": int(needed), "needed_GBps": r1(g), "needed_frac": frac(g)})
        if read is not None:
            g = gbs(read, t_hbm)
            rec.update({"read_bytes": int(read), "read_GBps": r1(g), "read_frac": frac(g)})
        rec.update(extra)
        return rec

    modes_out = {}
    modes_out["greedy"] = mode_record("greedy", *ms["greedy"], needed=greedy_bytes,
                                      read=read_bytes("greedy_sliced_kernel") or read_bytes("greedy_kernel"),
                                      mean_n=round(float(n_g.mean()), 4))
    if sv.sv_verify_greedy_workspace_bytes(B, K, V) > 0 and not args.no_lookahead_sweep:
        # the split walk's look-ahead depth L (rows read ahead of the decision): the same results, more
        # bytes loaded -- (min(K_b, n + L) + 1) rows of each sequence -- and the time they take
        la = {}
        try:
            for depth in (1, 2, K + 1):
                sv.sv_set_greedy_lookahead(depth)
                loaded = int(((np.minimum(kb, n_g + depth) + 1) * V * elem).sum()) + 4 * B * K + 8 * B
                la[str(depth)] = mode_record("greedy", *measure(greedy), needed=greedy_bytes, read=loaded)
        finally:
            sv.sv_set_greedy_lookahead()
        modes_out["greedy"]["lookahead"] = la
    sw_needed = accept_bytes + (warp_bytes_t + warp_bytes_d if logits else 0)
    rd_acc = read_bytes("accept_kernel")
    rd_warp = read_bytes("warp_coop_kernel", 2) if logits else 0
    modes_out["sampled_warps"] = mode_record(
        "sampled_warps", *ms["sampled_warps"], needed=sw_needed,
        read=None if rd_acc is None or rd_warp is None else rd_acc + rd_warp, mean_n=round(float(n_s.mean()), 4))
    if logits:
        n_f = o["fused"][0].cpu().numpy().astype(np.int64)
        # target rows 0..n and draft rows 0..min(n, kb-1), each read once
        fused_bytes = int(((n_f + 1 + np.minimum(n_f + 1, kb)) * V * elem).sum()) + 4 * B * (2 * K + 1) + 8 * B
        modes_out["sampled_fused"] = mode_record(
            "sampled_fused", *ms["sampled_fused"], needed=fused_bytes,
            read=read_bytes("accept_logits_sliced_kernel") or read_bytes("accept_logits_kernel"),
            mean_n=round(float(n_f.mean()), 4))
    if lse is not None:
        n_l = o["fused_lse"][0].cpu().numpy().astype(np.int64)
        # target rows 0..n, the draft row n at a rejection, one draft logit per examined position,
        # the normalisers of the examined positions
        examined = np.minimum(n_l + 1, kb)
        lse_bytes = int(((n_l + 1 + (n_l < kb)) * V * elem + examined * (elem + 4)).sum()) + 4 * B * (2 * K + 1) \
            + 8 * B
        modes_out["sampled_fused_lse"] = mode_record(
            "sampled_fused_lse", *ms["sampled_fused_lse"], needed=lse_bytes,
            read=read_bytes("accept_logits_sliced_kernel_lse") or read_bytes("accept_logits_kernel_lse"),
            mean_n=round(float(n_l.mean()), 4), same_as_fused=bool((n_l == n_f).all()))
    step_hbm, step_res = ms["step"]
    modes_out["step"] = mode_record("step", step_hbm, step_res, needed=sw_needed + greedy_bytes)

    out = {
        "metric": "verify rounds/s and achieved HBM GB/s (% of peak) for [B,K+1,V] verify",
        "value": round(1000.0 / step_hbm, 3),
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": S,
        "warmup": W,
        "ms_per_step": round(step_hbm, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "K": K, "V": V, "input_dtype": batch.dtype,
                   "temperature": T,
                   "step": ("warp(target)+warp(draft)+accept+greedy" if logits
                            else "accept+greedy (inputs are probabilities)"),
                   "inputs": f"{n} rotating copies of {rot.bytes_per_copy / 1e9:.3f} GB; value is the hbm timing"},
    }
    if logits:
        warp_ms = warp_t_ms + warp_d_ms
        achieved = gbs(warp_bytes_t + warp_bytes_d, warp_ms)
        wt = traffic.get("bytes_per_launch") if traffic.get("kernel_source_sha") == kernel_source_sha() else None
        out["roofline"] = {"bound": "hbm", "kernel": "warp_coop_kernel", "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": wt,
                           "algorithmic_bytes_per_launch": (warp_bytes_t + warp_bytes_d) // 2,
                           "avg_launch_ms": round(warp_ms / 2, 4)}
    else:  # probabilities in: the sampled verify is the step's largest kernel
        achieved = gbs(accept_bytes, accept_ms)
        out["roofline"] = {"bound": "hbm", "kernel": "accept_kernel", "achieved": round(achieved, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": read_bytes("accept_kernel"), "algorithmic_bytes_per_launch": int(accept_bytes),
                           "avg_launch_ms": round(accept_ms, 4)}
    out["modes"] = modes_out
    out["kernels"] = {
        "warp_target_ms": round(warp_t_ms, 4) if logits else None,
        "warp_draft_ms": round(warp_d_ms, 4) if logits else None,
        "accept_ms": round(accept_ms, 4), "greedy_ms": round(greedy_ms, 4),
        "warp_GBps": r1(gbs(warp_bytes_t + warp_bytes_d, warp_t_ms + warp_d_ms)) if logits else None,
        "accept_GBps_needed": r1(gbs(accept_bytes, accept_ms)),
        "greedy_GBps_needed": r1(gbs(greedy_bytes, greedy_ms)),
    }

    if logits:
        # the filtered warp (temperature, top-k, top-p) of target and draft rows
        tk = torch.full((B,), args.top_k, dtype=torch.int32, device=dev)
        tp = torch.full((B,), args.top_p, dtype=torch.float32, device=dev)

        def filtered(c):
            sv.sv_softmax_warp_filtered(rot.target[c], T, rot.lens[c], 1, tk, tp, out=p)
            sv.sv_softmax_warp_filtered(rot.draft[c], T, rot.lens[c], 0, tk, tp, out=q)
        fh, fr = measure(filtered)
        modes_out["filtered_warps"] = mode_record("filtered_warps", fh, fr, needed=warp_bytes_t + warp_bytes_d,
                                                  top_k=args.top_k, top_p=args.top_p)

        # the penalty stage of the target rows: a committed history of up to
        # 2048 tokens per sequence plus each row's draft prefix
        cap = 2048
        g = torch.Generator(device=dev).manual_seed(7)
        seq = torch.randint(0, V, (B, cap), generator=g, device=dev, dtype=torch.int32)
        seq_len = torch.randint(cap // 2, cap + 1, (B,), generator=g, device=dev, dtype=torch.int32)
        ws = torch.empty(sv.sv_apply_penalties_workspace_bytes(B, cap), dtype=torch.uint8, device=dev)

        def penalties(c):
            sv.sv_apply_penalties(rot.target[c], rot.lens[c], 1, seq, seq_len, rot.tokens[c], 1.2, 0.3, 0.1,
                                  out=p, workspace=ws)
        ph, pr = measure(penalties)
        pen_bytes = warp_bytes_t + int(seq_len.sum().item()) * 4
        modes_out["penalties_target"] = mode_record("penalties_target", ph, pr, needed=pen_bytes,
                                                    history_cap=cap)
        del seq, seq_len, ws

    # per-round latency, eager and replayed from a HIP graph (torch.cuda.CUDAGraph), resident inputs
    def latency_us(fn, reps=50):
        fn()
        torch.cuda.synchronize()
        eager = timed(lambda _: fn(), range(reps), stream) * 1e3
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            fn()
        graph.replay()
        torch.cuda.synchronize()
        return {"eager": round(eager, 2), "graph": round(timed(lambda _: graph.replay(), range(reps), stream) * 1e3, 2)}

    lat = {"greedy_round": latency_us(lambda: greedy(0))}
    lat["sampled_round_fused" if logits else "sampled_round"] = latency_us(lambda: (fused if logits else accept)(0))
    out["latency_us"] = lat

    # a measured stream-read rate: the greedy verify with draft tokens equal to
    # the target's argmax chain, so every live row of every sequence is read
    chain = batch.target.argmax(-1).to(torch.int32)[:, :K].contiguous()
    n_ch = torch.empty(B, dtype=torch.int32, device=dev)
    nx_ch = torch.empty(B, dtype=torch.int32, device=dev)
    sv.sv_verify_greedy(batch.target, chain, batch.lens, out=(n_ch, nx_ch))
    t_ch = timed(lambda _: sv.sv_verify_greedy(batch.target, chain, batch.lens, out=(n_ch, nx_ch)), range(5), stream)
    out["kernels"]["stream_read_GBps"] = r1(gbs(int(((n_ch.cpu().numpy().astype(np.int64) + 1) * V * elem).sum()),
                                                t_ch))
    del chain, n_ch, nx_ch

    if args.copy_calibrate:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = COPY_BYTES
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def traffic_from_counters(fetch_csv, write_csv, workload, out_path):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch).

    Each counter is scaled by what it reads for the calibration copy of
    COPY_BYTES (read once, written once) in the same run: on gfx950
    FETCH_SIZE reports about half the bytes a copy reads, WRITE_SIZE all of
    them. The roofline's figure is the warp's fast-path kernel, its two
    launches per step (target rows, draft rows) averaged like ``achieved``;
    every other library kernel is recorded per launch shape beside it. A
    shape's figure is the median over its launches: the run also makes
    launches outside the step with the same shape but other traffic (the
    greedy verify over every row, for the stream-read rate).
    """
    import csv
    import re

    kernel_re = re.compile(r"\b(warp_coop_kernel|warp_rows_kernel|warp_filter_kernel|accept_kernel|"
                           r"accept_logits_kernel|accept_logits_sliced_kernel|greedy_kernel|greedy_sliced_kernel|"
                           r"penalty_table_kernel|penalty_rows_kernel|fill_slots|fill_empty)\b")
    lse_re = re.compile(r"accept_logits(?:_sliced)?_kernel(?:<\w+, \w+, true>|ILb[01]ELb[01]ELb1E)")

    def load(path, counter):
        per, copy = {}, []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            m = kernel_re.search(r["Kernel_Name"])
            if m:
                k = m.group(1)
                if k.startswith("accept_logits") and lse_re.search(r["Kernel_Name"]):
                    k += "_lse"  # the instantiation with given draft normalisers
                per.setdefault((k, int(r["Grid_Size"])), []).append(v)
            elif "copyBuffer" in r["Kernel_Name"]:  # the runtime's device-to-device copy
                copy.append(v)
        big = [v for v in copy if v > 0.25 * COPY_BYTES]  # the calibration copies, not small transfers
        warp = {g: v for (k, g), v in per.items() if k == "warp_coop_kernel"}
        if not warp or not big:
            raise SystemExit(f"{path}: no warp kernel or calibration-copy dispatches with {counter}")
        factor = COPY_BYTES / (sum(big) / len(big))
        avg = {kg: statistics.median(v) * factor for kg, v in per.items()}
        per_launch = sum(avg[("warp_coop_kernel", g)] for g in warp) / len(warp)
        return factor, per_launch, avg

    ff, fetch, fetch_by = load(fetch_csv, "FETCH_SIZE")
    wf, write, write_by = load(write_csv, "WRITE_SIZE")
    kernels = {}
    for (k, g), v in sorted(fetch_by.items()):
        kernels.setdefault(k, {})[str(g)] = {"fetch": int(v), "write": int(write_by.get((k, g), 0))}
    rec = {"workload": workload, "kernel": "warp_coop_kernel", "kernel_source_sha": kernel_source_sha(),
           "library_source_sha": kernel_source_sha(all_sources=True),
           "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
           "fetch_bytes_per_launch": int(fetch), "write_bytes_per_launch": int(write),
           "bytes_per_launch": int(fetch + write),
           "per_grid": kernels["warp_coop_kernel"],
           "kernels": kernels,
           "source": [os.path.basename(fetch_csv), os.path.basename(write_csv)]}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def kernel_source_sha(all_sources=False):
    """Hash of the warp kernel's sources (or of every library source): measured
    traffic is void once they change."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "draft_token_verification_amd", "csrc")
    h = hashlib.sha256()
    files = sorted(os.listdir(d)) if all_sources else ["common.hpp", "warp.hip"]
    for f in files:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def cpu_baseline(batch, seconds):
    """The fp64 CPU oracle, as it stands, on a bounded sample of the workload's
    sequences: warp of the live target and draft rows, sampled verify on the
    oracle's own fp64 probabilities, greedy verify on the logits (probability
    workloads: the two verifies). Timed with every host thread and with one,
    each as the median over repeats of its sample (about half of ``seconds``
    each), scaled by B / sample to rounds/s of the whole batch."""
    import numpy as np
    import oracle

    B, K, V = batch.B, batch.K, batch.V
    affinity = len(os.sched_getaffinity(0))
    threads = min(affinity, int(os.environ.get("OMP_NUM_THREADS", affinity)))
    cap = max(1, int(4e9 // ((2 * K + 1) * V * 8)))  # the sample's fp64 probability rows under ~4 GB
    order = np.random.default_rng(0).permutation(B).tolist()

    def sample(n):
        sel = order[:n]
        return (batch.target[sel].cpu(), batch.draft[sel].cpu(), batch.tokens[sel].cpu(), batch.uniforms[sel].cpu(),
                None if batch.lens is None else batch.lens[sel].cpu())

    def run(tgt, drf, tok, uni, ln):
        t0 = time.perf_counter()
        if batch.kind == "logits":
            p = np.nan_to_num(oracle.softmax_warp(tgt, ln, 1, batch.temperature))
            q = np.nan_to_num(oracle.softmax_warp(drf, ln, 0, batch.temperature))
        else:
            p, q = tgt, drf
        oracle.accept(p, q, tok, uni, ln)
        oracle.verify_greedy(tgt, tok, ln)
        return time.perf_counter() - t0

    def leg(nthreads, n, budget):
        used = oracle.set_threads(nthreads)
        data = sample(n)
        times = [run(*data)]
        while sum(times) < budget or len(times) < 3:
            times.append(run(*data))
        med = statistics.median(times)
        return {"value": round(n / (med * B), 6), "unit": "rounds/s", "cores": used, "kind": "oracle",
                "sample": f"{n} of {B} sequences ({100.0 * n / B:.1f}%), median of {len(times)} repeats "
                          f"({med:.3f} s each), scaled by B/{n}"}

    n_all = min(B, cap, max(threads, 1) * 4)
    all_core = leg(threads, n_all, seconds / 2)
    single = leg(1, max(1, min(n_all, 2)), seconds / 2)
    oracle.set_threads(threads)
    all_core["what"] = ("warp of the live target and draft rows, sampled verify on the oracle's fp64 probs, greedy "
                        "on the logits" if batch.kind == "logits" else "sampled and greedy verify of the probs")
    all_core["single_thread"] = single
    return all_core


if __name__ == "__main__":
    main()
