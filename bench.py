"""Benchmark: MoE dispatch + combine on simulated ranks, one MI355X.

One step = one pass of the whole path over one batch: routing layout
(counts, rank prefix matrix, slots), dispatch scatter into the receive
layout, combine gather-reduce back to token order.  The expert between
dispatch and combine is the identity (combine reads the receive buffer),
so the step moves exactly the path's own bytes.

Default workload: 8 simulated ranks x 4096 tokens, hidden 7168 bf16, 256
experts, top-8 with Zipf(1.2) popularity, contiguous (normal-mode) layout.
The low-latency decode workload (8 x 128 tokens, packed masked layout, FP8
with fp32 scales) is timed alongside and reported under "low_latency".

`value` is algorithmic GB/s: the bytes the method must move (x read once,
K receive rows written, K rows read back, the output written, plus the
layout's index traffic) divided by the step time.  Inputs are resident in
HBM before the timed region.

Prints one JSON line.  Only one GPU is used: --gpus above 1 exits with a
message.
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

PEAK_HBM_GBPS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layout_bytes(w, send_head=True):
    R, T, K = w.R, w.T, w.K
    M = R * T * K
    b = 4 * M            # topk read
    b += 4 * M           # send_pos written
    b += R * T * R       # is_token_in_rank written
    if send_head:
        b += 4 * R * T * R
    return b


def step_bytes(w, rows):
    """Algorithmic bytes of layout, dispatch and combine for one step."""
    R, T, H, K, G = w.R, w.T, w.H, w.K, w.G
    N, M = R * T, R * T * K
    lay = layout_bytes(w) + 4 * rows  # + recv_src_idx
    if w.quant == 0:
        disp = 2 * H * N + 2 * H * M + 4 * M
    elif w.quant == 1:
        disp = 2 * H * N + (H + 4 * G) * M + 4 * M
    else:
        disp = 2 * H * N + (H + G) * M + 4 * M
    comb = 2 * H * M + 2 * H * N + 8 * M
    return lay, disp, comb


def kernel_hash():
    h = hashlib.sha256()
    for f in ["dispatch.hip", "combine.hip", "quant.hpp", "ep_device.hpp"]:
        with open(os.path.join(ROOT, "combine_ep_get_layout_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/
    counters.json), or None when absent or taken on different kernel code."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(kernel)
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("hbm_bytes_per_launch")


class Runner:
    """Buffers and launches of one workload; everything resident in HBM."""

    def __init__(self, w, torch, ep, inputs):
        self.w, self.torch, self.ep = w, torch, ep
        dev = "cuda"
        log(f"[bench] {w.name}: generating inputs")
        topk = inputs.gen_topk(w)
        x = inputs.gen_x(w)
        wt = inputs.gen_weights(w)
        self.p = ep.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
        self.topk = torch.from_numpy(topk).to(dev)
        self.x = torch.from_numpy(x).view(torch.bfloat16).to(dev)
        self.wt = torch.from_numpy(wt).to(dev)
        self.lay = ep.Layout(self.p)
        self.ws = ep.workspace(self.p)
        ep.get_layout(self.p, self.topk, self.lay, self.ws)
        torch.cuda.synchronize()
        if w.mode == ep.MODE_NORMAL:
            self.rows = int(self.lay.row_base[-1].item())  # untimed read-back of the receive size
        else:
            self.rows = w.E * w.R * w.T
        self.recv = ep.Recv(self.p, self.rows)
        if w.quant == ep.QUANT_NONE:
            self.y = self.recv.x  # identity expert
        else:
            # expert outputs in bf16 in the receive layout (values do not
            # change the data movement)
            self.y = torch.empty((self.rows, w.H), dtype=torch.bfloat16, device=dev)
            self.y.normal_()
        self.out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=dev)
        lb, db, cb = step_bytes(w, self.rows if w.mode == ep.MODE_NORMAL else w.R * w.T * w.K)
        self.bytes = {"layout": lb, "dispatch": db, "combine": cb}

    def step(self, ev=None):
        ep, p = self.ep, self.p
        if ev is not None:
            ev[0].record()
        ep.get_layout(p, self.topk, self.lay, self.ws)
        if ev is not None:
            ev[1].record()
        ep.dispatch(p, self.lay, self.x, recv=self.recv, ws=self.ws)
        if ev is not None:
            ev[2].record()
        ep.combine(p, self.lay, self.y, self.wt, self.out)
        if ev is not None:
            ev[3].record()

    def run(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        err = int(self.lay.err.item())
        if err:
            raise RuntimeError(f"device error word {err}")
        ph = {"layout": [], "dispatch": [], "combine": []}
        for e in evs:
            ph["layout"].append(e[0].elapsed_time(e[1]))
            ph["dispatch"].append(e[1].elapsed_time(e[2]))
            ph["combine"].append(e[2].elapsed_time(e[3]))
        ms = (t1 - t0) * 1e3 / steps
        return ms, {k: float(np.mean(v)) for k, v in ph.items()}, \
            {k: float(np.median(v)) for k, v in ph.items()}


def copy_probe(torch, nbytes=4 << 30, reps=10):
    """Device-to-device copy bandwidth (read + write bytes / time)."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(w, inputs, tokens_per_rank):
    """The plain C oracle on a bounded sample of the workload: the first
    `tokens_per_rank` tokens of every rank, layout + dispatch + combine,
    single-threaded, outputs preallocated and touched before timing."""
    from oracle import oracle as orc

    T = tokens_per_rank
    topk = np.ascontiguousarray(inputs.gen_topk(w)[:, :T])
    x = np.ascontiguousarray(inputs.gen_x(w)[:, :T])
    wt = np.ascontiguousarray(inputs.gen_weights(w)[:, :T])
    p = orc.Problem(w.R, T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
    lay = orc.layout(p, topk)
    rows = lay.total_rows
    recv = np.ones((rows, w.H), np.uint16)
    out = np.ones((w.R, T, w.H), np.uint16)
    t0 = time.perf_counter()
    lay = orc.layout(p, topk)
    orc.dispatch(p, x, topk, lay.send_pos, rows, out=(recv, None))
    orc.combine(p, recv, wt, lay.send_pos, out=out)
    dt = time.perf_counter() - t0
    sw = w.replace(T=T)
    lb, db, cb = step_bytes(sw, rows)
    gbps = (lb + db + cb) / dt / 1e9
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {T} of {w.T} tokens on each of the {w.R} ranks "
                      f"(layout + dispatch + combine, {dt:.2f} s, single thread)",
            "tokens_per_s": round(w.R * T / dt, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="normal_prefill")
    ap.add_argument("--no-ll", action="store_true", help="skip the low-latency workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=512)
    ap.add_argument("--calib", action="store_true",
                    help="also run a plain copy of 2^30 bytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: simulated ranks are partitions of one "
              "GPU's HBM; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_ep_get_layout_amd import ep, inputs

    ep.lib()  # fail loudly if the HIP library is missing
    w = inputs.WORKLOADS[args.workload]
    r = Runner(w, torch, ep, inputs)
    log(f"[bench] {w.name}: timing {args.steps} steps after {args.warmup} warm-up")
    ms, mean_ph, med_ph = r.run(args.steps, args.warmup)
    total = sum(r.bytes.values())
    gbps = total / (ms * 1e-3) / 1e9
    tok_s = w.N / (ms * 1e-3)
    dom = max(("dispatch", "combine"), key=lambda k: mean_ph[k])
    kname = {"dispatch": "dispatch_copy", "combine": "combine_rows"}[dom]
    ach = r.bytes[dom] / (mean_ph[dom] * 1e-3) / 1e9
    traffic = traffic_from_profile(kname)
    phases = {k: {"ms_mean": round(mean_ph[k], 4), "ms_median": round(med_ph[k], 4),
                  "bytes": r.bytes[k],
                  "GBps": round(r.bytes[k] / (mean_ph[k] * 1e-3) / 1e9, 1)} for k in mean_ph}
    del r
    torch.cuda.empty_cache()

    ll = None
    if not args.no_ll and args.workload != "ll_decode":
        wl = inputs.WORKLOADS["ll_decode"]
        rl = Runner(wl, torch, ep, inputs)
        ms_l, mean_l, _ = rl.run(max(args.steps, 20), args.warmup)
        tb = sum(rl.bytes.values())
        ll = {"workload": "ll_decode R8 T128 H7168 E256 K8 uniform, packed masked, fp8 e4m3 fp32 scales",
              "ms_per_step": round(ms_l, 4), "GBps": round(tb / (ms_l * 1e-3) / 1e9, 1),
              "tokens_per_s": round(wl.N / (ms_l * 1e-3), 1), "bytes_per_step": tb,
              "phase_ms": {k: round(v, 4) for k, v in mean_l.items()},
              "cache": "warm: the step's data fits in the 256 MB last-level cache"}
        del rl
        torch.cuda.empty_cache()

    if args.calib:
        a = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    probe = copy_probe(torch)
    cpu = None if args.no_cpu else cpu_baseline(w, inputs, args.cpu_tokens)

    line = {
        "metric": "dispatch+combine achieved HBM GB/s and tokens/s at 1 GPU (LL and normal)",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.quant == 0 else "fp8-e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name} R{w.R} T{w.T} H{w.H} E{w.E} K{w.K} "
                               f"{w.routing}{w.alpha if w.routing == 'zipf' else ''} "
                               f"{'contiguous' if w.mode == 0 else 'packed-masked'}",
                   "ranks": w.R, "tokens_per_rank": w.T, "hidden": w.H, "experts": w.E,
                   "topk": w.K, "bytes_per_step": total},
        "tokens_per_s": round(tok_s, 1),
        "phases": phases,
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic},
        "copy_probe_GBps": round(probe, 1),
        "low_latency": ll,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
