"""Benchmark: MoE dispatch + combine on simulated ranks, one MI355X.

One step = one pass of the whole path over one batch: the routing layout
(counts, rank prefix matrix, slots), the dispatch scatter into the receive
layout, and the combine gather-reduce back to token order.  The expert
between dispatch and combine is the identity for bf16 layouts (combine
reads the receive buffer), so the step moves exactly the path's own bytes;
FP8 layouts combine bf16 expert outputs of the receive shape.  In message
mode a step is the layout, the packer (table, payload, header / flag /
descriptors), the loopback delivery of the descriptors and the receiver
that unpacks the delivered messages into the low-latency layout.

The headline workload (`value`) is the normal-mode prefill shape: 8
simulated ranks x 4096 tokens, hidden 7168 bf16, 256 experts, top-8 with
Zipf(1.2) popularity, contiguous layout.  The other workloads of the method
are timed alongside under "workloads": low-latency decode (8 x 128 tokens,
packed masked, FP8 + fp32 scales), the FP8 training shape (16 x 8192,
hidden 4096, UE8M0 column-major scales), the 64-rank message path, and the
prefill routing in the rank-major (one row per token and destination rank)
layout.

`value` is algorithmic GB/s: the bytes the method must move (x read once,
K receive rows written, K rows read back, the output written, plus the
layout's index traffic) divided by the step time, with inputs resident in
HBM before the timed region.  Per-phase times (mean, median, p10, p90) come
from a second pass with HIP events on the stream the library launches on
(torch's current stream).  `roofline` is for the slowest phase that is a
single kernel launch, so that its event time is that kernel's duration
(the fused call, the FP8 normal-mode dispatch and the message packer and
delivery launch several kernels).  `without_layout` times the calls after the
layout alone (dispatch + combine), the same way as the headline.
Workloads whose data fit in the 256 MB last-level cache also report a
cold-cache step time (`cold`: 1 GiB overwritten before every step).

Prints one JSON line.  One GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
DEFAULT_WORKLOADS = ["normal_prefill", "ll_decode", "fp8_train", "messages", "rank_prefill"]
# workloads timed with the fused layout + dispatch call (measured on MI355X
# when it was introduced: low-latency decode 55.8 -> 53.0 us, FP8 training
# 2.867 -> 2.829 ms per step; the prefill step is 0.5% slower fused, 1.502
# against 1.494 ms, and keeps the two calls)
FUSED_WORKLOADS = {"ll_decode", "fp8_train"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def layout_rw(w, rows_written):
    """(read, written) bytes: topk read; send_pos / is_token_in_rank /
    send_head written, and one recv_src_idx entry per filled row."""
    R, T, K = w.R, w.T, w.K
    M = R * T * K
    wr = R * T * R + 4 * R * T * R + 4 * rows_written
    if w.mode != 2:
        wr += 4 * M
    return 4 * M, wr


def dispatch_rw(w, rows=None):
    """(read, written) bytes: x read once and a slot per routed pair; the
    rows (bf16, or codes and scales) written."""
    R, T, H, K, G = w.R, w.T, w.H, w.K, w.G
    N, M = R * T, R * T * K
    row = {0: 2 * H, 1: H + 4 * G, 2: H + G}[w.quant]
    if w.mode == 3:  # rank-major: one row per (token, rank), plus its top-k ids and weights
        return 2 * H * N + 4 * M + 8 * M, rows * (row + 8 * K)
    return 2 * H * N + 4 * M, row * M


def combine_rw(w, rows=None):
    """(read, written) bytes: the routed rows, slots and weights read; the
    output written."""
    R, T, H, K = w.R, w.T, w.H, w.K
    N, M = R * T, R * T * K
    if w.mode == 3:  # rank-major: each distinct row once, unweighted
        return 2 * H * rows + 4 * M, 2 * H * N
    return 2 * H * M + 8 * M, 2 * H * N


def layout_bytes(w, rows_written):
    return sum(layout_rw(w, rows_written))


def dispatch_bytes(w, rows=None):
    return sum(dispatch_rw(w, rows))


def combine_bytes(w, rows=None):
    return sum(combine_rw(w, rows))


# sources each profiled kernel is built from (its counters go stale when
# any of them changes)
KERNEL_SOURCES = {
    "dispatch_copy": ["dispatch.hip", "layout_rows.hpp", "ep_device.hpp", "ep_internal.hpp"],
    "dispatch_fp8": ["dispatch.hip", "layout_rows.hpp", "quant.hpp", "ep_device.hpp",
                     "ep_internal.hpp"],
    "combine_rows": ["combine.hip", "ep_device.hpp", "ep_internal.hpp"],
    "msg_pack_fp8": ["messages.hip", "msg_format.hpp", "quant.hpp", "ep_device.hpp",
                     "ep_internal.hpp"],
    "msg_pack_bf16": ["messages.hip", "msg_format.hpp", "ep_device.hpp", "ep_internal.hpp"],
    "msg_exec_puts": ["receive.hip", "msg_format.hpp", "ep_device.hpp", "ep_internal.hpp"],
    "msg_unpack": ["receive.hip", "msg_format.hpp", "ep_device.hpp", "ep_internal.hpp"],
}


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that a comment edit
    does not mark the counters of unchanged kernel code as stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "combine_ep_get_layout_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/
    counters.json), or None when absent or taken on different kernel code."""
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(f"{workload}:{kernel}")
    if not e or e.get("kernel_hash") != kernel_hash(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


class Runner:
    """Buffers and launches of one workload; everything resident in HBM."""

    def __init__(self, w, torch, ep, inputs, keep_host=False, fused=False):
        self.w, self.torch, self.ep = w, torch, ep
        self.fused = fused and w.mode in (ep.MODE_NORMAL, ep.MODE_LOW_LATENCY)
        dev = "cuda"
        log(f"[bench] {w.name}: generating inputs")
        topk = inputs.gen_topk(w)
        x = inputs.gen_x(w)
        wt = inputs.gen_weights(w)
        self.host = (topk, x, wt) if keep_host else None
        self.p = ep.Problem(w.R, w.T, w.H, w.E, w.K, mode=w.mode, quant=w.quant,
                            region_bytes=w.region_bytes, epoch=w.epoch)
        self.topk = torch.from_numpy(topk).to(dev)
        self.x = torch.from_numpy(x).view(torch.bfloat16).to(dev)
        self.wt = torch.from_numpy(wt).to(dev)
        self.lay = ep.Layout(self.p)
        self.ws = ep.workspace(self.p)
        ep.get_layout(self.p, self.topk, self.lay, self.ws)
        torch.cuda.synchronize()
        self.msgs = self.recv = self.y = self.out = None
        if w.mode == ep.MODE_MESSAGES:
            # untimed read-back of the per-pair counts to size the arena
            send_cap, desc_cap = ep.messages_capacity(self.p, self.lay.num_tokens_per_rank.cpu().numpy())
            self.msgs = ep.Messages(self.p, send_cap, desc_cap)
            ep.dispatch(self.p, self.lay, self.x, msgs=self.msgs, topk_idx=self.topk,
                        topk_weights=self.wt, ws=self.ws)
            torch.cuda.synchronize()
            table = self.msgs.table.cpu().numpy()
            nd = int(self.msgs.num_descriptors.item())
            msg_bytes = int(table[:, :, 2].sum())
            n_msg = int((table[:, :, 2] > 0).sum())
            # delivery into the receive arenas, then unpacking into the
            # low-latency layout (E*R*T rows)
            self.recv_cap = int(self.msgs.arena_base[1, -1].item())
            self.recv_arena = torch.empty(self.recv_cap, dtype=torch.uint8, device=dev)
            self.err = torch.zeros(1, dtype=torch.int32, device=dev)
            self.unp = ep.unpack_buffers(self.p)
            cb = 2 if w.quant == ep.QUANT_NONE else 1
            sb = {0: 0, 1: 4, 2: 1}[w.quant]
            routed = int((topk >= 0).sum())
            tokens_sent = int(table[:, :, 3].sum())
            row = w.H * cb + w.G * sb
            # (read, written): the packer reads x, the weights and the ids
            # and writes the messages, descriptors and table; delivery reads
            # the descriptors and copies the messages; the receiver reads
            # each routed row, the per-token metadata, header and flag, and
            # writes the rows, scales and source indices
            self.rw = {"layout": layout_rw(w, 0),
                       "dispatch": (2 * w.H * w.N + 8 * w.K * w.N,
                                    msg_bytes + 64 * nd + 64 * w.R * w.R),
                       "execute": (msg_bytes + 64 * nd, msg_bytes),
                       "unpack": (routed * row + tokens_sent * (4 * w.K + 4) + 32 * n_msg,
                                  routed * (row + 4))}
            self.bytes = {k: sum(v) for k, v in self.rw.items()}
            # the pack and delivery calls are several launches each
            self.kernels = {"unpack": "msg_unpack"}
            self.extra = {"messages": n_msg, "descriptors": nd, "message_bytes": msg_bytes}
            return
        if w.mode in (ep.MODE_NORMAL, ep.MODE_RANK_MAJOR):
            self.rows = int(self.lay.row_base[-1].item())  # untimed read-back of the receive size
            filled = self.rows
        else:
            self.rows = w.E * w.R * w.T
            filled = w.R * w.T * w.K
        self.recv = ep.Recv(self.p, self.rows)
        if w.quant == ep.QUANT_NONE:
            self.y = self.recv.x  # identity expert
        else:
            # bf16 expert outputs in the receive layout (values do not change
            # the data movement)
            self.y = torch.empty((self.rows, w.H), dtype=torch.bfloat16, device=dev)
            self.y.normal_()
        self.out = torch.empty((w.R, w.T, w.H), dtype=torch.bfloat16, device=dev)
        self.rw = {"layout": layout_rw(w, filled), "dispatch": dispatch_rw(w, self.rows),
                   "combine": combine_rw(w, self.rows)}
        self.bytes = {k: sum(v) for k, v in self.rw.items()}
        self.kernels = {"combine": "combine_rows"}
        # normal-mode FP8 dispatch also launches the scale transpose
        if w.quant == ep.QUANT_NONE or w.mode == ep.MODE_LOW_LATENCY:
            self.kernels["dispatch"] = "dispatch_copy" if w.quant == 0 else "dispatch_fp8"
        if self.fused:  # the fused call launches the layout's kernels too
            (lr, lw), (dr, dw) = self.rw["layout"], self.rw["dispatch"]
            self.rw = {"layout+dispatch": (lr + dr, lw + dw), "combine": self.rw["combine"]}
            self.bytes = {k: sum(v) for k, v in self.rw.items()}
            self.kernels = {"combine": "combine_rows"}
        self.extra = {}

    def phases(self):
        """The step's calls in order, one per timed phase, each checked and
        marshalled once (ep.prepare): a call in the timed loop only hands
        the cached arguments to the library, as a C caller would."""
        if getattr(self, "_phases", None) is not None:
            return self._phases
        ep, p = self.ep, self.p
        ph = [("layout", ep.prepare(ep.get_layout, p, self.topk, self.lay, self.ws))]
        if self.msgs is not None:
            ph.append(("dispatch", ep.prepare(ep.dispatch, p, self.lay, self.x, msgs=self.msgs,
                                              topk_idx=self.topk, topk_weights=self.wt,
                                              ws=self.ws)))
            ph.append(("execute", ep.prepare(ep.messages_execute, p, self.msgs, self.recv_arena,
                                             self.err)))
            ph.append(("unpack", ep.prepare(ep.messages_unpack, p, self.msgs, self.recv_arena,
                                            self.lay.num_tokens_per_expert, *self.unp,
                                            self.err)))
        elif self.fused:  # layout and dispatch in one call
            ph = [("layout+dispatch", ep.prepare(ep.dispatch_fused, p, self.topk, self.lay,
                                                 self.x, self.recv, self.ws)),
                  ("combine", ep.prepare(ep.combine, p, self.lay, self.y, self.wt, self.out))]
        else:
            if self.w.mode == ep.MODE_RANK_MAJOR:  # rows plus their top-k metadata
                ph.append(("dispatch", ep.prepare(ep.dispatch, p, self.lay, self.x, recv=self.recv,
                                                  topk_idx=self.topk, topk_weights=self.wt,
                                                  ws=self.ws)))
                ph.append(("combine", ep.prepare(ep.combine, p, self.lay, self.y, None,
                                                 self.out)))
            else:
                ph.append(("dispatch", ep.prepare(ep.dispatch, p, self.lay, self.x,
                                                  recv=self.recv, ws=self.ws)))
                ph.append(("combine", ep.prepare(ep.combine, p, self.lay, self.y, self.wt,
                                                 self.out)))
        self._phases = ph
        return ph

    def step(self, ev=None):
        for i, (_, call) in enumerate(self.phases()):
            if ev is not None:
                ev[i].record()
            call()
        if ev is not None:
            ev[-1].record()

    def run(self, steps, warmup):
        """Time `steps` whole steps with nothing else on the stream (the
        headline), then the same number of steps again with events between
        the calls (the per-phase split; an event costs a few microseconds of
        GPU time, so it stays out of the headline)."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / steps
        n_ph = len(self.phases())
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ph + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            self.step(evs[i])
        torch.cuda.synchronize()
        err = int(self.lay.err.item()) | (int(self.err.item()) if self.msgs is not None else 0)
        if err:
            raise RuntimeError(f"device error word {err}")
        names = [n for n, _ in self.phases()]
        ph = {k: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, k in enumerate(names)}
        return ms, ph

    def run_without_layout(self, steps):
        """The step's calls after the layout (dispatch and combine, or the
        message calls), timed like the headline: the layout's outputs stay
        valid since the routing does not change.  None when the layout is
        fused into the dispatch."""
        torch = self.torch
        calls = [c for n, c in self.phases() if n != "layout"]
        if len(calls) == len(self.phases()):
            return None
        for c in calls:
            c()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for c in calls:
                c()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def run_separate_y(self, steps):
        """The step with the combine reading a copy of the receive rows
        made once (untimed) instead of the receive rows themselves: the
        identity expert's output as a buffer of its own.  Returns the step
        time (ms, as the headline) and the mean per-call event times; None
        unless the expert output aliases the receive buffer (bf16 layouts)."""
        torch = self.torch
        if self.y is None or self.recv is None or self.y.data_ptr() != self.recv.x.data_ptr():
            return None
        self.y = self.recv.x.clone()
        self._phases = None
        try:
            for _ in range(3):
                self.step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                self.step()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            names = [n for n, _ in self.phases()]
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
                   for _ in range(steps)]
            for i in range(steps):
                self.step(evs[i])
            torch.cuda.synchronize()
            ph = {k: round(float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])), 4)
                  for i, k in enumerate(names)}
        finally:
            self.y = self.recv.x
            self._phases = None
            torch.cuda.empty_cache()
        return ms, ph

    def publish_curve(self, reps=20, batches=(0, 1, 4, 32)):
        """Delivery time (ms, mean of `reps` back-to-back calls, events
        around them) for each publication batch: 0 = every flag after a
        second launch; B = flags released every B messages per workgroup."""
        torch, ep = self.torch, self.ep
        out = {}
        for b in batches:
            call = ep.prepare(ep.messages_execute, self.p, self.msgs, self.recv_arena, self.err,
                              publish_batch=b)
            call()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                call()
            e.record()
            torch.cuda.synchronize()
            out[str(b)] = round(s.elapsed_time(e) / reps, 4)
        if int(self.err.item()):
            raise RuntimeError(f"device error word {int(self.err.item())}")
        return out

    def run_cold(self, steps, flush_bytes=1 << 30):
        """Step times with the last-level cache flushed before every step
        (a 1 GiB buffer overwritten, untimed); events bracket each step."""
        torch = self.torch
        scratch = torch.empty(flush_bytes // 4, dtype=torch.int32, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for i in range(steps):
            scratch.fill_(i)
            evs[i][0].record()
            self.step()
            evs[i][1].record()
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in evs]
        del scratch
        return t

    def report(self, steps, warmup, extra=True):
        w = self.w
        log(f"[bench] {w.name}: timing {steps} steps after {warmup} warm-up")
        ms, ph = self.run(steps, warmup)
        mean_ph = {k: float(np.mean(v)) for k, v in ph.items()}
        total = sum(self.bytes.values())
        phases = {k: {"ms_mean": round(mean_ph[k], 4),
                      "ms_median": round(float(np.median(v)), 4),
                      "ms_p10": round(float(np.percentile(v, 10)), 4),
                      "ms_p90": round(float(np.percentile(v, 90)), 4),
                      "bytes": self.bytes[k],
                      "GBps": round(self.bytes[k] / (mean_ph[k] * 1e-3) / 1e9, 1)}
                  for k, v in ph.items()}
        # the roofline's kernel: the slowest phase that is a single kernel
        # launch, so that its event time is that kernel's duration
        dom = max(self.kernels, key=lambda k: mean_ph[k])
        kname = self.kernels[dom]
        traffic = traffic_from_profile(kname, w.name)
        ach = self.bytes[dom] / (mean_ph[dom] * 1e-3) / 1e9
        mode = {0: "contiguous", 1: "packed-masked", 2: "messages", 3: "rank-major"}[w.mode]
        payload = {0: "bf16", 1: "fp8-e4m3 fp32 scales", 2: "fp8-e4m3 ue8m0 scales"}[w.quant]
        res = {
            "workload": f"{w.name} R{w.R} T{w.T} H{w.H} E{w.E} K{w.K} "
                        f"{w.routing}{w.alpha if w.routing == 'zipf' else ''} {mode} {payload}",
            "ms_per_step": round(ms, 4),
            "GBps": round(total / (ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(w.N / (ms * 1e-3), 1),
            "bytes_per_step": total,
            "calls": ("ep_dispatch_fused, ep_combine" if self.fused else
                      ", ".join("ep_" + n if n in ("dispatch", "combine") else
                                {"layout": "ep_get_layout", "execute": "ep_messages_execute",
                                 "unpack": "ep_messages_unpack"}[n] for n, _ in self.phases())),
            "phases": phases,
            "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1),
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(ach / PEAK_HBM_GBPS, 4),
                         "traffic": traffic},
        }
        if traffic is not None:  # counted HBM bytes over the same launch time
            res["roofline"]["traffic_GBps"] = round(traffic / (mean_ph[dom] * 1e-3) / 1e9, 1)
        # each phase's algorithmic bytes split into reads and writes (for
        # the mix ceiling, added once the probes have run)
        for k in phases:
            phases[k]["read_bytes"], phases[k]["written_bytes"] = self.rw[k]
        res["roofline"]["phase"] = dom
        # the calls after the layout alone (the bar's dispatch + combine)
        ms_nl = self.run_without_layout(steps) if extra else None
        if ms_nl is not None:
            b = total - self.bytes["layout"]
            res["without_layout"] = {"calls": ", ".join(n for n in phases if n != "layout"),
                                     "ms": round(ms_nl, 4),
                                     "GBps": round(b / (ms_nl * 1e-3) / 1e9, 1),
                                     "frac_of_peak": round(b / (ms_nl * 1e-3) / 1e9
                                                           / PEAK_HBM_GBPS, 4)}
        # the same step with the expert output in a buffer of its own: the
        # next dispatch then follows a combine that read other memory
        sep = self.run_separate_y(steps) if extra else None
        if sep is not None:
            res["separate_expert_output"] = {
                "note": "combine reads a copy of the receive rows made once, untimed",
                "ms_per_step": round(sep[0], 4),
                "GBps": round(total / (sep[0] * 1e-3) / 1e9, 1),
                "phase_ms": sep[1]}
        res.update(self.extra)
        if self.msgs is not None and extra:
            res["execute_ms_by_publish_batch"] = self.publish_curve()
        if total < 256e6:
            res["cache"] = "warm: the step's data fits in the 256 MB last-level cache"
        if total < 256e6 and extra:
            t = self.run_cold(steps)
            med = float(np.median(t))
            res["cold"] = {"note": "1 GiB overwritten before every step; events bracket each step",
                           "ms_median": round(med, 4),
                           "ms_p10": round(float(np.percentile(t, 10)), 4),
                           "ms_p90": round(float(np.percentile(t, 90)), 4),
                           "GBps": round(total / (med * 1e-3) / 1e9, 1)}
        return ms, res


PROBE_LIB = os.path.join(ROOT, "libbench_probe.so")
PROBE_KINDS = {"read": 0, "write": 1, "copy": 2}
# fan-out probe shape: row vectors (16 bytes each), rows, copies per row
FANOUT_SHAPE = (896, 32768, 8)


def bandwidth_probes(torch, nbytes=4 << 30, reps=5):
    """HBM read-only, write-only and copy rates of the hand-written probe
    kernels (bench_probe.hip), each the best over vectors in flight per
    thread (1, 2, 4, 8), plain or non-temporal accesses and three grid
    sizes; bytes moved / mean event time of `reps` launches on 4 GiB
    buffers.  These are the device's measured roofs for streams that only
    read or only write, against which the method's mix of reads and
    writes is measured."""
    import ctypes

    if not os.path.exists(PROBE_LIB):
        raise ImportError(f"{PROBE_LIB} is not built; run combine_ep_get_layout_amd/build.py")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.bench_probe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.bench_probe_launch.restype = ctypes.c_int
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    a.fill_(7)
    b.fill_(0)
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for name, kind in PROBE_KINDS.items():
        best = (0.0, None)
        for unroll in (1, 2, 4, 8):
            for nt in (0, 1):
                for blocks in (2048, 8192, 32768):
                    src, dst = (a, sink) if kind == 0 else (a, b)

                    def launch():
                        st = lib.bench_probe_launch(kind, src.data_ptr(), dst.data_ptr(), nbytes,
                                                    unroll, nt, blocks, stream)
                        if st != 0:
                            raise RuntimeError("probe launch failed")

                    launch()
                    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    s.record()
                    for _ in range(reps):
                        launch()
                    e.record()
                    torch.cuda.synchronize()
                    moved = nbytes * (2 if kind == 2 else 1)
                    rate = moved / (s.elapsed_time(e) / reps * 1e-3) / 1e9
                    if rate > best[0]:
                        best = (rate, {"unroll": unroll, "nt": nt, "blocks": blocks})
        out[name + "_GBps"] = round(best[0], 1)
        out[name + "_config"] = best[1]
    # the bf16 dispatch's mix at the prefill shape: 32,768 rows of 14,336
    # bytes, each read once and written to 8 rows (and the combine's below)
    lib.bench_fanout_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p]
    lib.bench_fanout_launch.restype = ctypes.c_int
    fv, fr, fk = FANOUT_SHAPE
    assert fr * fv * 16 <= nbytes and fk * fr * fv * 16 <= nbytes
    best = (0.0, None)
    for form in (0, 1):
        def launch():
            if lib.bench_fanout_launch(a.data_ptr(), b.data_ptr(), fv, fr, fk, form, stream) != 0:
                raise RuntimeError("fan-out probe launch failed")

        launch()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            launch()
        e.record()
        torch.cuda.synchronize()
        rate = fr * fv * 16 * (1 + fk) / (s.elapsed_time(e) / reps * 1e-3) / 1e9
        if rate > best[0]:
            best = (rate, {"row_bytes": fv * 16, "rows": fr, "copies": fk, "form": form})
    out["fanout_GBps"] = round(best[0], 1)
    out["fanout_config"] = best[1]
    # and the combine's: each of the 32,768 rows the xor of 8 rows
    lib.bench_fanin_launch.argtypes = lib.bench_fanout_launch.argtypes
    lib.bench_fanin_launch.restype = ctypes.c_int
    best = (0.0, None)
    for form in (0, 1):
        def launch():
            if lib.bench_fanin_launch(a.data_ptr(), b.data_ptr(), fv, fr, fk, form, stream) != 0:
                raise RuntimeError("fan-in probe launch failed")

        launch()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            launch()
        e.record()
        torch.cuda.synchronize()
        rate = fr * fv * 16 * (1 + fk) / (s.elapsed_time(e) / reps * 1e-3) / 1e9
        if rate > best[0]:
            best = (rate, {"row_bytes": fv * 16, "rows": fr, "copies": fk, "form": form})
    out["fanin_GBps"] = round(best[0], 1)
    out["fanin_config"] = best[1]
    del a, b, sink
    torch.cuda.empty_cache()
    out["source"] = ("bench_probe.hip (16-byte vector streams, 4 GiB buffers; fan-out: each row "
                     "read once and written to `copies` contiguous segments; fan-in: each row "
                     "the xor of `copies` rows of contiguous segments)")
    return out


def mix_ceiling(rw, probes):
    """Time (ms) at the probes' roofs for `rw` = (read, written) bytes when
    reads and writes take turns: read / read rate + written / write rate."""
    r, wr = rw
    return (r / (probes["read_GBps"] * 1e9) + wr / (probes["write_GBps"] * 1e9)) * 1e3


def add_mix_ceiling(res, probes, w=None):
    """Adds to a workload's result the time its reads and writes take at the
    probes' read-only and write-only rates, taking turns (the measured roof
    for that mix of traffic), and the measured fraction of it: per phase,
    for the roofline kernel's phase and for the whole step; also the step's
    rate as a fraction of the copy probe's (a stream that reads and writes
    equal amounts at once)."""
    phases = res["phases"]
    at = 0.0
    for v in phases.values():
        c = mix_ceiling((v["read_bytes"], v["written_bytes"]), probes)
        v["frac_of_mix_ceiling"] = round(c / v["ms_mean"], 4)
        at += c
    res["mix_ceiling"] = {"read_bytes": sum(v["read_bytes"] for v in phases.values()),
                          "written_bytes": sum(v["written_bytes"] for v in phases.values()),
                          "ms_at_probe_roofs": round(at, 4),
                          "GBps": round(res["bytes_per_step"] / (at * 1e-3) / 1e9, 1),
                          "frac": round(at / res["ms_per_step"], 4)}
    if probes.get("copy_GBps"):
        res["mix_ceiling"]["frac_of_copy_probe"] = round(res["GBps"] / probes["copy_GBps"], 4)
    res["roofline"]["frac_of_mix_ceiling"] = phases[res["roofline"]["phase"]]["frac_of_mix_ceiling"]
    # a bf16 expert-major dispatch of the fan-out probe's shape: its rate over
    # the probe's (the same mix of reads and writes with the simplest addresses)
    fv, fr, fk = FANOUT_SHAPE
    if (w is not None and probes.get("fanout_GBps") and "dispatch" in phases
            and w.quant == 0 and w.mode == 0 and (w.H * 2 // 16, w.N, w.K) == (fv, fr, fk)):
        phases["dispatch"]["frac_of_fanout_probe"] = round(
            phases["dispatch"]["GBps"] / probes["fanout_GBps"], 4)
        # and its combine over the fan-in probe's
        if probes.get("fanin_GBps") and "combine" in phases:
            phases["combine"]["frac_of_fanin_probe"] = round(
                phases["combine"]["GBps"] / probes["fanin_GBps"], 4)


def cpu_baseline(w, host, tokens_per_rank, min_seconds):
    """The plain C oracle on a bounded sample of the workload: the first
    `tokens_per_rank` tokens of every rank, layout + dispatch + combine,
    single-threaded, outputs preallocated and touched before timing.  The
    pass repeats until `min_seconds` have elapsed; the time per pass is
    reported."""
    from oracle import oracle as orc

    topk, x, wt = host
    T = tokens_per_rank
    topk = np.ascontiguousarray(topk[:, :T])
    x = np.ascontiguousarray(x[:, :T])
    wt = np.ascontiguousarray(wt[:, :T])
    p = orc.Problem(w.R, T, w.H, w.E, w.K, mode=w.mode, quant=w.quant)
    lay = orc.layout(p, topk)
    rows = lay.total_rows
    recv = np.ones((rows, w.H), np.uint16)
    out = np.ones((w.R, T, w.H), np.uint16)
    t0 = time.perf_counter()
    passes = 0
    ph = {"layout": 0.0, "dispatch": 0.0, "combine": 0.0}
    while True:
        ta = time.perf_counter()
        lay = orc.layout(p, topk)
        tb = time.perf_counter()
        orc.dispatch(p, x, topk, lay.send_pos, rows, out=(recv, None))
        tc = time.perf_counter()
        orc.combine(p, recv, wt, lay.send_pos, out=out)
        td = time.perf_counter()
        ph["layout"] += tb - ta
        ph["dispatch"] += tc - tb
        ph["combine"] += td - tc
        passes += 1
        total = td - t0
        if total >= min_seconds:
            break
    dt = total / passes
    sw = w.replace(T=T)
    nbytes = layout_bytes(sw, rows) + dispatch_bytes(sw) + combine_bytes(sw)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"first {T} of {w.T} tokens on each of the {w.R} ranks, layout + dispatch "
                      f"+ combine, {passes} passes in {total:.1f} s ({dt:.2f} s per pass), "
                      f"single thread",
            "tokens_per_s": round(w.R * T / dt, 1),
            "phase_s": {k: round(v / passes, 4) for k, v in ph.items()},
            "host": host_cpu()}


def host_cpu():
    """The host's logical CPU count and model (the oracle uses one of them)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default=",".join(DEFAULT_WORKLOADS),
                    help="comma-separated; the first is the headline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens per rank in the CPU-oracle sample (0 = all)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU-oracle pass repeats until this much time has elapsed")
    ap.add_argument("--fused", choices=["auto", "on", "off"], default="auto",
                    help="layout and dispatch in one call (ep_dispatch_fused): 'auto' uses it "
                         "for the workloads it measured faster on")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the without-layout and cold-cache passes (profiler runs, so "
                         "every launch of a kernel is a warm launch of the timed step)")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the bandwidth probes (and the mix-ceiling fractions)")
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
    names = [n for n in args.workloads.split(",") if n]
    head = None
    others = {}
    cpu = None
    for i, name in enumerate(names):
        w = inputs.WORKLOADS[name]
        fused = args.fused == "on" or (args.fused == "auto" and name in FUSED_WORKLOADS)
        r = Runner(w, torch, ep, inputs, keep_host=(i == 0 and not args.no_cpu), fused=fused)
        steps = args.steps if i == 0 else max(5, min(args.steps, 50))
        ms, res = r.report(steps, args.warmup, extra=not args.no_extra)
        if i == 0:
            head = (w, ms, res)
            if not args.no_cpu:
                host = r.host
        else:
            others[name] = res
        del r
        torch.cuda.empty_cache()
    if args.calib:
        a = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    # the probes run after the workloads, so that their 4 GiB streams do not
    # precede any timed step
    probes = None
    if not args.no_probes:
        log("[bench] bandwidth probes")
        probes = bandwidth_probes(torch)
        add_mix_ceiling(head[2], probes, head[0])
        for name, r_ in others.items():
            add_mix_ceiling(r_, probes, inputs.WORKLOADS[name])
    w, ms, res = head
    if not args.no_cpu and w.mode != ep.MODE_MESSAGES:
        cpu = cpu_baseline(w, host, min(args.cpu_tokens or w.T, w.T), args.cpu_seconds)

    quant_dtype = {0: "bf16", 1: "fp8-e4m3+bf16", 2: "fp8-e4m3+bf16"}[w.quant]
    line = {
        "metric": "dispatch+combine achieved HBM GB/s and tokens/s at 1 GPU (LL and normal)",
        "value": res["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": quant_dtype,
        "data": "synthetic",
        "config": {"workload": res["workload"], "ranks": w.R, "tokens_per_rank": w.T,
                   "hidden": w.H, "experts": w.E, "topk": w.K,
                   "bytes_per_step": res["bytes_per_step"]},
        "tokens_per_s": res["tokens_per_s"],
        "phases": res["phases"],
        "roofline": res["roofline"],
        "without_layout": res.get("without_layout"),
        "separate_expert_output": res.get("separate_expert_output"),
        "mix_ceiling": res.get("mix_ceiling"),
        "bandwidth_probes": probes,
        "workloads": others,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
