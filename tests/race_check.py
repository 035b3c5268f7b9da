"""Race check: every output of a whole step is bit-identical whether it
runs on the full chip or on a stream restricted to 8 compute units
(hipExtStreamCreateWithCUMask), which changes how blocks are scheduled and
interleaved.  Slot order is deterministic by construction and no output
depends on the order of atomics, so nothing may differ.  Covers the
chunked layout with normal bf16 dispatch and combine, the fused low-latency
FP8 call, rank-major FP8 with per-row metadata, and the message path
(packer, delivery, receiver).

Run as a child process by tests/test_gpu_race.py: a CU-masked stream needs
a hardware queue of its own, and a runtime that cannot provide one must not
leave the test session's process in a failed state.  Prints "race ok",
"race skip: ..." or the first difference, and exits 0 unless outputs
differ or a step fails."""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np
import torch

from combine_ep_get_layout_amd import ep, inputs
from gpu_util import DEV, h, problems, say

N, LL, MSG, RM = ep.MODE_NORMAL, ep.MODE_LOW_LATENCY, ep.MODE_MESSAGES, ep.MODE_RANK_MAJOR
QN, QF, QU = ep.QUANT_NONE, ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0
CASES = [
    # name, R, T, H, E, K, mode, quant, fused
    ("normal_bf16", 4, 2000, 256, 32, 4, N, QN, False),   # chunked layout (32k entries)
    ("ll_fp8_fused", 8, 128, 512, 64, 8, LL, QF, True),
    ("rank_major_ue8", 4, 1500, 512, 16, 6, RM, QU, False),
    ("messages", 8, 200, 256, 32, 4, MSG, QF, False),
]
# 32-bit words of CU mask bits: 8 neighbouring CUs
MASK = [0xFF] + [0] * 7


def masked_stream():
    """(library, stream) or None when the runtime cannot create one."""
    for name in ("libamdhip64.so", "libamdhip64.so.7"):
        try:
            hip = ctypes.CDLL(name)
            break
        except OSError:
            hip = None
    if hip is None:
        return None
    s = ctypes.c_void_p()
    mask = (ctypes.c_uint32 * len(MASK))(*MASK)
    st = hip.hipExtStreamCreateWithCUMask(ctypes.byref(s), ctypes.c_uint32(len(MASK)), mask)
    if st != 0:
        hip.hipGetLastError()
        return None
    return hip, s


def run(c, stream):
    """One whole step on `stream`; returns every output as numpy."""
    name, R, T, H, E, K, mode, quant, fused = c
    w = inputs.small(f"race_{name}", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=55,
                     region_bytes=4096)
    topk = inputs.masked_topk(w, inputs.gen_topk(w), 0.05, 0.05, seed=3)
    p, _ = problems(w)
    tk = torch.from_numpy(topk).to(DEV)
    x = torch.from_numpy(inputs.gen_x(w)).view(torch.bfloat16).to(DEV)
    wt = torch.from_numpy(inputs.gen_weights(w)).to(DEV)
    lay = ep.Layout(p)
    ws = ep.workspace(p)
    outs = {}
    torch.cuda.synchronize()
    if mode == MSG:
        ep.get_layout(p, tk, lay, ws, stream=stream)
        torch.cuda.synchronize()
        send_cap, desc_cap = ep.messages_capacity(p, h(lay.num_tokens_per_rank))
        msgs = ep.Messages(p, send_cap, desc_cap)
        msgs.send_arena.zero_()
        msgs.descriptors.zero_()  # slots past the count stay comparable
        torch.cuda.synchronize()
        ep.dispatch(p, lay, x, msgs=msgs, topk_idx=tk, topk_weights=wt, ws=ws, stream=stream)
        torch.cuda.synchronize()
        recv_cap = int(msgs.arena_base[1, -1].item())
        arena = torch.zeros(max(recv_cap, 16), dtype=torch.uint8, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        out, cnt, src = ep.unpack_buffers(p)
        out.x.zero_()
        out.scales.zero_()
        torch.cuda.synchronize()
        ep.messages_execute(p, msgs, arena[:recv_cap], err, stream=stream)
        ep.messages_unpack(p, msgs, arena[:recv_cap], lay.num_tokens_per_expert, out, cnt, src,
                           err, stream=stream)
        torch.cuda.synchronize()
        for k in ("send_arena", "table", "arena_base", "descriptors", "num_descriptors"):
            outs[k] = h(getattr(msgs, k))
        outs.update(arena=h(arena), rows=h(out.x), scales=h(out.scales), cnt=h(cnt), src=h(src),
                    msg_err=h(err))
    else:
        cap = ep.max_recv_rows(p)
        recv = ep.Recv(p, cap)
        recv.x.view(torch.uint8).zero_()
        if recv.scales is not None:
            recv.scales.view(torch.uint8).zero_()
        lay.recv_src_idx.fill_(-7)
        if recv.topk_idx is not None:  # rows past the filled ones stay comparable
            recv.topk_idx.fill_(0)
            recv.topk_weights.fill_(0)
        torch.cuda.synchronize()
        if fused:
            ep.dispatch_fused(p, tk, lay, x, recv, ws, stream=stream)
        else:
            ep.get_layout(p, tk, lay, ws, stream=stream)
            kw = dict(topk_idx=tk, topk_weights=wt) if mode == RM else {}
            ep.dispatch(p, lay, x, recv=recv, ws=ws, stream=stream, **kw)
        y = recv.x if quant == QN else torch.from_numpy(
            inputs.gen_y(w, cap)).view(torch.bfloat16).to(DEV)
        out = torch.empty((R, T, H), dtype=torch.bfloat16, device=DEV)
        torch.cuda.synchronize()
        ep.combine(p, lay, y, None if mode == RM else wt, out, stream=stream)
        torch.cuda.synchronize()
        outs.update(rows=h(recv.x.view(torch.uint8)), out=h(out.view(torch.int16)))
        if recv.scales is not None:
            outs["scales"] = h(recv.scales.view(torch.uint8))
        if recv.topk_idx is not None:
            outs.update(meta_idx=h(recv.topk_idx), meta_w=h(recv.topk_weights))
    for f in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank",
              "rank_prefix_matrix", "recv_tokens_per_expert", "expert_start", "rows_per_rank",
              "row_base", "send_pos", "send_head", "recv_src_idx", "err"):
        t = getattr(lay, f)
        if t is not None:
            outs[f] = h(t)
    return outs


def main() -> int:
    refs = {}
    for c in CASES:  # the full chip first, before any masked queue exists
        say("race", c[0], "full chip")
        refs[c[0]] = run(c, None)
        e = refs[c[0]]
        if int(e["err"][0]) not in (0, ep.DEVERR_LL_OVERFLOW) or int(e.get("msg_err", [0])[0]):
            print("race error words", c[0], int(e["err"][0]), flush=True)
            return 1
    ms = masked_stream()
    if ms is None:
        print("race skip: no CU-masked stream on this runtime", flush=True)
        return 0
    hip, s = ms
    try:
        stream = torch.cuda.ExternalStream(s.value)
        for c in CASES:
            say("race", c[0], "8 CUs")
            got, ref = run(c, stream), refs[c[0]]
            if got.keys() != ref.keys():
                print("race outputs differ in kind", c[0], flush=True)
                return 1
            for k in ref:
                if not np.array_equal(got[k], ref[k]):
                    print("race differs", c[0], k, flush=True)
                    return 1
    finally:
        torch.cuda.synchronize()
        hip.hipStreamDestroy(s)
    print("race ok", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
