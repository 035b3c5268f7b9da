"""GPU parity of message delivery (ep_messages_execute) and the receiver
(ep_messages_unpack) against the oracle, through the C ABI.

Small problems: the whole receive arena and every unpacked buffer (rows,
scales, recv_src_idx, recv_count) are compared byte for byte with the
oracle, both sides starting from the same fill values; the unpacked layout
also equals the GPU's own low-latency dispatch of the same routing.
Corrupted flags, headers and descriptors are rejected identically.
The 64-rank message workload: the whole receive arena against the oracle,
and sampled unpacked tokens against the oracle's quantisation of each
token on its own."""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import DEV, gpu_layout, h, problems, say, sweep_cases

pytestmark = pytest.mark.gpu

CASES = [
    # name, R, T, H, E, K, quant, region bytes, masked fraction, duplicate fraction
    ("r1", 1, 9, 128, 4, 2, ep.QUANT_FP8_F32, 256, 0.0, 0.0),
    ("r2_small_regions", 2, 17, 256, 8, 3, ep.QUANT_FP8_F32, 64, 0.2, 0.0),
    ("r3_bf16", 3, 12, 128, 6, 2, ep.QUANT_NONE, 4096, 0.0, 0.0),
    ("r4_ue8m0", 4, 20, 256, 16, 4, ep.QUANT_FP8_UE8M0, 512, 0.1, 0.3),
    ("r5", 5, 7, 384, 10, 5, ep.QUANT_FP8_F32, 2 << 20, 0.0, 0.0),
    ("r8_wide", 8, 40, 1024, 64, 8, ep.QUANT_FP8_F32, 8192, 0.05, 0.0),
    ("r16_many_local", 16, 24, 256, 512, 6, ep.QUANT_FP8_F32, 1024, 0.0, 0.0),
    ("r4_bf16_dups", 4, 33, 128, 8, 8, ep.QUANT_NONE, 128, 0.1, 0.4),
    ("r256", 256, 2, 128, 256, 4, ep.QUANT_FP8_F32, 4096, 0.0, 0.0),  # the rank limit
    # a 1,240,832-byte arena in 38,776 regions of 32 bytes: region indices
    # near the 16-bit key limit, one descriptor per 32 bytes
    ("r1_1mib_arena_32b_regions", 1, 600, 1024, 2, 2, ep.QUANT_NONE, 32, 0.0, 0.0),
    # messages of up to 2,400 entries: the receiver ranks and copies them
    # in two segments of at most 2,048
    ("r2_two_segments", 2, 300, 256, 8, 8, ep.QUANT_FP8_UE8M0, 4096, 0.1, 0.0),
    # 128 scale groups per token: more than one per lane of a wavefront
    ("r2_h16384_f32", 2, 6, 16384, 4, 2, ep.QUANT_FP8_F32, 2 << 20, 0.0, 0.0),
    ("r2_h16384_ue8m0", 2, 6, 16384, 4, 2, ep.QUANT_FP8_UE8M0, 2 << 20, 0.0, 0.5),
]
FILL = 0x5C


def run_gpu(w, p, topk, x, wt, publish_batch=0, spin_limit=0):
    """Layout, pack, execute (flags published every `publish_batch`
    messages, 0: after a second launch) and unpack (polling each flag up to
    `spin_limit` times) on the GPU; returns every buffer."""
    gl, ws = gpu_layout(p, topk)
    send_cap, desc_cap = ep.messages_capacity(p, h(gl.num_tokens_per_rank))
    msgs = ep.Messages(p, send_cap, desc_cap)
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), msgs=msgs,
                topk_idx=torch.from_numpy(topk).to(DEV), topk_weights=torch.from_numpy(wt).to(DEV),
                ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == 0
    recv_cap = int(h(msgs.arena_base)[1, -1])
    arena = torch.full((recv_cap + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_execute(p, msgs, arena[:recv_cap], err, publish_batch=publish_batch)
    out, cnt, src = ep.unpack_buffers(p)
    out.x.view(torch.uint8).fill_(FILL)
    if out.scales is not None:
        out.scales.view(torch.uint8).fill_(FILL)
    ep.messages_unpack(p, msgs, arena[:recv_cap], gl.num_tokens_per_expert, out, cnt, src, err,
                       spin_limit=spin_limit)
    torch.cuda.synchronize()
    return gl, ws, msgs, arena, recv_cap, out, cnt, src, err


def oracle_side(w, po, topk, x, wt, send_cap, desc_cap, recv_cap, cnt_expert):
    om = orc.messages(po, x, topk, wt, send_cap, desc_cap)
    assert om.err == 0
    arena = np.full(recv_cap + 64, 0xA5, np.uint8)
    e1, arena = orc.messages_execute(po, om, recv_cap, arena)
    u = orc.messages_unpack(po, arena[:recv_cap], om.table, cnt_expert, fill_codes=FILL)
    return om, arena, e1, u


def compare_unpacked(w, out, cnt, src, u):
    rows = w.E * w.R * w.T
    g = h(out.x.view(torch.uint16) if w.quant == ep.QUANT_NONE else out.x)[:rows]
    assert np.array_equal(g, u.recv)
    if w.quant != ep.QUANT_NONE:
        gs = h(out.scales.view(torch.uint8))[: u.scales.view(np.uint8).size]
        assert np.array_equal(gs, u.scales.view(np.uint8))
    assert np.array_equal(h(cnt), u.recv_count)
    assert np.array_equal(h(src)[:rows], u.recv_src_idx)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_execute_and_unpack_match_oracle(case):
    check_case(case)


def check_case(case, publish_batch=0, spin_limit=0, **kw):
    name, R, T, H, E, K, quant, rb, mfrac, dfrac = case
    say("receive", name, publish_batch, spin_limit)
    w = inputs.small(f"recv_{name}", R=R, T=T, H=H, E=E, K=K, mode=ep.MODE_MESSAGES, quant=quant,
                     seed=61, region_bytes=rb, epoch=5, **kw)
    topk = inputs.gen_topk(w)
    if mfrac or dfrac:
        topk = inputs.masked_topk(w, topk, mfrac, dfrac, seed=3)
    x, wt = inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    gl, ws, msgs, arena, recv_cap, out, cnt, src, err = run_gpu(w, p, topk, x, wt, publish_batch,
                                                                spin_limit)
    om, oarena, e1, u = oracle_side(w, po, topk, x, wt, msgs.send_capacity, msgs.desc_capacity,
                                    recv_cap, h(gl.num_tokens_per_expert))
    assert e1 == 0
    assert int(h(err)[0]) == u.err
    assert np.array_equal(h(arena), oarena)  # the whole arena, padding and canary tail included
    compare_unpacked(w, out, cnt, src, u)
    # the unpacked layout is what low-latency dispatch of the same routing stores
    pl = ep.Problem(R, T, H, E, K, mode=ep.MODE_LOW_LATENCY, quant=quant)
    ll, lws = gpu_layout(pl, topk)
    rl = ep.Recv(pl, E * R * T)
    ep.dispatch(pl, ll, torch.from_numpy(x).view(torch.bfloat16).to(DEV), recv=rl, ws=lws)
    torch.cuda.synchronize()
    sp = h(ll.send_pos)
    rows = torch.from_numpy(np.unique(sp[sp >= 0]).astype(np.int64)).to(DEV)
    assert torch.equal(out.x[rows], rl.x[rows])
    assert torch.equal(src[rows], ll.recv_src_idx[rows])
    assert torch.equal(cnt, ll.recv_tokens_per_expert)
    assert int(h(ll.err)[0]) == int(h(err)[0])
    return h(msgs.arena_base)


BATCH_CASES = [c for c in CASES if c[0] in ("r2_small_regions", "r4_ue8m0", "r8_wide", "r16_many_local",
                                            "r4_bf16_dups", "r256")]


@pytest.mark.parametrize("batch", [1, 2, 4, 32])
@pytest.mark.parametrize("case", BATCH_CASES, ids=[c[0] for c in BATCH_CASES])
def test_batched_publication_delivers_the_same_bytes(case, batch):
    """Flags published every 1, 2, 4 or 32 messages per workgroup, in one
    launch: the receive arena and the unpacked layout equal the oracle's
    (which delivers in no particular order) byte for byte, and the receiver
    polls each flag (at most 1,000 times) before checking it."""
    check_case(case, publish_batch=batch, spin_limit=1000)


def draw(i):
    """A random message-mode case and publication batch (0: the two-launch
    delivery): ranks, experts, top-k, tokens, payload format, hidden size,
    region size (down to 64 bytes, so puts split), masked and duplicate ids."""
    g = np.random.default_rng(9100 + i)
    R = int(g.choice([1, 2, 3, 4, 5, 8, 16]))
    E = R * int(g.integers(1, 9))
    K = int(g.integers(1, min(E, 9) + 1))
    T = int(g.choice([1, 7, 40, 100]))
    quant = int(g.choice([ep.QUANT_NONE, ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0]))
    H = int(8 * g.integers(1, 100)) if quant == ep.QUANT_NONE else int(128 * g.integers(1, 9))
    rb = int(g.choice([64, 256, 4096, 2 << 20]))
    case = (f"fuzz{i}", R, T, H, E, K, quant, rb, float(g.choice([0.0, 0.2])),
            float(g.choice([0.0, 0.3])) if K > 1 else 0.0)
    return case, int(g.choice([0, 0, 1, 4, 32]))


FUZZ = [draw(i) for i in range(sweep_cases(12))]


@pytest.mark.parametrize("i", range(len(FUZZ)))
def test_random_cases_match_oracle(i):
    case, batch = FUZZ[i]
    check_case(case, publish_batch=batch, spin_limit=1000 if batch else 0)


def test_polling_receiver_gives_up_on_a_missing_flag():
    """A message whose flag never shows the epoch: the receiver polls it 16
    times, gives up with the message bit and leaves that message's rows
    untouched; every other message is unpacked as the oracle does."""
    w = inputs.small("recv_spin", R=4, T=20, H=256, E=16, K=4, mode=ep.MODE_MESSAGES,
                     quant=ep.QUANT_FP8_F32, seed=73, region_bytes=512, epoch=9)
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    gl, ws, msgs, arena, recv_cap, out, cnt, src, err = run_gpu(w, p, topk, x, wt, 4, 16)
    assert int(h(err)[0]) == 0
    table = h(msgs.table)
    t21 = table[2, 1]
    assert t21[3] > 0
    bad = arena.clone()
    bad[int(t21[1] + 16 + t21[4])] ^= 0x40  # the flag's epoch word never arrives
    out2, cnt2, src2 = ep.unpack_buffers(p)
    out2.x.fill_(FILL)
    out2.scales.view(torch.uint8).fill_(FILL)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_unpack(p, msgs, bad[:recv_cap], gl.num_tokens_per_expert, out2, cnt2, src2, err2,
                       spin_limit=16)
    torch.cuda.synchronize()
    u = orc.messages_unpack(po, h(bad)[:recv_cap], table, h(gl.num_tokens_per_expert),
                            fill_codes=FILL)
    assert u.err == orc.ERR_MESSAGE and int(h(err2)[0]) == ep.DEVERR_MESSAGE
    compare_unpacked(w, out2, cnt2, src2, u)


@pytest.mark.parametrize("alpha,skewed", [(None, False), (2.5, True)], ids=["uniform", "zipf"])
def test_unpack_block_orders_32_ranks(alpha, skewed):
    """32 ranks: the receiver's block order follows the receive loads (one
    die per destination when balanced, runs of 16 sources per die when one
    destination receives more than twice the mean); both orders give the
    oracle's bytes."""
    kw = {} if alpha is None else {"routing": "zipf", "alpha": alpha}
    base = check_case((f"r32_{'zipf' if alpha else 'uniform'}", 32, 24, 256, 64, 4,
                       ep.QUANT_FP8_F32, 2048, 0.0, 0.0), **kw)
    sizes = np.diff(base[1])
    assert (sizes.max() * 32 > 2 * base[1][-1]) == skewed


def test_unpack_rejects_corrupt_flag_and_header_like_the_oracle():
    w = inputs.small("recv_bad", R=4, T=20, H=256, E=16, K=4, mode=ep.MODE_MESSAGES,
                     quant=ep.QUANT_FP8_F32, seed=71, region_bytes=512, epoch=9)
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    gl, ws, msgs, arena, recv_cap, out, cnt, src, err = run_gpu(w, p, topk, x, wt)
    assert int(h(err)[0]) == 0
    table = h(msgs.table)
    t12, t30 = table[1, 2], table[3, 0]
    assert t12[3] > 0 and t30[3] > 0
    bad = arena.clone()
    bad[int(t12[1] + 16 + t12[4])] ^= 1  # stale flag
    bad[int(t30[1] + 8)] ^= 1            # wrong token count in the header
    out2, cnt2, src2 = ep.unpack_buffers(p)
    out2.x.fill_(FILL)
    out2.scales.view(torch.uint8).fill_(FILL)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_unpack(p, msgs, bad[:recv_cap], gl.num_tokens_per_expert, out2, cnt2, src2, err2)
    torch.cuda.synchronize()
    u = orc.messages_unpack(po, h(bad)[:recv_cap], table, h(gl.num_tokens_per_expert),
                            fill_codes=FILL)
    assert u.err == orc.ERR_MESSAGE and int(h(err2)[0]) == ep.DEVERR_MESSAGE
    compare_unpacked(w, out2, cnt2, src2, u)


def test_execute_rejects_corrupt_descriptor_like_the_oracle():
    w = inputs.small("recv_desc", R=2, T=17, H=256, E=8, K=3, mode=ep.MODE_MESSAGES,
                     quant=ep.QUANT_FP8_F32, seed=72, region_bytes=64, epoch=3)
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    gl, ws, msgs, arena, recv_cap, out, cnt, src, err = run_gpu(w, p, topk, x, wt)
    nd = int(h(msgs.num_descriptors)[0])
    msgs.descriptors[1, 36] = 0x7F  # source rank out of range (a payload piece)
    arena2 = torch.full((recv_cap + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    err2 = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_execute(p, msgs, arena2[:recv_cap], err2)
    torch.cuda.synchronize()
    om = orc.Messages(0, h(msgs.send_arena), h(msgs.table), h(msgs.arena_base),
                      h(msgs.descriptors)[:nd], nd)
    e, oarena = orc.messages_execute(po, om, recv_cap, np.full(recv_cap + 64, 0xA5, np.uint8))
    assert e == orc.ERR_MESSAGE and int(h(err2)[0]) == ep.DEVERR_MESSAGE
    assert np.array_equal(h(arena2), oarena)


def test_region_index_past_16_bits_is_rejected_like_the_oracle():
    """The same 1,240,832-byte arena in 16-byte regions (77,552 of them): a
    key's 16-bit region index cannot name the pieces past region 65535, so
    the packer writes them with all-ones keys and raises the capacity bit;
    delivery rejects them (no such rank: the message bit) and leaves their
    bytes, the flag among them, undelivered; the receiver then finds no
    flag and skips the message.  Every descriptor, the error words, the
    receive arena and the unpacked buffers equal the oracle's."""
    R, T, H, E, K, rb = 1, 600, 1024, 2, 2, 16
    w = inputs.small("recv_rb16", R=R, T=T, H=H, E=E, K=K, mode=ep.MODE_MESSAGES,
                     quant=ep.QUANT_NONE, seed=61, region_bytes=rb, epoch=5)
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    say("receive: 16-byte regions over 1 MiB")
    gl, ws = gpu_layout(p, topk)
    send_cap, desc_cap = ep.messages_capacity(p, h(gl.num_tokens_per_rank))
    assert send_cap == 1240832 and desc_cap == 1240832 // 16
    msgs = ep.Messages(p, send_cap, desc_cap)
    ep.dispatch(p, gl, torch.from_numpy(x).view(torch.bfloat16).to(DEV), msgs=msgs,
                topk_idx=torch.from_numpy(topk).to(DEV), topk_weights=torch.from_numpy(wt).to(DEV),
                ws=ws)
    torch.cuda.synchronize()
    assert int(h(gl.err)[0]) == ep.DEVERR_CAPACITY
    om = orc.messages(po, x, topk, wt, send_cap, desc_cap)
    assert om.err == orc.ERR_CAPACITY and om.num_desc == desc_cap
    assert np.array_equal(h(msgs.descriptors), om.desc)
    assert np.array_equal(h(msgs.send_arena), om.send_arena)
    arena = torch.full((send_cap + 64,), 0xA5, dtype=torch.uint8, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    ep.messages_execute(p, msgs, arena[:send_cap], err)
    out, cnt, src = ep.unpack_buffers(p)
    out.x.view(torch.uint8).fill_(FILL)
    ep.messages_unpack(p, msgs, arena[:send_cap], gl.num_tokens_per_expert, out, cnt, src, err)
    torch.cuda.synchronize()
    e1, oarena = orc.messages_execute(po, om, send_cap, np.full(send_cap + 64, 0xA5, np.uint8))
    assert e1 == orc.ERR_MESSAGE
    u = orc.messages_unpack(po, oarena[:send_cap], om.table, h(gl.num_tokens_per_expert),
                            fill_codes=FILL)
    assert int(h(err)[0]) == (e1 | u.err) == ep.DEVERR_MESSAGE
    assert np.array_equal(h(arena), oarena)
    compare_unpacked(w, out, cnt, src, u)


def test_workload_messages_delivery_and_unpack():
    """R64 T256 H7168 E256 top-8 (0.94 GB of messages): the whole receive
    arena against the oracle; recv_count and recv_src_idx of every row
    against the oracle's low-latency layout; codes and scales of sampled
    tokens against the oracle's quantisation of each token alone."""
    w = inputs.WORKLOADS["messages"]
    topk, x, wt = inputs.gen_topk(w), inputs.gen_x(w), inputs.gen_weights(w)
    p, po = problems(w)
    say("receive workload: GPU")
    gl, ws, msgs, arena, recv_cap, out, cnt, src, err = run_gpu(w, p, topk, x, wt)
    assert int(h(err)[0]) == 0
    say("receive workload: oracle pack + execute")
    om = orc.messages(po, x, topk, wt, msgs.send_capacity, msgs.desc_capacity)
    _, oarena = orc.messages_execute(po, om, recv_cap, np.full(recv_cap + 64, 0xA5, np.uint8))
    assert np.array_equal(h(arena), oarena)
    del oarena
    pl = orc.Problem(w.R, w.T, w.H, w.E, w.K, mode=orc.MODE_LL, quant=w.quant)
    ol = orc.layout(pl, topk)
    assert np.array_equal(h(cnt), ol.recv_tokens_per_expert)
    g_src = h(src)
    filled = ol.recv_src_idx >= 0
    assert np.array_equal(g_src[filled], ol.recv_src_idx[filled])
    assert (g_src[~filled] == -1).all()
    # sampled tokens: every routed row of the token holds its codes and scales
    rng = np.random.default_rng(5)
    RT, G = w.R * w.T, w.G
    p1 = orc.Problem(1, 1, w.H, 1, 1, quant=w.quant)
    for st in rng.choice(w.R * w.T, 48, replace=False):
        s, t = divmod(int(st), w.T)
        _, codes, scales = orc.dispatch(p1, x[s, t][None, None], np.zeros((1, 1, 1), np.int32),
                                        np.zeros((1, 1, 1), np.int32), 1)
        for r in ol.send_pos[s, t]:
            if r < 0:
                continue
            e, pos = divmod(int(r), RT)
            assert np.array_equal(h(out.x[r]), codes[0])
            gi = torch.arange(G, device=DEV) * RT + e * G * RT + pos
            assert np.array_equal(h(out.scales[gi]), scales[:G])
