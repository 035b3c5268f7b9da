"""GPU sweep of the HIP path's E4M3 encoder over the bf16 input domain, bit
for bit against the oracle (whose encoder is pinned exhaustively to
PyTorch's float8_e4m3fn cast), through every kernel that quantises: the
normal and low-latency dispatch (separate and fused calls; one wavefront of
four pairs per lane at hidden 4096, eight wavefronts at 7168) and the
message packer, each with fp32 (amax / 448) and UE8M0 scales.

The token rows are built from 128-channel groups ("DeepEP" deep dive,
sec. 1.2: one scale per 128 channels):
  A. every bf16 magnitude up to 448, both signs, 127 to a group beside a
     channel of +-448: the scale is exactly 1 in both forms, so every code is
     the direct encoding of its input -- every E4M3 tie, subnormal and -0
     of the bf16 grid;
  B. every finite bf16 pattern (65,280), shuffled into groups: arbitrary
     group maxima, so the scaled inputs take every size, most of them
     subnormal or flushed to zero, and the 1e-4 amax floor binds;
  C. the normal values of A with their exponents shifted by k beside
     448 * 2^k, k from -100 to 100: power-of-two scales, so the codes are
     those of A again (k = -100 takes the amax floor instead).
"""
import numpy as np
import pytest
import torch

from combine_ep_get_layout_amd import ep, inputs
from oracle import oracle as orc
from gpu_util import DEV, h, say

pytestmark = pytest.mark.gpu

N, LL = ep.MODE_NORMAL, ep.MODE_LOW_LATENCY
QF, QU = ep.QUANT_FP8_F32, ep.QUANT_FP8_UE8M0
BF16_448 = 0x43E0  # 1.75 * 2^8


def sweep_groups() -> np.ndarray:
    """[n][128] uint16 bf16 groups (A, B, C above)."""
    rng = np.random.default_rng(4729)
    groups = []
    mags = np.arange(0, BF16_448 + 1, dtype=np.uint16)
    vals = np.concatenate([mags, mags | 0x8000])
    for j, i in enumerate(range(0, vals.size, 127)):  # A
        g = np.zeros(128, np.uint16)
        pos = (7 * j) % 128
        g[pos] = BF16_448 | (0x8000 if j % 2 else 0)
        chunk = vals[i:i + 127]
        g[np.delete(np.arange(128), pos)[:chunk.size]] = chunk
        groups.append(g)
    allp = np.arange(65536, dtype=np.uint32)
    finite = allp[(allp & 0x7F80) != 0x7F80].astype(np.uint16)  # B
    rng.shuffle(finite)
    groups.extend(finite.reshape(-1, 128))
    exp = (mags.astype(np.int32) >> 7) & 0xFF
    for k in (-100, -40, -9, -1, 3, 30, 100):  # C
        e2 = exp + k
        keep = (exp > 0) & (e2 >= 1) & (e2 <= 254)
        sh = ((e2[keep] << 7) | (mags[keep] & 0x7F)).astype(np.uint16)
        sv = np.concatenate([sh, sh | 0x8000])
        top = np.uint16(((135 + k) << 7) | 0x60)  # 448 * 2^k
        for j, i in enumerate(range(0, sv.size, 127)):
            g = np.zeros(128, np.uint16)
            pos = (11 * j + 5) % 128
            g[pos] = top
            chunk = sv[i:i + 127]
            g[np.delete(np.arange(128), pos)[:chunk.size]] = chunk
            groups.append(g)
    return np.stack(groups)


def sweep_x(R: int, T: int, H: int) -> np.ndarray:
    """[R][T][H] bf16 rows holding every sweep group at least once."""
    g = sweep_groups()
    G = H // 128
    need = R * T * G
    assert need >= g.shape[0], (need, g.shape[0])
    return g[np.arange(need) % g.shape[0]].reshape(R, T, H)


def run_dispatch(p, topk, x, fused):
    tk = torch.from_numpy(topk).to(DEV)
    xg = torch.from_numpy(x).view(torch.bfloat16).to(DEV)
    cap = ep.max_recv_rows(p)
    lay = ep.Layout(p)
    recv = ep.Recv(p, cap)
    recv.x.fill_(0x33)
    recv.scales.view(torch.uint8).fill_(0x33)
    ws = ep.workspace(p)
    if fused:
        ep.dispatch_fused(p, tk, lay, xg, recv, ws)
    else:
        ep.get_layout(p, tk, lay, ws)
        ep.dispatch(p, lay, xg, recv=recv, ws=ws)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    return recv, cap


# mode, hidden, tokens per rank (the fused kernels run above 6,144 entries)
SHAPES = [(N, 4096, 400), (LL, 7168, 400), (N, 1024, 1600), (LL, 2048, 800)]


@pytest.mark.parametrize("quant", [QF, QU], ids=["f32", "ue8m0"])
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{'ll' if s[0] else 'normal'}_h{s[1]}" for s in SHAPES])
def test_encoder_sweep_dispatch(shape, fused, quant):
    mode, H, T = shape
    R, E, K = 2, 16, 8
    say("e4m3 sweep", mode, H, T, fused, quant)
    x = sweep_x(R, T, H)
    w = inputs.small("e4m3_sweep", R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=31)
    topk = inputs.gen_topk(w)
    p = ep.Problem(R, T, H, E, K, mode=mode, quant=quant)
    po = orc.Problem(R, T, H, E, K, mode=mode, quant=quant)
    recv, cap = run_dispatch(p, topk, x, fused)
    ol = orc.layout(po, topk)
    err, ocodes, oscales = orc.dispatch(po, x, topk, ol.send_pos, cap)
    assert err == 0
    rows = np.unique(ol.send_pos[ol.send_pos >= 0])
    assert np.array_equal(h(recv.x)[rows], ocodes[rows])
    G, RT = H // 128, R * T
    g = np.arange(G)
    si = ((rows[:, None] // RT * G + g) * RT + rows[:, None] % RT if mode == LL
          else g[None, :] * cap + rows[:, None]).reshape(-1)
    assert np.array_equal(h(recv.scales)[si], oscales[si])


@pytest.mark.parametrize("quant", [QF, QU], ids=["f32", "ue8m0"])
def test_encoder_sweep_messages(quant):
    """The message packer's encoder (one wavefront of seven pairs per lane at
    hidden 7168): every message byte against the oracle's."""
    R, T, H, E, K = 2, 200, 7168, 8, 4
    x = sweep_x(R, T, H)
    w = inputs.small("e4m3_sweep_msg", R=R, T=T, H=H, E=E, K=K, mode=ep.MODE_MESSAGES,
                     quant=quant, seed=32)
    topk, wt = inputs.gen_topk(w), inputs.gen_weights(w)
    kw = dict(mode=ep.MODE_MESSAGES, quant=quant, region_bytes=1 << 20, epoch=3)
    p, po = ep.Problem(R, T, H, E, K, **kw), orc.Problem(R, T, H, E, K, **kw)
    tk = torch.from_numpy(topk).to(DEV)
    lay = ep.Layout(p)
    ws = ep.workspace(p)
    ep.get_layout(p, tk, lay, ws)
    torch.cuda.synchronize()
    send_cap, desc_cap = ep.messages_capacity(p, h(lay.num_tokens_per_rank))
    msgs = ep.Messages(p, send_cap, desc_cap)
    ep.dispatch(p, lay, torch.from_numpy(x).view(torch.bfloat16).to(DEV), msgs=msgs,
                topk_idx=tk, topk_weights=torch.from_numpy(wt).to(DEV), ws=ws)
    torch.cuda.synchronize()
    assert int(h(lay.err)[0]) == 0
    om = orc.messages(po, x, topk, wt, send_cap, desc_cap)
    assert om.err == 0
    table = h(msgs.table)
    assert np.array_equal(table, om.table)
    arena = h(msgs.send_arena)
    for s in range(R):
        for d in range(R):
            off, _, reg = table[s, d, :3]
            if reg:
                assert np.array_equal(arena[off:off + reg], om.send_arena[off:off + reg]), (s, d)
