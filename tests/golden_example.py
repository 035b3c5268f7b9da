"""The hand-worked routing example in tests/golden/layout_worked_example.json
(its derivation and page citations are in the file): expected layouts for
the normal (alignment 1 and 4), low-latency and rank-major modes, and exact
combine results with the identity expert.  Shared by the oracle test and
the GPU test; holds no method arithmetic beyond building the inputs the
file describes."""
from __future__ import annotations

import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
EX = json.load(open(os.path.join(HERE, "golden", "layout_worked_example.json")))
R, T, H, E, K = (EX["problem"][k] for k in ("R", "T", "H", "E", "K"))
TOPK = np.array(EX["topk_idx"], np.int32)
W = np.array(EX["topk_weights"], np.float32)
# mode name -> (mode number, expert alignment, fixture section)
MODES = {"normal_align1": (0, 1), "normal_align4": (0, 4), "low_latency": (1, 1),
         "rank_major": (3, 1)}
COMMON = ["num_tokens_per_expert", "num_tokens_per_rank", "is_token_in_rank",
          "rank_prefix_matrix", "recv_tokens_per_expert", "send_head"]
PER_MODE = ["expert_start", "rows_per_rank", "row_base", "send_pos"]


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that bf16 holds exactly."""
    b = np.ascontiguousarray(v, np.float32).view(np.uint32)
    assert not np.any(b & 0xFFFF), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def x_values() -> np.ndarray:
    tok = np.arange(R * T, dtype=np.float32).reshape(R, T, 1)
    ch = np.arange(H, dtype=np.float32).reshape(1, 1, H)
    return (tok + 1) * (ch + 1) / 4


def expected_out(section: str) -> np.ndarray:
    key = "rank_major_combine_scale" if section == "rank_major" else "combine_scale"
    scale = np.array(EX[key], np.float32).reshape(R, T, 1)
    return bf16_bits(x_values() * scale)


def expected_rows(section: str) -> dict[int, int]:
    """Receive row -> source token (s*T + t) for every filled row; -1 for
    alignment padding rows."""
    sec = EX[section]
    if "recv_src_idx" in sec:
        return {r: v for r, v in enumerate(sec["recv_src_idx"])}
    return {int(r): v for r, v in sec["filled_rows"].items()}


def check_layout(get, section: str):
    """`get(name)` returns the layout array of that name as numpy."""
    for f in COMMON:
        assert np.array_equal(get(f), np.array(EX[f])), f
    sec = EX[section]
    for f in PER_MODE:
        assert np.array_equal(get(f), np.array(sec[f])), (section, f)
    src = get("recv_src_idx")
    for r, v in expected_rows(section).items():
        assert int(src[r]) == v, (section, r)


# The hand-quantised FP8 group (tests/golden/e4m3_worked_example.json).
FP8 = json.load(open(os.path.join(HERE, "golden", "e4m3_worked_example.json")))


def fp8_input_and_codes():
    """x as bf16 bits [1][1][H] and the expected E4M3 codes [H]."""
    H8 = FP8["problem"]["H"]
    x = np.zeros(H8, np.float32)
    codes = np.zeros(H8, np.uint8)
    for ch in FP8["channels"]:
        x[ch["c"]] = ch["x"]
        codes[ch["c"]] = int(ch["code"], 16)
    return bf16_bits(x).reshape(1, 1, H8), codes


# The hand-worked messages (tests/golden/message_worked_example.json).
MSG = json.load(open(os.path.join(HERE, "golden", "message_worked_example.json")))


def message_inputs():
    """x [R][T][H] bf16 bits (each token the hand-quantised group), routing and
    weights as the file gives them, and the group's expected codes."""
    x1, codes = fp8_input_and_codes()
    pr = MSG["problem"]
    x = np.repeat(x1, pr["R"] * pr["T"], axis=0).reshape(pr["R"], pr["T"], pr["H"])
    return (x, np.array(MSG["topk_idx"], np.int32), np.array(MSG["topk_weights"], np.float32),
            codes)


def _u32(b, o):
    return int.from_bytes(bytes(b[o:o + 4]), "little")


def _be(b, o, n):
    return int.from_bytes(bytes(b[o:o + n]), "big")


def check_messages(table, arena_base, desc, num_desc, arena, codes):
    """Table, arena bases, every descriptor field and every message byte the
    file fixes, against the hand derivation."""
    assert np.array_equal(np.asarray(table).reshape(-1), np.array(MSG["table"]).reshape(-1))
    assert np.array_equal(np.asarray(arena_base).reshape(-1),
                          np.array(MSG["arena_base"]).reshape(-1))
    assert int(num_desc) == MSG["num_descriptors"]
    k = MSG["descriptor_constants"]
    for i, want in enumerate(MSG["descriptors"]):
        d = np.asarray(desc[i], np.uint8)
        w0, w1 = _be(d, 0, 4), _be(d, 4, 4)
        got = {"wqe": w0 >> 8, "qpn": w1 >> 8, "raddr": _be(d, 16, 8), "rkey": _be(d, 24, 4),
               "len": _be(d, 32, 4), "lkey": _be(d, 36, 4), "laddr": _be(d, 40, 8)}
        assert got == want, i
        assert w0 & 0xFF == k["opcode"] and w1 & 0xFF == k["ds"], i
        assert list(d[8:12]) == [0, 0, 0, k["cq_update"]], i
        assert not d[12:16].any() and not d[28:32].any() and not d[48:64].any(), i
    sec = MSG["sections"]
    for m in MSG["messages"]:
        b = np.asarray(arena[m["send_offset"]:m["send_offset"] + 224], np.uint8)
        assert [_u32(b, 4 * j) for j in range(4)] == m["header"]
        assert [_u32(b, 208 + 4 * j) for j in range(4)] == m["flag"]
        lo, hi = sec["codes"]
        assert np.array_equal(b[lo:hi], codes)
        lo, hi = sec["scales"]
        assert np.frombuffer(bytes(b[lo:lo + 4]), np.float32)[0] == np.float32(MSG["fp32_scale"])
        assert not b[lo + 4:hi].any()
        lo, hi = sec["weights"]
        assert np.frombuffer(bytes(b[lo:lo + 4]), np.float32)[0] == np.float32(m["weight"])
        assert not b[lo + 4:hi].any()
        lo, hi = sec["expert_ids"]
        assert _u32(b, lo) == m["expert_id"] and not b[lo + 4:hi].any()
        lo, hi = sec["src_token"]
        assert _u32(b, lo) == m["src_token"] and not b[lo + 4:hi].any()


def check_unpacked(recv_rows, scales, recv_count, recv_src_idx, codes):
    """The receiver's low-latency layout against the hand derivation."""
    u = MSG["unpacked"]
    assert [int(c) for c in np.asarray(recv_count).reshape(-1)] == u["recv_count"]
    for r, st in u["rows"].items():
        r = int(r)
        assert np.array_equal(np.asarray(recv_rows)[r], codes), r
        assert int(np.asarray(recv_src_idx).reshape(-1)[r]) == st, r
        si = u["scale_index"][str(r)]
        assert np.asarray(scales).reshape(-1)[si] == np.float32(MSG["fp32_scale"]), r


# Duplicate expert ids (tests/golden/layout_duplicates.json).
DUP = json.load(open(os.path.join(HERE, "golden", "layout_duplicates.json")))
DUP_MODES = {"normal": 0, "low_latency": 1, "rank_major": 3}


def dup_inputs():
    pr = DUP["problem"]
    R2, T2, H2 = pr["R"], pr["T"], pr["H"]
    tok = np.arange(R2 * T2, dtype=np.float32).reshape(R2, T2, 1)
    ch = np.arange(H2, dtype=np.float32).reshape(1, 1, H2)
    x = (tok + 1) * (ch + 1) / 4
    return (np.array(DUP["topk_idx"], np.int32), np.array(DUP["topk_weights"], np.float32),
            bf16_bits(x), x)


def check_dup_layout(get, section):
    for f in COMMON:
        assert np.array_equal(get(f), np.array(DUP[f])), f
    sec = DUP[section]
    assert np.array_equal(get("send_pos"), np.array(sec["send_pos"])), section
    if "row_base" in sec:
        assert np.array_equal(get("row_base"), np.array(sec["row_base"])), section
    src = get("recv_src_idx")
    rows = ({r: v for r, v in enumerate(sec["recv_src_idx"])} if "recv_src_idx" in sec
            else {int(r): v for r, v in sec["filled_rows"].items()})
    for r, v in rows.items():
        assert int(src[r]) == v, (section, r)
    return rows


def dup_expected_out(section, x):
    key = "rank_major_combine_scale" if section == "rank_major" else "combine_scale"
    pr = DUP["problem"]
    return bf16_bits(x * np.array(DUP[key], np.float32).reshape(pr["R"], pr["T"], 1))
