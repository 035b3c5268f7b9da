"""NumPy front-end for the plain C oracle (``ep_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use this module; the product library never imports it.
It shares no code with the HIP implementation.  Every function returns
fresh NumPy arrays computed by the single-threaded C routines; see
``ep_oracle.h`` for the passages each routine follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ep_oracle.c")
_LIB = os.path.join(_HERE, "libep_oracle.so")

MODE_NORMAL, MODE_LL, MODE_MSG, MODE_RANK = 0, 1, 2, 3
Q_NONE, Q_FP8_F32, Q_FP8_UE8M0 = 0, 1, 2
ERR_TOPK_RANGE, ERR_LL_OVERFLOW, ERR_CAPACITY, ERR_MESSAGE = 1, 2, 4, 8


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "ep_oracle.h"))
    ):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


class _Problem(ctypes.Structure):
    _fields_ = [
        ("R", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("align", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("quant", ctypes.c_int32),
        ("region_bytes", ctypes.c_int64), ("epoch", ctypes.c_uint32),
        ("pad_", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.POINTER(_Problem)
        vp = ctypes.c_void_p
        i64 = ctypes.c_int64
        _lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
        _lib.orc_e4m3_encode.restype = ctypes.c_uint8
        _lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        _lib.orc_e4m3_decode.restype = ctypes.c_float
        _lib.orc_bf16_from_double.argtypes = [ctypes.c_double]
        _lib.orc_bf16_from_double.restype = ctypes.c_uint16
        _lib.orc_fp8_scale_f32.argtypes = [ctypes.c_float]
        _lib.orc_fp8_scale_f32.restype = ctypes.c_float
        _lib.orc_fp8_scale_ue8m0.argtypes = [ctypes.c_float]
        _lib.orc_fp8_scale_ue8m0.restype = ctypes.c_uint8
        _lib.orc_e4m3_encode_array.argtypes = [vp, vp, i64]
        _lib.orc_e4m3_encode_array.restype = None
        _lib.orc_recv_rows.argtypes = [P, vp]
        _lib.orc_recv_rows.restype = i64
        _lib.orc_layout.argtypes = [P, vp] + [vp] * 11 + [i64]
        _lib.orc_layout.restype = ctypes.c_int
        _lib.orc_dispatch.argtypes = [P, vp, vp, vp, vp, vp, i64]
        _lib.orc_dispatch.restype = ctypes.c_int
        _lib.orc_dequant_rows.argtypes = [P, vp, vp, i64, vp, i64, vp]
        _lib.orc_dequant_rows.restype = None
        _lib.orc_combine.argtypes = [P, vp, i64, vp, vp, vp, i64, vp]
        _lib.orc_combine.restype = ctypes.c_int
        _lib.orc_msg_body_bytes.argtypes = [P, i64, vp]
        _lib.orc_msg_body_bytes.restype = i64
        _lib.orc_messages.argtypes = [P, vp, vp, vp, vp, i64, vp, vp, vp, i64, vp]
        _lib.orc_messages.restype = ctypes.c_int
        _lib.orc_rank_topk.argtypes = [P, vp, vp, vp, i64, vp, vp]
        _lib.orc_rank_topk.restype = ctypes.c_int
        _lib.orc_messages_execute.argtypes = [P, vp, i64, vp, vp, i64, vp, i64]
        _lib.orc_messages_execute.restype = ctypes.c_int
        _lib.orc_messages_unpack.argtypes = [P, vp, i64, vp, vp, vp, vp, vp, vp]
        _lib.orc_messages_unpack.restype = ctypes.c_int
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


@dataclass
class Problem:
    R: int
    T: int
    H: int
    E: int
    K: int
    align: int = 1
    mode: int = MODE_NORMAL
    quant: int = Q_NONE
    region_bytes: int = 2 << 20
    epoch: int = 1

    def c(self) -> _Problem:
        return _Problem(self.R, self.T, self.H, self.E, self.K, self.align, self.mode,
                        self.quant, self.region_bytes, self.epoch, 0)

    @property
    def L(self) -> int:
        return self.E // self.R

    @property
    def G(self) -> int:
        return self.H // 128


# ---------------------------------------------------------------- codecs
def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def e4m3_decode(code: int) -> float:
    return float(lib().orc_e4m3_decode(int(code)))


def bf16_from_double(v: float) -> int:
    return int(lib().orc_bf16_from_double(float(v)))


def fp8_scale_f32(amax: float) -> float:
    return float(lib().orc_fp8_scale_f32(float(amax)))


def fp8_scale_ue8m0(amax: float) -> int:
    return int(lib().orc_fp8_scale_ue8m0(float(amax)))


# ---------------------------------------------------------------- layout
@dataclass
class Layout:
    err: int
    num_tokens_per_rank: np.ndarray      # [R][R]
    num_tokens_per_expert: np.ndarray    # [R][E]
    is_token_in_rank: np.ndarray         # [R][T][R] u8
    rank_prefix_matrix: np.ndarray       # [R][R]
    recv_tokens_per_expert: np.ndarray   # [E]
    expert_start: np.ndarray             # [E]
    rows_per_rank: np.ndarray            # [R]
    row_base: np.ndarray                 # [R+1]
    send_pos: np.ndarray                 # [R][T][K]
    send_head: np.ndarray                # [R][T][R]
    recv_src_idx: np.ndarray             # [rows]

    @property
    def total_rows(self) -> int:
        return int(self.row_base[-1])


def recv_rows(p: Problem, topk: np.ndarray) -> int:
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    return int(lib().orc_recv_rows(ctypes.byref(p.c()), _ptr(topk)))


def layout(p: Problem, topk: np.ndarray, recv_cap: int | None = None) -> Layout:
    R, T, E, K = p.R, p.T, p.E, p.K
    topk = np.ascontiguousarray(topk, dtype=np.int32).reshape(R, T, K)
    if recv_cap is None:
        recv_cap = recv_rows(p, topk)
    o = dict(
        num_tokens_per_rank=np.zeros((R, R), np.int32),
        num_tokens_per_expert=np.zeros((R, E), np.int32),
        is_token_in_rank=np.zeros((R, T, R), np.uint8),
        rank_prefix_matrix=np.zeros((R, R), np.int32),
        recv_tokens_per_expert=np.zeros(E, np.int32),
        expert_start=np.zeros(E, np.int32),
        rows_per_rank=np.zeros(R, np.int32),
        row_base=np.zeros(R + 1, np.int32),
        send_pos=np.zeros((R, T, K), np.int32),
        send_head=np.zeros((R, T, R), np.int32),
        recv_src_idx=np.zeros(max(recv_cap, 1), np.int32),
    )
    err = lib().orc_layout(
        ctypes.byref(p.c()), _ptr(topk), _ptr(o["num_tokens_per_rank"]),
        _ptr(o["num_tokens_per_expert"]), _ptr(o["is_token_in_rank"]),
        _ptr(o["rank_prefix_matrix"]), _ptr(o["recv_tokens_per_expert"]),
        _ptr(o["expert_start"]), _ptr(o["rows_per_rank"]), _ptr(o["row_base"]),
        _ptr(o["send_pos"]), _ptr(o["send_head"]), _ptr(o["recv_src_idx"]), recv_cap,
    )
    o["recv_src_idx"] = o["recv_src_idx"][:recv_cap]
    return Layout(err=err, **o)


def rank_topk(p: Problem, topk: np.ndarray, w: np.ndarray, send_pos: np.ndarray, cap: int):
    """Rank-major receive metadata: (err, recv_topk_idx [cap][K] (-1 fill),
    recv_topk_weights [cap][K] (0 fill))."""
    K = p.K
    idx = np.full((max(cap, 1), K), -1, np.int32)
    wts = np.zeros((max(cap, 1), K), np.float32)
    err = lib().orc_rank_topk(ctypes.byref(p.c()), _ptr(np.ascontiguousarray(topk, np.int32)),
                              _ptr(np.ascontiguousarray(w, np.float32)),
                              _ptr(np.ascontiguousarray(send_pos, np.int32)), cap, _ptr(idx),
                              _ptr(wts))
    return err, idx[:cap], wts[:cap]


# ---------------------------------------------------------------- dispatch
def dispatch(p: Problem, x: np.ndarray, topk: np.ndarray, send_pos: np.ndarray, cap: int,
             out=None):
    """Returns (err, recv, scales).  recv: uint16 [cap][H] (bf16 bits) or
    uint8 [cap][H] codes; scales: None, float32 or uint8, column-major.
    ``out`` = (recv, scales) preallocated by the caller, else fresh zeros."""
    R, T, H, K, G = p.R, p.T, p.H, p.K, p.G
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(R, T, H)
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    send_pos = np.ascontiguousarray(send_pos, dtype=np.int32)
    if out is not None:
        recv, scales = out
    elif p.quant == Q_NONE:
        recv = np.zeros((cap, H), np.uint16)
        scales = None
    else:
        recv = np.zeros((cap, H), np.uint8)
        n_sc = G * (p.R * p.T * p.E if p.mode == MODE_LL else cap)
        scales = np.zeros(n_sc, np.float32 if p.quant == Q_FP8_F32 else np.uint8)
    err = lib().orc_dispatch(ctypes.byref(p.c()), _ptr(x), _ptr(topk), _ptr(send_pos),
                             _ptr(recv), _ptr(scales), cap)
    return err, recv, scales


def dequant_rows(p: Problem, codes: np.ndarray, scales: np.ndarray, cap: int,
                 rows: np.ndarray) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    y = np.zeros((rows.size, p.H), np.uint16)
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    lib().orc_dequant_rows(ctypes.byref(p.c()), _ptr(codes), _ptr(scales), cap, _ptr(rows),
                           rows.size, _ptr(y))
    return y


# ---------------------------------------------------------------- combine
def combine(p: Problem, y: np.ndarray, w: np.ndarray, send_pos: np.ndarray,
            tokens: np.ndarray | None = None, out: np.ndarray | None = None):
    """Returns (err, out) with out uint16 bf16 bits: [R][T][H], or
    [len(tokens)][H] when a flat token list (s*T+t) is given (``out`` may
    be preallocated by the caller)."""
    y = np.ascontiguousarray(y, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    send_pos = np.ascontiguousarray(send_pos, dtype=np.int32)
    y_rows = y.shape[0] if y.ndim == 2 else y.size // p.H
    if tokens is None:
        out = np.zeros((p.R, p.T, p.H), np.uint16) if out is None else out
        err = lib().orc_combine(ctypes.byref(p.c()), _ptr(y), y_rows, _ptr(w), _ptr(send_pos),
                                None, 0, _ptr(out))
    else:
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.zeros((tokens.size, p.H), np.uint16) if out is None else out
        err = lib().orc_combine(ctypes.byref(p.c()), _ptr(y), y_rows, _ptr(w), _ptr(send_pos),
                                _ptr(tokens), tokens.size, _ptr(out))
    return err, out


# ---------------------------------------------------------------- messages
def msg_body_bytes(p: Problem, n: int):
    sec = np.zeros(6, np.int64)
    body = lib().orc_msg_body_bytes(ctypes.byref(p.c()), int(n), _ptr(sec))
    return int(body), sec


@dataclass
class Messages:
    err: int
    send_arena: np.ndarray   # uint8 [send_cap]
    table: np.ndarray        # int64 [R][R][8]
    arena_base: np.ndarray   # int64 [2][R+1]
    desc: np.ndarray         # uint8 [num_desc][64]
    num_desc: int


def messages(p: Problem, x: np.ndarray, topk: np.ndarray, w: np.ndarray,
             send_cap: int, desc_cap: int) -> Messages:
    R = p.R
    x = np.ascontiguousarray(x, dtype=np.uint16)
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    arena = np.zeros(max(send_cap, 1), np.uint8)
    table = np.zeros((R, R, 8), np.int64)
    base = np.zeros((2, R + 1), np.int64)
    desc = np.zeros((max(desc_cap, 1), 64), np.uint8)
    nd = np.zeros(1, np.int64)
    err = lib().orc_messages(ctypes.byref(p.c()), _ptr(x), _ptr(topk), _ptr(w), _ptr(arena),
                             send_cap, _ptr(table), _ptr(base), _ptr(desc), desc_cap, _ptr(nd))
    n = int(nd[0])
    return Messages(err, arena[:send_cap], table, base, desc[:min(n, desc_cap)], n)


def messages_execute(p: Problem, m: Messages, recv_cap: int, recv_arena: np.ndarray | None = None):
    """Executes the descriptors of `m` (loopback) into a receive arena of
    recv_cap bytes (fresh zeros unless `recv_arena` is given, which is
    updated in place).  Returns (err, recv_arena)."""
    if recv_arena is None:
        recv_arena = np.zeros(max(recv_cap, 1), np.uint8)
    desc = np.ascontiguousarray(m.desc, np.uint8)
    err = lib().orc_messages_execute(ctypes.byref(p.c()), _ptr(m.send_arena), m.send_arena.size,
                                     _ptr(m.arena_base), _ptr(desc), desc.shape[0],
                                     _ptr(recv_arena), recv_cap)
    return err, recv_arena


@dataclass
class Unpacked:
    err: int
    recv: np.ndarray          # [E*R*T][H] uint16 (bf16) or uint8 codes
    scales: np.ndarray | None  # [E][G][R*T] float32 or uint8, flattened
    recv_count: np.ndarray    # [E] int32
    recv_src_idx: np.ndarray  # [E*R*T] int32, -1 where not written


def messages_unpack(p: Problem, recv_arena: np.ndarray, table: np.ndarray,
                    cnt_expert: np.ndarray, fill_codes: int = 0) -> Unpacked:
    """Receiver: unpacks every valid message of the receive arena into the
    low-latency layout.  Rows and scales not written keep `fill_codes` (bytes)."""
    R, T, H, E = p.R, p.T, p.H, p.E
    rows = E * R * T
    if p.quant == Q_NONE:
        recv = np.full((rows, H), fill_codes * 0x0101, np.uint16)
        scales = None
    else:
        recv = np.full((rows, H), fill_codes, np.uint8)
        dt = np.float32 if p.quant == Q_FP8_F32 else np.uint8
        scales = np.zeros(max(p.G * rows, 1), dt)
        scales.view(np.uint8)[:] = fill_codes
    cnt = np.zeros(E, np.int32)
    src = np.full(max(rows, 1), -1, np.int32)
    arena = np.ascontiguousarray(recv_arena, np.uint8)
    err = lib().orc_messages_unpack(ctypes.byref(p.c()), _ptr(arena), arena.size,
                                    _ptr(np.ascontiguousarray(table, np.int64)),
                                    _ptr(np.ascontiguousarray(cnt_expert, np.int32)),
                                    _ptr(recv), _ptr(scales), _ptr(cnt), _ptr(src))
    return Unpacked(err, recv, scales, cnt, src[:rows])
