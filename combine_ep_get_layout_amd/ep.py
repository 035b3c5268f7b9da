"""Thin ctypes binding of libep (include/ep.h): argument marshalling only.

Every step runs in the HIP library; this module turns torch tensors into
device pointers, fills the C structs, passes the current HIP stream and
raises ``EPError`` on a non-zero status.  It loads ``libep.so`` from the
package directory and raises if the library has not been built (there is
no fallback).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

MODE_NORMAL, MODE_LOW_LATENCY, MODE_MESSAGES, MODE_RANK_MAJOR = 0, 1, 2, 3
QUANT_NONE, QUANT_FP8_F32, QUANT_FP8_UE8M0 = 0, 1, 2
DEVERR_TOPK_RANGE, DEVERR_LL_OVERFLOW, DEVERR_CAPACITY, DEVERR_MESSAGE = 1, 2, 4, 8

EXPORTS = ["ep_workspace_bytes", "ep_max_recv_rows", "ep_messages_capacity", "ep_get_layout",
           "ep_dispatch", "ep_dispatch_fused", "ep_dispatch_fused_noalloc", "ep_combine",
           "ep_messages_execute", "ep_messages_unpack", "ep_status_string"]
NOALLOC_SCRATCH_BYTES = 64 << 20  # EP_NOALLOC_SCRATCH_BYTES
ERR_SCRATCH = -8


class EPError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


class CProblem(ctypes.Structure):
    _fields_ = [("num_ranks", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_topk", ctypes.c_int32), ("expert_alignment", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("quant", ctypes.c_int32),
                ("region_bytes", ctypes.c_int64), ("epoch", ctypes.c_uint32),
                ("reserved", ctypes.c_int32)]


_vp = ctypes.c_void_p


class CLayout(ctypes.Structure):
    _fields_ = [("num_tokens_per_rank", _vp), ("num_tokens_per_expert", _vp),
                ("is_token_in_rank", _vp), ("rank_prefix_matrix", _vp),
                ("recv_tokens_per_expert", _vp), ("expert_start", _vp),
                ("rows_per_rank", _vp), ("row_base", _vp), ("send_pos", _vp),
                ("send_head", _vp), ("recv_src_idx", _vp), ("recv_capacity", ctypes.c_int64),
                ("err", _vp)]


class CRecv(ctypes.Structure):
    _fields_ = [("x", _vp), ("scales", _vp), ("capacity", ctypes.c_int64),
                ("topk_idx", _vp), ("topk_weights", _vp)]


class CMessages(ctypes.Structure):
    _fields_ = [("send_arena", _vp), ("send_capacity", ctypes.c_int64), ("table", _vp),
                ("arena_base", _vp), ("descriptors", _vp), ("desc_capacity", ctypes.c_int64),
                ("num_descriptors", _vp)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run combine_ep_get_layout_amd/build.py")
        l = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(CProblem)
        l.ep_workspace_bytes.argtypes = [P]
        l.ep_workspace_bytes.restype = ctypes.c_size_t
        l.ep_max_recv_rows.argtypes = [P]
        l.ep_max_recv_rows.restype = ctypes.c_int64
        I64P = ctypes.POINTER(ctypes.c_int64)
        l.ep_messages_capacity.argtypes = [P, _vp, I64P, I64P, I64P]
        l.ep_messages_capacity.restype = ctypes.c_int
        l.ep_get_layout.argtypes = [P, _vp, ctypes.POINTER(CLayout), _vp, ctypes.c_size_t, _vp]
        l.ep_get_layout.restype = ctypes.c_int
        l.ep_dispatch.argtypes = [P, ctypes.POINTER(CLayout), _vp, _vp, _vp,
                                  ctypes.POINTER(CRecv), ctypes.POINTER(CMessages), _vp,
                                  ctypes.c_size_t, _vp]
        l.ep_dispatch.restype = ctypes.c_int
        l.ep_dispatch_fused.argtypes = [P, _vp, ctypes.POINTER(CLayout), _vp,
                                        ctypes.POINTER(CRecv), _vp, ctypes.c_size_t, _vp]
        l.ep_dispatch_fused.restype = ctypes.c_int
        l.ep_dispatch_fused_noalloc.argtypes = [P, _vp, ctypes.POINTER(CLayout), _vp,
                                                ctypes.POINTER(CRecv), _vp]
        l.ep_dispatch_fused_noalloc.restype = ctypes.c_int
        l.ep_combine.argtypes = [P, ctypes.POINTER(CLayout), _vp, ctypes.c_int64, _vp, _vp, _vp]
        l.ep_combine.restype = ctypes.c_int
        l.ep_messages_execute.argtypes = [P, ctypes.POINTER(CMessages), _vp, ctypes.c_int64,
                                          ctypes.c_int32, _vp, _vp]
        l.ep_messages_execute.restype = ctypes.c_int
        l.ep_messages_unpack.argtypes = [P, ctypes.POINTER(CMessages), _vp, ctypes.c_int64, _vp,
                                         ctypes.POINTER(CRecv), _vp, _vp, ctypes.c_int32, _vp,
                                         _vp]
        l.ep_messages_unpack.restype = ctypes.c_int
        l.ep_status_string.argtypes = [ctypes.c_int]
        l.ep_status_string.restype = ctypes.c_char_p
        _lib = l
    return _lib


def status_string(status: int) -> str:
    return lib().ep_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise EPError(status, what)


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libep takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libep takes contiguous tensors")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class _Args:
    """A libep entry point's name, its C arguments except the stream, and
    the ctypes objects those arguments point into (kept alive with them)."""

    def __init__(self, name: str, args: tuple, keep: tuple = ()):
        self.name, self.args, self.keep = name, args, keep


def _invoke(a: _Args, stream) -> None:
    _check(getattr(lib(), a.name)(*a.args, _stream(stream)), a.name)


class Call:
    """One libep call whose arguments were checked and marshalled once, when
    it was made (ep.prepare): calling it hands the cached C structs, device
    pointers and stream handle to the library and nothing else.  The
    tensors it was made from must stay alive and unchanged in size; their
    contents may change between calls."""

    def __init__(self, a: _Args, stream=None):
        self.name = a.name
        self._fn = getattr(lib(), a.name)
        self._args = a.args + (_stream(stream),)
        self._keep = a.keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            raise EPError(st, self.name)


def prepare(fn, *args, stream=None, **kw) -> Call:
    """ep.prepare(ep.dispatch, p, layout, x, recv=..., ws=...) checks the
    arguments as fn would and returns a Call that repeats the call with
    them on `stream` (torch's current stream when it was prepared by
    default)."""
    return Call(_ARGS[fn](*args, **kw), stream)


@dataclass
class Problem:
    R: int
    T: int
    H: int
    E: int
    K: int
    align: int = 1
    mode: int = MODE_NORMAL
    quant: int = QUANT_NONE
    region_bytes: int = 2 << 20
    epoch: int = 1

    def c(self) -> CProblem:
        return CProblem(self.R, self.T, self.H, self.E, self.K, self.align, self.mode, self.quant,
                        self.region_bytes, self.epoch, 0)

    @property
    def L(self) -> int:
        return self.E // self.R

    @property
    def G(self) -> int:
        return self.H // 128


def workspace_bytes(p: Problem) -> int:
    return int(lib().ep_workspace_bytes(ctypes.byref(p.c())))


def max_recv_rows(p: Problem) -> int:
    return int(lib().ep_max_recv_rows(ctypes.byref(p.c())))


class Layout:
    """Device buffers of one ep_get_layout call (the dispatch handle)."""

    def __init__(self, p: Problem, device="cuda", recv_capacity: int | None = None,
                 send_head: bool = True, recv_src_idx: bool = True):
        R, T, E, K = p.R, p.T, p.E, p.K
        i32 = dict(dtype=torch.int32, device=device)
        self.num_tokens_per_rank = torch.empty((R, R), **i32)
        self.num_tokens_per_expert = torch.empty((R, E), **i32)
        self.is_token_in_rank = torch.empty((R, T, R), dtype=torch.uint8, device=device)
        self.rank_prefix_matrix = torch.empty((R, R), **i32)
        self.recv_tokens_per_expert = torch.empty(E, **i32)
        self.expert_start = torch.empty(E, **i32)
        self.rows_per_rank = torch.empty(R, **i32)
        self.row_base = torch.empty(R + 1, **i32)
        self.send_pos = torch.empty((R, T, K), **i32) if p.mode != MODE_MESSAGES else None
        need_head = send_head or p.mode == MODE_MESSAGES
        self.send_head = torch.empty((R, T, R), **i32) if need_head else None
        if recv_capacity is None:
            recv_capacity = max_recv_rows(p) if p.mode != MODE_MESSAGES else 0
        self.recv_capacity = int(recv_capacity)
        self.recv_src_idx = (torch.empty(max(self.recv_capacity, 1), **i32)
                             if recv_src_idx and p.mode != MODE_MESSAGES else None)
        self.err = torch.zeros(1, **i32)

    def c(self) -> CLayout:
        return CLayout(_ptr(self.num_tokens_per_rank), _ptr(self.num_tokens_per_expert),
                       _ptr(self.is_token_in_rank), _ptr(self.rank_prefix_matrix),
                       _ptr(self.recv_tokens_per_expert), _ptr(self.expert_start),
                       _ptr(self.rows_per_rank), _ptr(self.row_base), _ptr(self.send_pos),
                       _ptr(self.send_head), _ptr(self.recv_src_idx),
                       self.recv_capacity if self.recv_src_idx is not None else 0,
                       _ptr(self.err))


def workspace(p: Problem, device="cuda") -> torch.Tensor:
    n = workspace_bytes(p)
    if n == 0:
        raise EPError(-3, "workspace size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _need(cond: bool, what: str):
    if not cond:
        raise ValueError(what)


def get_layout(p: Problem, topk_idx: torch.Tensor, layout: Layout, ws: torch.Tensor,
               stream=None) -> None:
    _invoke(_get_layout_args(p, topk_idx, layout, ws), stream)


def _get_layout_args(p: Problem, topk_idx: torch.Tensor, layout: Layout,
                     ws: torch.Tensor) -> _Args:
    R, T, E, K = p.R, p.T, p.E, p.K
    _need(topk_idx.dtype == torch.int32 and topk_idx.numel() == R * T * K, "topk_idx [R][T][K] int32")
    _need(layout.num_tokens_per_expert.numel() == R * E and layout.is_token_in_rank.numel() == R * T * R,
          "layout buffers do not match the problem")
    _need(layout.send_pos is None or layout.send_pos.numel() == R * T * K, "send_pos [R][T][K]")
    _need(layout.send_head is None or layout.send_head.numel() == R * T * R, "send_head [R][T][R]")
    _need(layout.recv_src_idx is None or layout.recv_src_idx.numel() >= layout.recv_capacity,
          "recv_src_idx smaller than recv_capacity")
    _need(ws.numel() >= workspace_bytes(p), "workspace too small")
    pc, cl = p.c(), layout.c()
    return _Args("ep_get_layout", (ctypes.byref(pc), _ptr(topk_idx), ctypes.byref(cl), _ptr(ws),
                                   ws.numel()), (pc, cl))


class Recv:
    """Receive buffers of normal / low-latency / rank-major dispatch.  In
    rank-major mode `meta` also allocates the per-row top-k ids and weights."""

    def __init__(self, p: Problem, capacity: int, device="cuda", meta: bool = True):
        self.capacity = int(capacity)
        if p.quant == QUANT_NONE:
            self.x = torch.empty((self.capacity, p.H), dtype=torch.bfloat16, device=device)
            self.scales = None
        else:
            self.x = torch.empty((self.capacity, p.H), dtype=torch.uint8, device=device)
            n = p.G * (p.E * p.R * p.T if p.mode == MODE_LOW_LATENCY else self.capacity)
            dt = torch.float32 if p.quant == QUANT_FP8_F32 else torch.uint8
            self.scales = torch.empty(max(n, 1), dtype=dt, device=device)
        self.topk_idx = self.topk_weights = None
        if p.mode == MODE_RANK_MAJOR and meta:
            self.topk_idx = torch.empty((max(self.capacity, 1), p.K), dtype=torch.int32,
                                        device=device)
            self.topk_weights = torch.empty((max(self.capacity, 1), p.K), dtype=torch.float32,
                                            device=device)

    def c(self) -> CRecv:
        return CRecv(_ptr(self.x), _ptr(self.scales), self.capacity, _ptr(self.topk_idx),
                     _ptr(self.topk_weights))


class Messages:
    """Send arena, per-message table and descriptors of message mode."""

    def __init__(self, p: Problem, send_capacity: int, desc_capacity: int, device="cuda"):
        R = p.R
        self.send_capacity = int(send_capacity)
        self.desc_capacity = int(desc_capacity)
        self.send_arena = torch.empty(max(self.send_capacity, 16), dtype=torch.uint8,
                                      device=device)
        self.table = torch.empty((R, R, 8), dtype=torch.int64, device=device)
        self.arena_base = torch.empty((2, R + 1), dtype=torch.int64, device=device)
        self.descriptors = torch.empty((max(self.desc_capacity, 1), 64), dtype=torch.uint8,
                                       device=device)
        self.num_descriptors = torch.zeros(1, dtype=torch.int64, device=device)

    def c(self) -> CMessages:
        return CMessages(_ptr(self.send_arena), self.send_capacity, _ptr(self.table),
                         _ptr(self.arena_base), _ptr(self.descriptors), self.desc_capacity,
                         _ptr(self.num_descriptors))


def dispatch(p: Problem, layout: Layout, x: torch.Tensor, *, recv: Recv | None = None,
             msgs: Messages | None = None, topk_idx: torch.Tensor | None = None,
             topk_weights: torch.Tensor | None = None, ws: torch.Tensor | None = None,
             stream=None) -> None:
    _invoke(_dispatch_args(p, layout, x, recv=recv, msgs=msgs, topk_idx=topk_idx,
                           topk_weights=topk_weights, ws=ws), stream)


def _dispatch_args(p: Problem, layout: Layout, x: torch.Tensor, *, recv: Recv | None = None,
                   msgs: Messages | None = None, topk_idx: torch.Tensor | None = None,
                   topk_weights: torch.Tensor | None = None,
                   ws: torch.Tensor | None = None) -> _Args:
    R, T, H, E, K = p.R, p.T, p.H, p.E, p.K
    _need(x.dtype == torch.bfloat16 and x.numel() == R * T * H, "x [R][T][H] bf16")
    if p.mode != MODE_MESSAGES:
        _need(recv is not None and layout.send_pos is not None, "recv buffers and send_pos")
        if p.mode == MODE_RANK_MAJOR and (recv.topk_idx is not None or recv.topk_weights is not None):
            _need(topk_idx is not None and topk_idx.dtype == torch.int32
                  and topk_idx.numel() == R * T * K, "topk_idx [R][T][K] int32 (row metadata)")
            _need(recv.topk_weights is None or (topk_weights is not None
                  and topk_weights.dtype == torch.float32 and topk_weights.numel() == R * T * K),
                  "topk_weights [R][T][K] fp32 (row metadata)")
            for t_ in (recv.topk_idx, recv.topk_weights):
                _need(t_ is None or t_.numel() >= recv.capacity * K, "row metadata [capacity][K]")
        _need(recv.x.shape[0] >= recv.capacity and recv.x.shape[1] == H, "recv x [capacity][H]")
        if p.quant != QUANT_NONE:
            n = p.G * (E * R * T if p.mode == MODE_LOW_LATENCY else recv.capacity)
            _need(recv.scales is not None and recv.scales.numel() >= n, "recv scales")
            _need(recv.x.element_size() == 1, "FP8 codes are bytes")
        else:
            _need(recv.x.element_size() == 2, "bf16 rows")
    else:
        _need(msgs is not None and layout.send_head is not None, "message buffers and send_head")
        _need(topk_idx is not None and topk_idx.dtype == torch.int32 and topk_idx.numel() == R * T * K,
              "topk_idx [R][T][K] int32")
        _need(topk_weights is not None and topk_weights.dtype == torch.float32
              and topk_weights.numel() == R * T * K, "topk_weights [R][T][K] fp32")
        _need(msgs.send_arena.numel() >= msgs.send_capacity, "send arena")
        _need(msgs.descriptors.shape[0] >= msgs.desc_capacity, "descriptors")
        _need(ws is not None and ws.numel() >= workspace_bytes(p), "workspace too small")
    pc, cl = p.c(), layout.c()
    cr = recv.c() if recv is not None else None
    cm = msgs.c() if msgs is not None else None
    return _Args("ep_dispatch", (ctypes.byref(pc), ctypes.byref(cl), _ptr(x), _ptr(topk_idx),
                                 _ptr(topk_weights), ctypes.byref(cr) if cr is not None else None,
                                 ctypes.byref(cm) if cm is not None else None, _ptr(ws),
                                 ws.numel() if ws is not None else 0), (pc, cl, cr, cm))


def dispatch_fused(p: Problem, topk_idx: torch.Tensor, layout: Layout, x: torch.Tensor,
                   recv: Recv, ws: torch.Tensor, stream=None) -> None:
    """Layout and dispatch in one call (normal / low-latency modes): fills
    `layout` exactly as get_layout does and `recv` as dispatch does."""
    _invoke(_dispatch_fused_args(p, topk_idx, layout, x, recv, ws), stream)


def _check_fused(p: Problem, topk_idx: torch.Tensor, layout: Layout, x: torch.Tensor,
                 recv: Recv) -> None:
    R, T, H, E, K = p.R, p.T, p.H, p.E, p.K
    _need(p.mode in (MODE_NORMAL, MODE_LOW_LATENCY), "normal or low-latency problem")
    _need(topk_idx.dtype == torch.int32 and topk_idx.numel() == R * T * K, "topk_idx [R][T][K] int32")
    _need(layout.num_tokens_per_expert.numel() == R * E and layout.is_token_in_rank.numel() == R * T * R,
          "layout buffers do not match the problem")
    _need(layout.send_pos is not None and layout.send_pos.numel() == R * T * K, "send_pos [R][T][K]")
    _need(layout.send_head is None or layout.send_head.numel() == R * T * R, "send_head [R][T][R]")
    _need(layout.recv_src_idx is None or layout.recv_src_idx.numel() >= layout.recv_capacity,
          "recv_src_idx smaller than recv_capacity")
    _need(x.dtype == torch.bfloat16 and x.numel() == R * T * H, "x [R][T][H] bf16")
    _need(recv.x.shape[0] >= recv.capacity and recv.x.shape[1] == H, "recv x [capacity][H]")
    if p.quant != QUANT_NONE:
        n = p.G * (E * R * T if p.mode == MODE_LOW_LATENCY else recv.capacity)
        _need(recv.scales is not None and recv.scales.numel() >= n, "recv scales")
        _need(recv.x.element_size() == 1, "FP8 codes are bytes")
    else:
        _need(recv.x.element_size() == 2, "bf16 rows")


def _dispatch_fused_args(p: Problem, topk_idx: torch.Tensor, layout: Layout, x: torch.Tensor,
                         recv: Recv, ws: torch.Tensor) -> _Args:
    _check_fused(p, topk_idx, layout, x, recv)
    _need(ws.numel() >= workspace_bytes(p), "workspace too small")
    pc, cl, cr = p.c(), layout.c(), recv.c()
    return _Args("ep_dispatch_fused", (ctypes.byref(pc), _ptr(topk_idx), ctypes.byref(cl), _ptr(x),
                                       ctypes.byref(cr), _ptr(ws), ws.numel()), (pc, cl, cr))


def dispatch_fused_noalloc(p: Problem, topk_idx: torch.Tensor, layout: Layout, x: torch.Tensor,
                           recv: Recv, stream=None) -> None:
    """dispatch_fused with the library's fixed scratch array instead of a
    workspace (ep_dispatch_fused_noalloc): nothing is allocated."""
    _invoke(_dispatch_fused_noalloc_args(p, topk_idx, layout, x, recv), stream)


def _dispatch_fused_noalloc_args(p: Problem, topk_idx: torch.Tensor, layout: Layout,
                                 x: torch.Tensor, recv: Recv) -> _Args:
    _check_fused(p, topk_idx, layout, x, recv)
    pc, cl, cr = p.c(), layout.c(), recv.c()
    return _Args("ep_dispatch_fused_noalloc", (ctypes.byref(pc), _ptr(topk_idx), ctypes.byref(cl),
                                               _ptr(x), ctypes.byref(cr)), (pc, cl, cr))


def combine(p: Problem, layout: Layout, y: torch.Tensor, topk_weights: torch.Tensor,
            out: torch.Tensor, stream=None) -> None:
    _invoke(_combine_args(p, layout, y, topk_weights, out), stream)


def _combine_args(p: Problem, layout: Layout, y: torch.Tensor, topk_weights: torch.Tensor,
                  out: torch.Tensor) -> _Args:
    R, T, H, K = p.R, p.T, p.H, p.K
    _need(y.dtype == torch.bfloat16 and y.dim() == 2 and y.shape[1] == H, "y [rows][H] bf16")
    if p.mode != MODE_RANK_MAJOR or topk_weights is not None:
        _need(topk_weights.dtype == torch.float32 and topk_weights.numel() == R * T * K,
              "topk_weights [R][T][K] fp32")
    _need(out.dtype == torch.bfloat16 and out.numel() == R * T * H, "out [R][T][H] bf16")
    _need(layout.send_pos is not None and layout.send_pos.numel() == R * T * K, "send_pos")
    cl = layout.c()
    y_rows = y.shape[0]
    pc = p.c()
    return _Args("ep_combine", (ctypes.byref(pc), ctypes.byref(cl), _ptr(y), y_rows,
                                _ptr(topk_weights), _ptr(out)), (pc, cl))


def messages_execute(p: Problem, msgs: Messages, recv_arena: torch.Tensor, err: torch.Tensor,
                     stream=None, publish_batch: int = 0) -> None:
    """Loopback delivery of the descriptors of `msgs` into `recv_arena`
    (uint8; msgs.arena_base[1][R] bytes suffice), flags published every
    `publish_batch` messages per workgroup (0: all after a second launch).
    Error bits are OR-ed into err[0]."""
    _invoke(_messages_execute_args(p, msgs, recv_arena, err, publish_batch), stream)


def _messages_execute_args(p: Problem, msgs: Messages, recv_arena: torch.Tensor,
                           err: torch.Tensor, publish_batch: int = 0) -> _Args:
    _need(p.mode == MODE_MESSAGES, "message-mode problem")
    _need(recv_arena.dtype == torch.uint8, "recv_arena bytes")
    _need(err.dtype == torch.int32 and err.numel() >= 1, "err int32")
    _need(msgs.table.numel() == p.R * p.R * 8 and msgs.arena_base.numel() == 2 * (p.R + 1),
          "message table / arena bases")
    _need(publish_batch >= 0, "publish_batch >= 0")
    pc, cm = p.c(), msgs.c()
    return _Args("ep_messages_execute", (ctypes.byref(pc), ctypes.byref(cm), _ptr(recv_arena),
                                         recv_arena.numel(), int(publish_batch), _ptr(err)),
                 (pc, cm))


def unpack_buffers(p: Problem, device="cuda") -> tuple[Recv, torch.Tensor, torch.Tensor]:
    """Low-latency receive buffers for messages_unpack: (rows and scales
    [E*R*T], recv_count [E], recv_src_idx [E*R*T] filled with -1)."""
    rows = p.E * p.R * p.T
    recv = Recv(p, rows, device=device)
    count = torch.zeros(p.E, dtype=torch.int32, device=device)
    src = torch.full((max(rows, 1),), -1, dtype=torch.int32, device=device)
    return recv, count, src


def messages_unpack(p: Problem, msgs: Messages, recv_arena: torch.Tensor,
                    num_tokens_per_expert: torch.Tensor, out: Recv, recv_count: torch.Tensor,
                    recv_src_idx: torch.Tensor, err: torch.Tensor, stream=None,
                    spin_limit: int = 0) -> None:
    """Receiver: checks every delivered message (polling its flag up to
    `spin_limit` times first) and unpacks it into the low-latency layout
    `out` (capacity >= E*R*T).  Error bits are OR-ed into err[0]."""
    _invoke(_messages_unpack_args(p, msgs, recv_arena, num_tokens_per_expert, out, recv_count,
                                  recv_src_idx, err, spin_limit), stream)


def _messages_unpack_args(p: Problem, msgs: Messages, recv_arena: torch.Tensor,
                          num_tokens_per_expert: torch.Tensor, out: Recv, recv_count: torch.Tensor,
                          recv_src_idx: torch.Tensor, err: torch.Tensor,
                          spin_limit: int = 0) -> _Args:
    R, T, E = p.R, p.T, p.E
    rows = E * R * T
    _need(p.mode == MODE_MESSAGES, "message-mode problem")
    _need(recv_arena.dtype == torch.uint8, "recv_arena bytes")
    _need(num_tokens_per_expert.dtype == torch.int32 and num_tokens_per_expert.numel() == R * E,
          "num_tokens_per_expert [R][E] int32")
    _need(out.capacity >= rows and out.x.shape[0] >= rows and out.x.shape[1] == p.H,
          "out rows [E*R*T][H]")
    _need(out.x.element_size() == (2 if p.quant == QUANT_NONE else 1), "out row element size")
    if p.quant != QUANT_NONE:
        _need(out.scales is not None and out.scales.numel() >= p.G * rows, "out scales")
    _need(recv_count.dtype == torch.int32 and recv_count.numel() == E, "recv_count [E]")
    _need(recv_src_idx.dtype == torch.int32 and recv_src_idx.numel() >= rows, "recv_src_idx")
    _need(err.dtype == torch.int32 and err.numel() >= 1, "err int32")
    _need(msgs.table.numel() == R * R * 8, "message table")
    pc, cm, cr = p.c(), msgs.c(), out.c()
    return _Args("ep_messages_unpack", (ctypes.byref(pc), ctypes.byref(cm), _ptr(recv_arena),
                                        recv_arena.numel(), _ptr(num_tokens_per_expert),
                                        ctypes.byref(cr), _ptr(recv_count), _ptr(recv_src_idx),
                                        int(spin_limit), _ptr(err)), (pc, cm, cr))


_ARGS = {get_layout: _get_layout_args, dispatch: _dispatch_args,
         dispatch_fused: _dispatch_fused_args, dispatch_fused_noalloc: _dispatch_fused_noalloc_args,
         combine: _combine_args, messages_execute: _messages_execute_args,
         messages_unpack: _messages_unpack_args}


def messages_sizes(p: Problem, counts=None) -> tuple[int, int, int]:
    """ep_messages_capacity: (send arena bytes, receive arena bytes,
    descriptors).  `counts`: host [R][R] tokens per (source, destination)
    for exact sizes, or None for bounds that hold for every routing."""
    import numpy as np

    c = None
    if counts is not None:
        c = np.ascontiguousarray(counts, dtype=np.int32)
        _need(c.size == p.R * p.R, "counts [R][R]")
    out = [ctypes.c_int64(0) for _ in range(3)]
    _check(lib().ep_messages_capacity(ctypes.byref(p.c()),
                                      c.ctypes.data if c is not None else None,
                                      *[ctypes.byref(v) for v in out]), "ep_messages_capacity")
    return out[0].value, out[1].value, out[2].value


def messages_capacity(p: Problem, counts=None) -> tuple[int, int]:
    """(send arena bytes, descriptors) for Messages(), from
    ep_messages_capacity (at least 16 bytes and one descriptor, so the
    buffers are never empty)."""
    send, _, desc = messages_sizes(p, counts)
    return max(send, 16), max(desc, 1)
