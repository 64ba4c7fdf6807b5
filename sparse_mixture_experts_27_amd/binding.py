"""Thin ctypes binding of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP library.  Torch
tensors provide device memory and the current HIP stream.  If the library is missing
the calls raise; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
_lib = None

MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_GELU, MOE_ACT_SWIGLU = 0, 1
WEIGHT_MODES = {"renormalized": 0, "softmax": 1}
PRIORITIES = {"token": 0, "slot": 1}
OVERFLOWS = {"drop": 0, "reroute": 1}
MOE_LAYOUT_LINEAR, MOE_LAYOUT_PACKED = 0, 1
MOE_SCRATCH_BYTES = 64 << 20          # the fixed scratch of moe_layer_forward_noalloc, per GPU
STATUS = {0: "MOE_OK", 1: "MOE_EINVAL", 2: "MOE_EUNSUPPORTED", 3: "MOE_EWORKSPACE", 4: "MOE_EHIP"}

# entry points declared in include/moe.h
EXPORTS = ("moe_status_string", "moe_last_error", "moe_route_workspace_bytes", "moe_route",
           "moe_capacity", "moe_dispatch_workspace_bytes",
           "moe_dispatch", "moe_pack_weights", "moe_expert_ffn_workspace_bytes", "moe_expert_ffn", "moe_combine",
           "moe_routing_stats_workspace_bytes", "moe_routing_stats",
           "moe_layer_workspace_bytes", "moe_layer_plan", "moe_layer_forward", "moe_layer_forward_noalloc")


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class Tile(C.Structure):
    """moe_tile_t: explicit rows per M-tile and waves per workgroup (0 = automatic)."""
    _fields_ = [("rows", C.c_int32), ("waves", C.c_int32)]


class FfnPlan(C.Structure):
    _fields_ = [("tile_rows", C.c_int32), ("tile_waves", C.c_int32), ("down_splits", C.c_int32)]


class LayerArgs(C.Structure):
    _fields_ = [("dt", C.c_int32), ("act", C.c_int32), ("out_dt", C.c_int32), ("weights", C.c_int32),
                ("priority", C.c_int32), ("overflow", C.c_int32), ("layout", C.c_int32),
                ("T", C.c_int64), ("d", C.c_int64), ("F", C.c_int64),
                ("E", C.c_int32), ("k", C.c_int32), ("capacity", C.c_int64),
                ("x", C.c_void_p), ("w_r", C.c_void_p), ("bias", C.c_void_p),
                ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
                ("s_gate", C.c_void_p), ("s_up", C.c_void_p), ("s_down", C.c_void_p),
                ("out", C.c_void_p),
                ("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("logits", C.c_void_p),
                ("counts", C.c_void_p), ("offsets", C.c_void_p), ("perm", C.c_void_p),
                ("inv", C.c_void_p), ("n_dropped", C.c_void_p),
                ("ws", C.c_void_p), ("ws_bytes", C.c_size_t),
                ("stage_events", C.POINTER(C.c_void_p)),
                ("stats", C.c_void_p), ("lambda_balance", C.c_float), ("lambda_aux", C.c_float),
                ("gamma_aux", C.c_float), ("tile", Tile)]

STAT_NAMES = ("balance_ratio", "l_balance", "l_aux", "entropy", "drop_rate")

STAGE_EVENTS = 7
STAGES = ("route", "dispatch", "ffn_schedule", "ffn_up", "ffn_down", "combine")


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmoe.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m sparse_mixture_experts_27_amd.build`")
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [C.c_int]
        L.moe_last_error.restype = C.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route_workspace_bytes.argtypes = [i64, i64, i32, C.c_int]
        L.moe_route.restype = C.c_int
        L.moe_route.argtypes = [vp, vp, vp, C.c_int, i64, i64, i32, i32, C.c_int, vp, vp, vp, vp, sz, vp]
        L.moe_capacity.restype = i64
        L.moe_capacity.argtypes = [i64, i32, i32, C.c_double, i64]
        L.moe_dispatch_workspace_bytes.restype = sz
        L.moe_dispatch_workspace_bytes.argtypes = [i64, i32, i32]
        L.moe_dispatch.restype = C.c_int
        L.moe_dispatch.argtypes = [vp, vp, i64, i32, i32, i64, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_pack_weights.restype = C.c_int
        L.moe_pack_weights.argtypes = [vp, vp, i64, i64, i64, vp]
        L.moe_expert_ffn_workspace_bytes.restype = sz
        L.moe_expert_ffn_workspace_bytes.argtypes = [i64, i32, i64, i64, C.c_int, C.c_int, C.POINTER(Tile)]
        L.moe_expert_ffn.restype = C.c_int
        L.moe_expert_ffn.argtypes = [vp, vp, i32, vp, i32, i64, i64, i64, C.c_int, C.c_int, C.c_int,
                                     vp, vp, vp, vp, C.POINTER(Tile), vp, sz, vp]
        L.moe_combine.restype = C.c_int
        L.moe_combine.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, C.c_int, vp, vp]
        L.moe_routing_stats_workspace_bytes.restype = sz
        L.moe_routing_stats_workspace_bytes.argtypes = [i64]
        L.moe_routing_stats.restype = C.c_int
        L.moe_routing_stats.argtypes = [vp, vp, vp, i64, i32, i32, C.c_float, C.c_float, C.c_float, vp, vp, sz, vp]
        L.moe_layer_workspace_bytes.restype = sz
        L.moe_layer_workspace_bytes.argtypes = [C.POINTER(LayerArgs)]
        L.moe_layer_plan.restype = C.c_int
        L.moe_layer_plan.argtypes = [C.POINTER(LayerArgs), C.POINTER(FfnPlan)]
        L.moe_layer_forward.restype = C.c_int
        L.moe_layer_forward.argtypes = [C.POINTER(LayerArgs), vp]
        L.moe_layer_forward_noalloc.restype = C.c_int
        L.moe_layer_forward_noalloc.argtypes = [C.POINTER(LayerArgs), vp]
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MoEError(status, lib().moe_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _req(t: Optional[torch.Tensor], name: str, dtype=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------
def route(x, w_r, k, bias=None, weights="renormalized"):
    """-> (topk_idx int32 [T,k], topk_w f32 [T,k], logits f32 [T,E])."""
    T, d = x.shape
    E = w_r.shape[1]
    for t, n in ((x, "x"), (w_r, "w_r")):
        _req(t, n, x.dtype, x.device)
    _req(bias, "bias", torch.float32, x.device)
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    ws = _ws(lib().moe_route_workspace_bytes(T, d, E, _dt(x)), x.device)
    _check(lib().moe_route(_ptr(x), _ptr(w_r), _ptr(bias), _dt(x), T, d, E, k, WEIGHT_MODES[weights],
                           _ptr(idx), _ptr(w), _ptr(logits), _ptr(ws), ws.numel(), _stream(x.device)))
    return idx, w, logits


def capacity_rule(T, k, E, factor=1.0, min_capacity=0) -> int:
    """Per-expert capacity max(min_capacity, ceil(factor*T*k/E)) (moe_capacity)."""
    return int(lib().moe_capacity(int(T), int(k), int(E), float(factor), int(min_capacity)))


@dataclass
class Dispatch:
    counts: torch.Tensor
    offsets: torch.Tensor
    perm: torch.Tensor
    inv: torch.Tensor
    n_dropped: torch.Tensor


def dispatch(topk_idx, E, capacity=0, priority="token", overflow="drop", logits=None) -> Dispatch:
    """priority "token" | "slot"; overflow "drop" | "reroute" (needs the router logits)."""
    _req(topk_idx, "topk_idx", torch.int32)
    T, k = topk_idx.shape
    if logits is not None:
        _req(logits, "logits", torch.float32, topk_idx.device)
    dev = topk_idx.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.full((T * k,), -1, dtype=torch.int32, device=dev)
    inv = torch.empty((T, k), dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    ws = _ws(lib().moe_dispatch_workspace_bytes(T, E, k), dev)
    _check(lib().moe_dispatch(_ptr(topk_idx), _ptr(logits), T, E, k, int(capacity), PRIORITIES[priority],
                              OVERFLOWS[overflow], _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(nd),
                              _ptr(ws), ws.numel(), _stream(dev)))
    return Dispatch(counts, offsets, perm, inv, nd)


def pack_weights(w):
    """bf16 expert weights [G, N, K] (or [N, K]) in the nn.Linear layout -> a new tensor of
    the same shape holding them in the packed layout (moe_pack_weights)."""
    _req(w, "w", torch.bfloat16)
    shape = w.shape
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    G, N, K = w3.shape
    out = torch.empty_like(w)
    _check(lib().moe_pack_weights(_ptr(w3), _ptr(out), G, N, K, _stream(w.device)))
    assert out.shape == shape
    return out


def _tile(tile) -> Optional[Tile]:
    """(rows, waves) -> moe_tile_t, None -> automatic."""
    if tile is None:
        return None
    return Tile(int(tile[0]), int(tile[1]))


def expert_ffn(x, offsets, w_gate, w_up, w_down, max_rows, perm=None, k=1, act="swiglu", packed=False,
               tile=None):
    """-> y f32 [max_rows, d] (rows past offsets[G] unspecified).  packed: the weights were
    reordered by pack_weights.  tile: (rows per M-tile, waves) or None (automatic)."""
    G = w_gate.shape[0]
    F, d = w_gate.shape[1], w_gate.shape[2]
    dev = x.device
    for t, n in ((x, "x"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _req(t, n, x.dtype, dev)
    _req(offsets, "offsets", torch.int32, dev)
    _req(perm, "perm", torch.int32, dev)
    a = MOE_ACT_SWIGLU if act == "swiglu" else MOE_ACT_GELU
    y = torch.empty((max(max_rows, 1), d), dtype=torch.float32, device=dev)
    t = _tile(tile)
    tp = None if t is None else C.byref(t)
    ws = _ws(lib().moe_expert_ffn_workspace_bytes(max_rows, G, d, F, a, _dt(x), tp), dev)
    _check(lib().moe_expert_ffn(_ptr(x), _ptr(perm), k, _ptr(offsets), G, max_rows, d, F, a, _dt(x),
                                MOE_LAYOUT_PACKED if packed else MOE_LAYOUT_LINEAR, _ptr(w_gate), _ptr(w_up),
                                _ptr(w_down), _ptr(y), tp, _ptr(ws), ws.numel(), _stream(dev)))
    return y[:max_rows]


def combine(y, inv, topk_w, out_dtype, shared=None):
    """-> out [T, d] of out_dtype."""
    T, k = inv.shape
    d = y.shape[1]
    dev = inv.device
    _req(y, "y", torch.float32, dev)
    _req(inv, "inv", torch.int32, dev)
    _req(topk_w, "topk_w", torch.float32, dev)
    _req(shared, "shared", torch.float32, dev)
    out = torch.empty((T, d), dtype=out_dtype, device=dev)
    _check(lib().moe_combine(_ptr(y), y.shape[0], _ptr(inv), _ptr(topk_w), _ptr(shared), T, d, k,
                             MOE_BF16 if out_dtype == torch.bfloat16 else MOE_F32, _ptr(out),
                             _stream(dev)))
    return out


def routing_stats(logits, counts, n_dropped, k, lambda_balance=0.01, lambda_aux=0.01, gamma_aux=100.0):
    """-> f32 [5 + E]: balance ratio, L_balance, L_aux, entropy, drop rate, utilization[E]."""
    T, E = logits.shape
    dev = logits.device
    _req(logits, "logits", torch.float32, dev)
    _req(counts, "counts", torch.int32, dev)
    _req(n_dropped, "n_dropped", torch.int32, dev)
    stats = torch.empty(5 + E, dtype=torch.float32, device=dev)
    ws = _ws(lib().moe_routing_stats_workspace_bytes(T), dev)
    _check(lib().moe_routing_stats(_ptr(logits), _ptr(counts), _ptr(n_dropped), T, E, k, lambda_balance,
                                   lambda_aux, gamma_aux, _ptr(stats), _ptr(ws), ws.numel(), _stream(dev)))
    return stats


class Layer:
    """One MoE layer with its weights; forward() runs moe_layer_forward.

    Buffers for the output, the routing results and the workspace are allocated once
    (per token count) and reused, so repeated calls allocate nothing.  packed=True
    stores bf16 expert weights (routed and shared) in the packed layout: they are
    reordered once here, into new tensors (the caller's tensors are left as they are).
    prepacked=True: the expert weights given are already packed (pack_weights).
    capacity_factor: if given, the capacity of each call is capacity_rule(T, k, E,
    capacity_factor, min_capacity) for its T tokens (instead of the fixed `capacity`).
    tile: (rows per M-tile, waves) of the expert FFN, or None for the automatic choice.
    noalloc=True: forward() calls moe_layer_forward_noalloc, which runs on the library's
    fixed device scratch (MOE_SCRATCH_BYTES per GPU) instead of a workspace tensor.
    """

    def __init__(self, w_r, w_gate, w_up, w_down, k, act="swiglu", bias=None, capacity=0,
                 s_gate=None, s_up=None, s_down=None, out_dtype=torch.float32, stats=False,
                 lambda_balance=0.01, lambda_aux=0.01, gamma_aux=100.0, weights="renormalized",
                 priority="token", overflow="drop", packed=False, prepacked=False, capacity_factor=None,
                 min_capacity=0, tile=None, noalloc=False):
        self.w_r, self.bias = w_r, bias
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        self.s_gate, self.s_up, self.s_down = s_gate, s_up, s_down
        self.k, self.capacity = k, int(capacity)
        self.capacity_factor, self.min_capacity = capacity_factor, int(min_capacity)
        if out_dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("out_dtype must be float32 or bfloat16")
        self.out_dtype = out_dtype
        self.want_stats = bool(stats)
        self.weight_mode = WEIGHT_MODES[weights]
        self.priority = PRIORITIES[priority]
        self.overflow = OVERFLOWS[overflow]
        self.stat_coeffs = (lambda_balance, lambda_aux, gamma_aux)
        self.tile = (0, 0) if tile is None else (int(tile[0]), int(tile[1]))
        self.noalloc = bool(noalloc)
        self.act = MOE_ACT_SWIGLU if act == "swiglu" else MOE_ACT_GELU
        self.E = w_r.shape[1]
        self.F, self.d = w_gate.shape[1], w_gate.shape[2]
        dev = w_r.device
        for t, n in ((w_r, "w_r"), (w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down"),
                     (s_gate, "s_gate"), (s_up, "s_up"), (s_down, "s_down")):
            _req(t, n, w_r.dtype, dev)
        _req(bias, "bias", torch.float32, dev)
        self.layout = MOE_LAYOUT_PACKED if packed or prepacked else MOE_LAYOUT_LINEAR
        if packed and not prepacked:
            self.w_gate, self.w_up, self.w_down, self.s_gate, self.s_up, self.s_down = (
                None if t is None else pack_weights(t)
                for t in (w_gate, w_up, w_down, s_gate, s_up, s_down))
        self._T = None

    def _args(self, x):
        T = x.shape[0]
        a = LayerArgs()
        a.dt, a.act = _dt(x), self.act
        a.out_dt = MOE_BF16 if self.out_dtype == torch.bfloat16 else MOE_F32
        a.weights = self.weight_mode
        a.priority = self.priority
        a.overflow = self.overflow
        a.layout = self.layout
        a.T, a.d, a.F, a.E, a.k = T, self.d, self.F, self.E, self.k
        a.capacity = (self.capacity if self.capacity_factor is None else
                      capacity_rule(T, self.k, self.E, self.capacity_factor, self.min_capacity))
        a.x, a.w_r, a.bias = _ptr(x), _ptr(self.w_r), _ptr(self.bias)
        a.w_gate, a.w_up, a.w_down = _ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down)
        a.s_gate, a.s_up, a.s_down = _ptr(self.s_gate), _ptr(self.s_up), _ptr(self.s_down)
        if self.want_stats:
            a.stats = _ptr(self.stats)
            a.lambda_balance, a.lambda_aux, a.gamma_aux = self.stat_coeffs
        a.tile = Tile(*self.tile)
        return a

    def plan(self, T: int) -> dict:
        """The expert-FFN plan moe_layer_forward uses for T tokens (moe_layer_plan)."""
        a = LayerArgs()
        a.dt = _dt(self.w_r)
        a.act = self.act
        a.T, a.d, a.F, a.E, a.k = T, self.d, self.F, self.E, self.k
        a.capacity = (self.capacity if self.capacity_factor is None else
                      capacity_rule(T, self.k, self.E, self.capacity_factor, self.min_capacity))
        a.s_gate = _ptr(self.s_gate)
        a.tile = Tile(*self.tile)
        p = FfnPlan()
        _check(lib().moe_layer_plan(C.byref(a), C.byref(p)))
        return dict(tile_rows=p.tile_rows, tile_waves=p.tile_waves, down_splits=p.down_splits)

    def _buffers(self, x):
        T, dev, k = x.shape[0], x.device, self.k
        if self._T == T and self._dev == dev and self._dtype == x.dtype:
            return
        self.out = torch.empty((T, self.d), dtype=self.out_dtype, device=dev)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.logits = torch.empty((T, self.E), dtype=torch.float32, device=dev)
        self.counts = torch.empty(self.E, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        self.perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        self.inv = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.n_dropped = torch.empty(1, dtype=torch.int32, device=dev)
        if self.want_stats:
            self.stats = torch.empty(5 + self.E, dtype=torch.float32, device=dev)
        self.ws = None if self.noalloc else _ws(lib().moe_layer_workspace_bytes(C.byref(self._args(x))), dev)
        self._T, self._dev, self._dtype = T, dev, x.dtype

    def forward(self, x, stage_events=None):
        """stage_events: optional list of 7 torch.cuda.Event (already created) recorded at
        the stage boundaries on the current stream."""
        _req(x, "x", self.w_r.dtype, self.w_r.device)
        self._buffers(x)
        a = self._args(x)
        a.out = _ptr(self.out)
        a.topk_idx, a.topk_w, a.logits = _ptr(self.topk_idx), _ptr(self.topk_w), _ptr(self.logits)
        a.counts, a.offsets, a.perm = _ptr(self.counts), _ptr(self.offsets), _ptr(self.perm)
        a.inv, a.n_dropped = _ptr(self.inv), _ptr(self.n_dropped)
        if self.ws is not None:
            a.ws, a.ws_bytes = _ptr(self.ws), self.ws.numel()
        if stage_events is not None:
            if len(stage_events) != STAGE_EVENTS:
                raise ValueError(f"need {STAGE_EVENTS} events")
            arr = (C.c_void_p * STAGE_EVENTS)(*[ev.cuda_event for ev in stage_events])
            a.stage_events = C.cast(arr, C.POINTER(C.c_void_p))
        fwd = lib().moe_layer_forward_noalloc if self.noalloc else lib().moe_layer_forward
        _check(fwd(C.byref(a), _stream(x.device)))
        return self.out

    __call__ = forward
