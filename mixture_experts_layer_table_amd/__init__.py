"""Python binding of libmok (the MI355X MoE-layer library).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmok.so``; PyTorch provides device memory and the stream. Importing this
package raises if the library has not been built
(``python mixture_experts_layer_table_amd/build.py``).

Two levels, after the pages' ops / functional split ("Mixture-of-Kittens (MoK)"
project summary, Functional API and Key-concepts table):

* ``mok_*`` — one function per C-ABI entry point, same names and arguments;
  tensors are passed as raw pointers and the caller owns every buffer.
* ``MoKConfig``, ``get_workspace``, ``build_schedule``, ``forward``,
  ``backward``, ``mxfp8_quantize`` — allocate the caller-side buffers with
  torch and call the entry points above.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

__version__ = "0.1.0"

# Device memory and streams come from PyTorch, so the library must run on the
# HIP runtime torch has loaded: import torch first, so that libmok's dependency
# on libamdhip64.so.7 resolves to that same copy instead of a second runtime.
import torch  # noqa: E402,F401

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmok.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with "
                      "`python mixture_experts_layer_table_amd/build.py` (there is no fallback)")
_lib = ctypes.CDLL(_LIB_PATH)

MOK_OK, MOK_ERROR_INVALID_VALUE, MOK_ERROR_UNSUPPORTED, MOK_ERROR_BUFFER_TOO_SMALL, \
    MOK_ERROR_LAUNCH_FAILED = range(5)
MOK_BF16, MOK_MXFP8, MOK_MXFP8_WGRAD = 0, 1, 2
MOK_SCHEDULE_OVERFLOW, MOK_BAD_EXPERT_ID, MOK_SCHEDULER_STALLED, MOK_SCHEDULE_MISMATCH = 1, 2, 4, 8
MOK_DEBUG_IDENTITY_EXPERT, MOK_DEBUG_SEPARATE_LAUNCHES, MOK_DEBUG_WHOLE_PASS, MOK_DEBUG_FORCE_STALL = 1, 2, 4, 8

EXPORTS = ("mok_config_default", "mok_config_autosize", "mok_query_sizes", "mok_schedule_layout_query",
           "mok_build_schedule", "mok_forward", "mok_backward", "mok_mxfp8_quantize", "mok_route",
           "mok_route_backward", "mok_status_string", "mok_kernel_timing_enable", "mok_kernel_timing_read",
           "mok_last_error", "mok_forward_noalloc", "mok_item_trace_enable", "mok_item_trace_read")
MOK_TRACE_FWD_GEMMS, MOK_TRACE_BWD_GEMMS, MOK_TRACE_WGRAD_GATE_UP, MOK_TRACE_WGRAD_DOWN, MOK_TRACE_OTHER = range(5)
MOK_ITEM_TRACE_CAPACITY = 65536
MOK_NOALLOC_SCRATCH_BYTES = 64 << 20


class mok_config(ctypes.Structure):
    _fields_ = [("minibatch_rows", ctypes.c_int32), ("precision", ctypes.c_int32),
                ("macrobatch_tokens", ctypes.c_int64), ("ring_bytes", ctypes.c_int64),
                ("capacity_multiplier", ctypes.c_float), ("debug_flags", ctypes.c_uint32),
                ("persistent_workgroups", ctypes.c_int32)]


class mok_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32)]


class mok_weights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("gate_elems", ctypes.c_void_p), ("gate_scales", ctypes.c_void_p),
                ("up_elems", ctypes.c_void_p), ("up_scales", ctypes.c_void_p),
                ("down_elems", ctypes.c_void_p), ("down_scales", ctypes.c_void_p)]


class mok_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double),
                ("max_ms", ctypes.c_double)]


class mok_item_record(ctypes.Structure):
    _fields_ = [("t_claim", ctypes.c_uint64), ("t_start", ctypes.c_uint64), ("t_kloop", ctypes.c_uint64),
                ("t_end", ctypes.c_uint64), ("launch", ctypes.c_uint32), ("kernel", ctypes.c_uint8),
                ("item_class", ctypes.c_uint8), ("xcd", ctypes.c_uint16), ("item", ctypes.c_uint32),
                ("workgroup", ctypes.c_uint32)]


class mok_schedule_layout(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int64), ("NM", ctypes.c_int64), ("G", ctypes.c_int64),
                ("cap", ctypes.c_int64)] + \
        [(n, ctypes.c_size_t) for n in ("status", "n_seg", "counts", "offsets", "mcounts", "moffsets",
                                       "perm", "inv", "canon", "mb_start", "segments", "total_bytes")]


_P = ctypes.c_void_p
_sz = ctypes.POINTER(ctypes.c_size_t)
_sigs = {
    "mok_config_default": [ctypes.POINTER(mok_config)],
    "mok_config_autosize": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape), ctypes.c_int32],
    "mok_query_sizes": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape), _sz, _sz, _sz],
    "mok_schedule_layout_query": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape),
                                  ctypes.POINTER(mok_schedule_layout)],
    "mok_build_schedule": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape), _P, _P,
                           ctypes.c_size_t, _P],
    "mok_forward": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape), _P, ctypes.c_size_t, _P,
                    ctypes.c_size_t, _P, _P, ctypes.POINTER(mok_weights), _P, _P, ctypes.c_size_t, _P],
    "mok_backward": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape), _P, ctypes.c_size_t, _P,
                     ctypes.c_size_t, _P, _P, ctypes.POINTER(mok_weights), _P, ctypes.c_size_t, _P, _P, _P,
                     _P, _P, _P, _P],
    "mok_forward_noalloc": [ctypes.POINTER(mok_config), ctypes.POINTER(mok_shape), _P, ctypes.c_size_t, _P, _P,
                            ctypes.POINTER(mok_weights), _P, _P, ctypes.c_size_t, _P],
    "mok_mxfp8_quantize": [_P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                           _P, _P, _P],
    "mok_route": [_P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P],
    "mok_route_backward": [_P, _P, _P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P],
    "mok_kernel_timing_enable": [ctypes.c_int32],
    "mok_item_trace_enable": [ctypes.c_int32],
    "mok_item_trace_read": [ctypes.POINTER(mok_item_record), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)],
    "mok_kernel_timing_read": [ctypes.POINTER(mok_kernel_stat), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)],
}
for _name, _args in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.mok_status_string.argtypes = [ctypes.c_int]
_lib.mok_status_string.restype = ctypes.c_char_p
_lib.mok_last_error.argtypes = []
_lib.mok_last_error.restype = ctypes.c_char_p


class MokError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = mok_last_error() if status == MOK_ERROR_LAUNCH_FAILED else ""
        super().__init__(f"{where}: {mok_status_string(status)}" + (f" ({detail})" if detail else ""))
        self.status = status


def _check(status: int, where: str):
    if status != MOK_OK:
        raise MokError(status, where)


def mok_status_string(status: int) -> str:
    return _lib.mok_status_string(status).decode()


def mok_last_error() -> str:
    return _lib.mok_last_error().decode()


# ----------------------------------------------------------------------------- raw entry points

def mok_config_default(cfg):
    return _lib.mok_config_default(ctypes.byref(cfg))


def mok_config_autosize(cfg, shape, n_cu):
    return _lib.mok_config_autosize(ctypes.byref(cfg), ctypes.byref(shape), n_cu)


def mok_query_sizes(cfg, shape, workspace, schedule, fwd_ctx):
    return _lib.mok_query_sizes(ctypes.byref(cfg), ctypes.byref(shape), workspace, schedule, fwd_ctx)


def mok_schedule_layout_query(cfg, shape, layout):
    return _lib.mok_schedule_layout_query(ctypes.byref(cfg), ctypes.byref(shape), ctypes.byref(layout))


def mok_build_schedule(cfg, shape, topk_ids, schedule, schedule_bytes, stream):
    return _lib.mok_build_schedule(ctypes.byref(cfg), ctypes.byref(shape), topk_ids, schedule,
                                   schedule_bytes, stream)


def mok_forward(cfg, shape, schedule, schedule_bytes, workspace, workspace_bytes, x, topk_w, weights, out,
                fwd_ctx, fwd_ctx_bytes, stream):
    return _lib.mok_forward(ctypes.byref(cfg), ctypes.byref(shape), schedule, schedule_bytes, workspace,
                            workspace_bytes, x, topk_w, ctypes.byref(weights), out, fwd_ctx, fwd_ctx_bytes,
                            stream)


def mok_backward(cfg, shape, schedule, schedule_bytes, workspace, workspace_bytes, x, topk_w, weights,
                 fwd_ctx, fwd_ctx_bytes, dy, dx, dw_gate, dw_up, dw_down, dtopk_w, stream):
    return _lib.mok_backward(ctypes.byref(cfg), ctypes.byref(shape), schedule, schedule_bytes, workspace,
                             workspace_bytes, x, topk_w, ctypes.byref(weights), fwd_ctx, fwd_ctx_bytes,
                             dy, dx, dw_gate, dw_up, dw_down, dtopk_w, stream)


def mok_forward_noalloc(cfg, shape, schedule, schedule_bytes, x, topk_w, weights, out, fwd_ctx, fwd_ctx_bytes,
                        stream):
    return _lib.mok_forward_noalloc(ctypes.byref(cfg), ctypes.byref(shape), schedule, schedule_bytes, x, topk_w,
                                    ctypes.byref(weights), out, fwd_ctx, fwd_ctx_bytes, stream)


def mok_mxfp8_quantize(src, batch, rows, K, src_is_k_by_rows, elems, scales, stream):
    return _lib.mok_mxfp8_quantize(src, batch, rows, K, src_is_k_by_rows, elems, scales, stream)


def mok_route(logits, T, E, k, topk_ids, topk_w, stream):
    return _lib.mok_route(logits, T, E, k, topk_ids, topk_w, stream)


def mok_route_backward(topk_ids, topk_w, dtopk_w, T, E, k, dlogits, stream):
    return _lib.mok_route_backward(topk_ids, topk_w, dtopk_w, T, E, k, dlogits, stream)


def mok_kernel_timing_enable(enable):
    return _lib.mok_kernel_timing_enable(enable)


def mok_kernel_timing_read(stats, capacity, count):
    return _lib.mok_kernel_timing_read(stats, capacity, count)


def mok_item_trace_enable(enable):
    return _lib.mok_item_trace_enable(enable)


def mok_item_trace_read(records, capacity, count):
    return _lib.mok_item_trace_read(records, capacity, count)


def item_trace_read():
    """The per-item trace records so far as a numpy structured array (synchronises)."""
    import numpy as np
    cap = MOK_ITEM_TRACE_CAPACITY
    arr = (mok_item_record * cap)()
    n = ctypes.c_int32()
    _check(mok_item_trace_read(arr, cap, ctypes.byref(n)), "mok_item_trace_read")
    dt = np.dtype([("t_claim", "<u8"), ("t_start", "<u8"), ("t_kloop", "<u8"), ("t_end", "<u8"),
                   ("launch", "<u4"), ("kernel", "u1"), ("item_class", "u1"), ("xcd", "<u2"),
                   ("item", "<u4"), ("workgroup", "<u4")])
    assert dt.itemsize == ctypes.sizeof(mok_item_record)
    buf = np.frombuffer(bytes(arr), dtype=dt)
    return buf[:min(n.value, cap)].copy(), n.value


def kernel_times(enable_after: bool = False):
    """Read (and clear) the per-kernel timing records: {name: (launches, total_ms, max_ms)}."""
    cap = 64
    arr = (mok_kernel_stat * cap)()
    n = ctypes.c_int32()
    _check(mok_kernel_timing_read(arr, cap, ctypes.byref(n)), "mok_kernel_timing_read")
    out = {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms, arr[i].max_ms) for i in range(min(n.value, cap))}
    if not enable_after:
        _check(mok_kernel_timing_enable(0), "mok_kernel_timing_enable")
    return out


# ----------------------------------------------------------------------------- functional layer

@dataclasses.dataclass
class MoKConfig:
    """Layer knobs; none of them changes any output bit."""
    minibatch_rows: int = 512
    macrobatch_tokens: int = 0
    ring_bytes: int = 256 << 20
    capacity_multiplier: float = 1.0
    precision: int = MOK_BF16
    debug_flags: int = 0
    persistent_workgroups: int = 0      # 0: one per compute unit

    def c(self) -> mok_config:
        return mok_config(self.minibatch_rows, self.precision, self.macrobatch_tokens,
                          self.ring_bytes, self.capacity_multiplier, self.debug_flags,
                          self.persistent_workgroups)


def _shape(T, H, I, E, k) -> mok_shape:
    return mok_shape(T, H, I, E, k)


def autosize_config(config: MoKConfig, T, H, I, E, k, n_cu: int = 0) -> MoKConfig:
    """Copy of ``config`` with the mini-batch sized by the two-wave rule (mok_config_autosize)."""
    c = config.c()
    _check(mok_config_autosize(c, _shape(T, H, I, E, k), n_cu), "mok_config_autosize")
    return dataclasses.replace(config, minibatch_rows=c.minibatch_rows, ring_bytes=c.ring_bytes)


def query_sizes(config: MoKConfig, T, H, I, E, k):
    ws, sc, cx = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(mok_query_sizes(config.c(), _shape(T, H, I, E, k), ctypes.byref(ws), ctypes.byref(sc),
                           ctypes.byref(cx)), "mok_query_sizes")
    return ws.value, sc.value, cx.value


def schedule_layout(config: MoKConfig, T, H, I, E, k) -> mok_schedule_layout:
    lay = mok_schedule_layout()
    _check(mok_schedule_layout_query(config.c(), _shape(T, H, I, E, k), lay), "mok_schedule_layout_query")
    return lay


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype, shape, device=None):
    """The C ABI receives raw pointers and no sizes for most tensors, so every
    tensor is checked here before a call: dtype (an int64 id tensor read as
    int32 would route silently wrong), exact shape (a short output would be
    written past its end), contiguity and device."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _require_bytes(t, name, nbytes, device=None):
    """A caller-given uint8 buffer of at least nbytes (workspace, schedule, fwd_ctx)."""
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous 1-D uint8 tensor")
    if t.numel() < nbytes:
        raise ValueError(f"{name}: {t.numel()} bytes, need {nbytes}")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name}: on {t.device}, expected {device}")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


@dataclasses.dataclass
class Workspace:
    """Caller-owned device buffers for one layer shape (made once, reused)."""
    config: MoKConfig
    T: int
    H: int
    I: int
    E: int
    k: int
    buffer: "object"        # torch.uint8 tensor
    schedule_bytes: int
    fwd_ctx_bytes: int


def get_workspace(config: MoKConfig, *, device, num_local_tokens: int, hidden_size: int,
                  intermediate_size: int, num_experts: int, topk: int) -> Workspace:
    import torch
    ws, sc, cx = query_sizes(config, num_local_tokens, hidden_size, intermediate_size, num_experts, topk)
    buf = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
    return Workspace(config, num_local_tokens, hidden_size, intermediate_size, num_experts, topk, buf,
                     sc, cx)


def build_schedule(ws: Workspace, topk_ids, schedule=None):
    """topk_ids: int32 [T,k] on the device. Returns the schedule buffer (uint8 tensor)."""
    import torch
    dev = ws.buffer.device
    _require(topk_ids, "topk_ids", torch.int32, (ws.T, ws.k), dev)
    if schedule is None:
        schedule = torch.empty(max(ws.schedule_bytes, 256), dtype=torch.uint8, device=dev)
    _require_bytes(schedule, "schedule", ws.schedule_bytes, dev)
    _check(mok_build_schedule(ws.config.c(), _shape(ws.T, ws.H, ws.I, ws.E, ws.k), _ptr(topk_ids),
                              _ptr(schedule), schedule.numel(), _stream()), "mok_build_schedule")
    return schedule


def weights_bf16(w_gate, w_up, w_down) -> mok_weights:
    """The struct keeps references to the tensors, so their memory lives as long as it does."""
    w = mok_weights(w_gate.data_ptr(), w_up.data_ptr(), w_down.data_ptr(), None, None, None, None, None, None)
    w._tensors = (w_gate, w_up, w_down)
    w._kind = "bf16"
    return w


def weights_mxfp8(gate, up, down, orientation: str = "") -> mok_weights:
    """Each argument is an (elems, scales) pair of uint8 tensors (kept referenced
    by the struct); orientation "fwd" or "bwd" when known (MXFP8Weights sets it)."""
    w = mok_weights(None, None, None, gate[0].data_ptr(), gate[1].data_ptr(), up[0].data_ptr(),
                    up[1].data_ptr(), down[0].data_ptr(), down[1].data_ptr())
    w._tensors = (gate, up, down)
    w._kind = "mxfp8" + (":" + orientation if orientation else "")
    return w


def _check_weights(ws: "Workspace", weights: mok_weights, orientation: str):
    """Shapes, dtypes and devices of the tensors a weight struct refers to."""
    import torch
    tensors = getattr(weights, "_tensors", None)
    if tensors is None:          # a hand-made struct: nothing to check against
        return
    dev = ws.buffer.device
    E, H, I = ws.E, ws.H, ws.I
    mx = ws.config.precision in (MOK_MXFP8, MOK_MXFP8_WGRAD)
    kind = getattr(weights, "_kind", "")
    if not mx:
        if not kind.startswith("bf16"):
            raise ValueError("BF16 mode needs bf16 weights (weights_bf16)")
        for t, n, sh in zip(tensors, ("w_gate", "w_up", "w_down"), ((E, H, I), (E, H, I), (E, I, H))):
            _require(t, n, torch.bfloat16, sh, dev)
        return
    if not kind.startswith("mxfp8"):
        raise ValueError("MXFP8 mode needs quantized weights (MXFP8Weights)")
    if ":" in kind and kind.split(":")[1] != orientation:
        raise ValueError(f"MXFP8 weights quantized for {kind.split(':')[1]}, used in {orientation}")
    if orientation == "fwd":        # quantized along the forward contraction axes
        shapes = ((E, I, H), (E, I, H), (E, H, I))
    else:
        shapes = ((E, H, I), (E, H, I), (E, I, H))
    for (el, sc), n, sh in zip(tensors, ("gate", "up", "down"), shapes):
        _require(el, n + " elements", torch.uint8, sh, dev)
        _require(sc, n + " scales", torch.uint8, sh[:2] + (sh[2] // 32,), dev)


class MXFP8Weights:
    """Expert weights quantized once for MXFP8 mode, in both orientations the
    layer needs (quantized along the contraction axis of each GEMM):
    ``fwd`` for mok_forward (W_gate^T, W_up^T [E,I,H] along H; W_down^T
    [E,H,I] along I) and ``bwd`` for mok_backward (W_gate, W_up [E,H,I] along
    I; W_down [E,I,H] along H). Holds the uint8 tensors the pointers refer to."""

    def __init__(self, w_gate, w_up, w_down):
        self.fwd_gate = mxfp8_quantize(w_gate, True)
        self.fwd_up = mxfp8_quantize(w_up, True)
        self.fwd_down = mxfp8_quantize(w_down, True)
        self.bwd_gate = mxfp8_quantize(w_gate, False)
        self.bwd_up = mxfp8_quantize(w_up, False)
        self.bwd_down = mxfp8_quantize(w_down, False)
        self.fwd = weights_mxfp8(self.fwd_gate, self.fwd_up, self.fwd_down, "fwd")
        self.bwd = weights_mxfp8(self.bwd_gate, self.bwd_up, self.bwd_down, "bwd")


def forward(ws: Workspace, schedule, x, topk_w, weights: mok_weights, out=None, fwd_ctx=None):
    """Returns (out bf16 [T,H], fwd_ctx uint8)."""
    import torch
    dev = ws.buffer.device
    if out is None:
        out = torch.empty((ws.T, ws.H), dtype=torch.bfloat16, device=dev)
    if fwd_ctx is None:
        fwd_ctx = torch.empty(max(ws.fwd_ctx_bytes, 256), dtype=torch.uint8, device=dev)
    _require_bytes(schedule, "schedule", ws.schedule_bytes, dev)
    _require(x, "x", torch.bfloat16, (ws.T, ws.H), dev)
    _require(topk_w, "topk_w", torch.float32, (ws.T, ws.k), dev)
    _require(out, "out", torch.bfloat16, (ws.T, ws.H), dev)
    _require_bytes(fwd_ctx, "fwd_ctx", ws.fwd_ctx_bytes, dev)
    _check_weights(ws, weights, "fwd")
    _check(mok_forward(ws.config.c(), _shape(ws.T, ws.H, ws.I, ws.E, ws.k), _ptr(schedule),
                       schedule.numel(), _ptr(ws.buffer), ws.buffer.numel(), _ptr(x), _ptr(topk_w), weights, _ptr(out),
                       _ptr(fwd_ctx), fwd_ctx.numel(), _stream()), "mok_forward")
    return out, fwd_ctx


def forward_noalloc(ws: Workspace, schedule, x, topk_w, weights: mok_weights, out, fwd_ctx):
    """forward() through mok_forward_noalloc: the library's static scratch
    instead of ws.buffer (ws supplies the config and shape only). out and
    fwd_ctx are caller-given; nothing is allocated here or in the call."""
    import torch
    dev = ws.buffer.device
    _require_bytes(schedule, "schedule", ws.schedule_bytes, dev)
    _require(x, "x", torch.bfloat16, (ws.T, ws.H), dev)
    _require(topk_w, "topk_w", torch.float32, (ws.T, ws.k), dev)
    _require(out, "out", torch.bfloat16, (ws.T, ws.H), dev)
    _require_bytes(fwd_ctx, "fwd_ctx", ws.fwd_ctx_bytes, dev)
    _check_weights(ws, weights, "fwd")
    _check(mok_forward_noalloc(ws.config.c(), _shape(ws.T, ws.H, ws.I, ws.E, ws.k), _ptr(schedule),
                               schedule.numel(), _ptr(x), _ptr(topk_w), weights, _ptr(out), _ptr(fwd_ctx),
                               fwd_ctx.numel(), _stream()), "mok_forward_noalloc")
    return out, fwd_ctx


def backward(ws: Workspace, schedule, fwd_ctx, x, topk_w, weights: mok_weights, dy, grads=None):
    """Returns dict(dx, dw_gate, dw_up, dw_down, dtopk_w)."""
    import torch
    dev = ws.buffer.device
    shapes = dict(dx=((ws.T, ws.H), torch.bfloat16), dw_gate=((ws.E, ws.H, ws.I), torch.bfloat16),
                  dw_up=((ws.E, ws.H, ws.I), torch.bfloat16), dw_down=((ws.E, ws.I, ws.H), torch.bfloat16),
                  dtopk_w=((ws.T, ws.k), torch.float32))
    if grads is None:
        grads = {n: torch.empty(sh, dtype=dt, device=dev) for n, (sh, dt) in shapes.items()}
    for n, (sh, dt) in shapes.items():
        _require(grads[n], n, dt, sh, dev)
    _require_bytes(schedule, "schedule", ws.schedule_bytes, dev)
    _require_bytes(fwd_ctx, "fwd_ctx", ws.fwd_ctx_bytes, dev)
    _require(x, "x", torch.bfloat16, (ws.T, ws.H), dev)
    _require(topk_w, "topk_w", torch.float32, (ws.T, ws.k), dev)
    _require(dy, "dy", torch.bfloat16, (ws.T, ws.H), dev)
    _check_weights(ws, weights, "bwd")
    _check(mok_backward(ws.config.c(), _shape(ws.T, ws.H, ws.I, ws.E, ws.k), _ptr(schedule),
                        schedule.numel(), _ptr(ws.buffer), ws.buffer.numel(), _ptr(x), _ptr(topk_w), weights,
                        _ptr(fwd_ctx), fwd_ctx.numel(), _ptr(dy), _ptr(grads["dx"]),
                        _ptr(grads["dw_gate"]), _ptr(grads["dw_up"]), _ptr(grads["dw_down"]),
                        _ptr(grads["dtopk_w"]), _stream()), "mok_backward")
    return grads


def mxfp8_quantize(src, src_is_k_by_rows: bool):
    """src bf16 [B, rows, K] (or [B, K, rows] when src_is_k_by_rows). Returns
    (elems uint8 [B, rows, K], scales uint8 [B, rows, K/32])."""
    import torch
    if src.dim() != 3:
        raise ValueError(f"src: expected [B, rows, K] or [B, K, rows], got shape {tuple(src.shape)}")
    _require(src, "src", torch.bfloat16, tuple(src.shape))
    B = src.shape[0]
    rows, K = (src.shape[2], src.shape[1]) if src_is_k_by_rows else (src.shape[1], src.shape[2])
    elems = torch.empty((B, rows, K), dtype=torch.uint8, device=src.device)
    scales = torch.empty((B, rows, K // 32), dtype=torch.uint8, device=src.device)
    _check(mok_mxfp8_quantize(_ptr(src), B, rows, K, int(src_is_k_by_rows), _ptr(elems), _ptr(scales),
                              _stream()), "mok_mxfp8_quantize")
    return elems, scales


def route(logits, k: int):
    """logits fp32 [T, E] on the device. Returns (topk_ids int32 [T, k],
    topk_w fp32 [T, k]): the k largest logits per row and their softmax weights
    renormalised over the chosen k."""
    import torch
    T, E = logits.shape
    _require(logits, "logits", torch.float32, (T, E))
    ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(mok_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream()), "mok_route")
    return ids, w


def route_backward(topk_ids, topk_w, dtopk_w, E: int):
    """Logit gradient fp32 [T, E] of route() for the upstream gradient dtopk_w [T, k]."""
    import torch
    T, k = topk_ids.shape
    _require(topk_ids, "topk_ids", torch.int32, (T, k))
    _require(topk_w, "topk_w", torch.float32, (T, k), topk_ids.device)
    _require(dtopk_w, "dtopk_w", torch.float32, (T, k), topk_ids.device)
    dl = torch.empty((T, E), dtype=torch.float32, device=topk_ids.device)
    _check(mok_route_backward(_ptr(topk_ids), _ptr(topk_w), _ptr(dtopk_w), T, E, k, _ptr(dl), _stream()),
           "mok_route_backward")
    return dl


def read_schedule(schedule, layout: mok_schedule_layout, E: int):
    """Copy the schedule table's fields to host numpy arrays (synchronises)."""
    import numpy as np
    host = schedule.cpu().numpy()

    def i32(off, n):
        return host[off: off + 4 * n].view(np.int32).copy()
    R, NM, G = layout.R, layout.NM, layout.G
    n_seg = int(i32(layout.n_seg, 1)[0])
    return dict(status=int(host[layout.status: layout.status + 4].view(np.uint32)[0]), n_seg=n_seg,
                counts=i32(layout.counts, E), offsets=i32(layout.offsets, E + 1),
                mcounts=i32(layout.mcounts, NM * E).reshape(NM, E),
                moffsets=i32(layout.moffsets, NM * (E + 1)).reshape(NM, E + 1),
                perm=i32(layout.perm, R), inv=i32(layout.inv, R), canon=i32(layout.canon, R),
                mb_start=i32(layout.mb_start, G + 1),
                segments=i32(layout.segments, 4 * min(n_seg, layout.cap)).reshape(-1, 4))
