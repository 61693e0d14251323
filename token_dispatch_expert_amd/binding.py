"""ctypes binding of the C ABI declared in include/moe.h.

Argument marshalling only: each function checks that it got device tensors of the expected
dtype and layout, reads the sizes off their shapes, and passes raw pointers and the current
HIP stream to the library. Every step of the layer runs in the library's HIP kernels; there is
no fallback of any kind. The library is the in-tree `libmoe.so` built by
`__graft_entry__.build()`; if it is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int, c_size_t, c_void_p

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libmoe.so"

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3FN, MOE_BF16_BLOCKED, MOE_FP8_E4M3FN_BLOCKED = 0, 1, 2, 3, 4

_DTYPE_ENUM = {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16,
               torch.float8_e4m3fn: MOE_FP8_E4M3FN, torch.uint8: MOE_FP8_E4M3FN}

ENTRY_POINTS = (
    "moe_status_string", "moe_route", "moe_permute_workspace_size", "moe_permute",
    "moe_ffn_workspace_size", "moe_grouped_ffn", "moe_combine", "moe_layer_workspace_size",
    "moe_layer", "moe_expert_capacity", "moe_permute_capped", "moe_layer_capped",
    "moe_route_gemm", "moe_route_gemm_workspace_size", "moe_permute_noalloc",
    "moe_block_weights",
)

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def load_library(path: str | None = None):
    """Load libmoe.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    P, I, S = c_void_p, c_int, c_size_t
    sig = {
        "moe_status_string": ([I], ctypes.c_char_p),
        "moe_route": ([P, I, I, I, P, P, P, P], I),
        "moe_permute_workspace_size": ([I, I, I], S),
        "moe_permute": ([P, I, P, I, I, I, I, P, P, P, P, P, P, S, P], I),
        "moe_ffn_workspace_size": ([I, I, I, I, I, I], S),
        "moe_grouped_ffn": ([P, I, P, I, I, I, I, P, P, P, I, P, P, P, P, P, S, P], I),
        "moe_combine": ([P, P, P, I, I, I, P, I, P], I),
        "moe_layer_workspace_size": ([I, I, I, I, I, I, I], S),
        "moe_layer": ([P, P, I, I, I, I, I, I, P, P, P, I, P, P, P,
                       P, P, P, P, P, P, P, P, P, I, P, S, P], I),
        "moe_expert_capacity": ([I, I, I, I], I),
        "moe_route_gemm": ([P, I, P, I, I, I, I, I, P, P, P, P, P, S, P], I),
        "moe_route_gemm_workspace_size": ([I, I, I], S),
        "moe_permute_capped": ([P, I, P, I, I, I, I, I, P, P, P, P, P, P, S, P], I),
        "moe_permute_noalloc": ([P, I, P, I, I, I, I, P, P, P, P, P, P], I),
        "moe_block_weights": ([P, P, I, I, I, I, P], I),
        "moe_layer_capped": ([P, P, I, I, I, I, I, I, I, P, P, P, I, P, P, P,
                              P, P, P, P, P, P, P, P, P, I, P, S, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != MOE_OK:
        msg = load_library().moe_status_string(status).decode()
        raise MoeError(status, msg)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _dt(t, name):
    try:
        return _DTYPE_ENUM[t.dtype]
    except KeyError:
        raise TypeError(f"{name}: unsupported dtype {t.dtype}") from None


# ----------------------------------------------------------------------------------------
# workspace
# ----------------------------------------------------------------------------------------
def moe_permute_workspace_size(T: int, E: int, k: int) -> int:
    return int(load_library().moe_permute_workspace_size(T, E, k))


def moe_ffn_workspace_size(rows: int, E: int, d: int, d_ff: int, act_dtype, w_dtype) -> int:
    return int(load_library().moe_ffn_workspace_size(rows, E, d, d_ff,
                                                     _DTYPE_ENUM[act_dtype], _DTYPE_ENUM[w_dtype]))


def moe_layer_workspace_size(T: int, E: int, k: int, d: int, d_ff: int, act_dtype, w_dtype) -> int:
    return int(load_library().moe_layer_workspace_size(T, E, k, d, d_ff, _DTYPE_ENUM[act_dtype],
                                                       _DTYPE_ENUM[w_dtype]))


class Workspace:
    """A device byte buffer (allocated by torch) handed to the library as scratch."""

    def __init__(self, nbytes: int, device="cuda"):
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 16), dtype=torch.uint8, device=device)

    @property
    def ptr(self):
        return c_void_p(self.buf.data_ptr()) if self.nbytes > 0 else None


# ----------------------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------------------
def moe_route(logits, k: int, topk_ids, topk_gates, counts=None, stream=None):
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(topk_gates, torch.float32, (T, k), "topk_gates")
    if counts is not None:
        _need(counts, torch.int32, (E,), "counts")
    _check(load_library().moe_route(_ptr(logits), T, E, k, _ptr(topk_ids), _ptr(topk_gates),
                                    _ptr(counts), _stream(stream)))


def moe_route_gemm_workspace_size(T: int, E: int, k: int) -> int:
    return load_library().moe_route_gemm_workspace_size(T, E, k)


def moe_route_gemm(x, w_router, k: int, topk_ids, topk_gates, counts=None, logits=None,
                   workspace: "Workspace | None" = None, stream=None):
    """Router scores x @ w_router^T (fp32) and top-k gating; logits optional. Small batches
    need a workspace of moe_route_gemm_workspace_size bytes (allocated here if not given)."""
    T, d = x.shape
    E = w_router.shape[0]
    if workspace is None:
        workspace = Workspace(moe_route_gemm_workspace_size(T, E, k), device=x.device)
    _need(w_router, x.dtype, (E, d), "w_router")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(topk_gates, torch.float32, (T, k), "topk_gates")
    if counts is not None:
        _need(counts, torch.int32, (E,), "counts")
    if logits is not None:
        _need(logits, torch.float32, (T, E), "logits")
    _check(load_library().moe_route_gemm(
        _ptr(x), _dt(x, "x"), _ptr(w_router), _dt(w_router, "w_router"), T, E, k, d,
        _ptr(logits), _ptr(topk_ids), _ptr(topk_gates), _ptr(counts), workspace.ptr,
        workspace.nbytes, _stream(stream)))


def moe_permute(x, topk_ids, E: int, counts, offsets, sorted_to_flat, flat_to_sorted, x_sorted,
                workspace: Workspace, stream=None, capacity: int | None = None):
    """capacity (optional): most kept assignments per expert (moe_permute_capped)."""
    T, d = x.shape
    k = topk_ids.shape[1]
    R = T * k
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(counts, torch.int32, (E,), "counts")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(sorted_to_flat, torch.int32, (R,), "sorted_to_flat")
    _need(flat_to_sorted, torch.int32, (R,), "flat_to_sorted")
    _need(x_sorted, x.dtype, (R, d), "x_sorted")
    lib = load_library()
    head = (_ptr(x), _dt(x, "x"), _ptr(topk_ids), T, E, k, d)
    tail = (_ptr(counts), _ptr(offsets), _ptr(sorted_to_flat), _ptr(flat_to_sorted),
            _ptr(x_sorted), workspace.ptr, workspace.nbytes, _stream(stream))
    if capacity is None:
        _check(lib.moe_permute(*head, *tail))
    else:
        _check(lib.moe_permute_capped(*head, int(capacity), *tail))


def moe_permute_noalloc(x, topk_ids, E: int, counts, offsets, sorted_to_flat, flat_to_sorted,
                        x_sorted, stream=None):
    """moe_permute without a workspace: the library's static per-GPU scratch (no allocation)."""
    T, d = x.shape
    k = topk_ids.shape[1]
    R = T * k
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(counts, torch.int32, (E,), "counts")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(sorted_to_flat, torch.int32, (R,), "sorted_to_flat")
    _need(flat_to_sorted, torch.int32, (R,), "flat_to_sorted")
    _need(x_sorted, x.dtype, (R, d), "x_sorted")
    _check(load_library().moe_permute_noalloc(
        _ptr(x), _dt(x, "x"), _ptr(topk_ids), T, E, k, d, _ptr(counts), _ptr(offsets),
        _ptr(sorted_to_flat), _ptr(flat_to_sorted), _ptr(x_sorted), _stream(stream)))


# bytes of the static scratch behind moe_permute_noalloc (MOE_PERMUTE_NOALLOC_SCRATCH_BYTES)
PERMUTE_NOALLOC_SCRATCH_BYTES = 4 << 20


def moe_expert_capacity(T: int, E: int, k: int, factor_percent: int) -> int:
    """ceil(C * T * k / E) for C = factor_percent / 100 (exact; -1 for invalid sizes)."""
    return load_library().moe_expert_capacity(T, E, k, int(factor_percent))


def _weights(w_gate, w_up, w_down, s_gate, s_up, s_down, blocked=False):
    """blocked: the bf16 or fp8 weights are in their blocked layout (see moe_block_weights); the
    tensors keep their [E, d_ff, d] / [E, d, d_ff] shapes."""
    E, d_ff, d = w_gate.shape
    _need(w_up, w_gate.dtype, (E, d_ff, d), "w_up")
    _need(w_down, w_gate.dtype, (E, d, d_ff), "w_down")
    w_dt = _dt(w_gate, "w_gate")
    if blocked:
        if w_dt not in (MOE_BF16, MOE_FP8_E4M3FN):
            raise TypeError("blocked weights are bfloat16 or float8_e4m3fn")
        w_dt = MOE_BF16_BLOCKED if w_dt == MOE_BF16 else MOE_FP8_E4M3FN_BLOCKED
    if w_dt == MOE_FP8_E4M3FN:
        for s, shp, n in ((s_gate, (E, -(-d_ff // 128), -(-d // 128)), "s_gate"),
                          (s_up, (E, -(-d_ff // 128), -(-d // 128)), "s_up"),
                          (s_down, (E, -(-d // 128), -(-d_ff // 128)), "s_down")):
            if s is None:
                raise ValueError(f"{n} is required for fp8 weights")
            _need(s, torch.float32, shp, n)
    return E, d, d_ff, w_dt


def moe_block_weights(src, dst, stream=None):
    """dst [E, N, K] <- src [E, N, K] (bfloat16 or float8_e4m3fn) in its blocked layout."""
    if src.dim() != 3:
        raise ValueError("src: expected [E, N, K]")
    E, N, K = src.shape
    if src.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError(f"src: expected bfloat16 or float8_e4m3fn, got {src.dtype}")
    _need(src, src.dtype, (E, N, K), "src")
    _need(dst, src.dtype, (E, N, K), "dst")
    _check(load_library().moe_block_weights(_ptr(src), _ptr(dst), _dt(src, "src"), E, N, K,
                                            _stream(stream)))


def moe_grouped_ffn(x_sorted, offsets, w_gate, w_up, w_down, y_sorted, workspace: Workspace,
                    s_gate=None, s_up=None, s_down=None, stream=None, weights_blocked=False):
    rows, d_x = x_sorted.shape
    E, d, d_ff, w_dt = _weights(w_gate, w_up, w_down, s_gate, s_up, s_down, weights_blocked)
    if d_x != d:
        raise ValueError("x_sorted and weights disagree on d")
    _need(offsets, torch.int32, (E + 1,), "offsets")
    _need(y_sorted, torch.float32, (rows, d), "y_sorted")
    _check(load_library().moe_grouped_ffn(
        _ptr(x_sorted), _dt(x_sorted, "x_sorted"), _ptr(offsets), rows, E, d, d_ff, _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), w_dt, _ptr(s_gate), _ptr(s_up), _ptr(s_down), _ptr(y_sorted),
        workspace.ptr, workspace.nbytes, _stream(stream)))


def _y_dt(y):
    """The combine's output format, from y's dtype: float32 or bfloat16."""
    if y.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"y: expected float32 or bfloat16, got {y.dtype}")
    return _DTYPE_ENUM[y.dtype]


def moe_combine(y_sorted, flat_to_sorted, topk_gates, y, stream=None):
    """y (float32 or bfloat16) receives the gate-weighted sums; bfloat16 is the fp32 sum
    rounded to nearest even."""
    T, k = topk_gates.shape
    R, d = y_sorted.shape
    if R != T * k:
        raise ValueError("y_sorted rows must equal T*k")
    _need(y_sorted, torch.float32, (R, d), "y_sorted")
    _need(flat_to_sorted, torch.int32, (R,), "flat_to_sorted")
    _need(topk_gates, torch.float32, (T, k), "topk_gates")
    _need(y, y.dtype, (T, d), "y")
    _check(load_library().moe_combine(_ptr(y_sorted), _ptr(flat_to_sorted), _ptr(topk_gates), T,
                                      k, d, _ptr(y), _y_dt(y), _stream(stream)))


def moe_layer(logits, x, w_gate, w_up, w_down, k: int, out: dict, workspace: Workspace,
              s_gate=None, s_up=None, s_down=None, stream=None, capacity: int | None = None,
              weights_blocked=False):
    """out holds the caller's buffers: topk_ids, topk_gates, counts, offsets, sorted_to_flat,
    flat_to_sorted, x_sorted, y_sorted, y (see `layer_buffers`; y float32 or bfloat16).
    capacity (optional): most kept assignments per expert (moe_layer_capped).
    weights_blocked: bf16 weights in the MOE_BF16_BLOCKED layout (moe_block_weights)."""
    T, E = logits.shape
    _need(logits, torch.float32, (T, E), "logits")
    Ew, d, d_ff, w_dt = _weights(w_gate, w_up, w_down, s_gate, s_up, s_down, weights_blocked)
    if Ew != E or x.shape != (T, d):
        raise ValueError("logits, x and weights disagree on T, E or d")
    R = T * k
    shapes = dict(topk_ids=(torch.int32, (T, k)), topk_gates=(torch.float32, (T, k)),
                  counts=(torch.int32, (E,)), offsets=(torch.int32, (E + 1,)),
                  sorted_to_flat=(torch.int32, (R,)), flat_to_sorted=(torch.int32, (R,)),
                  x_sorted=(x.dtype, (R, d)), y_sorted=(torch.float32, (R, d)),
                  y=(out["y"].dtype, (T, d)))
    for n, (dt, shp) in shapes.items():
        _need(out[n], dt, shp, n)
    o = out
    lib = load_library()
    head = (_ptr(logits), _ptr(x), _dt(x, "x"), T, E, k, d, d_ff)
    tail = (_ptr(w_gate), _ptr(w_up), _ptr(w_down), w_dt, _ptr(s_gate), _ptr(s_up), _ptr(s_down),
            _ptr(o["topk_ids"]), _ptr(o["topk_gates"]), _ptr(o["counts"]), _ptr(o["offsets"]),
            _ptr(o["sorted_to_flat"]), _ptr(o["flat_to_sorted"]), _ptr(o["x_sorted"]),
            _ptr(o["y_sorted"]), _ptr(o["y"]), _y_dt(o["y"]), workspace.ptr, workspace.nbytes,
            _stream(stream))
    if capacity is None:
        _check(lib.moe_layer(*head, *tail))
    else:
        _check(lib.moe_layer_capped(*head, int(capacity), *tail))


def layer_buffers(T: int, E: int, k: int, d: int, act_dtype, device="cuda",
                  y_dtype=torch.float32) -> dict:
    """Allocate (with torch) every output buffer moe_layer writes."""
    R = T * k
    z = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)  # noqa: E731
    return dict(topk_ids=z((T, k), torch.int32), topk_gates=z((T, k), torch.float32),
                counts=z((E,), torch.int32), offsets=z((E + 1,), torch.int32),
                sorted_to_flat=z((R,), torch.int32), flat_to_sorted=z((R,), torch.int32),
                x_sorted=z((R, d), act_dtype), y_sorted=z((R, d), torch.float32),
                y=z((T, d), y_dtype))
