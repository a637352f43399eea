"""Python binding of libmoe.so (ctypes): argument marshalling only.

Every step of the layer runs in the library's HIP kernels; PyTorch is used
here only to hold device memory and to name the current stream.  If the
library is missing, every call raises MoEError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
NUM_STAGES = 7
STAGE_NAMES = ("router", "tile_rank", "dispatch_scan", "scatter", "expert_gemm1_swiglu",
               "expert_gemm2_down", "combine")
_DTYPES = {torch.float32: MOE_DTYPE_F32, torch.bfloat16: MOE_DTYPE_BF16}

EXPORTED = ("moe_last_error", "moe_workspace_size", "moe_layer_forward",
            "moe_layer_forward_static", "moe_route",
            "moe_dispatch_workspace_size", "moe_dispatch", "moe_expert_ffn_workspace_size",
            "moe_expert_ffn", "moe_combine", "moe_balance_workspace_size", "moe_balance_stats",
            "moe_backward_workspace_size", "moe_layer_backward", "moe_timing_enable",
            "moe_timing_read", "moe_timing_stages")


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"moe status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libmoe.so and declare its C signatures (loading needs no GPU)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise MoEError(-1, f"{path} is not built (python -m mixture_experts_ffn_fp32_amd.build)")
    L = ctypes.CDLL(path)
    vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    szp = ctypes.POINTER(ctypes.c_size_t)
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    sigs = {
        "moe_workspace_size": [i, i, i, i, i, i, i, szp],
        "moe_layer_forward": [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, sz, vp],
        "moe_layer_forward_static": [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp],
        "moe_route": [vp, vp, f, i, i, i, i, i, vp, vp, vp, vp],
        "moe_dispatch_workspace_size": [i, i, i, szp],
        "moe_dispatch": [vp, i, i, i, vp, vp, vp, vp, sz, vp],
        "moe_expert_ffn_workspace_size": [i, i, i, i, szp],
        "moe_expert_ffn": [vp, vp, vp, i, i, i, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_combine": [vp, vp, vp, i, i, i, i, i, vp, vp],
        "moe_balance_workspace_size": [i, i, szp],
        "moe_balance_stats": [vp, vp, i, i, i, vp, i, ctypes.c_float, ctypes.c_float, vp, vp, vp,
                              vp, vp, vp, sz, vp],
        "moe_backward_workspace_size": [i, i, i, i, i, i, i, szp],
        "moe_layer_backward": [vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp,
                               sz, vp],
        "moe_timing_enable": [i],
        "moe_timing_read": [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)],
        "moe_timing_stages": [ctypes.c_uint],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise MoEError(status, load_library().moe_last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(*tensors, dtype=None):
    """Every tensor must live on a GPU, be contiguous and (if given) of dtype."""
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise MoEError(1, "tensors must be on a GPU device")
        if not t.is_contiguous():
            raise MoEError(1, "tensors must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise MoEError(1, f"expected dtype {dtype}, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t) -> int:
    if t.dtype not in _DTYPES:
        raise MoEError(2, f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _infer_I(W_routed, N: int, d: int) -> int:
    n = W_routed.numel()
    if N <= 0 or d <= 0 or n % (3 * N * d) != 0:
        raise MoEError(1, "W_routed must hold N blocks of 3*I*d elements")
    return n // (3 * N * d)


def workspace_size(T, d, I, N, K, K_s, dtype_code) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(T, d, I, N, K, K_s, dtype_code, ctypes.byref(out)))
    return out.value


def layer_forward(u, E_gate, W_routed, W_shared, N: int, K: int, K_s: int, gate_bias=None,
                  out=None, workspace=None):
    """h = u + sum_shared FFN(u) + sum_topK g FFN(u); see include/moe.h."""
    L = load_library()
    T, d = u.shape
    dt = _dtype_code(u)
    _dev(u, E_gate, W_routed, W_shared, dtype=u.dtype)
    _dev(gate_bias, dtype=torch.float32)
    I = _infer_I(W_routed, N, d)
    h = torch.empty_like(u) if out is None else out
    _dev(h, dtype=u.dtype)
    need = workspace_size(T, d, I, N, K, K_s, dt)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=u.device)
    _dev(workspace)
    _check(L.moe_layer_forward(_p(u), _p(E_gate), _p(W_routed), _p(W_shared), N, K, K_s, T, d, I,
                               dt, _p(gate_bias), _p(h), _p(workspace),
                               workspace.numel() * workspace.element_size(), _stream()))
    return h


def layer_forward_static(u, E_gate, W_routed, W_shared, N: int, K: int, K_s: int,
                         gate_bias=None, out=None):
    """The layer forward with the library's static device scratch as its workspace (no
    device allocation inside the call; `out` may be given so that none is made here
    either).  Shapes needing more than MOE_STATIC_SCRATCH_BYTES raise MoEError."""
    L = load_library()
    T, d = u.shape
    dt = _dtype_code(u)
    _dev(u, E_gate, W_routed, W_shared, dtype=u.dtype)
    _dev(gate_bias, dtype=torch.float32)
    I = _infer_I(W_routed, N, d)
    h = torch.empty_like(u) if out is None else out
    _dev(h, dtype=u.dtype)
    _check(L.moe_layer_forward_static(_p(u), _p(E_gate), _p(W_routed), _p(W_shared), N, K, K_s,
                                      T, d, I, dt, _p(gate_bias), _p(h), _stream()))
    return h


def backward_workspace_size(T, d, I, N, K, K_s, dtype_code) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_backward_workspace_size(T, d, I, N, K, K_s, dtype_code,
                                                      ctypes.byref(out)))
    return out.value


def layer_backward(u, E_gate, W_routed, W_shared, N: int, K: int, K_s: int, dh, gate_bias=None,
                   workspace=None):
    """Gradients of sum(dh * h) for h = layer_forward(u, ...); see include/moe.h.

    Returns (du, dE_gate, dgate_bias, dW_routed, dW_shared or None); every gradient
    but du is float32, the weight gradients in the layout of their weights.  The
    bias gradient is the same whether or not a bias is given.
    """
    L = load_library()
    T, d = u.shape
    dt = _dtype_code(u)
    _dev(u, E_gate, W_routed, W_shared, dh, dtype=u.dtype)
    _dev(gate_bias, dtype=torch.float32)
    I = _infer_I(W_routed, N, d)
    dev = u.device
    # an empty batch writes nothing: its weight gradients are zeros
    alloc = torch.zeros if T == 0 else torch.empty
    du = torch.empty_like(u)
    dE = alloc(E_gate.shape, dtype=torch.float32, device=dev)
    db = alloc(N, dtype=torch.float32, device=dev)
    dWr = alloc(W_routed.shape, dtype=torch.float32, device=dev)
    dWs = None if K_s == 0 else alloc(W_shared.shape, dtype=torch.float32, device=dev)
    need = backward_workspace_size(T, d, I, N, K, K_s, dt)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _dev(workspace)
    _check(L.moe_layer_backward(_p(u), _p(E_gate), _p(W_routed), _p(W_shared), N, K, K_s, T, d, I,
                                dt, _p(gate_bias), _p(dh), _p(du), _p(dE), _p(db), _p(dWr),
                                _p(dWs), _p(workspace),
                                workspace.numel() * workspace.element_size(), _stream()))
    return du, dE, db, dWr, dWs


def route(u, E_gate, K: int, gate_bias=None, want_scores: bool = False):
    """(idx [T][K] int32, gate [T][K] float32, scores [T][N] float32 or None)."""
    L = load_library()
    T, d = u.shape
    N = E_gate.shape[0]
    _dev(u, E_gate, dtype=u.dtype)
    _dev(gate_bias, dtype=torch.float32)
    idx = torch.empty((T, K), dtype=torch.int32, device=u.device)
    gate = torch.empty((T, K), dtype=torch.float32, device=u.device)
    scores = torch.empty((T, N), dtype=torch.float32, device=u.device) if want_scores else None
    _check(L.moe_route(_p(u), _p(E_gate), _p(gate_bias), T, d, N, K, _dtype_code(u), _p(idx),
                       _p(gate), _p(scores), _stream()))
    return idx, gate, scores


def dispatch(idx, N: int):
    """(counts [N], offsets [N+1], sorted_pair [T*K]) int32, grouped by expert, stable."""
    L = load_library()
    T, K = idx.shape
    _dev(idx, dtype=torch.int32)
    out = ctypes.c_size_t(0)
    _check(L.moe_dispatch_workspace_size(T, N, K, ctypes.byref(out)))
    ws = torch.empty(max(out.value, 1), dtype=torch.uint8, device=idx.device)
    counts = torch.empty(N, dtype=torch.int32, device=idx.device)
    offsets = torch.empty(N + 1, dtype=torch.int32, device=idx.device)
    sorted_pair = torch.empty(max(T * K, 1), dtype=torch.int32, device=idx.device)
    _check(L.moe_dispatch(_p(idx), T, N, K, _p(counts), _p(offsets), _p(sorted_pair), _p(ws),
                          ws.numel(), _stream()))
    return counts, offsets, sorted_pair[:T * K]


def expert_ffn(u, W_routed, W_shared, N: int, K: int, K_s: int, offsets, sorted_pair, gate):
    """(H_routed [T*K][I], H_shared [T][K_s*I] or None, Y [T*K][d], Y_shared [T][d] or None)."""
    L = load_library()
    T, d = u.shape
    dt = _dtype_code(u)
    _dev(u, W_routed, W_shared, dtype=u.dtype)
    _dev(offsets, sorted_pair, dtype=torch.int32)
    _dev(gate, dtype=torch.float32)
    I = _infer_I(W_routed, N, d)
    out = ctypes.c_size_t(0)
    _check(L.moe_expert_ffn_workspace_size(T, N, K, K_s, ctypes.byref(out)))
    ws = torch.empty(max(out.value, 1), dtype=torch.uint8, device=u.device)
    H = torch.empty((T * K, I), dtype=u.dtype, device=u.device)
    Y = torch.empty((T * K, d), dtype=u.dtype, device=u.device)
    Hs = torch.empty((T, K_s * I), dtype=u.dtype, device=u.device) if K_s > 0 else None
    Ys = torch.empty((T, d), dtype=u.dtype, device=u.device) if K_s > 0 else None
    _check(L.moe_expert_ffn(_p(u), _p(W_routed), _p(W_shared), T, d, I, N, K, K_s, dt,
                            _p(offsets), _p(sorted_pair), _p(gate), _p(H), _p(Hs), _p(Y), _p(Ys),
                            _p(ws), ws.numel(), _stream()))
    return H, Hs, Y, Ys


def combine(u, Y, Y_shared, K: int, K_s: int):
    """h = u + Y_shared + sum_k Y[t*K+k]."""
    L = load_library()
    T, d = u.shape
    _dev(u, Y, Y_shared, dtype=u.dtype)
    h = torch.empty_like(u)
    _check(L.moe_combine(_p(u), _p(Y), _p(Y_shared), T, d, K, K_s, _dtype_code(u), _p(h),
                         _stream()))
    return h


def balance_stats(scores, idx, K: int, group_of=None, alpha1: float = 1.0, alpha2: float = 1.0):
    """Balance statistics of one batch: dict of f [N], P [N], L_ExpBal and, with
    group_of (a length-N sequence of device-group ids 0..D-1), f_dev [D],
    P_dev [D], L_DevBal.  Tensors are float32 on the scores' device."""
    L = load_library()
    T, N = scores.shape
    _dev(scores, dtype=torch.float32)
    _dev(idx, dtype=torch.int32)
    if idx.shape != (T, K):
        raise MoEError(1, "idx must be [T][K]")
    D = 0
    groups = None
    if group_of is not None:
        g = [int(x) for x in group_of]
        if len(g) != N:
            raise MoEError(1, "group_of must have N entries")
        D = max(g) + 1 if g else 0
        groups = (ctypes.c_int32 * N)(*g)
    out = ctypes.c_size_t(0)
    _check(L.moe_balance_workspace_size(T, N, ctypes.byref(out)))
    dev = scores.device
    ws = torch.empty(max(out.value, 1), dtype=torch.uint8, device=dev)
    f = torch.empty(N, dtype=torch.float32, device=dev)
    P = torch.empty(N, dtype=torch.float32, device=dev)
    fd = torch.empty(max(D, 1), dtype=torch.float32, device=dev)
    Pd = torch.empty(max(D, 1), dtype=torch.float32, device=dev)
    losses = torch.empty(2, dtype=torch.float32, device=dev)
    _check(L.moe_balance_stats(_p(scores), _p(idx), T, N, K, groups, D, alpha1, alpha2, _p(f),
                               _p(P), _p(fd), _p(Pd), _p(losses), _p(ws), ws.numel(), _stream()))
    res = {"f": f, "P": P, "L_ExpBal": losses[0]}
    if group_of is not None:
        res.update({"f_dev": fd[:D], "P_dev": Pd[:D], "L_DevBal": losses[1]})
    return res


def timing_enable(on: bool = True, stages=None):
    """Per-stage event timing on or off; `stages` (names) limits it to those stages."""
    L = load_library()
    mask = 0xFFFFFFFF if stages is None else sum(1 << STAGE_NAMES.index(s) for s in stages)
    _check(L.moe_timing_stages(mask))
    _check(L.moe_timing_enable(1 if on else 0))


def timing_read():
    """{stage name: (total ms, launches)} for the stage launches since the last read."""
    ms = (ctypes.c_double * NUM_STAGES)()
    n = (ctypes.c_int * NUM_STAGES)()
    _check(load_library().moe_timing_read(ms, n))
    return {STAGE_NAMES[i]: (ms[i], n[i]) for i in range(NUM_STAGES)}
