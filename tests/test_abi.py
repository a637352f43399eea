"""The C ABI on the CPU: the library loads, exports what include/moe.h declares,
and rejects bad arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

mx = pytest.importorskip("mixture_experts_ffn_fp32_amd")
from mixture_experts_ffn_fp32_amd import moe as binding  # noqa: E402

OK, INVALID, UNSUPPORTED, WORKSPACE, ALIGNMENT = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libmoe.so is not built: run python -m mixture_experts_ffn_fp32_amd.build")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} not exported"


def _ws(lib, *shape):
    out = ctypes.c_size_t(0)
    st = lib.moe_workspace_size(*shape, ctypes.byref(out))
    return st, out.value


def test_workspace_size_validation(lib):
    # T, d, I, N, K, K_s, dtype
    assert _ws(lib, 8192, 2048, 1408, 64, 6, 2, 1)[0] == OK
    assert _ws(lib, 0, 2048, 1408, 64, 6, 2, 1) == (OK, 0)
    cases = [
        ((8192, 2048, 1400, 64, 6, 2, 1), UNSUPPORTED),   # I not a multiple of 64
        ((8192, 2000, 1408, 64, 6, 2, 1), UNSUPPORTED),   # d not a multiple of 64
        ((8192, 2048, 1408, 64, 65, 2, 1), INVALID),      # K > N
        ((8192, 2048, 1408, 64, 0, 2, 1), INVALID),       # K < 1
        ((8192, 2048, 1408, 0, 1, 2, 1), INVALID),        # N < 1
        ((8192, 2048, 1408, 257, 6, 2, 1), UNSUPPORTED),  # N > 256
        ((8192, 2048, 1408, 64, 6, 17, 1), UNSUPPORTED),  # K_s > 16
        ((8192, 2048, 1408, 64, 6, -1, 1), INVALID),
        ((-1, 2048, 1408, 64, 6, 2, 1), INVALID),
        ((8192, 2048, 1408, 64, 6, 2, 7), UNSUPPORTED),   # dtype
        ((8192, 0, 1408, 64, 6, 2, 1), INVALID),
    ]
    for shape, want in cases:
        st, _ = _ws(lib, *shape)
        assert st == want, (shape, st, lib.moe_last_error())
        assert lib.moe_last_error().decode()


def test_operands_past_2gib_are_refused(lib):
    """Operand rows are addressed as 32-bit byte offsets inside a 2 GiB buffer range:
    shapes whose u, H_routed, H_shared or one expert's weights would span more are
    refused with MOE_ERR_UNSUPPORTED instead of computing a wrong h."""
    # T, d, I, N, K, K_s, dtype
    cases = [
        (32768, 2048, 1536, 64, 12, 2, 0),     # f32 H_routed: 32768*12*1536*4 = 2.4 GB
        (65536, 16384, 64, 8, 1, 0, 1),        # bf16 u: 65536*16384*2 = 2 GiB
        (65536, 1024, 2048, 8, 1, 16, 1),      # bf16 H_shared: 65536*16*2048*2 = 4 GiB
        (1, 16384, 32768, 8, 1, 0, 1),         # one expert block 3*I*d*2 = 3 GiB
    ]
    for shape in cases:
        st, _ = _ws(lib, *shape)
        assert st == UNSUPPORTED, (shape, st)
        assert "2^31" in lib.moe_last_error().decode()
    # the largest workload shape stays well inside the limit
    assert _ws(lib, 16384, 4096, 1536, 128, 12, 4, 1)[0] == OK
    out = ctypes.c_size_t(0)
    assert lib.moe_backward_workspace_size(16384, 4096, 1536, 128, 12, 4, 1,
                                           ctypes.byref(out)) == OK
    # the backward's [da dc] rows: 2 * H_routed
    assert lib.moe_backward_workspace_size(20000, 1024, 4096, 64, 8, 0, 1,
                                           ctypes.byref(out)) == UNSUPPORTED
    assert lib.moe_workspace_size(20000, 1024, 4096, 64, 8, 0, 1, ctypes.byref(out)) == OK


def test_workspace_size_grows_with_tokens(lib):
    sizes = [_ws(lib, T, 2048, 1408, 64, 6, 2, 1)[1] for T in (1, 64, 65, 1000, 8192)]
    assert sizes == sorted(sizes) and len(set(sizes)) == len(sizes)
    # at least the token-proportional buffers: H (T*K + T*K_s) * I and Y (T*K + T) * d
    T = 8192
    assert sizes[-1] >= 2 * (T * 8 * 1408 + T * 7 * 2048)


def _fwd(lib, u=16, E=16, Wr=16, Ws=16, h=1 << 20, ws=1 << 24, wsb=1 << 40, N=64, K=6, K_s=2, T=8,
         d=2048, I=1408, dt=1, bias=None):
    p = lambda x: None if x is None else ctypes.c_void_p(x)   # noqa: E731
    return lib.moe_layer_forward(p(u), p(E), p(Wr), p(Ws), N, K, K_s, T, d, I, dt, p(bias), p(h),
                                 p(ws), wsb, None)


def test_forward_validation_never_reaches_the_gpu(lib):
    # every case fails validation, which runs before any HIP call
    assert _fwd(lib, u=None) == INVALID
    assert _fwd(lib, u=8) == ALIGNMENT
    assert _fwd(lib, Ws=None) == INVALID
    assert _fwd(lib, bias=4) == ALIGNMENT
    assert _fwd(lib, ws=None) == INVALID
    assert _fwd(lib, wsb=1024) == WORKSPACE
    assert _fwd(lib, h=16) == INVALID                   # h overlaps u
    assert _fwd(lib, K=0) == INVALID
    assert _fwd(lib, I=100) == UNSUPPORTED
    assert _fwd(lib, dt=3) == UNSUPPORTED
    assert "aligned" in (_fwd(lib, u=8), lib.moe_last_error().decode())[1]


def test_empty_batch_is_a_no_op(lib):
    assert _fwd(lib, T=0, u=None, h=None, ws=None, wsb=0) == OK


def test_stage_validation(lib):
    p = ctypes.c_void_p
    assert lib.moe_route(None, p(16), None, 4, 64, 8, 9, 1, p(16), p(16), None, None) == INVALID
    assert lib.moe_route(p(16), p(16), None, 4, 65, 8, 2, 1, p(16), p(16), None, None) == UNSUPPORTED
    assert lib.moe_dispatch(p(16), 4, 8, 2, p(16), p(16), p(16), p(16), 0, None) == WORKSPACE
    out = ctypes.c_size_t(0)
    assert lib.moe_dispatch_workspace_size(4, 8, 2, ctypes.byref(out)) == OK and out.value > 0
    assert lib.moe_expert_ffn_workspace_size(4, 8, 2, 1, ctypes.byref(out)) == OK and out.value > 0
    assert lib.moe_combine(p(16), None, None, 4, 64, 2, 0, 1, p(4096), None) == INVALID
    assert lib.moe_combine(p(16), p(32), None, 4, 64, 2, 1, 1, p(4096), None) == INVALID


def test_binding_refuses_host_tensors():
    import torch
    u = torch.zeros(4, 64)
    with pytest.raises(mx.MoEError):
        mx.layer_forward(u, torch.zeros(8, 64), torch.zeros(8 * 3 * 64 * 64), None, 8, 2, 0)


def _bal(lib, scores=16, idx=32, T=8, N=8, K=2, group_of=None, D=0, f=64, P=96, fd=128, Pd=160,
         losses=192, ws=4096, wsb=1 << 30):
    p = lambda x: None if x is None else ctypes.c_void_p(x)   # noqa: E731
    g = None if group_of is None else (ctypes.c_int32 * len(group_of))(*group_of)
    return lib.moe_balance_stats(p(scores), p(idx), T, N, K, g, D, 1.0, 1.0, p(f), p(P), p(fd),
                                 p(Pd), p(losses), p(ws), wsb, None)


def test_balance_validation_never_reaches_the_gpu(lib):
    out = ctypes.c_size_t(0)
    assert lib.moe_balance_workspace_size(8, 8, ctypes.byref(out)) == OK and out.value > 0
    assert lib.moe_balance_workspace_size(0, 8, ctypes.byref(out)) == INVALID
    assert lib.moe_balance_workspace_size(8, 257, ctypes.byref(out)) == UNSUPPORTED
    assert _bal(lib, T=0) == INVALID                       # the statistics divide by T
    assert _bal(lib, K=9) == INVALID
    assert _bal(lib, scores=None) == INVALID
    assert _bal(lib, f=8) == ALIGNMENT
    assert _bal(lib, wsb=16) == WORKSPACE
    assert _bal(lib, group_of=[0, 0, 1, 1, 2, 2, 3, 3], D=4, fd=None) == INVALID
    assert _bal(lib, group_of=[0, 0, 1, 1, 2, 2, 3, 4], D=4) == INVALID   # id outside [0, D)
    assert "outside" in lib.moe_last_error().decode()
    assert _bal(lib, group_of=[0, 0, 1, 1, 3, 3, 3, 3], D=4) == INVALID   # group 2 is empty
    assert "no expert" in lib.moe_last_error().decode()
    assert _bal(lib, group_of=[0] * 8, D=9) == INVALID


def _bwd(lib, u=16, E=16, Wr=16, Ws=16, dh=1 << 20, du=1 << 22, dE=1 << 23, db=None,
         dWr=1 << 24, dWs=1 << 25, ws=1 << 44, wsb=1 << 40, N=64, K=6, K_s=2, T=8, d=2048,
         I=1408, dt=1, bias=None):
    p = lambda x: None if x is None else ctypes.c_void_p(x)   # noqa: E731
    return lib.moe_layer_backward(p(u), p(E), p(Wr), p(Ws), N, K, K_s, T, d, I, dt, p(bias),
                                  p(dh), p(du), p(dE), p(db), p(dWr), p(dWs), p(ws), wsb, None)


def test_backward_validation_never_reaches_the_gpu(lib):
    out = ctypes.c_size_t(0)
    assert lib.moe_backward_workspace_size(8, 2048, 1408, 64, 6, 2, 1, ctypes.byref(out)) == OK
    small = out.value
    assert lib.moe_backward_workspace_size(64, 2048, 1408, 64, 6, 2, 1, ctypes.byref(out)) == OK
    assert out.value > small > 0
    assert lib.moe_backward_workspace_size(0, 2048, 1408, 64, 6, 2, 1, ctypes.byref(out)) == OK
    assert out.value == 0
    assert lib.moe_backward_workspace_size(8, 2048, 1400, 64, 6, 2, 1,
                                           ctypes.byref(out)) == UNSUPPORTED
    assert _bwd(lib, dh=None) == INVALID
    assert _bwd(lib, du=None) == INVALID
    assert _bwd(lib, dE=None) == INVALID
    assert _bwd(lib, dWr=None) == INVALID
    assert _bwd(lib, dWs=None) == INVALID                 # K_s > 0 needs dW_shared
    assert _bwd(lib, db=8) == ALIGNMENT
    assert _bwd(lib, wsb=1024) == WORKSPACE
    assert _bwd(lib, du=16) == INVALID                    # du overlaps u
    assert "du overlaps u" in lib.moe_last_error().decode()
    assert _bwd(lib, du=(1 << 20) + 64) == INVALID        # du overlaps dh
    assert _bwd(lib, du=(1 << 44) + 256) == INVALID       # du overlaps the workspace
    assert _bwd(lib, dWr=(1 << 44) - 4096) == INVALID     # dW_routed overlaps the workspace
    assert _bwd(lib, K=65) == INVALID
    assert _bwd(lib, T=0, u=None, dh=None, du=None, ws=None, wsb=0) == OK


def test_backward_binding_refuses_host_tensors():
    import torch
    u = torch.zeros(4, 64)
    with pytest.raises(mx.MoEError):
        mx.layer_backward(u, torch.zeros(8, 64), torch.zeros(8 * 3 * 64 * 64), None, 8, 2, 0,
                          torch.zeros(4, 64))
