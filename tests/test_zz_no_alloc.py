"""The allocation-free entry point, fn_norm_linear_noalloc, through the C
ABI: its output equals that of fn_norm_linear (FN_FUSED, with a workspace
from torch) bit for bit, on two calls in a row, the second with a smaller
input (the shared scratch keeps the first call's values past the second
call's rows).  Both shapes take the row-statistics pass, the kernels that
use the scratch.  A shape that needs more scratch than the library holds is
refused before anything runs.  Every case prints its name first."""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import bits_of, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _noalloc(lib, x, Ws, eps, y):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return lib.fn_norm_linear_noalloc(P(x), 1, x.shape[0], x.shape[1], P(Ws), 1, Ws.shape[0], eps, P(y),
                                      0 if y.dtype == torch.float32 else 1, st)


@pytest.mark.parametrize("force_pass", [True, False])
def test_noalloc_matches_the_workspace_entry_point(gpu_lib, monkeypatch, force_pass):
    fn = gpu_lib
    lib = fn.load()
    if force_pass:
        monkeypatch.setenv("FN_PRESTATS", "1")
        shapes = [(3000, 1032, 700), (500, 520, 300)]
    else:  # the library's own choice: shapes large enough to take the pass
        monkeypatch.delenv("FN_PRESTATS", raising=False)
        shapes = [(4096, 4096, 4096), (2048, 4096, 4096)]
    for M, K, N in shapes:
        w = synth.workload("llama7b_qkv_prefill_bf16").with_shape(M, K, N)
        need = fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.FUSED, M, K, N, torch.bfloat16)
        assert need > 0, "the shape must use the scratch"
        x, g = to_dev(w.x()), torch.from_numpy(w.g()).cuda()
        Ws = fn.fold_weights(to_dev(w.w()), g)
        for od in (torch.float32, torch.bfloat16):
            _say(f"noalloc {M}x{K}x{N} out={od} (scratch {need} bytes) against fn_norm_linear")
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            y_ref = fn.norm_linear(x, Ws, w.eps_f32(), out_dtype=od, ws=ws)
            y = torch.full((M, N), float("nan"), dtype=od, device="cuda")
            assert _noalloc(lib, x, Ws, w.eps_f32(), y) == 0, lib.fn_last_error().decode()
            torch.cuda.synchronize()
            assert np.array_equal(bits_of(y), bits_of(y_ref))
            # and through the binding
            y2 = torch.full((M, N), float("nan"), dtype=od, device="cuda")
            fn.norm_linear_noalloc(x, Ws, w.eps_f32(), out=y2)
            torch.cuda.synchronize()
            assert np.array_equal(bits_of(y2), bits_of(y_ref))


def test_noalloc_refuses_more_than_its_scratch(gpu_lib, monkeypatch):
    fn = gpu_lib
    lib = fn.load()
    monkeypatch.setenv("FN_PRESTATS", "1")
    M, K, N = (1 << 20) + 64, 64, 256  # row statistics of more than 2^20 rows
    _say(f"noalloc refuses M={M}: more row statistics than the 4 MiB scratch holds")
    x = torch.zeros(16, 64, dtype=torch.bfloat16, device="cuda")
    y = torch.full((16, 16), 7.0, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    status = lib.fn_norm_linear_noalloc(P(x), 1, M, K, P(x), 1, N, 1e-6, P(y), 0, st)
    assert status == 5 and b"scratch" in lib.fn_last_error()
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
