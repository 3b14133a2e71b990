"""Python binding of libflashnorm (FlashNorm norm-then-project on MI355X).

Argument marshalling only: tensors are checked for device, dtype and
contiguity, outputs and workspaces are allocated with torch (device memory
is PyTorch's job here), and the raw pointers plus the current HIP stream go
to the C ABI declared in ``include/flashnorm.h``.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashnorm.so")

FN_OK = 0
FN_F32, FN_BF16, FN_E4M3 = 0, 1, 2
FUSED, UNFUSED, TWO_STREAM, FUSED_PACKED = 0, 1, 2, 3
(OP_NORM_LINEAR, OP_NORM_GLU_FFN, OP_LINEAR_QKNORM, OP_LINEAR_QKNORM_ROPE, OP_LAYERNORM_LINEAR,
 OP_NORM_LINEAR_FP8, OP_NORM_GLU_FFN_FP8, OP_LINEAR_LATENT_NORM) = range(8)

_STATUS = {0: "FN_OK", 1: "FN_E_NULL", 2: "FN_E_SHAPE", 3: "FN_E_DTYPE", 4: "FN_E_ALIGN",
           5: "FN_E_WORKSPACE", 6: "FN_E_UNSUPPORTED", 7: "FN_E_HIP", 8: "FN_E_ARG"}

_lib: Optional[ctypes.CDLL] = None


class FlashNormError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libflashnorm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with `python -m rmsnorm_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i64, c_int, c_vp, c_f, c_sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.fn_abi_version.restype = c_int
    lib.fn_last_error.restype = ctypes.c_char_p
    lib.fn_status_string.restype = ctypes.c_char_p
    lib.fn_status_string.argtypes = [c_int]
    lib.fn_workspace_bytes.argtypes = [c_int, c_int, c_i64, c_i64, c_i64, c_int, ctypes.POINTER(c_sz)]
    lib.fn_dispatch_name.argtypes = [c_int, c_int, c_i64, c_i64, c_i64, c_int, c_int, ctypes.c_char_p, c_sz]
    lib.fn_fold_weights.argtypes = [c_vp, c_int, c_vp, c_i64, c_i64, c_vp, c_int, c_vp]
    lib.fn_norm_linear.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_i64, c_vp, c_f, c_vp, c_int, c_int,
                                   c_vp, c_sz, c_vp, c_vp]
    lib.fn_norm_glu_ffn.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_int, c_i64, c_vp, c_f, c_vp, c_int,
                                    c_int, c_vp, c_sz, c_vp]
    lib.fn_linear_qknorm.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_int, c_int, c_int, c_vp, c_vp,
                                     c_i64, c_f, c_f, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_sz, c_vp]
    lib.fn_linear_qknorm_rope.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_int, c_int, c_int, c_vp,
                                          c_vp, c_i64, c_f, c_f, c_int, c_vp, c_vp, c_i64, c_int, c_vp, c_vp, c_int,
                                          c_int, c_vp, c_sz, c_vp]
    lib.fn_rope_table.argtypes = [ctypes.c_double, c_int, c_i64, c_vp, c_vp]
    lib.fn_fold_layernorm.argtypes = [c_vp, c_int, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_int, c_vp, c_vp, c_vp]
    lib.fn_layernorm_linear.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp,
                                        c_f, c_vp, c_int, c_int, c_vp, c_sz, c_vp]
    lib.fn_linear_latent_norm.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_vp,
                                          c_f, c_f, c_vp, c_vp, c_i64, c_int, c_vp, c_vp, c_int, c_int, c_vp, c_sz,
                                          c_vp]
    lib.fn_quantize_fp8.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp]
    lib.fn_norm_linear_fp8.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_f, c_vp, c_int, c_int,
                                       c_vp, c_sz, c_vp]
    lib.fn_norm_glu_ffn_fp8.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_f, c_vp,
                                        c_int, c_int, c_vp, c_sz, c_vp]
    lib.fn_decode_packed_bytes.argtypes = [c_int, c_i64, c_i64, ctypes.POINTER(c_sz)]
    lib.fn_pack_decode_weights.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_vp]
    lib.fn_pack_decode_weights_glu.argtypes = [c_vp, c_vp, c_int, c_i64, c_i64, c_vp, c_vp]
    for f in ("fn_workspace_bytes", "fn_dispatch_name", "fn_fold_weights", "fn_norm_linear", "fn_norm_glu_ffn",
              "fn_linear_qknorm", "fn_linear_qknorm_rope", "fn_rope_table", "fn_fold_layernorm",
              "fn_layernorm_linear", "fn_quantize_fp8", "fn_norm_linear_fp8", "fn_norm_glu_ffn_fp8",
              "fn_linear_latent_norm", "fn_decode_packed_bytes", "fn_pack_decode_weights",
              "fn_pack_decode_weights_glu"):
        getattr(lib, f).restype = c_int
    lib.fn_shutdown.restype = None
    lib.fn_norm_linear_noalloc.argtypes = [c_vp, c_int, c_i64, c_i64, c_vp, c_int, c_i64, c_f, c_vp, c_int, c_vp]
    lib.fn_norm_linear_noalloc.restype = c_int
    lib.fn_testing_skip_join.argtypes = [c_int]
    lib.fn_testing_skip_join.restype = c_int
    lib.fn_testing_gemm_events.argtypes = [c_vp, c_vp, c_int]
    lib.fn_testing_gemm_events.restype = c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != FN_OK:
        raise FlashNormError(status, load().fn_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FN_F32
    if t.dtype == torch.bfloat16:
        return FN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dt(code: int):
    return torch.float32 if code == FN_F32 else torch.bfloat16


def _ptr(t: Optional[torch.Tensor]):
    """The device address of a contiguous GPU tensor, as an int (the
    arguments are declared void*, so ctypes converts it)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


# The current device's current stream as a raw handle, without building a
# torch.cuda.Stream object (about 2.5 us a call through the public API,
# more than the rest of a small call's host work).
if hasattr(torch._C, "_cuda_getCurrentRawStream") and hasattr(torch._C, "_cuda_getDevice"):
    def _current_raw_stream() -> int:
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
else:  # pragma: no cover - older torch
    def _current_raw_stream() -> int:
        return torch.cuda.current_stream().cuda_stream


def _stream(s: Optional[torch.cuda.Stream]):
    return _current_raw_stream() if s is None else s.cuda_stream


def _gain(g: Optional[torch.Tensor]):
    if g is None:
        return None
    if g.dtype != torch.float32:
        raise TypeError("gains are float32")
    return g


_ws_cache = {}


def workspace_bytes(op: int, variant: int, M: int, K: int, N: int, x_dtype: torch.dtype) -> int:
    """Workspace the library needs for a call (memoised: a pure function of
    the arguments and of FN_PRESTATS, which selects the statistics pass)."""
    code = FN_F32 if x_dtype == torch.float32 else FN_BF16
    key = (op, variant, M, K, N, code, os.environ.get("FN_PRESTATS"))
    hit = _ws_cache.get(key)
    if hit is not None:
        return hit
    out = ctypes.c_size_t(0)
    _check(load().fn_workspace_bytes(op, variant, M, K, N, code, ctypes.byref(out)))
    if len(_ws_cache) < 4096:
        _ws_cache[key] = out.value
    return out.value


def dispatch_name(op: int, variant: int, M: int, K: int, N: int, x_dtype: torch.dtype,
                  y_dtype: torch.dtype) -> str:
    buf = ctypes.create_string_buffer(256)
    xc = FN_F32 if x_dtype == torch.float32 else FN_BF16
    yc = FN_F32 if y_dtype == torch.float32 else FN_BF16
    _check(load().fn_dispatch_name(op, variant, M, K, N, xc, yc, buf, 256))
    return buf.value.decode()


def _empty(shape, dtype, device, stream=None):
    """torch.empty from the caching-allocator pool of the stream the call is
    enqueued on.  The allocator ties a block to the stream that allocated
    it, so a workspace freed when the wrapper returns is handed out again
    only to later work on that same stream, never while the call's kernels
    may still be reading it from another one."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(op, variant, M, K, N, x, ws, stream=None):
    need = workspace_bytes(op, variant, M, K, N, x.dtype)
    if need == 0:
        return None, 0
    if ws is None:
        ws = _empty(need, torch.uint8, x.device, stream)
    return ws, ws.numel() * ws.element_size()


class PackedWeight:
    """A weight in the decode-packed layout (``pack_decode_weights``): the
    uint8 buffer and the row-major shape it was packed from.  The op
    wrappers take it in place of the weight tensor and call the
    FUSED_PACKED variant."""

    def __init__(self, data: torch.Tensor, N: int, K: int, dtype: torch.dtype, pair: bool = False):
        self.data, self.N, self.K, self.dtype, self.pair = data, N, K, dtype, pair


def _packed_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return FN_BF16
    if dtype == torch.uint8:
        return FN_E4M3
    raise TypeError("decode-packed weights are bf16 or fp8 codes (uint8)")


def decode_packed_bytes(N: int, K: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(load().fn_decode_packed_bytes(_packed_code(dtype), N, K, ctypes.byref(out)))
    return out.value


def pack_decode_weights(W: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> PackedWeight:
    """Re-lay a row-major [N x K] weight (bf16 W*, or uint8 fp8 codes) for
    the weight-streaming kernel: 16-row slabs, each 64-byte K step stored as
    the 64 contiguous 16-byte pieces of one wave load."""
    lib = load()
    N, K = W.shape
    code = _packed_code(W.dtype)
    nbytes = decode_packed_bytes(N, K, W.dtype)
    if out is None:
        out = _empty(nbytes, torch.uint8, W.device, stream)
    elif out.dtype != torch.uint8 or out.numel() < nbytes:
        raise ValueError(f"out must be a uint8 buffer of at least {nbytes} bytes")
    _check(lib.fn_pack_decode_weights(_ptr(W), code, N, K, _ptr(out), _stream(stream)))
    return PackedWeight(out, N, K, W.dtype)


def pack_decode_weights_glu(W_gate: torch.Tensor, W_up: torch.Tensor, out: Optional[torch.Tensor] = None,
                            stream=None) -> PackedWeight:
    """Gate and up weights (bf16, or uint8 fp8 codes) in one decode-packed
    buffer, each K step holding the gate slab's pieces then the up slab's;
    pass it as the gate weight with the up weight None."""
    lib = load()
    if W_up.shape != W_gate.shape or W_up.dtype != W_gate.dtype:
        raise ValueError("W_gate and W_up must have the same shape and dtype")
    N, K = W_gate.shape
    nbytes = 2 * decode_packed_bytes(N, K, W_gate.dtype)
    if out is None:
        out = _empty(nbytes, torch.uint8, W_gate.device, stream)
    elif out.dtype != torch.uint8 or out.numel() < nbytes:
        raise ValueError(f"out must be a uint8 buffer of at least {nbytes} bytes")
    _check(lib.fn_pack_decode_weights_glu(_ptr(W_gate), _ptr(W_up), _packed_code(W_gate.dtype), N, K, _ptr(out),
                                          _stream(stream)))
    return PackedWeight(out, N, K, W_gate.dtype, pair=True)


def _weight(W, variant: int, K: int, allow_pair: bool = False):
    """(rows, pointer, variant) of a weight argument: a tensor keeps the
    caller's variant, a PackedWeight selects FUSED_PACKED."""
    if isinstance(W, PackedWeight):
        if variant not in (FUSED, FUSED_PACKED):
            raise ValueError("packed weights are read by the fused variant only")
        if W.pair and not allow_pair:
            raise ValueError("a gate/up pair buffer is the gate weight of a GLU op, not a single weight")
        if W.K != K:
            raise ValueError(f"packed weight has K={W.K}, x has K={K}")
        return W.N, _ptr(W.data), FUSED_PACKED
    if variant == FUSED_PACKED:
        raise ValueError("FUSED_PACKED takes a PackedWeight from pack_decode_weights")
    return W.shape[0], W, variant


def fold_weights(W: torch.Tensor, g: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """W* = round(g[k] * W[n, k]) (exact product, one rounding to out_dtype)."""
    lib = load()
    N, K = W.shape
    out_dtype = W.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((N, K), out_dtype, W.device, stream)
    _check(lib.fn_fold_weights(_ptr(W), _dt(W), _ptr(_gain(g)), N, K, _ptr(out), _dt(out), _stream(stream)))
    return out


def norm_linear(x: torch.Tensor, W: torch.Tensor, eps: float, g: Optional[torch.Tensor] = None,
                variant: int = FUSED, out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, stream=None, aux_stream=None) -> torch.Tensor:
    """y = RMSNorm(x) . W^T: fused (W folded, g None), unfused (W unfolded, g given) or two-stream."""
    lib = load()
    M, K = x.shape
    N, Wp, variant = _weight(W, variant, K)
    wdt = FN_BF16 if variant == FUSED_PACKED else _dt(W)
    Wp = Wp if variant == FUSED_PACKED else _ptr(W)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_NORM_LINEAR, variant, M, K, N, x, ws, stream)
    aux = None
    if variant == TWO_STREAM:
        if aux_stream is None:
            raise ValueError("the two-stream variant needs aux_stream")
        aux = ctypes.c_void_p(aux_stream.cuda_stream)
        if wsp is not None:
            wsp.record_stream(aux_stream)
    _check(lib.fn_norm_linear(_ptr(x), _dt(x), M, K, Wp, wdt, N, _ptr(_gain(g)), float(eps), _ptr(out),
                              _dt(out), variant, _ptr(wsp), wsb, _stream(stream), aux))
    return out


def norm_linear_noalloc(x: torch.Tensor, W_star: torch.Tensor, eps: float, out: torch.Tensor,
                        stream=None) -> torch.Tensor:
    """The fused norm_linear into a caller-provided `out`, allocating
    nothing (the row statistics go to the library's static device scratch;
    calls that overlap on one GPU race)."""
    lib = load()
    M, K = x.shape
    N = W_star.shape[0]
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M} x {N}]")
    _check(lib.fn_norm_linear_noalloc(_ptr(x), _dt(x), M, K, _ptr(W_star), _dt(W_star), N, float(eps), _ptr(out),
                                      _dt(out), _stream(stream)))
    return out


def norm_glu_ffn(x: torch.Tensor, W_gate: torch.Tensor, W_up: torch.Tensor, eps: float,
                 g: Optional[torch.Tensor] = None, variant: int = FUSED, out_dtype: Optional[torch.dtype] = None,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """h = SiLU(s * x.Wg*^T) * (s * x.Wu*^T) (fused) or the unfused baseline."""
    lib = load()
    M, K = x.shape
    if isinstance(W_gate, PackedWeight) and W_gate.pair and W_up is not None:
        raise ValueError("with the gate/up pair layout the up weight is None")
    N, Gp, v1 = _weight(W_gate, variant, K, allow_pair=True)
    if isinstance(W_gate, PackedWeight) and W_gate.pair:
        Up = None
    else:
        Nu, Up, _ = _weight(W_up, variant, K)
        if Nu != N or isinstance(W_gate, PackedWeight) != isinstance(W_up, PackedWeight):
            raise ValueError("W_gate and W_up must have the same shape and layout")
    variant = v1
    wdt = FN_BF16 if variant == FUSED_PACKED else _dt(W_gate)
    if variant != FUSED_PACKED:
        if W_up.shape != W_gate.shape:
            raise ValueError("W_gate and W_up must have the same shape")
        Gp, Up = _ptr(W_gate), _ptr(W_up)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_NORM_GLU_FFN, variant, M, K, N, x, ws, stream)
    _check(lib.fn_norm_glu_ffn(_ptr(x), _dt(x), M, K, Gp, Up, wdt, N, _ptr(_gain(g)),
                               float(eps), _ptr(out), _dt(out), variant, _ptr(wsp), wsb, _stream(stream)))
    return out


def linear_qknorm(x: torch.Tensor, W_qkv: torch.Tensor, n_q_heads: int, n_kv_heads: int, head_dim: int,
                  g_q: torch.Tensor, g_k: torch.Tensor, eps_x: float, eps_head: float, v_mode: int = 0,
                  g1: Optional[torch.Tensor] = None, variant: int = FUSED, out_dtype: Optional[torch.dtype] = None,
                  out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """QKV projection with per-head RMSNorm on q/k; the first RMSNorm dropped (fused)."""
    lib = load()
    M, K = x.shape
    N = W_qkv.shape[0]
    stride = 0 if g_q.dim() == 1 else g_q.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_LINEAR_QKNORM, variant, M, K, N, x, ws, stream)
    _check(lib.fn_linear_qknorm(_ptr(x), _dt(x), M, K, _ptr(W_qkv), _dt(W_qkv), n_q_heads, n_kv_heads, head_dim,
                                _ptr(_gain(g_q)), _ptr(_gain(g_k)), stride, float(eps_x), float(eps_head), v_mode,
                                _ptr(_gain(g1)), _ptr(out), _dt(out), variant, _ptr(wsp), wsb, _stream(stream)))
    return out


def rope_table(base: float, rot_dim: int, n_pos: int, device="cuda", out: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """[n_pos x rot_dim] float32 table of (cos, sin)(p * base^(-2i/rot_dim)) pairs."""
    lib = load()
    if out is None:
        out = _empty((n_pos, rot_dim), torch.float32, device, stream)
    _check(lib.fn_rope_table(float(base), rot_dim, n_pos, _ptr(out), _stream(stream)))
    return out


def linear_qknorm_rope(x: torch.Tensor, W_qkv: torch.Tensor, n_q_heads: int, n_kv_heads: int, head_dim: int,
                       g_q: torch.Tensor, g_k: torch.Tensor, eps_x: float, eps_head: float,
                       positions: torch.Tensor, table: torch.Tensor, v_mode: int = 0,
                       g1: Optional[torch.Tensor] = None, variant: int = FUSED,
                       out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                       ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """``linear_qknorm``, then q and k heads turned by the rotary embedding of
    each row's position (``positions`` int32 [M]; ``table`` from ``rope_table``,
    its width is the number of rotated columns per head)."""
    lib = load()
    M, K = x.shape
    N = W_qkv.shape[0]
    if positions.dtype != torch.int32:
        raise TypeError("positions are int32")
    if table.dtype != torch.float32 or table.dim() != 2:
        raise TypeError("table is a 2-D float32 tensor")
    stride = 0 if g_q.dim() == 1 else g_q.shape[1]
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_LINEAR_QKNORM_ROPE, variant, M, K, N, x, ws, stream)
    _check(lib.fn_linear_qknorm_rope(_ptr(x), _dt(x), M, K, _ptr(W_qkv), _dt(W_qkv), n_q_heads, n_kv_heads,
                                     head_dim, _ptr(_gain(g_q)), _ptr(_gain(g_k)), stride, float(eps_x),
                                     float(eps_head), v_mode, _ptr(positions), _ptr(table), table.shape[0],
                                     table.shape[1], _ptr(_gain(g1)), _ptr(out), _dt(out), variant, _ptr(wsp), wsb,
                                     _stream(stream)))
    return out


def fold_layernorm(W: torch.Tensor, g: torch.Tensor, beta: Optional[torch.Tensor] = None,
                   bias: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None, stream=None):
    """Offline LayerNorm fold: (W* = round(g W), colsum of the stored W*,
    b* = W beta + bias), the last two float32 [N]."""
    lib = load()
    N, K = W.shape
    out_dtype = W.dtype if out_dtype is None else out_dtype
    Ws = _empty((N, K), out_dtype, W.device, stream)
    c = _empty(N, torch.float32, W.device, stream)
    b = _empty(N, torch.float32, W.device, stream)
    _check(lib.fn_fold_layernorm(_ptr(W), _dt(W), _ptr(_gain(g)), _ptr(_gain(beta)), _ptr(_gain(bias)), N, K,
                                 _ptr(Ws), _dt(Ws), _ptr(c), _ptr(b), _stream(stream)))
    return Ws, c, b


def layernorm_linear(x: torch.Tensor, W: torch.Tensor, eps: float, colsum: Optional[torch.Tensor] = None,
                     b_star: Optional[torch.Tensor] = None, g: Optional[torch.Tensor] = None,
                     beta: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                     variant: int = FUSED, out_dtype: Optional[torch.dtype] = None,
                     out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """y = LayerNorm(x; g, beta) . W^T + bias: fused (W, colsum, b_star from
    ``fold_layernorm``) or unfused (W unfolded with g, beta, bias)."""
    lib = load()
    M, K = x.shape
    N, Wp, variant = _weight(W, variant, K)
    wdt = FN_BF16 if variant == FUSED_PACKED else _dt(W)
    Wp = Wp if variant == FUSED_PACKED else _ptr(W)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_LAYERNORM_LINEAR, variant, M, K, N, x, ws, stream)
    _check(lib.fn_layernorm_linear(_ptr(x), _dt(x), M, K, Wp, wdt, N, _ptr(_gain(colsum)),
                                   _ptr(_gain(b_star)), _ptr(_gain(g)), _ptr(_gain(beta)), _ptr(_gain(bias)),
                                   float(eps), _ptr(out), _dt(out), variant, _ptr(wsp), wsb, _stream(stream)))
    return out


def quantize_fp8(W: torch.Tensor, stream=None):
    """Per-output-channel OCP E4M3 quantisation: (codes uint8 [N x K],
    scales float32 [N]); the dequantised weight is scales[n] * value(code)."""
    lib = load()
    N, K = W.shape
    codes = _empty((N, K), torch.uint8, W.device, stream)
    scales = _empty(N, torch.float32, W.device, stream)
    _check(lib.fn_quantize_fp8(_ptr(W), _dt(W), N, K, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def _codes(t: torch.Tensor):
    if t.dtype != torch.uint8:
        raise TypeError("fp8 weights are uint8 codes")
    return _ptr(t)


def norm_linear_fp8(x: torch.Tensor, W8: torch.Tensor, scales: torch.Tensor, eps: float,
                    g: Optional[torch.Tensor] = None, variant: int = FUSED, out_dtype: Optional[torch.dtype] = None,
                    out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = RMSNorm(x) . W^T with fp8 W (codes and channel scales); for M > 16
    x is quantised per row to fp8 as well (see fn_norm_linear_fp8)."""
    lib = load()
    M, K = x.shape
    N, Wp, variant = _weight(W8, variant, K)
    Wp = Wp if variant == FUSED_PACKED else _codes(W8)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_NORM_LINEAR_FP8, variant, M, K, N, x, ws, stream)
    _check(lib.fn_norm_linear_fp8(_ptr(x), _dt(x), M, K, Wp, _ptr(_gain(scales)), N, _ptr(_gain(g)),
                                  float(eps), _ptr(out), _dt(out), variant, _ptr(wsp), wsb, _stream(stream)))
    return out


def norm_glu_ffn_fp8(x: torch.Tensor, W8_gate: torch.Tensor, s_gate: torch.Tensor, W8_up: torch.Tensor,
                     s_up: torch.Tensor, eps: float, g: Optional[torch.Tensor] = None, variant: int = FUSED,
                     out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """h = SiLU(s q_g a) * (s q_u b) on fp8 gate and up weights; for M > 16
    x is quantised per row to fp8 as well (see fn_norm_glu_ffn_fp8)."""
    lib = load()
    M, K = x.shape
    if isinstance(W8_gate, PackedWeight) and W8_gate.pair and W8_up is not None:
        raise ValueError("with the gate/up pair layout the up codes are None")
    N, Gp, v1 = _weight(W8_gate, variant, K, allow_pair=True)
    if isinstance(W8_gate, PackedWeight) and W8_gate.pair:
        Up = None
    else:
        Nu, Up, _ = _weight(W8_up, variant, K)
        if Nu != N or isinstance(W8_gate, PackedWeight) != isinstance(W8_up, PackedWeight):
            raise ValueError("W8_gate and W8_up must have the same shape and layout")
    variant = v1
    if variant != FUSED_PACKED:
        if W8_up.shape != W8_gate.shape:
            raise ValueError("W8_gate and W8_up must have the same shape")
        Gp, Up = _codes(W8_gate), _codes(W8_up)
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_NORM_GLU_FFN_FP8, variant, M, K, N, x, ws, stream)
    _check(lib.fn_norm_glu_ffn_fp8(_ptr(x), _dt(x), M, K, Gp, _ptr(_gain(s_gate)), Up,
                                   _ptr(_gain(s_up)), N, _ptr(_gain(g)), float(eps), _ptr(out), _dt(out), variant,
                                   _ptr(wsp), wsb, _stream(stream)))
    return out


def linear_latent_norm(x: torch.Tensor, W: torch.Tensor, n_q_latent: int, n_kv_latent: int, n_rope: int,
                       g_q_latent: Optional[torch.Tensor], g_kv_latent: Optional[torch.Tensor], eps_x: float,
                       eps_latent: float, positions: Optional[torch.Tensor] = None,
                       table: Optional[torch.Tensor] = None, g1: Optional[torch.Tensor] = None,
                       variant: int = FUSED, out_dtype: Optional[torch.dtype] = None,
                       out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """MLA attention input: [q latent | kv latent | rope part] with each latent
    RMS-normalised over its width, the first RMSNorm dropped (fused)."""
    lib = load()
    M, K = x.shape
    N = W.shape[0]
    if N != n_q_latent + n_kv_latent + n_rope:
        raise ValueError("W must have n_q_latent + n_kv_latent + n_rope rows")
    if positions is not None and positions.dtype != torch.int32:
        raise TypeError("positions are int32")
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = _empty((M, N), out_dtype, x.device, stream)
    wsp, wsb = _workspace(OP_LINEAR_LATENT_NORM, variant, M, K, N, x, ws, stream)
    n_pos, rot = (table.shape[0], table.shape[1]) if (positions is not None and table is not None) else (0, 0)
    _check(lib.fn_linear_latent_norm(_ptr(x), _dt(x), M, K, _ptr(W), _dt(W), n_q_latent, n_kv_latent, n_rope,
                                     _ptr(_gain(g_q_latent)), _ptr(_gain(g_kv_latent)), float(eps_x),
                                     float(eps_latent), _ptr(positions), _ptr(table) if positions is not None else None,
                                     n_pos, rot, _ptr(_gain(g1)), _ptr(out), _dt(out), variant, _ptr(wsp), wsb,
                                     _stream(stream)))
    return out
