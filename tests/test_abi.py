"""The C ABI library without a GPU: it loads, exports every entry point the
header declares, and answers the calls that do no device work."""

import ctypes
import glob
import os
import re

import pytest
import torch

import rmsnorm_linear_amd as fn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashnorm.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared(paths=None):
    names = set()
    for path in HEADERS if paths is None else paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(fn_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fn.LIB_PATH):
        pytest.fail("libflashnorm.so is not built (python -m rmsnorm_linear_amd.build)")
    return fn.load()


def test_header_declares_the_entry_points():
    assert HEADER in HEADERS and len(HEADERS) >= 2
    assert "fn_testing_skip_join" in _declared()
    names = _declared([HEADER])
    for want in ("fn_fold_weights", "fn_norm_linear", "fn_norm_glu_ffn", "fn_linear_qknorm",
                 "fn_linear_qknorm_rope", "fn_rope_table", "fn_fold_layernorm", "fn_layernorm_linear",
                 "fn_quantize_fp8", "fn_norm_linear_fp8", "fn_norm_glu_ffn_fp8", "fn_linear_latent_norm",
                 "fn_decode_packed_bytes", "fn_pack_decode_weights",
                 "fn_workspace_bytes", "fn_last_error", "fn_abi_version"):
        assert want in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    assert lib.fn_abi_version() == 3
    assert lib.fn_status_string(0) == b"FN_OK"
    assert lib.fn_status_string(4) == b"FN_E_ALIGN"


def test_workspace_bytes(lib):
    # fused: nothing, except the row-statistics pass of large shapes (one
    # float32 scale per row; LayerNorm also a mean)
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.FUSED, 1024, 4096, 4096, torch.bfloat16) == 0
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.FUSED, 4096, 4096, 12288, torch.bfloat16) == 4096 * 4
    assert fn.workspace_bytes(fn.OP_LAYERNORM_LINEAR, fn.FUSED, 4096, 4096, 12288, torch.bfloat16) == 2 * 4096 * 4
    assert fn.workspace_bytes(fn.OP_LAYERNORM_LINEAR, fn.FUSED, 16, 4096, 12288, torch.bfloat16) == 0
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.FUSED, 4096, 4096, 12288, torch.float32) == 0
    # unfused: the normalised activations in the input dtype, padded to 256 B
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.UNFUSED, 100, 520, 7, torch.bfloat16) == 104192
    # two-stream: float32 product plus one float32 scale per row
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.TWO_STREAM, 64, 256, 512, torch.bfloat16) == 64 * 512 * 4 + 256
    with pytest.raises(fn.FlashNormError) as e:
        fn.workspace_bytes(fn.OP_NORM_LINEAR, 9, 1, 8, 1, torch.bfloat16)
    assert e.value.status == 8


def test_workspace_bytes_memo_follows_the_statistics_switch(lib, monkeypatch):
    """The binding memoises workspace sizes; FN_PRESTATS, which decides
    whether the fused path runs a statistics pass (and needs its row
    scales), is part of the key, so a size taken with the pass off is never
    handed to a call that runs it."""
    bf = torch.bfloat16
    args = (fn.OP_NORM_LINEAR, fn.FUSED, 4096, 4096, 12288, bf)
    monkeypatch.setenv("FN_PRESTATS", "0")
    assert fn.workspace_bytes(*args) == 0
    monkeypatch.setenv("FN_PRESTATS", "1")
    assert fn.workspace_bytes(*args) == 4096 * 4
    monkeypatch.setenv("FN_PRESTATS", "0")
    assert fn.workspace_bytes(*args) == 0
    monkeypatch.delenv("FN_PRESTATS")
    assert fn.workspace_bytes(*args) == 4096 * 4
    # a memoised answer equals the library's own
    out = ctypes.c_size_t(0)
    assert lib.fn_workspace_bytes(fn.OP_NORM_LINEAR, fn.UNFUSED, 100, 520, 7, 1, ctypes.byref(out)) == 0
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.UNFUSED, 100, 520, 7, bf) == out.value
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.UNFUSED, 100, 520, 7, bf) == out.value


def test_dispatch_choices(lib):
    bf = torch.bfloat16
    assert "decode" in fn.dispatch_name(fn.OP_NORM_GLU_FFN, fn.FUSED, 16, 4096, 11008, bf, torch.float32)
    assert "decode" in fn.dispatch_name(fn.OP_NORM_GLU_FFN, fn.FUSED, 1, 4096, 11008, bf, torch.float32)
    big = fn.dispatch_name(fn.OP_NORM_LINEAR, fn.FUSED, 4096, 4096, 12288, bf, torch.float32)
    assert "row_scale+gemm_bf16<256x256w3,plain" in big
    assert "ln_stats+gemm_bf16<256x256w3,layernorm" in fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, fn.FUSED, 4096, 4096,
                                                                      12288, bf, bf)
    assert "row_scale" not in fn.dispatch_name(fn.OP_NORM_LINEAR, fn.FUSED, 2048, 576, 1536, bf, bf)
    q = fn.dispatch_name(fn.OP_LINEAR_QKNORM, fn.FUSED, 1024, 2560, 4096, bf, torch.float32)
    assert "qknorm" in q and "x256" in q
    r = fn.dispatch_name(fn.OP_LINEAR_QKNORM_ROPE, fn.FUSED, 1024, 2560, 4096, bf, bf)
    assert "qknorm_rope" in r and "x256" in r
    ln = fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, fn.UNFUSED, 4096, 4096, 12288, bf, bf)
    assert "layernorm+" in ln and "256x256w3" in ln
    assert "decode_bf16<layernorm" in fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, fn.FUSED, 1, 4096, 16384, bf, bf)
    assert "gemm_f32<16x32,layernorm>" in fn.dispatch_name(fn.OP_LAYERNORM_LINEAR, fn.FUSED, 128, 576, 960,
                                                            torch.float32, torch.float32)
    assert fn.dispatch_name(fn.OP_NORM_GLU_FFN_FP8, fn.FUSED, 1, 4096, 11008, bf, bf) == "fused:decode_fp8<glu,bf16>"
    assert fn.dispatch_name(fn.OP_NORM_LINEAR_FP8, fn.UNFUSED, 4, 4096, 300, bf, torch.float32) == \
        "unfused:rmsnorm+decode_fp8<plain,f32>"
    lat = fn.dispatch_name(fn.OP_LINEAR_LATENT_NORM, fn.FUSED, 4096, 7168, 2112, bf, bf)
    assert "latent" in lat and lat.endswith("+latent_norm")
    # the latent op always needs its workspace (float32 latent product and sums)
    assert fn.workspace_bytes(fn.OP_LINEAR_LATENT_NORM, fn.FUSED, 64, 128, 576, bf) == 64 * 576 * 4 + 64 * 18 * 4
    assert fn.workspace_bytes(fn.OP_LINEAR_LATENT_NORM, fn.UNFUSED, 64, 128, 576, bf) == \
        64 * 576 * 4 + 64 * 18 * 4 + 64 * 128 * 2
    # decode batch sizes of the head-norm ops: the weight-streaming kernel's
    # float32 product in the workspace, then the head norms per (row, head)
    assert fn.dispatch_name(fn.OP_LINEAR_QKNORM_ROPE, fn.FUSED, 4, 2560, 4096, bf, bf) == \
        "fused:decode_bf16<plain,f32>+qk_finish<qknorm_rope,bf16>"
    assert fn.workspace_bytes(fn.OP_LINEAR_QKNORM, fn.FUSED, 4, 2560, 4096, bf) == 4 * 4096 * 4
    assert fn.workspace_bytes(fn.OP_LINEAR_QKNORM, fn.UNFUSED, 16, 2560, 4096, bf) == 16 * 2560 * 2 + 16 * 4096 * 4
    # above the decode rows the head-norm tile takes over
    assert "gemm_bf16" in fn.dispatch_name(fn.OP_LINEAR_QKNORM_ROPE, fn.FUSED, 17, 2560, 4096, bf, bf)
    assert fn.workspace_bytes(fn.OP_LINEAR_QKNORM, fn.FUSED, 17, 2560, 4096, bf) == 0
    assert "rmsnorm+" in fn.dispatch_name(fn.OP_NORM_LINEAR, fn.UNFUSED, 4096, 4096, 12288, bf, bf)
    assert "gemm_f32" in fn.dispatch_name(fn.OP_NORM_LINEAR, fn.FUSED, 128, 576, 960, torch.float32, torch.float32)


def test_validation_runs_before_any_device_work(lib):
    """Invalid calls return their status without touching the (absent) GPU."""
    bad_ptr = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    st = None
    assert lib.fn_norm_linear(None, 1, 4, 8, bad_ptr, 1, 4, None, 1e-6, bad_ptr, 0, 0, None, 0, st, None) == 1
    assert lib.fn_norm_linear(bad_ptr, 1, 4, 8, bad_ptr, 1, 4, None, -1.0, bad_ptr, 0, 0, None, 0, st, None) == 8
    assert b"eps" in lib.fn_last_error()
    # bf16 K beyond the prefill kernel's 32-bit tile offsets
    assert lib.fn_norm_linear(bad_ptr, 1, 4, (1 << 21) + 8, bad_ptr, 1, 4, None, 1e-6, bad_ptr, 0, 0, None, 0, st,
                              None) == 6
    assert lib.fn_norm_linear(ctypes.c_void_p(0x1002), 1, 4, 8, bad_ptr, 1, 4, None, 1e-6, bad_ptr, 0, 0, None, 0,
                              st, None) == 4
    assert lib.fn_norm_linear(bad_ptr, 0, 4, 8, bad_ptr, 0, 4, None, 1e-6, bad_ptr, 1, 0, None, 0, st, None) == 3
    assert lib.fn_fold_weights(bad_ptr, 1, bad_ptr, 4, 12, bad_ptr, 1, st) == 4
    assert lib.fn_fold_weights(bad_ptr, 1, bad_ptr, 4, 16, ctypes.c_void_p(0x1010), 1, st) == 8  # partial overlap
    assert lib.fn_linear_qknorm(bad_ptr, 1, 4, 8, bad_ptr, 1, 1, 1, 96, bad_ptr, bad_ptr, 0, 1e-6, 1e-6, 0, None,
                                bad_ptr, 0, 0, None, 0, st) == 2
    # rotary arguments: missing table, misaligned positions, rot_dim not a
    # multiple of 4 or above head_dim, empty table
    q = lambda pos, tab, n_pos, rot: lib.fn_linear_qknorm_rope(  # noqa: E731
        bad_ptr, 1, 4, 8, bad_ptr, 1, 1, 1, 64, bad_ptr, bad_ptr, 0, 1e-6, 1e-6, 0, pos, tab, n_pos, rot, None,
        bad_ptr, 0, 0, None, 0, st)
    assert q(bad_ptr, None, 16, 64) == 1
    assert q(ctypes.c_void_p(0x1004), bad_ptr, 16, 64) == 4
    assert q(bad_ptr, bad_ptr, 16, 62) == 2
    assert q(bad_ptr, bad_ptr, 16, 128) == 2
    assert q(bad_ptr, bad_ptr, 0, 64) == 2
    assert lib.fn_rope_table(10000.0, 63, 16, bad_ptr, st) == 2
    assert lib.fn_rope_table(1.0, 64, 16, bad_ptr, st) == 8
    assert lib.fn_rope_table(10000.0, 64, 0, bad_ptr, st) == 0
    # LayerNorm: fused needs colsum and takes no unfolded parameters; unfused
    # needs g and takes no folded vectors; folds need their outputs
    ln = lambda cs, bs, g, beta, bias, v: lib.fn_layernorm_linear(  # noqa: E731
        bad_ptr, 1, 4, 8, bad_ptr, 1, 4, cs, bs, g, beta, bias, 1e-5, bad_ptr, 1, v, None, 0, st)
    assert ln(None, None, None, None, None, 0) == 1
    assert ln(bad_ptr, None, bad_ptr, None, None, 0) == 8
    assert ln(None, None, None, None, None, 1) == 1
    assert ln(None, bad_ptr, bad_ptr, None, None, 1) == 8
    assert ln(ctypes.c_void_p(0x1008), None, None, None, None, 0) == 4
    assert ln(bad_ptr, None, None, None, None, 2) == 6
    assert lib.fn_fold_layernorm(bad_ptr, 1, bad_ptr, None, None, 4, 16, bad_ptr, 1, None, bad_ptr, st) == 1
    assert lib.fn_fold_layernorm(bad_ptr, 1, bad_ptr, None, None, 4, 12, bad_ptr, 1, ctypes.c_void_p(0x9000),
                                 ctypes.c_void_p(0xa000), st) == 4
    assert lib.fn_fold_layernorm(bad_ptr, 1, bad_ptr, None, None, 4, 16, ctypes.c_void_p(0x2000), 1,
                                 ctypes.c_void_p(0x9000), ctypes.c_void_p(0x9008), st) == 8  # colsum/b_star overlap
    assert lib.fn_fold_layernorm(None, 1, None, None, None, 0, 16, None, 1, None, None, st) == 0
    # fp8: M above the decode rows without the workspace the row
    # quantisation needs, or with packed weights; K not a multiple of 16, g
    # with fused, missing scales, overlapping quantiser outputs
    f8 = lambda M, K, q, g, v: lib.fn_norm_linear_fp8(  # noqa: E731
        bad_ptr, 1, M, K, bad_ptr, q, 4, g, 1e-6, bad_ptr, 1, v, None, 0, st)
    assert f8(17, 64, bad_ptr, None, 0) == 5
    assert f8(17, 64, bad_ptr, None, 3) == 6
    assert f8(4, 40, bad_ptr, None, 0) == 4
    assert f8(4, 64, bad_ptr, bad_ptr, 0) == 8
    assert f8(4, 64, None, None, 0) == 1
    assert f8(4, 64, bad_ptr, None, 1) == 1
    assert lib.fn_quantize_fp8(bad_ptr, 1, 4, 40, ctypes.c_void_p(0x9000), ctypes.c_void_p(0xa000), st) == 4
    assert lib.fn_quantize_fp8(bad_ptr, 1, 4, 64, ctypes.c_void_p(0x1010), ctypes.c_void_p(0xa000), st) == 8
    # latent: widths not multiples of 32 / 4, no latent, missing gain
    la = lambda nq, nkv, nr, gq, gkv: lib.fn_linear_latent_norm(  # noqa: E731
        bad_ptr, 1, 4, 64, bad_ptr, 1, nq, nkv, nr, gq, gkv, 1e-6, 1e-6, None, None, 0, 0, None, bad_ptr, 1, 0,
        bad_ptr, 1 << 20, st)
    assert la(48, 0, 0, bad_ptr, None) == 2
    assert la(32, 32, 6, bad_ptr, bad_ptr) == 2
    assert la(0, 0, 64, None, None) == 2
    assert la(32, 32, 0, bad_ptr, None) == 1
    # zero-size fold is a valid no-op
    assert lib.fn_fold_weights(None, 1, None, 0, 16, None, 1, st) == 0


def test_empty_batch_takes_null_row_pointers(lib):
    """M = 0 reads and writes no row, so x, y (h) and positions may be NULL,
    as an empty tensor's are; with M > 0 the same calls fail FN_E_NULL."""
    w = ctypes.c_void_p(0x1000)  # never dereferenced
    st = None
    for M, want in ((0, 0), (3, 1)):
        assert lib.fn_norm_linear(None, 1, M, 64, w, 1, 32, None, 1e-6, None, 0, 0, None, 0, st, None) == want
        assert lib.fn_norm_glu_ffn(None, 1, M, 64, w, w, 1, 32, None, 1e-6, None, 0, 0, None, 0, st) == want
        assert lib.fn_linear_qknorm(None, 1, M, 64, w, 1, 1, 1, 64, w, w, 0, 1e-6, 1e-6, 0, None, None, 0, 0,
                                    None, 0, st) == want
        assert lib.fn_linear_qknorm_rope(None, 1, M, 64, w, 1, 1, 1, 64, w, w, 0, 1e-6, 1e-6, 0, None, w, 16, 64,
                                         None, None, 0, 0, None, 0, st) == want
        assert lib.fn_layernorm_linear(None, 1, M, 64, w, 1, 32, w, None, None, None, None, 1e-5, None, 0, 0,
                                       None, 0, st) == want
        assert lib.fn_norm_linear_fp8(None, 1, M, 64, w, w, 32, None, 1e-6, None, 0, 0, None, 0, st) == want
        assert lib.fn_norm_glu_ffn_fp8(None, 1, M, 64, w, w, w, w, 32, None, 1e-6, None, 0, 0, None, 0, st) == want
        assert lib.fn_linear_latent_norm(None, 1, M, 64, w, 1, 32, 32, 0, w, w, 1e-6, 1e-6, None, None, 0, 0,
                                         None, None, 0, 0, w, 1 << 20, st) == want
    # weights stay required even for an empty batch
    assert lib.fn_norm_linear(None, 1, 0, 64, None, 1, 32, None, 1e-6, None, 0, 0, None, 0, st, None) == 1


def test_decode_packed_layout_queries(lib):
    """Sizes of the decode-packed layout, its validation, and which ops take
    FUSED_PACKED (the weight-streaming ones, M <= 16, bf16 x)."""
    bf, u8 = torch.bfloat16, torch.uint8
    # ceil(N / 16) slabs x ceil(K * bytes / 64) steps x 1 KB
    assert fn.decode_packed_bytes(11008, 4096, bf) == 688 * 128 * 1024
    assert fn.decode_packed_bytes(11008, 4096, u8) == 688 * 64 * 1024
    assert fn.decode_packed_bytes(77, 520, bf) == 5 * 17 * 1024
    assert fn.decode_packed_bytes(1, 16, u8) == 1024
    assert fn.decode_packed_bytes(0, 64, bf) == 0
    out = ctypes.c_size_t(0)
    assert lib.fn_decode_packed_bytes(0, 16, 64, ctypes.byref(out)) == 3   # float32 weights are not packed
    assert lib.fn_decode_packed_bytes(1, 16, 12, ctypes.byref(out)) == 4   # bf16 K % 8
    assert lib.fn_decode_packed_bytes(2, 16, 24, ctypes.byref(out)) == 4   # fp8 K % 16
    assert lib.fn_decode_packed_bytes(1, -1, 64, ctypes.byref(out)) == 2
    bad = ctypes.c_void_p(0x1000)
    assert lib.fn_pack_decode_weights(None, 1, 16, 64, bad, None) == 1
    assert lib.fn_pack_decode_weights(bad, 1, 16, 64, ctypes.c_void_p(0x1008), None) == 4
    assert lib.fn_pack_decode_weights(bad, 1, 16, 64, ctypes.c_void_p(0x1400), None) == 8  # overlaps W
    assert lib.fn_pack_decode_weights(None, 1, 0, 64, None, None) == 0
    # the packed variant: decode ops only, M <= 16, bf16 x; no workspace
    for op in (fn.OP_NORM_LINEAR, fn.OP_NORM_GLU_FFN, fn.OP_LAYERNORM_LINEAR, fn.OP_NORM_LINEAR_FP8,
               fn.OP_NORM_GLU_FFN_FP8):
        assert fn.workspace_bytes(op, fn.FUSED_PACKED, 16, 4096, 11008, bf) == 0
        assert fn.dispatch_name(op, fn.FUSED_PACKED, 4, 4096, 11008, bf, bf).startswith("fused_packed:decode_")
    for op in (fn.OP_LINEAR_QKNORM, fn.OP_LINEAR_QKNORM_ROPE, fn.OP_LINEAR_LATENT_NORM):
        with pytest.raises(fn.FlashNormError, match="UNSUPPORTED"):
            fn.dispatch_name(op, fn.FUSED_PACKED, 4, 4096, 4096, bf, bf)
    with pytest.raises(fn.FlashNormError, match="UNSUPPORTED"):
        fn.dispatch_name(fn.OP_NORM_LINEAR, fn.FUSED_PACKED, 17, 4096, 4096, bf, bf)
    w = ctypes.c_void_p(0x1000)
    assert lib.fn_norm_linear(w, 1, 17, 64, w, 1, 32, None, 1e-6, w, 1, 3, None, 0, None, None) == 6
    assert lib.fn_norm_linear(w, 0, 4, 64, w, 0, 32, None, 1e-6, w, 0, 3, None, 0, None, None) == 6
    assert lib.fn_norm_glu_ffn(w, 1, 17, 64, w, w, 1, 32, None, 1e-6, w, 1, 3, None, 0, None) == 6
    assert lib.fn_norm_linear_fp8(w, 1, 17, 64, w, w, 32, None, 1e-6, w, 1, 3, None, 0, None) == 6
    assert lib.fn_linear_qknorm(w, 1, 4, 64, w, 1, 1, 1, 64, w, w, 0, 1e-6, 1e-6, 0, None, w, 1, 3, None, 0,
                                None) == 6
    assert lib.fn_norm_linear(w, 1, 4, 64, w, 1, 32, None, 1e-6, w, 1, 4, None, 0, None, None) == 8
    # an empty batch with packed weights is a valid no-op
    assert lib.fn_norm_glu_ffn(None, 1, 0, 64, w, w, 1, 32, None, 1e-6, None, 1, 3, None, 0, None) == 0
    # the gate/up pair layout: the up weight may be NULL only with FUSED_PACKED
    assert lib.fn_pack_decode_weights_glu(bad, None, 1, 16, 64, ctypes.c_void_p(0x900000), None) == 1
    assert lib.fn_pack_decode_weights_glu(bad, ctypes.c_void_p(0x800000), 1, 16, 64, ctypes.c_void_p(0x800400),
                                          None) == 8  # overlaps W_up
    assert lib.fn_pack_decode_weights_glu(None, None, 2, 0, 64, None, None) == 0
    assert lib.fn_norm_glu_ffn(w, 1, 4, 64, w, None, 1, 32, None, 1e-6, w, 1, 0, None, 0, None) == 1
    assert lib.fn_norm_glu_ffn_fp8(w, 1, 4, 64, w, w, None, w, 32, None, 1e-6, w, 1, 0, None, 0, None) == 1
    assert lib.fn_norm_glu_ffn(None, 1, 0, 64, w, None, 1, 32, None, 1e-6, None, 1, 3, None, 0, None) == 0


def test_pair_buffer_rejected_by_single_weight_ops(lib):
    """A gate/up pair buffer is only the gate weight of a GLU op: the
    single-weight wrappers refuse it before touching any device memory."""
    P = fn.PackedWeight(torch.empty(2048, dtype=torch.uint8), 16, 64, torch.bfloat16, pair=True)
    x = torch.empty(4, 64, dtype=torch.bfloat16)
    for call in (lambda: fn.norm_linear(x, P, 1e-6), lambda: fn.layernorm_linear(x, P, 1e-5),
                 lambda: fn.norm_linear_fp8(x, P, torch.ones(16), 1e-6)):
        with pytest.raises(ValueError, match="pair"):
            call()
    with pytest.raises(ValueError, match="None"):
        fn.norm_glu_ffn(x, P, P, 1e-6)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library the binding raises; there is no fallback."""
    monkeypatch.setattr(fn, "LIB_PATH", str(tmp_path / "libflashnorm.so"))
    monkeypatch.setattr(fn, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        fn.load()
    with pytest.raises(RuntimeError):
        fn.workspace_bytes(fn.OP_NORM_LINEAR, fn.FUSED, 1, 8, 8, torch.bfloat16)


def test_product_path_does_not_import_the_oracle():
    """The package (binding and build script) never imports the oracle."""
    pkg = os.path.join(ROOT, "rmsnorm_linear_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            with open(os.path.join(pkg, name)) as f:
                text = f.read()
            assert "import oracle" not in text and "from oracle" not in text, name


def test_fp8_prefill_workspace_and_dispatch(lib):
    """Above 16 rows the fp8 ops quantise x into the workspace: the codes
    (padded to 256 bytes), then one float32 factor per row (and, unfused,
    the normalised bf16 x before them)."""
    bf = torch.bfloat16
    M, K, N = 300, 1040, 700
    codes, fac = (M * K + 255) // 256 * 256, (M * 4 + 255) // 256 * 256
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR_FP8, fn.FUSED, M, K, N, bf) == codes + fac
    assert fn.workspace_bytes(fn.OP_NORM_GLU_FFN_FP8, fn.UNFUSED, M, K, N, bf) == \
        (M * K * 2 + 255) // 256 * 256 + codes + fac
    assert fn.workspace_bytes(fn.OP_NORM_LINEAR_FP8, fn.FUSED, 16, K, N, bf) == 0
    d = fn.dispatch_name(fn.OP_NORM_LINEAR_FP8, fn.FUSED, 4096, 4096, 12288, bf, bf)
    assert d.startswith("fused:quant_rows+gemm_fp8<") and d.endswith(",plain,bf16>"), d
    assert fn.dispatch_name(fn.OP_NORM_GLU_FFN_FP8, fn.UNFUSED, 2048, 576, 1536, bf, torch.float32).startswith(
        "unfused:rmsnorm+quant_rows+gemm_fp8<")


def test_noalloc_refuses_before_any_device_work(lib):
    """The allocation-free entry point validates like fn_norm_linear and
    refuses a shape whose row statistics exceed its static scratch, before
    any HIP call (so this runs without a GPU)."""
    bad = ctypes.c_void_p(0x1000)  # never dereferenced
    import os
    old = os.environ.get("FN_PRESTATS")
    os.environ["FN_PRESTATS"] = "1"
    try:
        assert lib.fn_norm_linear_noalloc(bad, 1, (1 << 20) + 64, 64, bad, 1, 256, 1e-6, bad, 0, None) == 5
        assert b"scratch" in lib.fn_last_error()
        assert lib.fn_norm_linear_noalloc(bad, 1, 64, 64, bad, 0, 256, 1e-6, bad, 0, None) == 3
        assert lib.fn_norm_linear_noalloc(bad, 1, -1, 64, bad, 1, 256, 1e-6, bad, 0, None) == 2
    finally:
        if old is None:
            del os.environ["FN_PRESTATS"]
        else:
            os.environ["FN_PRESTATS"] = old


def test_gemm_timing_hook_checks_its_arrays(lib):
    """The measurement hook only stores its arguments: NULL arrays with
    n > 0 are refused (and leave it off), n <= 0 turns it off; no HIP call."""
    assert lib.fn_testing_gemm_events(None, None, 4) == 1
    assert b"NULL" in lib.fn_last_error()
    assert lib.fn_testing_gemm_events(None, None, 0) == 0
    assert lib.fn_testing_gemm_events(None, None, -3) == 0
