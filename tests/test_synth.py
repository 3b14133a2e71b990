"""The seeded input generator: published SplitMix64 outputs, counter-based
sub-ranges, distribution moments, storage rounding."""

import numpy as np
import torch

import synth
from synth.gen import T_X, _GOLDEN


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0: state += 0x9E3779B97F4A7C15, then the output mix.
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    idx = np.arange(1, 5, dtype=np.uint64)
    with np.errstate(over="ignore"):
        got = synth.splitmix64_mix(idx * _GOLDEN)
    assert [int(v) for v in got] == want


def test_counter_based_subranges():
    full = synth.normal(123, T_X, 1001)
    for a, b in [(0, 1), (1, 2), (3, 700), (999, 1001), (500, 1001)]:
        part = synth.normal(123, T_X, b - a, a)
        assert np.array_equal(part, full[a:b])
    assert not np.array_equal(synth.normal(124, T_X, 100), full[:100])
    assert not np.array_equal(synth.normal(123, T_X + 1, 100), full[:100])


def test_normal_moments():
    v = synth.normal(7, 0, 1 << 20)
    assert abs(v.mean()) < 5e-3 and abs(v.std() - 1) < 5e-3
    u = synth.uniform01(7, 1, 1 << 20)
    assert u.min() > 0 and u.max() <= 1 and abs(u.mean() - 0.5) < 2e-3


def test_bf16_storage_matches_torch_cast():
    f = (synth.normal(9, 0, 1 << 16) * 3).astype(np.float32)
    bits = synth.bf16_bits_from_f32(f)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, want)
    back = synth.bf16_bits_to_f64(bits)
    assert np.array_equal(back, torch.from_numpy(f).to(torch.bfloat16).double().numpy())


def test_workload_rows_regenerate_and_distributions():
    w = synth.workload("smollm2_ffn_prefill_bf16")
    x = w.x()
    assert x.shape == (2048, 576) and x.dtype == np.uint16
    assert np.array_equal(w.x_rows(100, 164), x[100:164])
    W = synth.stored_to_f64(w.w())
    assert W.shape == (1536, 576)
    assert abs(W.std() * np.sqrt(576) - 1) < 0.01
    g = w.g()
    assert g.dtype == np.float32 and abs(g.mean() - 1) < 0.02 and abs(g.std() - 0.1) < 0.01
    rs = np.sqrt(np.mean(synth.stored_to_f64(x) ** 2, axis=1))
    # rows scaled by lognormal(0, 0.5): log RMS has std about 0.5
    assert abs(np.std(np.log(rs)) - 0.5) < 0.05
    q = synth.workload("qknorm_attn_in_bf16")
    assert q.N == 4096 and q.n_q_heads == 8 and q.n_kv_heads == 4 and q.head_dim == 256
    f0 = synth.workload("smollm2_qkv_f32")
    assert f0.x().dtype == np.float32 and f0.w().shape == (960, 576)
