"""Counter-based SplitMix64 + Box-Muller generator and the workload recipes.

Generator
---------
SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014; constants as published there and in Vigna's
reference code) is used as a *counter-based* mixer: word ``i`` of stream
``(seed, tensor_id)`` is ``mix(key + (i + 1) * GOLDEN)`` with
``key = mix(seed XOR (tensor_id + 1) * 0xD1B54A32D192ED03)``.  Any sub-range of
a stream can therefore be regenerated on its own, which the full-size parity
tests use to sample rows.

Uniforms in (0, 1] take the top 53 bits: ``((w >> 11) + 1) * 2**-53``.
Normals use the Box-Muller transform on consecutive word pairs
``(u1, u2) = (word 2j, word 2j+1)``: ``sqrt(-2 ln u1) * cos(2 pi u2)`` is draw
``2j`` and ``sqrt(-2 ln u1) * sin(2 pi u2)`` is draw ``2j + 1``.  Draws are
formed in float64.

Storage
-------
A value is drawn in float64, rounded once to float32 (IEEE round to nearest
even), and for bf16 tensors rounded once more from that float32 to bf16
(round to nearest even on the bit pattern).  bf16 tensors are kept as their
uint16 bit patterns; ``stored_to_f64`` upcasts either kind exactly.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_KEYMUL = 0xD1B54A32D192ED03
_MASK64 = (1 << 64) - 1
_CHUNK = 1 << 22


def splitmix64_mix(z: np.ndarray) -> np.ndarray:
    """The SplitMix64 output function applied elementwise to uint64 words."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _stream_key(seed: int, tensor_id: int) -> np.uint64:
    mixed = (int(seed) ^ (((tensor_id + 1) * _KEYMUL) & _MASK64)) & _MASK64
    return splitmix64_mix(np.array([mixed], dtype=np.uint64))[0]


def _words(seed: int, tensor_id: int, start: int, count: int) -> np.ndarray:
    key = _stream_key(seed, tensor_id)
    idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return splitmix64_mix(key + idx * _GOLDEN)


def uniform01(seed: int, tensor_id: int, count: int, start: int = 0) -> np.ndarray:
    """``count`` uniforms in (0, 1] (float64) from word ``start`` on."""
    w = _words(seed, tensor_id, start, count)
    return ((w >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal(seed: int, tensor_id: int, count: int, start: int = 0) -> np.ndarray:
    """``count`` standard normal draws (float64) from draw ``start`` on."""
    out = np.empty(count, dtype=np.float64)
    done = 0
    while done < count:
        n = min(_CHUNK, count - done)
        first = start + done
        pair0 = first // 2
        npairs = (first + n + 1) // 2 - pair0
        u = uniform01(seed, tensor_id, 2 * npairs, 2 * pair0)
        u1, u2 = u[0::2], u[1::2]
        rad = np.sqrt(-2.0 * np.log(u1))
        ang = 2.0 * math.pi * u2
        both = np.empty(2 * npairs, dtype=np.float64)
        both[0::2] = rad * np.cos(ang)
        both[1::2] = rad * np.sin(ang)
        off = first - 2 * pair0
        out[done:done + n] = both[off:off + n]
        done += n
    return out


def bf16_bits_from_f32(f: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits."""
    b = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def stored_to_f64(arr: np.ndarray) -> np.ndarray:
    """Exact float64 view of a stored tensor (float32 or bf16 bits)."""
    if arr.dtype == np.uint16:
        return bf16_bits_to_f64(arr)
    return np.asarray(arr, dtype=np.float64)


def _store(v64: np.ndarray, dtype: str) -> np.ndarray:
    f = v64.astype(np.float32)
    if dtype == F32:
        return f
    if dtype == BF16:
        return bf16_bits_from_f32(f)
    raise ValueError(dtype)


# Tensor ids: one independent stream per tensor of a workload.
T_X, T_ROWSCALE, T_G, T_W, T_WUP, T_GQ, T_GK, T_G1, T_POS, T_MEAN, T_BETA, T_BIAS, T_GQL, T_GKVL = range(14)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload.

    ``kind`` is ``"linear"`` (RMSNorm then one projection), ``"glu"``
    (RMSNorm then gate and up projections with a SiLU gated unit) or
    ``"qknorm"`` (RMSNorm, QKV projection, per-head RMSNorm on q and k) or
    ``"qknorm_rope"`` (the same, then the rotary embedding of q and k at
    each row's token position), ``"layernorm"`` (LayerNorm with gain and
    bias, then one projection with bias) or ``"latent"`` (MLA attention
    input: RMSNorm, one projection to [q latent | kv latent | rope part],
    an RMSNorm on each latent, the rotary embedding on the rope part).
    Weights are stored ``[N x K]`` (output features by input features,
    input features contiguous), the layout of a linear layer's checkpoint.
    """

    name: str
    kind: str
    M: int
    K: int
    N: int  # output columns per projection (qknorm: (nq + 2 nkv) * head_dim)
    dtype: str  # storage dtype of x and the weights
    eps: float
    seed: int
    row_sigma: float  # rows of x are scaled by exp(row_sigma * N(0, 1))
    n_q_heads: int = 0
    n_kv_heads: int = 0
    head_dim: int = 0
    eps_head: float = 0.0
    rope_base: float = 0.0  # qknorm_rope: theta_i = rope_base^(-2i / rot_dim)
    rot_dim: int = 0        # qknorm_rope: rotated columns per head
    n_pos: int = 0          # qknorm_rope: positions lie in [0, n_pos)
    mean_sigma: float = 0.0  # rows of x get an offset mean_sigma * N(0, 1) before the row scale
    fp8: bool = False  # weights stored as per-channel E4M3 (1 byte + a float32 scale per row)
    n_q_latent: int = 0   # latent: widths of the q latent, kv latent and rope part (N is their sum)
    n_kv_latent: int = 0
    n_rope: int = 0

    def flops(self) -> int:
        """Algorithmic flops: 2 M K N over every projection."""
        nproj = 2 if self.kind == "glu" else 1
        return 2 * self.M * self.K * self.N * nproj

    def out_cols(self) -> int:
        return self.N

    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def algo_bytes(self, out_bytes: int) -> int:
        """Algorithmic HBM bytes: x and W* read once, y written once (and,
        with the rotary embedding, the positions and one table row per row;
        with LayerNorm, the two float32 vectors over N)."""
        nproj = 2 if self.kind == "glu" else 1
        e = self.elem_bytes()
        we = 1 if self.fp8 else e
        b = self.M * self.K * e + nproj * self.N * self.K * we + self.M * self.N * out_bytes
        if self.fp8:
            b += nproj * self.N * 4  # channel scales
        if self.kind == "qknorm_rope" or (self.kind == "latent" and self.rot_dim):
            b += self.M * 4 + self.M * self.rot_dim * 4
        if self.kind == "layernorm":
            b += 2 * self.N * 4  # column sums and folded bias
        return b

    def with_rows(self, M: int, seed: Optional[int] = None) -> "Workload":
        return dataclasses.replace(self, M=M, seed=self.seed if seed is None else seed)

    def with_shape(self, M: int, K: int, N: int) -> "Workload":
        return dataclasses.replace(self, M=M, K=K, N=N)

    # ---- draws ---------------------------------------------------------
    def x_rows(self, r0: int, r1: int) -> np.ndarray:
        """Rows [r0, r1) of x, stored in the workload dtype."""
        K = self.K
        base = normal(self.seed, T_X, (r1 - r0) * K, r0 * K).reshape(r1 - r0, K)
        if self.mean_sigma:
            base = base + self.mean_sigma * normal(self.seed, T_MEAN, r1 - r0, r0)[:, None]
        scale = np.exp(self.row_sigma * normal(self.seed, T_ROWSCALE, r1 - r0, r0))
        return _store(base * scale[:, None], self.dtype)

    def x(self) -> np.ndarray:
        return self.x_rows(0, self.M)

    def _weight(self, tid: int, rows: int, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
        r1 = rows if r1 is None else r1
        K = self.K
        v = normal(self.seed, tid, (r1 - r0) * K, r0 * K).reshape(r1 - r0, K)
        return _store(v / math.sqrt(K), self.dtype)

    def w(self, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
        """Projection weight (gate weight for ``glu``), ``[N x K]``."""
        return self._weight(T_W, self.N, r0, r1)

    def w_up(self, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
        return self._weight(T_WUP, self.N, r0, r1)

    def _gain(self, tid: int, n: int) -> np.ndarray:
        return (1.0 + 0.1 * normal(self.seed, tid, n)).astype(np.float32)

    def g(self) -> np.ndarray:
        """RMSNorm gain over the K input features (float32)."""
        return self._gain(T_G, self.K)

    def beta(self) -> np.ndarray:
        """LayerNorm bias over the K input features (float32): 0.1 N(0, 1)."""
        return (0.1 * normal(self.seed, T_BETA, self.K)).astype(np.float32)

    def bias(self) -> np.ndarray:
        """The linear layer's bias over the N outputs (float32): 0.1 N(0, 1)."""
        return (0.1 * normal(self.seed, T_BIAS, self.N)).astype(np.float32)

    def g_q_latent(self) -> np.ndarray:
        return self._gain(T_GQL, self.n_q_latent)

    def g_kv_latent(self) -> np.ndarray:
        return self._gain(T_GKVL, self.n_kv_latent)

    def g_q(self) -> np.ndarray:
        return self._gain(T_GQ, self.head_dim)

    def g_k(self) -> np.ndarray:
        return self._gain(T_GK, self.head_dim)

    def positions(self) -> np.ndarray:
        """Token positions [M] (int32) of a packed prefill batch: consecutive
        runs (sequences) of 64..512 tokens, lengths uniform, each run
        continuing a context whose length is uniform in [0, n_pos - length],
        so the batch touches positions across the whole table."""
        u = uniform01(self.seed, T_POS, 2 * self.M + 2)
        out = np.empty(self.M, dtype=np.int32)
        m = k = 0
        while m < self.M:
            length = min(64 + int(u[k] * 449), self.n_pos)
            start = int(u[k + 1] * (self.n_pos - length + 1))
            k += 2
            length = min(length, self.M - m)
            out[m:m + length] = start + np.arange(length)
            m += length
        return out

    def eps_f32(self) -> float:
        return float(np.float32(self.eps))

    def eps_head_f32(self) -> float:
        return float(np.float32(self.eps_head))


def _seed(i: int) -> int:
    return 0x5EED0000 + i


WORKLOADS: Dict[str, Workload] = {
    # SmolLM2-135M-shaped QKV norm+projection, float32 end to end.
    "smollm2_qkv_f32": Workload("smollm2_qkv_f32", "linear", 128, 576, 960, F32, 1e-5, _seed(0), 0.5),
    # SmolLM2-135M-shaped FFN gate+up, prefill, bf16 storage.
    "smollm2_ffn_prefill_bf16": Workload("smollm2_ffn_prefill_bf16", "glu", 2048, 576, 1536, BF16, 1e-5, _seed(1), 0.5),
    # Llama-7B-shaped QKV projection, prefill, bf16.
    "llama7b_qkv_prefill_bf16": Workload("llama7b_qkv_prefill_bf16", "linear", 4096, 4096, 12288, BF16, 1e-6, _seed(2), 0.5),
    # Llama-7B-shaped FFN gate+up in decode, batch 1 / 4 / 16 rows.
    "llama7b_ffn_decode_m1_bf16": Workload("llama7b_ffn_decode_m1_bf16", "glu", 1, 4096, 11008, BF16, 1e-6, 0x5EED0030, 0.5),
    "llama7b_ffn_decode_m4_bf16": Workload("llama7b_ffn_decode_m4_bf16", "glu", 4, 4096, 11008, BF16, 1e-6, 0x5EED0031, 0.5),
    "llama7b_ffn_decode_m16_bf16": Workload("llama7b_ffn_decode_m16_bf16", "glu", 16, 4096, 11008, BF16, 1e-6, 0x5EED0032, 0.5),
    # The same decode FFN with the folded gate and up weights in fp8 (E4M3,
    # one float32 scale per output channel); x and outputs stay bf16.
    "llama7b_ffn_decode_m1_fp8": Workload("llama7b_ffn_decode_m1_fp8", "glu", 1, 4096, 11008, BF16, 1e-6, 0x5EED0030, 0.5,
                                          fp8=True),
    "llama7b_ffn_decode_m4_fp8": Workload("llama7b_ffn_decode_m4_fp8", "glu", 4, 4096, 11008, BF16, 1e-6, 0x5EED0031, 0.5,
                                          fp8=True),
    "llama7b_ffn_decode_m16_fp8": Workload("llama7b_ffn_decode_m16_fp8", "glu", 16, 4096, 11008, BF16, 1e-6, 0x5EED0032,
                                           0.5, fp8=True),
    # The Llama-7B QKV prefill with the folded weight in fp8 (E4M3 per output
    # channel); the op quantises x per row to E4M3 as well, for the fp8
    # matrix cores.  Same draws as the bf16 workload.
    "llama7b_qkv_prefill_fp8": Workload("llama7b_qkv_prefill_fp8", "linear", 4096, 4096, 12288, BF16, 1e-6, _seed(2),
                                        0.5, fp8=True),
    # The SmolLM2 FFN prefill with fp8 gate and up weights (and fp8 x in the op).
    "smollm2_ffn_prefill_fp8": Workload("smollm2_ffn_prefill_fp8", "glu", 2048, 576, 1536, BF16, 1e-5, _seed(1), 0.5,
                                        fp8=True),
    # QK-norm attention input: 8 q heads, 4 k heads, 4 v heads of 256.
    "qknorm_attn_in_bf16": Workload("qknorm_attn_in_bf16", "qknorm", 1024, 2560, 16 * 256, BF16, 1e-6, _seed(4), 1.0,
                                    n_q_heads=8, n_kv_heads=4, head_dim=256, eps_head=1e-6),
    # The same attention input with the rotary embedding of q and k after the
    # head norms: base 10^4, every column of a head rotated, 32768 positions.
    "qknorm_rope_attn_in_bf16": Workload("qknorm_rope_attn_in_bf16", "qknorm_rope", 1024, 2560, 16 * 256, BF16, 1e-6,
                                         0x5EED0050, 1.0, n_q_heads=8, n_kv_heads=4, head_dim=256, eps_head=1e-6,
                                         rope_base=10000.0, rot_dim=256, n_pos=32768),
    # MLA attention input at DeepSeek-V2 width: hidden 5120 -> q latent 1536,
    # kv latent 512, rope part 64; a 2048-token prefill chunk; rows scaled
    # by lognormal(0, 1); rotary embedding on the rope part (base 10^4).
    "mla_latent_attn_in_bf16": Workload("mla_latent_attn_in_bf16", "latent", 2048, 5120, 2112, BF16, 1e-6, 0x5EED0070,
                                        1.0, eps_head=1e-6, rope_base=10000.0, rot_dim=64, n_pos=32768,
                                        n_q_latent=1536, n_kv_latent=512, n_rope=64),
    # LayerNorm then a biased projection: a 4096-wide QKV prefill (the width
    # of the LayerNorm models at 6-7B scale) and a 4096 -> 16384 first FFN
    # layer in decode.  Rows are N(offset, 1) with offset ~ N(0, 1), then
    # scaled by lognormal(0, 0.5).
    "ln_qkv_prefill_bf16": Workload("ln_qkv_prefill_bf16", "layernorm", 4096, 4096, 12288, BF16, 1e-5, 0x5EED0060,
                                    0.5, mean_sigma=1.0),
    "ln_fc1_decode_m1_bf16": Workload("ln_fc1_decode_m1_bf16", "layernorm", 1, 4096, 16384, BF16, 1e-5, 0x5EED0061,
                                      0.5, mean_sigma=1.0),
    "ln_fc1_decode_m16_bf16": Workload("ln_fc1_decode_m16_bf16", "layernorm", 16, 4096, 16384, BF16, 1e-5,
                                       0x5EED0062, 0.5, mean_sigma=1.0),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
