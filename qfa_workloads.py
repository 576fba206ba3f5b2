"""Seeded synthetic inputs for the block-quantized attention workloads.

This module only draws random numbers and casts them to the input dtype of a
workload. It holds none of the quantization or attention arithmetic, and it is
the one module that both the CPU oracle's callers and the GPU path's callers
share. Every draw comes from a ``torch.Generator`` seeded with the workload's
seed, on the device the caller asks for (CPU draws and GPU draws differ; a run
always hands the same tensors to both sides).

Workloads (names carry their sizes):

* ``tiny_int8_s256_d64``      B=1, H=1, S=256, D=64, fp32 N(0,1), INT8, non-causal.
* ``int8_causal_h32_s4096``   B=1, H=32, S=4096, D=128, fp16 N(0,1), four fixed
                              K channels scaled by 20 (LLaMA-2-7B head shape), causal.
* ``fp8_rot_b2_h24_s4608``    B=2, H=24, S=4608, D=128, bf16 N(0,1); Q and K
                              multiplied by a seeded random orthogonal 128x128
                              matrix before the bf16 cast; FP8 e4m3fn, non-causal.
* ``int8_kv_decode_b32_h32``  B=32, Hq=Hkv=32, D=128, one fp16 query token,
                              context lengths uniform in [4096, 8192].
* ``gqa64x8_int4kv_causal_s16384`` B=1, Hq=64, Hkv=8, S=16384, D=128, fp16
                              N(0,1), 1% of K elements scaled by 10, causal.
"""
from __future__ import annotations

import dataclasses
import math

import torch

BNSD = "bnsd"
BSND = "bsnd"

_TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPES[name]


@dataclasses.dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    in_dtype: str          # "f32" | "f16" | "bf16"
    seed: int
    q_qtype: str           # "int8" | "fp8" | "int4"
    k_qtype: str
    v_qtype: str
    q_block: int           # rows per Q scale block
    kv_block: int          # rows per K/V scale block (1 = per token)
    q_scale_dtype: str     # "f32" | "f16"
    kv_scale_dtype: str
    causal: bool
    out_dtype: str
    softmax_scale: float   # exact float32 value handed to the kernels
    k_outlier_channels: int = 0      # fixed channels of K multiplied by k_outlier_factor
    k_outlier_frac: float = 0.0      # Bernoulli fraction of K elements multiplied
    k_outlier_factor: float = 1.0
    rotate_qk: bool = False

    def attention_ops(self) -> int:
        """Algorithmic ops (multiply and add counted separately) of the two
        contractions, unmasked pairs only."""
        if self.causal:
            return 2 * self.B * self.Hq * self.D * self.S * (self.S + 1)
        return 4 * self.B * self.Hq * self.S * self.S * self.D


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S_max: int
    len_lo: int
    len_hi: int            # inclusive
    seed: int
    kv_qtype: str
    kv_block: int
    kv_scale_dtype: str
    q_dtype: str
    out_dtype: str
    softmax_scale: float


def _f32(x: float) -> float:
    return float(torch.tensor(x, dtype=torch.float32).item())


TINY = PrefillWorkload(
    name="tiny_int8_s256_d64", B=1, Hq=1, Hkv=1, S=256, D=64, in_dtype="f32", seed=1,
    q_qtype="int8", k_qtype="int8", v_qtype="int8", q_block=128, kv_block=256,
    q_scale_dtype="f32", kv_scale_dtype="f32", causal=False, out_dtype="f32",
    softmax_scale=0.125)

INT8_CAUSAL = PrefillWorkload(
    name="int8_causal_h32_s4096", B=1, Hq=32, Hkv=32, S=4096, D=128, in_dtype="f16", seed=2,
    q_qtype="int8", k_qtype="int8", v_qtype="int8", q_block=128, kv_block=256,
    q_scale_dtype="f32", kv_scale_dtype="f32", causal=True, out_dtype="f16",
    softmax_scale=_f32(1.0 / math.sqrt(128)), k_outlier_channels=4, k_outlier_factor=20.0)

FP8_ROT = PrefillWorkload(
    name="fp8_rot_b2_h24_s4608", B=2, Hq=24, Hkv=24, S=4608, D=128, in_dtype="bf16", seed=3,
    q_qtype="fp8", k_qtype="fp8", v_qtype="fp8", q_block=128, kv_block=256,
    q_scale_dtype="f32", kv_scale_dtype="f32", causal=False, out_dtype="bf16",
    softmax_scale=_f32(1.0 / math.sqrt(128)), rotate_qk=True)

GQA_INT4 = PrefillWorkload(
    name="gqa64x8_int4kv_causal_s16384", B=1, Hq=64, Hkv=8, S=16384, D=128, in_dtype="f16",
    seed=5, q_qtype="int8", k_qtype="int4", v_qtype="int4", q_block=128, kv_block=1,
    q_scale_dtype="f32", kv_scale_dtype="f16", causal=True, out_dtype="f16",
    softmax_scale=_f32(1.0 / math.sqrt(128)), k_outlier_frac=0.01, k_outlier_factor=10.0)

DECODE = DecodeWorkload(
    name="int8_kv_decode_b32_h32", B=32, Hq=32, Hkv=32, D=128, S_max=8192, len_lo=4096,
    len_hi=8192, seed=4, kv_qtype="int8", kv_block=256, kv_scale_dtype="f16", q_dtype="f16",
    out_dtype="f16", softmax_scale=_f32(1.0 / math.sqrt(128)))

# The INT8 causal prefill shape with packed INT4 V codes (INT8 Q and K, one
# scale per 256 keys): the mixed-precision variant of the pages' INT8/INT4 layers.
INT8QK_INT4V = dataclasses.replace(INT8_CAUSAL, name="int8qk_int4v_causal_h32_s4096",
                                   v_qtype="int4")

# The decode shape above with a packed INT4 cache (two codes per byte, one
# fp16 scale per 256-token block): half the cache bytes of INT8.
DECODE_INT4 = dataclasses.replace(DECODE, name="int4_kv_decode_b32_h32", kv_qtype="int4")

# The same decode shape with grouped KV heads: 32 query heads over 8 (groups
# of 4) with the INT8 cache, over 2 (groups of 16) with the packed INT4 cache.
DECODE_GQA4 = dataclasses.replace(DECODE, name="int8_kv_decode_b32_h32_gqa4", Hkv=8)
DECODE_GQA16_INT4 = dataclasses.replace(DECODE_INT4, name="int4_kv_decode_b32_h32_gqa16", Hkv=2)

PREFILL_WORKLOADS = {w.name: w for w in (TINY, INT8_CAUSAL, FP8_ROT, GQA_INT4)}


def scaled(w: PrefillWorkload, **changes) -> PrefillWorkload:
    """The same recipe at other sizes (used for small parity cases)."""
    return dataclasses.replace(w, **changes)


def random_orthogonal(D: int, gen: torch.Generator) -> torch.Tensor:
    """Haar-random orthogonal D x D matrix in float64: the Q factor of a Gaussian
    matrix with the signs of R's diagonal moved onto Q's columns (Mezzadri 2007)."""
    g = torch.randn(D, D, generator=gen, dtype=torch.float64, device=gen.device)
    qm, rm = torch.linalg.qr(g.cpu())
    qm = qm * torch.sign(torch.diagonal(rm)).unsqueeze(0)
    return qm.to(gen.device)


def _randn(shape, gen) -> torch.Tensor:
    return torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device)


def make_prefill_inputs(w: PrefillWorkload, device="cpu", layout: str = BNSD):
    """Q [B,Hq,S,D], K and V [B,Hkv,S,D] in ``w.in_dtype`` (BNSD), or the BSND
    transposes [B,S,H,D] made contiguous.

    Draw order from one generator: outlier channels (if any), Q, K, V, then the
    outlier mask (if any), then the rotation (if any).
    """
    gen = torch.Generator(device=device).manual_seed(w.seed)
    dt = torch_dtype(w.in_dtype)
    chans = None
    if w.k_outlier_channels:
        chans = torch.randperm(w.D, generator=gen, device=device)[: w.k_outlier_channels]
    q = _randn((w.B, w.Hq, w.S, w.D), gen)
    k = _randn((w.B, w.Hkv, w.S, w.D), gen)
    v = _randn((w.B, w.Hkv, w.S, w.D), gen)
    if chans is not None:
        k[..., chans] *= w.k_outlier_factor
    if w.k_outlier_frac > 0:
        mask = torch.rand(k.shape, generator=gen, device=device) < w.k_outlier_frac
        k = torch.where(mask, k * w.k_outlier_factor, k)
        del mask
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if w.rotate_qk:
        rot = random_orthogonal(w.D, gen)
        q = (q.double() @ rot).to(dt)
        k = (k.double() @ rot).to(dt)
    if layout == BSND:
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    return q, k, v


def outlier_channels(w: PrefillWorkload, device="cpu"):
    """The fixed outlier channels of K (first draw of the workload's generator)."""
    gen = torch.Generator(device=device).manual_seed(w.seed)
    return torch.randperm(w.D, generator=gen, device=device)[: w.k_outlier_channels]


def make_decode_inputs(w: DecodeWorkload, device="cpu", B: int | None = None,
                       S_max: int | None = None, len_lo: int | None = None,
                       len_hi: int | None = None):
    """Returns (q [B,Hq,1,D], k_src, v_src [B,Hkv,S_max,D], lens int32 [B]).

    Rows at or beyond a sequence's length are zero in the sources. Draw order:
    lengths, q, then K and V one batch element at a time.
    """
    B = w.B if B is None else B
    S_max = w.S_max if S_max is None else S_max
    lo = w.len_lo if len_lo is None else len_lo
    hi = w.len_hi if len_hi is None else len_hi
    gen = torch.Generator(device=device).manual_seed(w.seed)
    lens = torch.randint(lo, hi + 1, (B,), generator=gen, device=device, dtype=torch.int64)
    dt = torch_dtype(w.q_dtype)
    q = _randn((B, w.Hq, 1, w.D), gen).to(dt)
    k = torch.zeros(B, w.Hkv, S_max, w.D, dtype=dt, device=device)
    v = torch.zeros(B, w.Hkv, S_max, w.D, dtype=dt, device=device)
    for b in range(B):
        L = int(lens[b])
        k[b, :, :L] = _randn((w.Hkv, L, w.D), gen).to(dt)
        v[b, :, :L] = _randn((w.Hkv, L, w.D), gen).to(dt)
    return q, k, v, lens.to(torch.int32)


def decode_kv_bytes(w: DecodeWorkload, lens, D: int | None = None) -> int:
    """Algorithmic HBM bytes of one decode pass: K and V codes of the valid rows,
    their block scales, the query and the output."""
    D = w.D if D is None else D
    code_bytes = D if w.kv_qtype != "int4" else D // 2
    sbytes = 2 if w.kv_scale_dtype == "f16" else 4
    qbytes = 2 if w.q_dtype != "f32" else 4
    obytes = 2 if w.out_dtype != "f32" else 4
    total = 0
    for L in [int(x) for x in lens]:
        nblk = -(-L // w.kv_block)
        total += w.Hkv * (2 * L * code_bytes + 2 * nblk * sbytes)
    total += len(lens) * w.Hq * D * (qbytes + obytes)
    return total
