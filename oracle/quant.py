"""Oracle: symmetric per-block quantization (test infrastructure only).

Definition followed, step by step:

1. Upcast the input to IEEE float32 (exact for fp16 and bf16).
2. A block is ``R`` consecutive sequence rows times all ``D`` channels of one
   (batch, head); the last block of a sequence may be short. Q uses R=128 and
   K/V R=256 ([MindIE-SD] FA quantization, "块量化" step: dynamic block
   quantization with Q block 128 and K/V block 256); INT4 K/V use R=1 (one
   group of D=128 channels per token and head, [OT-Quant] section 5.1 on
   group-wise quantization with groups of 128 and one FP16 scale each).
3. ``amax = max |x|`` over the block (exact in float32).
4. ``s = fl32(amax / qmax)`` with qmax = 127 for INT8 ([Ascend-INT8] section
   "对称量化 vs 非对称量化": symmetric scale max(abs(x))/127, zero point 0),
   448 for FP8 e4m3fn (its largest finite value) and 7 for INT4 (symmetric
   range of [-8, 7], [FA-INT8/INT4] INT4 layer). When scales are stored as fp16
   the scale is rounded to fp16 first and the codes use the rounded value.
5. ``t = fl32(x / s)`` (correctly rounded division, [Ascend-INT8] reference
   quantizer ``round(x / scale)``), then
   * INT8: ``clamp(rne(t), -128, 127)`` (same passage: round, clamp to
     [-128, 127]);
   * INT4: ``clamp(rne(t), -8, 7)``, two codes per byte, element 2k in the low
     nibble and 2k+1 in the high nibble as two's-complement nibbles
     ([OT-Quant] section 5.2, packed INT4 byte layout);
   * FP8: ``e4m3fn(rne(clamp(t, -448, 448)))`` ([MindIE-SD] FA quantization:
     Q/K/V quantized to float8_e4m3fn).
6. A block whose stored scale is 0 (all-zero block) gets all-zero codes.

Rounding is round-half-to-even throughout (numpy ``rint``; torch ``round`` in
the [Ascend-INT8] listing has the same rule).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

QMAX = {"int8": 127.0, "fp8": 448.0, "int4": 7.0}


def _to_f32(x) -> np.ndarray:
    """float32 numpy copy of a torch tensor (any float dtype) or numpy array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float32)


def _to_bnsd(a: np.ndarray, layout: str) -> np.ndarray:
    if layout == "bnsd":
        return a
    if layout == "bsnd":
        return np.ascontiguousarray(a.transpose(0, 2, 1, 3))
    raise ValueError(f"unknown layout {layout!r}")


def fp16_round(x) -> np.ndarray:
    """Round float32 values to the nearest IEEE binary16 value (ties to even)
    and return them as float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def e4m3fn_encode(t) -> np.ndarray:
    """Encode float32 values with |t| <= 448 as OCP FP8 E4M3 ("fn" flavour) bytes.

    Format (OCP 8-bit floating point specification): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
    m * 2^-9; no infinities; S.1111.111 is NaN; largest finite value 448.
    Rounding is to nearest, ties to even; the sign of a value that rounds to
    zero is kept (-0 encodes as 0x80).
    """
    t = np.asarray(t, dtype=np.float32)
    if not np.all(np.abs(t) <= 448.0):
        raise ValueError("e4m3fn_encode expects finite |t| <= 448")
    sign = np.signbit(t).astype(np.uint8) << np.uint8(7)
    a = np.abs(t).astype(np.float64)
    _, E = np.frexp(a)                      # a = f * 2**E with f in [0.5, 1)
    e = np.maximum(E - 1, -6)               # binade; subnormals share 2^-6's spacing
    quantum = np.ldexp(1.0, e - 3)          # 3 mantissa bits
    mag = np.rint(a / quantum) * quantum    # exact: quantum is a power of two
    _, E2 = np.frexp(mag)
    e2 = E2 - 1
    normal = mag >= 2.0 ** -6
    exp_field = np.where(normal, e2 + 7, 0)
    mant = np.where(normal, (mag / np.ldexp(1.0, e2) - 1.0) * 8.0, mag / 2.0 ** -9)
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    return (sign | code.astype(np.uint8)).astype(np.uint8)


def e4m3fn_decode(codes) -> np.ndarray:
    """Value of OCP E4M3 ("fn") bytes as float64 (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def pack_int4(c: np.ndarray) -> np.ndarray:
    """Two signed 4-bit codes per byte along the last axis: element 2k in the
    low nibble, element 2k+1 in the high nibble ([OT-Quant] section 5.2)."""
    c = c.astype(np.int64)
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(p) -> np.ndarray:
    """Inverse of ``pack_int4``: int8 codes in [-8, 7], last axis doubled."""
    p = np.asarray(p, dtype=np.uint8).astype(np.int64)
    lo = p & 0xF
    hi = p >> 4
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def block_quant(x, block_rows: int, qtype: str, scale_dtype: str = "f32",
                layout: str = "bnsd"):
    """Quantize ``x`` ([B,N,S,D] for "bnsd", [B,S,N,D] for "bsnd") per block of
    ``block_rows`` sequence rows of one (batch, head).

    Returns ``(codes, scales)``: codes in the input layout (int8 for INT8,
    uint8 e4m3fn bytes for FP8, uint8 packed pairs with last axis D/2 for INT4)
    and scales of shape [B, N, ceil(S/block_rows)] (float32, or float16 when
    ``scale_dtype == "f16"``).
    """
    if qtype not in QMAX:
        raise ValueError(f"unknown qtype {qtype!r}")
    if block_rows < 1:
        raise ValueError("block_rows must be >= 1")
    x32 = _to_bnsd(_to_f32(x), layout)
    B, N, S, D = x32.shape
    if qtype == "int4" and D % 2:
        raise ValueError("INT4 needs an even number of channels")
    R = block_rows
    nblk = -(-S // R)
    pad = nblk * R - S
    xp = np.pad(x32, ((0, 0), (0, 0), (0, pad), (0, 0))) if pad else x32
    blocks = xp.reshape(B, N, nblk, R, D)
    amax = np.abs(blocks).max(axis=(3, 4)) if S else np.zeros((B, N, 0), np.float32)
    s = (amax / np.float32(QMAX[qtype])).astype(np.float32)
    if scale_dtype == "f16":
        s = fp16_round(s)
    elif scale_dtype != "f32":
        raise ValueError(f"unknown scale dtype {scale_dtype!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (blocks / s[..., None, None]).astype(np.float32)
    t = np.where((s == 0)[..., None, None], np.float32(0.0), t)
    if qtype == "int8":
        codes = np.clip(np.rint(t), -128, 127).astype(np.int8)
    elif qtype == "int4":
        codes = np.clip(np.rint(t), -8, 7).astype(np.int8)
    else:
        codes = e4m3fn_encode(np.clip(t, np.float32(-448.0), np.float32(448.0)))
    codes = codes.reshape(B, N, nblk * R, D)[:, :, :S]
    if qtype == "int4":
        codes = pack_int4(codes)
    if layout == "bsnd":
        codes = np.ascontiguousarray(codes.transpose(0, 2, 1, 3))
    scales = s.astype(np.float16) if scale_dtype == "f16" else s
    return np.ascontiguousarray(codes), scales


def code_values(codes, qtype: str) -> np.ndarray:
    """Integer or e4m3 value of each code as float64 (INT4 unpacked)."""
    if qtype == "int8":
        return np.asarray(codes).astype(np.int8).astype(np.float64)
    if qtype == "int4":
        return unpack_int4(codes).astype(np.float64)
    if qtype == "fp8":
        return e4m3fn_decode(codes)
    raise ValueError(f"unknown qtype {qtype!r}")


def dequantize(codes, scales, block_rows: int, qtype: str, layout: str = "bnsd") -> np.ndarray:
    """``s_block * value(code)`` in float64, returned as BNSD [B,N,S,D]."""
    vals = _to_bnsd(code_values(codes, qtype), layout)
    B, N, S, D = vals.shape
    s = np.asarray(scales).astype(np.float64)
    row_scale = np.repeat(s, block_rows, axis=2)[:, :, :S]
    return vals * row_scale[..., None]


def bf16_round(y) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (8 significant bits,
    ties to even, one rounding) and return them as float64. Values are assumed
    normal in bfloat16 (no overflow or subnormal results)."""
    y = np.asarray(y, dtype=np.float64)
    m, e = np.frexp(y)  # y = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def _round_fraction16(v: Fraction, in_dtype: str) -> float:
    """Nearest value of ``in_dtype`` ("bf16": 8 significant bits, exponents
    down to -126; "f16": 11 bits, down to -14, subnormals below) to the exact
    rational ``v``, ties to even (``round`` of a Fraction rounds half to even)."""
    if v == 0:
        return 0.0
    bits, emin = (8, -126) if in_dtype == "bf16" else (11, -14)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - bits + 1)
    r = float(round(a / quantum) * quantum)
    return r if v > 0 else -r


def rotate16(x, w, in_dtype: str) -> np.ndarray:
    """``y[..., i] = round16(sum_k x[..., k] * w[i, k])`` as float64: the exact
    sum of products, rounded once to ``in_dtype`` ("bf16" or "f16"), nearest-even.

    Every product of a 16-bit x and a float32 w is exact in float64, so the
    float64 matrix product differs from the exact sum by at most
    ``D * 2^-53 * sum_k |x_k w_ik|`` (the bound for any summation order). Where
    the 16-bit roundings of the two ends of that interval agree, rounding is
    monotone, so the exact sum rounds to the same value; elsewhere the sum is
    recomputed in exact rational arithmetic and rounded from there.
    """
    if in_dtype not in ("bf16", "f16"):
        raise ValueError(f"unknown input dtype {in_dtype!r}")
    x64 = np.asarray(_to_f32(x), dtype=np.float64)
    w64 = np.asarray(_to_f32(w), dtype=np.float64)
    r16 = bf16_round if in_dtype == "bf16" else (lambda t: t.astype(np.float16).astype(np.float64))
    y = x64 @ w64.T
    err = 2.0 * x64.shape[-1] * 2.0 ** -53 * (np.abs(x64) @ np.abs(w64).T)  # 2x margin
    out = r16(y)
    for idx in np.argwhere(r16(y - err) != r16(y + err)):
        idx = tuple(idx)
        xs, ws = x64[idx[:-1]], w64[idx[-1]]
        exact = sum((Fraction(a) * Fraction(b) for a, b in zip(xs.tolist(), ws.tolist())),
                    Fraction(0))
        out[idx] = _round_fraction16(exact, in_dtype)
    return out


def rotate_block_quant(x, w, block_rows: int, qtype: str, in_dtype: str,
                       scale_dtype: str = "f32", layout: str = "bnsd"):
    """Rotate, then block-quantize ([MindIE-SD] FP8 attention: Q and K are
    multiplied by an orthogonal matrix before the dynamic block quantization).

    ``y = rotate16(x, w, in_dtype)``: the exact product of the 16-bit inputs
    rounded once to ``in_dtype``, with x in ``layout``; then ``block_quant`` on
    y. Returns (codes, scales) as ``block_quant`` does.
    """
    y = rotate16(x, w, in_dtype)
    return block_quant(y.astype(np.float32), block_rows, qtype, scale_dtype, layout)


def quantize_with_scale(values, s: float, qtype: str) -> np.ndarray:
    """Codes of float32 ``values`` for a given scale ``s``: step 5 of the
    definition above (``t = fl32(x / s)``, round half to even, clamp, or the
    e4m3fn encoding); all-zero codes when s is 0. INT4 codes are returned
    unpacked (int8 values in [-8, 7])."""
    v = np.asarray(values, dtype=np.float32)
    if not s != 0:
        return (np.zeros(v.shape, np.uint8) if qtype == "fp8" else np.zeros(v.shape, np.int8))
    t = (v / np.float32(s)).astype(np.float32)
    if qtype == "int8":
        return np.clip(np.rint(t), -128, 127).astype(np.int8)
    if qtype == "int4":
        return np.clip(np.rint(t), -8, 7).astype(np.int8)
    return e4m3fn_encode(np.clip(t, np.float32(-448.0), np.float32(448.0)))


def kv_append(codes, scales, x, positions, kv_block: int, qtype: str, scale_dtype: str = "f16",
              layout: str = "bnsd"):
    """Quantize one new token per sequence into an INT8 or packed-INT4 KV cache
    ([Ascend-INT8] section 3: the decode cache is stored quantized, so a new
    token is quantized into it; the block-scale update is this reading).

    codes [B,H,S_max,D] (INT4: D/2 packed bytes) and scales [B,H,ceil(S_max/R)]
    are the cache; x [B,H,D] holds the new key (or value) rows; token b goes to
    row ``positions[b]`` (a row outside [0, S_max) leaves sequence b alone).
    For the block r = p // R holding row p, with old rows [rR, p):

    * if the block has old rows, its scale s is nonzero and fl32(max|x| / s)
      <= qmax (or x is all zero), x is quantized with s and nothing else
      changes;
    * otherwise the block is requantized as one block: the old rows' values
      fl32(code * s) together with x go through ``block_quant`` (a new scale
      from their amax, new codes for every row of the block up to p).

    Returns new (codes, scales) arrays in the input layout; rows past p are
    not touched.
    """
    c = _to_bnsd(np.array(codes), layout).copy()
    sc = np.array(scales).copy()
    xv = np.asarray(_to_f32(x), dtype=np.float32)
    B, H, S_max = c.shape[0], c.shape[1], c.shape[2]
    R = kv_block
    qmax = np.float32(QMAX[qtype])
    for b in range(B):
        p = int(positions[b])
        if p < 0 or p >= S_max:
            continue
        r, row0 = p // R, (p // R) * R
        for h in range(H):
            xr = xv[b, h]
            ax = np.float32(np.abs(xr).max()) if xr.size else np.float32(0)
            fits = False
            s_old = np.float32(sc[b, h, r])
            if p > row0:
                if s_old > 0:
                    fits = bool(np.float32(ax / s_old) <= qmax)
                else:
                    fits = bool(ax == 0)
            if fits:
                q = quantize_with_scale(xr, s_old, qtype)
                c[b, h, p] = pack_int4(q[None])[0] if qtype == "int4" else q
                continue
            old = code_values(c[b, h, row0:p], qtype).astype(np.float32)
            vals = np.concatenate([(old * s_old).astype(np.float32), xr[None]], axis=0)
            nc, ns = block_quant(vals[None, None], p + 1 - row0, qtype, scale_dtype)
            c[b, h, row0:p + 1] = nc[0, 0]
            sc[b, h, r] = ns[0, 0, 0]
    if layout == "bsnd":
        c = np.ascontiguousarray(c.transpose(0, 2, 1, 3))
    return c, sc
