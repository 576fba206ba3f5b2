"""Pins of the oracle's quantizer against hand-computed fixtures, library
conversions (torch's float8_e4m3fn and float16 casts) and invariants that the
definition fixes. CPU only."""
import numpy as np
import pytest
import torch

import oracle
from oracle.quant import pack_int4
from golden_io import load


def _golden_block(name):
    g = load(name)
    x = np.array(g["input"], dtype=np.float32)
    n = x.size
    x = x.reshape(1, 1, *(g.get("layout_rows_by_channels") or (n, 1)))
    codes, scales = oracle.block_quant(x, g["block_rows"], g["qtype"], g["scale_dtype"])
    return g, codes, scales


@pytest.mark.parametrize("name", ["int8_ties.txt", "int8_scale_half.txt", "e4m3_points.txt",
                                  "int4_pack.txt"])
def test_golden_quant(name):
    g, codes, scales = _golden_block(name)
    assert float(scales.ravel()[0]) == g["scale"]
    want = np.array(g["codes"] if isinstance(g["codes"], list) else [g["codes"]])
    if g["qtype"] == "int8":
        assert codes.ravel().astype(np.int64).tolist() == want.tolist()
    else:
        assert codes.ravel().astype(np.int64).tolist() == (want & 0xFF).tolist()


def _torch_e4m3(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _e4m3_test_values() -> np.ndarray:
    """Every fp16 and bf16 value with |x| <= 448, the 128 fp32 neighbours on each
    side of every e4m3 rounding midpoint, and random fp32 bit patterns."""
    parts = []
    h = np.arange(1 << 16, dtype=np.uint16).view(np.float16).astype(np.float32)
    parts.append(h)
    bf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    parts.append(bf)
    pos = oracle.e4m3fn_decode(np.arange(0x7F, dtype=np.uint8))  # 0 .. 448
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    bits = mids.view(np.uint32).astype(np.int64)
    off = np.arange(-128, 129)
    near = (bits[:, None] + off[None, :]).ravel()
    near = near[near >= 0].astype(np.uint32).view(np.float32)
    parts += [near, -near]
    rng = np.random.default_rng(0)
    rb = rng.integers(0, 0x43E00001, size=1 << 20, dtype=np.uint32).view(np.float32)
    parts += [rb, -rb]
    x = np.concatenate(parts)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    return x


def test_e4m3_encode_matches_torch():
    x = _e4m3_test_values()
    assert x.size > 300_000
    np.testing.assert_array_equal(oracle.e4m3fn_encode(x), _torch_e4m3(x))


def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3fn_decode(codes), ref)
    assert np.isnan(oracle.e4m3fn_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_saturation_of_clamped_values():
    # 463.999 is clamped to 448 before encoding; encoding itself rejects > 448.
    t = np.clip(np.float32(463.999), -448, 448)
    assert oracle.e4m3fn_encode(np.array([t]))[0] == 0x7E
    with pytest.raises(ValueError):
        oracle.e4m3fn_encode(np.array([449.0], np.float32))


def test_fp16_round_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(1 << 18).astype(np.float32) * 10.0 ** rng.integers(-8, 4, 1 << 18),
        # float32 values around every fp16 rounding midpoint of the positive range
        ((np.arange(0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
          + np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2
         ).astype(np.float32),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).half().float().numpy()
    np.testing.assert_array_equal(oracle.fp16_round(x), ref)


def test_int4_pack_roundtrip():
    rng = np.random.default_rng(2)
    c = rng.integers(-8, 8, size=(3, 5, 128)).astype(np.int8)
    p = pack_int4(c)
    assert p.shape == (3, 5, 64) and p.dtype == np.uint8
    np.testing.assert_array_equal(oracle.unpack_int4(p), c)
    assert p[0, 0, 0] == ((int(c[0, 0, 0]) & 0xF) | ((int(c[0, 0, 1]) & 0xF) << 4))


def _random_input(shape, dtype, seed, zero_block=None, block_rows=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(*shape, generator=g) * torch.exp(torch.randn(shape[:2] + (1, 1), generator=g))
    if zero_block is not None:
        b, n, r = zero_block
        x[b, n, r * block_rows:(r + 1) * block_rows] = 0
    return x.to(dtype)


CASES = [
    # qtype, block_rows, scale dtype, in dtype, S, D
    ("int8", 128, "f32", torch.float16, 300, 128),
    ("int8", 256, "f32", torch.float32, 513, 64),
    ("int8", 256, "f16", torch.float16, 700, 128),
    ("fp8", 128, "f32", torch.bfloat16, 260, 128),
    ("fp8", 256, "f32", torch.bfloat16, 511, 128),
    ("int4", 1, "f16", torch.float16, 37, 128),
    ("int4", 16, "f32", torch.float32, 50, 64),
]


@pytest.mark.parametrize("qtype,R,sdt,dt,S,D", CASES)
def test_quant_invariants(qtype, R, sdt, dt, S, D):
    qmax = oracle.QMAX[qtype]
    x = _random_input((2, 3, S, D), dt, seed=S + D, zero_block=(1, 2, 0), block_rows=R)
    codes, scales = oracle.block_quant(x, R, qtype, sdt)
    nblk = -(-S // R)
    assert scales.shape == (2, 3, nblk)
    assert scales.dtype == (np.float16 if sdt == "f16" else np.float32)
    vals = oracle.code_values(codes, qtype)
    x64 = x.double().numpy()
    s64 = np.repeat(scales.astype(np.float64), R, axis=2)[:, :, :S, None]
    # I3: |code| <= qmax
    assert np.abs(vals).max() <= qmax
    # zero block: scale 0 and all-zero codes
    assert scales[1, 2, 0] == 0 and np.all(vals[1, 2, :R] == 0)
    # I1: every nonzero block reaches qmax exactly
    blk = np.pad(np.abs(vals), ((0, 0), (0, 0), (0, nblk * R - S), (0, 0))).reshape(
        2, 3, nblk, R * D).max(axis=3)
    np.testing.assert_array_equal(blk[scales != 0], qmax)
    # amax definition: scale = fl32(amax / qmax), rounded to fp16 when asked
    amax = np.pad(np.abs(x.float().numpy()), ((0, 0), (0, 0), (0, nblk * R - S), (0, 0))
                  ).reshape(2, 3, nblk, R * D).max(axis=3)
    s_ref = (amax / np.float32(qmax)).astype(np.float32)
    if sdt == "f16":
        s_ref = torch.from_numpy(s_ref).half().float().numpy()
    np.testing.assert_array_equal(scales.astype(np.float32), s_ref)
    # I2: reconstruction error at most half a code step (plus the fp32 quotient's rounding)
    err = np.abs(x64 - s64 * vals)
    if qtype in ("int8", "int4"):
        bound = s64 * (0.5 + qmax * 2.0 ** -23)
    else:
        t = np.abs(vals)
        e = np.maximum(np.floor(np.log2(np.maximum(t, 2.0 ** -9))), -6)
        bound = s64 * (2.0 ** (e - 4) * 1.0001 + 448 * 2.0 ** -23)
    assert np.all(err <= bound + 1e-300)


@pytest.mark.parametrize("qtype,R", [("int8", 128), ("fp8", 256), ("int4", 1)])
def test_quant_layouts_agree(qtype, R):
    """I4: BSND codes equal BNSD codes transposed, scales identical."""
    x = _random_input((2, 3, 300, 64), torch.float16, seed=7)
    c1, s1 = oracle.block_quant(x, R, qtype, "f32", layout="bnsd")
    c2, s2 = oracle.block_quant(x.transpose(1, 2).contiguous(), R, qtype, "f32", layout="bsnd")
    np.testing.assert_array_equal(c2, c1.transpose(0, 2, 1, 3))
    np.testing.assert_array_equal(s1, s2)


def test_quant_row_permutation_within_block():
    """I5: permuting rows inside a block permutes the codes and keeps the scale."""
    x = _random_input((1, 2, 256, 128), torch.float32, seed=9)
    perm = torch.randperm(128, generator=torch.Generator().manual_seed(3))
    xp = x.clone()
    xp[:, :, :128] = x[:, :, perm]
    c1, s1 = oracle.block_quant(x, 128, "int8")
    c2, s2 = oracle.block_quant(xp, 128, "int8")
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c2[:, :, :128], c1[:, :, perm.numpy()])
    np.testing.assert_array_equal(c2[:, :, 128:], c1[:, :, 128:])


def test_quant_fp16_scale_codes_use_rounded_scale():
    """With fp16 scales, codes come from the stored (rounded) scale."""
    x = np.array([[[[1.0, -0.3, 0.77, 0.5]]]], dtype=np.float32)  # amax 1 -> 1/7 rounds in fp16
    codes, scales = oracle.block_quant(x, 1, "int4", "f16")
    s = np.float32(np.float16(np.float32(1.0) / np.float32(7.0)))
    assert scales.astype(np.float32)[0, 0, 0] == s
    t = (x / s).astype(np.float32)
    expect = np.clip(np.rint(t), -8, 7).astype(np.int64).ravel()
    np.testing.assert_array_equal(oracle.unpack_int4(codes).ravel(), expect)


def test_dequantize_inverse_layouts():
    x = _random_input((1, 2, 130, 64), torch.bfloat16, seed=11)
    for layout, xin in (("bnsd", x), ("bsnd", x.transpose(1, 2).contiguous())):
        codes, scales = oracle.block_quant(xin, 64, "fp8", layout=layout)
        xh = oracle.dequantize(codes, scales, 64, "fp8", layout=layout)
        assert xh.shape == (1, 2, 130, 64)
        s = np.repeat(scales.astype(np.float64), 64, axis=2)[:, :, :130, None]
        assert np.all(np.abs(xh - x.double().numpy()) <= s * 16 * (1 + 1e-6))


# ---- rotation + block quantization ----------------------------------------

def test_bf16_round_matches_torch():
    """On float32 inputs (one rounding either way) the float64 bf16 rounding
    agrees with torch's float32 -> bfloat16 conversion (nearest-even)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(1 << 18) * 10.0 ** rng.integers(-20, 20, 1 << 18)).astype(np.float32)
    ref = torch.from_numpy(x).bfloat16().double().numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x.astype(np.float64)), ref)


def test_bf16_round_is_one_rounding():
    """A value just above (below) the midpoint of two adjacent bf16 values goes
    up (down); the exact midpoint goes to the even neighbour. A detour through
    float32 would round 'just above' to the midpoint first."""
    lo = np.array([1.0, 1.5, 3.0, -7.25, 1e-3], dtype=np.float64)
    lo = oracle.bf16_round(lo)
    m, e = np.frexp(lo)
    step = np.ldexp(np.ones_like(lo), e - 8)            # bf16 spacing at lo
    mid = lo + np.sign(lo) * step / 2
    up = lo + np.sign(lo) * step
    eps = np.abs(mid) * 2.0 ** -40
    np.testing.assert_array_equal(oracle.bf16_round(mid + np.sign(lo) * eps), up)
    np.testing.assert_array_equal(oracle.bf16_round(mid - np.sign(lo) * eps), lo)
    # ties to even: of lo and up, the one whose 8-bit significand is even
    sig_lo = np.rint(np.ldexp(np.frexp(lo)[0], 8)).astype(np.int64)
    np.testing.assert_array_equal(oracle.bf16_round(mid), np.where(sig_lo % 2 == 0, lo, up))


def _rand16(shape, dt, seed):
    t = torch.from_numpy(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))
    return t.to(torch.bfloat16 if dt == "bf16" else torch.float16)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("qtype", ["int8", "fp8"])
def test_rotate_identity_is_block_quant(dt, qtype):
    x = _rand16((1, 2, 70, 64), dt, 11)
    eye = np.eye(64, dtype=np.float32)
    c1, s1 = oracle.rotate_block_quant(x, eye, 32, qtype, dt)
    c0, s0 = oracle.block_quant(x, 32, qtype)
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(s1, s0)


def test_rotate_permutation_permutes_channels():
    x = _rand16((2, 1, 40, 64), "bf16", 12)
    perm = np.random.default_rng(3).permutation(64)
    w = np.zeros((64, 64), dtype=np.float32)
    w[np.arange(64), perm] = 1.0                        # y[..., i] = x[..., perm[i]]
    c1, s1 = oracle.rotate_block_quant(x, w, 64, "fp8", "bf16", layout="bnsd")
    c0, s0 = oracle.block_quant(x[..., perm], 64, "fp8")
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(s1, s0)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_rotate_rounds_sums_once(dt):
    """w with two ones per row: y = x_a + x_b exactly, which float32 holds, so
    torch's float32 -> 16-bit conversion is the single nearest-even rounding
    the definition asks for; codes and scales must match block_quant of it."""
    x = _rand16((1, 1, 96, 64), dt, 13)
    rng = np.random.default_rng(4)
    a, b = rng.permutation(64), rng.permutation(64)
    w = np.zeros((64, 64), dtype=np.float32)
    w[np.arange(64), a] += 1.0
    w[np.arange(64), b] += 1.0
    xf = x.float()
    y = (xf[..., a] + xf[..., b]).to(x.dtype)
    c1, s1 = oracle.rotate_block_quant(x, w, 32, "int8", dt, layout="bsnd")
    c0, s0 = oracle.block_quant(y, 32, "int8", layout="bsnd")
    np.testing.assert_array_equal(c1, c0)
    np.testing.assert_array_equal(s1, s0)


def _row_w(D, cols, vals=None):
    """w whose row 0 sums the listed channels of x (times vals); identity elsewhere."""
    w = np.eye(D, dtype=np.float32)
    w[0] = 0.0
    for j, c in enumerate(cols):
        w[0, c] = 1.0 if vals is None else vals[j]
    return w


@pytest.mark.parametrize("dt,terms,want", [
    # 1 + 2^-8 is the midpoint between bf16 1 and 1 + 2^-7; a float64 sum drops
    # the 2^-70 term and would round the tie to even (1.0). The exact sum lies
    # above the midpoint and rounds up.
    ("bf16", [(1.0, 1.0), (2.0 ** -8, 1.0), (2.0 ** -70, 1.0)], 1.0 + 2.0 ** -7),
    ("bf16", [(1.0, 1.0), (2.0 ** -8, 1.0), (-(2.0 ** -70), 1.0)], 1.0),
    # the same in fp16 (midpoint 1 + 2^-11); the tiny term is 2^-24 * 2^-40
    ("f16", [(1.0, 1.0), (2.0 ** -11, 1.0), (2.0 ** -24, 2.0 ** -40)], 1.0 + 2.0 ** -10),
    # exact ties round to even: 1 + 2^-8 -> 1, (1 + 2^-7) + 2^-8 -> 1 + 2^-6
    ("bf16", [(1.0, 1.0), (2.0 ** -8, 1.0)], 1.0),
    ("bf16", [(1.0 + 2.0 ** -7, 1.0), (2.0 ** -8, 1.0)], 1.0 + 2.0 ** -6),
    ("f16", [(1.0 + 2.0 ** -10, 1.0), (2.0 ** -11, 1.0)], 1.0 + 2.0 ** -9),
    # f16 subnormal result: 2^-24 + 2^-25 is a tie between 2^-24 and 2^-23
    ("f16", [(2.0 ** -24, 1.0), (2.0 ** -24, 0.5)], 2.0 ** -23),
])
def test_rotate16_rounds_the_exact_sum(dt, terms, want):
    D = 8
    x = torch.zeros(1, 1, 1, D, dtype=torch.float32)
    vals = []
    for c, (xv, wv) in enumerate(terms):
        x[0, 0, 0, c] = xv
        vals.append(wv)
    x = x.to(torch.bfloat16 if dt == "bf16" else torch.float16)
    assert [float(x[0, 0, 0, c]) for c in range(len(terms))] == [t[0] for t in terms]
    w = _row_w(D, range(len(terms)), vals)
    y = oracle.rotate16(x, w, dt)
    assert y[0, 0, 0, 0] == want
    # channels 1.. are the identity rows of w: y equals x there
    np.testing.assert_array_equal(y[0, 0, 0, 1:], x.double().numpy()[0, 0, 0, 1:])


def _neighbours16(v: float, dt):
    """The two 16-bit values adjacent to the 16-bit value nearest v (by bits)."""
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    c = torch.tensor([v], dtype=torch.float64).to(tdt)
    bits = c.view(torch.int16)
    out = [c]
    for d in (-1, 1):
        out.append((bits + d).view(tdt))
    return [float(t) for t in out], [int(t.view(torch.int16)) for t in out]


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_rotate16_brute_force(dt):
    """Tiny random case: every output against the exact rational sum. The
    result must be the closest of the candidate 16-bit values around it (the
    even one on a tie)."""
    from fractions import Fraction
    x = _rand16((1, 2, 3, 16), dt, 31)
    rot = np.linalg.qr(np.random.default_rng(7).standard_normal((16, 16)))[0]
    w = torch.from_numpy(rot).to(torch.bfloat16 if dt == "bf16" else torch.float16)
    y = oracle.rotate16(x, w, dt)
    xs, ws = x.double().numpy(), w.double().numpy()
    for idx in np.ndindex(*y.shape):
        exact = sum((Fraction(a) * Fraction(b) for a, b in zip(xs[idx[:-1]], ws[idx[-1]])),
                    Fraction(0))
        vals, bits = _neighbours16(float(exact), dt)
        dist = [abs(Fraction(v) - exact) for v in vals]
        best = min(dist)
        cands = [(v, b) for v, b, d in zip(vals, bits, dist) if d == best]
        if len(cands) > 1:  # a tie: the even significand
            cands = [c for c in cands if c[1] % 2 == 0]
        assert y[idx] == cands[0][0], (idx, float(exact), y[idx], cands)


# ---- quantizing into an existing scale; KV-cache append --------------------

@pytest.mark.parametrize("qtype", ["int8", "int4", "fp8"])
def test_quantize_with_scale_matches_block_quant(qtype):
    x = np.random.default_rng(21).standard_normal((1, 1, 40, 32)).astype(np.float32) * 3
    c, s = oracle.block_quant(x, 40, qtype)
    q = oracle.quantize_with_scale(x, s[0, 0, 0], qtype)
    if qtype == "int4":
        q = pack_int4(q)
    np.testing.assert_array_equal(q, c)


def _cache(B, H, S, D, R, qtype, sdt="f16"):
    codes = np.zeros((B, H, S, D // 2 if qtype == "int4" else D),
                     dtype=np.int8 if qtype == "int8" else np.uint8)
    scales = np.zeros((B, H, -(-S // R)), dtype=np.float16 if sdt == "f16" else np.float32)
    return codes, scales


@pytest.mark.parametrize("qtype,R", [("int8", 16), ("int4", 1), ("int4", 8)])
def test_kv_append_first_row_of_a_block_is_block_quant(qtype, R):
    rng = np.random.default_rng(22)
    codes, scales = _cache(2, 3, 40, 16, R, qtype)
    x = rng.standard_normal((2, 3, 16)).astype(np.float32)
    pos = np.array([R * 2, 0])
    c, s = oracle.kv_append(codes, scales, x, pos, R, qtype)
    for b in range(2):
        ref_c, ref_s = oracle.block_quant(x[b][:, None, :][None], 1, qtype, "f16")
        np.testing.assert_array_equal(c[b, :, pos[b]], ref_c[0, :, 0])
        np.testing.assert_array_equal(s[b, :, pos[b] // R], ref_s[0, :, 0])


@pytest.mark.parametrize("qtype", ["int8", "int4"])
def test_kv_append_rows_that_fit_equal_block_quant(qtype):
    """Row 0 holds the block's largest value, so every later row fits its scale
    and the appended block equals block_quant of the rows at once."""
    rng = np.random.default_rng(23)
    R, D = 8, 16
    rows = rng.standard_normal((R, D)).astype(np.float32)
    rows[0, 3] = 10.0
    codes, scales = _cache(1, 1, R, D, R, qtype)
    for p in range(R):
        codes, scales = oracle.kv_append(codes, scales, rows[p][None, None], [p], R, qtype)
    ref_c, ref_s = oracle.block_quant(rows[None, None], R, qtype, "f16")
    np.testing.assert_array_equal(codes, ref_c)
    np.testing.assert_array_equal(scales, ref_s)


def test_kv_append_raising_the_amax_requantizes_the_block():
    rng = np.random.default_rng(24)
    R, D = 8, 16
    rows = rng.standard_normal((4, D)).astype(np.float32)
    codes, scales = _cache(1, 1, R, D, R, "int8", "f32")
    for p in range(3):
        codes, scales = oracle.kv_append(codes, scales, rows[p][None, None], [p], R, "int8", "f32")
    big = rows[3] * 0 + 0.5
    big[5] = 50.0                                        # far above the block's amax
    c, s = oracle.kv_append(codes, scales, big[None, None], [3], R, "int8", "f32")
    assert s[0, 0, 0] == np.float32(np.float32(50.0) / np.float32(127.0))
    assert c[0, 0, 3, 5] == 127                          # the new maximum reaches qmax
    # old rows: block_quant of their dequantized fp32 values together with the new row
    old = (codes[0, 0, :3].astype(np.float32) * scales[0, 0, 0]).astype(np.float32)
    ref_c, ref_s = oracle.block_quant(np.concatenate([old, big[None]])[None, None], 4, "int8")
    np.testing.assert_array_equal(c[0, 0, :4], ref_c[0, 0])
    np.testing.assert_array_equal(c[0, 0, 4:], 0)        # rows past the new one untouched


def test_kv_append_out_of_range_position_changes_nothing():
    codes, scales = _cache(2, 1, 16, 16, 8, "int8")
    x = np.ones((2, 1, 16), np.float32)
    c, s = oracle.kv_append(codes, scales, x, [16, -1], 8, "int8")
    np.testing.assert_array_equal(c, codes)
    np.testing.assert_array_equal(s, scales)
