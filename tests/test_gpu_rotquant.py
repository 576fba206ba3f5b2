"""GPU parity of qfa_rotate_block_quant against the oracle's rotation (exact
product rounded once to 16 bits) followed by block quantization.

The GPU sums the 16-bit products in fp32 on the matrix unit. Where the exact
product lies within the fp32 error bound of a 16-bit rounding midpoint, either
neighbour is a correct rounding of a correctly computed sum, so those
elements ("ambiguous") may get any code between those of the two ends of
that interval (one step apart away from zero, several near zero); a block whose amax such an
element could change may get the other scale. Every block is compared: where the
GPU took the other scale, the oracle's 16-bit values are re-quantized with the
GPU's scale (after checking that an ambiguous element explains it) and the
codes compared as elsewhere; all other elements match byte for byte."""
import numpy as np
import pytest
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl
from gpu_util import SDT, say

pytestmark = pytest.mark.gpu


def _round16(y, dt):
    return oracle.bf16_round(y) if dt == "bf16" else y.astype(np.float16).astype(np.float64)


def _inputs(B, N, S, D, dt, layout, seed):
    gen = torch.Generator().manual_seed(seed)
    x = torch.randn(B, N, S, D, generator=gen, dtype=torch.float64)
    x[..., :3] *= 20.0  # a few outlier channels, which the rotation spreads
    rot = wl.random_orthogonal(D, gen)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    x = x.to(tdt)
    w = rot.t().contiguous().to(tdt)  # y = x . rot = x . w^T
    if layout == "bsnd":
        x = x.transpose(1, 2).contiguous()
    return x, w


def _scale_of(amax, qtype, sdt):
    """The stored scale the definition gives for a block with this amax."""
    s = np.float32(np.float32(amax) / np.float32(oracle.QMAX[qtype]))
    return np.float16(s) if sdt == "f16" else s


def _check(x, w, R, qtype, dt, sdt, layout, heads=None):
    say(f"rotate+quant {tuple(x.shape)} {dt} {qtype} R={R} scales={sdt} {layout} heads={heads}")
    gc, gs = qfa.rotate_block_quant(x.cuda(), w.cuda(), R, qtype, SDT[sdt], layout)
    torch.cuda.synchronize()
    xb = x if layout == "bnsd" else x.transpose(1, 2)
    gcb = gc.cpu() if layout == "bnsd" else gc.cpu().transpose(1, 2)
    gsb = gs.cpu()
    if heads is not None:
        xb, gcb, gsb = xb[:, heads], gcb[:, heads], gsb[:, heads]
    xb = xb.contiguous()
    y16 = oracle.rotate16(xb, w, dt)
    rc, rs = oracle.block_quant(y16.astype(np.float32), R, qtype, sdt, "bnsd")
    gcb = gcb.contiguous().numpy()
    gsb = gsb.numpy()
    # Ambiguous elements: the 16-bit rounding of the exact sum moved by a bound
    # on the fp32 accumulation error. The matrix unit adds D/16 partial sums
    # of 16 exact products, each rounded to fp32: at most ~(D/16 + 16) roundings
    # of 2^-24 relative to the sum of |products|; 2^-18 leaves a 4x margin.
    x64 = xb.double().numpy()
    w64 = w.double().numpy()
    y64 = x64 @ w64.T
    bound = 2.0 ** -18 * (np.abs(x64) @ np.abs(w64).T)
    lo16, hi16 = _round16(y64 - bound, dt), _round16(y64 + bound, dt)
    amb = lo16 != hi16
    B, N, S, D = x64.shape
    nblk = -(-S // R)
    other_scale = 0
    ndiff = 0
    for b in range(B):
        for n in range(N):
            for r in range(nblk):
                sl = slice(r * R, min(S, (r + 1) * R))
                yb = y16[b, n, sl]
                if gsb[b, n, r] == rs[b, n, r]:
                    ev = oracle.code_values(rc[b, n, sl], qtype)
                else:
                    # The GPU's amax must come from an ambiguous element taking
                    # its other 16-bit rounding. With that scale, every element
                    # the GPU rounded as the oracle did must get the oracle's
                    # code for it.
                    ab = amb[b, n, sl]
                    alts = np.where(yb[ab] == lo16[b, n, sl][ab], hi16[b, n, sl][ab],
                                    lo16[b, n, sl][ab])
                    # the GPU amax is some element's |value| (the oracle's, or
                    # an ambiguous element's alternative), at least the largest
                    # non-ambiguous |value|
                    cands = np.concatenate([np.abs(yb).ravel(), np.abs(alts)])
                    cands = cands[cands >= np.abs(yb[~ab]).max(initial=0.0)]
                    assert any(_scale_of(a, qtype, sdt) == gsb[b, n, r] for a in cands), \
                        (b, n, r, gsb[b, n, r], rs[b, n, r])
                    other_scale += 1
                    ev = oracle.code_values(
                        oracle.quantize_with_scale(yb.astype(np.float32), float(gsb[b, n, r]),
                                                   qtype), qtype)
                gv = oracle.code_values(gcb[b, n, sl], qtype)
                diff = gv != ev
                if diff.any():
                    assert amb[b, n, sl][diff].all(), \
                        f"code differs where the rounding is not ambiguous at block {(b, n, r)}"
                    # quantization is monotone: the GPU's code lies between the
                    # codes of the two ends of the element's rounding interval
                    sg = float(gsb[b, n, r])
                    clo = oracle.code_values(oracle.quantize_with_scale(
                        lo16[b, n, sl][diff].astype(np.float32), sg, qtype), qtype)
                    chi = oracle.code_values(oracle.quantize_with_scale(
                        hi16[b, n, sl][diff].astype(np.float32), sg, qtype), qtype)
                    g = gv[diff]
                    assert ((np.minimum(clo, chi) <= g) & (g <= np.maximum(clo, chi))).all(), \
                        ((b, n, r), g[:5], clo[:5], chi[:5])
                    ndiff += int(diff.sum())
    nblocks = B * N * nblk
    say(f"  ambiguous elements {int(amb.sum())} of {amb.size}; code differences {ndiff}; "
        f"blocks with the other scale {other_scale} of {nblocks} (all blocks compared)")
    assert other_scale <= max(1, nblocks // 100)


@pytest.mark.parametrize("case", [
    # B, N, S, D, dtype, R, qtype, scale dtype, layout
    (1, 2, 300, 128, "bf16", 128, "fp8", "f32", "bnsd"),
    (2, 1, 200, 64, "f16", 64, "int8", "f16", "bsnd"),
    (1, 2, 600, 128, "bf16", 256, "fp8", "f32", "bsnd"),
    (1, 3, 70, 128, "f16", 32, "int8", "f32", "bnsd"),
    # 8-wavefront workgroups (R > 128) with empty tiles and ragged tails
    (1, 2, 500, 128, "f16", 160, "int8", "f16", "bnsd"),
    (2, 1, 530, 64, "bf16", 224, "fp8", "f32", "bsnd"),
    (1, 1, 513, 128, "f16", 256, "fp8", "f16", "bnsd"),
], ids=lambda c: "_".join(map(str, c)))
def test_rotate_block_quant_small(case):
    B, N, S, D, dt, R, qtype, sdt, layout = case
    x, w = _inputs(B, N, S, D, dt, layout, seed=B * 1000 + S)
    _check(x, w, R, qtype, dt, sdt, layout)


@pytest.mark.parametrize("R", [128, 256])
def test_rotate_block_quant_full_size_sampled(R):
    """The FP8 workload's Q/K shape (2 x 24 heads x 4608 x 128, bf16): the
    kernel runs on the whole tensor; two heads are checked."""
    x, w = _inputs(2, 24, 4608, 128, "bf16", "bnsd", seed=R)
    _check(x, w, R, "fp8", "bf16", "f32", "bnsd", heads=[0, 23])


def test_rotate_block_quant_empty():
    w = torch.eye(128, dtype=torch.bfloat16, device="cuda")
    x = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    c, s = qfa.rotate_block_quant(x, w, 128, "fp8")
    assert c.shape == (1, 2, 0, 128) and s.shape == (1, 2, 0)


@pytest.mark.parametrize("R", [128, 256])
def test_rotate_block_quant_unaligned_codes(R):
    """Codes 8 bytes past a 16-byte boundary take the 4-byte store path; its
    bytes must equal those of the 16-byte path (checked against the oracle
    by the other tests)."""
    x, w = _inputs(1, 2, 400, 128, "bf16", "bnsd", seed=5 + R)
    x, w = x.cuda(), w.cuda()
    ref_c, ref_s = qfa.rotate_block_quant(x, w, R, "fp8")
    buf = torch.zeros(ref_c.numel() + 16, dtype=torch.uint8, device="cuda")
    codes = buf[8:8 + ref_c.numel()].view(ref_c.dtype).view(ref_c.shape)
    assert codes.data_ptr() % 16 == 8
    c, s = qfa.rotate_block_quant(x, w, R, "fp8", codes=codes)
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.uint8), ref_c.view(torch.uint8))
    assert torch.equal(s, ref_s)
    assert int(buf[:8].sum()) == 0 and int(buf[8 + ref_c.numel():].sum()) == 0
