"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

import block_quantized_flashattention_amd as qfa
import oracle
import qfa_workloads as wl

MAX_ABS = 1e-2
MEAN_ABS = 1e-3

SDT = {"f32": torch.float32, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def codes_np(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def assert_codes_equal(gpu_codes: torch.Tensor, gpu_scales: torch.Tensor, ref_codes, ref_scales,
                       what: str):
    gc, gs = codes_np(gpu_codes), gpu_scales.cpu().numpy()
    if gs.dtype != ref_scales.dtype or not np.array_equal(gs.view(np.uint8), ref_scales.view(np.uint8)):
        bad = np.argwhere(gs != ref_scales)
        raise AssertionError(f"{what}: scales differ at {len(bad)} blocks, first {bad[:3].tolist()}: "
                             f"gpu {gs[tuple(bad[0])] if len(bad) else None} "
                             f"ref {ref_scales[tuple(bad[0])] if len(bad) else None}")
    gcu, rcu = gc.view(np.uint8), np.asarray(ref_codes).view(np.uint8)
    if not np.array_equal(gcu, rcu):
        bad = np.argwhere(gcu != rcu)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} code bytes differ; first at {list(i)}: "
                             f"gpu 0x{int(gcu[i]):02x} ref 0x{int(rcu[i]):02x}")


def assert_close(out_gpu: torch.Tensor, ref: np.ndarray, what: str,
                 max_abs: float = MAX_ABS, mean_abs: float = MEAN_ABS):
    o = out_gpu.double().cpu().numpy() if isinstance(out_gpu, torch.Tensor) else out_gpu
    err = np.abs(o - ref)
    mx, mn = float(err.max()), float(err.mean())
    say(f"  {what}: max_abs={mx:.3e} mean_abs={mn:.3e} (n={err.size})")
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max_abs {mx:.3e} mean_abs {mn:.3e}"


def quantize_both(x: torch.Tensor, block_rows: int, qtype: str, sdt: str, layout: str, what: str,
                  heads=None):
    """GPU codes of x (already on the GPU) checked byte for byte against the
    oracle (all heads, or the listed ones). Returns the GPU codes and scales."""
    c, s = qfa.block_quant(x, block_rows, qtype, SDT[sdt], layout)
    torch.cuda.synchronize()
    if heads is None:
        rc, rs = oracle.block_quant(x.cpu(), block_rows, qtype, sdt, layout)
        assert_codes_equal(c, s, rc, rs, what)
    else:
        hsel = torch.tensor(list(heads), device=x.device)
        if layout == "bnsd":
            rc, rs = oracle.block_quant(x[:, hsel].cpu(), block_rows, qtype, sdt, layout)
            assert_codes_equal(c[:, hsel], s[:, hsel], rc, rs, what)
        else:
            rc, rs = oracle.block_quant(x[:, :, hsel].cpu(), block_rows, qtype, sdt, layout)
            assert_codes_equal(c[:, :, hsel], s[:, hsel], rc, rs, what)
    return c, s


def dequant_heads(codes: torch.Tensor, scales: torch.Tensor, block_rows: int, qtype: str,
                  layout: str, heads) -> np.ndarray:
    """Oracle dequantization of the listed heads (BNSD float64 [B, len(heads), S, D])."""
    hsel = torch.tensor(list(heads), device=codes.device)
    if layout == "bnsd":
        c = codes[:, hsel].cpu().numpy()
    else:
        c = codes[:, :, hsel].cpu().numpy()
    s = scales[:, hsel].cpu().numpy()
    return oracle.dequantize(c, s, block_rows, qtype, layout)


def prefill_parity(w: wl.PrefillWorkload, layout: str = "bnsd", heads=None, rows=None,
                   out_dtype=None, gen_device="cpu"):
    """Quantize Q/K/V on the GPU (codes checked against the oracle), run the
    attention forward and compare sampled (or all) output rows with the
    oracle's float64 attention on the dequantized codes."""
    say(f"prefill case {w.name} layout={layout} B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} D={w.D} "
        f"q={w.q_qtype} k={w.k_qtype} v={w.v_qtype} causal={w.causal}")
    q, k, v = wl.make_prefill_inputs(w, device=gen_device, layout=layout)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    group = w.Hq // w.Hkv
    qheads = list(range(w.Hq)) if heads is None else list(heads)
    kvheads = sorted({h // group for h in qheads})
    qc, qs = quantize_both(q, w.q_block, w.q_qtype, w.q_scale_dtype, layout, "Q codes", qheads)
    kc, ks = quantize_both(k, w.kv_block, w.k_qtype, w.kv_scale_dtype, layout, "K codes", kvheads)
    vc, vs = quantize_both(v, w.kv_block, w.v_qtype, w.kv_scale_dtype, layout, "V codes", kvheads)
    odt = wl.torch_dtype(out_dtype or w.out_dtype)
    out = qfa.fwd(qc, qs, kc, ks, vc, vs, q_qtype=w.q_qtype, k_qtype=w.k_qtype, v_qtype=w.v_qtype,
                  q_block=w.q_block, kv_block=w.kv_block, softmax_scale=w.softmax_scale,
                  causal=w.causal, layout=layout, out_dtype=odt)
    torch.cuda.synchronize()
    qh = dequant_heads(qc, qs, w.q_block, w.q_qtype, layout, qheads)
    kh = dequant_heads(kc, ks, w.kv_block, w.k_qtype, layout, kvheads)
    vh = dequant_heads(vc, vs, w.kv_block, w.v_qtype, layout, kvheads)
    kvpos = {h: i for i, h in enumerate(kvheads)}
    outc = out.cpu()
    errs_ref, errs_out = [], []
    for b in range(w.B):
        for hi, h in enumerate(qheads):
            r = np.arange(w.S) if rows is None else np.asarray(rows)
            kvi = kvpos[h // group]
            ref = oracle.attention_rows(qh[:, hi:hi + 1], kh[:, kvi:kvi + 1], vh[:, kvi:kvi + 1],
                                        w.softmax_scale, w.causal, b, 0, r)
            got = outc[b, h, r] if layout == "bnsd" else outc[b, r, h]
            errs_ref.append(ref)
            errs_out.append(got.double().numpy())
    assert_close(np.concatenate(errs_out), np.concatenate(errs_ref), f"{w.name} output")
    return out


def prefill_parity_every_head(w: wl.PrefillWorkload, rows_per_head: int = 3):
    """Every (batch, query head) of a full workload, a few rows each.

    The HIP path quantizes the whole Q, K and V and runs the forward in the
    launch configuration the benchmark times. The oracle quantizes K and V of
    every KV head (the GPU's codes and scales must equal them byte for byte)
    and, per query head, only the Q blocks that hold the sampled rows (blocks
    are independent, so a block-aligned slice quantizes as in the whole
    tensor; checked against the GPU's bytes too). The reference rows are the
    oracle's float64 attention on the oracle's own codes.
    """
    say(f"prefill every head {w.name} B={w.B} Hq={w.Hq} Hkv={w.Hkv} S={w.S} "
        f"{rows_per_head} rows per head")
    q, k, v = wl.make_prefill_inputs(w)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    qc, qs = qfa.block_quant(qg, w.q_block, w.q_qtype, SDT[w.q_scale_dtype])
    kc, ks = qfa.block_quant(kg, w.kv_block, w.k_qtype, SDT[w.kv_scale_dtype])
    vc, vs = qfa.block_quant(vg, w.kv_block, w.v_qtype, SDT[w.kv_scale_dtype])
    out = qfa.fwd(qc, qs, kc, ks, vc, vs, q_qtype=w.q_qtype, k_qtype=w.k_qtype, v_qtype=w.v_qtype,
                  q_block=w.q_block, kv_block=w.kv_block, softmax_scale=w.softmax_scale,
                  causal=w.causal, out_dtype=wl.torch_dtype(w.out_dtype))
    torch.cuda.synchronize()
    del qg, kg, vg
    rk, rks = oracle.block_quant(k, w.kv_block, w.k_qtype, w.kv_scale_dtype)
    rv, rvs = oracle.block_quant(v, w.kv_block, w.v_qtype, w.kv_scale_dtype)
    assert_codes_equal(kc, ks, rk, rks, "K codes, every head")
    assert_codes_equal(vc, vs, rv, rvs, "V codes, every head")
    kh = oracle.dequantize(rk, rks, w.kv_block, w.k_qtype)
    vh = oracle.dequantize(rv, rvs, w.kv_block, w.v_qtype)
    del rk, rv
    qcn, qsn, outc = qc.cpu().numpy(), qs.cpu().numpy(), out.cpu()
    group = w.Hq // w.Hkv
    S, R = w.S, w.q_block
    got, ref = [], []
    for b in range(w.B):
        for h in range(w.Hq):
            rng = np.random.default_rng(w.seed * 100003 + b * 1009 + h)
            rows = set(rng.integers(0, S, rows_per_head).tolist())
            rows.add(S - 1 if h % 2 else int(rng.integers(0, min(S, 2 * R))))
            rows = np.array(sorted(rows))
            qhat = np.zeros((1, 1, S, w.D))
            for blk in sorted({int(r) // R for r in rows}):
                sl = slice(blk * R, min(S, (blk + 1) * R))
                bc, bs = oracle.block_quant(q[b:b + 1, h:h + 1, sl], R, w.q_qtype,
                                            w.q_scale_dtype)
                assert_codes_equal(torch.from_numpy(np.ascontiguousarray(qcn[b:b + 1, h:h + 1, sl])),
                                   torch.from_numpy(qsn[b:b + 1, h:h + 1, blk:blk + 1]), bc, bs,
                                   f"Q block {blk} of head {h}")
                qhat[0, 0, sl] = oracle.dequantize(bc, bs, R, w.q_qtype)[0, 0]
            kvh = h // group
            ref.append(oracle.attention_rows(qhat, kh[b:b + 1, kvh:kvh + 1], vh[b:b + 1, kvh:kvh + 1],
                                             w.softmax_scale, w.causal, 0, 0, rows))
            got.append(outc[b, h, rows].double().numpy())
    assert_close(np.concatenate(got), np.concatenate(ref), f"{w.name} every head")
