"""Benchmark: block-quantized FlashAttention on one MI355X.

One step = quantize Q, K and V (one qfa_block_quant_multi call) and run the
attention forward (qfa_fwd) on the largest single-GPU workload,
``gqa64x8_int4kv_causal_s16384``: B=1, 64 query heads over 8 KV heads, S=16384,
D=128, fp16 inputs (1% of K elements x10), Q in INT8 per 128-row block, K and V
in packed INT4 with one fp16 scale per token, causal, fp16 output; inputs
resident in HBM. ``value`` is the attention's algorithmic ops (unmasked pairs,
multiply and add counted) per second of the whole step. The dominant kernel
(the forward) is also timed alone with HIP events and reported against the
dense INT8 MFMA peak (``roofline``).

Sub-objects: the same step on the INT8 causal (``int8_causal_h32_s4096``) and
FP8 rotated (``fp8_rot_b2_h24_s4608``) workloads, the tiny INT8 workload's
latency, the quantizer and the fused rotate+quantize (after a 512 MiB cache
flush and cache-resident), the INT8 and INT4 KV-cache decode (after a flush),
the KV append, and the mixed INT8 Q/K + INT4 V forward. ``attainable`` holds what
plain library kernels reach on the same box (fp16 and INT8
GEMMs, a 512 MiB copy), and every MFMA roofline carries ``frac_attainable``
against the INT8 GEMM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # dense INT8 MFMA, MI355X
PEAK_FP8_TFLOPS = 5000.0     # dense FP8 MFMA
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20      # larger than the 256 MiB last-level cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def settle(torch, fn, seconds=0.1):
    """Run ``fn`` untimed for about ``seconds`` of GPU time before the warmup
    steps: the GPU's clocks ramp up over the first tens of milliseconds of
    sustained work."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def _sdt(torch, name):
    return {"f32": torch.float32, "f16": torch.float16}[name]


def prepare_step(torch, qfa, wl, w):
    """Inputs of workload ``w`` on the GPU and the two marshalled calls of one
    step: quantize Q/K/V (one qfa_block_quant_multi) and the forward."""
    q, k, v = wl.make_prefill_inputs(w, device="cuda")
    jobs = [dict(x=q, block_rows=w.q_block, qtype=w.q_qtype, scale_dtype=_sdt(torch, w.q_scale_dtype)),
            dict(x=k, block_rows=w.kv_block, qtype=w.k_qtype,
                 scale_dtype=_sdt(torch, w.kv_scale_dtype)),
            dict(x=v, block_rows=w.kv_block, qtype=w.v_qtype,
                 scale_dtype=_sdt(torch, w.kv_scale_dtype))]
    quant, outs = qfa.prepare_block_quant_multi(jobs)
    quant()
    (qc, qs), (kc, ks), (vc, vs) = outs
    out = torch.empty(q.shape, dtype=wl.torch_dtype(w.out_dtype), device="cuda")
    attn, _ = qfa.prepare_fwd(qc, qs, kc, ks, vc, vs, q_qtype=w.q_qtype, k_qtype=w.k_qtype,
                              v_qtype=w.v_qtype, q_block=w.q_block, kv_block=w.kv_block,
                              softmax_scale=w.softmax_scale, causal=w.causal, out=out)
    nbytes = sum(t.numel() * t.element_size() for t in (q, k, v, qc, kc, vc, qs, ks, vs))
    keep = (q, k, v, qc, qs, kc, ks, vc, vs, out)
    return quant, attn, nbytes, keep


def time_step(torch, quant, attn, steps, warmup):
    """Exactly ``steps`` steps between two synchronizations (wall clock), with
    HIP events around each call on the stream they run on."""
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        quant()
        if ev is not None:
            ev[1].record()
        attn()
        if ev is not None:
            ev[2].record()

    settle(torch, step)
    for _ in range(warmup):
        step()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    quant_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    fwd_ms = sum(b.elapsed_time(c) for _, b, c in evs) / steps
    return wall * 1e3 / steps, fwd_ms, quant_ms


def time_calls(torch, fn, n, flush=None):
    """Median time of ``n`` single calls (HIP events); with ``flush`` a buffer
    larger than the last-level cache is read (not written, so no write-back
    lands in the timed call) before each one."""
    times = []
    for _ in range(n):
        if flush is not None:
            flush.max()
        torch.cuda.synchronize()
        a, b = _events(torch)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    return sorted(times)[len(times) // 2]


def mfma_roofline(ops, ms, peak, traffic=None, kernel=None):
    achieved = ops / (ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if kernel:
        r["kernel"] = kernel
        r["kernel_ms"] = round(ms, 4)
    return r


def hbm_roofline(nbytes, ms, traffic=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}


def profiled_traffic(profile, source):
    """HBM bytes per dispatch from a committed rocprofv3 summary, or None when
    the kernel source has changed since the counters were taken."""
    import hashlib
    import re
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
        src = open(os.path.join(ROOT, source), "rb").read()
    except OSError:
        return None
    m = re.search(r"sha256 prefix `([0-9a-f]+)`", text)
    t = re.search(r"traffic_bytes_per_dispatch: (\d+)", text)
    if not m or not t or hashlib.sha256(src).hexdigest()[:len(m.group(1))] != m.group(1):
        return None
    return int(t.group(1))


PREFILL_SRC = "block_quantized_flashattention_amd/csrc/prefill.hip"
QUANT_SRC = "block_quantized_flashattention_amd/csrc/quant.hip"
DECODE_SRC = "block_quantized_flashattention_amd/csrc/decode.hip"


def bench_prefill_step(torch, qfa, wl, w, steps, warmup, peak, flush):
    """One workload's step (quantize Q/K/V + forward): step wall time, forward
    and quantizer event times, the quantizer alone after a cache flush."""
    quant, attn, qbytes, keep = prepare_step(torch, qfa, wl, w)
    ms_step, fwd_ms, quant_ms = time_step(torch, quant, attn, steps, warmup)
    quant_flushed = time_calls(torch, quant, 10, flush)
    ops = w.attention_ops()
    del keep
    torch.cuda.empty_cache()
    prof = f"fwd_{w.name}.md"
    return {
        "workload": w.name,
        "ms_per_step": round(ms_step, 4),
        "value": round(ops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TOPS",
        "fwd_ms": round(fwd_ms, 4),
        "roofline": mfma_roofline(ops, fwd_ms, peak, profiled_traffic(prof, PREFILL_SRC)),
        "quantize": {"ms": round(quant_ms, 4), "ms_flushed": round(quant_flushed, 4),
                     "bytes": qbytes,
                     "roofline": hbm_roofline(qbytes, quant_flushed),
                     "roofline_cached": hbm_roofline(qbytes, quant_ms)},
    }


def bench_tiny_latency(torch, qfa, wl, steps, warmup):
    """The tiny INT8 workload (one workgroup): per-call latency of the step and
    of the forward alone."""
    w = wl.TINY
    quant, attn, _, keep = prepare_step(torch, qfa, wl, w)

    def step():
        quant()
        attn()
    for _ in range(warmup + 5):
        step()
    n = max(steps, 20)
    step_ms = time_calls(torch, step, n)
    fwd_ms = time_calls(torch, attn, n)
    del keep
    return {"workload": w.name, "step_latency_us": round(step_ms * 1e3, 2),
            "fwd_latency_us": round(fwd_ms * 1e3, 2),
            "note": "one workgroup: launch-bound, correctness and latency only"}


def bench_forward(torch, qfa, wl, w, steps, warmup):
    """Forward alone on workload ``w`` (codes quantized once): average kernel
    time from per-call HIP events over back-to-back calls."""
    quant, attn, _, keep = prepare_step(torch, qfa, wl, w)
    settle(torch, attn)
    for _ in range(warmup):
        attn()
    torch.cuda.synchronize()
    evs = [_events(torch) for _ in range(steps)]
    for a, b in evs:
        a.record()
        attn()
        b.record()
    torch.cuda.synchronize()
    del keep
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def bench_fwd_lowp(torch, qfa, wl, steps, warmup):
    """The FP8 workload's forward with P.V on the fp8 matrix unit (qfa_fwd_lowp:
    fp8 pass, then the fp16 pass over the work items the accuracy gate
    flagged) against qfa_fwd on the same codes: average kernel-pair time over
    back-to-back calls, and the fraction of work items that fell back."""
    w = wl.FP8_ROT
    q, k, v = wl.make_prefill_inputs(w, device="cuda")
    qc, qs = qfa.block_quant(q, w.q_block, "fp8")
    kc, ks = qfa.block_quant(k, w.kv_block, "fp8")
    vc, vs = qfa.block_quant(v, w.kv_block, "fp8")
    del q, k, v
    kw = dict(q_qtype="fp8", k_qtype="fp8", v_qtype="fp8", q_block=w.q_block,
              kv_block=w.kv_block, softmax_scale=w.softmax_scale, causal=w.causal,
              out_dtype=wl.torch_dtype(w.out_dtype))
    f16, _ = qfa.prepare_fwd(qc, qs, kc, ks, vc, vs, **kw)
    flp, _, ws = qfa.prepare_fwd_lowp(qc, qs, kc, ks, vc, vs, **kw)

    def avg(f):
        settle(torch, f)
        for _ in range(warmup):
            f()
        torch.cuda.synchronize()
        evs = [_events(torch) for _ in range(steps)]
        for a, b in evs:
            a.record()
            f()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps
    t16, tlp = avg(f16), avg(flp)
    nitems = ws.numel() // 8
    flagged = float(ws.cpu()[:8 * nitems].view(nitems, 8).any(dim=1).float().mean())
    ops = w.attention_ops()
    return {"workload": w.name, "fwd_ms": round(t16, 4), "fwd_lowp_ms": round(tlp, 4),
            "speedup": round(t16 / tlp, 3), "fallback_items": round(flagged, 4),
            "roofline": mfma_roofline(ops, tlp, PEAK_FP8_TFLOPS),
            "note": "one launch: fp8 P.V, and a workgroup whose gate flags a row recomputes "
                    "its work item with the fp16 product before exiting"}


def bench_rotate_quant(torch, qfa, wl, steps, warmup, flush):
    """Fused rotation + FP8 block quantization of Q (128-row blocks) and K
    (256-row blocks) of the FP8 workload's shape: the pair's time, cache
    resident (average of back-to-back pairs) and after a flush (median), and
    the algorithmic bytes (bf16 read once, e4m3 codes and fp32 scales written
    once)."""
    w = wl.FP8_ROT
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    q = torch.randn(w.B, w.Hq, w.S, w.D, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn(w.B, w.Hkv, w.S, w.D, generator=gen, device="cuda").to(torch.bfloat16)
    wt = wl.random_orthogonal(w.D, gen).t().contiguous().to(torch.bfloat16)
    lq, _, _ = qfa.prepare_rotate_block_quant(q, wt, w.q_block, "fp8")
    lk, _, _ = qfa.prepare_rotate_block_quant(k, wt, w.kv_block, "fp8")

    def pair():
        lq()
        lk()
    settle(torch, pair)
    for _ in range(warmup):
        pair()
    torch.cuda.synchronize()
    evs = [_events(torch) for _ in range(steps)]
    for a, b in evs:
        a.record()
        pair()
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    ms_flushed = time_calls(torch, pair, 10, flush)
    nq, nk = q.numel(), k.numel()
    nbytes = 3 * (nq + nk) + 4 * (w.B * w.Hq * -(-w.S // w.q_block) + w.B * w.Hkv * -(-w.S // w.kv_block))
    return {"workload": w.name, "ms": round(ms, 4), "ms_flushed": round(ms_flushed, 4),
            "bytes": nbytes, "roofline": hbm_roofline(nbytes, ms_flushed),
            "roofline_cached": hbm_roofline(nbytes, ms)}


def bench_kv_append(torch, qfa, wl, steps, warmup):
    """One decode step's cache update on the decode workload's shape: the new K
    and V rows of every sequence quantized into INT8 caches (fp16 scales per
    256 rows), at positions inside existing blocks: both rows in one launch, and
    as two launches. Average times from per-call HIP events."""
    w = wl.DECODE
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    kc = torch.randint(-127, 128, (w.B, w.Hkv, w.S_max, w.D), generator=gen, device="cuda",
                       dtype=torch.int8)
    vc = kc.clone()
    nblk = -(-w.S_max // w.kv_block)
    ks = torch.full((w.B, w.Hkv, nblk), 0.05, dtype=torch.float16, device="cuda")
    vs = ks.clone()
    pos = torch.randint(w.len_lo, w.len_hi, (w.B,), generator=gen, device="cuda",
                        dtype=torch.int32)
    xk = torch.randn(w.B, w.Hkv, w.D, generator=gen, device="cuda").to(torch.float16)
    xv = torch.randn(w.B, w.Hkv, w.D, generator=gen, device="cuda").to(torch.float16)
    ak = qfa.kv_append(xk, pos, kc, ks, w.kv_block, "int8", prepare=True)
    av = qfa.kv_append(xv, pos, vc, vs, w.kv_block, "int8", prepare=True)
    akv = qfa.kv_append_kv(xk, xv, pos, kc, ks, vc, vs, w.kv_block, "int8", prepare=True)

    def pair():
        ak()
        av()

    def avg(fn):
        for _ in range(warmup + 5):
            fn()
        torch.cuda.synchronize()
        evs = [_events(torch) for _ in range(steps)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps
    two = avg(pair)
    one = avg(akv)
    return {"workload": w.name, "ms": round(one, 4), "ms_two_calls": round(two, 4),
            "note": "latency of one decode step's K and V row appends: one qfa_kv_append_kv "
                    "launch (ms), two qfa_kv_append launches (ms_two_calls); no roofline: a few "
                    "KB per call"}


def bench_decode(torch, qfa, wl, w, steps, warmup, flush, prof):
    q, k, v, lens = wl.make_decode_inputs(w, device="cuda")
    sdt = torch.float16
    kc, ks = qfa.block_quant(k, w.kv_block, w.kv_qtype, sdt)
    vc, vs = qfa.block_quant(v, w.kv_block, w.kv_qtype, sdt)
    del k, v
    out = torch.empty_like(q)
    ws = torch.empty(qfa.decode_workspace_bytes(w.B, w.Hq, w.S_max, w.D), dtype=torch.uint8,
                     device="cuda")
    call, _ = qfa.prepare_decode(q, kc, vc, ks, vs, lens, kv_qtype=w.kv_qtype,
                                 kv_block=w.kv_block, softmax_scale=w.softmax_scale, out=out,
                                 workspace=ws)
    for _ in range(warmup):
        call()
    ms = time_calls(torch, call, max(steps, 10), flush)
    nbytes = wl.decode_kv_bytes(w, lens.cpu().tolist())
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4),
            "bytes": nbytes,
            "roofline": hbm_roofline(nbytes, ms, profiled_traffic(prof, DECODE_SRC))}


def measure_attainable(torch, flush):
    """What plain library kernels reach on this machine, on the same stream and
    clocks as the timed kernels, so that the MFMA roofline fractions can be
    read against a measured ceiling as well as the nominal peak: a 8192^3
    fp16 GEMM, where torch provides it a 8192^3 INT8 GEMM (torch._int_mm),
    and a 512 MiB device copy (read + write bytes; torch's copy is no
    read-only ceiling, so HBM fractions stay against the nominal 8 TB/s)."""
    dst = torch.empty_like(flush)
    copy_ms = time_calls(torch, lambda: dst.copy_(flush), 7)
    del dst
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.float16)
    b = torch.randn(n, n, device="cuda", dtype=torch.float16)
    gemm_ms = time_calls(torch, lambda: torch.matmul(a, b), 7)
    r = {"hbm_copy_gbs": round(2 * FLUSH_BYTES / (copy_ms * 1e-3) / 1e9, 1),
         "fp16_gemm_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
         "int8_gemm_tops": None,
         "note": "copy: torch copy_ of 512 MiB, read + write bytes; gemm: torch.matmul / "
                 "torch._int_mm, 8192^3; medians of 7"}
    del a, b
    try:
        a8 = torch.randint(-127, 128, (n, n), device="cuda", dtype=torch.int8)
        b8 = torch.randint(-127, 128, (n, n), device="cuda", dtype=torch.int8)
        i8_ms = time_calls(torch, lambda: torch._int_mm(a8, b8), 7)
        r["int8_gemm_tops"] = round(2 * n ** 3 / (i8_ms * 1e-3) / 1e12, 1)
        del a8, b8
    except Exception as e:  # not every torch build has an INT8 GEMM on this GPU
        log(f"int8 gemm probe unavailable: {type(e).__name__}")
    torch.cuda.empty_cache()
    return r


def add_attainable(rec, att):
    """frac_attainable beside every MFMA roofline's frac: the achieved rate
    over the INT8 GEMM's (the dense INT8 and FP8 peaks are equal)."""
    def visit(d):
        for k, v in d.items():
            if isinstance(v, dict):
                if k.startswith("roofline"):
                    if v.get("bound") == "mfma":
                        ref = att["int8_gemm_tops"]
                        v["frac_attainable"] = round(v["achieved"] / ref, 4) if ref else None
                else:
                    visit(v)
    visit(rec)


def cpu_baseline(wl, target_s=10.0):
    """The oracle (quantize + float64 causal attention) on blocks of 512 query
    rows of the headline workload, cycling over heads and row blocks until
    about ``target_s`` seconds have passed; ops/s in TOPS (the algorithmic ops
    of exactly the rows computed)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    w = wl.GQA_INT4
    q, k, v = wl.make_prefill_inputs(w)
    group = w.Hq // w.Hkv
    rows_per, done, ops, kv_cache = 512, 0, 0, {}
    t0 = time.perf_counter()
    while True:
        h = (done * 7) % w.Hq                      # spread over heads and KV heads
        r0 = ((done * 13) % (w.S // rows_per)) * rows_per
        kvh = h // group
        if kvh not in kv_cache:
            kc, ks = oracle.block_quant(k[:, kvh:kvh + 1], w.kv_block, w.k_qtype, w.kv_scale_dtype)
            vc, vs = oracle.block_quant(v[:, kvh:kvh + 1], w.kv_block, w.v_qtype, w.kv_scale_dtype)
            kv_cache[kvh] = (oracle.dequantize(kc, ks, w.kv_block, w.k_qtype),
                             oracle.dequantize(vc, vs, w.kv_block, w.v_qtype))
        kh, vh = kv_cache[kvh]
        qb = q[:, h:h + 1, r0:r0 + rows_per]
        qc, qs = oracle.block_quant(qb, w.q_block, w.q_qtype, w.q_scale_dtype)
        qh = oracle.dequantize(qc, qs, w.q_block, w.q_qtype)
        rows = np.arange(r0, r0 + rows_per)
        qfull = np.zeros((1, 1, w.S, w.D))
        qfull[0, 0, r0:r0 + rows_per] = qh[0, 0]
        oracle.attention_rows(qfull, kh, vh, w.softmax_scale, True, 0, 0, rows)
        ops += int(sum(4 * w.D * (i + 1) for i in rows))
        done += 1
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} blocks of {rows_per} query rows of {w.name} (spread over heads): "
                      f"quantize Q block + K/V head (INT4 per token) and float64 causal attention "
                      f"of those rows, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline step only (for profiler runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels shard by head or batch with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_quantized_flashattention_amd as qfa
    import qfa_workloads as wl

    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
    w = wl.GQA_INT4
    log(f"headline step: {w.name}, warmup {args.warmup}, steps {args.steps}")
    head = bench_prefill_step(torch, qfa, wl, w, args.steps, args.warmup, PEAK_INT8_TOPS, flush)
    log(f"{w.name}: step {head['ms_per_step']:.3f} ms, forward {head['fwd_ms']:.3f} ms "
        f"({head['roofline']['achieved']:.0f} TOPS), quantize {head['quantize']['ms']:.3f} ms "
        f"({head['quantize']['ms_flushed']:.3f} ms flushed)")
    rec = {
        "metric": "quantized FA prefill TOPS + decode KV GB/s, % of MI355X MFMA/HBM peak",
        "value": head["value"],
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                   "causal": w.causal, "q_qtype": w.q_qtype, "kv_qtype": w.k_qtype,
                   "q_block": w.q_block, "kv_block": w.kv_block,
                   "step": "block_quant_multi(Q,K,V) + fwd"},
        "roofline": dict(head["roofline"], kernel="fwd_kernel<128,int4kv,causal,per-token>",
                         kernel_ms=head["fwd_ms"]),
        "quantize": head["quantize"],
    }
    if not args.only_headline:
        for key, pw, peak in (("int8_causal", wl.INT8_CAUSAL, PEAK_INT8_TOPS),
                              ("fp8_rot", wl.FP8_ROT, PEAK_FP8_TFLOPS)):
            log(f"step: {pw.name}")
            r = bench_prefill_step(torch, qfa, wl, pw, args.steps, args.warmup, peak, flush)
            log(f"{pw.name}: step {r['ms_per_step']:.3f} ms, forward {r['fwd_ms']:.3f} ms "
                f"({r['roofline']['achieved']:.0f} TOPS)")
            rec[key] = r
        rec["tiny"] = bench_tiny_latency(torch, qfa, wl, args.steps, args.warmup)
        log(f"tiny: step {rec['tiny']['step_latency_us']} us, forward {rec['tiny']['fwd_latency_us']} us")
        mw = wl.INT8QK_INT4V
        mms = bench_forward(torch, qfa, wl, mw, args.steps, args.warmup)
        rec["fwd_int8qk_int4v"] = {"workload": mw.name, "fwd_ms": round(mms, 4),
                                   "roofline": mfma_roofline(mw.attention_ops(), mms, PEAK_INT8_TOPS)}
        log(f"forward {mw.name}: {mms:.3f} ms")
        rec["fwd_lowp_pv"] = bench_fwd_lowp(torch, qfa, wl, args.steps, args.warmup)
        log(f"fp8 P.V forward: {rec['fwd_lowp_pv']['fwd_lowp_ms']:.4f} ms against "
            f"{rec['fwd_lowp_pv']['fwd_ms']:.4f} ms, fallback items "
            f"{rec['fwd_lowp_pv']['fallback_items']:.2%}")
        rec["rotate_quantize"] = bench_rotate_quant(torch, qfa, wl, args.steps, args.warmup, flush)
        log(f"rotate+quantize: {rec['rotate_quantize']['ms']:.4f} ms cached, "
            f"{rec['rotate_quantize']['ms_flushed']:.4f} ms flushed")
        rec["kv_append"] = bench_kv_append(torch, qfa, wl, args.steps, args.warmup)
        if not args.no_decode:
            for key, dwl, prof in (("decode", wl.DECODE, "decode_int8_kv_b32_h32.md"),
                                   ("decode_int4", wl.DECODE_INT4, "decode_int4_kv_b32_h32.md"),
                                   ("decode_gqa4", wl.DECODE_GQA4, "decode_int8_kv_b32_h32_gqa4.md"),
                                   ("decode_gqa16_int4", wl.DECODE_GQA16_INT4,
                                    "decode_int4_kv_b32_h32_gqa16.md")):
                rec[key] = bench_decode(torch, qfa, wl, dwl, args.steps, args.warmup, flush, prof)
                log(f"{key} {rec[key]['ms']:.3f} ms, {rec[key]['value']:.0f} GB/s")
    att = measure_attainable(torch, flush)
    log(f"attainable: {att}")
    rec["attainable"] = att
    add_attainable(rec, att)
    if args.copy_probe:
        # A plain elementwise copy of known size: reads 1 GiB (fp32), writes 512 MiB (fp16).
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty(1 << 28, dtype=torch.float16, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: 3 fp32->fp16 copies, 1 GiB read + 512 MiB written each")
        del src, dst
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on the host")
        rec["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
