"""Benchmark: block-quantized FlashAttention on one MI355X.

One step = quantize Q, K and V (one qfa_block_quant_multi call) and run the INT8 causal
attention forward (qfa_fwd) on the LLaMA-2-7B head shape workload
``int8_causal_h32_s4096`` (B=1, H=32, S=4096, D=128, fp16 inputs with four
outlier K channels), inputs resident in HBM. ``value`` is the attention's
algorithmic ops (unmasked pairs, multiply and add counted) per second of the
whole step. The dominant kernel (the forward) is also timed alone with HIP
events and reported against the dense INT8 MFMA peak; the decode kernel on the
``int8_kv_decode_b32_h32`` workload is reported in GB/s against HBM peak.

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
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def settle(torch, fn, seconds=0.1):
    """Run ``fn`` untimed for about ``seconds`` of GPU time before the warmup
    steps: the GPU's clocks ramp up over the first tens of milliseconds of
    sustained work (the first ~25 ms of forwards run up to ~10% slower)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def bench_prefill(torch, qfa, wl, steps, warmup):
    w = wl.INT8_CAUSAL
    q, k, v = wl.make_prefill_inputs(w, device="cuda")
    sdt = torch.float32
    qc, qs = qfa.block_quant(q, w.q_block, w.q_qtype, sdt)
    kc, ks = qfa.block_quant(k, w.kv_block, w.k_qtype, sdt)
    vc, vs = qfa.block_quant(v, w.kv_block, w.v_qtype, sdt)
    out = torch.empty_like(q)

    jobs = [dict(x=q, block_rows=w.q_block, qtype=w.q_qtype, scale_dtype=sdt, codes=qc, scales=qs),
            dict(x=k, block_rows=w.kv_block, qtype=w.k_qtype, scale_dtype=sdt, codes=kc, scales=ks),
            dict(x=v, block_rows=w.kv_block, qtype=w.v_qtype, scale_dtype=sdt, codes=vc, scales=vs)]

    # Arguments are marshalled once: each step is then two ctypes calls, so the
    # host enqueues faster than the GPU runs and the events time the kernels,
    # not host-side gaps between them.
    quant, _ = qfa.prepare_block_quant_multi(jobs)
    attn, _ = qfa.prepare_fwd(qc, qs, kc, ks, vc, vs, q_qtype=w.q_qtype, k_qtype=w.k_qtype,
                              v_qtype=w.v_qtype, q_block=w.q_block, kv_block=w.kv_block,
                              softmax_scale=w.softmax_scale, causal=w.causal, out=out)

    def step(ev=None):
        if ev is not None:
            ev[2].record()
        quant()
        if ev is not None:
            ev[0].record()
        attn()
        if ev is not None:
            ev[1].record()

    settle(torch, step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [_events(torch) + (torch.cuda.Event(enable_timing=True),) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in evs) / steps
    quant_ms = sum(c.elapsed_time(a) for a, b, c in evs) / steps
    ops = w.attention_ops()
    return w, wall, fwd_ms, quant_ms, ops


def bench_forward(torch, qfa, wl, w, steps, warmup):
    """Forward alone on workload ``w`` (codes quantized once): average kernel
    time from per-call HIP events over ``steps`` back-to-back calls."""
    q, k, v = wl.make_prefill_inputs(w, device="cuda")
    sdt = torch.float32
    qc, qs = qfa.block_quant(q, w.q_block, w.q_qtype, sdt)
    kc, ks = qfa.block_quant(k, w.kv_block, w.k_qtype, sdt)
    vc, vs = qfa.block_quant(v, w.kv_block, w.v_qtype, sdt)
    out = torch.empty_like(q)
    del q, k, v
    attn, _ = qfa.prepare_fwd(qc, qs, kc, ks, vc, vs, q_qtype=w.q_qtype, k_qtype=w.k_qtype,
                              v_qtype=w.v_qtype, q_block=w.q_block, kv_block=w.kv_block,
                              softmax_scale=w.softmax_scale, causal=w.causal, out=out)
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
    return sum(a.elapsed_time(b) for a, b in evs) / steps


def bench_rotate_quant(torch, qfa, wl, steps, warmup):
    """Fused rotation + FP8 block quantization of Q (128-row blocks) and K
    (256-row blocks) of the FP8 workload's shape: average time of the pair
    from per-call HIP events, and the algorithmic bytes (bf16 read once, e4m3
    codes and fp32 scales written once)."""
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
    nq, nk = q.numel(), k.numel()
    nbytes = 3 * (nq + nk) + 4 * (w.B * w.Hq * -(-w.S // w.q_block) + w.B * w.Hkv * -(-w.S // w.kv_block))
    return w, ms, nbytes


def bench_kv_append(torch, qfa, wl, steps, warmup):
    """One decode step's cache update on the decode workload's shape: the new K
    and V rows of every sequence quantized into INT8 caches (fp16 scales per
    256 rows), at positions inside existing blocks. Average time of the pair
    from per-call HIP events."""
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

    def pair():
        ak()
        av()
    for _ in range(warmup + 5):
        pair()
    torch.cuda.synchronize()
    evs = [_events(torch) for _ in range(steps)]
    for a, b in evs:
        a.record()
        pair()
        b.record()
    torch.cuda.synchronize()
    return w, sum(a.elapsed_time(b) for a, b in evs) / steps


def bench_decode(torch, qfa, wl, w, steps, warmup):
    q, k, v, lens = wl.make_decode_inputs(w, device="cuda")
    sdt = torch.float16
    kc, ks = qfa.block_quant(k, w.kv_block, w.kv_qtype, sdt)
    vc, vs = qfa.block_quant(v, w.kv_block, w.kv_qtype, sdt)
    del k, v
    out = torch.empty_like(q)
    ws = torch.empty(qfa.decode_workspace_bytes(w.B, w.Hq, w.S_max, w.D), dtype=torch.uint8,
                     device="cuda")
    # A buffer larger than the 256 MiB last-level cache, read (not written)
    # between timed calls: the cache then holds clean lines of this buffer, so
    # the KV cache comes from HBM and no write-back of the flush itself lands
    # inside the timed region.
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    call, _ = qfa.prepare_decode(q, kc, vc, ks, vs, lens, kv_qtype=w.kv_qtype,
                                 kv_block=w.kv_block, softmax_scale=w.softmax_scale, out=out,
                                 workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        flush.max()
        torch.cuda.synchronize()
        a, b = _events(torch)
        a.record()
        call()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    nbytes = wl.decode_kv_bytes(w, lens.cpu().tolist())
    return w, ms, nbytes


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


def cpu_baseline(wl, target_s=10.0):
    """The oracle (quantize + float64 attention) on whole heads of the bench
    workload, cycling over the heads until about ``target_s`` seconds have
    passed; ops/s in TOPS."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    w = wl.INT8_CAUSAL
    q, k, v = wl.make_prefill_inputs(w)
    done_heads, ops, t0 = 0, 0, time.perf_counter()
    while True:
        h = done_heads % w.Hq
        qc, qs = oracle.block_quant(q[:, h:h + 1], w.q_block, w.q_qtype)
        kc, ks = oracle.block_quant(k[:, h:h + 1], w.kv_block, w.k_qtype)
        vc, vs = oracle.block_quant(v[:, h:h + 1], w.kv_block, w.v_qtype)
        oracle.attention(oracle.dequantize(qc, qs, w.q_block, w.q_qtype),
                         oracle.dequantize(kc, ks, w.kv_block, w.k_qtype),
                         oracle.dequantize(vc, vs, w.kv_block, w.v_qtype),
                         w.softmax_scale, w.causal)
        done_heads += 1
        ops += 2 * w.D * w.S * (w.S + 1)
        if time.perf_counter() - t0 >= target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done_heads} head passes (cycling over the {w.Hq} heads) of {w.name}: "
                      f"quantize Q/K/V + float64 causal attention, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
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

    log(f"prefill: {wl.INT8_CAUSAL.name}, warmup {args.warmup}, steps {args.steps}")
    w, wall, fwd_ms, quant_ms, ops = bench_prefill(torch, qfa, wl, args.steps, args.warmup)
    ms_step = wall * 1e3 / args.steps
    # Algorithmic bytes of the three quantizer calls: fp16 inputs read once,
    # int8 codes and fp32 scales written once.
    nel = w.B * w.Hq * w.S * w.D
    qbytes = 3 * nel * 2 + 3 * nel + 4 * (w.B * w.Hq * (w.S // w.q_block) + 2 * w.B * w.Hkv * (w.S // w.kv_block))
    value = ops / (ms_step * 1e-3) / 1e12
    achieved = ops / (fwd_ms * 1e-3) / 1e12
    log(f"prefill step {ms_step:.3f} ms, forward kernel {fwd_ms:.3f} ms, {achieved:.1f} TOPS, "
        f"quantize Q/K/V {quant_ms:.3f} ms")
    rec = {
        "metric": "quantized FA prefill TOPS + decode KV GB/s, % of MI355X MFMA/HBM peak",
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.Hq, "S": w.S, "D": w.D,
                   "causal": w.causal, "qtype": "int8", "q_block": w.q_block,
                   "kv_block": w.kv_block, "step": "block_quant_multi(Q,K,V) + fwd"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_INT8_TOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": profiled_traffic("fwd_int8_causal_h32_s4096.md",
                                                 "block_quantized_flashattention_amd/csrc/prefill.hip"),
                     "kernel": "fwd_kernel<128,int8,causal>",
                     "kernel_ms": round(fwd_ms, 4)},
        "quantize": {"ms": round(quant_ms, 4), "bytes": qbytes,
                     "roofline": {"bound": "hbm",
                                  "achieved": round(qbytes / (quant_ms * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                  "frac": round(qbytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                  "traffic": profiled_traffic(
                                      "block_quant_qkv_int8_causal_h32_s4096.md",
                                      "block_quantized_flashattention_amd/csrc/quant.hip")}},
    }
    # The same shape with packed INT4 V codes (INT8 Q and K): forward only.
    mw = wl.INT8QK_INT4V
    log(f"forward: {mw.name}")
    mms = bench_forward(torch, qfa, wl, mw, args.steps, args.warmup)
    mtops = mw.attention_ops() / (mms * 1e-3) / 1e12
    log(f"forward {mw.name} {mms:.3f} ms, {mtops:.1f} TOPS")
    rec["fwd_int8qk_int4v"] = {"workload": mw.name, "ms": round(mms, 4),
                               "roofline": {"bound": "mfma", "achieved": round(mtops, 2),
                                            "peak": PEAK_INT8_TOPS, "unit": "TFLOP/s",
                                            "frac": round(mtops / PEAK_INT8_TOPS, 4),
                                            "traffic": None}}
    rw, rms, rbytes = bench_rotate_quant(torch, qfa, wl, args.steps, args.warmup)
    rgbs = rbytes / (rms * 1e-3) / 1e9
    log(f"rotate+quantize Q/K of {rw.name}: {rms:.3f} ms, {rgbs:.0f} GB/s")
    rec["rotate_quantize"] = {"workload": rw.name, "ms": round(rms, 4), "bytes": rbytes,
                              "roofline": {"bound": "hbm", "achieved": round(rgbs, 1),
                                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                           "frac": round(rgbs / PEAK_HBM_GBS, 4),
                                           "traffic": None}}
    aw, ams = bench_kv_append(torch, qfa, wl, args.steps, args.warmup)
    log(f"kv append (K and V of {aw.B} x {aw.Hkv} heads): {ams * 1e3:.1f} us")
    rec["kv_append"] = {"workload": aw.name, "ms": round(ams, 4),
                        "note": "latency of one decode step's K and V row appends (two launches); "
                                "no roofline: a few KB per call"}
    if not args.no_decode:
        # INT8 cache, then the same shape with a packed INT4 cache.
        for key, dwl, prof in (("decode", wl.DECODE, "decode_int8_kv_b32_h32.md"),
                               ("decode_int4", wl.DECODE_INT4, "decode_int4_kv_b32_h32.md")):
            log(f"{key}: {dwl.name}")
            dw, dms, nbytes = bench_decode(torch, qfa, wl, dwl, max(args.steps, 10), args.warmup)
            gbs = nbytes / (dms * 1e-3) / 1e9
            log(f"{key} {dms:.3f} ms, {gbs:.0f} GB/s")
            rec[key] = {"workload": dw.name, "value": round(gbs, 1), "unit": "GB/s",
                        "ms": round(dms, 4), "bytes": nbytes,
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                                     "traffic": profiled_traffic(
                                         prof, "block_quantized_flashattention_amd/csrc/decode.hip")}}
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
