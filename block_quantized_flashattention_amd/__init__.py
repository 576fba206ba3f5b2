"""Block-quantized FlashAttention for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``libqfa.so``; the functions keep the C ABI's names
(``block_quant``, ``fwd``, ``decode``, ``decode_workspace_bytes``). This module
only marshals arguments: torch tensors supply device memory and the current
stream, and every step of the computation runs in the library's HIP kernels.
There is no CPU fallback: calling into a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqfa.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "qfa.h")

QTYPES = {"int8": 0, "fp8": 1, "int4": 2}
LAYOUTS = {"bnsd": 0, "bsnd": 1}
FLOATS = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
QMAX = {"int8": 127, "fp8": 448, "int4": 7}

_lib = None


class QFAError(RuntimeError):
    """A nonzero status from libqfa."""

    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().qfa_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status}: {msg}")


def lib() -> ctypes.CDLL:
    """The loaded libqfa.so (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_quantized_flashattention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.qfa_version.argtypes = []
    L.qfa_version.restype = i
    L.qfa_status_string.argtypes = [i]
    L.qfa_status_string.restype = ctypes.c_char_p
    L.qfa_block_quant.argtypes = [vp, i, i, i, i, i, i, i, i, vp, vp, i, vp]
    L.qfa_block_quant.restype = i
    L.qfa_block_quant_multi.argtypes = [ctypes.POINTER(QuantJob), i, vp]
    L.qfa_block_quant_multi.restype = i
    L.qfa_kv_append.argtypes = [vp, i, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.qfa_kv_append.restype = i
    L.qfa_kv_append_kv.argtypes = [vp, vp, i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp]
    L.qfa_kv_append_kv.restype = i
    L.qfa_rotate_block_quant.argtypes = [vp, i, vp, i, i, i, i, i, i, i, vp, vp, i, vp]
    L.qfa_rotate_block_quant.restype = i
    L.qfa_fwd.argtypes = [vp, vp, i, i, i, vp, vp, i, vp, vp, i, i, i,
                          i, i, i, i, i, i, i, i, f, vp, i, vp]
    L.qfa_fwd.restype = i
    L.qfa_fwd_lowp.argtypes = [vp, vp, i, i, i, vp, vp, i, vp, vp, i, i, i,
                          i, i, i, i, i, i, i, i, f, vp, i, vp, sz, vp]
    L.qfa_fwd_lowp.restype = i
    L.qfa_fwd_lowp_workspace_bytes.argtypes = [i, i, i, i]
    L.qfa_fwd_lowp_workspace_bytes.restype = sz
    L.qfa_decode_workspace_bytes.argtypes = [i, i, i, i]
    L.qfa_decode_workspace_bytes.restype = sz
    L.qfa_decode.argtypes = [vp, i, i, i, i, i, vp, vp, vp, vp, i, i, i, i, i, vp, f, vp, i,
                             vp, sz, vp]
    L.qfa_decode.restype = i
    L.qfa_decode_noalloc_max_bytes.argtypes = []
    L.qfa_decode_noalloc_max_bytes.restype = sz
    L.qfa_decode_noalloc.argtypes = [vp, i, i, i, i, i, vp, vp, vp, vp, i, i, i, i, i, vp, f, vp, i,
                                     vp]
    L.qfa_decode_noalloc.restype = i
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/qfa.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*QFA_API\s+(?:int|size_t|const char\*)\s+(qfa_\w+)\s*\(", text,
                                 flags=re.M)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise QFAError(fn, status)


def _dev(t: torch.Tensor, name: str):
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous GPU tensor")


def code_dtype(qtype: str) -> torch.dtype:
    return torch.int8 if qtype == "int8" else torch.uint8


def _expect(t: torch.Tensor, shape, dtypes, name: str):
    """Raise ValueError unless ``t`` has exactly ``shape`` and one of ``dtypes``.
    The library trusts the sizes it is given, so a mismatched tensor would be
    read or written out of bounds on the GPU."""
    if tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")


def _code_shape(shape_bnsd_like, qtype: str):
    """Shape of the codes of a tensor of this shape: the last dim halves for INT4."""
    d = shape_bnsd_like[-1]
    return tuple(shape_bnsd_like[:-1]) + (d // 2 if qtype == "int4" else d,)


_SCALE_DTYPES = (torch.float32, torch.float16)


class QuantJob(ctypes.Structure):
    """Mirror of qfa_quant_job (include/qfa.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("B", ctypes.c_int),
                ("N", ctypes.c_int), ("S", ctypes.c_int), ("D", ctypes.c_int),
                ("layout", ctypes.c_int), ("block_rows", ctypes.c_int), ("qtype", ctypes.c_int),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("scale_dtype", ctypes.c_int)]


def _quant_outputs(x, block_rows, qtype, scale_dtype, layout, codes, scales):
    _dev(x, "x")
    if layout == "bnsd":
        B, N, S, D = x.shape
    else:
        B, S, N, D = x.shape
    if qtype not in QTYPES or x.dtype not in FLOATS or block_rows < 1:
        raise ValueError("unknown qtype or input dtype, or block_rows < 1")
    cshape = _code_shape(x.shape, qtype)
    if codes is None:
        codes = torch.empty(cshape, dtype=code_dtype(qtype), device=x.device)
    if scales is None:
        scales = torch.empty(B, N, -(-S // block_rows), dtype=scale_dtype, device=x.device)
    _dev(codes, "codes")
    _dev(scales, "scales")
    _expect(codes, cshape, (code_dtype(qtype),), "codes")
    _expect(scales, (B, N, -(-S // block_rows)), _SCALE_DTYPES, "scales")
    job = QuantJob(_ptr(x), FLOATS[x.dtype], B, N, S, D, LAYOUTS[layout], block_rows,
                   QTYPES[qtype], _ptr(codes), _ptr(scales), FLOATS[scales.dtype])
    return job, codes, scales


def prepare_block_quant_multi(jobs, stream=None):
    """Marshal one ``block_quant_multi`` call once; returns (launch, outputs).

    ``launch()`` issues the same call again (same tensors, same stream) at the
    cost of one ctypes call, for loops that repeat a call on fixed buffers.
    """
    descs, outs = [], []
    for j in jobs:
        job, codes, scales = _quant_outputs(j["x"], j["block_rows"], j["qtype"],
                                            j.get("scale_dtype", torch.float32),
                                            j.get("layout", "bnsd"), j.get("codes"),
                                            j.get("scales"))
        descs.append(job)
        outs.append((codes, scales))
    arr = (QuantJob * max(len(descs), 1))(*descs)
    n, st, f = len(descs), _stream(stream), lib().qfa_block_quant_multi

    def launch():
        _check("qfa_block_quant_multi", f(arr, n, st))
    return launch, outs


def block_quant_multi(jobs, stream=None):
    """Quantize several tensors in shared launches; returns [(codes, scales), ...].

    Each job is a dict with the arguments of ``block_quant``: x, block_rows,
    qtype, and optionally scale_dtype (float32), layout ("bnsd"), codes, scales.
    Results are bit-identical to one ``block_quant`` call per job.
    """
    descs, outs = [], []
    for j in jobs:
        job, codes, scales = _quant_outputs(j["x"], j["block_rows"], j["qtype"],
                                            j.get("scale_dtype", torch.float32),
                                            j.get("layout", "bnsd"), j.get("codes"),
                                            j.get("scales"))
        descs.append(job)
        outs.append((codes, scales))
    arr = (QuantJob * max(len(descs), 1))(*descs)
    _check("qfa_block_quant_multi", lib().qfa_block_quant_multi(arr, len(descs), _stream(stream)))
    return outs


def block_quant(x: torch.Tensor, block_rows: int, qtype: str, scale_dtype=torch.float32,
                layout: str = "bnsd", codes=None, scales=None, stream=None):
    """Quantize ``x`` per block of ``block_rows`` rows; returns (codes, scales).

    x: [B,N,S,D] (bnsd) or [B,S,N,D] (bsnd); codes in the same layout (last dim
    D/2 for int4, int8 for INT8, uint8 for FP8 e4m3fn and packed INT4); scales
    [B,N,ceil(S/block_rows)] of ``scale_dtype``.
    """
    _dev(x, "x")
    if layout == "bnsd":
        B, N, S, D = x.shape
    else:
        B, S, N, D = x.shape
    if qtype not in QTYPES or x.dtype not in FLOATS or block_rows < 1:
        raise ValueError("unknown qtype or input dtype, or block_rows < 1")
    cshape = _code_shape(x.shape, qtype)
    if codes is None:
        codes = torch.empty(cshape, dtype=code_dtype(qtype), device=x.device)
    if scales is None:
        scales = torch.empty(B, N, -(-S // block_rows), dtype=scale_dtype, device=x.device)
    _dev(codes, "codes")
    _dev(scales, "scales")
    _expect(codes, cshape, (code_dtype(qtype),), "codes")
    _expect(scales, (B, N, -(-S // block_rows)), _SCALE_DTYPES, "scales")
    _check("qfa_block_quant", lib().qfa_block_quant(
        _ptr(x), FLOATS[x.dtype], B, N, S, D, LAYOUTS[layout], block_rows, QTYPES[qtype],
        _ptr(codes), _ptr(scales), FLOATS[scales.dtype], _stream(stream)))
    return codes, scales


def kv_append(x: torch.Tensor, positions: torch.Tensor, codes: torch.Tensor,
              scales: torch.Tensor, kv_block: int, qtype: str, layout: str = "bnsd",
              stream=None, prepare: bool = False):
    """Quantize x [B, H, D] into the cache (codes, scales) at row positions[b]
    of each sequence, in place (see qfa_kv_append); returns (codes, scales), or
    with ``prepare=True`` a launcher that repeats the marshalled call."""
    for t, n in ((x, "x"), (positions, "positions"), (codes, "codes"), (scales, "scales")):
        _dev(t, n)
    if positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    B, H, D = x.shape
    S_max = codes.shape[2] if layout == "bnsd" else codes.shape[1]
    cs = (B, H, S_max, D) if layout == "bnsd" else (B, S_max, H, D)
    _expect(codes, _code_shape(cs, qtype), (code_dtype(qtype),), "codes")
    _expect(scales, (B, H, -(-S_max // kv_block)), _SCALE_DTYPES, "scales")
    _expect(positions, (B,), (torch.int32,), "positions")
    if x.dtype not in FLOATS:
        raise ValueError(f"x has dtype {x.dtype}")
    args = (_ptr(x), FLOATS[x.dtype], _ptr(positions), _ptr(codes), _ptr(scales), B, H, S_max, D,
            LAYOUTS[layout], kv_block, QTYPES[qtype], FLOATS[scales.dtype], _stream(stream))
    f = lib().qfa_kv_append
    if prepare:
        def launch():
            _check("qfa_kv_append", f(*args))
        return launch
    _check("qfa_kv_append", f(*args))
    return codes, scales


def kv_append_kv(xk: torch.Tensor, xv: torch.Tensor, positions: torch.Tensor,
                 k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                 v_scales: torch.Tensor, kv_block: int, qtype: str, layout: str = "bnsd",
                 stream=None, prepare: bool = False):
    """``kv_append`` of a decode step's K and V rows in one launch (see
    qfa_kv_append_kv); returns (k_codes, k_scales, v_codes, v_scales), or with
    ``prepare=True`` a launcher that repeats the marshalled call."""
    for t, n in ((xk, "xk"), (xv, "xv"), (positions, "positions"), (k_codes, "k_codes"),
                 (k_scales, "k_scales"), (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, n)
    if positions.dtype != torch.int32:
        raise ValueError("positions must be int32")
    B, H, D = xk.shape
    _expect(xv, (B, H, D), (xk.dtype,), "xv")
    S_max = k_codes.shape[2] if layout == "bnsd" else k_codes.shape[1]
    cs = (B, H, S_max, D) if layout == "bnsd" else (B, S_max, H, D)
    for c, s, n in ((k_codes, k_scales, "k"), (v_codes, v_scales, "v")):
        _expect(c, _code_shape(cs, qtype), (code_dtype(qtype),), f"{n}_codes")
        _expect(s, (B, H, -(-S_max // kv_block)), _SCALE_DTYPES, f"{n}_scales")
    if v_scales.dtype != k_scales.dtype:
        raise ValueError("k_scales and v_scales must have the same dtype")
    _expect(positions, (B,), (torch.int32,), "positions")
    if xk.dtype not in FLOATS:
        raise ValueError(f"xk has dtype {xk.dtype}")
    args = (_ptr(xk), _ptr(xv), FLOATS[xk.dtype], _ptr(positions), _ptr(k_codes), _ptr(k_scales),
            _ptr(v_codes), _ptr(v_scales), B, H, S_max, D, LAYOUTS[layout], kv_block,
            QTYPES[qtype], FLOATS[k_scales.dtype], _stream(stream))
    f = lib().qfa_kv_append_kv
    if prepare:
        def launch():
            _check("qfa_kv_append_kv", f(*args))
        return launch
    _check("qfa_kv_append_kv", f(*args))
    return k_codes, k_scales, v_codes, v_scales


def rotate_block_quant(x: torch.Tensor, w: torch.Tensor, block_rows: int, qtype: str,
                       scale_dtype=torch.float32, layout: str = "bnsd", codes=None, scales=None,
                       stream=None):
    """y = x . w^T rounded to x's 16-bit type, block-quantized like ``block_quant``;
    returns (codes, scales). x: [B,N,S,D] (bnsd) or [B,S,N,D] (bsnd), fp16 or
    bf16; w: [D, D] of the same dtype (pass R^T to rotate by R)."""
    launch, codes, scales = prepare_rotate_block_quant(x, w, block_rows, qtype, scale_dtype,
                                                       layout, codes, scales, stream)
    launch()
    return codes, scales


def prepare_rotate_block_quant(x: torch.Tensor, w: torch.Tensor, block_rows: int, qtype: str,
                               scale_dtype=torch.float32, layout: str = "bnsd", codes=None,
                               scales=None, stream=None):
    """Marshal one ``rotate_block_quant`` call once; returns (launch, codes, scales)."""
    _dev(x, "x")
    _dev(w, "w")
    if layout == "bnsd":
        B, N, S, D = x.shape
    else:
        B, S, N, D = x.shape
    if codes is None:
        codes = torch.empty(x.shape, dtype=code_dtype(qtype), device=x.device)
    if scales is None:
        scales = torch.empty(B, N, -(-S // block_rows), dtype=scale_dtype, device=x.device)
    _dev(codes, "codes")
    _dev(scales, "scales")
    if w.dtype != x.dtype or tuple(w.shape) != (D, D):
        raise ValueError("w must be [D, D] with the dtype of x")
    _expect(codes, x.shape, (code_dtype(qtype),), "codes")
    _expect(scales, (B, N, -(-S // block_rows)), _SCALE_DTYPES, "scales")
    args = (_ptr(x), FLOATS[x.dtype], _ptr(w), B, N, S, D, LAYOUTS[layout], block_rows,
            QTYPES[qtype], _ptr(codes), _ptr(scales), FLOATS[scales.dtype], _stream(stream))
    f = lib().qfa_rotate_block_quant

    def launch():
        _check("qfa_rotate_block_quant", f(*args))
    return launch, codes, scales


def _fwd_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, q_qtype, k_qtype, v_qtype,
              q_block, kv_block, softmax_scale, causal, layout, out_dtype, out, stream):
    for t, n in ((q_codes, "q_codes"), (q_scales, "q_scales"), (k_codes, "k_codes"),
                 (k_scales, "k_scales"), (v_codes, "v_codes"), (v_scales, "v_scales")):
        _dev(t, n)
    if layout == "bnsd":
        B, Hq, Sq, D = q_codes.shape
        Hkv, Sk = k_codes.shape[1], k_codes.shape[2]
    else:
        B, Sq, Hq, D = q_codes.shape
        Sk, Hkv = k_codes.shape[1], k_codes.shape[2]
    for qt in (q_qtype, k_qtype, v_qtype):
        if qt not in QTYPES:
            raise ValueError(f"unknown code type {qt!r}")
    if q_qtype == "int4":
        raise ValueError("Q codes cannot be INT4")
    if q_block < 1 or kv_block < 1:
        raise ValueError("block sizes must be >= 1")
    if out is None:
        out = torch.empty(q_codes.shape, dtype=out_dtype, device=q_codes.device)
    _dev(out, "out")
    qshape = (B, Hq, Sq, D) if layout == "bnsd" else (B, Sq, Hq, D)
    kvshape = (B, Hkv, Sk, D) if layout == "bnsd" else (B, Sk, Hkv, D)
    _expect(q_codes, qshape, (code_dtype(q_qtype),), "q_codes")
    _expect(k_codes, _code_shape(kvshape, k_qtype), (code_dtype(k_qtype),), "k_codes")
    _expect(v_codes, _code_shape(kvshape, v_qtype), (code_dtype(v_qtype),), "v_codes")
    _expect(q_scales, (B, Hq, -(-Sq // q_block)), _SCALE_DTYPES, "q_scales")
    _expect(k_scales, (B, Hkv, -(-Sk // kv_block)), _SCALE_DTYPES, "k_scales")
    _expect(v_scales, (B, Hkv, -(-Sk // kv_block)), (k_scales.dtype,), "v_scales")
    _expect(out, qshape, tuple(FLOATS), "out")
    args = (_ptr(q_codes), _ptr(q_scales), QTYPES[q_qtype], q_block, FLOATS[q_scales.dtype],
            _ptr(k_codes), _ptr(k_scales), QTYPES[k_qtype], _ptr(v_codes), _ptr(v_scales),
            QTYPES[v_qtype], kv_block, FLOATS[k_scales.dtype], B, Hq, Hkv, Sq, Sk, D,
            LAYOUTS[layout], int(bool(causal)), float(softmax_scale), _ptr(out),
            FLOATS[out.dtype], _stream(stream))
    return args, out


def fwd(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, *, q_qtype: str, k_qtype: str,
        v_qtype: str, q_block: int, kv_block: int, softmax_scale: float, causal: bool = False,
        layout: str = "bnsd", out_dtype=torch.float16, out=None, stream=None):
    """Attention forward on block-quantized codes; returns out [B,Hq,Sq,D] (or BSND)."""
    args, out = _fwd_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, q_qtype,
                          k_qtype, v_qtype, q_block, kv_block, softmax_scale, causal, layout,
                          out_dtype, out, stream)
    _check("qfa_fwd", lib().qfa_fwd(*args))
    return out


def prepare_fwd(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, *, q_qtype: str,
                k_qtype: str, v_qtype: str, q_block: int, kv_block: int, softmax_scale: float,
                causal: bool = False, layout: str = "bnsd", out_dtype=torch.float16, out=None,
                stream=None):
    """Marshal one ``fwd`` call once; returns (launch, out).

    ``launch()`` issues the same forward again (same tensors, same stream) at
    the cost of one ctypes call, for loops that repeat a call on fixed buffers.
    """
    args, out = _fwd_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, q_qtype,
                          k_qtype, v_qtype, q_block, kv_block, softmax_scale, causal, layout,
                          out_dtype, out, stream)
    f = lib().qfa_fwd

    def launch():
        _check("qfa_fwd", f(*args))
    return launch, out


def fwd_lowp_workspace_bytes(B: int, Hq: int, Hkv: int, Sq: int) -> int:
    return int(lib().qfa_fwd_lowp_workspace_bytes(B, Hq, Hkv, Sq))


def _lowp_workspace(args, workspace, device):
    B, Hq, Hkv, Sq = args[13], args[14], args[15], args[16]
    need = fwd_lowp_workspace_bytes(B, Hq, Hkv, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=device)
    _dev(workspace, "workspace")
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    return args[:-1] + (_ptr(workspace), workspace.numel(), args[-1]), workspace


def fwd_lowp(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, *, q_qtype: str,
             k_qtype: str, v_qtype: str, q_block: int, kv_block: int, softmax_scale: float,
             causal: bool = False, layout: str = "bnsd", out_dtype=torch.float16, out=None,
             workspace=None, stream=None):
    """``fwd`` with P.V on the fp8 matrix unit (e4m3 Q/K/V, block scales) and
    the accuracy-gated fp16 fallback; returns (out, workspace). Byte 8*w + v
    of the workspace is 1 where wavefront v of work item w fell back."""
    args, out = _fwd_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, q_qtype,
                          k_qtype, v_qtype, q_block, kv_block, softmax_scale, causal, layout,
                          out_dtype, out, stream)
    args, workspace = _lowp_workspace(args, workspace, q_codes.device)
    _check("qfa_fwd_lowp", lib().qfa_fwd_lowp(*args))
    return out, workspace


def prepare_fwd_lowp(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, *, q_qtype: str,
                     k_qtype: str, v_qtype: str, q_block: int, kv_block: int,
                     softmax_scale: float, causal: bool = False, layout: str = "bnsd",
                     out_dtype=torch.float16, out=None, workspace=None, stream=None):
    """Marshal one ``fwd_lowp`` call once; returns (launch, out, workspace)."""
    args, out = _fwd_args(q_codes, q_scales, k_codes, k_scales, v_codes, v_scales, q_qtype,
                          k_qtype, v_qtype, q_block, kv_block, softmax_scale, causal, layout,
                          out_dtype, out, stream)
    args, workspace = _lowp_workspace(args, workspace, q_codes.device)
    f = lib().qfa_fwd_lowp

    def launch():
        _check("qfa_fwd_lowp", f(*args))
    return launch, out, workspace


def decode_workspace_bytes(B: int, Hq: int, S_max: int, D: int) -> int:
    return int(lib().qfa_decode_workspace_bytes(B, Hq, S_max, D))


def _decode_args(q, k_cache, v_cache, k_scales, v_scales, seq_lens, kv_qtype, kv_block,
                 softmax_scale, layout, out_dtype, out, workspace, stream):
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (k_scales, "k_scales"),
                 (v_scales, "v_scales"), (seq_lens, "seq_lens")):
        _dev(t, n)
    if seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32")
    B, D = q.shape[0], q.shape[-1]
    Hq = q.numel() // (B * D) if B * D else 0
    if layout == "bnsd":
        Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    else:
        S_max, Hkv = k_cache.shape[1], k_cache.shape[2]
    if kv_qtype not in QTYPES or kv_block < 1:
        raise ValueError("unknown kv_qtype or kv_block < 1")
    if q.dim() != 4 or q.numel() != B * Hq * D or q.dtype not in FLOATS:
        raise ValueError(f"q must be [B, Hq, 1, D] (or [B, 1, Hq, D]) float, got {tuple(q.shape)}")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    cshape = (B, Hkv, S_max, D) if layout == "bnsd" else (B, S_max, Hkv, D)
    _expect(k_cache, _code_shape(cshape, kv_qtype), (code_dtype(kv_qtype),), "k_cache")
    _expect(v_cache, _code_shape(cshape, kv_qtype), (code_dtype(kv_qtype),), "v_cache")
    _expect(k_scales, (B, Hkv, -(-S_max // kv_block)), _SCALE_DTYPES, "k_scales")
    _expect(v_scales, (B, Hkv, -(-S_max // kv_block)), (k_scales.dtype,), "v_scales")
    _expect(seq_lens, (B,), (torch.int32,), "seq_lens")
    _expect(out, q.shape, tuple(FLOATS), "out")
    head = (_ptr(q), FLOATS[q.dtype], B, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache), _ptr(k_scales),
            _ptr(v_scales), QTYPES[kv_qtype], kv_block, FLOATS[k_scales.dtype], S_max,
            LAYOUTS[layout], _ptr(seq_lens), float(softmax_scale), _ptr(out), FLOATS[out.dtype])
    if workspace is False:  # the no-alloc entry point takes no workspace
        return head + (_stream(stream),), out, None
    need = decode_workspace_bytes(B, Hq, S_max, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    args = head + (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    return args, out, workspace


def decode(q, k_cache, v_cache, k_scales, v_scales, seq_lens, *, kv_qtype: str, kv_block: int,
           softmax_scale: float, layout: str = "bnsd", out_dtype=None, out=None, workspace=None,
           stream=None):
    """One query token per sequence against a quantized KV cache; returns out [B,Hq,1,D]."""
    args, out, _ = _decode_args(q, k_cache, v_cache, k_scales, v_scales, seq_lens, kv_qtype,
                                kv_block, softmax_scale, layout, out_dtype, out, workspace, stream)
    _check("qfa_decode", lib().qfa_decode(*args))
    return out


def decode_noalloc_max_bytes() -> int:
    return int(lib().qfa_decode_noalloc_max_bytes())


def decode_noalloc(q, k_cache, v_cache, k_scales, v_scales, seq_lens, *, kv_qtype: str,
                   kv_block: int, softmax_scale: float, layout: str = "bnsd", out=None,
                   out_dtype=None, stream=None):
    """``decode`` without a workspace: the split-K partials go to the library's
    static per-device scratch (qfa_decode_noalloc). ``out`` may be given so
    that the call allocates nothing at all; calls that overlap on one GPU race."""
    args, out, _ = _decode_args(q, k_cache, v_cache, k_scales, v_scales, seq_lens, kv_qtype,
                                kv_block, softmax_scale, layout, out_dtype, out, False, stream)
    _check("qfa_decode_noalloc", lib().qfa_decode_noalloc(*args))
    return out


def prepare_decode(q, k_cache, v_cache, k_scales, v_scales, seq_lens, *, kv_qtype: str,
                   kv_block: int, softmax_scale: float, layout: str = "bnsd", out_dtype=None,
                   out=None, workspace=None, stream=None):
    """Marshal one ``decode`` call once; returns (launch, out).

    ``launch()`` issues the same decode again (same tensors, workspace and
    stream) at the cost of one ctypes call.
    """
    args, out, workspace = _decode_args(q, k_cache, v_cache, k_scales, v_scales, seq_lens,
                                        kv_qtype, kv_block, softmax_scale, layout, out_dtype, out,
                                        workspace, stream)
    f = lib().qfa_decode

    def launch():
        _check("qfa_decode", f(*args))
    launch.workspace = workspace  # keeps a workspace allocated here alive
    return launch, out


__all__ = ["block_quant", "block_quant_multi", "prepare_block_quant_multi", "rotate_block_quant",
           "prepare_rotate_block_quant", "kv_append", "kv_append_kv", "fwd", "prepare_fwd", "fwd_lowp",
           "prepare_fwd_lowp", "fwd_lowp_workspace_bytes",
           "decode", "prepare_decode", "decode_workspace_bytes", "decode_noalloc",
           "decode_noalloc_max_bytes", "lib", "header_functions",
           "QFAError", "QTYPES", "LAYOUTS", "FLOATS", "QMAX", "code_dtype"]
