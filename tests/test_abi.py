"""The C ABI: the library loads, exports every function the header declares,
and rejects invalid calls with the documented status before touching the
device. CPU only: every call here returns during host-side validation."""
import ctypes

import pytest

import block_quantized_flashattention_amd as qfa

OK, NULL, SHAPE, ENUM, UNSUP, WS = 0, 1, 2, 3, 4, 5
I8, F8, I4 = 0, 1, 2
F32, F16, BF16 = 0, 1, 2
BNSD, BSND = 0, 1
P = ctypes.c_void_p(256)  # a non-null, 256-byte-aligned stand-in never dereferenced
MIS = ctypes.c_void_p(258)


@pytest.fixture(scope="module")
def L():
    return qfa.lib()


def test_exports_every_declared_function(L):
    names = qfa.header_functions()
    assert set(names) == {"qfa_version", "qfa_status_string", "qfa_block_quant",
                          "qfa_block_quant_multi", "qfa_rotate_block_quant", "qfa_kv_append",
                          "qfa_kv_append_kv",
                          "qfa_fwd", "qfa_fwd_lowp", "qfa_fwd_lowp_workspace_bytes",
                          "qfa_decode_workspace_bytes", "qfa_decode",
                          "qfa_decode_noalloc_max_bytes", "qfa_decode_noalloc"}
    for n in names:
        assert hasattr(L, n), n


def test_status_strings(L):
    for s in range(8):
        assert L.qfa_status_string(s) != b"unknown status"
    assert L.qfa_status_string(99) == b"unknown status"
    assert L.qfa_version() >= 100


def quant(L, x=P, dt=F16, B=1, N=2, S=300, D=128, layout=BNSD, R=128, qt=I8, codes=P, scales=P,
          sdt=F32):
    return L.qfa_block_quant(x, dt, B, N, S, D, layout, R, qt, codes, scales, sdt, None)


def test_block_quant_validation(L):
    assert quant(L, dt=7) == ENUM
    assert quant(L, layout=2) == ENUM
    assert quant(L, qt=3) == ENUM
    assert quant(L, sdt=BF16) == ENUM
    assert quant(L, D=12) == SHAPE
    assert quant(L, D=0) == SHAPE
    assert quant(L, D=2048) == SHAPE
    assert quant(L, R=0) == SHAPE
    assert quant(L, B=-1) == SHAPE
    assert quant(L, x=None) == NULL
    assert quant(L, scales=None) == NULL
    assert quant(L, x=MIS) == UNSUP
    # empty tensors are valid and launch nothing, even with null pointers
    assert quant(L, S=0, x=None, codes=None, scales=None) == OK
    assert quant(L, B=0, x=None, codes=None, scales=None) == OK


def job(x=P, dt=F16, B=1, N=2, S=300, D=128, layout=BNSD, R=128, qt=I8, codes=P, scales=P,
        sdt=F32):
    return qfa.QuantJob(x, dt, B, N, S, D, layout, R, qt, codes, scales, sdt)


def multi(L, *jobs, n=None):
    arr = (qfa.QuantJob * max(len(jobs), 1))(*jobs)
    return L.qfa_block_quant_multi(arr, len(jobs) if n is None else n, None)


def test_block_quant_multi_validation(L):
    assert multi(L) == OK                      # no jobs: nothing to do
    assert multi(L, job(), n=-1) == SHAPE
    assert multi(L, job(), n=17) == SHAPE
    assert L.qfa_block_quant_multi(None, 2, None) == NULL
    # every job is checked before anything runs; the first failure is returned
    assert multi(L, job(dt=7), job(x=None)) == ENUM
    assert multi(L, job(S=0, x=None), job(D=12)) == SHAPE
    assert multi(L, job(S=0, x=None), job(scales=None)) == NULL
    assert multi(L, job(B=0, x=None, codes=None, scales=None)) == OK
    assert multi(L, job(S=0, x=None), job(x=MIS)) == UNSUP


def rot(L, x=P, dt=BF16, w=P, B=1, N=2, S=300, D=128, layout=BNSD, R=128, qt=F8, codes=P,
        scales=P, sdt=F32):
    return L.qfa_rotate_block_quant(x, dt, w, B, N, S, D, layout, R, qt, codes, scales, sdt, None)


def test_rotate_block_quant_validation(L):
    assert rot(L, dt=7) == ENUM
    assert rot(L, qt=9) == ENUM
    assert rot(L, D=12) == SHAPE
    assert rot(L, R=0) == SHAPE
    assert rot(L, dt=F32) == UNSUP             # 16-bit inputs only
    assert rot(L, D=96) == UNSUP
    assert rot(L, qt=I4) == UNSUP
    assert rot(L, R=100) == UNSUP              # block rows: multiples of 32, at most 256
    assert rot(L, R=288) == UNSUP
    assert rot(L, w=None) == NULL
    assert rot(L, x=None) == NULL
    assert rot(L, w=MIS) == UNSUP              # misaligned
    assert rot(L, S=0, x=None, w=None) == OK   # empty: nothing to do


def app(L, x=P, dt=F16, pos=P, codes=P, scales=P, B=2, H=4, S=512, D=128, layout=BNSD, R=256,
        qt=I8, sdt=F16):
    return L.qfa_kv_append(x, dt, pos, codes, scales, B, H, S, D, layout, R, qt, sdt, None)


def test_kv_append_validation(L):
    assert app(L, dt=7) == ENUM
    assert app(L, qt=9) == ENUM
    assert app(L, sdt=BF16) == ENUM
    assert app(L, S=0) == SHAPE
    assert app(L, D=12) == SHAPE
    assert app(L, R=0) == SHAPE
    assert app(L, qt=F8) == UNSUP
    assert app(L, D=264) == UNSUP
    assert app(L, D=520, qt=I4) == UNSUP
    assert app(L, pos=None) == NULL
    assert app(L, scales=None) == NULL
    assert app(L, scales=ctypes.c_void_p(257)) == UNSUP
    assert app(L, B=0, x=None, pos=None, codes=None, scales=None) == OK


def app2(L, xk=P, xv=P, dt=F16, pos=P, kc=P, ks=P, vc=P, vs=P, B=2, H=4, S=512, D=128,
         layout=BNSD, R=256, qt=I8, sdt=F16):
    return L.qfa_kv_append_kv(xk, xv, dt, pos, kc, ks, vc, vs, B, H, S, D, layout, R, qt, sdt,
                              None)


def test_kv_append_kv_validation(L):
    """The K and V append in one launch checks both caches' arguments as the
    single append does, and launches nothing on an error."""
    assert app2(L, dt=7) == ENUM
    assert app2(L, qt=F8) == UNSUP
    assert app2(L, D=12) == SHAPE
    assert app2(L, xk=None) == NULL
    assert app2(L, xv=None) == NULL
    assert app2(L, vc=None) == NULL
    assert app2(L, vs=None) == NULL
    assert app2(L, ks=ctypes.c_void_p(257)) == UNSUP
    assert app2(L, vs=ctypes.c_void_p(257)) == UNSUP
    assert app2(L, B=0, xk=None, xv=None, pos=None, kc=None, ks=None, vc=None, vs=None) == OK


def fwd(L, q=P, qs=P, qqt=I8, qb=128, qsd=F32, k=P, ks=P, kqt=I8, v=P, vs=P, vqt=I8, kb=256,
        ksd=F32, B=1, Hq=4, Hkv=2, Sq=100, Sk=100, D=128, layout=BNSD, causal=1, scale=0.1,
        out=P, odt=F16):
    return L.qfa_fwd(q, qs, qqt, qb, qsd, k, ks, kqt, v, vs, vqt, kb, ksd, B, Hq, Hkv, Sq, Sk, D,
                     layout, causal, ctypes.c_float(scale), out, odt, None)


def test_fwd_validation(L):
    assert fwd(L, qqt=5) == ENUM
    assert fwd(L, odt=4) == ENUM
    assert fwd(L, qsd=BF16) == ENUM
    assert fwd(L, Hq=3, Hkv=2) == SHAPE
    assert fwd(L, Hkv=0) == SHAPE
    assert fwd(L, qb=0) == SHAPE
    assert fwd(L, causal=2) == SHAPE
    assert fwd(L, D=96) == UNSUP
    assert fwd(L, Sq=10, Sk=20, causal=1) == UNSUP
    assert fwd(L, Sq=10, Sk=0, causal=0) == SHAPE
    assert fwd(L, scale=float("nan")) == SHAPE
    assert fwd(L, qqt=F8) == UNSUP             # fp8 Q with int8 K
    assert fwd(L, qqt=I4) == UNSUP             # int4 Q
    assert fwd(L, kqt=I4, qqt=F8) == UNSUP
    assert fwd(L, out=None) == NULL
    assert fwd(L, v=None) == NULL
    assert fwd(L, q=MIS) == UNSUP
    assert fwd(L, Sq=0, Sk=0, q=None, k=None, v=None, out=None) == OK


def dec(L, q=P, qdt=F16, B=2, Hq=4, Hkv=2, D=128, k=P, v=P, ks=P, vs=P, qt=I8, kb=256, sdt=F16,
        S_max=4096, layout=BNSD, lens=P, scale=0.1, out=P, odt=F16, ws=P, wsb=1 << 20):
    return L.qfa_decode(q, qdt, B, Hq, Hkv, D, k, v, ks, vs, qt, kb, sdt, S_max, layout, lens,
                        ctypes.c_float(scale), out, odt, ws, wsb, None)


def test_decode_validation(L):
    need = L.qfa_decode_workspace_bytes(2, 4, 4096, 128)
    assert need == 2 * 4 * 4 * 130 * 4
    assert L.qfa_decode_workspace_bytes(2, 4, 4096, 96) == 0
    assert dec(L, qdt=9) == ENUM
    assert dec(L, qt=7) == ENUM
    assert dec(L, Hq=5) == SHAPE
    assert dec(L, S_max=0) == SHAPE
    assert dec(L, D=32) == UNSUP
    assert dec(L, qt=F8) == UNSUP
    assert dec(L, Hq=64, Hkv=2) == UNSUP
    # Rows of one (batch, KV head) must stay within 32-bit byte offsets:
    # (S_max + 1024) * row_stride < 2^31 (row_stride = Hkv * D in BSND).
    assert dec(L, B=0, layout=BSND, Hq=16, Hkv=16, S_max=(1 << 20) - 1024) == UNSUP
    assert dec(L, B=0, layout=BSND, Hq=16, Hkv=16, S_max=(1 << 20) - 1025) == OK
    assert dec(L, B=0, layout=BSND, Hq=16, Hkv=16, S_max=(1 << 20) - 1024, qt=I4) == OK
    assert dec(L, lens=None) == NULL
    assert dec(L, ws=None) == WS
    assert dec(L, wsb=need - 1) == WS
    assert dec(L, k=MIS, wsb=need) == UNSUP
    assert dec(L, B=0, q=None, k=None, v=None) == OK


def dec_na(L, q=P, qdt=F16, B=2, Hq=4, Hkv=2, D=128, k=P, v=P, ks=P, vs=P, qt=I8, kb=256,
           sdt=F16, S_max=4096, layout=BNSD, lens=P, scale=0.1, out=P, odt=F16):
    return L.qfa_decode_noalloc(q, qdt, B, Hq, Hkv, D, k, v, ks, vs, qt, kb, sdt, S_max, layout,
                                lens, ctypes.c_float(scale), out, odt, None)


def test_decode_noalloc_validation(L):
    """The allocation-free decode validates as qfa_decode does and refuses a
    call whose split-K partials would not fit the static scratch, before any
    device call (these return during host-side validation)."""
    SCRATCH = 7
    cap = L.qfa_decode_noalloc_max_bytes()
    assert cap == 8 << 20
    assert dec_na(L, qdt=9) == ENUM
    assert dec_na(L, Hq=5) == SHAPE
    assert dec_na(L, D=32) == UNSUP
    assert dec_na(L, lens=None) == NULL
    assert dec_na(L, k=MIS) == UNSUP
    assert dec_na(L, B=0, q=None, k=None, v=None) == OK
    # D=128: B * Hq * ceil(S_max/1024) * 130 floats must fit 8 MiB.
    assert L.qfa_decode_workspace_bytes(32, 32, 16384, 128) > cap
    assert dec_na(L, B=32, Hq=32, Hkv=32, S_max=16384) == SCRATCH
    assert dec_na(L, B=32, Hq=32, Hkv=32, S_max=16384, lens=None) == NULL  # validation first
    assert L.qfa_status_string(SCRATCH) != b"unknown status"


def fwd_lp(L, ws=P, wsb=1 << 20, **kw):
    args = dict(q=P, qs=P, qqt=F8, qb=128, qsd=F32, k=P, ks=P, kqt=F8, v=P, vs=P, vqt=F8, kb=256,
                ksd=F32, B=1, Hq=4, Hkv=2, Sq=300, Sk=300, D=128, layout=BNSD, causal=0, scale=0.1,
                out=P, odt=F16)
    args.update(kw)
    a = args
    return L.qfa_fwd_lowp(a["q"], a["qs"], a["qqt"], a["qb"], a["qsd"], a["k"], a["ks"], a["kqt"],
                          a["v"], a["vs"], a["vqt"], a["kb"], a["ksd"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Sk"], a["D"], a["layout"], a["causal"],
                          ctypes.c_float(a["scale"]), a["out"], a["odt"], ws, wsb, None)


def test_fwd_lowp_validation(L):
    """fp8 P.V: e4m3 Q/K/V with block scales only, a workspace of one byte per
    work item and wavefront; validated like qfa_fwd before any device call."""
    need = L.qfa_fwd_lowp_workspace_bytes(1, 4, 2, 300)
    # 2 KV heads x group 2 (both heads of a group in one workgroup: 128 rows
    # each) x ceil(300 / 128) row blocks, 8 bytes each
    assert need == 2 * 3 * 8
    assert L.qfa_fwd_lowp_workspace_bytes(1, 3, 2, 300) == 0
    assert fwd_lp(L, qqt=I8, kqt=I8, vqt=I8) == UNSUP
    assert fwd_lp(L, kb=100) == UNSUP                  # per-key scales
    assert fwd_lp(L, ws=None) == WS
    assert fwd_lp(L, wsb=need - 1) == WS
    assert fwd_lp(L, ws=ctypes.c_void_p(260), wsb=need) == UNSUP  # 8-byte alignment
    assert fwd_lp(L, qqt=5) == ENUM
    assert fwd_lp(L, Hq=3) == SHAPE
    assert fwd_lp(L, v=None) == NULL
    assert fwd_lp(L, Sq=0, Sk=0, q=None, k=None, v=None, out=None, ws=None) == OK
