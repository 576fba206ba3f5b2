"""The forward kernel's address arithmetic, checked on the CPU: the index
functions the kernel uses (compiled for the host into libqfa_ixcheck.so) are
walked over every workgroup, thread and fetched tile of a launch, and every
code and scale address must lie inside its tensor; every output row must be
computed exactly once. A tensor extent one byte short must be caught, which
shows that the walk reaches each tensor's last byte."""
import ctypes
import os

import pytest

import qfa_workloads as wl
from block_quantized_flashattention_amd import build as qbuild

KINDS = {"Q codes": 1, "K codes": 2, "V codes": 4, "Q scales": 8, "K/V scales": 16, "output": 32}


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(qbuild.IXCHECK_LIB):
        qbuild.build_ixcheck()
    lib = ctypes.CDLL(qbuild.IXCHECK_LIB)
    i = ctypes.c_int
    lib.qfa_ixcheck_fwd.argtypes = [i] * 15 + [ctypes.POINTER(i), ctypes.c_char_p, i]
    lib.qfa_ixcheck_fwd.restype = ctypes.c_long
    return lib


def check(L, B, Hq, Hkv, Sq, Sk, D, layout="bnsd", kqt="int8", vqt="int8", q_block=128,
          kv_block=256, q_f16=False, kv_f16=False, causal=True, shrink=0):
    kinds = ctypes.c_int(0)
    msg = ctypes.create_string_buffer(256)
    n = L.qfa_ixcheck_fwd(B, Hq, Hkv, Sq, Sk, D, layout == "bsnd", kqt == "int4", vqt == "int4",
                          q_block, kv_block, q_f16, kv_f16, causal, shrink, ctypes.byref(kinds),
                          msg, 256)
    return n, kinds.value, msg.value.decode()


def _workload_args(w):
    return dict(B=w.B, Hq=w.Hq, Hkv=w.Hkv, Sq=w.S, Sk=w.S, D=w.D, kqt=w.k_qtype, vqt=w.v_qtype,
                q_block=w.q_block, kv_block=w.kv_block, q_f16=w.q_scale_dtype == "f16",
                kv_f16=w.kv_scale_dtype == "f16", causal=w.causal)


@pytest.mark.parametrize("w", [wl.INT8_CAUSAL, wl.FP8_ROT, wl.GQA_INT4, wl.INT8QK_INT4V, wl.TINY],
                         ids=lambda w: w.name)
def test_full_workloads_in_bounds(L, w):
    n, kinds, msg = check(L, **_workload_args(w))
    assert n == 0, msg


CASES = [
    # B, Hq, Hkv, S, D, layout, K, V, q_block, kv_block, q_f16, kv_f16, causal
    (1, 1, 1, 1, 128, "bnsd", "int8", "int8", 128, 256, False, False, True),
    (1, 1, 1, 1, 64, "bsnd", "int4", "int4", 1, 1, True, True, False),
    (2, 3, 1, 63, 128, "bnsd", "int8", "int4", 128, 256, False, True, True),
    (1, 4, 4, 65, 64, "bsnd", "int8", "int8", 77, 64, True, False, False),
    (3, 6, 2, 300, 128, "bsnd", "int4", "int4", 128, 1, False, True, True),
    (1, 16, 1, 257, 128, "bnsd", "int4", "int4", 128, 16, False, True, True),
    (4, 8, 2, 1000, 64, "bnsd", "int8", "int8", 32, 100, True, True, False),   # xcd order
    (8, 8, 8, 130, 128, "bsnd", "int8", "int4", 128, 128, False, False, True),
    (1, 12, 4, 700, 128, "bnsd", "int8", "int8", 128, 192, False, False, True),  # group 3
    (2, 48, 8, 333, 128, "bsnd", "int4", "int4", 64, 1, False, True, True),     # group 6
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_small_and_ragged_shapes_in_bounds(L, case):
    B, Hq, Hkv, S, D, layout, kqt, vqt, qb, kb, qf, kf, causal = case
    n, kinds, msg = check(L, B, Hq, Hkv, S, S, D, layout, kqt, vqt, qb, kb, qf, kf, causal)
    assert n == 0, msg


def test_rectangular_noncausal_in_bounds(L):
    for Sq, Sk in [(1, 5000), (4097, 3), (200, 1000)]:
        n, kinds, msg = check(L, 2, 4, 2, Sq, Sk, 128, causal=False, kv_block=1, kv_f16=True,
                              kqt="int4", vqt="int4")
        assert n == 0, (Sq, Sk, msg)


@pytest.mark.parametrize("case", CASES[:6], ids=lambda c: "_".join(map(str, c)))
def test_walk_reaches_every_tensor_end(L, case):
    """With each extent one element short, every tensor must be flagged: the
    walk does read the last byte of each, so it is not vacuous."""
    B, Hq, Hkv, S, D, layout, kqt, vqt, qb, kb, qf, kf, causal = case
    n, kinds, msg = check(L, B, Hq, Hkv, S, S, D, layout, kqt, vqt, qb, kb, qf, kf, causal,
                          shrink=1)
    assert n > 0
    for name, bit in KINDS.items():
        assert kinds & bit, f"{name} never reaches its last element"


def test_rejects_unsupported_shape(L):
    assert check(L, 1, 3, 2, 10, 10, 128)[0] == -1      # Hq not a multiple of Hkv
    assert check(L, 1, 2, 2, 10, 20, 128)[0] == -1      # causal with Sq != Sk
