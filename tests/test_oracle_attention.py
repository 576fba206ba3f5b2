"""Pins of the oracle's attention and decode against a library routine
(torch's scaled_dot_product_attention in float64 on the CPU), closed forms and
special cases. CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import qfa_workloads as wl


def _rand(shape, seed):
    return torch.randn(*shape, generator=torch.Generator().manual_seed(seed), dtype=torch.float64)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 4), (8, 2)])
def test_attention_matches_sdpa(causal, Hq, Hkv):
    B, S, D = 2, 67, 32
    q, k, v = _rand((B, Hq, S, D), 1), _rand((B, Hkv, S, D), 2), _rand((B, Hkv, S, D), 3)
    scale = 0.3
    ref = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale,
                                         enable_gqa=Hq != Hkv).numpy()
    out = oracle.attention(q.numpy(), k.numpy(), v.numpy(), scale, causal)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_attention_noncausal_rectangular():
    q, k, v = _rand((1, 2, 5, 16), 4), _rand((1, 2, 40, 16), 5), _rand((1, 2, 40, 16), 6)
    ref = F.scaled_dot_product_attention(q, k, v, scale=0.25).numpy()
    np.testing.assert_allclose(oracle.attention(q.numpy(), k.numpy(), v.numpy(), 0.25), ref,
                               rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_values():
    """All keys equal: every score in a row is the same, so o_i is the mean of
    the attended values (the prefix mean when causal)."""
    S, D = 50, 8
    q = _rand((1, 1, S, D), 7).numpy()
    k = np.repeat(_rand((1, 1, 1, D), 8).numpy(), S, axis=2)
    v = _rand((1, 1, S, D), 9).numpy()
    out = oracle.attention(q, k, v, 0.7, causal=False)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0].mean(0), (S, D)), atol=1e-13)
    outc = oracle.attention(q, k, v, 0.7, causal=True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(outc[0, 0], prefix, atol=1e-13)


def test_one_hot_score_copies_value_row():
    """One key scoring 60 above all others: the output is that key's value row
    (the others weigh at most S * e^-60)."""
    S, D = 32, 16
    q = np.zeros((1, 1, 4, D))
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, S, D))
    k[0, 0, 13, 0] = 60.0
    v = _rand((1, 1, S, D), 10).numpy()
    out = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0, 13], (4, D)), atol=1e-20 + 1e-24 * S)


def test_causal_first_row_is_first_value():
    q, k, v = (_rand((1, 3, 20, 8), s).numpy() for s in (11, 12, 13))
    out = oracle.attention(q, k, v, 1.3, causal=True)
    np.testing.assert_array_equal(out[0, :, 0], v[0, :, 0])


def test_gqa_equals_mha_with_repeated_heads():
    q = _rand((1, 8, 30, 16), 14).numpy()
    k, v = _rand((1, 2, 30, 16), 15).numpy(), _rand((1, 2, 30, 16), 16).numpy()
    out = oracle.attention(q, k, v, 0.5, causal=True)
    rep = oracle.attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.5, causal=True)
    np.testing.assert_array_equal(out, rep)


def test_attention_rows_match_full():
    q, k, v = (_rand((2, 4, 40, 8), s).numpy() for s in (17, 18, 19))
    k, v = k[:, :2], v[:, :2]
    full = oracle.attention(q, k, v, 0.9, causal=True)
    rows = [0, 5, 39]
    part = oracle.attention_rows(q, k, v, 0.9, True, 1, 3, rows)
    np.testing.assert_allclose(part, full[1, 3, rows], atol=1e-14)


def test_decode_is_last_causal_row_and_single_query_sdpa():
    B, Hq, Hkv, S, D = 3, 4, 2, 64, 16
    lens = np.array([64, 1, 37])
    q = _rand((B, Hq, 1, D), 20).numpy()
    k, v = _rand((B, Hkv, S, D), 21).numpy(), _rand((B, Hkv, S, D), 22).numpy()
    out = oracle.decode(q, k, v, lens, 0.4)
    for b in range(B):
        L = int(lens[b])
        ref = F.scaled_dot_product_attention(
            torch.from_numpy(q[b:b + 1]), torch.from_numpy(k[b:b + 1, :, :L]),
            torch.from_numpy(v[b:b + 1, :, :L]), scale=0.4, enable_gqa=True).numpy()
        np.testing.assert_allclose(out[b:b + 1], ref, atol=1e-12)
        # the same query appended as the last row of a causal prefill of length L
        qq = np.concatenate([np.zeros((1, Hq, L - 1, D)), q[b:b + 1]], axis=2)
        full = oracle.attention(qq, k[b:b + 1, :, :L], v[b:b + 1, :, :L], 0.4, causal=True)
        np.testing.assert_allclose(out[b, :, 0], full[0, :, L - 1], atol=1e-12)
    assert np.array_equal(out[1, :, 0], v[1, np.arange(Hq) // 2, 0])


def test_tiny_workload_end_to_end_fidelity():
    """The tiny INT8 workload: the oracle's attention on dequantized codes stays
    close to unquantized attention (quantization fidelity, not a parity gate)."""
    w = wl.TINY
    q, k, v = wl.make_prefill_inputs(w)
    qc, qs = oracle.block_quant(q, w.q_block, w.q_qtype)
    kc, ks = oracle.block_quant(k, w.kv_block, w.k_qtype)
    vc, vs = oracle.block_quant(v, w.kv_block, w.v_qtype)
    qh = oracle.dequantize(qc, qs, w.q_block, w.q_qtype)
    kh = oracle.dequantize(kc, ks, w.kv_block, w.k_qtype)
    vh = oracle.dequantize(vc, vs, w.kv_block, w.v_qtype)
    out = oracle.attention(qh, kh, vh, w.softmax_scale, w.causal)
    ref = F.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                         scale=w.softmax_scale).numpy()
    assert np.abs(out - ref).max() < 0.03
    assert np.abs(out - ref).mean() < 0.005
