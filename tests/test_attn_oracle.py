"""Pins for the sparse-attention oracle, checked against things other than the
oracle itself: torch's scaled_dot_product_attention and logsumexp in float64
on the gathered rows, and closed forms (uniform weights give the mean, one
key gives itself, a dominant key wins, padding and order do not matter).
No GPU needed."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W


def _bf16(g, shape, scale=1.0):
    return W.to_bf16_bits((g.standard_normal(shape) * scale).astype(np.float32))


def _f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def _random_idx(g, B, T, S, k, pad_frac=0.2):
    idx = np.empty((B, T, k), np.int32)
    for b in range(B):
        for t in range(T):
            n = min(S, k)
            sel = g.choice(S, n, replace=False)
            row = np.full(k, -1, np.int32)
            row[:n] = sel
            drop = g.random(k) < pad_frac
            row[drop] = -1
            idx[b, t] = row
    return idx


@pytest.mark.parametrize("seed,B,T,S,H,k,dqk,dv", [(1, 1, 3, 50, 2, 16, 24, 16), (2, 2, 2, 300, 3, 64, 40, 32),
                                                  (3, 1, 2, 20, 1, 32, 8, 8)])
def test_matches_torch_sdpa_and_logsumexp(seed, B, T, S, H, k, dqk, dv):
    g = np.random.Generator(np.random.PCG64(seed))
    q = _bf16(g, (B, T, H, dqk))
    c = _bf16(g, (B, S, dqk))
    idx = _random_idx(g, B, T, S, k)
    scale = 1.0 / math.sqrt(dqk)
    out, lse = oracle.sparse_attention(q, c, idx, scale, dv)
    qf, cf = _f64(q), _f64(c)
    for b in range(B):
        for t in range(T):
            sel = idx[b, t][idx[b, t] >= 0]
            K = torch.from_numpy(cf[b, sel])
            V = torch.from_numpy(cf[b, sel, :dv])
            Q = torch.from_numpy(qf[b, t])  # [H, dqk]
            ref = torch.nn.functional.scaled_dot_product_attention(Q[:, None, :], K[None], V[None],
                                                                   scale=scale)[:, 0, :]
            got = out[b * T + t]
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)
            ref_lse = torch.logsumexp(scale * (Q @ K.T), dim=-1).numpy()
            np.testing.assert_allclose(lse[b * T + t], ref_lse, rtol=1e-12, atol=1e-12)


def test_uniform_weights_give_the_mean():
    g = np.random.Generator(np.random.PCG64(4))
    q = np.zeros((1, 1, 2, 16), np.uint16)  # all scores 0
    c = _bf16(g, (1, 40, 16))
    idx = np.array([[[3, 9, -1, 27, 1]]], np.int32)
    out, lse = oracle.sparse_attention(q, c, idx, 0.5, 12)
    mean = _f64(c)[0, [3, 9, 27, 1], :12].mean(0)
    np.testing.assert_allclose(out[0, 0], mean, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(out[0, 1], mean, rtol=1e-15, atol=1e-15)
    assert lse[0, 0] == pytest.approx(math.log(4), abs=1e-15)


def test_single_key_is_returned_exactly():
    g = np.random.Generator(np.random.PCG64(5))
    q = _bf16(g, (1, 1, 3, 16))
    c = _bf16(g, (1, 10, 16))
    idx = np.array([[[-1, 7, -1]]], np.int32)
    out, lse = oracle.sparse_attention(q, c, idx, 0.25, 16)
    cf = _f64(c)[0, 7]
    for h in range(3):
        np.testing.assert_array_equal(out[0, h], cf)
        assert lse[0, h] == pytest.approx(0.25 * float(_f64(q)[0, 0, h] @ cf), rel=1e-15)


def test_dominant_key_wins():
    # score 60 for key 4, 0 for the rest: the weights of the others are e^-60
    q = np.zeros((1, 1, 1, 8), np.float32)
    q[..., 0] = 60.0
    c = np.zeros((1, 6, 8), np.float32)
    c[0, :, 1:] = np.arange(6)[:, None] + 1.0
    c[0, 4, 0] = 1.0
    out, _ = oracle.sparse_attention(W.to_bf16_bits(q), W.to_bf16_bits(c),
                                     np.array([[[0, 1, 2, 3, 4, 5]]], np.int32), 1.0, 8)
    np.testing.assert_allclose(out[0, 0, 1:], np.full(7, 5.0), rtol=1e-20, atol=5 * 6 * math.exp(-60))
    assert out[0, 0, 0] == pytest.approx(1.0, abs=1e-20 + 6 * math.exp(-60))


def test_padding_order_and_out_of_range_entries_do_not_matter():
    g = np.random.Generator(np.random.PCG64(6))
    q = _bf16(g, (1, 1, 2, 32))
    c = _bf16(g, (1, 100, 32))
    base = np.array([5, 17, 42, 99, 0], np.int32)
    a, la = oracle.sparse_attention(q, c, base[None, None], 0.2, 16)
    noisy = np.array([-1, 42, 100, 0, -7, 99, 5, 17, 1000], np.int32)
    b, lb = oracle.sparse_attention(q, c, noisy[None, None], 0.2, 16)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(la, lb, rtol=1e-14, atol=1e-15)


def test_no_valid_entry_gives_zero_and_minus_inf():
    q = np.ones((1, 1, 2, 8), np.uint16)
    c = np.ones((1, 4, 8), np.uint16)
    out, lse = oracle.sparse_attention(q, c, np.array([[[-1, 4, -2]]], np.int32), 1.0, 8)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_streams_use_their_own_cache():
    g = np.random.Generator(np.random.PCG64(8))
    q = _bf16(g, (2, 1, 1, 16))
    c = _bf16(g, (2, 20, 16))
    idx = np.array([[[3, 4]], [[3, 4]]], np.int32)
    out, _ = oracle.sparse_attention(q, c, idx, 0.3, 16)
    for b in range(2):
        one, _ = oracle.sparse_attention(q[b:b + 1], c[b:b + 1], idx[b:b + 1], 0.3, 16)
        np.testing.assert_array_equal(out[b], one[0])
    assert not np.allclose(out[0], out[1])
