"""Pins for the CPU oracle, checked against things other than the oracle itself:
the OCP E4M3 encoding table (and torch's independent float8 codec), a
hand-worked example, closed-form special cases, an exact rational brute force
on tiny inputs, a reduction to numpy's lexsort, invariants and metamorphic
relations. No GPU needed."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _wl(q, k, w, k_scale=None, q_dtype=W.F32, k_dtype=W.F32, offset=0, topk=4):
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    B, T, H, D = q.shape
    S = k.shape[1]
    return W.Workload("t", q, k, k_scale, np.ascontiguousarray(w, dtype=np.float32), B, T, S,
                      H, D, offset, topk, q_dtype, k_dtype, [(0, T, S, offset)])


# --------------------------------------------------------------------------- E4M3

def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ocp_anchors.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                c, ocp, fnuz = line.split()
                rows.append((int(c, 16), float(ocp), float(fnuz)))
    return rows


def test_e4m3_anchors_ocp_not_fnuz():
    for code, ocp, fnuz in _golden_e4m3():
        got = oracle.e4m3_decode(code)
        if math.isnan(ocp):
            assert math.isnan(got), hex(code)
        else:
            assert got == ocp and math.copysign(1, got) == math.copysign(1, ocp), hex(code)
        if not math.isnan(fnuz) and fnuz != 0:
            assert got != fnuz, f"{code:#x} decoded with the FNUZ reading"


def test_e4m3_fnuz_column_is_torch_fnuz():
    # The fixture's FNUZ column agrees with torch's own fnuz codec, so the
    # "not FNUZ" check above tests against the real alternative reading.
    for code, _ocp, fnuz in _golden_e4m3():
        t = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fnuz).float().item()
        assert (math.isnan(t) and math.isnan(fnuz)) or t == fnuz, hex(code)


def test_e4m3_all_codes_match_torch_ocp():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        got = oracle.e4m3_decode(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c] and math.copysign(1, got) == math.copysign(1, ref[c]), c


def test_quantizer_roundtrip_within_half_ulp():
    # The generator's per-token encoding: |decode(code)*scale - x| <= 2^-4 of
    # |x| rounded up to the subnormal step, and amax maps to 448.
    g = np.random.Generator(np.random.PCG64(11))
    x = g.standard_normal((64, 128), dtype=np.float32)
    codes, scale = W.quantize_e4m3_per_token(x)
    dec = np.array([oracle.e4m3_decode(c) for c in range(256)])[codes] * scale[:, None]
    amax = np.abs(x).max(1)
    assert np.all(np.abs(np.abs(dec).max(1) - amax) <= amax * 2 ** -4)
    step = scale[:, None] * 2.0 ** -9
    assert np.all(np.abs(dec - x) <= np.maximum(np.abs(x) * 2 ** -4, step) * 1.0000001)


# --------------------------------------------------------------------------- hand example

def test_hand_worked_example():
    q = np.zeros((1, 4, 2, 2), np.float32)
    k = np.zeros((1, 4, 2), np.float32)
    w = np.zeros((1, 4, 2), np.float32)
    expects, scores = [], []
    with open(os.path.join(GOLDEN, "hand_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tag, *v = line.split()
            if tag == "k":
                k[0, int(v[0])] = [float(v[1]), float(v[2])]
            elif tag == "q":
                q[0, int(v[0]), int(v[1])] = [float(v[2]), float(v[3])]
            elif tag == "w":
                w[0, int(v[0]), int(v[1])] = float(v[2])
            elif tag == "expect":
                expects.append((int(v[0]), int(v[1]), [int(x) for x in v[2:]]))
            elif tag == "score":
                scores.append((int(v[0]), int(v[1]), float(v[2])))
    for topk, t, exp in expects:
        idx, *_ = oracle.select(_wl(q, k, w, topk=topk), rows=[t])
        assert list(idx[0]) == exp, (topk, t)
    wl = _wl(q, k, w)
    got = oracle.score_pairs(wl, [s[0] for s in scores], [s[1] for s in scores])
    assert list(got) == [s[2] for s in scores]
    assert math.isnan(oracle.score_pairs(wl, [0], [1])[0])  # causal: t=0 cannot see s=1


# --------------------------------------------------------------------------- closed forms

def _fp8_ramp(T, S, H, D, scale, offset=0):
    q = np.zeros((1, T, H, D), np.float32)
    q[..., 0] = 1.0
    k = np.full((1, S, D), 0x38, np.uint8)  # E4M3 1.0
    w = np.full((1, T, H), 0.5, np.float32)
    return _wl(q, k, w, k_scale=scale.reshape(1, S).astype(np.float32),
               k_dtype=W.FP8, offset=offset)


@pytest.mark.parametrize("offset", [0, 37])
def test_all_equal_scores_pick_lowest_indices(offset):
    # K == 0: every score is exactly 0, the answer is {0 .. min(k,L)-1}.
    T, S, k = 9, 9 + offset, 5
    g = np.random.Generator(np.random.PCG64(3))
    q = g.standard_normal((1, T, 3, 4)).astype(np.float32)
    w = g.standard_normal((1, T, 3)).astype(np.float32)
    wl = _wl(q, np.zeros((1, S, 4), np.float32), w, offset=offset, topk=k)
    idx, val, *_ = oracle.select(wl)
    for t in range(T):
        L = offset + t + 1
        m = min(k, L)
        assert list(idx[t]) == list(range(m)) + [-1] * (k - m)
        assert np.all(val[t, :m] == 0)


@pytest.mark.parametrize("offset", [0, 20])
def test_increasing_scores_pick_last_visible(offset):
    # score(t,s) = sum_h 0.5 * scale[s] with a strictly increasing scale:
    # the top-k are the last min(k, L) visible keys. Pins the causal bound
    # (s <= offset + t, inclusive) and that the per-token scale is applied.
    T, H, D, k = 12, 4, 8, 5
    S = T + offset
    scale = 1.0 + np.arange(S) * 2.0 ** -20
    wl = _fp8_ramp(T, S, H, D, scale, offset)
    wl.topk = k
    idx, val, *_ = oracle.select(wl)
    for t in range(T):
        L = offset + t + 1
        m = min(k, L)
        assert list(idx[t, :m]) == list(range(L - m, L))
        assert np.all(idx[t, m:] == -1)
        assert np.allclose(val[t, :m], 0.5 * H * scale[L - m:L], rtol=0, atol=0)


def test_decreasing_scores_pick_first():
    T, H, D, k = 10, 2, 4, 3
    scale = 2.0 - np.arange(T) * 2.0 ** -20
    wl = _fp8_ramp(T, T, H, D, scale)
    wl.topk = k
    idx, *_ = oracle.select(wl)
    for t in range(T):
        m = min(k, t + 1)
        assert list(idx[t, :m]) == list(range(m))


def test_h1_d1_reduces_to_lexsort():
    # H=1, D=1, w=1: score = max(0, q*k). The selection equals numpy's
    # lexsort on (index asc within score desc).
    g = np.random.Generator(np.random.PCG64(5))
    T = S = 64
    q = g.integers(-3, 4, (1, T, 1, 1)).astype(np.float32)
    k = g.integers(-5, 6, (1, S, 1)).astype(np.float32)
    w = np.ones((1, T, 1), np.float32)
    topk = 7
    idx, *_ = oracle.select(_wl(q, k, w, topk=topk))
    for t in range(T):
        L = t + 1
        sc = np.maximum(0.0, q[0, t, 0, 0] * k[0, :L, 0].astype(np.float64))
        order = np.lexsort((np.arange(L), -sc))[:min(topk, L)]
        exp = sorted(order.tolist())
        assert list(idx[t, :len(exp)]) == exp


def test_relu_is_per_head_and_weight_after_relu():
    # H=2, D=1, q=(1,-1), w=(1,1): score = max(0,k) + max(0,-k) = |k|.
    # Dropping the ReLU would make every score 0 (then the first k win).
    # w=(2,-1), q=(1,1): score = max(0,k); putting w inside the ReLU would
    # give 2*max(0,k) + max(0,-k) instead.
    g = np.random.Generator(np.random.PCG64(9))
    S = 40
    k = g.permutation(np.arange(-20, 20)).astype(np.float32).reshape(1, S, 1)
    q = np.tile(np.array([1.0, -1.0], np.float32).reshape(1, 1, 2, 1), (1, S, 1, 1))
    w = np.ones((1, S, 2), np.float32)
    idx, *_ = oracle.select(_wl(q, k, w, topk=5), rows=[S - 1])
    exp = sorted(np.lexsort((np.arange(S), -np.abs(k[0, :, 0])))[:5].tolist())
    assert list(idx[0]) == exp
    q2 = np.ones((1, S, 2, 1), np.float32)
    w2 = np.tile(np.array([2.0, -1.0], np.float32).reshape(1, 1, 2), (1, S, 1))
    idx2, val2, *_ = oracle.select(_wl(q2, k, w2, topk=25), rows=[S - 1])
    sc = np.maximum(0.0, k[0, :, 0])
    exp2 = sorted(np.lexsort((np.arange(S), -sc))[:25].tolist())
    assert list(idx2[0]) == exp2


def test_negative_weights_zero_ties():
    # H=1, D=1, q=1, w=-1: score = -max(0,k): 0 (in fact -0.0) for k <= 0 and
    # -k below that. Zeros must tie with each other regardless of sign and
    # go to the lowest indices first.
    k = np.array([3, -1, 0, 2, -4, 1, -2, 5], np.float32).reshape(1, 8, 1)
    q = np.ones((1, 8, 1, 1), np.float32)
    w = -np.ones((1, 8, 1), np.float32)
    idx, val, *_ = oracle.select(_wl(q, k, w, topk=6), rows=[7])
    # zeros at 1,2,4,6 ; then -1 (s5), -2 (s3)
    assert list(idx[0]) == [1, 2, 3, 4, 5, 6]
    idx, *_ = oracle.select(_wl(q, k, w, topk=2), rows=[7])
    assert list(idx[0]) == [1, 2]


def test_short_rows_are_padded():
    g = np.random.Generator(np.random.PCG64(4))
    T = 6
    q = g.standard_normal((1, T, 2, 3)).astype(np.float32)
    k = g.standard_normal((1, T, 3)).astype(np.float32)
    w = g.standard_normal((1, T, 2)).astype(np.float32)
    idx, val, *_ = oracle.select(_wl(q, k, w, topk=8))
    for t in range(T):
        assert sorted(idx[t, :t + 1].tolist()) == list(range(t + 1))
        assert np.all(idx[t, t + 1:] == -1) and np.all(np.isnan(val[t, t + 1:]))


# --------------------------------------------------------------------------- brute force

def _brute(q, k, w, offset, topk, scale=None):
    """Exact rational arithmetic, plain loops."""
    B, T, H, D = q.shape
    out = []
    for b in range(B):
        for t in range(T):
            L = offset + t + 1
            sc = []
            for s in range(L):
                tot = Fraction(0)
                for h in range(H):
                    dot = Fraction(0)
                    for d in range(D):
                        kv = Fraction(float(k[b, s, d]))
                        if scale is not None:
                            kv *= Fraction(float(scale[b, s]))
                        dot += Fraction(float(q[b, t, h, d])) * kv
                    tot += Fraction(float(w[b, t, h])) * max(Fraction(0), dot)
                sc.append((tot, s))
            sel = sorted(sc, key=lambda x: (-x[0], x[1]))[:topk]
            out.append((sorted(s for _, s in sel), {s: v for v, s in sc}))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_matches_exact_brute_force(seed):
    g = np.random.Generator(np.random.PCG64(100 + seed))
    B = int(g.integers(1, 3))
    T = int(g.integers(1, 7))
    offset = int(g.integers(0, 5))
    S = T + offset + int(g.integers(0, 3))
    H = int(g.integers(1, 4))
    D = int(g.integers(1, 6))
    topk = int(g.choice([1, 2, 3, 7]))
    integer = seed % 2 == 0
    if integer:
        q = g.integers(-3, 4, (B, T, H, D)).astype(np.float32)
        k = g.integers(-3, 4, (B, S, D)).astype(np.float32)
        w = g.choice([0.5, 1.0, 2.0, -1.0], (B, T, H)).astype(np.float32)
    else:
        q = (g.standard_normal((B, T, H, D))).astype(np.float32)
        k = (g.standard_normal((B, S, D))).astype(np.float32)
        w = g.standard_normal((B, T, H)).astype(np.float32)
    wl = _wl(q, k, w, offset=offset, topk=topk)
    idx, val, kth, rms, _ = oracle.select(wl)
    ref = _brute(q, k, w, offset, topk)
    for r, (sel, scores) in enumerate(ref):
        got = [i for i in idx[r] if i >= 0]
        assert got == sel, (r, got, sel)
        for j, s in enumerate(got):
            assert val[r, j] == pytest.approx(float(scores[s]), rel=1e-12, abs=1e-12)


def test_fp8_matches_exact_brute_force():
    g = np.random.Generator(np.random.PCG64(77))
    B, T, H, D, offset, topk = 2, 5, 3, 6, 3, 4
    S = T + offset
    q16 = W.to_bf16_bits(g.standard_normal((B, T, H, D)).astype(np.float32))
    codes, scale = W.quantize_e4m3_per_token(g.standard_normal((B, S, D)).astype(np.float32))
    w = g.standard_normal((B, T, H)).astype(np.float32)
    wl = _wl(q16, codes, w, k_scale=scale, q_dtype=W.BF16, k_dtype=W.FP8, offset=offset,
             topk=topk)
    idx, val, *_ = oracle.select(wl)
    lut = np.array([oracle.e4m3_decode(c) for c in range(256)])
    kdec = lut[codes]
    ref = _brute(W.bf16_bits_to_f32(q16), kdec, w, offset, topk, scale=scale)
    for r, (sel, scores) in enumerate(ref):
        assert [i for i in idx[r] if i >= 0] == sel


# --------------------------------------------------------------------------- invariants

def test_invariants_and_metamorphic_relations():
    g = np.random.Generator(np.random.PCG64(21))
    B, T, H, D, offset, topk = 2, 24, 5, 7, 30, 16
    S = T + offset
    q = g.standard_normal((B, T, H, D)).astype(np.float32)
    k = g.standard_normal((B, S, D)).astype(np.float32)
    w = g.standard_normal((B, T, H)).astype(np.float32)
    wl = _wl(q, k, w, offset=offset, topk=topk)
    idx, val, kth, rms, _ = oracle.select(wl)
    for r in range(B * T):
        t = r % T
        L = offset + t + 1
        sel = idx[r][idx[r] >= 0]
        assert len(sel) == min(topk, L)
        assert np.all(np.diff(sel) > 0) and sel.max() <= offset + t
        allsc = oracle.score_pairs(wl, np.full(L, r), np.arange(L))
        chosen = np.zeros(L, bool)
        chosen[sel] = True
        if (~chosen).any():
            assert allsc[~chosen].max() <= allsc[chosen].min()
            tie = allsc[chosen].min()
            # equal scores: every selected index below every unselected one
            if np.any(allsc[~chosen] == tie):
                assert np.where(chosen & (allsc == tie))[0].max() < \
                    np.where(~chosen & (allsc == tie))[0].min()
        assert rms[r] == pytest.approx(np.sqrt(np.mean(allsc ** 2)), rel=1e-12)
    # head permutation changes nothing
    perm = g.permutation(H)
    idx_p, val_p, *_ = oracle.select(_wl(q[:, :, perm], k, w[:, :, perm], offset=offset,
                                         topk=topk))
    assert np.array_equal(idx_p, idx)
    assert np.allclose(val_p, val, rtol=1e-12, equal_nan=True)
    # w * 2 doubles the scores, indices unchanged
    idx_2, val_2, *_ = oracle.select(_wl(q, k, w * 2, offset=offset, topk=topk))
    assert np.array_equal(idx_2, idx)
    assert np.allclose(val_2, 2 * val, rtol=1e-12, equal_nan=True)
    # keys beyond the causal horizon change nothing
    k_more = np.concatenate([k, g.standard_normal((B, 9, D)).astype(np.float32) * 50], 1)
    idx_m, *_ = oracle.select(_wl(q, k_more, w, offset=offset, topk=topk))
    assert np.array_equal(idx_m, idx)


def test_chunked_equals_unchunked():
    # Row t of a chunk with offset_c = offset + t0 is the same row as in the
    # unchunked problem: query t0+j sees keys <= offset + t0 + j.
    wl = W.prefill_fp8(seed=8, T=96, S=96, H=4, D=16, topk=10, chunk=32)
    idx, *_ = oracle.select(wl)
    for (t0, tc, sc, oc) in wl.chunks:
        sub = W.Workload("c", wl.q[:, t0:t0 + tc], wl.k[:, :sc], wl.k_scale[:, :sc],
                         wl.w[:, t0:t0 + tc], 1, tc, sc, wl.H, wl.D, oc, wl.topk, wl.q_dtype,
                         wl.k_dtype, [(0, tc, sc, oc)])
        idx_c, *_ = oracle.select(sub)
        assert np.array_equal(idx_c, idx[t0:t0 + tc])


def test_integer_config_scores_are_exact_halves():
    wl = W.tiny(T=64, S=64)
    idx, val, *_ = oracle.select(wl)
    v = val[~np.isnan(val)]
    assert np.all(v * 2 == np.round(v * 2))
    assert np.all(np.abs(v) <= 4 * 2 * 64 * 9)


def test_fp64_query_path_equals_fp32_path():
    # queries given as exact doubles (the fp8 x fp8 scorer's dequantised
    # queries) reduce to the pinned fp32 path on fp32-representable values
    wl = W.tiny(seed=5, T=64, S=64)
    a = oracle.select(wl)
    q64 = W.Workload(wl.name, wl.q.astype(np.float64), wl.k, wl.k_scale, wl.w, wl.B, wl.T, wl.S, wl.H, wl.D,
                     wl.offset, wl.topk, 3, wl.k_dtype, wl.chunks)
    b = oracle.select(q64)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
