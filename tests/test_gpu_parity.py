"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every test names its workload, seed and shape in its id; inputs are seeded.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as ds
import workloads as W
from parity import check_invariants, compare_rows, run_select, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _impl_auto():
    prev = ds.set_impl("auto")
    yield
    ds.set_impl(prev)


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ fp8 codec

@pytest.mark.parametrize("impl", ["opt", "ref"])
def test_e4m3_decode_through_scorer(impl):
    # K row s holds code s in dim 0; q = +e0 (t=0) or -e0 (t=1) on head 0 only,
    # w = e_head0, scale 1: score(t, s) = max(0, +-decode(s)). Every OCP code
    # except the two NaNs is recovered exactly; the FNUZ reading would halve
    # them.
    ds.set_impl(impl)
    S, T, H, D = 256, 2, 64, 128
    k = np.zeros((1, S, D), np.uint8)
    k[0, :, 0] = np.arange(256)
    q = np.zeros((1, T, H, D), np.float32)
    q[0, 0, 0, 0], q[0, 1, 0, 0] = 1.0, -1.0
    w = np.zeros((1, T, H), np.float32)
    w[0, :, 0] = 1.0
    dev = (torch.from_numpy(q).to(torch.bfloat16).cuda(), torch.from_numpy(k).cuda(),
           torch.ones((1, S), dtype=torch.float32, device="cuda"), torch.from_numpy(w).cuda())
    sc = ds.score(*dev, causal_offset=S - T).cpu().numpy()[0]
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for code in range(256):
        if np.isnan(ref[code]):
            continue
        if code <= S - T:  # t = 0 sees s <= 254
            assert sc[0, code] == max(0.0, ref[code]), (code, sc[0, code], ref[code])
        assert sc[1, code] == max(0.0, -ref[code]), (code, sc[1, code], ref[code])
    assert sc[0, 255] == -np.inf


# ------------------------------------------------------------------ exact configs

def test_tiny_all_rows_exact():
    wl = W.tiny()
    _say("tiny T=S=1024 H=4 D=64 fp32 ints seed=1")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(wl.T), gi, gv, exact=True)


@pytest.mark.parametrize("impl", ["auto", "ref"])
def test_int_prefill_2k_all_rows_exact(impl):
    ds.set_impl(impl)
    wl = W.prefill_bf16_int(seed=102, T=2048, S=2048)
    _say(f"8k-int recipe at T=S=2048 seed=102 impl={impl}")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(wl.T), gi, gv, exact=True)


def test_int_prefill_8k_full_size_exact():
    wl = W.prefill_bf16_int()
    _say("8k-int T=S=8192 H=64 D=128 seed=102")
    gi, gv = run_select(wl)
    check_invariants(wl, gi)
    rows = W.sample_rows(wl, 96)
    compare_rows(wl, rows, gi[rows], gv[rows], exact=True)


# ------------------------------------------------------------------ float configs

def test_prefill_8k_bf16():
    wl = W.prefill_bf16()
    _say("8k T=S=8192 bf16 seed=2")
    gi, gv = run_select(wl)
    check_invariants(wl, gi)
    rows = W.sample_rows(wl, 96)
    swaps = compare_rows(wl, rows, gi[rows], gv[rows], exact=False)
    _say("near-tie swaps", swaps)


def test_prefill_64k_fp8_chunked():
    wl = W.prefill_fp8()
    _say("64k T=S=65536 fp8 K, 16 chunks of 4096, seed=3")
    gi, gv = run_select(wl)
    check_invariants(wl, gi)
    rows = W.sample_rows_per_chunk(wl, 4)  # 4 per chunk (first, last, 2 drawn) + rows 510..512
    assert len(rows) == 4 * len(wl.chunks) + 3 and rows[0] == 0 and rows[-1] == wl.T - 1
    swaps = compare_rows(wl, rows, gi[rows], gv[rows], exact=False)
    _say("near-tie swaps", swaps)


def test_decode_256k_fp8():
    wl = W.decode()
    _say("decode B=8 T=1 S=262144 fp8 K seed=4")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    swaps = compare_rows(wl, np.arange(wl.B), gi, gv, exact=False)
    _say("near-tie swaps", swaps)


def test_long_prefill_1m_fp8():
    wl = W.long_prefill()
    _say("1m T=2048 S=1048576 offset=1046528 fp8 K seed=5")
    gi, gv = run_select(wl)
    check_invariants(wl, gi)
    rows = W.sample_rows(wl, 64)  # rows 0 and 2047 plus 62 drawn
    assert len(rows) == 64 and rows[0] == 0 and rows[-1] == wl.T - 1
    swaps = compare_rows(wl, rows, gi[rows], gv[rows], exact=False)
    _say("near-tie swaps", swaps)


# ------------------------------------------------------------------ edge cases

@pytest.mark.parametrize("T,offset,extra,topk,B", [
    (13, 0, 0, 512, 1),      # ragged tail, all rows shorter than k
    (37, 600, 5, 512, 2),    # ragged, offset, keys beyond the horizon, batch 2
    (9, 100, 0, 1, 1),       # k = 1
    (21, 3000, 0, 7, 1),     # small k, long rows
    (64, 511, 0, 512, 1),    # rows of exactly k keys at the first query
    (8, 4000, 100, 100, 3),  # batch 3
])
def test_edge_shapes_fp8(T, offset, extra, topk, B):
    wl = W.prefill_fp8(seed=31 + T, T=T, S=T + offset + extra, offset=offset, topk=topk, B=B,
                       chunk=T)
    wl.chunks = [(0, T, wl.S, offset)]  # the whole cache, including keys past the horizon
    _say(f"edge fp8 B={B} T={T} offset={offset} extra={extra} k={topk}")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(wl.B * wl.T), gi, gv, exact=False)


def test_all_equal_scores_tie_break():
    # K = 0: every score is exactly 0; the answer is {0..min(k,L)-1}.
    wl = W.prefill_bf16(seed=5, T=40, S=1200, offset=1160, topk=512)
    wl.k[:] = 0
    gi, gv = run_select(wl)
    for r in range(wl.T):
        L = wl.offset + r + 1
        assert list(gi[r, :min(512, L)]) == list(range(min(512, L)))
        assert np.all(gv[r, :min(512, L)] == 0)


@pytest.mark.parametrize("direction", [1, -1])
def test_monotone_rows_stress_streaming(direction):
    # Scores strictly monotone in s: rising rows admit every key (the most
    # buffer refills), falling rows admit almost none after the first k.
    T, S = 16, 20000
    off = S - T
    q = np.zeros((1, T, 64, 128), np.float32)
    q[..., 0] = 1.0
    k = np.full((1, S, 128), 0x38, np.uint8)   # E4M3 1.0 in every dim
    scale = (1.0 + direction * np.arange(S) * 2.0 ** -20).astype(np.float32).reshape(1, S)
    w = np.full((1, T, 64), 0.5, np.float32)
    wl = W.Workload("mono", W.to_bf16_bits(q), k, scale, w, 1, T, S, 64, 128, off, 512, W.BF16,
                    W.FP8, [(0, T, S, off)])
    gi, gv = run_select(wl)
    for t in range(T):
        L = off + t + 1
        exp = list(range(L - 512, L)) if direction > 0 else list(range(512))
        assert list(gi[t]) == exp


def test_negative_weights_zero_ties():
    # w < 0 everywhere: every score <= 0, many exactly 0 (some -0.0). Zeros tie.
    wl = W.prefill_bf16_int(seed=9, T=24, S=3000, offset=2976, topk=512)
    wl.w[:] = -np.abs(wl.w)
    gi, gv = run_select(wl)
    compare_rows(wl, np.arange(wl.T), gi, gv, exact=True)


# ------------------------------------------------------------------ consistency

@pytest.mark.parametrize("T", [1024, 300])
def test_fused_equals_score_then_topk(T):
    # T=1024 runs the prefill kernel, whose scorer arithmetic is that of
    # ds4idx_score: bit-identical. T=300 runs the split-key kernel, which sums
    # the same products in another order: equal up to fp32 rounding.
    wl = W.prefill_fp8(seed=12, T=T, S=5000, offset=5000 - T, chunk=T)
    q, k, ks, w = to_device(wl)
    idx, vals = ds.select(q, k, ks, w, wl.offset, 512)
    sc = ds.score(q, k, ks, w, wl.offset)
    idx2, vals2 = ds.topk(sc, 512, wl.offset)
    torch.cuda.synchronize()
    if T == 1024:
        assert torch.equal(idx, idx2)
        assert torch.equal(vals, vals2)
    else:
        # both paths against the oracle on every row
        rows = np.arange(wl.T)
        for name, (gi, gv) in (("fused", (idx, vals)), ("score+topk", (idx2, vals2))):
            gi = gi.reshape(wl.T, 512).cpu().numpy()
            gv = gv.reshape(wl.T, 512).cpu().numpy()
            check_invariants(wl, gi)
            swaps = compare_rows(wl, rows, gi, gv, exact=False)
            _say(f"T={T} {name}: near-tie swaps against the oracle {swaps}")
    # the scorer's masked region is -inf, the visible part finite
    lim = wl.offset + torch.arange(wl.T, device="cuda")
    cols = torch.arange(wl.S, device="cuda")
    masked = cols[None, :] > lim[:, None]
    assert torch.all(torch.isneginf(sc[0][masked]))
    assert torch.all(torch.isfinite(sc[0][~masked]))


def test_scorer_values_against_oracle():
    wl = W.prefill_fp8(seed=13, T=64, S=3000, offset=2936, chunk=64)
    sc = ds.score(*to_device(wl), causal_offset=wl.offset).cpu().numpy()[0]
    g = np.random.Generator(np.random.PCG64(0))
    rows = g.integers(0, wl.T, 400)
    keys = np.array([g.integers(0, wl.offset + r + 1) for r in rows])
    ref = oracle.score_pairs(wl, rows, keys)
    _, _, _, rms, _ = oracle.select(wl, rows=np.unique(rows))
    rmsd = dict(zip(np.unique(rows).tolist(), rms))
    tol = 1e-2 * np.maximum(np.abs(ref), np.array([rmsd[r] for r in rows]))
    assert np.all(np.abs(sc[rows, keys] - ref) <= tol)


def test_rollback_ref_matches_opt_on_integers():
    wl = W.prefill_bf16_int(seed=41, T=256, S=4096, offset=3840)
    dev = to_device(wl)
    ds.set_impl("opt")
    a, av = run_select(wl, dev=dev)
    ds.set_impl("ref")
    b, bv = run_select(wl, dev=dev)
    assert np.array_equal(a, b) and np.array_equal(av, bv)


def test_deterministic_repeat():
    wl = W.prefill_fp8(seed=14, T=512, S=20000, offset=19488, chunk=512)
    dev = to_device(wl)
    a, av = run_select(wl, dev=dev)
    b, bv = run_select(wl, dev=dev)
    assert np.array_equal(a, b) and np.array_equal(av.view(np.uint32), bv.view(np.uint32))


@pytest.mark.parametrize("impl", ["auto", "ref"])
def test_large_k(impl):
    # k = 1500 > 512: the split-key kernel (few rows) or the plain kernels.
    ds.set_impl(impl)
    wl = W.prefill_fp8(seed=15, T=20, S=30000, offset=29980, topk=1500, chunk=20)
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(wl.T), gi, gv, exact=False)


@pytest.mark.parametrize("B,T,S,offset,topk,kdt", [
    (3, 1, 20000, 19999, 512, "fp8"),     # partial last partition
    (2, 5, 8192 * 3, 8192 * 3 - 5, 512, "fp8"),  # several queries per stream, exact partitions
    (1, 2, 700, 698, 512, "fp8"),         # rows shorter than k
    (2, 3, 40000, 39997, 64, "bf16"),     # bf16 keys
    (4, 1, 9000, 8999, 1, "fp8"),         # k = 1
])
def test_split_kernel_shapes(B, T, S, offset, topk, kdt):
    if kdt == "fp8":
        wl = W.prefill_fp8(seed=60 + T, T=T, S=S, offset=offset, topk=topk, B=B, chunk=T)
    else:
        wl = W.prefill_bf16(seed=60 + T, T=T, S=S, offset=offset, topk=topk, B=B)
    wl.chunks = [(0, T, S, offset)]
    _say(f"split B={B} T={T} S={S} offset={offset} k={topk} {kdt}")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(B * T), gi, gv, exact=False)
    # three calls on one workspace: the arrival counters must return to zero
    q, k, ks, w = to_device(wl)
    ws = ds.new_workspace(ds.make_problem(q, k, offset), topk)
    for _ in range(3):
        idx, _v = ds.select(q, k, ks, w, offset, topk, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(idx.reshape(B * T, topk).cpu().numpy(), gi)


def test_split_int_exact():
    wl = W.prefill_bf16_int(seed=77, T=2, S=50000, offset=49998, topk=512, B=3)
    gi, gv = run_select(wl, poison=True)
    compare_rows(wl, np.arange(6), gi, gv, exact=True)


@pytest.mark.parametrize("lo,hi,kind", [(-4, 4, "fp8"), (-1, 1, "fp8"), (-1, 1, "bf16")])
def test_split_int_decode_ties_exact(lo, hi, kind):
    # Decode shape (one query per stream, 262144 keys: 32 partitions whose
    # short lists are merged). Integer values make every fp32 sum exact, so
    # the oracle's indices are the answer bit for bit. Values in [-1, 1] leave
    # few distinct scores, so the k-th score is shared by many keys spread
    # over many 64-slot chunks of the merge, and the ties kept must be the
    # lowest indices.
    wl = W.int_decode(seed=80 + hi, B=2, S=262144, lo=lo, hi=hi, kind=kind)
    _say(f"split integer decode ties [{lo}, {hi}] {kind}")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(2), gi, gv, exact=True)


@pytest.mark.parametrize("S", [100000, 300000])
def test_split_all_equal_scores(S):
    # K = 0 on a long cache with few rows (the split-key kernel): every score
    # is 0, so each partition's k-th key shares its bin with all 8192 keys
    # (exact partition selection), no short list fits, and at 300k keys the
    # merge holds more candidates than it stages (selection from the lists).
    B, T = 2, 2
    wl = W.prefill_fp8(seed=21, T=T, S=S, offset=S - T, topk=512, B=B, chunk=T)
    wl.chunks = [(0, T, S, S - T)]
    wl.k[:] = 0
    _say(f"split all-equal B={B} T={T} S={S}")
    gi, gv = run_select(wl, poison=True)
    assert np.array_equal(gi, np.tile(np.arange(512, dtype=gi.dtype), (B * T, 1)))
    assert np.all(gv == 0)


def test_split_hot_partition():
    # Partition 0 holds every one of the top k scores: its short list lies
    # above the row bound, so the merge must read the full candidate lists.
    # Scores are 32 * scale exactly (q = e_0, every key 1.0, w = 0.5) and
    # distinct, so the answer is the last k keys of partition 0.
    S = 40000
    q = np.zeros((1, 1, 64, 128), np.float32)
    q[..., 0] = 1.0
    k = np.full((1, S, 128), 0x38, np.uint8)
    s = np.arange(S)
    scale = np.where(s < 8192, 2.0 + s * 2.0 ** -20, 1.0 + s * 2.0 ** -20).astype(np.float32).reshape(1, S)
    w = np.full((1, 1, 64), 0.5, np.float32)
    wl = W.Workload("hot", W.to_bf16_bits(q), k, scale, w, 1, 1, S, 64, 128, S - 1, 512, W.BF16,
                    W.FP8, [(0, 1, S, S - 1)])
    _say("split hot partition S=40000")
    gi, gv = run_select(wl, poison=True)
    assert list(gi[0]) == list(range(8192 - 512, 8192))
    assert np.array_equal(gv[0], (32.0 * scale[0, 8192 - 512:8192]).astype(np.float32))


@pytest.mark.parametrize("S,topk,B", [
    (1048576, 512, 2),   # 128 partitions: the largest short-list grid the direct merge takes
    (262144, 2048, 2),   # k = 2048: short lists beyond one merge batch (the general path)
    (300000, 96, 3),     # partial last partition, small k
])
def test_split_long_cache_decode(S, topk, B):
    wl = W.decode(seed=40 + B, B=B, S=S, topk=topk)
    _say(f"split decode B={B} S={S} k={topk}")
    gi, gv = run_select(wl, poison=True)
    check_invariants(wl, gi)
    compare_rows(wl, np.arange(wl.B * wl.T), gi, gv, exact=False)


# ------------------------------------------------------------------ partition lengths

def _split_cases():
    c = {}
    c["decode B=3 S=100000"] = W.decode(seed=91, B=3, S=100000, topk=512)
    w = W.prefill_fp8(seed=92, T=5, S=40000, offset=39995, topk=512, chunk=5)
    w.chunks = [(0, 5, 40000, 39995)]
    c["fp8 T=5 S=40000"] = w
    w = W.prefill_bf16(seed=93, T=3, S=30001, offset=29998, topk=300, B=2)
    w.chunks = [(0, 3, 30001, 29998)]
    c["bf16 B=2 T=3 S=30001 k=300"] = w
    c["decode B=2 S=262144 k=2048"] = W.decode(seed=94, B=2, S=262144, topk=2048)
    w = W.decode(seed=95, B=2, S=50000, topk=512)
    w.k[:] = 0  # every score 0: exact partition selection, tie-break by index
    c["all-equal B=2 S=50000"] = w
    return c


@pytest.mark.parametrize("keys", [8192, 12288, 16384])
def test_split_partition_lengths_identical(keys):
    # Scores and the exact selection do not depend on how the keys are split,
    # so every partition length returns the same indices and values, bit for
    # bit, as the automatic choice (the first case is also checked against
    # the oracle).
    prev = ds.set_split(0)
    try:
        for n, (name, wl) in enumerate(_split_cases().items()):
            _say(f"split length {keys}: {name}")
            dev = to_device(wl)
            ds.set_split(0)
            ai, av = run_select(wl, dev=dev, poison=True)
            ds.set_split(keys)
            gi, gv = run_select(wl, dev=dev, poison=True)
            check_invariants(wl, gi)
            assert np.array_equal(gi, ai), f"{name}: indices differ between lengths"
            assert np.array_equal(gv.view(np.uint32), av.view(np.uint32)), f"{name}: values differ"
            if n == 0:
                compare_rows(wl, np.arange(wl.B * wl.T), gi, gv, exact=False)
    finally:
        ds.set_split(prev)


# ------------------------------------------------------------------ randomised shapes

def _random_case(g, case):
    kind = g.choice(["prefill", "long", "decode", "decode"])
    kdt = g.choice(["fp8", "bf16", "int"])
    topk = int(g.choice([1, 5, 64, 100, 257, 512, 512, 1024, 2048]))
    B = int(g.integers(1, 4))
    if kind == "prefill":
        T, offset = int(g.integers(1, 300)), int(g.integers(0, 20000 // B))
    elif kind == "long":  # long rows: several threshold raises per token
        T, offset = int(g.integers(1, 40)), int(g.integers(20000, 90000 // B))
    else:
        T, offset = int(g.integers(1, 4)), int(g.integers(500, 300000 // B))
    S, seed = offset + T, 5000 + case
    if kdt == "fp8":
        wl = W.prefill_fp8(seed=seed, T=T, S=S, offset=offset, topk=topk, B=B, chunk=T)
    elif kdt == "bf16":
        wl = W.prefill_bf16(seed=seed, T=T, S=S, offset=offset, topk=topk, B=B)
    else:
        wl = W.prefill_bf16_int(seed=seed, T=T, S=S, offset=offset, topk=topk, B=B)
    wl.chunks = [(0, T, S, offset)]
    return wl, f"{kind} {kdt} B={B} T={T} S={S} offset={offset} k={topk} seed={seed}"


@pytest.mark.parametrize("group", range(4))
def test_randomised_shapes(group):
    # 12 seeded cases per group: prefill-, long-row- and decode-shaped problems
    # (both hot kernels and every k path), E4M3, bf16 and integer keys; every
    # row against the oracle (bit for bit on integers).
    g = np.random.Generator(np.random.PCG64(900 + group))
    for case in range(12):
        wl, desc = _random_case(g, 12 * group + case)
        _say("random", desc)
        gi, gv = run_select(wl, poison=True)
        check_invariants(wl, gi)
        compare_rows(wl, np.arange(wl.B * wl.T), gi, gv, exact=wl.integer_valued)
