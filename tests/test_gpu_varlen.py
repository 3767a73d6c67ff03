"""GPU parity of ragged batches (ds4idx_select_varlen) through the C ABI:
every stream against the CPU oracle (bit-exact on integer inputs, within the
float tolerance otherwise), and against ds4idx_select on the same stream where
both calls take the same kernel (then bit-exact on any input)."""
import numpy as np
import pytest
import torch

import sparse_attention_token_lightning_amd as ds
import workloads as W
from parity import check_invariants, compare_rows, run_select, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _dev(rg: W.Ragged):
    q = torch.from_numpy(rg.q.view(np.int16)).view(torch.bfloat16).cuda()
    if rg.k_dtype == W.BF16:
        k = torch.from_numpy(rg.k.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        k = torch.from_numpy(rg.k).cuda()
    ks = None if rg.k_scale is None else torch.from_numpy(rg.k_scale).cuda()
    w = torch.from_numpy(rg.w).cuda()
    return (q, k, ks, w, torch.from_numpy(rg.cu_q).cuda(), torch.from_numpy(rg.cu_k).cuda())


def _max_k(rg):
    return int(np.diff(rg.cu_k).max())


def run_varlen(rg: W.Ragged, topk=None, dev=None, workspace=None, poison=True):
    topk = rg.topk if topk is None else topk
    q, k, ks, w, cq, ck = dev if dev is not None else _dev(rg)
    idx = torch.full((q.shape[0], topk), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    vals = torch.full((q.shape[0], topk), float("nan"), dtype=torch.float32, device="cuda")
    if not poison:
        idx.zero_()
        vals.zero_()
    ds.select_varlen(q, k, ks, w, cq, ck, _max_k(rg), topk, idx=idx, vals=vals, workspace=workspace)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), vals.cpu().numpy()


def _route_is_split(rg, topk):
    # with the prefill kernel's key parts off, only the split-key kernel needs
    # a workspace
    q, k, _, _, cq, ck = _dev(rg)
    p = ds.make_varlen_problem(q, k, cq, ck, _max_k(rg))
    prev = ds.set_prefill_split(-1)
    try:
        return ds.varlen_workspace_bytes(p, topk) > 0
    finally:
        ds.set_prefill_split(prev)


def _rows_for_oracle(T, n=16):
    if T <= n:
        return np.arange(T)
    g = np.random.Generator(np.random.PCG64(T))
    return np.unique(np.concatenate([[0, T - 1], g.integers(0, T, n - 2)]))


def check_against_oracle(rg: W.Ragged, gi, gv, exact: bool, topk=None, n=16):
    topk = rg.topk if topk is None else topk
    for b in range(rg.B):
        wl = rg.stream(b)
        if wl.T == 0:
            continue
        q0 = int(rg.cu_q[b])
        check_invariants(wl, gi[q0:q0 + wl.T], topk=topk)
        rows = _rows_for_oracle(wl.T, n)
        compare_rows(wl, rows, gi[q0 + rows], gv[q0 + rows], exact=exact, topk=topk)


def check_against_single_stream_calls(rg: W.Ragged, gi, gv, topk=None):
    topk = rg.topk if topk is None else topk
    for b in range(rg.B):
        wl = rg.stream(b)
        if wl.T == 0:
            continue
        q0 = int(rg.cu_q[b])
        si, sv = run_select(wl, topk=topk)
        np.testing.assert_array_equal(gi[q0:q0 + wl.T], si, err_msg=f"stream {b} indices")
        np.testing.assert_array_equal(gv[q0:q0 + wl.T], sv, err_msg=f"stream {b} values")


DECODE_MIX = [(1, 1), (1, 100), (1, 511), (1, 512), (1, 513), (0, 77), (1, 8191), (1, 8192),
              (1, 8193), (3, 70000), (1, 262144), (1, 300000), (2, 5)]
PREFILL_MIX = [(700, 700), (1, 20000), (300, 9000), (0, 50), (129, 129), (5, 4099), (17, 60000)]


# The two ragged batches bench.py times, at their full shapes (the same
# recipe; bench.py carves its bytes from the decode and 64k workloads).
BENCH_DECODE_MIX = [(1, 4096 + 910 * b) for b in range(64)]
BENCH_PREFILL_MIX = [(1024, 32768), (512, 16384), (256, 8192), (256, 8192)]


def test_bench_ragged_decode_mix():
    # 64 streams x 1 query, 2,096,704 keys in all: the split-key kernel with
    # more partitions than CUs
    rg = W.ragged(47, BENCH_DECODE_MIX)
    assert _route_is_split(rg, rg.topk)
    _say("ragged decode, the bench mix: 64 streams of 4096 + 910 b keys, seed=47")
    gi, gv = run_varlen(rg)
    check_against_single_stream_calls(rg, gi, gv)
    check_against_oracle(rg, gi, gv, exact=False)


def test_bench_ragged_prefill_mix():
    # a 2048-token budget: 1024/512/256/256 new tokens on caches of
    # 32768/16384/8192/8192 keys, one prefill-kernel launch
    rg = W.ragged(48, BENCH_PREFILL_MIX)
    assert not _route_is_split(rg, rg.topk)
    _say("ragged prefill, the bench mix: 2048 tokens over 4 streams, seed=48")
    gi, gv = run_varlen(rg)
    check_against_oracle(rg, gi, gv, exact=False, n=16)


def test_ragged_decode_batch_fp8():
    # few rows: the split-key kernel. Each stream equals its own ds4idx_select
    # call (same kernel) bit for bit, and the oracle within tolerance.
    rg = W.ragged(41, DECODE_MIX)
    assert _route_is_split(rg, rg.topk)
    _say(f"ragged decode fp8 seed=41 streams={DECODE_MIX}")
    gi, gv = run_varlen(rg)
    check_against_single_stream_calls(rg, gi, gv)
    check_against_oracle(rg, gi, gv, exact=False)


def test_ragged_decode_batch_int_exact():
    rg = W.ragged(42, DECODE_MIX, kind="int")
    _say(f"ragged decode int seed=42 streams={DECODE_MIX}")
    gi, gv = run_varlen(rg)
    check_against_oracle(rg, gi, gv, exact=True)


def test_ragged_decode_k1024():
    mix = [(1, 300), (1, 1023), (1, 1024), (1, 1025), (2, 50000), (1, 200000)]
    rg = W.ragged(43, mix, topk=1024)
    _say(f"ragged decode k=1024 seed=43 streams={mix}")
    gi, gv = run_varlen(rg, topk=1024)
    check_against_single_stream_calls(rg, gi, gv, topk=1024)
    check_against_oracle(rg, gi, gv, exact=False, topk=1024)


def test_ragged_prefill_batch_fp8():
    # many rows: the prefill kernel, streams of every size mixed
    rg = W.ragged(44, PREFILL_MIX)
    assert not _route_is_split(rg, rg.topk)
    _say(f"ragged prefill fp8 seed=44 streams={PREFILL_MIX}")
    gi, gv = run_varlen(rg)
    check_against_oracle(rg, gi, gv, exact=False)


def test_ragged_prefill_batch_int_exact():
    rg = W.ragged(45, PREFILL_MIX, kind="int")
    _say(f"ragged prefill int seed=45 streams={PREFILL_MIX}")
    gi, gv = run_varlen(rg)
    check_against_oracle(rg, gi, gv, exact=True, n=64)


def test_ragged_prefill_bf16_keys_and_long_streams_match_single_calls():
    # streams long enough that their own ds4idx_select also takes the prefill
    # kernel: bit-identical outputs
    mix = [(1024, 1024), (2048, 6000), (1100, 1100), (0, 10)]
    rg = W.ragged(46, mix, kind="bf16")
    _say(f"ragged prefill bf16 seed=46 streams={mix}")
    gi, gv = run_varlen(rg)
    check_against_single_stream_calls(rg, gi, gv)
    check_against_oracle(rg, gi, gv, exact=False)


def test_uniform_decode_as_ragged_is_identical():
    # the 256k decode problem (8 streams x 1 query x 262144 keys) written as a
    # ragged batch gives the uniform call's outputs bit for bit
    wl = W.decode()
    _say("uniform decode 8 x 262144 as a ragged batch")
    dev = to_device(wl)
    ui, uv = run_select(wl, dev=dev)
    q, k, ks, w = dev
    cq = torch.arange(0, wl.B + 1, dtype=torch.int32, device="cuda")
    ck = torch.arange(0, wl.B + 1, dtype=torch.int64, device="cuda") * wl.S
    idx, vals = ds.select_varlen(q.reshape(wl.B, wl.H, wl.D), k.reshape(wl.B * wl.S, wl.D),
                                 ks.reshape(-1), w.reshape(wl.B, wl.H), cq, ck, wl.S, wl.topk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ui)
    np.testing.assert_array_equal(vals.cpu().numpy(), uv)


def test_workspace_reuse_across_ragged_batches():
    a = W.ragged(47, DECODE_MIX)
    b = W.ragged(48, [(1, 40000), (2, 9000), (1, 300000), (1, 64)])
    _say("ragged workspace reuse")
    da, db = _dev(a), _dev(b)
    n = max(ds.varlen_workspace_bytes(ds.make_varlen_problem(d[0], d[1], d[4], d[5], _max_k(r)), 512)
            for r, d in ((a, da), (b, db)))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    first = run_varlen(a, dev=da, workspace=ws)
    other = run_varlen(b, dev=db, workspace=ws)
    again = run_varlen(a, dev=da, workspace=ws)
    np.testing.assert_array_equal(first[0], again[0])
    np.testing.assert_array_equal(first[1], again[1])
    check_against_oracle(b, other[0], other[1], exact=False)


@pytest.mark.parametrize("keys", [8192, 12288, 16384])
def test_ragged_partition_lengths_identical(keys):
    # The ragged decode mixes under every partition length return what the
    # automatic choice returns (12288 for the bench mix), bit for bit.
    prev = ds.set_split(0)
    try:
        for name, mix, seed in (("bench decode mix", BENCH_DECODE_MIX, 47), ("decode mix", DECODE_MIX, 41)):
            rg = W.ragged(seed, mix)
            dev = _dev(rg)
            _say(f"ragged {name}, partition length {keys}")
            ds.set_split(0)
            ai, av = run_varlen(rg, dev=dev)
            ds.set_split(keys)
            gi, gv = run_varlen(rg, dev=dev)
            assert np.array_equal(gi, ai), f"{name}: indices differ between lengths"
            assert np.array_equal(gv.view(np.uint32), av.view(np.uint32)), f"{name}: values differ"
    finally:
        ds.set_split(prev)


PARTS_MIX = [(300, 8000), (40, 3000), (1, 7999), (64, 64), (9, 6001)]


@pytest.mark.parametrize("keys", [0, 2048, 5000])
def test_ragged_prefill_key_parts_identical(keys):
    # Splitting an 8-token block's keys into parts changes neither the
    # scores nor the exact selection: the parted launch returns the unsplit
    # launch's indices and values bit for bit, and matches the oracle
    # (exactly on integer inputs). With 2048-key parts the 8000-key stream
    # takes 4 parts, the 3000-key one 2, the 64-key one 1.
    prev = ds.get_prefill_split()
    try:
        cases = [("bench prefill mix", BENCH_PREFILL_MIX, 48, "fp8"), ("parts mix", PARTS_MIX, 49, "fp8"),
                 ("parts mix int", PARTS_MIX, 50, "int"), ("parts mix bf16", PARTS_MIX, 51, "bf16")]
        for name, mix, seed, kind in cases:
            rg = W.ragged(seed, mix, kind=kind)
            dev = _dev(rg)
            _say(f"ragged prefill key parts {keys}: {name} ({kind})")
            ds.set_prefill_split(-1)
            ri, rv = run_varlen(rg, dev=dev)
            ds.set_prefill_split(keys)
            gi, gv = run_varlen(rg, dev=dev)
            assert np.array_equal(gi, ri), f"{name}: indices differ with key parts"
            assert np.array_equal(gv.view(np.uint32), rv.view(np.uint32)), f"{name}: values differ with key parts"
            if name != "bench prefill mix" or keys == 0:
                check_against_oracle(rg, gi, gv, exact=(kind == "int"), n=8)
    finally:
        ds.set_prefill_split(prev)


PLAN_CASES = [
    ("110 short streams", [(1, 300 + 37 * b) for b in range(110)], 512, 61),
    ("one long stream, 50 short", [(1, 1_000_000)] + [(1, 1000 + 13 * b) for b in range(50)], 512, 62),
    ("k = 2048", [(1, 40000 + 1000 * b) for b in range(24)], 2048, 63),
    ("several queries per stream", [(5, 9000), (1, 120000), (12, 40000), (1, 513), (0, 10), (3, 3)], 512, 64),
]


@pytest.mark.parametrize("name,mix,topk,seed", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_planned_parts_match_fixed_length(name, mix, topk, seed):
    # With the automatic length a batch of at most 256 rows takes parts
    # planned on the device (equal parts per row, the shortest length whose
    # parts start in one round); a fixed length takes the plain partitions.
    # Both select exactly, so they agree bit for bit; rows against the oracle.
    rg = W.ragged(seed, mix, topk=topk)
    assert _route_is_split(rg, topk)
    dev = _dev(rg)
    prev = ds.set_split(0)
    try:
        _say(f"planned parts: {name}, k={topk}")
        ai, av = run_varlen(rg, topk=topk, dev=dev)
        ds.set_split(16384)
        gi, gv = run_varlen(rg, topk=topk, dev=dev)
    finally:
        ds.set_split(prev)
    assert np.array_equal(ai, gi), f"{name}: indices differ from the fixed length"
    assert np.array_equal(av.view(np.uint32), gv.view(np.uint32)), f"{name}: values differ"
    check_against_oracle(rg, ai, av, exact=False, topk=topk, n=4)


@pytest.mark.parametrize("group", range(2))
def test_randomised_ragged_batches(group):
    # 10 seeded random stream mixes per group: empty streams, single tokens on
    # long caches and prefill-like streams in one batch; E4M3, bf16 and integer
    # keys; k from 1 to 2048. Every stream's invariants, and up to 24 rows per
    # stream against the oracle (bit for bit on integers). (A mixed batch runs
    # on one kernel for all its streams, so its values can differ from a
    # single-stream call by fp32 rounding: the oracle is the reference here.)
    g = np.random.Generator(np.random.PCG64(700 + group))
    for case in range(10):
        streams = []
        for _ in range(int(g.integers(1, 24))):
            T = int(g.choice([0, 1, 1, 2, int(g.integers(1, 200))]))
            streams.append((T, T + int(g.integers(0, 90000 if T <= 2 else 30000))))
        if sum(t for t, _ in streams) == 0:
            streams[0] = (1, max(1, streams[0][1]))
        kind = str(g.choice(["fp8", "int", "bf16"]))
        topk = int(g.choice([1, 64, 300, 512, 512, 2048]))
        rg = W.ragged(seed=7100 + 10 * group + case, streams=streams, topk=topk, kind=kind)
        _say(f"random ragged {kind} k={topk} streams={streams}")
        gi, gv = run_varlen(rg)
        check_against_oracle(rg, gi, gv, exact=(kind == "int"), n=24)

