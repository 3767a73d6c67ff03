"""GPU parity of the fp8 x fp8 scorer (ds4idx_select_qfp8) through the C ABI.

The scorer computes the indexer on dequantised queries; its oracle is the
same CPU oracle fed those exact values (scale x E4M3 decode, in fp64). The
parity cost of quantising Q, i.e. how far the selection moves from the
bf16-query selection, is measured here and reported."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as ds
import workloads as W
from parity import check_invariants, compare_rows

pytestmark = pytest.mark.gpu
F64 = 3  # the oracle's fp64 query dtype


def _say(*a):
    print(*a, flush=True)


def _decode_table():
    t = np.array([oracle.e4m3_decode(c) for c in range(256)])
    t[np.isnan(t)] = 0.0
    return t


def dequantised(wl: W.Workload, codes, scale) -> W.Workload:
    q = _decode_table()[codes] * scale[..., None].astype(np.float64)
    return W.Workload(wl.name + "/qfp8", np.ascontiguousarray(q), wl.k, wl.k_scale, wl.w, wl.B, wl.T, wl.S,
                      wl.H, wl.D, wl.offset, wl.topk, F64, wl.k_dtype, wl.chunks, wl.integer_valued)


def run_qfp8(wl: W.Workload, codes, scale, topk=None):
    topk = wl.topk if topk is None else topk
    q8 = torch.from_numpy(codes).cuda()
    qs = torch.from_numpy(scale).cuda()
    k = torch.from_numpy(wl.k).cuda()
    ks = torch.from_numpy(wl.k_scale).cuda()
    w = torch.from_numpy(wl.w).cuda()
    idx = torch.full((wl.B, wl.T, topk), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    vals = torch.full((wl.B, wl.T, topk), float("nan"), dtype=torch.float32, device="cuda")
    for (t0, tc, sc, oc) in wl.chunks:
        ds.select_qfp8(q8[:, t0:t0 + tc].contiguous(), qs[:, t0:t0 + tc].contiguous(), k[:, :sc].contiguous(),
                       ks[:, :sc].contiguous(), w[:, t0:t0 + tc].contiguous(), oc, topk,
                       idx=idx[:, t0:t0 + tc], vals=vals[:, t0:t0 + tc])
    torch.cuda.synchronize()
    return idx.reshape(wl.B * wl.T, topk).cpu().numpy(), vals.reshape(wl.B * wl.T, topk).cpu().numpy()


def _int_fp8_workload(seed, T, S, offset):
    g = np.random.Generator(np.random.PCG64(seed))
    kv = g.integers(-4, 5, (1, S, 128)).astype(np.float32)
    k8 = torch.from_numpy(kv).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    w = np.array([0.5, 1.0, 2.0], np.float32)[g.integers(0, 3, (1, T, 64))]
    wl = W.Workload("int-fp8", np.zeros((1, T, 64, 128), np.float32), k8, np.ones((1, S), np.float32), w, 1, T, S,
                    64, 128, offset, 512, W.F32, W.FP8, [(0, T, S, offset)], integer_valued=True)
    codes, scale = W.integer_fp8_queries(seed + 1, 1, T, 64, 128)
    return wl, codes, scale


@pytest.mark.parametrize("T,S,offset", [(1024, 1024, 0), (300, 5000, 4700)])
def test_integer_values_exact(T, S, offset):
    wl, codes, scale = _int_fp8_workload(61, T, S, offset)
    _say(f"qfp8 integer T={T} S={S} offset={offset}")
    gi, gv = run_qfp8(wl, codes, scale)
    dq = dequantised(wl, codes, scale)
    check_invariants(dq, gi)
    rows = np.arange(T) if T <= 400 else np.unique(np.r_[0, 510, 511, 512, T - 1, np.arange(0, T, 37)])
    compare_rows(dq, rows, gi[rows], gv[rows], exact=True)


def test_prefill_chunk_matches_dequantised_oracle():
    # the last 4096-query chunk of the 64k workload: 4096 queries over 65536 keys
    wl = W.prefill_fp8(T=65536)
    last = W.Workload(wl.name, wl.q[:, -4096:], wl.k, wl.k_scale, wl.w[:, -4096:], 1, 4096, wl.S, wl.H, wl.D,
                      wl.S - 4096, wl.topk, wl.q_dtype, wl.k_dtype, [(0, 4096, wl.S, wl.S - 4096)])
    codes, scale = W.fp8_queries(last)
    _say("qfp8 64k last chunk, 24 sampled rows")
    gi, gv = run_qfp8(last, codes, scale)
    dq = dequantised(last, codes, scale)
    check_invariants(dq, gi)
    g = np.random.Generator(np.random.PCG64(62))
    rows = np.unique(np.r_[0, 4095, g.integers(0, 4096, 22)])
    compare_rows(dq, rows, gi[rows], gv[rows], exact=False)
    # parity cost: overlap with the exact selection from the bf16 queries
    oi, _, _, _, _ = oracle.select(last, rows=rows)
    recall = np.mean([len(set(gi[r]) & set(oi[n])) / 512.0 for n, r in enumerate(rows)])
    _say(f"qfp8 recall of the bf16-query top-512 over {len(rows)} rows: {recall:.4f}")
    # 0.968 measured on these rows (0.971 over all 65536 rows): the guard
    # sits just under it, so a scorer that loses a further 1-2% of the exact
    # selection fails
    assert recall > 0.955
