"""The allocation-free select (ds4idx_select_noalloc) through the C ABI
against ds4idx_select with its own workspace: the same kernels, so indices and
values must be identical bit for bit. Several calls in a row on the one
per-GPU scratch array, each smaller than the one before, so that stale
counters or lists of an earlier call would show."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_token_lightning_amd as ds
import workloads as W
from parity import check_invariants, to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _both(wl, topk=None):
    topk = wl.topk if topk is None else topk
    q, k, ks, w = to_device(wl)
    ref_i, ref_v = ds.select(q, k, ks, w, wl.offset, topk)
    idx = torch.full((wl.B, wl.T, topk), 0x7F7F7F7F, dtype=torch.int32, device="cuda")
    vals = torch.full((wl.B, wl.T, topk), float("nan"), dtype=torch.float32, device="cuda")
    ds.select_noalloc(q, k, ks, w, wl.offset, idx, vals)
    torch.cuda.synchronize()
    return (ref_i.cpu().numpy(), ref_v.cpu().numpy()), (idx.cpu().numpy(), vals.cpu().numpy())


@pytest.mark.parametrize("seq", ["decode", "mixed"])
def test_noalloc_equals_select_calls_in_a_row(seq):
    if seq == "decode":
        # split-key kernel both times; the second call has fewer rows and keys
        calls = [W.decode(seed=81, B=6, S=200000, topk=512), W.decode(seed=82, B=2, S=30000, topk=512)]
    else:
        # k = 2048 lists, then a prefill-kernel problem (no scratch), then a
        # small split-key one after it
        calls = [W.decode(seed=83, B=2, S=262144, topk=2048),
                 W.prefill_fp8(seed=84, T=1024, S=3000, offset=1976, topk=512, chunk=1024),
                 W.prefill_bf16(seed=85, T=3, S=9000, offset=8997, topk=100)]
    for n, wl in enumerate(calls):
        _say(f"noalloc {seq} call {n}: B={wl.B} T={wl.T} S={wl.S} offset={wl.offset} k={wl.topk}")
        (ri, rv), (gi, gv) = _both(wl)
        assert np.array_equal(gi, ri), f"call {n}: indices differ from ds4idx_select"
        assert np.array_equal(gv.view(np.uint32), rv.view(np.uint32)), f"call {n}: values differ"
        check_invariants(wl, gi.reshape(wl.B * wl.T, -1))


def test_noalloc_rejects_oversize_problem():
    # 64 decode rows at 1M keys need more than the scratch array holds
    q = torch.empty((64, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((64, 1, 128), dtype=torch.uint8, device="cuda")  # shape only; never read
    p = ds.Problem(64, 1, 1 << 20, 64, 128, (1 << 20) - 1, ds.BF16, ds.FP8_E4M3)
    assert ds.workspace_bytes(p, 512) > ds.NOALLOC_SCRATCH_BYTES
    idx = torch.empty((64, 1, 512), dtype=torch.int32, device="cuda")
    st = ds.lib().ds4idx_select_noalloc(ctypes.byref(p), ds._ptr(q), ds._ptr(k), ds._ptr(idx), ds._ptr(q), 512,
                                        ds._ptr(idx), None, None)
    assert st == ds.ERR_SCRATCH
