"""Parity helpers: run the HIP path on a workload and compare with the oracle.

Comparison rules (the oracle is exact in fp64; the GPU accumulates in fp32):
* integer-valued workloads: every fp32 sum is exact, so index sets and values
  must match the oracle bit for bit;
* float workloads: values within a relative 1e-2 of max(|oracle|, row RMS),
  and index sets equal except for keys whose oracle score lies within that
  same tolerance of the oracle's k-th score (a swap across a near-tie).
Invariants checked on every GPU row: exactly min(k, L) indices, ascending,
unique, all <= offset + t, then -1 padding.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_attention_token_lightning_amd as ds
import workloads as W

RTOL = 1e-2


def to_device(wl: W.Workload, device="cuda"):
    if wl.q_dtype == W.BF16:
        q = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16)
    else:
        q = torch.from_numpy(wl.q)
    if wl.k_dtype == W.BF16:
        k = torch.from_numpy(wl.k.view(np.int16)).view(torch.bfloat16)
    else:
        k = torch.from_numpy(wl.k)
    ks = None if wl.k_scale is None else torch.from_numpy(wl.k_scale)
    w = torch.from_numpy(wl.w)
    return (q.to(device), k.to(device), None if ks is None else ks.to(device), w.to(device))


def run_select(wl: W.Workload, dev=None, topk=None, with_vals=True, poison=False):
    """All chunk calls of the workload through ds4idx_select; host arrays [B*T, k].
    Chunk c passes views: queries [t0, t0+T_c) and the first S_c cached keys."""
    topk = wl.topk if topk is None else topk
    q, k, ks, w = dev if dev is not None else to_device(wl)
    idx = torch.empty((wl.B, wl.T, topk), dtype=torch.int32, device=q.device)
    vals = torch.empty((wl.B, wl.T, topk), dtype=torch.float32, device=q.device) if with_vals else None
    if poison:
        idx.fill_(0x7F7F7F7F)
        if vals is not None:
            vals.fill_(float("nan"))
    assert len(wl.chunks) == 1 or wl.B == 1, "chunked workloads are single-stream"
    for (t0, tc, sc, oc) in wl.chunks:
        ds.select(q[:, t0:t0 + tc], k[:, :sc], None if ks is None else ks[:, :sc],
                  w[:, t0:t0 + tc], oc, topk, idx=idx[:, t0:t0 + tc],
                  vals=None if vals is None else vals[:, t0:t0 + tc], with_vals=with_vals)
    torch.cuda.synchronize()
    gi = idx.reshape(wl.B * wl.T, topk).cpu().numpy()
    gv = None if vals is None else vals.reshape(wl.B * wl.T, topk).cpu().numpy()
    return gi, gv


def visible(wl: W.Workload, rows: np.ndarray) -> np.ndarray:
    return wl.offset + (np.asarray(rows) % wl.T) + 1


def check_invariants(wl: W.Workload, gidx: np.ndarray, topk=None):
    topk = wl.topk if topk is None else topk
    rows = np.arange(gidx.shape[0])
    L = visible(wl, rows)
    m = np.minimum(L, topk)
    pos = np.arange(topk)[None, :]
    valid = pos < m[:, None]
    assert np.all(gidx[valid] >= 0), "missing index inside min(k, L)"
    assert np.all(gidx[~valid] == -1), "padding is not -1"
    lim = (wl.offset + rows % wl.T)[:, None]
    assert np.all(np.where(valid, gidx, -1) <= lim), "index beyond the causal limit"
    d = np.diff(gidx, axis=1)
    both = valid[:, 1:]
    assert np.all(d[both] > 0), "indices not strictly ascending"


def compare_rows(wl: W.Workload, rows, gidx, gvals, exact: bool, topk=None):
    """Compare GPU rows (aligned with `rows`) against the oracle. Returns the
    number of near-tie swaps (always 0 when exact)."""
    topk = wl.topk if topk is None else topk
    rows = np.asarray(rows, dtype=np.int64)
    oi, ov, kth, rms, _ = oracle.select(wl, rows=rows, topk=topk)
    swaps = 0
    for r in range(len(rows)):
        L = int(visible(wl, rows[r:r + 1])[0])
        m = min(L, topk)
        g = gidx[r, :m]
        o = oi[r, :m]
        assert np.all(gidx[r, m:] == -1)
        if exact:
            assert np.array_equal(g, o), f"row {rows[r]}: index sets differ"
            if gvals is not None:
                assert np.array_equal(gvals[r, :m].astype(np.float64), ov[r, :m]), \
                    f"row {rows[r]}: values differ"
            continue
        scale = max(abs(kth[r]), rms[r])
        gs, os_ = set(g.tolist()), set(o.tolist())
        diff = sorted(gs ^ os_)
        if diff:
            osc = oracle.score_pairs(wl, np.full(len(diff), rows[r]), np.array(diff))
            assert np.all(np.abs(osc - kth[r]) <= RTOL * scale), \
                f"row {rows[r]}: swapped keys are not near-ties of the k-th score"
            swaps += len(diff) // 2
        if gvals is not None:
            common = np.array(sorted(gs & os_), dtype=np.int64)
            gpos = np.searchsorted(g, common)
            opos = np.searchsorted(o, common)
            gv = gvals[r, gpos].astype(np.float64)
            refv = ov[r, opos]
            tol = RTOL * np.maximum(np.abs(refv), rms[r])
            assert np.all(np.abs(gv - refv) <= tol), f"row {rows[r]}: values out of tolerance"
    return swaps
