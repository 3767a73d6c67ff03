"""Benchmark: Lightning Indexer (score + top-512) on one MI355X.

One step = the 64k cold causal prefill: T = S = 65536 queries in 16 chunks of
4096 (chunk c: causal offset 4096c against the 4096(c+1) keys cached so far),
H = 64, D = 128, top-512, bf16 Q, OCP E4M3 K with per-token fp32 scale,
fp32 head weights, i.e. 16 ds4idx_select calls on one stream. Inputs are
seeded synthetic data resident in HBM before timing starts.

Printed (one JSON line): query-tok/s of the step, the roofline of the MFMA
select kernel (algorithmic bf16 flop per launch over its HIP-event-timed
average duration, against the 2.5 PFLOP/s dense bf16 peak), the 256k decode
latency (8 streams x 1 query x 262144 keys, rotated over 3 copies of the
inputs so the 256 MB last-level cache cannot hold them), and the CPU oracle
timed on a bounded sample of the same prefill rows. Also reported: the
key-cache writer (per-token E4M3 quantisation) filling the whole 256k decode
cache of 8 streams from bf16 keys, against the HBM peak; and two ragged
batches in one launch each (ds4idx_select_varlen): 64 decode streams whose
caches span 4096..61426 keys, and a 2048-token chunked-prefill budget spread
over four streams; and sparse attention (ds4idx_sparse_attention) of one
4096-query prefill chunk over 512 selected rows of a 65536-row latent cache,
64 heads, against the bf16 MFMA peak; and the fp8 x fp8 variant of the 64k
prefill (queries quantised per token and head by the key-cache writer, inside
the timed step), with its recall of the bf16-query selection over all rows; and
the remaining indexer workloads, one ds4idx_select call each: the tiny fp32
prefill (T = S = 1024, H = 4, D = 64), the 8k bf16 prefill and the 1M chunked
prefill (2048 queries after 1,046,528 cached E4M3 keys).

Before each timed 64k step a 512 MB buffer is written so the step starts
with a cold last-level cache (--no-flush to skip). Also reported: measured
ceilings in plain torch (HBM reads of 277 MB rotated over three copies by a sum
and by a library GEMV, a 277 MB device copy, an 8192^3 bf16 matmul) and from
the probe library's two kernels (a grid-stride read of the same bytes, an
MFMA-only loop), and the CPU oracle timed per workload with the host's
core count, CPU model and a one-thread rate.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "indexer query-tok/s at 64k causal prefill (score+top-512); decode µs at 256k"
BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
FP8_PEAK_TFLOPS = 5033.2    # dense fp8
HBM_PEAK_GBS = 8000.0


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-iters", type=int, default=60)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-writer", action="store_true")
    ap.add_argument("--no-ragged", action="store_true")
    ap.add_argument("--no-attention", action="store_true")
    ap.add_argument("--no-qfp8", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the tiny, 8k and 1M prefill workloads")
    ap.add_argument("--attention-iters", type=int, default=10)
    ap.add_argument("--warm-ms", type=float, default=30.0,
                    help="device time of the untimed calls queued before each per-call timed loop")
    ap.add_argument("--writer-iters", type=int, default=20)
    ap.add_argument("--no-cpu-configs", action="store_true",
                    help="skip the per-workload oracle timings (every row of the tiny, 8k, 8k-int and "
                         "decode workloads; sampled rows of the 64k and 1M prefills)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured ceilings (torch sum, GEMV and copy over 277 MB; bf16 matmul)")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not write a 512 MB buffer before each timed 64k step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 256 MiB once (the reference kernel that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    return ap.parse_args()


PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_attention_token_lightning_amd", "csrc")


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed, so an
    edit to comments or layout alone leaves the digest unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                   # string or char literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i) or text.startswith("/*", i) or c.isspace():
            if text.startswith("//", i):
                j = text.find("\n", i)
                i = n if j < 0 else j
            elif text.startswith("/*", i):
                j = text.find("*/", i + 2)
                i = n if j < 0 else j + 2
            else:
                i += 1
            if out and out[-1] != " ":                   # one space per gap outside literals
                out.append(" ")
        else:
            out.append(c)
            i += 1
    return "".join(out).strip()


def kernel_digest(src: str) -> str:
    import hashlib
    with open(os.path.join(CSRC, src), encoding="utf-8") as f:
        return hashlib.sha256(_code_only(f.read()).encode()).hexdigest()[:16]


def measured_traffic(summary: str = "mfma_select_64k_traffic.txt", src: str = "mfma_indexer.hip"):
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel's code (comments and layout aside) changed since the counters were
    taken."""
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256_16") != kernel_digest(src):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _to_device(wl, dev):
    """A workload's host arrays as device tensors (bf16 bits viewed as bf16)."""
    import numpy as np
    import torch

    import workloads as W

    def cv(a, dt):
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if dt == W.BF16 else torch.from_numpy(a)
        return t.to(dev)
    ks = None if wl.k_scale is None else torch.from_numpy(wl.k_scale).to(dev)
    return cv(wl.q, wl.q_dtype), cv(wl.k, wl.k_dtype), ks, torch.from_numpy(wl.w).to(dev)


def _probe_lib():
    """The ceiling probes' own library (outside the indexer's C ABI), or None
    if it was not built."""
    plib = os.path.join(os.path.dirname(CSRC), "libds4probe.so")
    if not os.path.exists(plib):
        return None
    probe = ctypes.CDLL(plib)
    probe.ds4probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p]
    probe.ds4probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.ds4probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p,
                                      ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return probe


def _time_calls(call, n: int, stream, warm_ms: float = 30.0):
    """Device time in microseconds, sorted, of n calls call(i) on `stream`.

    One untimed call gives the duration. Then enough untimed calls to fill about
    warm_ms of device time are queued right before the n timed ones, with no
    synchronisation between them. Queuing a call takes the host 10-20 us, less
    than any of these calls runs, so the device never waits for the host inside
    a timed event pair, and the timed calls run at the clocks of sustained load.
    (A spin kernel in place of the warm-up calls leaves the GPU near idle for its
    length, and the calls after it measured up to 12% slower while the clocks
    settled; their medians then disagreed with wall-clock time per call.)"""
    import math

    import torch
    call(0)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    call(1)
    e[1].record(stream)
    torch.cuda.synchronize()
    nwarm = max(2, min(2000, math.ceil(warm_ms / max(e[0].elapsed_time(e[1]), 1e-3))))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    for i in range(nwarm):
        call(2 + i)
    for j, x in enumerate(ev):
        x[0].record(stream)
        call(2 + nwarm + j)
        x[1].record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 for a, b in ev)


def _flops_64k(wl):
    """Algorithmic work of one step: 2*H*D flop per visible (query, key) pair;
    chunk c's query j (of T_c) sees offset_c + j + 1 keys."""
    pairs = sum(tc * oc + tc * (tc + 1) // 2 for (_, tc, _, oc) in wl.chunks)
    return 2 * wl.H * wl.D * pairs, pairs


def main():
    args = _parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the indexer path here runs on a single MI355X "
              "(rows shard across GPUs with no exchange; that path is not built). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import sparse_attention_token_lightning_amd as ds
    import workloads as W

    ds.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------------- 64k prefill
    wl = W.prefill_fp8()
    q = torch.from_numpy(wl.q.view(np.int16)).view(torch.bfloat16).to(dev)
    k = torch.from_numpy(wl.k).to(dev)
    ks = torch.from_numpy(wl.k_scale).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    idx = torch.empty((1, wl.T, wl.topk), dtype=torch.int32, device=dev)
    vals = torch.empty((1, wl.T, wl.topk), dtype=torch.float32, device=dev)
    ws = [ds.new_workspace(ds.make_problem(q[:, t0:t0 + tc], k[:, :sc], oc), wl.topk, dev)
          for (t0, tc, sc, oc) in wl.chunks]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        for c, (t0, tc, sc, oc) in enumerate(wl.chunks):
            if ev is not None:
                ev[c][0].record(stream)
            ds.select(q[:, t0:t0 + tc], k[:, :sc], ks[:, :sc], w[:, t0:t0 + tc], oc, wl.topk,
                      idx=idx[:, t0:t0 + tc], vals=vals[:, t0:t0 + tc], workspace=ws[c],
                      stream=stream)
            if ev is not None:
                ev[c][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in wl.chunks]
              for _ in range(args.steps)]
    # "Cold": before each timed step, 512 MB are written (twice the 256 MB
    # last-level cache), so no key, query or weight byte of the step is
    # cached when it starts. The write is outside the timed region: each step
    # is bracketed by synchronisations and timed on the host clock.
    flush = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    elapsed = 0.0
    step_ms = []
    for s in range(args.steps):
        if flush is not None:
            flush.fill_(s & 0xff)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        step(events[s])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t_start
        elapsed += dt
        step_ms.append(dt * 1e3)
    del flush
    step_ms.sort()
    launch_ms = [ev[0].elapsed_time(ev[1]) for st in events for ev in st]
    ms_per_step = elapsed * 1e3 / args.steps
    value = wl.T * args.steps / elapsed

    flops, pairs = _flops_64k(wl)
    n_launch = len(wl.chunks)
    avg_launch_s = (sum(launch_ms) / len(launch_ms)) * 1e-3
    achieved_tflops = flops / n_launch / avg_launch_s / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved_tflops / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(),
                "kernel": "mfma_indexer_kernel<fp8 keys, select>",
                "avg_launch_us": round(avg_launch_s * 1e6, 2),
                "flop_per_launch": flops // n_launch,
                "fp8_peak": FP8_PEAK_TFLOPS,
                "fp8_frac": round(achieved_tflops / FP8_PEAK_TFLOPS, 4),
                "cold": not args.no_flush}

    if args.copy_calibration:
        src = torch.ones(256 << 18, dtype=torch.float32, device=dev)  # 256 MiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    extra = {"step_ms_median": round(step_ms[len(step_ms) // 2], 3), "step_ms_min": round(step_ms[0], 3),
             "kernel_ms_per_step": round(sum(launch_ms) / args.steps, 3),
             "bf16_tflops_step_wall": round(flops / (ms_per_step * 1e-3) / 1e12, 1)}

    # ---------------------------------------------------------------- fp8 x fp8 prefill
    idx8 = None
    if not args.no_qfp8:
        q8 = torch.empty((1, wl.T, wl.H, wl.D), dtype=torch.uint8, device=dev)
        qs8 = torch.empty((1, wl.T, wl.H), dtype=torch.float32, device=dev)
        idx8 = torch.empty((1, wl.T, wl.topk), dtype=torch.int32, device=dev)
        vals8 = torch.empty((1, wl.T, wl.topk), dtype=torch.float32, device=dev)

        def qstep():
            for (t0, tc, sc, oc) in wl.chunks:
                ds.k_cache_write(q[0, t0:t0 + tc].reshape(tc * wl.H, wl.D), q8[0, t0:t0 + tc].reshape(tc * wl.H, wl.D),
                                 qs8[0, t0:t0 + tc].reshape(tc * wl.H), stream=stream)
                ds.select_qfp8(q8[:, t0:t0 + tc], qs8[:, t0:t0 + tc], k[:, :sc], ks[:, :sc], w[:, t0:t0 + tc], oc,
                               wl.topk, idx=idx8[:, t0:t0 + tc], vals=vals8[:, t0:t0 + tc], stream=stream)

        qstep()
        torch.cuda.synchronize()
        qe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        qe[0].record(stream)
        for _ in range(3):
            qstep()
        qe[1].record(stream)
        torch.cuda.synchronize()
        qms = qe[0].elapsed_time(qe[1]) / 3
        extra["select_qfp8_64k"] = {
            "workload": "the 64k prefill with E4M3 queries (one scale per token and head, quantised in the step)",
            "ms_per_step": round(qms, 3), "query_tok_s": round(wl.T / (qms * 1e-3), 1),
            "tflops": round(flops / (qms * 1e-3) / 1e12, 1),
            "fp8_frac": round(flops / (qms * 1e-3) / 1e12 / FP8_PEAK_TFLOPS, 4)}
        # Cost of the fp8 queries: the share of each row's bf16-query selection (the timed
        # step's output, parity-checked against the oracle by the tests) that the fp8
        # selection keeps, over all 65536 rows. Both index lists hold distinct
        # positions, so after sorting their concatenation every common position is an
        # adjacent equal pair.
        both = torch.sort(torch.cat([idx.reshape(wl.T, wl.topk), idx8.reshape(wl.T, wl.topk)], dim=1),
                          dim=1).values
        common = ((both[:, 1:] == both[:, :-1]) & (both[:, 1:] >= 0)).sum(dim=1)
        nvalid = (idx.reshape(wl.T, wl.topk) >= 0).sum(dim=1)
        recall = (common.double() / nvalid.double()).cpu().numpy()
        extra["select_qfp8_64k"]["recall_of_bf16_query_top512"] = round(float(recall.mean()), 4)
        extra["select_qfp8_64k"]["recall_min_row"] = round(float(recall.min()), 4)
        del both, common, nvalid

    hostwl = {"prefill_64k": wl}
    # ---------------------------------------------------------------- 256k decode
    if not args.no_decode:
        dl = W.decode()
        hostwl["decode_256k"] = dl
        sets = []
        qd = torch.from_numpy(dl.q.view(np.int16)).view(torch.bfloat16).to(dev)
        kd = torch.from_numpy(dl.k).to(dev)
        ksd = torch.from_numpy(dl.k_scale).to(dev)
        wd = torch.from_numpy(dl.w).to(dev)
        for r in range(3):
            sets.append((qd.clone(), kd.clone(), ksd.clone(), wd.clone()))
        del qd, kd, ksd, wd
        pd = ds.make_problem(sets[0][0], sets[0][1], dl.offset)
        wsd = ds.new_workspace(pd, dl.topk, dev)
        idd = torch.empty((dl.B, 1, dl.topk), dtype=torch.int32, device=dev)
        vd = torch.empty((dl.B, 1, dl.topk), dtype=torch.float32, device=dev)

        def dstep(i):
            a = sets[i % 3]
            ds.select(*a, dl.offset, dl.topk, idx=idd, vals=vd, workspace=wsd, stream=stream)

        dus = _time_calls(dstep, args.decode_iters, stream, args.warm_ms)
        dbytes = dl.k.nbytes + dl.k_scale.nbytes + dl.q.nbytes + dl.w.nbytes + dl.B * dl.topk * 8
        med = dus[len(dus) // 2]
        extra["decode_256k"] = {"us_median": round(med, 2), "us_min": round(dus[0], 2),
                                "alg_bytes": int(dbytes),
                                "GB_s": round(dbytes / (med * 1e-6) / 1e9, 1),
                                "hbm_frac": round(dbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic("split_decode_256k_traffic.txt",
                                                            "split_indexer.hip")}
        # ragged decode: 64 streams, one query each, cache lengths 4096 + 910 b
        # keys, packed from the same rotated bytes
        if not args.no_ragged:
            lens = 4096 + 910 * np.arange(64, dtype=np.int64)
            cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)])).to(dev)
            cu_q = torch.arange(0, 65, dtype=torch.int32, device=dev)
            rq = q[0, :64].contiguous()
            rw = w[0, :64].contiguous()
            nk = int(lens.sum())
            rsets = [(rq, a[1].reshape(-1, dl.D)[:nk], a[2].reshape(-1)[:nk]) for a in sets]
            rp = ds.make_varlen_problem(rq, rsets[0][1], cu_q, cu_k, int(lens.max()))
            rws = ds.new_varlen_workspace(rp, dl.topk, dev)
            ridx = torch.empty((64, dl.topk), dtype=torch.int32, device=dev)
            rvals = torch.empty((64, dl.topk), dtype=torch.float32, device=dev)

            def rstep(i):
                a = rsets[i % 3]
                ds.select_varlen(rq, a[1], a[2], rw, cu_q, cu_k, int(lens.max()), dl.topk, idx=ridx,
                                 vals=rvals, workspace=rws, stream=stream)

            rus = _time_calls(rstep, args.decode_iters, stream, args.warm_ms)
            rbytes = int(lens.sum()) * (dl.D + 4) + 64 * (dl.H * dl.D * 2 + dl.H * 4) + 64 * dl.topk * 8
            rmed = rus[len(rus) // 2]
            extra["ragged_decode_64"] = {
                "workload": "64 streams x 1 query, caches of 4096 + 910 b keys (2,096,704 in all), "
                            "H=64, D=128, top-512, E4M3 K, one ds4idx_select_varlen call",
                "us_median": round(rmed, 2), "us_min": round(rus[0], 2), "alg_bytes": rbytes,
                "GB_s": round(rbytes / (rmed * 1e-6) / 1e9, 1),
                "hbm_frac": round(rbytes / (rmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del sets

    # ---------------------------------------------------------------- ragged prefill
    # A 2048-token chunked-prefill budget over four streams (1024, 512, 256 and
    # 256 new tokens on caches of 32768, 16384, 8192 and 8192 keys), packed
    # from the 64k workload's first 2048 queries and its 65536 cached keys.
    if not args.no_ragged:
        Tq = np.array([1024, 512, 256, 256])
        Sk = np.array([32768, 16384, 8192, 8192])
        pcu_q = torch.from_numpy(np.concatenate([[0], np.cumsum(Tq)]).astype(np.int32)).to(dev)
        pcu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(Sk)]).astype(np.int64)).to(dev)
        pq = q[0, :2048].contiguous()
        pw = w[0, :2048].contiguous()
        pk, pks = k[0], ks[0]
        pidx = torch.empty((2048, wl.topk), dtype=torch.int32, device=dev)
        pvals = torch.empty((2048, wl.topk), dtype=torch.float32, device=dev)

        def pstep(i):
            ds.select_varlen(pq, pk, pks, pw, pcu_q, pcu_k, int(Sk.max()), wl.topk, idx=pidx,
                             vals=pvals, stream=stream)

        pus = _time_calls(pstep, 20, stream, args.warm_ms)
        pairs_r = int(sum(t * (s_ - t) + t * (t + 1) // 2 for t, s_ in zip(Tq, Sk)))
        pflop = 2 * wl.H * wl.D * pairs_r
        pmed = pus[len(pus) // 2]
        extra["ragged_prefill_2048"] = {
            "workload": "4 streams: 1024/512/256/256 new tokens on caches of 32768/16384/8192/8192 "
                        "keys, H=64, D=128, top-512, E4M3 K, one ds4idx_select_varlen call",
            "us_median": round(pmed, 2), "us_min": round(pus[0], 2),
            "query_tok_s": round(2048 / (pmed * 1e-6), 1), "flop": pflop,
            "tflops": round(pflop / (pmed * 1e-6) / 1e12, 1),
            "mfma_frac": round(pflop / (pmed * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    # ---------------------------------------------------------------- sparse attention
    if not args.no_attention:
        at = W.attention(seed=20, T=4096, S=65536, H=64, topk=512)
        aq = torch.from_numpy(at.q.view(np.int16)).view(torch.bfloat16).to(dev)
        akv = torch.from_numpy(at.kv.view(np.int16)).view(torch.bfloat16).to(dev)
        aidx = torch.from_numpy(at.idx).to(dev)
        aout = torch.empty((1, 4096, 64, at.d_v), dtype=torch.bfloat16, device=dev)
        def astep(i):
            ds.sparse_attention(aq, akv, aidx, at.softmax_scale, at.d_v, out=aout, stream=stream)

        aus = _time_calls(astep, args.attention_iters, stream, args.warm_ms)
        nsel = int((at.idx >= 0).sum())
        aflop = 2 * 64 * nsel * (at.q.shape[-1] + at.d_v)
        amed = aus[len(aus) // 2]
        row_bytes = at.q.shape[-1] * 2  # the gathered key rows (576 bf16; values are their first 512)
        # The gather probe: the same selected rows of the same cache, read
        # into registers with nothing else done (1024 workgroups, four rows
        # in flight per wavefront): what this GPU sustains on this gather.
        gprobe = _probe_lib()
        gather = {}
        if gprobe is not None:
            gsink = torch.empty(1024 * 512, dtype=torch.int32, device=dev)
            gst = ctypes.c_void_p(stream.cuda_stream)
            nidx = int(aidx.numel())

            def gpstep(i):
                st = gprobe.ds4probe_gather(akv.data_ptr(), row_bytes, int(akv.shape[-2]), aidx.data_ptr(), nidx,
                                            gsink.data_ptr(), 1024, gst)
                assert st == 0, st

            gus = _time_calls(gpstep, 20, stream, args.warm_ms)
            gpmed = gus[len(gus) // 2]
            gp_rate = nsel * row_bytes / (gpmed * 1e-6) / 1e9
            gather = {"gather_probe_us": round(gpmed, 2), "gather_probe_GB_s": round(gp_rate, 1),
                      "gather_frac": round(nsel * row_bytes / (amed * 1e-6) / 1e9 / gp_rate, 4)}
            del gsink
        extra["sparse_attention_4096"] = {
            "workload": "4096 queries x 64 heads, 512 selected rows each of a 65536-row bf16 latent cache "
                        "(key 576, value 512), bf16 out + fp32 lse",
            "us_median": round(amed, 2), "us_min": round(aus[0], 2),
            "query_tok_s": round(4096 / (amed * 1e-6), 1), "flop": aflop,
            "tflops": round(aflop / (amed * 1e-6) / 1e12, 1),
            "mfma_frac": round(aflop / (amed * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "gathered_GB_s": round(nsel * row_bytes / (amed * 1e-6) / 1e9, 1), **gather,
            "traffic": measured_traffic("sparse_attention_4096_traffic.txt", "sparse_attention.hip")}
        del aq, akv, aidx, aout

    # ---------------------------------------------------------------- key-cache writer
    if not args.no_writer:
        kn = W.new_keys()
        n_tok, kdim = kn.shape
        kin = torch.from_numpy(kn.view(np.int16)).view(torch.bfloat16).to(dev)
        del kn
        cache = torch.empty((n_tok, kdim), dtype=torch.uint8, device=dev)
        cscale = torch.empty((n_tok,), dtype=torch.float32, device=dev)
        def wstep(i):
            ds.k_cache_write(kin, cache, cscale, stream=stream)

        wus = _time_calls(wstep, args.writer_iters, stream, args.warm_ms)
        wbytes = n_tok * (2 * kdim + kdim + 4)
        wmed = wus[len(wus) // 2]
        extra["k_cache_write_256k"] = {
            "workload": f"{n_tok} bf16 keys (8 streams x 262144), D={kdim} -> E4M3 + fp32 scale",
            "us_median": round(wmed, 2), "us_min": round(wus[0], 2), "alg_bytes": int(wbytes),
            "GB_s": round(wbytes / (wmed * 1e-6) / 1e9, 1),
            "hbm_frac": round(wbytes / (wmed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("k_cache_write_256k_traffic.txt", "k_cache_writer.hip")}
        del kin, cache, cscale

    # ---------------------------------------------------------------- the other workloads
    # The tiny fp32 prefill, the 8k bf16 prefill and the 1M chunked prefill
    # (2048 queries after 1,046,528 cached E4M3 keys), one ds4idx_select call
    # each, timed with HIP events on the launch stream.
    if not args.no_others:
        for name, make in (("tiny_1024", W.tiny), ("prefill_8k", W.prefill_bf16),
                           ("prefill_1m", W.long_prefill)):
            ow = make()
            oq, ok_, oks, ow_ = _to_device(ow, dev)
            host_bytes = ow.nbytes()
            oidx = torch.empty((ow.B, ow.T, ow.topk), dtype=torch.int32, device=dev)
            ovals = torch.empty((ow.B, ow.T, ow.topk), dtype=torch.float32, device=dev)
            ows = ds.new_workspace(ds.make_problem(oq, ok_, ow.offset), ow.topk, dev)
            iters = 3 if name == "prefill_1m" else 20

            def ostep(i):
                ds.select(oq, ok_, oks, ow_, ow.offset, ow.topk, idx=oidx, vals=ovals, workspace=ows,
                          stream=stream)

            ous = _time_calls(ostep, iters, stream, args.warm_ms)
            omed = ous[len(ous) // 2]
            opairs = ow.B * (ow.T * ow.offset + ow.T * (ow.T + 1) // 2)
            oflop = 2 * ow.H * ow.D * opairs
            extra[name] = {
                "workload": f"B={ow.B} T={ow.T} S={ow.S} offset={ow.offset} H={ow.H} D={ow.D} "
                            f"top-{ow.topk}, Q {W.DTYPE_NAMES[ow.q_dtype]}, K {W.DTYPE_NAMES[ow.k_dtype]}",
                "us_median": round(omed, 2), "us_min": round(ous[0], 2),
                "query_tok_s": round(ow.B * ow.T / (omed * 1e-6), 1), "flop": oflop,
                "tflops": round(oflop / (omed * 1e-6) / 1e12, 1),
                "mfma_frac": round(oflop / (omed * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "input_bytes": int(host_bytes)}
            if name == "prefill_1m":
                extra[name]["traffic"] = measured_traffic("mfma_select_1m_kernel_stats.txt", "mfma_indexer.hip")
            hostwl[name] = ow  # host arrays, for the oracle timings below
            del oq, ok_, oks, ow_, oidx, ovals, ows, ow

    # ---------------------------------------------------------------- measured ceilings
    # What this GPU sustains in plain torch operations, beside the kernels'
    # fractions of the datasheet peaks: a read of the decode's 277 MB
    # (rotated over three copies, so the last-level cache holds none of it)
    # and a large bf16 matmul.
    if not args.no_ceilings:
        nbytes = 276989952
        bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device=dev) for _ in range(3)]

        def rstep(i):
            bufs[i % 3].sum()

        rus = _time_calls(rstep, 30, stream, args.warm_ms)
        rmed = rus[len(rus) // 2]
        # a library GEMV reads its matrix once: [16906 x 4096] fp32, the first 276,987,904 B
        grow = nbytes // 4 // 4096
        gbytes = grow * 4096 * 4
        mats = [b[:grow * 4096].view(grow, 4096) for b in bufs]
        vec = torch.ones(4096, dtype=torch.float32, device=dev)
        res = torch.empty(grow, dtype=torch.float32, device=dev)

        def gstep(i):
            torch.mv(mats[i % 3], vec, out=res)

        gus = _time_calls(gstep, 30, stream, args.warm_ms)
        gmed = gus[len(gus) // 2]
        # a device copy of 277 MB (read + write)
        dst = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)

        def cstep(i):
            dst.copy_(bufs[i % 3])

        cus_ = _time_calls(cstep, 30, stream, args.warm_ms)
        cmed = cus_[len(cus_) // 2]
        # The probe library's kernels: a plain grid-stride read of the same
        # rotated bytes (256 x 512 threads, four 16-byte loads in flight per
        # lane) and back-to-back 32x32x16 bf16 MFMAs (four chains per
        # wavefront, two wavefronts per SIMD).
        probe = _probe_lib()
        if probe is not None:
            sink = torch.empty(256 * 512, dtype=torch.int32, device=dev)
            sst = ctypes.c_void_p(stream.cuda_stream)

            def pstep(i):
                st = probe.ds4probe_hbm_read(bufs[i % 3].data_ptr(), nbytes, sink.data_ptr(), 256, sst)
                assert st == 0, st

            pus = _time_calls(pstep, 30, stream, args.warm_ms)
            pmed = pus[len(pus) // 2]
            cus_n = torch.cuda.get_device_properties(dev).multi_processor_count
            msink = torch.empty(2 * cus_n * 256, dtype=torch.float32, device=dev)
            iters = 8192

            def mfstep(i):
                st = probe.ds4probe_mfma(iters, 2 * cus_n, msink.data_ptr(), sst)
                assert st == 0, st

            mfus = _time_calls(mfstep, 10, stream, args.warm_ms)
            mfmed = mfus[len(mfus) // 2]
            mflop = 2 * cus_n * 4 * iters * 4 * 32768
            del sink, msink
        del bufs, mats, vec, res, dst
        n = 8192
        ma = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
        mb = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
        mc = torch.empty((n, n), dtype=torch.bfloat16, device=dev)

        def mstep(i):
            torch.matmul(ma, mb, out=mc)

        mus = _time_calls(mstep, 20, stream, args.warm_ms)
        mmed = mus[len(mus) // 2]
        del ma, mb, mc
        def rate(nb, us):
            return {"us_median": round(us, 2), "GB_s": round(nb / (us * 1e-6) / 1e9, 1),
                    "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

        extra["ceilings"] = {
            "hbm_read": {"what": "torch.sum over 276,989,952 B, rotated over 3 copies", **rate(nbytes, rmed)},
            "hbm_read_gemv": {"what": "torch.mv of a [16906 x 4096] fp32 matrix (276,987,904 B), rotated over "
                                      "3 copies", **rate(gbytes, gmed)},
            "hbm_copy": {"what": "torch copy_ of 276,989,952 B (read + write, counted twice)",
                         **rate(2 * nbytes, cmed)},
            **({"probe_hbm_read": {"what": "probe kernel: grid-stride read of 276,989,952 B, rotated over 3 copies, "
                                           "256 x 512 threads, four 16-byte loads in flight per lane",
                                   **rate(nbytes, pmed)},
                "probe_mfma_bf16": {"what": "probe kernel: v_mfma_f32_32x32x16_bf16, four chains per wavefront, "
                                            "two wavefronts per SIMD, register operands",
                                    "us_median": round(mfmed, 2),
                                    "tflops": round(mflop / (mfmed * 1e-6) / 1e12, 1),
                                    "frac_of_peak": round(mflop / (mfmed * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
               if probe is not None else {}),
            "bf16_matmul": {"what": "torch.matmul 8192 x 8192 x 8192 bf16",
                            "us_median": round(mmed, 2),
                            "tflops": round(2 * n ** 3 / (mmed * 1e-6) / 1e12, 1),
                            "frac_of_peak": round(2 * n ** 3 / (mmed * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}}

    # ---------------------------------------------------------------- CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        rng = np.random.Generator(np.random.PCG64(17))
        probe = np.sort(rng.choice(wl.T, 8, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        _, _, _, _, used = oracle.select(wl, rows=probe)
        t_probe = time.perf_counter() - t0
        keys_probe = int(sum(wl.offset + r + 1 for r in probe))
        rate = keys_probe / max(t_probe, 1e-6)                       # keys scored per second
        n = int(min(wl.T, max(8, args.cpu_seconds * rate / (pairs / wl.T))))
        rows = np.sort(rng.choice(wl.T, n, replace=False)).astype(np.int64)
        t0 = time.perf_counter()
        _, _, _, _, used = oracle.select(wl, rows=rows)
        t_cpu = time.perf_counter() - t0
        keys = int(sum(wl.offset + r + 1 for r in rows))
        full_s = t_cpu * pairs / keys
        cpu = {"value": round(wl.T / full_s, 2), "unit": "query-tok/s", "cores": int(used),
               "kind": "oracle",
               "sample": f"{n} uniformly drawn query rows of the 64k prefill ({keys} visible keys, "
                         f"{t_cpu:.1f} s measured), extrapolated by visible-key count to all "
                         f"{wl.T} rows ({pairs} keys)"}

    # Every workload's oracle time on the host: every row of the tiny, 8k,
    # 8k-int and decode workloads; the 64k prefill's 4 rows per chunk (each
    # chunk's first and last, 2 drawn) plus rows 510-512; 64 rows of the 1M
    # prefill (0 and 2047 included). Full-workload seconds are extrapolated
    # by visible keys. A 1-thread run of 4 rows of the 64k prefill (16k to 64k
    # visible keys) gives the per-core rate.
    if not args.no_cpu_baseline and not args.no_cpu_configs:
        import oracle
        per = {}
        plan = [("tiny_1024", lambda: hostwl.get("tiny_1024") or W.tiny(), None),
                ("prefill_8k", lambda: hostwl.get("prefill_8k") or W.prefill_bf16(), None),
                ("prefill_8k_int", W.prefill_bf16_int, None),
                ("prefill_64k", lambda: wl, lambda x: W.sample_rows_per_chunk(x, 4)),
                ("decode_256k", lambda: hostwl.get("decode_256k") or W.decode(), None),
                ("prefill_1m", lambda: hostwl.get("prefill_1m") or W.long_prefill(),
                 lambda x: W.sample_rows(x, 64))]
        for name, make, pick in plan:
            cw = make()
            rows = np.arange(cw.B * cw.T, dtype=np.int64) if pick is None else pick(cw)
            vis = lambda r: cw.offset + (np.asarray(r) % cw.T) + 1
            t0 = time.perf_counter()
            _, _, _, _, used = oracle.select(cw, rows=rows)
            t_meas = time.perf_counter() - t0
            keys = int(vis(rows).sum())
            all_keys = int(vis(np.arange(cw.B * cw.T)).sum())
            full_s = t_meas * all_keys / keys
            per[name] = {"rows": "all" if pick is None else f"{len(rows)} sampled",
                         "rows_measured": int(len(rows)), "s_measured": round(t_meas, 3),
                         "s_full_extrapolated": round(full_s, 2),
                         "query_tok_s": round(cw.B * cw.T / full_s, 2), "threads": int(used)}
            del cw
        one = np.array([16383, 32767, 49151, 65535], dtype=np.int64)  # chunk-end rows, 16k to 64k keys
        t0 = time.perf_counter()
        _, _, _, _, used1 = oracle.select(wl, rows=one, nthreads=1)
        t1 = time.perf_counter() - t0
        keys1 = int(sum(wl.offset + (r % wl.T) + 1 for r in one))
        cpu_model = None
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        extra["cpu_baseline_per_config"] = {
            "kind": "oracle", "nproc": os.cpu_count(), "cpu_model": cpu_model, "configs": per,
            "one_thread": {"threads": int(used1), "rows": len(one), "keys": keys1, "s": round(t1, 3),
                           "keys_per_s": round(keys1 / t1, 1),
                           "query_tok_s_64k_equivalent": round(keys1 / t1 / (pairs / wl.T), 3)}}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "64k cold causal prefill: T=S=65536 in 16 chunks of 4096 queries, "
                               "H=64, D=128, top-512, bf16 Q, OCP E4M3 K + per-token fp32 scale, "
                               "fp32 head weights",
                   "global_batch": 1, "seq_len": wl.T, "topk": wl.topk, "heads": wl.H,
                   "head_dim": wl.D},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
