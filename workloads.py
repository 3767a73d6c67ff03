"""Seeded synthetic inputs for the Lightning Indexer (score + top-k) workloads.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle. It generates input bytes and nothing else: it holds none of the
indexer's arithmetic (no scoring, no selection). The one transformation it
applies is the storage encoding of the inputs themselves:

* bf16 tensors are float32 draws rounded to nearest-even bf16 (torch's cast);
* fp8 key caches are OCP E4M3FN codes with one positive fp32 scale per key
  token: scale[s] = max(amax_s, 2^-126) / 448 and code = E4M3(RNE(clamp(k /
  scale, -448, 448))), the cast done by torch's ``float8_e4m3fn``.  The FP8
  format is OCP E4M3 (bias 7, max 448, NaN = S.1111.111), never the FNUZ
  variant whose reading of the same bits is off by 2x (the MI300X write-up,
  section on the FP8 format mismatch of the indexer cache).

The five workloads follow the shapes the pages' measurements revolve around
(64k cold prefill, 256k decode, the 1M window; first page, TL;DR and section
details; fourth page, performance table):

=========  ==========================================================================
tiny       T=S=1024, H=4, D=64, k=512; fp32 Q/K integers uniform in [-3,3];
           head weights in {0.5, 1, 2}. Every fp32 sum is exact.
8k         T=S=8192, H=64, D=128, k=512; bf16 Q/K = bf16(N(0,1)*0.25);
           w = N(0,1)*H^-0.5 (fp32).
8k-int     as 8k, Q/K integers uniform in [-4,4] (bf16, exact); w in {0.5,1,2}.
64k        T=S=65536 in 16 chunks of 4096 queries (chunk c: offset 4096c, S=4096(c+1));
           Q bf16(N(0,1)); K fp8 E4M3 + per-token scale of N(0,1) rows;
           w = N(0,1)*H^-0.5.
decode     8 independent streams, T=1, S=262144, offset 262143; Q/K/w as 64k.
1m         T=2048 after 1,046,528 cached tokens (S=1,048,576, offset=1,046,528).
=========  ==========================================================================

Random numbers: numpy ``Generator(PCG64(SeedSequence(seed)))`` with one
spawned child stream per tensor, so every tensor is reproducible on its own.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8_e4m3"}

E4M3_MAX = 448.0


@dataclasses.dataclass
class Workload:
    """Host arrays for one indexer problem (row-major, contiguous).

    q:       [B, T, H, D]  float32, or uint16 holding bf16 bits
    k:       [B, S, D]     float32, uint16 (bf16 bits) or uint8 (E4M3 codes)
    k_scale: [B, S]        float32 (fp8 keys only) else None
    w:       [B, T, H]     float32
    Query t of batch b sees keys s <= offset + t.
    """
    name: str
    q: np.ndarray
    k: np.ndarray
    k_scale: Optional[np.ndarray]
    w: np.ndarray
    B: int
    T: int
    S: int
    H: int
    D: int
    offset: int
    topk: int
    q_dtype: int
    k_dtype: int
    # Calls that make up one pass: (t0, T_c, S_c, offset_c). Chunk c sees the
    # cache filled so far, S_c = offset_c + T_c.
    chunks: List[Tuple[int, int, int, int]]
    integer_valued: bool = False

    def nbytes(self) -> int:
        n = self.q.nbytes + self.k.nbytes + self.w.nbytes
        if self.k_scale is not None:
            n += self.k_scale.nbytes
        return n


def _streams(seed: int, n: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest-even, torch's cast); return the uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_e4m3_per_token(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-token OCP E4M3 encoding of a key cache x[..., S, D] (float32).

    Returns (codes uint8 [..., S, D], scale float32 [..., S]) with
    scale = max(amax, 2^-126) / 448 and codes = E4M3(clamp(x / scale)).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (np.maximum(amax, np.float32(2.0 ** -126)) / np.float32(E4M3_MAX)).astype(np.float32)
    t = torch.from_numpy(x) / torch.from_numpy(scale)[..., None]
    t = t.clamp_(-E4M3_MAX, E4M3_MAX)
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


def _int_uniform(g, shape, lo, hi):
    return g.integers(lo, hi + 1, size=shape, dtype=np.int64).astype(np.float32)


def _pick_weights(g, shape):
    return np.array([0.5, 1.0, 2.0], dtype=np.float32)[g.integers(0, 3, size=shape)]


def tiny(seed: int = 1, T: int = 1024, S: int = 1024, H: int = 4, D: int = 64,
         topk: int = 512, offset: int = 0) -> Workload:
    gq, gk, gw = _streams(seed, 3)
    q = _int_uniform(gq, (1, T, H, D), -3, 3)
    k = _int_uniform(gk, (1, S, D), -3, 3)
    w = _pick_weights(gw, (1, T, H))
    return Workload("tiny", q, k, None, w, 1, T, S, H, D, offset, topk, F32, F32,
                    [(0, T, S, offset)], integer_valued=True)


def prefill_bf16(seed: int = 2, T: int = 8192, S: int = 8192, H: int = 64, D: int = 128,
                 topk: int = 512, offset: int = 0, B: int = 1, name: str = "8k") -> Workload:
    gq, gk, gw = _streams(seed, 3)
    q = to_bf16_bits(gq.standard_normal((B, T, H, D), dtype=np.float32) * np.float32(0.25))
    k = to_bf16_bits(gk.standard_normal((B, S, D), dtype=np.float32) * np.float32(0.25))
    w = gw.standard_normal((B, T, H), dtype=np.float32) * np.float32(H ** -0.5)
    return Workload(name, q, k, None, w, B, T, S, H, D, offset, topk, BF16, BF16,
                    [(0, T, S, offset)])


def prefill_bf16_int(seed: int = 102, T: int = 8192, S: int = 8192, H: int = 64, D: int = 128,
                     topk: int = 512, offset: int = 0, B: int = 1,
                     name: str = "8k-int") -> Workload:
    gq, gk, gw = _streams(seed, 3)
    q = to_bf16_bits(_int_uniform(gq, (B, T, H, D), -4, 4))
    k = to_bf16_bits(_int_uniform(gk, (B, S, D), -4, 4))
    w = _pick_weights(gw, (B, T, H))
    return Workload(name, q, k, None, w, B, T, S, H, D, offset, topk, BF16, BF16,
                    [(0, T, S, offset)], integer_valued=True)


def _fp8_cache(gk, B, S, D, block=1 << 20):
    codes = np.empty((B, S, D), dtype=np.uint8)
    scale = np.empty((B, S), dtype=np.float32)
    for b in range(B):
        for s0 in range(0, S, block):
            s1 = min(S, s0 + block)
            x = gk.standard_normal((s1 - s0, D), dtype=np.float32)
            codes[b, s0:s1], scale[b, s0:s1] = quantize_e4m3_per_token(x)
    return codes, scale


def prefill_fp8(seed: int = 3, T: int = 65536, S: int = 65536, H: int = 64, D: int = 128,
                topk: int = 512, offset: int = 0, B: int = 1, chunk: int = 4096,
                name: str = "64k") -> Workload:
    """Causal prefill of T queries in chunks against an fp8 cache that already
    holds the offset earlier tokens; chunk c covers queries [c*chunk, (c+1)*chunk)."""
    gq, gk, gw = _streams(seed, 3)
    q = to_bf16_bits(gq.standard_normal((B, T, H, D), dtype=np.float32))
    codes, scale = _fp8_cache(gk, B, S, D)
    w = gw.standard_normal((B, T, H), dtype=np.float32) * np.float32(H ** -0.5)
    chunks = []
    for t0 in range(0, T, chunk):
        tc = min(chunk, T - t0)
        chunks.append((t0, tc, offset + t0 + tc, offset + t0))
    return Workload(name, q, codes, scale, w, B, T, S, H, D, offset, topk, BF16, FP8, chunks)


def decode(seed: int = 4, B: int = 8, S: int = 262144, H: int = 64, D: int = 128,
           topk: int = 512, T: int = 1, name: str = "decode") -> Workload:
    gq, gk, gw = _streams(seed, 3)
    q = to_bf16_bits(gq.standard_normal((B, T, H, D), dtype=np.float32))
    codes, scale = _fp8_cache(gk, B, S, D)
    w = gw.standard_normal((B, T, H), dtype=np.float32) * np.float32(H ** -0.5)
    off = S - T
    return Workload(name, q, codes, scale, w, B, T, S, H, D, off, topk, BF16, FP8,
                    [(0, T, S, off)])


def long_prefill(seed: int = 5, T: int = 2048, S: int = 1048576, H: int = 64, D: int = 128,
                 topk: int = 512, name: str = "1m") -> Workload:
    gq, gk, gw = _streams(seed, 3)
    q = to_bf16_bits(gq.standard_normal((1, T, H, D), dtype=np.float32))
    codes, scale = _fp8_cache(gk, 1, S, D)
    w = gw.standard_normal((1, T, H), dtype=np.float32) * np.float32(H ** -0.5)
    off = S - T
    return Workload(name, q, codes, scale, w, 1, T, S, H, D, off, topk, BF16, FP8,
                    [(0, T, S, off)])


def int_decode(seed: int = 80, B: int = 2, S: int = 262144, H: int = 64, D: int = 128, topk: int = 512,
               lo: int = -4, hi: int = 4, kind: str = "fp8", name: str = "int-decode") -> Workload:
    """One query per stream against S cached keys, with integer values in
    [lo, hi]: bf16 queries, keys as exact E4M3 codes with scale 1 (kind "fp8")
    or as bf16, and w in {0.5, 1, 2}, so every fp32 sum is exact. A narrow
    range leaves few distinct scores: the k-th score is shared by many keys."""
    gq, gk, gw = _streams(seed, 3)
    q = to_bf16_bits(_int_uniform(gq, (B, 1, H, D), lo, hi))
    kv = _int_uniform(gk, (B, S, D), lo, hi)
    w = _pick_weights(gw, (B, 1, H))
    if kind == "fp8":
        codes = torch.from_numpy(kv).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
        return Workload(name, q, codes, np.ones((B, S), np.float32), w, B, 1, S, H, D, S - 1, topk, BF16, FP8,
                        [(0, 1, S, S - 1)], integer_valued=True)
    return Workload(name, q, to_bf16_bits(kv), None, w, B, 1, S, H, D, S - 1, topk, BF16, BF16,
                    [(0, 1, S, S - 1)], integer_valued=True)


CONFIGS = {
    "tiny": tiny,
    "8k": prefill_bf16,
    "8k-int": prefill_bf16_int,
    "64k": prefill_fp8,
    "decode": decode,
    "1m": long_prefill,
}


def make(name: str, **kw) -> Workload:
    return CONFIGS[name](**kw)


def sample_rows(wl: Workload, n: int, seed: int = 7) -> np.ndarray:
    """A bounded, seeded set of flat row ids (b*T + t) that always contains the
    first and last query of every chunk, the short rows around t = k-1 when the
    first chunk starts at offset 0, and the rest drawn uniformly."""
    fixed = set()
    for b in range(wl.B):
        for (t0, tc, _s, _o) in wl.chunks:
            fixed.add(b * wl.T + t0)
            fixed.add(b * wl.T + t0 + tc - 1)
        if wl.offset == 0:
            for t in (wl.topk - 2, wl.topk - 1, wl.topk):
                if 0 <= t < wl.T:
                    fixed.add(b * wl.T + t)
    rows = sorted(fixed)
    g = np.random.Generator(np.random.PCG64(seed))
    total = wl.B * wl.T
    while len(rows) < min(n, total):
        r = int(g.integers(0, total))
        if r not in fixed:
            fixed.add(r)
            rows.append(r)
    return np.array(sorted(rows), dtype=np.int64)


def sample_rows_per_chunk(wl: Workload, per_chunk: int = 4, seed: int = 7) -> np.ndarray:
    """Flat row ids with `per_chunk` rows from every chunk of every stream: the
    chunk's first and last query plus uniform draws inside it, and, when the
    first chunk starts at offset 0, the rows around t = k-1 (where rows reach
    k visible keys)."""
    g = np.random.Generator(np.random.PCG64(seed))
    rows = set()
    for b in range(wl.B):
        for (t0, tc, _s, _o) in wl.chunks:
            mine = {b * wl.T + t0, b * wl.T + t0 + tc - 1}
            while len(mine) < min(per_chunk, tc):
                mine.add(b * wl.T + t0 + int(g.integers(0, tc)))
            rows |= mine
        if wl.offset == 0:
            for t in (wl.topk - 2, wl.topk - 1, wl.topk):
                if 0 <= t < wl.T:
                    rows.add(b * wl.T + t)
    return np.array(sorted(rows), dtype=np.int64)


# --------------------------------------------------------------------------- key-cache writer

def new_keys(seed: int = 6, n: int = 8 * 262144, D: int = 128, log_spread: float = 0.0,
             dtype: int = BF16) -> np.ndarray:
    """Key vectors entering the key-cache writer: N(0,1) rows, each optionally
    multiplied by exp(U(-log_spread, log_spread)) so per-token scales differ.
    Returns uint16 bf16 bits (dtype BF16) or float32 values (dtype F32), [n, D].
    The default size is the 256k decode cache of 8 streams, written whole."""
    gk, gs = _streams(seed, 2)
    x = gk.standard_normal((n, D), dtype=np.float32)
    if log_spread > 0:
        x *= np.exp(gs.uniform(-log_spread, log_spread, (n, 1))).astype(np.float32)
    return to_bf16_bits(x) if dtype == BF16 else x


# --------------------------------------------------------------------------- ragged batches

@dataclasses.dataclass
class Ragged:
    """A ragged batch: streams packed along the rows.

    q [total_q, H, D] bf16 bits; k [total_k, D] E4M3 codes (or bf16 bits /
    float32); k_scale [total_k] (fp8 only); w [total_q, H]; cu_q int32 and
    cu_k int64 prefix sums [B + 1]. Stream b's query t sees its keys
    s <= S_b - T_b + t."""
    name: str
    q: np.ndarray
    k: np.ndarray
    k_scale: Optional[np.ndarray]
    w: np.ndarray
    cu_q: np.ndarray
    cu_k: np.ndarray
    H: int
    D: int
    topk: int
    q_dtype: int
    k_dtype: int

    @property
    def B(self) -> int:
        return len(self.cu_q) - 1

    def stream(self, b: int) -> Workload:
        """Stream b as a single-stream workload (offset S_b - T_b)."""
        q0, q1 = int(self.cu_q[b]), int(self.cu_q[b + 1])
        k0, k1 = int(self.cu_k[b]), int(self.cu_k[b + 1])
        T, S = q1 - q0, k1 - k0
        ks = None if self.k_scale is None else self.k_scale[k0:k1][None]
        return Workload(f"{self.name}/{b}", self.q[q0:q1][None], self.k[k0:k1][None], ks,
                        self.w[q0:q1][None], 1, T, S, self.H, self.D, S - T, self.topk,
                        self.q_dtype, self.k_dtype, [(0, T, S, S - T)])


def ragged(seed: int, streams, H: int = 64, D: int = 128, topk: int = 512, kind: str = "fp8",
           name: str = "ragged") -> Ragged:
    """Streams [(T_b, S_b), ...] with the 64k/decode recipe (kind "fp8": Q
    bf16(N(0,1)), K E4M3 + per-token scale of N(0,1) rows, w N(0,1)/8), bf16
    keys (kind "bf16"), or integers in [-4, 4] as bf16 with w in {0.5, 1, 2}
    (kind "int", every fp32 sum exact)."""
    T = np.array([t for t, _ in streams], dtype=np.int64)
    S = np.array([s for _, s in streams], dtype=np.int64)
    cu_q = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(S)]).astype(np.int64)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    gq, gk, gw = _streams(seed, 3)
    if kind == "int":
        q = to_bf16_bits(_int_uniform(gq, (tq, H, D), -4, 4))
        k = to_bf16_bits(_int_uniform(gk, (tk, D), -4, 4))
        w = _pick_weights(gw, (tq, H))
        return Ragged(name, q, k, None, w, cu_q, cu_k, H, D, topk, BF16, BF16)
    q = to_bf16_bits(gq.standard_normal((tq, H, D), dtype=np.float32))
    w = (gw.standard_normal((tq, H), dtype=np.float32) * np.float32(H ** -0.5)).astype(np.float32)
    if kind == "bf16":
        k = to_bf16_bits(gk.standard_normal((tk, D), dtype=np.float32))
        return Ragged(name, q, k, None, w, cu_q, cu_k, H, D, topk, BF16, BF16)
    codes, scale = _fp8_cache(gk, 1, tk, D)
    return Ragged(name, q, codes[0], scale[0], w, cu_q, cu_k, H, D, topk, BF16, FP8)


# --------------------------------------------------------------------------- sparse attention

@dataclasses.dataclass
class AttnInputs:
    """Sparse attention inputs: q [B,T,H,d_qk] and kv [B,S,d_qk] bf16 bits,
    idx [B,T,k] int32 (ascending selected positions, -1 padded)."""
    q: np.ndarray
    kv: np.ndarray
    idx: np.ndarray
    softmax_scale: float
    d_v: int


def attention(seed: int = 9, B: int = 1, T: int = 64, S: int = 4096, H: int = 64, topk: int = 512,
              d_qk: int = 576, d_v: int = 512, softmax_scale: Optional[float] = None,
              pad_frac: float = 0.0, causal_offset: Optional[int] = None) -> AttnInputs:
    """q, kv = bf16(N(0,1)); idx row t picks min(k, L) distinct positions
    uniformly from the L = offset + t + 1 visible ones (offset = S - T by
    default), ascending, -1 padded, then a fraction pad_frac of entries is
    replaced by -1. The default scale is d_qk^-1/2."""
    gq, gc, gi = _streams(seed, 3)
    q = to_bf16_bits(gq.standard_normal((B, T, H, d_qk), dtype=np.float32))
    kv = to_bf16_bits(gc.standard_normal((B, S, d_qk), dtype=np.float32))
    off = S - T if causal_offset is None else causal_offset
    idx = np.full((B, T, topk), -1, np.int32)
    for b in range(B):
        for t in range(T):
            L = off + t + 1
            n = min(topk, L)
            sel = np.sort(gi.choice(L, n, replace=False)) if L > n else np.arange(L)
            idx[b, t, :n] = sel
    if pad_frac > 0:
        idx[gi.random(idx.shape) < pad_frac] = -1
    scale = d_qk ** -0.5 if softmax_scale is None else softmax_scale
    return AttnInputs(q, kv, idx, float(scale), d_v)


# --------------------------------------------------------------------------- fp8 queries

def fp8_queries(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """The workload's queries in the storage encoding of the fp8 x fp8 scorer:
    one E4M3 row of D codes per (stream, token, head) with its fp32 scale, by
    the same per-row encoding as the fp8 key caches. Returns (codes uint8
    [B,T,H,D], scale float32 [B,T,H])."""
    q = bf16_bits_to_f32(wl.q) if wl.q_dtype == BF16 else np.asarray(wl.q, dtype=np.float32)
    B, T, H, D = q.shape
    codes, scale = quantize_e4m3_per_token(q.reshape(B * T * H, D))
    return codes.reshape(B, T, H, D), scale.reshape(B, T, H)


def integer_fp8_queries(seed: int, B: int, T: int, H: int, D: int, lo: int = -4, hi: int = 4):
    """Integer query values in [lo, hi] as exact E4M3 codes with scale 1."""
    g = _streams(seed, 1)[0]
    v = _int_uniform(g, (B, T, H, D), lo, hi)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, np.ones((B, T, H), np.float32)
