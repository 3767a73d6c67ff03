"""GPU parity of sparse attention (ds4idx_sparse_attention) through the C ABI
against the CPU oracle.

Tolerance, from the arithmetic. Scores, sums and accumulators are fp32; the
probabilities p_j enter the value sum rounded to bf16, p_j (1 + d_j) with
|d_j| <= 2^-9, and the output is rounded to bf16 (relative 2^-9 per element).

* Element bound (worst case): the weighted mean moves by at most 2^-9 of the
  largest selected value, so |out - ref| <= 2^-8 (max_j |v_j| + |ref|).
* Norm bound per (token, head), over the d_v outputs: with softmax weights
  w_j, the probability rounding adds e = sum_j w_j (d_j - dbar) v_j, where
  dbar = sum_j w_j d_j (the denominator may or may not see the rounding).
  The dbar part is at most 2^-9 |ref| in norm; the rest is a sum of
  independent rounding errors with standard deviation at most
  2^-9 / sqrt(3) * sqrt(sum_j w_j^2 |v_j|^2). Allowed:
      |out - ref|_2 <= 2^-8 |ref|_2 + 6 * 2^-9 / sqrt(3) * sqrt(sum_j w_j^2 |v_j|_2^2) + 1e-6
  (output rounding and dbar, plus six standard deviations; when at most 12
  keys carry the weight, the second term also covers the worst case
  2^-9 sum_j w_j |v_j|). On N(0,1) rows of 512 keys this is about 1% of
  |ref|_2, where dropping one selected key from the value sum alone moves the
  output by about 4%.
* lse within 2e-5 + 1e-5 |lse|."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as ds
import workloads as W

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def run_attention(a: W.AttnInputs):
    o, lse = ds.sparse_attention(_bf16_dev(a.q), _bf16_dev(a.kv), torch.from_numpy(a.idx).cuda(),
                                 a.softmax_scale, a.d_v)
    torch.cuda.synchronize()
    B, T, H, _ = a.q.shape
    o = o.float().cpu().numpy().reshape(B * T, H, a.d_v)
    return o, lse.cpu().numpy().reshape(B * T, H)


def check(a: W.AttnInputs, go, glse, rows=None):
    B, T, H, _ = a.q.shape
    rows = np.arange(B * T) if rows is None else np.asarray(rows)
    ro, rl = oracle.sparse_attention(a.q, a.kv, a.idx, a.softmax_scale, a.d_v, rows=rows)
    kvf = W.bf16_bits_to_f32(a.kv).astype(np.float64)
    qf = W.bf16_bits_to_f32(a.q).astype(np.float64).reshape(B * T, H, -1)
    S = a.kv.shape[1]
    for n, r in enumerate(rows):
        b = r // T
        sel = a.idx.reshape(B * T, -1)[r]
        sel = sel[(sel >= 0) & (sel < S)]
        vmax = np.abs(kvf[b, sel, :a.d_v]).max() if len(sel) else 0.0
        tol = 2.0 ** -8 * (vmax + np.abs(ro[n]))
        err = np.abs(go[r] - ro[n])
        assert np.all(err <= tol), f"row {r}: max error {err.max()} (worst head {np.unravel_index(np.argmax(err - tol), err.shape)})"
        if len(sel):
            # softmax weights of the selection (tolerance scale only)
            z = a.softmax_scale * (qf[r] @ kvf[b, sel].T)             # [H, n_sel]
            wgt = np.exp(z - z.max(axis=1, keepdims=True))
            wgt /= wgt.sum(axis=1, keepdims=True)
            vn2 = (kvf[b, sel, :a.d_v] ** 2).sum(axis=1)               # |v_j|^2
            spread = np.sqrt((wgt ** 2 * vn2[None, :]).sum(axis=1))    # [H]
            refn = np.linalg.norm(ro[n], axis=1)
            errn = np.linalg.norm(go[r] - ro[n], axis=1)
            ntol = 2.0 ** -8 * refn + 6.0 * 2.0 ** -9 / np.sqrt(3.0) * spread + 1e-6
            worst = int(np.argmax(errn / ntol))
            assert np.all(errn <= ntol), \
                f"row {r} head {worst}: |out-ref|_2 = {errn[worst]:.3e} > {ntol[worst]:.3e} (|ref|_2 = {refn[worst]:.3e})"
        if len(sel) == 0:
            assert np.all(np.isneginf(glse[r])) and np.all(go[r] == 0)
        else:
            np.testing.assert_allclose(glse[r], rl[n], rtol=1e-5, atol=2e-5, err_msg=f"row {r} lse")


@pytest.mark.parametrize("seed,B,T,S,H,k,pad", [(11, 2, 5, 700, 64, 64, 0.0), (12, 1, 16, 4096, 128, 512, 0.0),
                                                (13, 1, 9, 300, 64, 100, 0.3), (14, 3, 2, 50, 64, 33, 0.0),
                                                (15, 1, 4, 2000, 192, 256, 0.1)])
def test_random_rows(seed, B, T, S, H, k, pad):
    a = W.attention(seed=seed, B=B, T=T, S=S, H=H, topk=k, pad_frac=pad)
    _say(f"sparse attention seed={seed} B={B} T={T} S={S} H={H} k={k} pad={pad}")
    go, glse = run_attention(a)
    check(a, go, glse)


def test_peaked_scores():
    # a large scale makes the softmax nearly one-hot: the max subtraction and
    # the online rescaling carry the whole result
    a = W.attention(seed=16, T=8, S=3000, topk=512, softmax_scale=0.35)
    _say("sparse attention peaked scale=0.35")
    go, glse = run_attention(a)
    check(a, go, glse)


@pytest.mark.parametrize("direction", [1.0, -1.0])
def test_scores_rising_by_chunk(direction):
    # Scores (log2 units) that move by a per-head step from one 32-row chunk
    # of the selection to the next. Steps of 7 stay within the running max's
    # slack of 8, so the probabilities grow to 2^7 without a rescale; steps of
    # 10.5, 14 and 17.5 force a rescale at every chunk. Falling scores
    # (direction -1) never rescale after the first chunk. Only the last dim of
    # q is nonzero, so the score of row j is q[-1] * kv[j, -1] * scale; that
    # dim lies outside the values, so the tolerance stays set by the N(0,1)
    # values.
    B, T, S, H, k = 1, 4, 1024, 64, 512
    a = W.attention(seed=22, B=B, T=T, S=S, H=H, topk=k, softmax_scale=1.0)
    g = np.random.Generator(np.random.PCG64(23))
    ln2 = float(np.log(2.0))
    sel = np.sort(g.choice(S, k, replace=False))
    a.idx[:] = sel[None, None, :]
    kv = W.bf16_bits_to_f32(a.kv)
    z = direction * 7.0 * (np.arange(k) // 32) + g.uniform(-0.5, 0.5, k)  # log2 units for q0 = 1
    kv[0, sel, -1] = (z * ln2).astype(np.float32)
    a.kv[:] = W.to_bf16_bits(kv)
    q = np.zeros((B, T, H, a.q.shape[-1]), np.float32)
    q[..., -1] = (1.0 + 0.5 * (np.arange(H) % 4))[None, None, :]  # steps 7, 10.5, 14, 17.5
    a.q[:] = W.to_bf16_bits(q)
    _say(f"sparse attention scores moving by chunk, direction {direction}")
    go, glse = run_attention(a)
    check(a, go, glse)


def test_edge_rows():
    # no valid entry; one valid entry (out is that row's values exactly);
    # out-of-range entries; duplicates of the same position
    a = W.attention(seed=17, T=4, S=200, topk=40)
    a.idx[0, 0, :] = -1
    a.idx[0, 1, :] = -1
    a.idx[0, 1, 17] = 123
    a.idx[0, 2, ::3] = 200
    a.idx[0, 2, 1::5] = -9
    a.idx[0, 3, :10] = 77
    _say("sparse attention edge rows")
    go, glse = run_attention(a)
    check(a, go, glse)
    assert np.all(go[0] == 0) and np.all(np.isneginf(glse[0]))
    v = W.bf16_bits_to_f32(a.kv)[0, 123, :512]
    assert np.array_equal(go[1], np.broadcast_to(v, go[1].shape))


def test_indexer_output_feeds_attention():
    # the indexer's selection over a bf16 cache (its first 128 dims as the
    # indexer keys) drives the attention; both checked against the oracle
    B, T, S, H = 1, 64, 4096, 64
    wl = W.prefill_bf16(seed=18, T=T, S=S, offset=S - T)
    from parity import run_select
    gi, _ = run_select(wl)
    a = W.attention(seed=19, B=B, T=T, S=S, H=H, topk=512)
    a.idx[:] = gi.reshape(B, T, 512)
    _say("indexer selection feeding sparse attention")
    go, glse = run_attention(a)
    check(a, go, glse)


def test_prefill_chunk_full_size_sampled():
    # one 4096-query chunk of a long prefill: 4096 tokens x 64 heads attending
    # to 512 of 65536 cached rows; 24 sampled rows checked
    a = W.attention(seed=20, T=4096, S=65536, H=64, topk=512)
    _say("sparse attention T=4096 S=65536 H=64 k=512")
    go, glse = run_attention(a)
    g = np.random.Generator(np.random.PCG64(21))
    rows = np.unique(np.concatenate([[0, 4095], g.integers(0, 4096, 22)]))
    check(a, go, glse, rows=rows)


@pytest.mark.parametrize("seed,B,T,S,H,k,pad,sample", [
    (30, 1, 700, 3000, 64, 40, 0.0, None),    # 2 chunks per item: each item starts its own gathers
    (31, 2, 300, 2000, 64, 70, 0.0, None),    # 3 chunks (the last ragged): gathers run on into the next item
    (32, 1, 200, 5000, 128, 512, 0.0, None),  # two head tiles per query row
    (33, 3, 120, 900, 192, 96, 0.3, None),    # three head tiles, streams change within a workgroup's run
    (34, 1, 300, 4096, 64, 2048, 0.0, 40),    # the largest selection, 64 chunks
])
def test_many_items_per_workgroup(seed, B, T, S, H, k, pad, sample):
    # More (query row, head tile) items than CUs, so every workgroup takes a
    # run of consecutive items, carrying its gather ring (or restarting it)
    # from one item to the next; every row (or a sample with both ends)
    # against the oracle
    a = W.attention(seed=seed, B=B, T=T, S=S, H=H, topk=k, pad_frac=pad)
    _say(f"sparse attention many items seed={seed} B={B} T={T} S={S} H={H} k={k} pad={pad}")
    go, glse = run_attention(a)
    rows = None
    if sample:
        g = np.random.Generator(np.random.PCG64(seed))
        rows = np.unique(np.concatenate([[0, B * T - 1], g.integers(0, B * T, sample - 2)]))
    check(a, go, glse, rows=rows)


@pytest.mark.parametrize("group", range(2))
def test_randomised_attention(group):
    # 10 seeded random shapes per group: 1-3 streams, 1-119 queries, 64, 128 or
    # 192 heads, caches of 40 to 70000 rows, k from 1 to 2048 (odd counts and
    # ragged last chunks included), with and without padded entries; every row
    # (or 32 sampled rows with both ends) against the oracle.
    g = np.random.Generator(np.random.PCG64(800 + group))
    for case in range(10):
        B, T, H = int(g.integers(1, 4)), int(g.integers(1, 120)), int(g.choice([64, 128, 192]))
        S = int(g.integers(40, 70000))
        topk = min(int(g.choice([1, 17, 32, 33, 64, 96, 97, 128, 500, 512, 2048])), S)
        pad = float(g.choice([0.0, 0.0, 0.3]))
        a = W.attention(seed=8100 + 10 * group + case, B=B, T=T, S=S, H=H, topk=topk, pad_frac=pad)
        _say(f"random attention B={B} T={T} S={S} H={H} k={topk} pad={pad}")
        go, glse = run_attention(a)
        rows = None if B * T <= 64 else np.unique(np.concatenate([[0, B * T - 1], g.integers(0, B * T, 30)]))
        check(a, go, glse, rows=rows)

