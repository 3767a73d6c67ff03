"""GPU parity of the key-cache writer (per-token E4M3 quantisation) through
the C ABI against the CPU oracle: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_token_lightning_amd as ds
import workloads as W
from parity import compare_rows, run_select

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _dev_keys(k: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == W.BF16:
        return torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(k, dtype=np.float32)).cuda()


def _write(k: np.ndarray, dtype: int, rows=None, slots=None, fill=0xAA, misalign16=False):
    n, D = k.shape
    rows = n if rows is None else rows
    if misalign16:  # 8-byte but not 16-byte aligned rows: the 8-values-per-lane kernel
        buf = torch.full((rows * D + 16,), fill, dtype=torch.uint8, device="cuda")
        cache = buf[8:8 + rows * D].view(rows, D)
        assert cache.data_ptr() % 16 == 8
    else:
        cache = torch.full((rows, D), fill, dtype=torch.uint8, device="cuda")
    scale = torch.full((rows,), -1.0, dtype=torch.float32, device="cuda")
    sl = None if slots is None else torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    ds.k_cache_write(_dev_keys(k, dtype), cache, scale, sl)
    torch.cuda.synchronize()
    return cache.cpu().numpy(), scale.cpu().numpy()


def _exact(k, dtype, codes, scale):
    ref_codes, ref_scale = oracle.quantize_k(k, dtype)
    np.testing.assert_array_equal(scale.view(np.uint32), ref_scale.view(np.uint32))
    bad = np.argwhere(codes != ref_codes)
    assert len(bad) == 0, f"{len(bad)} codes differ, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("D,n", [(128, 1), (128, 37), (128, 4099), (8, 300), (64, 1000),
                                 (136, 129), (512, 65)])
def test_random_tokens_exact(dtype, D, n):
    _say(f"k-cache writer random n={n} D={D} dtype={W.DTYPE_NAMES[dtype]} seed={n + D}")
    k = W.new_keys(seed=n + D, n=n, D=D, log_spread=20.0, dtype=dtype)
    codes, scale = _write(k, dtype)
    _exact(k, dtype, codes, scale)


@pytest.mark.parametrize("misalign16", [False, True])
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_special_tokens_exact(dtype, misalign16):
    # zeros, -0, one nonzero, fp32 subnormals below the scale floor, huge and
    # tiny magnitudes, heavy tails, all-equal, small integers
    g = np.random.Generator(np.random.PCG64(9))
    D = 128
    k = g.standard_normal((12, D)).astype(np.float32)
    k[1] *= 1e30
    k[2] *= 1e-30
    k[3] = 0.0
    k[4] = 0.0
    k[4, D // 2] = -3.0
    k[5] = np.float32(2.0 ** -130)
    k[6] = g.standard_t(2, D)
    k[7] = -0.0
    k[8] = 1.0
    k[9] = g.integers(-4, 5, D)
    k[10] *= 2.0 ** 120
    k[11] *= 2.0 ** -120
    if dtype == W.BF16:
        k = W.to_bf16_bits(k)
    _say(f"k-cache writer special tokens dtype={W.DTYPE_NAMES[dtype]} misalign16={misalign16}")
    codes, scale = _write(k, dtype, misalign16=misalign16)
    _exact(k, dtype, codes, scale)


@pytest.mark.parametrize("misalign16", [False, True])
def test_quotients_near_every_midpoint_exact(misalign16):
    # Tokens whose quotients k / scale land on, and a few fp32 steps around,
    # every midpoint between adjacent E4M3 values, under scales that are not
    # powers of two: a division that is off by one step, or rounding that is
    # not to nearest-even, changes codes here. The scales span both division
    # paths of the kernel (scale >= 2^-80 and below) and the boundary.
    vals = np.array([oracle.e4m3_decode(c) for c in range(127)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    rows = []
    edge = 448.0 * 2.0 ** -80
    for amax in (448.0, 1.0, 3.0, 0.1, 1000.0, 7.0e-3, 2.0 ** 20 * 3, 2.0 ** 100 * 5, edge,
                 float(np.nextafter(np.float32(edge), np.float32(1))),
                 float(np.nextafter(np.float32(edge), np.float32(0))), 3.0 * 2.0 ** -85,
                 5.0 * 2.0 ** -100, 1.5 * 2.0 ** -110):
        sc = np.float32(amax) / np.float32(448.0)
        base = (mids.astype(np.float64) * np.float64(sc)).astype(np.float32)
        for step in (-2, -1, 0, 1, 2):
            v = base.copy()
            for _ in range(abs(step)):
                v = np.nextafter(v, np.float32(np.inf) if step > 0 else np.float32(0))
            for sign in (1.0, -1.0):
                row = np.zeros(128, np.float32)
                row[0] = np.float32(amax)
                row[1:1 + len(v)] = sign * v
                rows.append(row)
    k = np.stack(rows)
    _say(f"k-cache writer near-midpoint quotients: {len(rows)} tokens misalign16={misalign16}")
    codes, scale = _write(k, W.F32, misalign16=misalign16)
    _exact(k, W.F32, codes, scale)


def test_slots_scatter_and_skip():
    n, D, rows = 1000, 128, 1500
    g = np.random.Generator(np.random.PCG64(12))
    k = W.new_keys(seed=12, n=n, D=D, log_spread=5.0)
    slots = g.permutation(rows)[:n].astype(np.int64)
    slots[::97] = -1
    slots[5::101] = rows + 3
    _say(f"k-cache writer slots n={n} rows={rows}")
    codes, scale = _write(k, W.BF16, rows=rows, slots=slots)
    ref_codes, ref_scale = oracle.quantize_k(k, W.BF16)
    ok = (slots >= 0) & (slots < rows)
    np.testing.assert_array_equal(codes[slots[ok]], ref_codes[ok])
    np.testing.assert_array_equal(scale[slots[ok]].view(np.uint32), ref_scale[ok].view(np.uint32))
    untouched = np.setdiff1d(np.arange(rows), slots[ok])
    assert np.all(codes[untouched] == 0xAA) and np.all(scale[untouched] == -1.0)


def test_written_cache_feeds_the_indexer():
    # Keys written by the writer are byte-identical to the oracle's
    # quantisation, and the fused indexer over that cache matches the oracle.
    B, T, S, H, D = 1, 64, 4096, 64, 128
    keys = W.new_keys(seed=31, n=S, D=D)
    codes, scale = _write(keys, W.BF16)
    ref_codes, ref_scale = oracle.quantize_k(keys, W.BF16)
    np.testing.assert_array_equal(codes, ref_codes)
    np.testing.assert_array_equal(scale.view(np.uint32), ref_scale.view(np.uint32))
    gq, gw = W._streams(32, 2)
    q = W.to_bf16_bits(gq.standard_normal((B, T, H, D), dtype=np.float32))
    w = (gw.standard_normal((B, T, H)) * H ** -0.5).astype(np.float32)
    off = S - T
    wl = W.Workload("writer-fed", q, codes[None], scale[None], w, B, T, S, H, D, off, 512,
                    W.BF16, W.FP8, [(0, T, S, off)])
    _say(f"k-cache writer feeding select T={T} S={S}")
    gi, gv = run_select(wl)
    compare_rows(wl, np.arange(T), gi, gv, exact=False)


def test_full_decode_cache_sampled_exact():
    # The benchmark's launch: 8 streams x 262144 tokens of bf16 keys, D = 128,
    # written in one call; 4096 sampled tokens checked against the oracle.
    n, D = 8 * 262144, 128
    _say(f"k-cache writer full size n={n} D={D}")
    keys = W.new_keys(seed=6, n=n, D=D)
    codes, scale = _write(keys, W.BF16)
    g = np.random.Generator(np.random.PCG64(13))
    pick = np.unique(np.concatenate([[0, n - 1], g.integers(0, n, 4094)]))
    ref_codes, ref_scale = oracle.quantize_k(keys[pick], W.BF16)
    np.testing.assert_array_equal(codes[pick], ref_codes)
    np.testing.assert_array_equal(scale[pick].view(np.uint32), ref_scale.view(np.uint32))
