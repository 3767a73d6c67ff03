"""C-ABI checks that need no GPU: the library loads, exports every function
include/ds4idx.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import sparse_attention_token_lightning_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4idx.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4idx_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(ds.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ds.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.ds4idx_abi_version() == ds.ABI_VERSION


def test_status_strings():
    for s in range(6):
        assert ds.status_string(s)
    assert ds.status_string(99) == "unknown status"


def test_impl_switch():
    prev = ds.set_impl("ref")
    try:
        assert ds.get_impl() == ds.IMPL_REF
        assert ds.lib().ds4idx_set_impl(7) == -1
        assert ds.get_impl() == ds.IMPL_REF
    finally:
        ds.set_impl(prev)


def _prob(**kw):
    d = dict(B=1, T=16, S=32, H=64, D=128, causal_offset=16, q_dtype=ds.BF16, k_dtype=ds.FP8_E4M3)
    d.update(kw)
    return ds.Problem(**d)


FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: validation fails first
FAKE_MIS = ctypes.c_void_p(0x10004)   # 4-byte aligned, not 16


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(S=0), dict(H=0), dict(D=-1),
                                dict(causal_offset=-1), dict(causal_offset=17),
                                dict(q_dtype=2), dict(k_dtype=5), dict(q_dtype=-1)])
def test_invalid_problem_rejected(kw):
    L = ds.lib()
    p = _prob(**kw)
    args = (ctypes.byref(p), FAKE, FAKE, FAKE, FAKE)
    assert L.ds4idx_score(*args, FAKE, None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_select(*args, 512, FAKE, None, None, 0, None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_topk(ctypes.byref(p), FAKE, 512, FAKE, None, None, 0, None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_workspace_bytes(ctypes.byref(p), 512, ds.OP_SELECT) == ctypes.c_size_t(-1).value


def test_null_problem_rejected():
    L = ds.lib()
    assert L.ds4idx_score(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_workspace_bytes(None, 512, ds.OP_SELECT) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("which", ["q", "k", "w", "ks", "idx"])
def test_null_pointers_rejected(which):
    L = ds.lib()
    p = _prob()
    ptr = {n: FAKE for n in ("q", "k", "w", "ks", "idx")}
    ptr[which] = None
    st = L.ds4idx_select(ctypes.byref(p), ptr["q"], ptr["k"], ptr["ks"], ptr["w"], 512, ptr["idx"],
                         None, None, 0, None)
    assert st == ds.ERR_INVALID_ARG


def test_fp8_needs_scale_but_bf16_does_not_validate_it():
    L = ds.lib()
    p = _prob()
    assert L.ds4idx_score(ctypes.byref(p), FAKE, FAKE, None, FAKE, FAKE, None) == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["q", "k"])
def test_misaligned_inputs_rejected(which):
    L = ds.lib()
    p = _prob()
    q = FAKE_MIS if which == "q" else FAKE
    k = FAKE_MIS if which == "k" else FAKE
    assert L.ds4idx_select(ctypes.byref(p), q, k, FAKE, FAKE, 512, FAKE, None, None, 0,
                           None) == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("k", [0, -1, 2049])
def test_bad_k_rejected(k):
    L = ds.lib()
    p = _prob()
    assert L.ds4idx_select(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, k, FAKE, None, None, 0,
                           None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_topk(ctypes.byref(p), FAKE, k, FAKE, None, None, 0, None) == ds.ERR_INVALID_ARG


def test_workspace_sizes_and_checks():
    L = ds.lib()
    prev = ds.set_impl("auto")
    try:
        # Enough rows to fill the GPU: the MFMA prefill kernel, no workspace.
        p_pre = _prob(T=2048, S=4096, causal_offset=2048)
        assert ds.workspace_bytes(p_pre, 512, ds.OP_SCORE) == 0
        assert ds.workspace_bytes(p_pre, 512, ds.OP_TOPK) == 0
        assert ds.workspace_bytes(p_pre, 512) == 0
        # Few rows (decode-like): the split-key kernel; counters + candidates.
        p_dec = _prob(B=8, T=1, S=262144, causal_offset=262143)
        need = ds.workspace_bytes(p_dec, 512)
        parts = 262144 // 8192
        # per partition: bounds (16 bytes), 2k full-list and 16*ceil(k/parts) short-list slots of 8 bytes
        assert need >= 8 * 4 + 8 * parts * 16 + 8 * parts * (1024 + 256) * 8 and need % 256 == 0
        st = L.ds4idx_select(ctypes.byref(p_dec), FAKE, FAKE, FAKE, FAKE, 512, FAKE, None, None, 0, None)
        assert st == ds.ERR_WORKSPACE
        st = L.ds4idx_select(ctypes.byref(p_dec), FAKE, FAKE, FAKE, FAKE, 512, FAKE, None,
                             ctypes.c_void_p(0x10100), need - 1, None)
        assert st == ds.ERR_WORKSPACE
        st = L.ds4idx_select(ctypes.byref(p_dec), FAKE, FAKE, FAKE, FAKE, 512, FAKE, None,
                             ctypes.c_void_p(0x10080), need, None)  # not 256-byte aligned
        assert st == ds.ERR_WORKSPACE
        # The plain kernels materialise the scores.
        ds.set_impl("ref")
        assert ds.workspace_bytes(p_pre, 512) >= p_pre.B * p_pre.T * p_pre.S * 4
        # Forcing the MFMA family on a shape it does not cover.
        ds.set_impl("opt")
        p2 = _prob(H=4, D=64, q_dtype=ds.F32, k_dtype=ds.F32)
        assert L.ds4idx_score(ctypes.byref(p2), FAKE, FAKE, None, FAKE, FAKE, None) == ds.ERR_UNSUPPORTED
        assert L.ds4idx_select(ctypes.byref(p2), FAKE, FAKE, None, FAKE, 8, FAKE, None, None, 0,
                               None) == ds.ERR_UNSUPPORTED
    finally:
        ds.set_impl(prev)


FAKE8_MIS = ctypes.c_void_p(0x10004)  # 4-byte aligned, not 8


@pytest.mark.parametrize("kw", [dict(dtype=ds.FP8_E4M3), dict(dtype=7), dict(n=-1), dict(D=0),
                                dict(D=12), dict(D=520), dict(rows=0), dict(kin=None),
                                dict(cache=None), dict(scale=None), dict(kin=FAKE_MIS),
                                dict(cache=FAKE8_MIS), dict(slots=FAKE8_MIS)])
def test_k_cache_write_rejects_bad_arguments(kw):
    a = dict(kin=FAKE, dtype=ds.BF16, n=4, D=128, slots=None, cache=FAKE, scale=FAKE, rows=16)
    a.update(kw)
    st = ds.lib().ds4idx_k_cache_write(a["kin"], a["dtype"], a["n"], a["D"], a["slots"], a["cache"],
                                       a["scale"], a["rows"], None)
    assert st == ds.ERR_INVALID_ARG


def test_k_cache_write_empty_is_a_no_op():
    # n = 0 returns before touching any pointer or launching anything
    assert ds.lib().ds4idx_k_cache_write(None, ds.F32, 0, 128, None, None, None, 1, None) == ds.OK


def test_k_cache_write_grid_limit():
    st = ds.lib().ds4idx_k_cache_write(FAKE, ds.BF16, 1 << 40, 128, None, FAKE, FAKE, 16, None)
    assert st == ds.ERR_UNSUPPORTED


def _vprob(**kw):
    d = dict(B=3, total_q=10, total_k=1000, max_k=600, H=64, D=128, q_dtype=ds.BF16,
             k_dtype=ds.FP8_E4M3)
    d.update(kw)
    return ds.VarlenProblem(**d)


def _vselect(p, **ptrs):
    a = dict(cu_q=FAKE, cu_k=FAKE, q=FAKE, k=FAKE, ks=FAKE, w=FAKE, idx=FAKE, k_=512)
    a.update(ptrs)
    return ds.lib().ds4idx_select_varlen(ctypes.byref(p), a["cu_q"], a["cu_k"], a["q"], a["k"], a["ks"],
                                         a["w"], a["k_"], a["idx"], None, None, 0, None)


@pytest.mark.parametrize("kw", [dict(B=0), dict(total_q=-1), dict(total_k=-1), dict(max_k=0),
                                dict(H=0), dict(D=0), dict(q_dtype=2), dict(k_dtype=9)])
def test_varlen_invalid_problem_rejected(kw):
    p = _vprob(**kw)
    assert _vselect(p) == ds.ERR_INVALID_ARG
    assert ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(p), 512) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("which", ["cu_q", "cu_k", "q", "k", "ks", "w", "idx"])
def test_varlen_null_pointers_rejected(which):
    assert _vselect(_vprob(), **{which: None}) == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["cu_k", "q", "k"])
def test_varlen_misaligned_rejected(which):
    assert _vselect(_vprob(), **{which: FAKE_MIS}) == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("k", [0, 2049])
def test_varlen_bad_k_rejected(k):
    assert _vselect(_vprob(), k_=k) == ds.ERR_INVALID_ARG


def test_varlen_unsupported_shape_and_routing():
    assert _vselect(_vprob(H=4)) == ds.ERR_UNSUPPORTED
    assert _vselect(_vprob(q_dtype=ds.F32)) == ds.ERR_UNSUPPORTED
    # k > 512 needs the split-key kernel, which takes at most 65535 rows
    assert _vselect(_vprob(total_q=70000), k_=1024) == ds.ERR_UNSUPPORTED
    # few rows: split-key kernel with a workspace; missing workspace is reported
    assert _vselect(_vprob()) == ds.ERR_WORKSPACE
    p = _vprob()
    n = ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(p), 512)
    assert n > 0 and n % 256 == 0
    # many rows: the prefill kernel, no workspace
    p = _vprob(total_q=4096)
    assert ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(p), 512) == 0


def test_varlen_empty_batch_is_a_no_op():
    assert _vselect(_vprob(total_q=0)) == ds.OK


def _a256(n):
    return (n + 255) // 256 * 256


def test_varlen_workspace_matches_uniform_decode():
    # 8 streams of one query over 262144 keys: under every fixed partition
    # length the same split-key workspace as the uniform decode problem;
    # under the automatic length the ragged batch takes planned parts, whose
    # lists are sized per launched block: max(rows * ceil(max_k / 16384), 256)
    # blocks, each with 2k full-list and 2k short-list slots, plus a counter
    # per row
    v = _vprob(B=8, total_q=8, total_k=8 * 262144, max_k=262144)
    u = ds.Problem(8, 1, 262144, 64, 128, 262143, ds.BF16, ds.FP8_E4M3)
    prev = ds.set_split(0)
    try:
        for keys in ds.SPLIT_LENS:
            ds.set_split(keys)
            assert ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(v), 512) == \
                ds.lib().ds4idx_workspace_bytes(ctypes.byref(u), 512, ds.OP_SELECT)
        ds.set_split(0)
        blocks = max(8 * (262144 // 16384), 256)
        assert ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(v), 512) == \
            _a256(8 * 4) + _a256(blocks * 16) + 2 * _a256(blocks * 1024 * 8)
        # more rows than a plan takes: fixed-length partitions again
        w = _vprob(B=300, total_q=300, total_k=300 * 4096, max_k=4096)
        ds.set_split(8192)
        fixed = ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(w), 512)
        ds.set_split(0)
        assert ds.lib().ds4idx_varlen_workspace_bytes(ctypes.byref(w), 512) == fixed
    finally:
        ds.set_split(prev)


def test_split_length_switch_and_automatic_choice():
    prev = ds.set_split(0)
    try:
        assert ds.get_split() == 0
        with pytest.raises(ValueError):
            ds.set_split(10000)
        assert ds.get_split() == 0 and ds.lib().ds4idx_set_split(4096) == -1
        dec = ds.Problem(8, 1, 262144, 64, 128, 262143, ds.BF16, ds.FP8_E4M3)
        auto = ds.workspace_bytes(dec, 512)
        ds.set_split(8192)
        assert ds.workspace_bytes(dec, 512) == auto  # 8 x 32 partitions fill the 256 CUs
        ds.set_split(16384)
        assert ds.workspace_bytes(dec, 512) < auto   # half the partitions
        assert ds.set_split(0) == 16384
        # 10 streams: 320 partitions of 8192 keys would need two rounds; 12288
        # keys gives 220, one round
        ten = ds.Problem(10, 1, 262144, 64, 128, 262143, ds.BF16, ds.FP8_E4M3)
        auto10 = ds.workspace_bytes(ten, 512)
        ds.set_split(12288)
        assert ds.workspace_bytes(ten, 512) == auto10
        ds.set_split(0)
        # the ragged decode mix: 64 streams of 4096 + 910 b keys (2,096,704 in
        # all, at most 61426). With a fixed length, 2096704 / 8192 + 64 > 256
        # partitions of 8192 keys: the workspace for 8192 exceeds that for
        # 12288. The automatic length plans the parts on the device, with
        # lists for max(64 * ceil(61426 / 16384), 256) = 256 blocks.
        lens = [4096 + 910 * b for b in range(64)]
        v = _vprob(B=64, total_q=64, total_k=sum(lens), max_k=max(lens))
        assert ds.varlen_workspace_bytes(v, 512) == _a256(64 * 4) + _a256(256 * 16) + 2 * _a256(256 * 1024 * 8)
        ds.set_split(12288)
        w12 = ds.varlen_workspace_bytes(v, 512)
        ds.set_split(8192)
        assert ds.varlen_workspace_bytes(v, 512) > w12
    finally:
        ds.set_split(prev)


def _aprob(**kw):
    d = dict(B=1, T=4, S=100, H=64, topk=512, d_qk=576, d_v=512, softmax_scale=0.04)
    d.update(kw)
    return ds.AttnProblem(**d)


def _attn(p, **ptrs):
    a = dict(q=FAKE, kv=FAKE, idx=FAKE, o=FAKE, lse=None)
    a.update(ptrs)
    return ds.lib().ds4idx_sparse_attention(ctypes.byref(p), a["q"], a["kv"], a["idx"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw", [dict(B=0), dict(T=0), dict(S=0), dict(H=0), dict(topk=0), dict(topk=2049),
                                dict(d_qk=0), dict(d_v=600), dict(softmax_scale=float("nan")),
                                dict(softmax_scale=float("inf"))])
def test_attention_invalid_problem_rejected(kw):
    assert _attn(_aprob(**kw)) == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("which", ["q", "kv", "idx", "o"])
def test_attention_null_or_misaligned_rejected(which):
    assert _attn(_aprob(), **{which: None}) == ds.ERR_INVALID_ARG
    if which != "idx":
        assert _attn(_aprob(), **{which: FAKE_MIS}) == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(H=32), dict(H=96), dict(d_qk=512), dict(d_v=256)])
def test_attention_unsupported_shapes(kw):
    assert _attn(_aprob(**kw)) == ds.ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(q_dtype=ds.BF16), dict(k_dtype=ds.BF16), dict(T=0), dict(causal_offset=17)])
def test_qfp8_invalid_problem_rejected(kw):
    p = _prob(q_dtype=ds.FP8_E4M3, **{k: v for k, v in kw.items() if k != "q_dtype"})
    if "q_dtype" in kw:
        p.q_dtype = kw["q_dtype"]
    st = ds.lib().ds4idx_select_qfp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 512, FAKE, None, None)
    assert st == ds.ERR_INVALID_ARG


@pytest.mark.parametrize("which", [1, 2, 3, 4, 5, 7])
def test_qfp8_null_pointers_rejected(which):
    p = _prob(q_dtype=ds.FP8_E4M3)
    args = [ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 512, FAKE, None, None]
    args[which] = None
    assert ds.lib().ds4idx_select_qfp8(*args) == ds.ERR_INVALID_ARG


def test_qfp8_unsupported_shapes():
    for kw in (dict(H=32), dict(D=64)):
        p = _prob(q_dtype=ds.FP8_E4M3, **kw)
        assert ds.lib().ds4idx_select_qfp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 512, FAKE, None,
                                           None) == ds.ERR_UNSUPPORTED
    p = _prob(q_dtype=ds.FP8_E4M3)
    assert ds.lib().ds4idx_select_qfp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1024, FAKE, None,
                                       None) == ds.ERR_UNSUPPORTED


def test_noalloc_validates_before_any_hip_call():
    L = ds.lib()
    p = _prob(B=8, T=1, S=262144, causal_offset=262143)
    assert L.ds4idx_select_noalloc(ctypes.byref(p), None, FAKE, FAKE, FAKE, 512, FAKE, None,
                                   None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_select_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 512, None, None,
                                   None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_select_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, 0, FAKE, None,
                                   None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_select_noalloc(ctypes.byref(p), FAKE_MIS, FAKE, FAKE, FAKE, 512, FAKE, None,
                                   None) == ds.ERR_INVALID_ARG
    assert L.ds4idx_select_noalloc(None, FAKE, FAKE, FAKE, FAKE, 512, FAKE, None, None) == ds.ERR_INVALID_ARG
    # workspace beyond the scratch array: refused with its own status, no HIP call made
    big = _prob(B=64, T=1, S=1 << 20, causal_offset=(1 << 20) - 1)
    assert ds.workspace_bytes(big, 512) > ds.NOALLOC_SCRATCH_BYTES
    assert L.ds4idx_select_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 512, FAKE, None,
                                   None) == ds.ERR_SCRATCH
    assert ds.workspace_bytes(p, 512) <= ds.NOALLOC_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define DS4IDX_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == ds.NOALLOC_SCRATCH_BYTES


def test_prefill_split_switch_and_workspace():
    # The 2048-token ragged prefill budget (1024/512/256/256 new tokens on
    # caches of 32768/16384/8192/8192 keys): the prefill kernel with key parts
    # of 8192 by default, which need workspace; none with parts off.
    tq, sk = [1024, 512, 256, 256], [32768, 16384, 8192, 8192]
    v = _vprob(B=4, total_q=sum(tq), total_k=sum(sk), max_k=max(sk))
    prev = ds.set_prefill_split(0)
    try:
        assert ds.get_prefill_split() == 0
        auto = ds.varlen_workspace_bytes(v, 512)
        assert auto >= 2048 * 4 * 512 * 8  # counters, counts and 4 lists of k entries per row
        assert _vselect(v) == ds.ERR_WORKSPACE  # parts need a workspace; refused before any HIP call
        ds.set_prefill_split(-1)
        assert ds.get_prefill_split() == -1 and ds.varlen_workspace_bytes(v, 512) == 0
        ds.set_prefill_split(5000)
        assert ds.varlen_workspace_bytes(v, 512) == auto  # same layout: always 4 part slots per row
        # short caches: a single part, no workspace
        short = _vprob(B=4, total_q=2048, total_k=4 * 4096, max_k=4096)
        ds.set_prefill_split(0)
        assert ds.varlen_workspace_bytes(short, 512) == 0
        # a large batch balances without parts
        big = _vprob(B=2, total_q=8192, total_k=2 * 65536, max_k=65536)
        assert ds.varlen_workspace_bytes(big, 512) == 0
        ds.set_prefill_split(4096)
        assert ds.varlen_workspace_bytes(big, 512) > 0
    finally:
        ds.set_prefill_split(prev)
