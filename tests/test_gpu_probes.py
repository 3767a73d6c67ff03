"""The benchmark's ceiling probes (libds4probe.so) on the GPU: the read probe
touches every 16-byte word of its buffer exactly once (the XOR of its
per-thread folds equals the XOR of all words), the gather probe every word
of every valid indexed row once, and the MFMA probe runs."""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_attention_token_lightning_amd", "libds4probe.so")


def _lib():
    lib = ctypes.CDLL(LIB)
    lib.ds4probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    lib.ds4probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.ds4probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p,
                                    ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("words,blocks", [(4 * (1 << 20) + 36, 256), (1000, 3), (4, 1)])
def test_read_probe_reads_every_word_once(words, blocks):
    # words 32-bit words (a multiple of 4: whole 16-byte pieces)
    lib = _lib()
    g = np.random.Generator(np.random.PCG64(words))
    host = g.integers(0, 2 ** 32, words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(blocks * 512, dtype=torch.int32, device="cuda")
    st = lib.ds4probe_hbm_read(buf.data_ptr(), words * 4, sink.data_ptr(), blocks,
                               ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_mfma_probe_runs():
    lib = _lib()
    sink = torch.zeros(4 * 256, dtype=torch.float32, device="cuda")
    st = lib.ds4probe_mfma(16, 4, sink.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert np.all(np.isfinite(s)) and np.all(s > 0)  # positive operands near 1


@pytest.mark.parametrize("row_bytes,nrows,n,blocks", [(1152, 5000, 100003, 256), (2048, 64, 999, 7), (16, 3, 5, 1)])
def test_gather_probe_reads_every_indexed_row_once(row_bytes, nrows, n, blocks):
    lib = _lib()
    g = np.random.Generator(np.random.PCG64(n))
    rows = g.integers(0, 2 ** 32, (nrows, row_bytes // 4), dtype=np.uint32)
    idx = g.integers(-2, nrows + 3, n).astype(np.int32)  # a few out of range: skipped
    rbuf = torch.from_numpy(rows.view(np.int32)).cuda()
    ibuf = torch.from_numpy(idx).cuda()
    sink = torch.zeros(blocks * 512, dtype=torch.int32, device="cuda")
    st = lib.ds4probe_gather(rbuf.data_ptr(), row_bytes, nrows, ibuf.data_ptr(), n, sink.data_ptr(), blocks,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    valid = idx[(idx >= 0) & (idx < nrows)]
    want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(rows[valid], axis=1)) if len(valid) else np.uint32(0)
    assert got == want
