"""Host logic of bench.py (no GPU): the one-GPU guard and the gate that
reports counter-derived HBM traffic only for the kernel source it was
measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "--gpus 1" in (r.stdout + r.stderr)


def _summary(path, digest, hbm):
    with open(path, "w") as f:
        f.write("# comment: a line with a colon is not a field\n")
        f.write(f"kernel_code_sha256_16: {digest}\n")
        f.write("launches: 16\n")
        f.write(f"hbm_bytes_per_launch: {hbm}\n")


def test_traffic_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    digest = bench.kernel_digest("mfma_indexer.hip")
    _summary(tmp_path / "same.txt", digest, 123456789)
    assert bench.measured_traffic("same.txt", "mfma_indexer.hip") == 123456789
    # the same figure, taken on another source (a changed kernel): no figure
    _summary(tmp_path / "stale.txt", "0123456789abcdef", 123456789)
    assert bench.measured_traffic("stale.txt", "mfma_indexer.hip") is None
    # a summary for one kernel does not vouch for another kernel's source
    assert bench.measured_traffic("same.txt", "split_indexer.hip") is None
    assert bench.measured_traffic("missing.txt", "mfma_indexer.hip") is None


@pytest.mark.parametrize("summary", ["mfma_select_64k_traffic.txt", "mfma_select_1m_kernel_stats.txt",
                                     "split_decode_256k_traffic.txt", "k_cache_write_256k_traffic.txt",
                                     "sparse_attention_4096_traffic.txt"])
def test_committed_traffic_summaries_parse(summary):
    path = os.path.join(ROOT, "profiles", summary)
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert len(kv["kernel_code_sha256_16"]) == 16
    fetch, write = int(kv["fetch_bytes_per_launch"]), int(kv["write_bytes_per_launch"])
    assert int(kv["hbm_bytes_per_launch"]) == fetch + write > 0


def test_digest_ignores_comments_and_layout_only():
    src = 'int f(int x) {  // doubles\n  return 2 * x; /* no\noverflow */ }\nconst char *s = "a // b";\n'
    same = 'int f(int x) { return 2 * x; }\n// a new comment\nconst char *s = "a // b";'
    changed = 'int f(int x) { return 3 * x; }\nconst char *s = "a // b";'
    literal = 'int f(int x) { return 2 * x; }\nconst char *s = "a  // b";'
    assert bench._code_only(src) == bench._code_only(same)
    assert bench._code_only(src) != bench._code_only(changed)
    assert bench._code_only(src) != bench._code_only(literal)   # inside a literal, text counts


def test_probe_library_exports_its_kernels():
    # the ceiling probes bench.py times live in their own library, outside
    # the indexer's C ABI
    import ctypes
    path = os.path.join(ROOT, "sparse_attention_token_lightning_amd", "libds4probe.so")
    assert os.path.exists(path), "built by __graft_entry__.build()"
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "ds4probe_hbm_read") and hasattr(lib, "ds4probe_mfma") and hasattr(lib, "ds4probe_gather")
    lib.ds4probe_gather.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_void_p,
                                    ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    ok = (ctypes.c_void_p(0x1000), 1152, 10, ctypes.c_void_p(0x2000), 5, ctypes.c_void_p(0x3000), 1, None)
    for i, bad in [(1, 1000), (1, 4096), (2, 0), (4, 0), (6, 0), (0, None), (0, ctypes.c_void_p(0x1008))]:
        args = list(ok)
        args[i] = bad
        assert lib.ds4probe_gather(*args) != 0, (i, bad)
    # argument checks come before any HIP call
    lib.ds4probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_void_p]
    assert lib.ds4probe_hbm_read(ctypes.c_void_p(0x1000), 24, ctypes.c_void_p(0x2000), 1, None) != 0  # not x16
    assert lib.ds4probe_hbm_read(None, 32, ctypes.c_void_p(0x2000), 1, None) != 0
