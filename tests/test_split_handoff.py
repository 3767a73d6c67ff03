"""The split-key kernel's cross-workgroup handoff, checked in the gfx950
assembly this source compiles to (no GPU needed).

Every partition publishes its candidate lists and bounds with device-scope
stores, waits for all of its own stores to complete, passes a workgroup
barrier, and only then one lane increments the row's arrival counter; the
workgroup that sees the last increment reads the lists with device-scope loads
issued after the increment returned. The ordering rests on these instruction
properties, so a compiler change that drops one of them fails here:

* every 64-bit global store of the kernel (the lists and bounds are the only
  ones) carries sc1: device scope, written through to the point where all
  XCDs see it;
* the arrival atomic returns its old value, and between the last global store
  before it and the atomic there is an s_barrier preceded by
  s_waitcnt vmcnt(0): every wavefront's stores have completed at device scope;
* every 64-bit global load after the atomic (the merge's list and bound reads)
  carries sc1.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "sparse_attention_token_lightning_amd", "csrc", "split_indexer.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "split.s"
    from sparse_attention_token_lightning_amd import build as B
    flags = [f for f in B.FLAGS if f != "-fPIC"]
    r = subprocess.run([HIPCC, *flags, "-S", "--cuda-device-only", SRC, "-o", str(out)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(text):
    starts = [m.start() for m in re.finditer(r"^_Z\S*split_indexer_kernel\S*:", text, re.M)]
    assert len(starts) == 14, ("{E4M3, bf16} keys x ({uniform, ragged} x three partition lengths "
                               "+ ragged with planned parts)")
    for st in starts:
        body = text[st:]
        yield body[:body.index(".Lfunc_end")].split("\n")


def test_list_stores_are_device_scope(asm):
    for lines in _kernels(asm):
        st = [l for l in lines if re.match(r"\s*global_store_dwordx2\b", l)]
        assert st, "the lists are stored as 64-bit words"
        assert all(" sc1" in l for l in st), [l for l in st if " sc1" not in l]


def test_arrival_follows_completed_stores_and_barrier(asm):
    for lines in _kernels(asm):
        at = [j for j, l in enumerate(lines) if re.match(r"\s*global_atomic_\w+", l)]
        assert len(at) == 1, "one arrival atomic per kernel"
        a = at[0]
        assert re.match(r"\s*global_atomic_add\b.* sc0", lines[a]), "the arrival must return the old count"
        barrier = waited = False
        for l in reversed(lines[:a]):
            if re.match(r"\s*(global_store|global_atomic|buffer_store|flat_store)", l):
                break
            if re.match(r"\s*s_barrier\b", l):
                barrier = True
            elif barrier and re.match(r"\s*s_waitcnt\b.*vmcnt\(0\)", l):
                waited = True
                break
        assert barrier and waited, "stores -> s_waitcnt vmcnt(0) -> s_barrier -> arrival atomic"


def test_merge_loads_are_device_scope(asm):
    for lines in _kernels(asm):
        a = next(j for j, l in enumerate(lines) if re.match(r"\s*global_atomic_\w+", l))
        ld = [l for l in lines[a:] if re.match(r"\s*global_load_dwordx2\b", l)]
        assert ld, "the merge reads the lists as 64-bit words"
        assert all(" sc1" in l for l in ld), [l for l in ld if " sc1" not in l]
