"""The tiled kernels keep their next tile's HBM->LDS loads in flight while
they compute: in the gfx950 assembly the compiler emits no `s_waitcnt vmcnt(N)`
before an LDS read that would wait for loads issued since the workgroup's last
barrier (the next tile's prefetch).  Such waits appear when the compiler's
wait insertion cannot account for an explicit wait (written as asm, or missing
on one path round the loop) and drain the prefetch on every tile.  The check
compiles the kernel sources for gfx950 on the host and scans the assembly; the
label dQ kernel at d = 128 still has two such waits and is listed as known."""
import concurrent.futures
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from long_context_blockwise_amd import build as B  # noqa: E402

SOURCES = ("attn_fwd_bf16.hip", "attn_bwd_bf16.hip")
KNOWN = ("bwd_dq_kernelILi128ELi64ELi4ELi2ELi2E",)  # labels, d = 128


def _hipcc():
    try:
        return B._hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc for gfx950 not available")
    out = tmp_path_factory.mktemp("asm")

    def comp(src):
        dst = os.path.join(out, src + ".s")
        cmd = [hipcc, *B.COMMON, *B.DEVICE_FLAGS, "--cuda-device-only", "-S", os.path.join(B.CSRC, src), "-o", dst]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        with open(dst) as f:
            return f.read()

    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(comp, SOURCES)))


def draining_waits(text):
    """{kernel: [(N, loads issued since the last barrier)]} for every
    `s_waitcnt vmcnt(N)` directly before an LDS read with more than N such
    loads."""
    found = {}
    for m in re.finditer(r"\n(_ZN[^\n:]*):[^\n]*\n(.*?)\.Lfunc_end", text, re.S):
        lines = [l.strip() for l in m.group(2).split("\n")]
        lines = [l for l in lines if l and not l.startswith((";", "."))]
        bad = []
        for i, l in enumerate(lines):
            if not (l.startswith("s_waitcnt") and "vmcnt(" in l):
                continue
            if not any(x.startswith("ds_read") for x in lines[i + 1:i + 3]):
                continue
            n = int(re.search(r"vmcnt\((\d+)\)", l).group(1))
            since = 0
            for k in range(i - 1, -1, -1):
                if lines[k].startswith("s_barrier"):
                    break
                if lines[k].startswith(("buffer_load", "global_load")) and lines[k].endswith("lds"):
                    since += 1
            if since > n:
                bad.append((n, since))
        found[m.group(1)] = bad
    return found


@pytest.mark.parametrize("src", SOURCES)
def test_no_wait_drains_the_prefetch(asm, src):
    found = draining_waits(asm[src])
    tiled = [k for k in found if re.search(r"fwd_bf16|fwd_fp8kv|bwd_dq|bwd_dkdv", k)]
    assert len(tiled) >= 8, sorted(found)
    bad = {k: v for k, v in found.items() if v and not any(x in k for x in KNOWN)}
    assert not bad, bad


def test_scan_finds_a_draining_wait():
    """The scan itself: a wait for loads issued after the barrier is reported,
    one that leaves them in flight is not."""
    body = ("\ts_barrier\n\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n"
            "\tbuffer_load_dwordx4 v2, s[0:3], 0 offen lds\n\ts_waitcnt vmcnt({n})\n\tds_read_b128 v[4:7], v0\n")
    for n, expect in ((0, [(0, 2)]), (1, [(1, 2)]), (2, [])):
        text = "\n_ZN4testE: ; @x\n" + body.format(n=n) + ".Lfunc_end0:\n"
        assert draining_waits(text) == {"_ZN4testE": expect}
