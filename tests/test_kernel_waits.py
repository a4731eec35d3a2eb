"""Checks on the gfx950 assembly of the tiled kernels, compiled on the host.

Waits: the kernels keep their next tile's HBM->LDS loads in flight while they
compute, so the compiler must emit no `s_waitcnt vmcnt(N)` before an LDS read
that would wait for loads issued since the workgroup's last barrier (the next
tile's prefetch).  Such waits appear when the compiler's wait insertion cannot
account for an explicit wait (written as asm, or missing on one path round the
loop) and drain the prefetch on every tile.  The label dQ kernel at d = 128
still has two such waits and is listed as known.

Wait states around MFMAs written as inline asm: the compiler sees no matrix
instruction inside asm and inserts none of the wait states the ISA requires
around one.  A vector write of a source register (for instance a copy of a
resident fragment into AGPRs that the compiler places just before) needs 2
wait states before the MFMA reads it; a result needs more than a dozen before
another instruction other than the next MFMA of the same accumulation chain
touches it (20 covers every MFMA size on gfx950).  Missing the first gave
wrong (NaN) key gradients in a reordered dK/dV loop."""
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


MFMA_SRC_WAITS = 2     # vector write of a register -> MFMA reads it
MFMA_RESULT_WAITS = 20  # MFMA writes a register -> another instruction touches it


def _regs(tok):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", tok):
        out |= {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    for m in re.finditer(r"(?<![\w\[:])([va])(\d+)\b", tok):
        out.add((m.group(1), int(m.group(2))))
    return out


def _wait_states(ins):
    m = re.match(r"s_nop\s+(\d+)", ins)
    return int(m.group(1)) + 1 if m else 1


def asm_mfma_hazards(text):
    """{kernel: [(what, wait states, instruction)]} for every MFMA inside an
    inline-asm block with (a) a vector instruction writing one of its source
    registers fewer than MFMA_SRC_WAITS wait states before it, or (b) an
    instruction touching its result registers within MFMA_RESULT_WAITS wait
    states after it, other than a later MFMA accumulating into exactly the same
    registers.  Program order along the listing, within a basic block for (a)."""
    found = {}
    for m in re.finditer(r"\n(_ZN[^\n:]*):[^\n]*\n(.*?)\.Lfunc_end", text, re.S):
        ins, in_asm = [], False
        for raw in m.group(2).split("\n"):
            l = raw.split(";;")[0].strip() if not raw.strip().startswith(";;#ASM") else raw.strip()
            if l.startswith(";;#ASMSTART"):
                in_asm = True
            elif l.startswith(";;#ASMEND"):
                in_asm = False
            elif l.startswith(".LBB"):
                ins.append(("", "label"))
            elif l and not l.startswith((";", ".")):
                ins.append((l.split(";")[0].strip(), "asm" if in_asm else "c"))
        bad = []
        for i, (l, kind) in enumerate(ins):
            if kind != "asm" or not l.startswith("v_mfma"):
                continue
            ops = [o.strip() for o in l.split(None, 1)[1].split(",")]
            dst, src = _regs(ops[0]), _regs(",".join(ops[1:]))
            w = 0
            for j in range(i - 1, -1, -1):
                lj, kj = ins[j]
                if kj == "label" or w >= MFMA_SRC_WAITS:
                    break
                if lj.startswith("v_") and not lj.startswith("v_mfma") and " " in lj and \
                        _regs(lj.split(None, 1)[1].split(",")[0]) & src:
                    bad.append(("source written", w, lj))
                w += _wait_states(lj)
            w = 0
            for lj, kj in ins[i + 1:]:
                if w >= MFMA_RESULT_WAITS:
                    break
                if kj == "label" or lj.startswith("s_") or " " not in lj:
                    w += 0 if kj == "label" else _wait_states(lj)
                    continue
                if lj.startswith("v_mfma"):
                    o2 = [o.strip() for o in lj.split(None, 1)[1].split(",")]
                    chained = _regs(o2[0]) == dst and _regs(o2[3]) == dst and not (_regs(o2[1]) | _regs(o2[2])) & dst
                    if not chained and _regs(lj.split(None, 1)[1]) & dst:
                        bad.append(("result read by an MFMA", w, lj))
                elif _regs(lj.split(None, 1)[1]) & dst:
                    bad.append(("result touched", w, lj))
                w += _wait_states(lj)
        found[m.group(1)] = bad
    return found


@pytest.mark.parametrize("src", SOURCES)
def test_asm_mfma_wait_states(asm, src):
    found = asm_mfma_hazards(asm[src])
    with_asm = [k for k in found if re.search(r"bwd_dkdv|fwd_bf16_wide|bwd_d[qk]", k)]
    assert with_asm, sorted(found)
    bad = {k: v[:3] for k, v in found.items() if v}
    assert not bad, bad


def test_scan_finds_mfma_hazards():
    """The scan itself, on hand-written listings."""
    def listing(body):
        return "\n_ZN4testE: ; @x\n" + body + ".Lfunc_end0:\n"

    mfma = "\t;;#ASMSTART\n\t{nop}v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]\n\t;;#ASMEND\n"
    copy = "\tv_accvgpr_write_b32 a3, v7\n"
    # a copy into a source AGPR right before the MFMA, then with s_nop 1 in front
    assert [b[0] for b in asm_mfma_hazards(listing(copy + mfma.format(nop="")))["_ZN4testE"]] == ["source written"]
    assert asm_mfma_hazards(listing(copy + mfma.format(nop="s_nop 1\n\t")))["_ZN4testE"] == []
    # the result read by a VALU instruction too soon, then after 21 wait states
    use = "\tv_exp_f32 v20, v3\n"
    assert [b[0] for b in asm_mfma_hazards(listing(mfma.format(nop="") + use))["_ZN4testE"]] == ["result touched"]
    settle = "\ts_nop 7\n\ts_nop 7\n\ts_nop 4\n"
    assert asm_mfma_hazards(listing(mfma.format(nop="") + settle + use))["_ZN4testE"] == []
    # the next MFMA of the same chain is fine, one reading the result as a source is not
    assert asm_mfma_hazards(listing(mfma.format(nop="") + mfma.format(nop="")))["_ZN4testE"] == []
    other = "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], v[20:23], v[32:47]\n"
    assert [b[0] for b in asm_mfma_hazards(listing(mfma.format(nop="") + other))["_ZN4testE"]] == \
        ["result read by an MFMA"]
