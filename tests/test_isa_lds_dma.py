"""The direct HBM->LDS loads of the built kernels are waited for before any LDS read (CPU only).

The kernels stage a wave's long code streams (and the decode table) with
global_load_lds, whose data lands in LDS asynchronously and is counted by
vmcnt, not by the LDS counter.  An LDS read reached while such a load may
still be in flight would decode stale bits.  This test compiles the library's
kernels for gfx950 to AMD assembly and runs a dataflow pass over each
kernel's control-flow graph: on every path from a global_load_lds to a
ds_read there must be an s_waitcnt whose vmcnt drains that load (vmcnt(n)
with n at most the vector-memory operations issued after it).  The same pass
is run on a planted hazard to show it finds one.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_matvec_amd", "csrc", "kernels.hip")
VMEM = ("global_load", "buffer_load", "global_store", "buffer_store", "global_atomic", "buffer_atomic")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    """The library's kernels compiled for gfx950 to AMD assembly, once for this module."""
    return _assembly(tmp_path_factory.mktemp("isa"))


def _assembly(tmp_path):
    out = str(tmp_path / "kernels.s")
    from decode_matvec_amd.build import FLAGS
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC", "-pthread")]
    cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), *flags, "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail(r.stderr[-2000:])
    return open(out).read()


def _kernels(asm):
    for m in re.finditer(r"^(_Z\S+):\s*;", asm, re.M):
        end = asm.find(".Lfunc_end", m.end())
        yield m.group(1), asm[m.end():end]


def hazards(body):
    """(line, instruction) of LDS reads some path reaches with an LDS DMA not yet drained."""
    lines = [l.split(";")[0].strip() for l in body.split("\n")]
    lines = [l for l in lines if l and not l.startswith(".") or re.match(r"^\.LBB\S+:$", l or "")]
    # basic blocks: split at labels and after branches
    blocks, labels, cur = [], {}, []
    for l in lines:
        if re.match(r"^\.LBB\S+:$", l):
            if cur:
                blocks.append(cur)
            cur = []
            labels[l[:-1]] = len(blocks)
            continue
        cur.append(l)
        if l.split()[0].startswith(("s_branch", "s_cbranch", "s_endpgm", "s_setpc")):
            blocks.append(cur)
            cur = []
    if cur:
        blocks.append(cur)
    # labels map to the index of the block that starts after them
    succ = []
    for i, b in enumerate(blocks):
        op = b[-1].split()[0] if b else ""
        s = []
        if op.startswith(("s_branch", "s_cbranch")):
            tgt = b[-1].split()[-1]
            if tgt in labels:
                s.append(labels[tgt])
        if not op.startswith(("s_branch", "s_endpgm", "s_setpc")) and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    # state: None = no DMA outstanding, else the number of VMEM ops issued since the oldest outstanding DMA
    state_in = [None] * len(blocks)
    visited = [False] * len(blocks)
    found = set()
    work = [0]
    visited[0] = True

    def join(a, b):
        if a is None:
            return b
        if b is None:
            return a
        return min(a, b)   # fewer ops issued since the DMA: a smaller vmcnt is needed to drain it

    while work:
        i = work.pop()
        st = state_in[i]
        for l in blocks[i]:
            op = l.split()[0]
            if op.startswith("global_load_lds") or (op.startswith("buffer_load") and " lds" in l):
                st = 0
            elif op.startswith(VMEM):
                if st is not None:
                    st += 1
            elif op == "s_waitcnt":
                m = re.search(r"vmcnt\((\d+)\)", l)
                if m and st is not None and int(m.group(1)) <= st:
                    st = None
            elif op.startswith(("ds_read", "ds_load")) and st is not None:
                found.add(l)
        for j in succ[i]:
            new = join(state_in[j], st) if visited[j] else st
            if not visited[j] or new != state_in[j]:
                visited[j] = True
                state_in[j] = new
                work.append(j)
    return sorted(found)


def test_dataflow_finds_a_planted_hazard():
    planted = """
        s_mov_b32 m0, s4
        global_load_lds_dwordx4 v[4:5], off
        s_cbranch_scc1 .LBB0_2
        s_waitcnt vmcnt(0)
.LBB0_2:
        ds_read_b32 v1, v2
        s_endpgm
"""
    assert hazards(planted) == ["ds_read_b32 v1, v2"]
    safe = planted.replace("s_cbranch_scc1 .LBB0_2\n", "")
    assert hazards(safe) == []


def test_every_lds_read_waits_for_the_lds_dma(asm):
    checked = 0
    bad = {}
    for name, body in _kernels(asm):
        if "global_load_lds" not in body:
            continue
        checked += 1
        h = hazards(body)
        if h:
            bad[name] = h[:3]
    assert checked >= 20, checked          # matvec, group, dequant and gather instances
    assert not bad, bad


def test_gather_code_base_is_not_sign_extended(asm):
    """Regression: a helper that restated a pointer as wave-uniform widened the signed 32-bit result of
    readfirstlane into the pointer's high word, so the gather's code-plane buffer base became 0xFFFF_xxxxxxxx
    whenever bit 31 of the low word was set (a GPU memory fault).  No gather kernel sign-extends a 32-bit
    value into 64 bits."""
    gathers = [(name, body) for name, body in _kernels(asm) if "gather_kernel" in name]
    assert len(gathers) >= 8, len(gathers)
    bad = [name for name, body in gathers if "s_bfe_i64" in body]
    assert not bad, bad
