"""The hand-counted LDS waits of the attention kernels, and the absence of
per-lane scratch memory in every kernel, checked on the gfx950 assembly
(CPU only: hipcc cross-compiles).

In the hot loops of the forward, dK/dV and dQ kernels every LDS read is an
inline-assembly ds_read followed later by an explicit `s_waitcnt
lgkmcnt(N)`; the N of each wait is counted by hand from the fixed order of
the reads. A wrong N, or the compiler moving a use above its wait, would let
an instruction read a register whose LDS load has not landed. This test
compiles the kernels to assembly with the library's own flags and walks
each kernel body in order: a register written by an LDS read is pending
until a wait retires that read (lgkmcnt(N) retires all but the newest N
outstanding reads; other LDS and scalar operations are ignored, which can
only keep more reads pending), and no instruction may read or overwrite a
pending register.

Scratch: a run-time index into an array member of a by-value kernel
argument (the segment table) makes the compiler copy the whole argument to
per-lane scratch memory, which cost the dK/dV kernel a quarter of its speed;
every kernel must report a private segment of 0 bytes.
"""

import functools
import re
import subprocess

import pytest

from long_context_kv_amd import build as B

KERNELS = {
    "attn_fwd.hip": ["attn_fwd_bf16_kernel"],
    "attn_bwd.hip": ["attn_bwd_kv_kernel", "attn_bwd_dq_kernel"],
}


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _violations(body):
    pending = []          # register sets of the outstanding LDS reads, oldest first
    bad = []
    for line in body:
        op = line.split()[0]
        args = [a.strip() for a in line[len(op):].split(",")]
        if op.startswith("ds_read"):
            live = set().union(*pending) if pending else set()
            dst = _regs(args[0])
            used = set()
            for a in args[1:]:
                used |= _regs(a.split()[0] if a else "")
            if (dst | used) & live:
                bad.append(line)
            pending.append(dst)
            continue
        if op == "s_waitcnt" and "lgkmcnt" in line:
            n = int(re.search(r"lgkmcnt\((\d+)\)", line).group(1))
            pending = pending[len(pending) - n:] if n < len(pending) else pending
            if n == 0:
                pending = []
            continue
        live = set().union(*pending) if pending else set()
        used = set()
        for a in args:
            used |= _regs(a.split()[0] if a else "")
        if used & live:
            bad.append(line)
    return bad


@functools.lru_cache(maxsize=None)
def _asm(src, tmp):
    out = f"{tmp}/{src}.s"
    cmd = [B.HIPCC, *B.COMMON, "-x", "hip", "-S", "--cuda-device-only", str(B.CSRC / src),
           "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    with open(out) as fh:
        return fh.read()


@pytest.fixture(scope="module")
def asm_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("asm"))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("src", sorted(KERNELS))
def test_inline_lds_reads_are_waited_for(src, asm_dir):
    asm = _asm(src, asm_dir)
    checked = 0
    for name in KERNELS[src]:
        for m in re.finditer(r"^(_Z\w*" + name + r"\w*):", asm, re.M):
            end = asm.index(".Lfunc_end", m.end())
            body = [l.strip() for l in asm[m.end():end].splitlines()]
            body = [l for l in body if l and not l.startswith((";", ".")) and not l.endswith(":")]
            assert any(l.startswith("ds_read") for l in body), m.group(1)
            bad = _violations(body)
            assert not bad, (m.group(1), bad[:5])
            checked += 1
    assert checked >= len(KERNELS[src]) * 2, checked    # head_dim 64 and 128


@pytest.mark.timeout(900)
@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_no_kernel_uses_scratch(src, asm_dir):
    asm = _asm(src, asm_dir)
    names = re.findall(r"^\s+\.name:\s+(_Z\S+)$", asm, re.M)
    priv = [int(x) for x in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)$", asm, re.M)]
    assert names and len(names) == len(priv), src
    bad = {n: b for n, b in zip(names, priv) if b}
    assert not bad, bad
