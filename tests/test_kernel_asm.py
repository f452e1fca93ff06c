"""The hand-counted LDS waits of the attention kernels, and the absence of
per-lane scratch memory in every kernel, checked on the gfx950 assembly
(CPU only: hipcc cross-compiles).

In the hot loops of the forward, dK/dV and dQ kernels every LDS read is an
inline-assembly ds_read followed later by an explicit `s_waitcnt
lgkmcnt(N)`; the N of each wait is counted by hand from the fixed order of
the reads. A wrong N, or the compiler moving a use above its wait, would let
an instruction read a register whose LDS load has not landed. This test
compiles the kernels to assembly with the library's own flags and walks
each kernel's control-flow graph (basic blocks split at labels and branches),
carrying the LDS reads still pending along every path to a fixed point: a
register written by an LDS read is pending until a wait retires that read
(lgkmcnt(N) retires all but the newest N outstanding reads; other LDS and
scalar operations are ignored, which can only keep more reads pending;
where paths join, the pending lists are merged newest-first, position by
position, which again can only keep more pending), and no instruction may
read or overwrite a pending register.

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


def _step(state, line, bad):
    """Apply one instruction to the pending-read list; report violations."""
    op = line.split()[0]
    args = [x.strip() for x in line[len(op):].split(",")]
    live = set().union(*state) if state else set()
    if op.startswith("ds_read"):
        dst = _regs(args[0])
        used = set()
        for x in args[1:]:
            used |= _regs(x.split()[0] if x else "")
        if (dst | used) & live and bad is not None:
            bad.append(line)
        return state + (frozenset(dst),)
    if op == "s_waitcnt" and "lgkmcnt" in line:
        n = int(re.search(r"lgkmcnt\((\d+)\)", line).group(1))
        return state[len(state) - n:] if n < len(state) else state if n else ()
    used = set()
    for x in args:
        used |= _regs(x.split()[0] if x else "")
    if used & live and bad is not None:
        bad.append(line)
    return state


def _merge(a, b, cap=64):
    """Pending lists of two paths joined: newest-first union per position."""
    n = max(len(a), len(b))
    out = []
    for k in range(1, n + 1):
        x = a[-k] if k <= len(a) else frozenset()
        y = b[-k] if k <= len(b) else frozenset()
        out.append(x | y)
    out.reverse()
    if len(out) > cap:
        out = [frozenset().union(*out[: len(out) - cap + 1])] + out[len(out) - cap + 1:]
    return tuple(out)


def _blocks(lines):
    """Basic blocks of a function body: (label, instructions, successors)."""
    blocks, cur, label = [], [], None
    for ln in lines:
        m = re.match(r"^(\.LBB\w+):", ln)
        if m:
            if cur or label is not None:
                blocks.append([label, cur])
            label, cur = m.group(1), []
            continue
        if not ln or ln.startswith((";", ".")) or ln.endswith(":"):
            continue
        cur.append(ln)
        op = ln.split()[0]
        if op.startswith(("s_branch", "s_cbranch", "s_endpgm")):
            blocks.append([label, cur])
            label, cur = None, []
    if cur or label is not None:
        blocks.append([label, cur])
    index = {lab: i for i, (lab, _) in enumerate(blocks) if lab}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        last = ins[-1].split() if ins else [""]
        nxt = [i + 1] if i + 1 < len(blocks) else []
        if last[0] == "s_endpgm":
            succ.append([])
        elif last[0] == "s_branch":
            succ.append([index[last[1]]])
        elif last[0].startswith("s_cbranch"):
            succ.append([index[last[1]]] + nxt)
        else:
            succ.append(nxt)
    return [ins for _, ins in blocks], succ


def _violations(lines):
    blocks, succ = _blocks(lines)
    entry = [None] * len(blocks)
    entry[0] = ()
    work = [0]
    while work:
        i = work.pop()
        st = entry[i]
        for ln in blocks[i]:
            st = _step(st, ln, None)
        for j in succ[i]:
            new = st if entry[j] is None else _merge(entry[j], st)
            if new != entry[j]:
                entry[j] = new
                work.append(j)
    bad = []
    for i, ins in enumerate(blocks):
        if entry[i] is None:
            continue          # unreachable
        st = entry[i]
        for ln in ins:
            st = _step(st, ln, bad)
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
            assert any(l.startswith("ds_read") for l in body), m.group(1)
            bad = _violations(body)
            assert not bad, (m.group(1), bad[:5])
            checked += 1
    assert checked >= len(KERNELS[src]) * 2, checked    # head_dim 64 and 128


@pytest.mark.timeout(900)
def test_checker_flags_a_weakened_wait(asm_dir):
    """The checker is not vacuous: a copy of the forward kernel whose S-phase
    wait lets two more reads stay pending than the k-step may leave (6
    instead of 4) is reported."""
    import pathlib
    import shutil
    tree = pathlib.Path(asm_dir) / "weak"
    shutil.copytree(B.CSRC, tree / "csrc")
    f = tree / "csrc" / "attn_fwd.hip"
    text = f.read_text()
    assert text.count("        lds_wait<4>();") == 1
    f.write_text(text.replace("        lds_wait<4>();", "        lds_wait<6>();"))
    out = str(tree / "fwd.s")
    cmd = [B.HIPCC, *[c if not c.startswith(f"-I{B.CSRC}") else f"-I{tree / 'csrc'}"
                      for c in B.COMMON],
           "-x", "hip", "-S", "--cuda-device-only", str(f), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    asm = open(out).read()
    m = re.search(r"^(_Z\w*attn_fwd_bf16_kernelILi128E\w*):", asm, re.M)
    end = asm.index(".Lfunc_end", m.end())
    assert _violations([l.strip() for l in asm[m.end():end].splitlines()])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_no_kernel_uses_scratch(src, asm_dir):
    asm = _asm(src, asm_dir)
    names = re.findall(r"^\s+\.name:\s+(_Z\S+)$", asm, re.M)
    priv = [int(x) for x in re.findall(r"^\s+\.private_segment_fixed_size:\s+(\d+)$", asm, re.M)]
    assert names and len(names) == len(priv), src
    bad = {n: b for n, b in zip(names, priv) if b}
    assert not bad, bad
