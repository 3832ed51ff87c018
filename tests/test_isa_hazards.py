"""MFMA results read too early across a branch: a check on the built gfx950 assembly.

On gfx950 the software keeps a number of independent instructions (wait states) between an
MFMA and the next instruction that reads or overwrites its destination registers; the compiler
pads that distance with `s_nop`. Inside one basic block it does. One case was found where it
did not: a uniform branch over a softmax tail mask, placed right after the last score MFMAs,
left the branch target reading the accumulators one and three wait states after the MFMAs on the
taken path (the library's kernel keeps `s_nop 7` there). The results were wrong,
deterministically, on every first tile of a segment.

This test compiles every HIP source to assembly with the library's own flags and walks each
MFMA's successors over fall-through and taken branches. An access to the MFMA's destination
that is reached across a branch or a label must be at least as far from the MFMA as the
compiler keeps the same kind of access (by MFMA opcode: a VALU or memory read, a write, an MFMA
operand A/B) inside a block in the same compile. Where the compiler marks a register
`implicit-def` on a path (its value is undefined there, so nothing computed from a read of it
on that path can matter), reads of that register on that path are not counted; writes still
are (an MFMA result landing after them would overwrite them). The scanner is itself checked on
a planted case of the failing shape, on its padded form, and on the implicit-def rule.
"""
import concurrent.futures
import os
import re
import shutil
import subprocess

import pytest

from mla_latent_kv_14_amd import build as B

HIPCC = B.HIPCC if os.path.exists(B.HIPCC) else shutil.which("hipcc")

# instructions whose every VGPR operand is read (no destination register)
_STORE = re.compile(r"^(ds_write|ds_store|global_store|buffer_store|flat_store|scratch_store|"
                    r"global_atomic|buffer_atomic|ds_add|ds_max|ds_min)")
FALLBACK = {"16x16": 8, "32x32": 20}  # used only where no compile has an in-block sample


def _regs(tok):
    m = re.fullmatch(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"v(\d+)", tok)
    return {int(m.group(1))} if m else set()


_IMPLICIT = re.compile(r";\s*implicit-def:\s*\$vgpr(\d+)\s*$")


def parse(text):
    """Instructions as (opcode, operands); labels as ("LABEL", name); functions as ("FUNC",);
    the compiler's `implicit-def: $vgprN` notes as ("UNDEF", ["vN"])."""
    ins, labels = [], {}
    for ln in text.split("\n"):
        m = _IMPLICIT.search(ln)
        if m and not ln.split(";")[0].strip():
            ins.append(("UNDEF", ["v" + m.group(1)]))
            continue
        s = ln.split(";")[0].strip()
        if not s:
            continue
        m = re.match(r"^(\.?[\w.$]+):", s)
        if m:
            name = m.group(1)
            if name.startswith(".LBB"):
                labels[name] = len(ins)
                ins.append(("LABEL", [name]))
            elif not name.startswith("."):
                ins.append(("FUNC", [name]))
            continue
        if s.startswith("."):
            continue
        parts = s.replace(",", " ").split()
        ins.append((parts[0], parts[1:]))
    return ins, labels


def _kind(op, args, dst):
    """How an instruction touches the MFMA destination `dst`: 'read', 'write', 'mfma' or None."""
    if op.startswith("v_mfma"):
        src_ab = set().union(set(), *[_regs(x) for x in args[1:3]])
        return "mfma" if src_ab & dst else None
    if op == "s_waitcnt" or op.startswith("s_"):
        return None
    vr = [_regs(x) for x in args]
    if not vr:
        return None
    if _STORE.match(op):
        return "read" if set().union(*vr) & dst else None
    if vr[0] & dst:
        return "write"
    if len(vr) > 1 and set().union(*vr[1:]) & dst:
        return "read"
    return None


def _read_regs(op, args):
    """The VGPRs an instruction reads (an MFMA: its A and B operands)."""
    if op.startswith("v_mfma"):
        return set().union(set(), *[_regs(x) for x in args[1:3]])
    vr = [_regs(x) for x in args]
    if not vr:
        return set()
    return set().union(*vr) if _STORE.match(op) else set().union(set(), *vr[1:])


def _ws(op, args):
    if op in ("LABEL", "FUNC", "UNDEF"):
        return 0
    if op == "s_nop":
        return int(args[0], 0) + 1
    return 1


def _shape(op):
    return "32x32" if "32x32" in op else "16x16"


def in_block_minima(ins):
    """Smallest distance the compiler keeps, inside one block, between an MFMA and the first
    access of each kind to its destination, keyed by (MFMA opcode, kind)."""
    mins = {}
    for i, (op, args) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        dst, w = _regs(args[0]), 0
        for o, a in ins[i + 1:]:
            if o in ("LABEL", "FUNC") or o.startswith("s_cbranch") or o in ("s_branch",
                                                                             "s_endpgm"):
                break
            if o == "UNDEF":
                continue
            k = _kind(o, a, dst)
            if k is not None:
                key = (op, k)
                mins[key] = min(mins.get(key, 1 << 30), w)
                break
            w += _ws(o, a)
    return mins


def cross_branch_violations(ins, labels, mins):
    """Accesses to an MFMA's destination reached across a branch or a label closer to the MFMA
    than the in-block minimum for their kind."""
    bad = []
    for i, (op, args) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        bound = {k: mins.get((op, k), FALLBACK[_shape(op)]) for k in ("read", "write", "mfma")}
        horizon = max(bound.values())
        dst = _regs(args[0])
        # (position, wait states so far, crossed a branch or label, registers undefined here)
        stack, seen = [(i + 1, 0, False, frozenset())], set()
        while stack:
            j, w, crossed, und = stack.pop()
            if j >= len(ins) or w >= horizon or (j, w, crossed, und) in seen:
                continue
            seen.add((j, w, crossed, und))
            o, a = ins[j]
            if o in ("FUNC", "s_endpgm"):
                continue
            if o == "LABEL":
                stack.append((j + 1, w, True, und))
                continue
            if o == "UNDEF":
                stack.append((j + 1, w, crossed, und | (_regs(a[0]) & dst)))
                continue
            k = _kind(o, a, dst)
            if k in ("read", "mfma") and not ((_read_regs(o, a) & dst) - und):
                k = None  # it reads only registers undefined on this path
            if k is not None:
                # MFMA chains that take the destination back as srcC exactly are not accesses
                if crossed and w < bound[k]:
                    bad.append((" ".join([op] + args), " ".join([o] + a), w, bound[k]))
                continue  # the path ends at the first access
            nw = w + _ws(o, a)
            if o.startswith("s_cbranch") or o == "s_branch":
                if a and a[0] in labels:
                    stack.append((labels[a[0]], nw, True, und))
                if o != "s_branch":
                    stack.append((j + 1, nw, True, und))
                continue
            stack.append((j + 1, nw, crossed, und))
    return bad


def merged_minima(texts):
    """In-block minima over several compiles (the compiler applies one rule everywhere)."""
    mins = {}
    for t in texts:
        for k, v in in_block_minima(parse(t)[0]).items():
            mins[k] = min(mins.get(k, v), v)
    return mins


def scan(text, mins=None):
    ins, labels = parse(text)
    return cross_branch_violations(ins, labels, in_block_minima(ins) if mins is None else mins)


# The failing shape (abridged from the variant's assembly): the last score MFMA, a uniform
# branch over a tail mask, and the join reading the accumulator. A padded in-block copy first
# gives the scanner its bound for this opcode.
PLANTED = """
k:
  v_mfma_f32_16x16x32_bf16 v[10:13], v[20:23], v[30:33], v[10:13]
  s_nop 7
  v_add_f32_e32 v40, v10, v11
  v_mfma_f32_16x16x32_bf16 v[74:77], v[86:89], v[66:69], v[94:97]
  s_cmp_gt_i32 s26, 31
  s_cbranch_scc1 .LBB1_170
  v_cmp_gt_i32_e32 vcc, s16, v134
  s_nop 1
  v_cndmask_b32_e32 v152, v146, v152, vcc
  v_cmp_gt_i32_e32 vcc, s16, v137
  s_nop 1
  v_cndmask_b32_e32 v151, v146, v151, vcc
  v_cmp_gt_i32_e32 vcc, s16, v138
  s_nop 1
  v_cndmask_b32_e32 v150, v146, v150, vcc
.LBB1_170:
  v_add_f32_e32 v74, v74, v78
  s_endpgm
"""


def test_scanner_flags_the_planted_case():
    bad = scan(PLANTED)
    assert len(bad) == 1, bad
    mfma, use, w, bound = bad[0]
    assert "v[74:77]" in mfma and use.startswith("v_add_f32_e32 v74") and w == 2 and bound == 8


def test_scanner_passes_the_padded_case():
    padded = PLANTED.replace("  s_cbranch_scc1 .LBB1_170\n", "  s_nop 7\n  s_cbranch_scc1 .LBB1_170\n")
    assert scan(padded) == []


def test_scanner_counts_the_mask_path():
    # with the branch not taken, the mask block's twelve wait states are enough: only the taken
    # edge is reported (moving the target past the mask would leave no violation)
    no_branch = PLANTED.replace("  s_cbranch_scc1 .LBB1_170\n", "")
    assert scan(no_branch) == []


def test_scanner_drops_registers_undefined_on_the_path():
    # the compiler's note that the accumulator's registers are undefined on the taken path ends
    # the check for them there; a register the note leaves out is still checked
    read = PLANTED.replace("  v_add_f32_e32 v74, v74, v78\n", "  v_add_f32_e32 v40, v74, v78\n")
    assert len(scan(read)) == 1
    undef = read.replace("  s_cbranch_scc1 .LBB1_170\n",
                         "  ; implicit-def: $vgpr74\n  s_cbranch_scc1 .LBB1_170\n")
    assert scan(undef) == []
    other = read.replace("  s_cbranch_scc1 .LBB1_170\n",
                         "  ; implicit-def: $vgpr75\n  s_cbranch_scc1 .LBB1_170\n")
    assert len(scan(other)) == 1
    # a write to an undefined register still has to wait for the MFMA's result
    write = undef.replace("  v_add_f32_e32 v40, v74, v78\n", "  v_mov_b32_e32 v74, 0\n")
    assert len(scan(write)) == 1


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_built_kernels_keep_mfma_wait_states_across_branches(tmp_path):
    flags = [f for f in B.FLAGS if f != "-fPIC"]

    def asm(src):
        out = tmp_path / (os.path.basename(src) + ".s")
        r = subprocess.run([HIPCC] + flags + ["--cuda-device-only", "-S", src, "-o", str(out)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        texts = list(ex.map(asm, B.sources()))
    mins = merged_minima([t for _, t in texts])
    n_mfma = 0
    report = []
    for src, text in texts:
        n_mfma += text.count("v_mfma")
        for mfma, use, w, bound in scan(text, mins):
            report.append("%s: %s -> %s after %d wait states (in-block %d)"
                          % (os.path.basename(src), mfma, use, w, bound))
    assert n_mfma > 100  # the sources do hold the MFMA kernels
    assert not report, "\n".join(report[:20])
