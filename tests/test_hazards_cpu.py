"""Static check of the wait states the hand-written PV MFMAs rely on.

The fast path of attn_bf16_kernel issues its O^T += V^T P^T products as
inline assembly (accumulators bound to accumulation VGPRs), so the compiler
does not insert the wait states the CDNA4 ISA reference guide requires
around those matrix (XDL) instructions; the kernel supplies them itself
(an `s_nop 1` before each, a fence of 8 x `s_nop 15` before the
accumulators are touched by anything else).  This test compiles
attn_bf16.hip for gfx950 with the library's own flags, walks the assembly of
attn_bf16_kernel<128> and <64> along every control-flow path, and checks:

  (a) a vector-ALU write of a VGPR/AGPR that an inline-asm MFMA reads as
      source A or B is at least 2 wait states before it (a matrix
      instruction writing it: at least 19);
  (b) no instruction other than another inline-asm MFMA with the same
      accumulator reads or writes an inline-asm MFMA's accumulator within
      19 wait states of it (more than the 16 passes of a 32x32x16 MFMA);
  (c) two inline-asm MFMAs into the same accumulator have at least
      2*MT - 1 other MFMAs between them inside a block of straight-line code.

Wait states are counted as one per instruction and N + 1 per `s_nop N`.
A planted-mistake test shows each rule fires on a small hand-written
sequence.
"""
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

RAW_NEED_VALU = 2      # VALU write -> MFMA source A/B read
RAW_NEED_XDL = 19      # MFMA write -> source read, or any other access of its result

REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+))(?!\w)")
LABEL = re.compile(r"^(\.?[A-Za-z_$][\w.$]*):")


def regs(text):
    """The VGPR/AGPR numbers named in an operand string: {('v', n), ('a', n)}."""
    out = set()
    for m in REG.finditer(text):
        kind = m.group(1)
        if m.group(4) is not None:
            out.add((kind, int(m.group(4))))
        else:
            out.update((kind, r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    return out


class Inst:
    def __init__(self, op, args, in_asm):
        self.op = op
        self.args = [a.strip() for a in args.split(",")] if args.strip() else []
        self.in_asm = in_asm

    @property
    def waits(self):
        if self.op == "s_nop":
            return int(self.args[0], 0) + 1
        return 1

    @property
    def is_mfma(self):
        return self.op.startswith("v_mfma")

    @property
    def is_valu(self):
        return self.op.startswith("v_") and not self.is_mfma

    def defs(self):
        """Registers the instruction writes (VGPR/AGPR only)."""
        if not self.args:
            return set()
        op = self.op
        if op.startswith(("global_store", "buffer_store", "scratch_store", "ds_write",
                          "ds_store", "flat_store", "global_load_lds", "buffer_load_lds")):
            return set()
        if op.startswith(("v_cmp", "v_readlane", "v_readfirstlane")) or not (
                op.startswith(("v_", "global_load", "buffer_load", "scratch_load", "ds_read",
                               "ds_load", "flat_load", "global_atomic", "ds_bpermute",
                               "ds_permute", "ds_swizzle"))):
            return set()
        return regs(self.args[0])

    def uses(self):
        """Registers the instruction reads (VGPR/AGPR), or all operands."""
        if not self.args:
            return set()
        if self.defs():
            return set().union(*(regs(a) for a in self.args[1:])) if len(self.args) > 1 else set()
        return set().union(*(regs(a) for a in self.args))

    def touches(self):
        return self.defs() | self.uses()


def parse(asm_text):
    """Instructions and labels of one function: (insts, label -> index)."""
    insts, labels = [], {}
    in_asm = False
    for raw in asm_text.splitlines():
        line = raw.split(";")[0].rstrip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        if raw.strip().startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.strip().startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line.strip():
            continue
        m = LABEL.match(line.strip())
        if m and not raw.startswith("\t"):
            labels[m.group(1)] = len(insts)
            continue
        s = line.strip()
        if s.startswith("."):
            continue
        op, _, args = s.partition(" ")
        insts.append(Inst(op, args, in_asm))
    return insts, labels


def successors(insts, labels, i):
    ins = insts[i]
    out = []
    if ins.op.startswith("s_cbranch") or ins.op == "s_branch":
        tgt = ins.args[0]
        if tgt in labels:
            out.append(labels[tgt])
        if ins.op == "s_branch":
            return out
    if ins.op == "s_endpgm" or ins.op == "s_setpc_b64":
        return out
    if i + 1 < len(insts):
        out.append(i + 1)
    return out


def predecessors_map(insts, labels):
    preds = {i: [] for i in range(len(insts))}
    for i in range(len(insts)):
        for j in successors(insts, labels, i):
            preds[j].append(i)
    return preds


def writers_within(insts, preds, j, targets, limit):
    """Instructions on some path before j that write one of `targets`, with the
    wait states between them and j; paths are followed back until `limit`
    wait states have accumulated."""
    found = []
    stack = [(p, 0) for p in preds[j]]
    seen = {}
    while stack:
        i, dist = stack.pop()
        if dist >= limit or seen.get(i, limit + 1) <= dist:
            continue
        seen[i] = dist
        ins = insts[i]
        if ins.defs() & targets:
            found.append((i, dist))
            continue
        for p in preds[i]:
            stack.append((p, dist + ins.waits))
    return found


def accesses_within(insts, labels, j, targets, limit):
    """Instructions on some path after j that read or write `targets`, within
    `limit` wait states of j."""
    found = []
    stack = [(s, 0) for s in successors(insts, labels, j)]
    seen = {}
    while stack:
        i, dist = stack.pop()
        if dist >= limit or seen.get(i, limit + 1) <= dist:
            continue
        seen[i] = dist
        ins = insts[i]
        if ins.touches() & targets:
            found.append((i, dist))
            continue
        for s in successors(insts, labels, i):
            stack.append((s, dist + ins.waits))
    return found


def check(insts, labels, mt):
    """Violations of rules (a), (b), (c) for the inline-asm MFMAs."""
    preds = predecessors_map(insts, labels)
    bad = []
    asm_mfma = [i for i, x in enumerate(insts) if x.in_asm and x.is_mfma]
    for j in asm_mfma:
        m = insts[j]
        dst, src_a, src_b = regs(m.args[0]), regs(m.args[1]), regs(m.args[2])
        # (a) writes of the A/B sources shortly before
        for i, dist in writers_within(insts, preds, j, src_a | src_b, RAW_NEED_XDL):
            w = insts[i]
            need = RAW_NEED_XDL if w.is_mfma else (RAW_NEED_VALU if w.is_valu else 0)
            if dist < need:
                bad.append("(a) %s at %d writes a source of the MFMA at %d, %d wait states before "
                           "(needs %d)" % (w.op, i, j, dist, need))
        # (b) other accesses of the accumulator shortly after
        for i, dist in accesses_within(insts, labels, j, dst, RAW_NEED_XDL):
            o = insts[i]
            if o.in_asm and o.is_mfma and regs(o.args[0]) == dst and regs(o.args[3]) == dst:
                continue  # the next accumulation into it (rule (c) below)
            bad.append("(b) %s at %d touches the accumulator of the MFMA at %d, %d wait states "
                       "after it" % (o.op, i, j, dist))
        # (c) the next inline-asm MFMA into the same accumulator, in straight-line code
        between = 0
        for i in range(j + 1, len(insts)):
            o = insts[i]
            if o.op.startswith(("s_cbranch", "s_branch", "s_endpgm")):
                break
            if o.in_asm and o.is_mfma:
                if regs(o.args[0]) == dst:
                    if between < 2 * mt - 1:
                        bad.append("(c) MFMAs at %d and %d accumulate into the same registers "
                                   "with %d MFMAs between" % (j, i, between))
                    break
                between += 1
            elif o.is_mfma:
                between += 1
    return bad


def kernel_asm(asm, name):
    start = asm.index("\n" + name + ":")
    end = asm.index("s_endpgm", start)
    # through the end of the function (the fallback path sits after the first s_endpgm)
    nxt = asm.find("\n\t.section", end)
    fend = asm.find(".Lfunc_end", start)
    return asm[start:fend if fend != -1 else nxt]


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    from block_sparse_video_solattn_amd import build
    out = str(tmp_path_factory.mktemp("asm") / "attn_bf16.s")
    cmd = [build.hipcc()] + [f for f in build.flags() if f not in ("-shared", "-fPIC")] + [
        "--cuda-device-only", "-S", "-x", "hip",
        os.path.join(build.CSRC, "attn_bf16.hip"), "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-4000:]
    with open(out) as f:
        return f.read()


@pytest.mark.parametrize("D,n_asm_mfma", [(128, 32), (64, 16)])
def test_pv_mfma_wait_states(device_asm, D, n_asm_mfma):
    name = "_ZN7solattn16attn_bf16_kernelILi%dEEEvNS_8AttnArgsE" % D
    insts, labels = parse(kernel_asm(device_asm, name))
    asm_mfma = [x for x in insts if x.in_asm and x.is_mfma]
    fences = sum(1 for i in range(len(insts) - 7)
                 if all(insts[i + k].in_asm and insts[i + k].op == "s_nop"
                        and insts[i + k].args == ["15"] for k in range(8)))
    # the checks must have something to check: every PV MFMA of the two
    # halves of the unrolled loop body, and the fence after the loop
    assert len(asm_mfma) == n_asm_mfma, len(asm_mfma)
    assert fences >= 1
    bad = check(insts, labels, D // 32)
    assert not bad, "\n".join(bad[:20])


SNIPPET = """
f:
\tv_cvt_pk_bf16_f32 v10, v1, v2
\t;;#ASMSTART
\t{nop}
\tv_mfma_f32_32x32x16_bf16 a[0:15], a[32:35], v[8:11], a[0:15]
\t;;#ASMEND
\t;;#ASMSTART
\ts_nop 1
\tv_mfma_f32_32x32x16_bf16 a[16:31], a[32:35], v[12:15], a[16:31]
\t;;#ASMEND
\t{after}
\ts_endpgm
"""


ASM_MFMA0 = ("\t;;#ASMSTART\n\ts_nop 1\n"
             "\tv_mfma_f32_32x32x16_bf16 a[0:15], a[32:35], v[12:15], a[0:15]\n\t;;#ASMEND")


@pytest.mark.parametrize("nop,after,mt,rule", [
    ("s_nop 1", "s_nop 0", 4, None),                                # correct
    ("s_nop 0", "s_nop 0", 4, "(a)"),                               # one wait state short
    ("s_nop 1", "v_accvgpr_read_b32 v3, a20", 4, "(b)"),            # result read too early
    ("s_nop 1", "v_mov_b32 v9, 0", 4, None),                        # unrelated register: fine
    ("s_nop 1", ASM_MFMA0.lstrip("\t"), 4, "(c)"),                  # same accumulator, 1 MFMA apart
    ("s_nop 1", ASM_MFMA0.lstrip("\t"), 1, None),                   # ... allowed when MT = 1
])
def test_checker_catches_planted_mistakes(nop, after, mt, rule):
    insts, labels = parse(SNIPPET.format(nop=nop, after=after))
    bad = check(insts, labels, mt)
    if rule is None:
        assert not bad, bad
    else:
        assert any(b.startswith(rule) for b in bad), bad


def test_checker_catches_close_accumulations():
    text = "f:\n" + "".join(
        "\t;;#ASMSTART\n\ts_nop 1\n\tv_mfma_f32_32x32x16_bf16 a[%d:%d], a[64:67], v[8:11], a[%d:%d]\n"
        "\t;;#ASMEND\n" % (16 * r, 16 * r + 15, 16 * r, 16 * r + 15) for r in (0, 1, 0)) + "\ts_endpgm\n"
    insts, labels = parse(text)
    assert any(b.startswith("(c)") for b in check(insts, labels, 4))
    assert not [b for b in check(insts, labels, 1) if b.startswith("(c)")]
