"""Static checks on the compiled GEMM main loop (CPU only: hipcc cross-compiles
gfx950 device code without a GPU).

The GEMM issues its MFMAs as inline asm so that their order among the loads,
waits and barriers is kept.  The compiler's hazard recognizer does not look
inside asm, so it inserts no wait states between a plain VALU write of a
register (an accumulator being zeroed, a copy) and an asm MFMA that reads it,
nor between an asm MFMA and a plain instruction that reads or overwrites its
result.  Either would read a stale value with no error.  This test compiles
gemm.hip with the library's flags and walks every control-flow path backwards
from each MFMA (and forwards from it) to check the distances, in wait states:

  * VALU writes a register that the MFMA reads:  at least 2 apart
  * the MFMA's result used or overwritten by any non-MFMA instruction: at
    least 18 apart after a 16x16x32 bf16 MFMA and 19 after a 32x32x16 one
    (more than each one's pipeline depth; 19 is the distance the CDNA3 table
    gives for the longest, 16-pass, MFMAs)
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "gemm_epilogue_bf16_amd", "csrc", "gemm.hip")

VALU_TO_MFMA = 2
MFMA_TO_USE = 18
MFMA32_TO_USE = 19


def _regs(tok):
    m = re.match(r"([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([va])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _operands(inst):
    parts = inst.split(None, 1)
    if len(parts) < 2:
        return []
    return [o.strip() for o in parts[1].split(",")]


def _cost(inst):
    if inst.startswith("s_nop"):
        return int(inst.split()[1], 0) + 1
    return 1


class Kernel:
    def __init__(self, name, lines):
        self.name = name
        self.ins = []        # ("I", text) or ("L", label)
        for l in lines:
            s = l.split(";")[0].strip()
            if not s:
                continue
            if s.endswith(":"):
                self.ins.append(("L", s[:-1]))
            elif not s.startswith("."):
                self.ins.append(("I", s))
        self.label_at = {t: k for k, (kind, t) in enumerate(self.ins) if kind == "L"}
        self.branches_to = {}
        for k, (kind, t) in enumerate(self.ins):
            if kind == "I" and t.startswith("s_cbranch") or t.startswith("s_branch"):
                ops = t.split()
                if len(ops) > 1 and ops[1] in self.label_at:
                    self.branches_to.setdefault(ops[1], []).append(k)

    def preds(self, k):
        """Positions whose instruction may run right before position k."""
        out = []
        if self.ins[k][0] == "L":
            out += self.branches_to.get(self.ins[k][1], [])
        if k > 0:
            kind, t = self.ins[k - 1]
            if not (kind == "I" and (t.startswith("s_branch") or t.startswith("s_endpgm"))):
                out.append(k - 1)
        return out

    def succs(self, k):
        kind, t = self.ins[k]
        out = []
        if kind == "I" and (t.startswith("s_branch") or t.startswith("s_cbranch")):
            tgt = t.split()[1]
            if tgt in self.label_at:
                out.append(self.label_at[tgt])
            if t.startswith("s_branch"):
                return out
        if kind == "I" and t.startswith("s_endpgm"):
            return out
        if k + 1 < len(self.ins):
            out.append(k + 1)
        return out

    def walk(self, start, step, budget, visit):
        """Visit instructions within `budget` wait states of `start` along
        every path (step = preds or succs)."""
        seen = {}
        stack = [(n, 0) for n in step(start)]
        while stack:
            k, d = stack.pop()
            if d >= budget or seen.get(k, budget + 1) <= d:
                continue
            seen[k] = d
            kind, t = self.ins[k]
            nd = d
            if kind == "I":
                visit(t, d)
                nd = d + _cost(t)
            stack += [(n, nd) for n in step(k)]


def _kernels(asm):
    out, cur, name = [], None, None
    for l in asm.splitlines():
        m = re.match(r"^(_Z\S*gemm_bf16_kernel\S*):", l)
        if m:
            name, cur = m.group(1), []
            continue
        if cur is not None:
            if l.startswith(".Lfunc_end"):
                out.append(Kernel(name, cur))
                cur = None
            else:
                cur.append(l)
    return out


def _hazards(k):
    found = []
    for pos, (kind, t) in enumerate(k.ins):
        if kind != "I" or not t.startswith("v_mfma"):
            continue
        ops = _operands(t)
        dst = _regs(ops[0])
        srcs = set().union(*(_regs(o) for o in ops[1:]))

        def before(u, d):
            if u.startswith("v_") and not u.startswith("v_mfma"):
                o = _operands(u)
                if o and _regs(o[0]) & srcs:
                    found.append(f"{d} wait states: '{u}' then '{t}'")

        def after(u, d):
            if u.startswith("v_mfma"):
                return
            if any(_regs(o) & dst for o in _operands(u)):
                found.append(f"{d} wait states: '{t}' then '{u}'")

        k.walk(pos, k.preds, VALU_TO_MFMA, before)
        k.walk(pos, k.succs, MFMA32_TO_USE if "32x32" in t else MFMA_TO_USE, after)
    return found


def _compile_asm(tmp_path_factory, defines=()):
    from gemm_epilogue_bf16_amd import build as B

    try:
        cc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "gemm.s")
    cmd = [cc, *B.common_flags(), *B.EXTRA_FLAGS.get("gemm.hip", []), *defines, "-x", "hip",
           "--cuda-device-only", "-S", SRC, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    return _compile_asm(tmp_path_factory)


@pytest.fixture(scope="module")
def gemm_asm_m32(tmp_path_factory):
    """The build option that runs the 256x256 tile on the 32x32x16 MFMA."""
    return _compile_asm(tmp_path_factory, ("-DFMLP_TILE256_M32=1",))


def test_every_gemm_kernel_compiled(gemm_asm):
    ks = _kernels(gemm_asm)
    assert len(ks) >= 8   # 2 tiles x (bf16, geglu, gathered geglu, scaled fp32)
    for k in ks:
        assert sum(1 for kind, t in k.ins if kind == "I" and t.startswith("v_mfma")) > 0, k.name


def test_no_mfma_hazard_in_asm_loop(gemm_asm):
    problems = []
    for k in _kernels(gemm_asm):
        for h in _hazards(k):
            problems.append(f"{k.name[:80]}: {h}")
    assert not problems, "\n".join(problems[:20])


def _kmajor(name):
    """the k-major template argument (last) of a gemm_bf16_kernel symbol"""
    m = re.search(r"ELb[01]ELi(\d)EEEv", name)
    return int(m.group(1)) if m else 0


@pytest.mark.parametrize("m32", [False, True])
def test_tile256_mfma_shape(gemm_asm, gemm_asm_m32, m32):
    # the k-major operand forms (the backward's row contractions) always run
    # on 16x16x32 MFMAs: their transposing reads give 16-column fragments
    ks = [k for k in _kernels(gemm_asm_m32 if m32 else gemm_asm) if "ILi256ELi256E" in k.name
          and (not m32 or _kmajor(k.name) == 0)]
    assert ks
    want = "v_mfma_f32_32x32x16_bf16" if m32 else "v_mfma_f32_16x16x32_bf16"
    for k in ks:
        m = [t for kind, t in k.ins if kind == "I" and t.startswith("v_mfma")]
        assert m and all(t.startswith(want) for t in m), k.name


def test_no_mfma_hazard_with_32x32_tiles(gemm_asm_m32):
    problems = []
    for k in _kernels(gemm_asm_m32):
        for h in _hazards(k):
            problems.append(f"{k.name[:80]}: {h}")
    assert not problems, "\n".join(problems[:20])


def test_checker_sees_a_planted_hazard():
    """The checker itself: a zeroing write right before the MFMA that reads it,
    reached over a branch, and a read of an MFMA result too soon, are found."""
    asm = "\n".join([
        "_Z1x_gemm_bf16_kernel:",
        "  v_accvgpr_write_b32 a3, 0",
        "  s_branch .LBB0_2",
        ".LBB0_1:",
        "  s_nop 7",
        ".LBB0_2:",
        "  v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]",
        "  s_nop 7",
        "  v_accvgpr_read_b32 v8, a2",
        "  s_endpgm",
        ".Lfunc_end0:",
    ])
    (k,) = _kernels(asm)
    h = _hazards(k)
    assert any("v_accvgpr_write_b32 a3" in x for x in h)
    assert any("v_accvgpr_read_b32 v8" in x for x in h)
