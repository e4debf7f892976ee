"""The inline-assembly matrix-core instructions of the wide product kernel,
checked on the built code object (no GPU needed).

The wide product (k_gemm_bf16_wide) keeps two of its six 32-row output blocks
per wave in VGPRs and accumulates them with v_mfma_f32_32x32x16_bf16 written
as inline assembly, which the compiler does not look inside.  The source
brackets those MFMAs with a guard of wait states (four `s_nop 7`) after the
accumulators are zeroed and before the epilogue reads them.  This test
disassembles the library's gfx950 code object and checks, for both
instantiations:

- there are exactly two guards, and every inline (VGPR-accumulator) MFMA lies
  between them;
- between the guards, no instruction other than those MFMAs names any of
  their accumulator VGPRs;
- every branch between the guards lands between them, so no path leaves or
  enters the region except through a guard;
- two inline MFMAs into the same accumulator block are at least 6 MFMAs apart
  in the instruction stream, also around each loop that holds them, as the
  source's fences arrange.
"""
import os
import re
import shutil
import subprocess

import pytest

import newton_schulz_03_amd as nsa

LLVM = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
WIDE = ("_ZN4muon16k_gemm_bf16_wideILb0EEEvNS_9LaunchCtxENS_8GemmArgsE",
        "_ZN4muon16k_gemm_bf16_wideILb1EEEvNS_9LaunchCtxENS_8GemmArgsE")
GUARD = ("s_nop 7",) * 4
INLINE = re.compile(r"\bv_mfma_f32_32x32x16_bf16 v\[(\d+):(\d+)\]")
VRANGE = re.compile(r"\bv\[(\d+):(\d+)\]")
VSINGLE = re.compile(r"\bv(\d+)\b")
ADDR = re.compile(r"//\s*([0-9A-Fa-f]+):")
BRANCH = re.compile(r"^(s_branch|s_cbranch_\w+)\s+(\d+)")


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip(f"{path} not found")
    return path


@pytest.fixture(scope="module")
def disassembly(tmp_path_factory):
    """The gfx950 disassembly of every translation unit of the library."""
    lib = nsa.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("library not built")
    d = tmp_path_factory.mktemp("isa")
    fat = d / "fat.bin"
    subprocess.run([_tool("llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib,
                    str(d / "lib.stripped")], check=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)]
    text = []
    for n, s in enumerate(starts):
        e = starts[n + 1] if n + 1 < len(starts) else len(data)
        b, co = d / f"b{n}.bin", d / f"co{n}.o"
        b.write_bytes(data[s:e])
        subprocess.run([_tool("clang-offload-bundler"), "--unbundle", "--type=o", f"--input={b}",
                        f"--targets={TARGET}", f"--output={co}"], check=True)
        text.append(subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", str(co)],
                                   check=True, capture_output=True, text=True).stdout)
    shutil.rmtree(d, ignore_errors=True)
    return "\n".join(text)


def _function(text, name):
    """(instruction text, address) of every instruction of function `name`."""
    out, inside = [], False
    for line in text.splitlines():
        if re.match(r"^[0-9a-f]+ <", line):
            inside = line.rstrip().endswith(f"<{name}>:")
            continue
        if inside and line.startswith("\t"):
            ins = line.strip().split("//")[0].strip()
            m = ADDR.search(line)
            if ins and m:
                out.append((ins, int(m.group(1), 16)))
    return out


def _vregs(ins):
    ops = ins.split(None, 1)[1] if " " in ins else ""
    regs = set()
    for a, b in VRANGE.findall(ops):
        regs.update(range(int(a), int(b) + 1))
    for a in VSINGLE.findall(VRANGE.sub("", ops)):
        regs.add(int(a))
    return regs


@pytest.mark.parametrize("name", WIDE)
def test_inline_mfma_accumulators_are_guarded(disassembly, name):
    code = _function(disassembly, name)
    assert code, f"{name} not found in the code object"
    mnem = [i for i, _ in code]
    guards = [k for k in range(len(mnem) - 3) if tuple(mnem[k:k + 4]) == GUARD]
    assert len(guards) == 2, guards
    lo, hi = guards[0] + 4, guards[1]  # the region between the guards
    inline = [k for k, ins in enumerate(mnem) if INLINE.match(ins)]
    assert inline and all(lo <= k < hi for k in inline), "an inline MFMA outside the guards"
    blocks = {tuple(map(int, INLINE.match(mnem[k]).groups())) for k in inline}
    acc = set()
    for a, b in blocks:
        acc.update(range(a, b + 1))
    assert len(acc) == 16 * len(blocks) == 128, sorted(blocks)
    inline_set = set(inline)
    for k in range(lo, hi):
        if k in inline_set:
            continue
        touched = _vregs(mnem[k]) & acc
        assert not touched, f"{mnem[k]} names accumulator VGPRs {sorted(touched)}"
    lo_addr, hi_addr = code[lo][1], code[hi][1]
    for k in range(lo, hi):
        m = BRANCH.match(mnem[k])
        if not m:
            continue
        off = int(m.group(2))
        off = off - 65536 if off >= 32768 else off
        target = code[k][1] + 4 + 4 * off
        assert lo_addr <= target <= hi_addr, f"{mnem[k]} at {code[k][1]:#x} leaves the region"


def _min_distance(mfma, cyclic):
    """Fewest MFMAs from an inline MFMA to the next one into the same block,
    along `mfma` (and around it again when it is a loop body)."""
    pos = {}
    for p, ins in enumerate(mfma):
        m = INLINE.match(ins)
        if m:
            pos.setdefault(m.groups(), []).append(p)
    best = None
    for ps in pos.values():
        gaps = [b - a for a, b in zip(ps, ps[1:])]
        if cyclic:
            gaps.append(len(mfma) - ps[-1] + ps[0])
        for g in gaps:
            best = g if best is None else min(best, g)
    return best


@pytest.mark.parametrize("name", WIDE)
def test_dependent_inline_mfmas_are_six_apart(disassembly, name):
    code = _function(disassembly, name)
    mnem = [i for i, _ in code]
    straight = _min_distance([i for i in mnem if i.startswith("v_mfma")], cyclic=False)
    assert straight is not None and straight >= 6, straight
    loops = 0
    for k, (ins, addr) in enumerate(code):  # around each loop that holds inline MFMAs
        m = BRANCH.match(ins)
        if not m:
            continue
        off = int(m.group(2))
        off = off - 65536 if off >= 32768 else off
        if off >= 0:
            continue
        head = next(j for j, (_, a) in enumerate(code) if a == addr + 4 + 4 * off)
        body = [i for i in mnem[head:k + 1] if i.startswith("v_mfma")]
        if any(INLINE.match(i) for i in body):
            loops += 1
            d = _min_distance(body, cyclic=True)
            assert d >= 6, (head, k, d)
    assert loops >= 1
