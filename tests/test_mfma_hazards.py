"""Wait states around the inline-assembly MFMAs, checked in the built library.

The four-wave kernels issue their MFMAs as inline assembly (accumulators tied to
AGPRs) and make their int4 and 1-bit operand planes with single vector
instructions placed between them.  The compiler does not insert the wait states
that the matrix core needs between a vector instruction writing a VGPR and an
MFMA reading it as a source (two on CDNA3/CDNA4, per the hazard tables of AMD's
instruction set reference), nor between an MFMA writing its accumulators and a
later non-MFMA read of them; the kernels schedule both themselves.  This test
disassembles the device code of the built library (our own build, with the ROCm
tools) and checks, along every control-flow path of every kernel:
- no vector instruction writes a source VGPR of an MFMA within 2 wait states
  before it;
- in the four-wave kernels, no instruction other than an MFMA reads an MFMA's
  accumulators within 19 wait states after it (the longest requirement for a
  16-pass result; the kernels pad 32).
A taken branch is counted as no wait state (conservative)."""
import os
import re
import shutil
import subprocess

import pytest

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
BUNDLER = os.path.join(ROCM, "llvm", "bin", "clang-offload-bundler")
OBJDUMP = os.path.join(ROCM, "llvm", "bin", "llvm-objdump")

_FUNC = re.compile(r"^([0-9a-f]+) <(\S+)>:$")
_ADDR = re.compile(r"//\s*([0-9A-Fa-f]+):")
_TARGET = re.compile(r"<(\S+?)\+0x([0-9a-f]+)>\s*$")
_RANGE = re.compile(r"^([va])\[(\d+):(\d+)\]$")
_ONE = re.compile(r"^([va])(\d+)$")
_BRANCH = re.compile(r"^s_(c)?branch")


def _regs(op, kind):
    op = op.strip()
    m = _RANGE.match(op)
    if m and m.group(1) == kind:
        return set(range(int(m.group(2)), int(m.group(3)) + 1))
    m = _ONE.match(op)
    if m and m.group(1) == kind:
        return {int(m.group(2))}
    return set()


def _operands(text):
    parts = text.split(None, 1)
    if len(parts) < 2:
        return []
    body = re.split(r"\s(?:op_sel|cbsz|blgp|offset|offen|lds|glc|sc0|sc1|nt)", parts[1])[0]
    return [o.strip() for o in body.split(",") if o.strip()]


def _wait_states(text):
    m = re.match(r"s_nop\s+(\d+)", text)
    if m:
        return int(m.group(1)) + 1
    if _BRANCH.match(text):
        return 0
    return 1


class Func:
    def __init__(self, name, start):
        self.name, self.start = name, start
        self.ins = []      # (address, text)
        self.target = {}   # instruction index -> branch target address

    def add(self, addr, line):
        text = line.split("//")[0].strip()
        if not text:
            return
        if _BRANCH.match(text):
            m = _TARGET.search(line)
            assert m and m.group(1) == self.name, line
            self.target[len(self.ins)] = self.start + int(m.group(2), 16)
        self.ins.append((addr, text))

    def finish(self):
        self.index = {a: i for i, (a, _) in enumerate(self.ins)}
        self.preds = [[] for _ in self.ins]
        self.succs = [[] for _ in self.ins]
        for i, (a, t) in enumerate(self.ins):
            op = t.split()[0]
            falls = op not in ("s_branch", "s_endpgm", "s_setpc_b64")
            if falls and i + 1 < len(self.ins):
                self._edge(i, i + 1)
            if i in self.target:
                j = self.index.get(self.target[i])
                assert j is not None, t
                self._edge(i, j)

    def _edge(self, i, j):
        self.succs[i].append(j)
        self.preds[j].append(i)


def _disassemble(lib_path, workdir):
    fat = os.path.join(workdir, "fatbin.bin")
    dev = os.path.join(workdir, "device.co")
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", lib_path, fat], check=True)
    subprocess.run([BUNDLER, "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True)
    out = subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", dev], check=True, capture_output=True, text=True).stdout
    funcs, cur = [], None
    for line in out.splitlines():
        m = _FUNC.match(line)
        if m:
            cur = Func(m.group(2), int(m.group(1), 16))
            funcs.append(cur)
            continue
        if cur is None or not line.startswith("\t"):
            continue
        a = _ADDR.search(line)
        if not a:
            continue
        cur.add(int(a.group(1), 16), line)
    for f in funcs:
        f.finish()
    return funcs


def _is_valu(text):
    return text.startswith("v_") and not text.startswith("v_mfma")


def _mfma_source_hazards(f, need=2):
    """(vector instruction, MFMA, wait states between) with fewer than `need`."""
    bad = []
    for k, (_, t) in enumerate(f.ins):
        if not t.startswith("v_mfma"):
            continue
        src = set().union(*[_regs(o, "v") for o in _operands(t)[1:]])
        stack, seen = [(p, 0) for p in f.preds[k]], set()
        while stack:
            i, w = stack.pop()
            if (i, w) in seen:
                continue
            seen.add((i, w))
            u = f.ins[i][1]
            if _is_valu(u):
                ops = _operands(u)
                if ops and _regs(ops[0], "v") & src:
                    bad.append((u, t, w))
            w2 = w + _wait_states(u)
            if w2 < need:
                stack.extend((p, w2) for p in f.preds[i])
    return bad


def _accumulator_read_hazards(f, need=19):
    """(MFMA, reader, wait states between) for non-MFMA reads of an MFMA's
    accumulators with fewer than `need` wait states after it."""
    bad = []
    for k, (_, t) in enumerate(f.ins):
        if not t.startswith("v_mfma"):
            continue
        dst = _regs(_operands(t)[0], "a")
        stack, seen = [(s, 0) for s in f.succs[k]], set()
        while stack:
            i, w = stack.pop()
            if (i, w) in seen:
                continue
            seen.add((i, w))
            u = f.ins[i][1]
            if not u.startswith("v_mfma"):
                ops = _operands(u)
                # a read: any operand but a VGPR/AGPR destination of an ALU op
                reads = ops[1:] if u.startswith("v_") else ops
                if any(_regs(o, "a") & dst for o in reads):
                    bad.append((t, u, w))
            w2 = w + _wait_states(u)
            if w2 < need:
                stack.extend((s, w2) for s in f.succs[i])
    return bad


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    for tool in (BUNDLER, OBJDUMP):
        if not os.path.exists(tool):
            pytest.skip(f"{tool} not installed")
    if shutil.which("objcopy") is None:
        pytest.skip("objcopy not installed")
    from bit_integer_gemm_amd import _build
    _build.ensure_built()
    return _disassemble(_build.LIB, str(tmp_path_factory.mktemp("disasm")))


def test_every_kernel_was_disassembled(kernels):
    names = [f.name for f in kernels]
    w4 = [n for n in names if "mfma_w4_kernel" in n]
    # 256x256 and 256x192: int8, int4, linear, 1-bit (FP4); 192x256: int8, linear
    assert len(w4) == 10, w4
    assert sum("mfma_gemm_kernel" in n for n in names) >= 9
    for f in kernels:
        if "mfma_w4_kernel" in f.name:
            whole = "Li8ELi8E" in f.name      # FM = FN = 8
            assert sum(t.startswith("v_mfma") for _, t in f.ins) >= (256 if whole else 192), f.name


def test_no_vector_write_within_two_wait_states_of_an_mfma_source(kernels):
    checked, found = 0, []
    for f in kernels:
        checked += sum(t.startswith("v_mfma") for _, t in f.ins)
        found += [(f.name,) + h for h in _mfma_source_hazards(f)]
    assert checked > 5000
    assert not found, found[:10]


def test_four_wave_accumulators_are_read_after_the_mfma_pipeline_drains(kernels):
    found = []
    for f in kernels:
        if "mfma_w4_kernel" in f.name:
            found += [(f.name,) + h for h in _accumulator_read_hazards(f)]
    assert not found, found[:10]


def test_the_checker_finds_a_planted_hazard():
    """The checker itself, on a hand-made listing: a plane made one instruction
    before the MFMA that reads it is reported; two instructions before is not;
    a hazard reached only through a loop's back edge is reported too."""
    def func(lines):
        f = Func("k", 0)
        for i, t in enumerate(lines):
            f.add(4 * i, t)
        f.finish()
        return f
    near = func(["v_and_b32 v4, s2, v8", "s_nop 0",
                 "v_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[12:15], a[0:3]", "s_endpgm"])
    assert len(_mfma_source_hazards(near)) == 1
    far = func(["v_and_b32 v4, s2, v8", "s_nop 1",
                "v_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[12:15], a[0:3]", "s_endpgm"])
    assert _mfma_source_hazards(far) == []
    other = func(["v_and_b32 v20, s2, v8",
                  "v_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[12:15], a[0:3]", "s_endpgm"])
    assert _mfma_source_hazards(other) == []
    loop = func(["s_nop 7",
                 "v_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[12:15], a[0:3]",
                 "s_nop 7",
                 "v_lshlrev_b64 v[12:13], 4, v[12:13]",
                 "s_cbranch_scc1 65532 // <k+0x4>",
                 "s_endpgm"])
    assert len(_mfma_source_hazards(loop)) == 1
    acc = func(["v_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[12:15], a[0:3]", "s_nop 7",
                "v_accvgpr_read_b32 v0, a1", "s_endpgm"])
    assert len(_accumulator_read_hazards(acc)) == 1
    acc_ok = func(["v_mfma_i32_16x16x64_i8 a[0:3], v[4:7], v[12:15], a[0:3]", "s_nop 7", "s_nop 7",
                   "s_nop 7", "v_accvgpr_read_b32 v0, a1", "s_endpgm"])
    assert _accumulator_read_hazards(acc_ok) == []
