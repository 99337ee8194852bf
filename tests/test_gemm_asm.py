"""Static check of the NS GEMM's gfx950 assembly (CPU only: hipcc emits it).

The GEMM issues its LDS fragment reads as inline ds_read_b128 (and, for the
apply's [k][n] operand, ds_read_b64_tr_b16), which the
compiler does not track with the LDS counter: it treats the destination
registers as written when the asm issues. A compiler-inserted copy or any
other use of such a register before the explicit `s_waitcnt lgkmcnt(0)`
would read (or be clobbered by) data still in flight, silently. This test
compiles the kernel source the way the library build does and checks, for
every ns_gemm_kernel instantiation, that
  * no instruction other than the reads themselves names a register with an
    inline read in flight, and
  * no inline read is in flight at a label or a branch (control-flow joins
    are where register allocation places copies).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


REG = re.compile(r"\b([va])(?:\[(\d+):(\d+)\]|(\d+)\b)")


def regs_of(operands: str):
    out = set()
    for kind, lo, hi, one in REG.findall(operands):
        if one:
            out.add((kind, int(one)))
        else:
            out.update((kind, r) for r in range(int(lo), int(hi) + 1))
    return out


def check_function(lines):
    """Returns a list of violations for one kernel's assembly lines."""
    pending = set()
    in_asm = False
    bad = []
    for n, raw in enumerate(lines):
        line = raw.split(";")[0].strip() if not raw.lstrip().startswith(";;#ASM") else raw.strip()
        if raw.strip().startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if raw.strip().startswith(";;#ASMEND"):
            in_asm = False
            continue
        if not line:
            continue
        if line.endswith(":"):
            if pending:
                bad.append(f"line {n}: label {line} with inline LDS reads in flight")
            continue
        op, _, rest = line.partition(" ")
        if op.startswith("s_waitcnt"):
            if re.search(r"lgkmcnt\(0\)", rest):
                pending.clear()
            continue
        if in_asm and op in ("ds_read_b128", "ds_read_b64_tr_b16"):
            dst, _, addr = rest.partition(",")
            if regs_of(addr) & pending:
                bad.append(f"line {n}: address of an inline read is in flight: {line}")
            pending |= regs_of(dst)
            continue
        if op.startswith("s_cbranch") or op == "s_branch" or op == "s_endpgm":
            if pending:
                bad.append(f"line {n}: {op} with inline LDS reads in flight")
            continue
        hit = regs_of(rest) & pending
        if hit:
            bad.append(f"line {n}: '{line}' touches in-flight registers {sorted(hit)[:4]}")
    return bad


@pytest.fixture(scope="module")
def gemm_asm(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "ns_gemm.s"
    src = os.path.join(ROOT, "muonclip_step_amd", "csrc", "ns_gemm.hip")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "muonclip_step_amd", "csrc"),
           "--cuda-device-only", "-S", src, "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def kernels(asm: str):
    out = {}
    cur, body = None, []
    for line in asm.splitlines():
        m = re.match(r"^(_ZN2mc14ns_gemm_kernel\S*):", line)
        if m:
            cur, body = m.group(1), []
            continue
        if cur is not None:
            body.append(line)
            if line.strip().startswith("s_endpgm"):
                out[cur] = body
                cur = None
    return out


def test_checker_flags_a_planted_copy():
    # a copy of a register whose read is still in flight, then the wait
    planted = [";;#ASMSTART", "ds_read_b128 v[2:5], v33", ";;#ASMEND",
               "v_mov_b64_e32 v[10:11], v[2:3]", "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert check_function(planted)
    clean = [";;#ASMSTART", "ds_read_b128 v[2:5], v33", ";;#ASMEND",
             "s_waitcnt lgkmcnt(0)", "v_mov_b64_e32 v[10:11], v[2:3]", "s_endpgm"]
    assert not check_function(clean)
    at_label = [";;#ASMSTART", "ds_read_b128 v[2:5], v33", ";;#ASMEND", ".LBB0_1:",
                "s_waitcnt lgkmcnt(0)", "s_endpgm"]
    assert check_function(at_label)


def test_ns_gemm_inline_reads_are_waited_before_use(gemm_asm):
    ks = kernels(gemm_asm)
    assert len(ks) >= 12, sorted(ks)
    problems = {}
    for name, body in ks.items():
        assert any("ds_read_b128" in l for l in body), name
        if "ILi1EEEv" in name:   # the apply instantiations read B with transposing reads
            assert any("ds_read_b64_tr_b16" in l for l in body), name
        bad = check_function(body)
        if bad:
            problems[name] = bad[:5]
    assert not problems, problems
