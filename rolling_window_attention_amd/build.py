"""Build librfattn.so in-tree with the ROCm toolchain for gfx950.

One shared library holds the C ABI (include/rfattn.h), the host validation and
bookkeeping, and the three HIP kernel families.  Always recompiles.

api.hip and rope_roll.hip are ordinary hipcc translation units.  window_attn.hip
takes a longer route because its kernels split each lane's 256 vector registers
unevenly between VGPRs and accumulation registers (160 + 96), which the compiler
only does for a per-function IR attribute ("amdgpu-agpr-alloc"); by default it
halves the file (128 + 128) once a kernel uses accumulation registers:

  hipcc --cuda-device-only -emit-llvm -> device bitcode
  set "amdgpu-agpr-alloc" on the attention kernels      (text edit of the IR)
  llc -> gfx950 assembly -> checks below -> assembler -> lld -> code object
  clang-offload-bundler -> fat binary
  hipcc --cuda-host-only -fcuda-include-gpubinary       (host stubs + that binary)

The attention kernels keep the output accumulators in the fixed accumulation
registers a0..a63, written and read only by inline assembly, which the register
allocator does not know about.  The generated assembly is therefore checked
before it is assembled:
  * no other instruction of those kernels may name a0..a63, and the kernels
    must be granted at least 64 accumulation registers;
  * their MFMAs are inline assembly, so the compiler's hazard recognizer does
    not see them: a scan over the control-flow graph requires at least 12 wait
    states (instructions issued, s_nop n counting n+1) between an MFMA writing
    a register and any non-MFMA instruction touching it or an MFMA taking it as
    an A/B operand (12 is what the compiler itself inserts for these MFMAs),
    and 2 between a VALU write and an MFMA reading the register;
  * the whole file has no packed-fp32 VALU instructions, which the build
    disables.
"""
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librfattn.so")
PLAIN_SOURCES = ["api.hip", "rope_roll.hip", "qkv_proj.hip"]
ATTN_SOURCE = "window_attn.hip"
ATTN_KERNEL_PREFIX = "_ZN6rfattn18window_attn_kernel"
ATTN_AGPRS = 96        # a[0:63]: O^T accumulators; 32 more: the Q' fragments
ATTN_FIXED_AGPRS = 64  # a0..a63 are owned by the kernels' inline assembly
ARCH = "gfx950"
CUID = "rfattn_window_attn"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]
# every MFMA builtin (if any) in the VGPR form; the accumulation registers are
# managed by hand
ATTN_DEVICE_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
PACKED_FP32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")
# hipcc's host pass warns that it does not know the packed-fp32 feature: harmless
NOISE = "is not a recognized feature for this target"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build librfattn")


def llvm_tool(name):
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for cand in (os.path.join(rocm, "llvm", "bin", name), os.path.join(rocm, "lib", "llvm", "bin", name)):
        if os.path.exists(cand):
            return cand
    raise RuntimeError(f"{name} not found next to {hipcc()}")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if NOISE not in l)
    if res.returncode != 0:
        raise RuntimeError(f"{os.path.basename(cmd[0])} failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def set_agpr_alloc(ll_text, n):
    """Add "amdgpu-agpr-alloc"="n" to the attribute groups of the attention kernels."""
    groups = set(re.findall(r"define [^\n]*@" + ATTN_KERNEL_PREFIX + r"[^\n]*? (#\d+)\b[^\n]*\{", ll_text))
    if not groups:
        raise RuntimeError("attention kernels not found in the device bitcode")
    out = []
    for line in ll_text.split("\n"):
        m = re.match(r"attributes (#\d+) = \{", line)
        if m and m.group(1) in groups:
            line = re.sub(r' "amdgpu-agpr-alloc"="[^"]*"', "", line)
            line = line.replace("= {", f'= {{ "amdgpu-agpr-alloc"="{n}"', 1)
        out.append(line)
    return "\n".join(out)


MFMA_RESULT_WAIT = 12   # MFMA writes a register -> another instruction touches it
VALU_TO_MFMA_WAIT = 2   # VALU writes a register -> an MFMA reads it
_NO_VDST = ("v_cmp", "v_readlane", "v_readfirstlane", "s_", "ds_write", "buffer_store", "global_store",
            "scratch_store", "flat_store")


def _vregs(tok):
    """Vector registers named by one operand: v5, v[4:7], a3, a[0:3]."""
    tok = tok.split()[0] if tok else tok
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return [f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)]
    return [tok] if re.fullmatch(r"[va]\d+", tok) else []


def mfma_hazards(fn_lines, name):
    """Wait-state hazards around MFMAs in one function's assembly (see module doc)."""
    blocks, cur, lab = [], [], "entry"
    for line in fn_lines:
        code = line.split(";")[0].strip()
        m = re.match(r"^(\.?[\w$.]+):$", code)
        if m:
            blocks.append((lab, cur))
            cur, lab = [], m.group(1)
            continue
        if not code or code.startswith("."):
            continue
        parts = code.split(None, 1)
        ops = [o.strip() for o in parts[1].split(",")] if len(parts) > 1 else []
        cur.append((parts[0], ops))
        if parts[0].startswith("s_cbranch") or parts[0] == "s_branch":  # a branch ends a block
            blocks.append((lab, cur))
            cur, lab = [], f"{lab}+{len(blocks)}"
    blocks.append((lab, cur))
    index = {b[0]: i for i, b in enumerate(blocks)}
    succ = []
    for i, (_, ins) in enumerate(blocks):
        s = [index[o[0]] for mn, o in ins if (mn.startswith("s_cbranch") or mn == "s_branch") and o and o[0] in index]
        last = ins[-1][0] if ins else ""
        if last not in ("s_branch", "s_endpgm", "s_setpc_b64") and i + 1 < len(blocks):
            s.append(i + 1)
        succ.append(s)
    state = [None] * len(blocks)
    state[0] = ({}, {})
    work, problems = [0], set()
    while work:
        b = work.pop()
        mf, vw = dict(state[b][0]), dict(state[b][1])
        for mn, ops in blocks[b][1]:
            if mn.startswith("v_mfma"):
                for k, op in enumerate(ops[1:4]):
                    for r in _vregs(op):
                        if mf.get(r, 0) > 0 and k != 2:  # the C operand is interlocked in hardware
                            problems.add(f"{name}: {mn} takes MFMA result {r} as an A/B operand too early")
                        if vw.get(r, 0) > 0:
                            problems.add(f"{name}: {mn} reads VALU-written {r} too early")
            elif not mn.startswith("s_"):
                for op in ops:
                    for r in _vregs(op):
                        if mf.get(r, 0) > 0:
                            problems.add(f"{name}: {mn} {', '.join(ops)} touches MFMA result {r} too early")
            w = int(ops[0], 0) + 1 if mn == "s_nop" else 1
            for d in (mf, vw):
                for r in list(d):
                    d[r] -= w
                    if d[r] <= 0:
                        del d[r]
            if mn.startswith("v_mfma"):
                for r in _vregs(ops[0]):
                    mf[r] = MFMA_RESULT_WAIT
            elif mn.startswith("v_") and ops and not mn.startswith(_NO_VDST):
                for r in _vregs(ops[0]):
                    vw[r] = VALU_TO_MFMA_WAIT
        for t in succ[b]:
            if state[t] is None:
                state[t] = (dict(mf), dict(vw))
                work.append(t)
                continue
            changed = False
            for old, new in zip(state[t], (mf, vw)):
                for r, x in new.items():
                    if old.get(r, 0) < x:
                        old[r] = x
                        changed = True
            if changed:
                work.append(t)
    return sorted(problems)


def check_attention_asm(asm_text):
    """Raise if the compiler touched a0..a63 in the attention kernels, if those
    kernels were granted fewer than 64 accumulation registers, if an MFMA
    hazard is not covered by enough wait states, or if any packed-fp32 VALU
    instruction was emitted."""
    problems = []
    fn, in_asm, seen = None, False, set()
    for line in asm_text.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            fn, in_asm = m.group(1), False
        if ";;#ASMSTART" in line:
            in_asm = True
            continue
        if ";;#ASMEND" in line:
            in_asm = False
            continue
        code = line.split(";")[0].strip()
        if not code or code.startswith("."):
            continue
        if PACKED_FP32.search(code):
            problems.append(f"packed-fp32 instruction in {fn}: {code}")
        if fn is None or not fn.startswith(ATTN_KERNEL_PREFIX):
            continue
        seen.add(fn)
        if in_asm:
            continue
        for lo, hi in re.findall(r"\ba\[(\d+):(\d+)\]", code):
            if int(lo) < ATTN_FIXED_AGPRS:
                problems.append(f"compiler-generated use of a[{lo}:{hi}] in {fn}: {code}")
        for r in re.findall(r"\ba(\d+)\b", code):
            if int(r) < ATTN_FIXED_AGPRS:
                problems.append(f"compiler-generated use of a{r} in {fn}: {code}")
    if not seen:
        problems.append("attention kernels not found in the generated assembly")
    # wait-state hazards around the MFMAs, per attention kernel
    fns, name = {}, None
    for line in asm_text.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1) if m.group(1).startswith(ATTN_KERNEL_PREFIX) else None
            if name:
                fns[name] = []
            continue
        if name and line.startswith(".Lfunc_end"):
            name = None
        elif name:
            fns[name].append(line)
    for fname, body in fns.items():
        problems += mfma_hazards(body, fname)
    # kernel descriptors: accumulation registers = next_free_vgpr - accum_offset
    for name, body in re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm_text, re.S):
        if not name.startswith(ATTN_KERNEL_PREFIX):
            continue
        nfv = int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", body).group(1))
        acc = int(re.search(r"\.amdhsa_accum_offset (\d+)", body).group(1))
        if nfv - acc < ATTN_FIXED_AGPRS:
            problems.append(f"{name}: only {nfv - acc} accumulation registers allocated")
    if problems:
        raise RuntimeError("attention kernel assembly check failed:\n  " + "\n  ".join(problems[:20]))


def build_attention(td, verbose=False):
    """window_attn.hip -> host object carrying its own gfx950 fat binary."""
    src = os.path.join(CSRC, ATTN_SOURCE)
    bc, ll, asm = (os.path.join(td, "wa" + e) for e in (".bc", ".ll", ".s"))
    dev_o, hsaco, fatbin, host_o = (os.path.join(td, n) for n in ("wa_dev.o", "wa.hsaco", "wa.hipfb", "wa_host.o"))
    _run([hipcc(), *COMMON_FLAGS, *ATTN_DEVICE_FLAGS, f"-cuid={CUID}", "--cuda-device-only", "-emit-llvm",
          "-c", src, "-o", bc], verbose)
    _run([llvm_tool("llvm-dis"), bc, "-o", ll], verbose)
    with open(ll) as f:
        text = f.read()
    with open(ll, "w") as f:
        f.write(set_agpr_alloc(text, ATTN_AGPRS))
    _run([llvm_tool("llc"), "-O3", "-mtriple=amdgcn-amd-amdhsa", f"-mcpu={ARCH}", "--relocation-model=pic",
          "-amdgpu-mfma-vgpr-form=1", ll, "-o", asm], verbose)
    with open(asm) as f:
        check_attention_asm(f.read())
    _run([llvm_tool("clang"), "-x", "assembler", "-target", "amdgcn-amd-amdhsa", f"-mcpu={ARCH}", "-c", asm,
          "-o", dev_o], verbose)
    _run([llvm_tool("lld"), "-flavor", "gnu", "-m", "elf64_amdgpu", "--no-undefined", "-shared", dev_o,
          "-o", hsaco], verbose)
    _run([llvm_tool("clang-offload-bundler"), "-type=o", "-bundle-align=4096",
          f"-targets=host-x86_64-unknown-linux-gnu,hipv4-amdgcn-amd-amdhsa--{ARCH}",
          "-input=/dev/null", f"-input={hsaco}", f"-output={fatbin}"], verbose)
    _run([hipcc(), *COMMON_FLAGS, f"-cuid={CUID}", "--cuda-host-only", "-Xclang", "-fcuda-include-gpubinary",
          "-Xclang", fatbin, "-c", src, "-o", host_o], verbose)
    return host_o


def build(verbose=False):
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="rfattn_build_") as td:
        objs = []
        for name in PLAIN_SOURCES:
            obj = os.path.join(td, name + ".o")
            _run([hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, name), "-o", obj], verbose)
            objs.append(obj)
        objs.append(build_attention(td, verbose))
        _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
