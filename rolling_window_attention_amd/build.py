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
before it is assembled: no other instruction of those kernels may name a0..a63,
and the kernels must be granted at least 64 accumulation registers.  The whole
file is also checked for packed-fp32 VALU instructions, which the build
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
PLAIN_SOURCES = ["api.hip", "rope_roll.hip"]
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


def check_attention_asm(asm_text):
    """Raise if the compiler touched a0..a63 in the attention kernels, if those
    kernels were granted fewer than 64 accumulation registers, or if any
    packed-fp32 VALU instruction was emitted."""
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
