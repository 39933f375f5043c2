"""Build libfa_fwd.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m exact_attention_17_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa_fwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Werror=array-bounds",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


INST = "fa_fwd_inst.hip"  # compiled once per (d_head, dtype, part of the configuration space)
SPACE_PARTS = 4           # kSpaceParts in csrc/fa_internal.h


def units():
    """(source, object name, extra defines) for every compile unit."""
    out = []
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith((".hip", ".cpp")):
            continue
        src = os.path.join(CSRC, f)
        if f == INST:
            for d in (32, 64, 128):
                for f16 in (0, 1):
                    for part in range(SPACE_PARTS):
                        out.append((src, "fa_fwd_inst_d%d_%s_p%d.o" % (d, "fp16" if f16 else "bf16", part),
                                    ["-DFA_INST_D=%d" % d, "-DFA_INST_F16=%d" % f16, "-DFA_INST_PART=%d" % part]))
        else:
            out.append((src, f + ".o", []))
    return out


def sources():
    return sorted({u[0] for u in units()})


def _compile(unit, extra):
    src, objname, defines = unit
    obj = os.path.join(BUILD, objname)
    cmd = [HIPCC] + FLAGS + defines + extra + ["-c", src, "-o", obj]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in p.stdout.splitlines() if "is not a recognized feature" not in ln)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, out))
    return obj, out


def build(jobs=None, extra=(), verbose=False):
    """Compile every source under csrc/ and link libfa_fwd.so.  Returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        # longest units first (the instantiation parts), so the pool drains evenly
        todo = sorted(units(), key=lambda u: u[0].endswith(INST), reverse=True)
        results = list(ex.map(lambda u: _compile(u, list(extra)), todo))
    if verbose:
        for obj, out in results:
            if out.strip():
                print(out)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
