"""Build the HIP library in-tree with hipcc for gfx950.

The forward kernels are instantiated in several translation units
(csrc/fwd_*.hip) that compile in parallel, then link with the host/ABI unit
(csrc/ssm_scan.hip) into libssm_scan.so next to this file.
"""
import concurrent.futures as cf
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssm_scan.so")
OBJDIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: plain fp32 VALU ops only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


MICRO_SRC = os.path.join(CSRC, "microbench", "rates.hip")
MICRO_EXE = os.path.join(PKG, "ssm_rates_microbench")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(verbose=False, jobs=None):
    """Compile every csrc/*.hip (in parallel) and link libssm_scan.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJDIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda so: _run([HIPCC] + FLAGS + ["-c", "-o", so[1], so[0]]),
                           zip(srcs, objs)))
    tmp = LIB + ".tmp%d" % os.getpid()
    outs.append(_run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    os.replace(tmp, LIB)
    # the rate microbenchmark behind the roofline figures (a separate executable)
    tmp = MICRO_EXE + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-o", tmp, MICRO_SRC])
    os.replace(tmp, MICRO_EXE)
    return LIB


def device_asm(out_dir):
    """Write the gfx950 assembly of each unit into out_dir (for reading the
    generated code)."""
    os.makedirs(out_dir, exist_ok=True)
    res = []
    for s in sources():
        o = os.path.join(out_dir, os.path.basename(s)[:-4] + ".s")
        subprocess.check_call([HIPCC] + FLAGS + ["--cuda-device-only", "-S", "-o", o, s])
        res.append(o)
    return res


if __name__ == "__main__":
    print(build(verbose=True))
