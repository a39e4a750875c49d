"""Build the HIP library in-tree with hipcc for gfx950."""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "ssm_scan.hip")
LIB = os.path.join(PKG, "libssm_scan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: plain fp32 VALU ops only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose=False):
    """Compile csrc/ssm_scan.hip into libssm_scan.so next to this file."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp, SRC]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_path):
    """Write the gfx950 assembly of the library (for reading the code generated)."""
    cmd = [HIPCC] + [f for f in FLAGS if f not in ("-shared", "-fPIC")] + [
        "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-o", out_path, SRC]
    subprocess.check_call(cmd)
    return out_path


if __name__ == "__main__":
    print(build(verbose=True))
