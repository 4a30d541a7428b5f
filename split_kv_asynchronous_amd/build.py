"""Compiles the HIP sources under csrc/ (decode, prefill, calibration, flat GEMM, read probe) into libfd_attn.so (gfx950 only).

Each source is compiled to an object file in its own hipcc process (in
parallel), then the objects are linked into the shared library."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f)
        for f in ("fd_attn.hip", "fd_prefill.hip", "fd_calib.hip", "fd_gemm.hip", "fd_probe.hip")]
LIB = os.path.join(HERE, "libfd_attn.so")
OBJDIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Wall", "-Wno-unused-result",
         # no packed fp32 arithmetic in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device feature flag; that warning is harmless
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    pid = os.getpid()
    objs = [os.path.join(OBJDIR, os.path.basename(s) + ".%d.o" % pid) for s in SRCS]
    cmds = [[HIPCC] + FLAGS + ["-c", "-o", o, s] for s, o in zip(SRCS, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        results = list(ex.map(_run, cmds))
    try:
        for (rc, out), s in zip(results, SRCS):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (os.path.basename(s), out))
            if verbose and out.strip():
                print(out)
        tmp = LIB + ".tmp%d" % pid
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
        if verbose:
            print(" ".join(link), flush=True)
        rc, out = _run(link)
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("link failed:\n" + out)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
