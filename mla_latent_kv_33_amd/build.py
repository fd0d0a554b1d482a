"""Build libmla.so (the HIP kernels and the C ABI of include/mla.h) in-tree
with hipcc for gfx950.  Each source compiles to its own object in parallel;
the objects are then linked into the shared library."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
SOURCES = ["mla_api.hip", "gemm.hip", "elementwise.hip", "decode_simt.hip",
           "decode_mfma.hip", "absorb.hip", "prefill_mha.hip", "peaks.hip",
           "gemv.hip", "merged.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Wno-inline-asm",
         # no packed-fp32 VALU forms (v_pk_*_f32) anywhere in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return proc.returncode, out


def build(verbose: bool = False, sources=SOURCES, lib=LIB,
          extra_flags=()) -> str:
    """Compile every source and link them into `lib` (libmla.so next to this
    file by default); returns the library path.  Always recompiles.
    `extra_flags` go to every compile (not to the link)."""
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o")
                for s in sources]
        cmds = [[HIPCC, *FLAGS, *extra_flags, "-c", os.path.join(CSRC, s),
                 "-o", o]
                for s, o in zip(sources, objs)]
        jobs = max(1, min(len(cmds), os.cpu_count() or 1, 16))
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        logs = []
        for s, (rc, out) in zip(sources, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {s} ({rc}):\n{out}")
            if out.strip():
                logs.append(out)
        tmp = lib + ".tmp"
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                        *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError(f"hipcc link failed ({rc}):\n{out}")
        if out.strip():
            logs.append(out)
    if verbose and logs:
        print("\n".join(logs), file=sys.stderr)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
