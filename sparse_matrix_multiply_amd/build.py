"""Build libmmac.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every HIP source (csrc/*.hip and the per-type-pair kernel instantiations in
csrc/inst/*.hip) is compiled with hipcc for --offload-arch=gfx950 into
sparse_matrix_multiply_amd/_build/, in parallel, then linked into
sparse_matrix_multiply_amd/libmmac.so; the matrix-instruction rate
microbenchmark (csrc/rate/) becomes libmmac_rate.so.  Usage: python -m sparse_matrix_multiply_amd.build
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmmac.so")
RATE_LIB = os.path.join(HERE, "libmmac_rate.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def sources():
    """Every .hip file under csrc/ and csrc/inst/ (one kernel set per file)."""
    out = []
    for d in (CSRC, os.path.join(CSRC, "inst")):
        out += [os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip")]
    return sorted(out)


def _compile(src, verbose):
    rel = os.path.relpath(src, CSRC)[:-4].replace(os.sep, "_")   # inst/dense_bf16 -> inst_dense_bf16
    obj = os.path.join(OUT, rel + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is expected
    msg = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg and verbose:
        print(msg)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every HIP source for gfx950 and link libmmac.so; returns its path."""
    os.makedirs(OUT, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    # the matrix-instruction rate microbenchmark: a library of its own (measurement only)
    rate_src = os.path.join(CSRC, "rate", "matrix_rate.hip")
    cmd = [HIPCC] + FLAGS + ["-shared", rate_src, "-o", RATE_LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {rate_src}:\n{r.stdout}")
    os.replace(RATE_LIB + ".tmp", RATE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
