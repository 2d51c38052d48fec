"""Build libkvq.so (the HIP kernels and the C ABI of include/kvq.h) in-tree
for gfx950 with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.hip", "kvq_quantize.hip", "kvq_decode_valu.hip", "kvq_decode_mfma.hip", "kvq_certify.hip", "kvq_adaptive.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-pass-failed",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


STAMP = LIB + ".srchash"  # hash of the sources and flags the library was built from


def source_hash() -> str:
    """sha256 over the sources (csrc/, include/kvq.h) and the compiler flags."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(sources(), key=os.path.basename):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    # the flags with the repository's location taken out (the tree is built
    # in one place and may run from another)
    h.update(" ".join(f.replace(ROOT, "<root>") for f in FLAGS).encode())
    return h.hexdigest()


def is_current() -> bool:
    """True when libkvq.so exists and was built from the present sources."""
    if not os.path.exists(LIB) or not os.path.exists(STAMP):
        return False
    with open(STAMP) as fh:
        return fh.read().strip() == source_hash()


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [HIPCC, *FLAGS, *srcs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(LIB + ".tmp", LIB)
    with open(STAMP + ".tmp", "w") as fh:
        fh.write(source_hash() + "\n")
    os.replace(STAMP + ".tmp", STAMP)
    return LIB


def sources():
    return [os.path.join(CSRC, s) for s in os.listdir(CSRC) if s.endswith((".hip", ".hpp", ".h"))] + \
        [os.path.join(ROOT, "include", "kvq.h")]


if __name__ == "__main__":
    print(build(verbose=True))
