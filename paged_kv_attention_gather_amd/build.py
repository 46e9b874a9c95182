"""Build libpagedattn.so for gfx950 with hipcc, in the package directory.

    python -m paged_kv_attention_gather_amd.build

compiles csrc/pa_kernels.hip (the attention kernels), csrc/kv_write.hip (the
cache append write) and csrc/pagedattn_api.cpp (the C ABI) into one shared
library next to this file.  Every HIP source is compiled
with packed fp32 VALU ops disabled.
"""
import os
import shutil
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["pa_kernels.hip", "kv_write.hip", "pagedattn_api.cpp"]


def source_digest() -> str:
    """First 16 hex digits of the SHA-256 of every kernel source and header
    (in a fixed order): identifies the code that a set of counters measured."""
    import hashlib
    h = hashlib.sha256()
    files = sorted(os.listdir(CSRC)) + ["../../include/pagedattn.h"]
    for name in files:
        path = os.path.normpath(os.path.join(CSRC, name))
        if os.path.isfile(path):
            h.update(name.encode())
            h.update(open(path, "rb").read())
    return h.hexdigest()[:16]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpagedattn.so)")


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    cc = hipcc()
    tmp = tempfile.mkdtemp(prefix="pagedattn_build_")
    try:
        objs = []
        procs = []
        for src in SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            cmd = [cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        for cmd, pr in procs:
            out, _ = pr.communicate()
            out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
            if pr.returncode != 0:
                raise RuntimeError("hipcc failed:\n%s\n%s" % (" ".join(cmd), out))
            if verbose and out.strip():
                print(out)
        tmp_lib = os.path.join(tmp, LIB_NAME)
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib] + objs
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
        shutil.move(tmp_lib, LIB_PATH)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
