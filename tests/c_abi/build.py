"""Builds the plain-C caller of the C ABI (closed_form.c) next to its source.

It is compiled as C99 with gcc against include/attn.h and the HIP runtime
headers, and linked to the in-tree libattn.so (found through an $ORIGIN
rpath, so the built tree can move) and to libamdhip64. Run the binary on a
machine with a GPU; it exits 0 when every closed-form check passes.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "closed_form.c")
EXE = os.path.join(HERE, "closed_form")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CFLAGS = ["-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include")]


def build(verbose=False):
    libdir = os.path.join(ROOT, "long_context_decode_kv_amd")
    cmd = (["gcc"] + CFLAGS + [SRC, "-o", EXE + ".tmp", "-L", libdir, "-l:libattn.so",
                               "-Wl,-rpath,$ORIGIN/../../long_context_decode_kv_amd",
                               "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                               "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed for %s:\n%s" % (SRC, r.stderr))
    os.replace(EXE + ".tmp", EXE)
    if verbose:
        print("built", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
