"""Build libsage_attn.so in-tree with hipcc for gfx950 (MI355X)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsage_attn.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["prologue.hip", "attn_fwd.hip", "attn_bwd.hip", "sage_abi.cpp"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         # no packed fp32 (v_pk_*_f32) code generation
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (device code is not instrumented): a
# separate build, loaded through SAGE_ATTN_LIBRARY with the sanitizer runtime preloaded, that the
# host ABI tests run under.
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_OUT = os.path.join(BUILD, "sanitize", "libsage_attn.so")


def build(verbose=False, sanitize=False):
    """Compile every source for gfx950 and link the library in-tree (sanitize: the host-sanitized
    build under _build/sanitize, -O1)."""
    bdir = os.path.join(BUILD, "sanitize") if sanitize else BUILD
    target = SANITIZE_OUT if sanitize else OUT
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1"] + SANITIZE if sanitize else FLAGS
    os.makedirs(bdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + flags + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
        if p.returncode != 0:
            failed.append(src)
            print("\n".join(lines), file=sys.stderr)
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = target + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + (SANITIZE[:4] if sanitize else [])
    subprocess.check_call(link + ["-o", tmp] + objs)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
