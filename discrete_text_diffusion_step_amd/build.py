"""Build libdgstep.so for gfx950 with hipcc (cross-compiles without a GPU).

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel),
then linked into discrete_text_diffusion_step_amd/libdgstep.so next to this
file.  Packed-fp32 instructions are disabled for the device code.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdgstep.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result"]


def _compile(src, build_dir=BUILD, defines=()):
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj


def build(verbose=False, out=OUT, defines=(), build_dir=BUILD):
    """Compile and link; `defines` are extra NAME=VALUE preprocessor settings
    (tile-shape knobs of the streaming products), `out` the library path."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def build_host_sanitized(out_dir):
    """A library for checking the host code: dg_api.hip (argument checks,
    workspace carving, launch order) compiled with AddressSanitizer and
    UndefinedBehaviorSanitizer on its host side only, linked with the kernel
    objects of the regular build.  Returns the library path; a program that
    loads it must itself be linked with the same sanitizers (clang)."""
    os.makedirs(out_dir, exist_ok=True)
    if not all(os.path.exists(os.path.join(BUILD, f + ".o")) for f in os.listdir(CSRC) if f.endswith(".hip")):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    obj = os.path.join(out_dir, "dg_api_san.o")
    cmd = [HIPCC] + FLAGS + san + ["-c", os.path.join(CSRC, "dg_api.hip"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized compile failed:\n" + r.stderr)
    kernels = [os.path.join(BUILD, f + ".o") for f in sorted(os.listdir(CSRC))
               if f.endswith(".hip") and f != "dg_api.hip"]
    out = os.path.join(out_dir, "libdgstep_san.so")
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out, obj] + kernels
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitized link failed:\n" + r.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
