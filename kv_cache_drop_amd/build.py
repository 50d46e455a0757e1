"""Build libakv.so (host runtime + gfx950 HIP kernels) in-tree with hipcc."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libakv.so")
SOURCES = ["akv_runtime.cpp", "akv_kernels.hip", "akv_copy.hip", "akv_decode.hip", "akv_tree.cpp"]
ARCH = os.environ.get("AKV_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of the device code (hipcc flag; the host
# pass prints a harmless "not a recognized feature" warning).
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU checks
# of the runtime; each flag is for the host pass only, device code is built
# as usual).  The result goes to a file of its own, loaded only when
# AKV_LIB_PATH names it (with the sanitizer runtime preloaded).
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SANITIZED_LIB = os.path.join(HERE, "libakv_sanitized.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    out = SANITIZED_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [hipcc] + FLAGS + (SANITIZE if sanitize else []) + ["-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
