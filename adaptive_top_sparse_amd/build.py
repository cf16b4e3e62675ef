"""Build libtwilight.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Each source compiles to an object in ``_build/`` in parallel, then one link produces the
shared library next to this file, where the Python binding loads it.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(HERE, "libtwilight.so")
SOURCES = ["twilight_api.hip", "cache_kernels.hip", "quest_kernels.hip",
           "estimate_kernels.hip", "topp_kernels.hip", "decode_kernels.hip"]
ARCH = os.environ.get("TWILIGHT_ARCH", "gfx950")
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 forms are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def _compile(src: str, verbose: bool, build_dir: str, extra) -> str:
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = ["hipcc", *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    err = "\n".join(line for line in res.stderr.splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if err and verbose:
        print(err, flush=True)
    return obj


def build(verbose: bool = False, out: str = OUT, defines=(), build_dir: str = BUILD) -> str:
    """Compile and link the library to `out`; `defines` are extra -D flags (tuning
    constants), built in their own `build_dir`."""
    os.makedirs(build_dir, exist_ok=True)
    extra = [f"-D{d}" for d in defines]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), SOURCES))
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
