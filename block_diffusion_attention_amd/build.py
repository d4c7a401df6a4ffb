"""Build libflashblock.so (gfx950) in-tree with hipcc.

Run as ``python -m block_diffusion_attention_amd.build`` or through
``__graft_entry__.build()``. Always recompiles (a few seconds per file,
files compiled in parallel).
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashblock.so")
# the benchmark's streaming-read probe (not part of the FlashBlock ABI)
PROBE_LIB = os.path.join(PKG, "libfbprobe.so")
PROBE_SOURCES = ["probe_stream.hip"]
SOURCES = ["fb_host.hip", "k1_prefix.hip", "k2_block.hip", "k3_decide.hip", "k4_pages.hip", "k5_rows.hip", "k6_sparse.hip", "k7_cache.hip", "k8_proxy.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
    # packed fp32 VALU ops stay off: plain scalar float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return r


def _compile(src, out_dir, extra):
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    _run([HIPCC, *CFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def _link(objs, lib_path):
    tmp = lib_path + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, lib_path)


def build(verbose=True, extra_flags=(), lib_path=LIB, out_dir=OUT_DIR, probe=True):
    """Compile every source and link lib_path (and the benchmark's probe
    library). extra_flags (e.g. -D tuning macros) and another lib_path/out_dir
    serve tuning builds."""
    os.makedirs(out_dir, exist_ok=True)
    extra = list(extra_flags)
    srcs = SOURCES + (PROBE_SOURCES if probe else [])
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, out_dir, extra), srcs)))
    _link([objs[s] for s in SOURCES], lib_path)
    if verbose:
        print("built", lib_path)
    if probe:
        _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
        if verbose:
            print("built", PROBE_LIB)
    return lib_path


if __name__ == "__main__":
    build()
    sys.exit(0)
