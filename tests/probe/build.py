"""Build tests/probe/libmoe_probe.so: the test-only probe entry points
(probe_api.cpp) linked with the library's kernel objects.  Run after the main
build (mixture_experts_layer_13_amd/build.py), whose objects in _build/ it
links; the public libmoe.so is not touched."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from mixture_experts_layer_13_amd import build as pkg_build  # noqa: E402

LIB = os.path.join(HERE, "libmoe_probe.so")
KERNEL_SOURCES = [s for s in pkg_build.SOURCES if s != "moe_api.cpp"]


def build(verbose=False):
    objs = [os.path.join(pkg_build.OBJ_DIR, os.path.splitext(s)[0] + ".o") for s in KERNEL_SOURCES]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"kernel objects missing (run the main build first): {missing}")
    obj = os.path.join(pkg_build.OBJ_DIR, "probe_api.o")
    cmd = [pkg_build.HIPCC, "-x", "hip"] + pkg_build.FLAGS + \
        ["-I", pkg_build.CSRC, "-c", os.path.join(HERE, "probe_api.cpp"), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on probe_api.cpp:\n" + r.stdout + r.stderr)
    tmp = LIB + ".tmp"
    subprocess.run([pkg_build.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, obj] + objs,
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
