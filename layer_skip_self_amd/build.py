"""Build the gfx950 engine library ``liblss.so`` and the streaming-read
ceiling benchmark ``lss_stream`` in-tree with hipcc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblss.so")
SOURCES = ["lss_engine.hip", "lss_router.cpp"]
STREAM = os.path.join(HERE, "lss_stream")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fixed rounding: no contraction of separate multiplies and adds
    "-ffp-contract=off",
    # no packed fp32 math (v_pk_* f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc(flags, dst, sources, verbose):
    tmp = dst + ".tmp"
    cmd = [HIPCC] + flags + ["-o", tmp] + [os.path.join(CSRC, s) for s in sources]
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, dst)


def build(verbose=False):
    """Compile ``liblss.so`` and ``lss_stream`` (always recompiles)."""
    _hipcc(FLAGS, LIB, SOURCES, verbose)
    _hipcc([f for f in FLAGS if f not in ("-fPIC", "-shared")], STREAM, ["lss_stream.hip"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
