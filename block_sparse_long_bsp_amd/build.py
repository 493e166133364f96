"""Build the HIP library ``libbsp_attn.so`` in-tree for gfx950."""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "bsp_attn.hip")
LIB = os.path.join(PKG, "libbsp_attn.so")
# matrix-core rate probe used by the benchmark's roofline report (not part of the attention ABI)
PROBE_SRC = os.path.join(PKG, "csrc", "mfma_peak.hip")
PROBE_LIB = os.path.join(PKG, "libbsp_mfma_peak.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the K/V copies set M0 in inline assembly (see lds_copy16); the M0 clobber warning is expected
    "-Wno-inline-asm",
    # device code has no NaN operands (scores are finite or -inf by construction),
    # so fmaxf lowers to v_max3_f32 without operand canonicalisation
    "-Xarch_device", "-fno-honor-nans",
    "-I", INCLUDE,
]


def _compile(src, lib, extra=(), verbose=False) -> str:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra) + [src, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError("hipcc failed for %s" % src)
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, lib)
    return lib


def build(extra=(), verbose=False) -> str:
    """Compile ``csrc/bsp_attn.hip`` to ``libbsp_attn.so`` and the matrix-core
    probe ``csrc/mfma_peak.hip`` to ``libbsp_mfma_peak.so`` (always recompiles)."""
    _compile(PROBE_SRC, PROBE_LIB, verbose=verbose)
    return _compile(SRC, LIB, extra, verbose)


if __name__ == "__main__":
    print(build(extra=sys.argv[1:], verbose=True))
