"""Build libattn.so (the HIP kernels + C ABI) in-tree with hipcc for gfx950.

    python -m transformer_scaled_dot_03_amd.build

The library is written next to this file; the Python binding loads it from
there.  Build happens on any host with ROCm (no GPU needed: hipcc
cross-compiles for gfx950).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libattn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["attn_fwd_kernel.hip", "attn_bwd_kernel.hip", "attn_decode_kernel.hip", "attn_gemm_kernel.hip",
           "attn_mha.hip", "attn_api.hip"]
# libraries each target links beyond the HIP runtime
LINK: dict[str, list[str]] = {}
# measurement aid for the benchmark: pure matrix-core loop (include/mfma_probe.h)
PROBE_LIB_PATH = os.path.join(PKG, "libmfma_probe.so")
PROBE_SOURCES = ["mfma_probe.hip"]
# test-only copy of the library whose forward waits for every K/V tile load
# before reading LDS (no load overlaps compute): the race check of the staging
SERIAL_TEST_LIB_PATH = os.path.join(PKG, "libattn_serial_test.so")
TARGETS = [(LIB_PATH, SOURCES), (PROBE_LIB_PATH, PROBE_SOURCES)]
TEST_TARGETS = [(SERIAL_TEST_LIB_PATH, SOURCES, ["-DATTN_FWD_TEST_SERIAL_STAGING=1", "-DATTN_BWD_TEST_SERIAL_STAGING=1",
                                                 "-DATTN_GEMM_TEST_SERIAL_STAGING=1"])]
ARCH = "gfx950"

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the device code (kept out on
# purpose; hipcc's host pass warns that it does not know the feature).
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libattn.so")


def build(verbose: bool = False, extra_flags: list[str] | None = None, tests: bool = True) -> str:
    """Compile every library (always recompiles), and the test-only libraries
    unless tests=False; return the attention library's path."""
    for path, sources in TARGETS:
        _build_one(path, sources, verbose, extra_flags)
    if tests:
        for path, sources, flags in TEST_TARGETS:
            _build_one(path, sources, verbose, [*(extra_flags or []), *flags])
    return LIB_PATH


def _build_one(lib_path: str, sources: list[str], verbose: bool, extra_flags: list[str] | None) -> None:
    srcs = [os.path.join(CSRC, s) for s in sources]
    fd, tmp = tempfile.mkstemp(prefix=".lib.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", *srcs, "-o", tmp,
           *LINK.get(os.path.basename(lib_path), [])]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed (%d):\n%s\n%s" % (res.returncode, " ".join(cmd), res.stderr))
        if verbose:
            noise = "is not a recognized feature for this target"
            msg = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
            if msg.strip():
                print(msg, file=sys.stderr)
        # every kernel stub and entry point must resolve: load it now (RTLD_NOW)
        import ctypes
        ctypes.CDLL(tmp, mode=os.RTLD_NOW | os.RTLD_LOCAL)
        os.replace(tmp, lib_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)


if __name__ == "__main__":
    print(build(verbose=True))
