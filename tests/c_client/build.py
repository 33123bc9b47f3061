"""Build the plain C client of libspec_verify.so (a test program) with gcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "verify_client.c")
BIN = os.path.join(HERE, "verify_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", os.path.join(ROOT, "rejection_sampling_verify_08_amd", "lib"), "-lspec_verify",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../rejection_sampling_verify_08_amd/lib",
           "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("gcc failed:\n" + res.stdout + res.stderr)
    return BIN


if __name__ == "__main__":
    build(verbose=True)
