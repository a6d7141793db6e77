"""Build the test-only device library (tests/native/libdevice_sweep.so) with
the library's own compiler flags, so its encoders compile as the kernels'
do.  Called by the repository's build entry point."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libdevice_sweep.so")


def build(verbose: bool = False) -> str:
    from compressed_sparse_kv_append_amd import _build as b
    src = os.path.join(HERE, "device_sweep.hip")
    tmp = LIB + ".tmp"
    cmd = [b.HIPCC, *b.FLAGS, "-shared", "-x", "hip", src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
