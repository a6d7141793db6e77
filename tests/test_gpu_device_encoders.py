"""The kernels' own encoders over every finite fp32 bit pattern, on the GPU:
the E2M1 code of the FP4 planes [P1 §3.1 (per-group scale, values relative
to it); P2 四、"P4 main KV" (E2M1)] and the bf16 rounding of the window rows.

A test-only kernel (tests/native/device_sweep.hip, built with the library's
flags from the library's device.hpp) reduces the 4,278,190,080 codes of each
encoder to an order-independent checksum, sum of (code + 1) * splitmix64
finaliser(pattern) mod 2^64; the oracle's encoders give the stored values
(tests/golden/encoder_checksums.json, re-derived by the CPU test of the
exhaustive tool), so one differing code anywhere changes a checksum.
"""
import ctypes as C
import json
import os

import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "native", "libdevice_sweep.so")


def test_device_encoders_match_the_oracle_on_every_fp32_pattern():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(LIB), "tests/native/libdevice_sweep.so is not built (run __graft_entry__.build())"
    L = C.CDLL(LIB)
    L.cskv_test_encoder_sweep.argtypes = [C.c_uint64, C.c_uint64, C.POINTER(C.c_uint64)]
    L.cskv_test_encoder_sweep.restype = C.c_int
    out = (C.c_uint64 * 2)()
    assert L.cskv_test_encoder_sweep(0, 1 << 32, out) == 0
    with open(os.path.join(HERE, "golden", "encoder_checksums.json")) as f:
        g = json.load(f)
    assert f"0x{out[0]:016x}" == g["e2m1_sum"], "E2M1 encoder differs from the oracle on some fp32 pattern"
    assert f"0x{out[1]:016x}" == g["bf16_sum"], "bf16 rounding differs from the oracle on some fp32 pattern"
