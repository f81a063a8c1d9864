"""The LDS read-rate probe library (a measurement tool next to the decode
library, run by bench.py --probe-lds) loads, exports its entry point and
rejects unsupported arguments before any device work (no GPU needed)."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.cpu

PROBE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                     "mla_latent_decode_absorbed_amd", "libmla_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(PROBE):
        pytest.skip("libmla_probe.so is not built")
    import torch  # noqa: F401  (the HIP runtime the libraries share)
    lib = ctypes.CDLL(PROBE)
    lib.mla_probe_lds_read_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(ctypes.c_double)]
    lib.mla_probe_lds_read_rate.restype = ctypes.c_int
    return lib


def test_probe_rejects_unsupported_shapes(probe):
    v = ctypes.c_double(0.0)
    assert probe.mla_probe_lds_read_rate(3, 8, 1, ctypes.byref(v)) == -1
    assert probe.mla_probe_lds_read_rate(256, 7, 1, ctypes.byref(v)) == -1
    assert probe.mla_probe_lds_read_rate(2048, 8, 0, ctypes.byref(v)) == -1
    assert probe.mla_probe_lds_read_rate(256, 8, 1, None) == -1
