"""The device Philox4x64-10 words and uniforms, as the sampling kernels draw them (through
libsvprobe.so's probe, which calls the kernels' own device functions), equal the oracle's
word for word."""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_verify_sv_amd as sv
from gpu_helpers import say
from oracle import philox as P

pytestmark = pytest.mark.gpu


def _probe():
    lib = ctypes.CDLL(os.path.join(os.path.dirname(sv.LIB_PATH), "libsvprobe.so"))
    lib.sv_probe_philox.restype = ctypes.c_int
    lib.sv_probe_philox.argtypes = [ctypes.c_uint64] * 6 + [ctypes.c_int32, ctypes.c_void_p,
                                                            ctypes.c_void_p, ctypes.c_void_p]
    return lib


@pytest.mark.parametrize("seed,offset,b,purpose,row,j0,n", [
    (0x5EED, 0, 0, P.ACCEPT, 1, 0, 4),                 # accept tests, first draft
    (0x5EED, 7, 3, P.ACCEPT, 31, 0, 4),
    (0x5EED, 5, 0, P.RESAMPLE, 12, 0, 152064),          # a whole 152,064-token race row
    (2**64 - 1, 2**63 + 11, 65535, P.RESAMPLE, 63, 1_000_001, 4099),   # wide words, odd start
    (0, 0, 0, P.RESAMPLE, 0, 0, 1),
])
def test_device_words_equal_oracle(gpu_lib, seed, offset, b, purpose, row, j0, n):
    lib = _probe()
    words = torch.empty(n, dtype=torch.int64, device="cuda")
    unif = torch.empty(n, dtype=torch.float64, device="cuda")
    say(f"[philox] seed={seed:#x} offset={offset} b={b} purpose={purpose} row={row} j0={j0} n={n}")
    st = lib.sv_probe_philox(seed, offset, b, purpose, row, j0, n, words.data_ptr(),
                             unif.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    j = np.arange(j0, j0 + n, dtype=np.uint64)
    ref_w = P.raw_words(seed, offset, b, purpose, row, j)
    ref_u = P.uniforms(seed, offset, b, purpose, row, j)
    np.testing.assert_array_equal(words.cpu().numpy().view(np.uint64), ref_w)
    np.testing.assert_array_equal(unif.cpu().numpy(), ref_u)
