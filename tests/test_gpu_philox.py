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


def test_race_variate_matches_log1p(gpu_lib):
    """The races' exponential variate -ln(1 - u) (an atanh series, not the library log1p)
    stays within 4 ulp of numpy's -log1p(-u) over the uniforms the races draw and the ends
    of [0, 1)."""
    lib = _probe()
    lib.sv_probe_neg_log1m.restype = ctypes.c_int
    lib.sv_probe_neg_log1m.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p]
    j = np.arange(0, 400_000, dtype=np.uint64)
    u = P.uniforms(0xC0FFEE, 3, 1, P.RESAMPLE, 5, j)
    k = np.arange(1, 54, dtype=np.float64)
    ends = np.concatenate([[0.0, 2.0 ** -53, 1.0 - 2.0 ** -53, 0.5, 1.0 - 2.0 ** -0.5,
                            2.0 ** -0.5, 0.25, 0.75],
                           2.0 ** -k, 1.0 - 2.0 ** -k])
    u = np.concatenate([u, ends]).astype(np.float64)
    say(f"[race variate] n={len(u)}")
    du = torch.from_numpy(u).cuda()
    de = torch.empty_like(du)
    assert lib.sv_probe_neg_log1m(du.data_ptr(), de.data_ptr(), len(u),
                                  torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    e = de.cpu().numpy()
    ref = -np.log1p(-u)
    zero = u == 0.0
    assert np.all(e[zero] == 0.0) and np.all(e[~zero] > 0)
    ulp = np.spacing(np.maximum(np.abs(ref), np.finfo(np.float64).tiny))
    err = np.abs(e - ref) / ulp
    say(f"  max error {err.max():.2f} ulp, mean {err.mean():.3f} ulp")
    assert err.max() <= 4.0
