"""The fp32 -> bf16 hi + lo split that every MFMA product with an fp32
operand uses (split4 of the library's device code, run on test data through
libldv_checks.so) against its definition written out in numpy: hi = x
rounded to bf16 (to nearest, ties to even), lo = (x - hi) rounded the same
way, x - hi taken exactly in fp32.  The device computes x - hi from a packed
bf16 dot product instead of a subtraction; the two must agree bit for bit
for every |x| from 1e-30 to 1e30, and on exact powers of two, rounding ties
of both parities and signed zeros."""
import ctypes
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "speculative_decoding_verify_amd",
                   "libldv_checks.so")


def bf16_rne_bits(x):
    """bf16 bit patterns of fp32 values, rounded to nearest, ties to even
    (finite inputs whose rounding stays finite)."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def reference_split(x):
    hi = bf16_rne_bits(x)
    hi_f = (hi.astype(np.uint32) << 16).view(np.float32)
    rem = (x - hi_f).astype(np.float32)  # exact: hi holds the top 8 of x's 24 mantissa bits
    return hi, bf16_rne_bits(rem)


def inputs(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.uniform(1.0, 2.0, n)
    expo = rng.integers(-99, 99, n)  # |x| from about 1.6e-30 to 1.3e30
    sign = rng.choice([-1.0, 1.0], n)
    x = (sign * mant * np.exp2(expo)).astype(np.float32)
    k = n // 8
    x[:k] = np.float32(2.0) ** rng.integers(-99, 99, k).astype(np.float32)          # powers of two
    ties = rng.integers(0, 1 << 16, k).astype(np.uint32) << 16 | np.uint32(0x8000)  # ties, both parities
    ties = ties & np.uint32(0x3FFFFFFF) | np.uint32(0x3F000000)                      # kept in range
    x[k:2 * k] = ties.view(np.float32)
    x[2 * k:2 * k + 4] = np.array([0.0, -0.0, 1.0, -1.0], np.float32)
    return x


def test_reference_rounds_to_nearest_even():
    """The reference itself (CPU): round-to-nearest-even on exact cases, and
    hi + lo holds x to about 2^-17, where truncating both parts would give a
    different split on most of the test's values."""
    as_f = lambda u: np.array([u], np.uint32).view(np.float32)
    assert bf16_rne_bits(np.float32(1.0)) == 0x3F80
    assert bf16_rne_bits(as_f(0x3F808000))[0] == 0x3F80  # tie, even below
    assert bf16_rne_bits(as_f(0x3F818000))[0] == 0x3F82  # tie, even above
    assert bf16_rne_bits(as_f(0x3F808001))[0] == 0x3F81  # above the tie
    assert bf16_rne_bits(as_f(0xBF807FFF))[0] == 0xBF80  # below the tie, negative
    x = inputs(1 << 14, 3)
    hi, lo = reference_split(x)
    hf = (hi.astype(np.uint32) << 16).view(np.float32)
    lf = (lo.astype(np.uint32) << 16).view(np.float32)
    nz = x != 0
    err = np.abs(hf.astype(np.float64) + lf - x)[nz] / np.abs(x[nz])
    assert err.max() <= 2.0 ** -16
    trunc_hi = (x.view(np.uint32) >> 16).astype(np.uint16)
    assert np.mean(trunc_hi != hi) > 0.3


@pytest.mark.gpu
def test_split_matches_its_definition():
    assert os.path.exists(LIB), "libldv_checks.so is not built (python -c 'import __graft_entry__ as g; g.build()')"
    lib = ctypes.CDLL(LIB)
    lib.ldv_check_split.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
                                    ctypes.c_void_p]
    n = 1 << 22
    x = inputs(n, 7101)
    assert np.all((np.abs(x) == 0) | ((np.abs(x) >= 1e-30) & (np.abs(x) <= 1e30)))
    dx = torch.from_numpy(x).cuda()
    hi = torch.empty(n, dtype=torch.int16, device="cuda")
    lo = torch.empty(n, dtype=torch.int16, device="cuda")
    st = torch.cuda.current_stream()
    rc = lib.ldv_check_split(ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(hi.data_ptr()),
                             ctypes.c_void_p(lo.data_ptr()), n, ctypes.c_void_p(st.cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    ghi = hi.cpu().numpy().view(np.uint16)
    glo = lo.cpu().numpy().view(np.uint16)
    rhi, rlo = reference_split(x)
    bad_hi = np.flatnonzero(ghi != rhi)
    bad_lo = np.flatnonzero(glo != rlo)
    assert bad_hi.size == 0, "hi differs at %s" % x[bad_hi[:5]]
    assert bad_lo.size == 0, "lo differs at %s" % x[bad_lo[:5]]
