"""The exact sign of a float32/bf16 dot product (the fixed-point sum of
exact_dot.h that the hashing kernels fall back to near a tie), built for the
host with g++ and checked against math.fsum of the exact float64 products.

The hashing steps set a plane's bit when the projection is >= 0 (SOCKET
overview page, "Core mechanism: soft LSH", item 1); the sign must be exact
for any rows, including sums that cancel to within the rounding of every
float64 order and sums whose exact value needs many float64 partials.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hash_scored_top_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "exact_dot_check.cpp")


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = tmp_path_factory.mktemp("exact_dot") / "libexactdot.so"
    subprocess.run(["g++", "-std=c++17", "-O2", "-shared", "-fPIC", "-I", CSRC, SRC, "-o", str(out)],
                   check=True)
    so = ctypes.CDLL(str(out))
    fp = ctypes.POINTER(ctypes.c_float)
    hp = ctypes.POINTER(ctypes.c_uint16)
    so.hst_check_dot_nonneg_f32.argtypes = [fp, fp, ctypes.c_int]
    so.hst_check_dot_nonneg_bf16.argtypes = [hp, hp, ctypes.c_int]
    so.hst_check_dot_words_f32.argtypes = [fp, fp, ctypes.c_int, ctypes.POINTER(ctypes.c_uint64)]
    return so


def sign_f32(lib, a, b):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    fp = ctypes.POINTER(ctypes.c_float)
    return bool(lib.hst_check_dot_nonneg_f32(a.ctypes.data_as(fp), b.ctypes.data_as(fp), len(a)))


def fsum_nonneg(a, b):
    # float32 x float32 is exact in float64; fsum rounds the exact sum once,
    # which keeps its sign (and gives 0.0 only for an exact zero)
    return math.fsum(float(x) * float(y) for x, y in zip(np.float32(a), np.float32(b))) >= 0.0


def grow_expansion_len(products):
    """Number of float64 partials Shewchuk's growing expansion (with zero
    elimination) holds after adding the products in order (its maximum over
    the run)."""
    h, most = [], 0
    for x in products:
        k = []
        for y in h:
            hi = x + y
            bv = hi - x
            lo = (x - (hi - bv)) + (y - bv)
            if lo != 0.0:
                k.append(lo)
            x = hi
        k.append(x)
        h = k
        most = max(most, len(h))
    return most


def test_random_rows_match_fsum(lib):
    rng = np.random.default_rng(20260101)
    for n in (1, 2, 7, 64, 128, 513):
        for _ in range(40):
            a = rng.standard_normal(n).astype(np.float32)
            b = rng.standard_normal(n).astype(np.float32)
            assert sign_f32(lib, a, b) == fsum_nonneg(a, b)


def test_cancellation_to_a_tiny_residue(lib):
    # x.y - x.y + r: the float64 sum in any order is dominated by rounding of
    # the large terms; the exact sum is r
    rng = np.random.default_rng(7)
    for _ in range(200):
        n = int(rng.integers(2, 60))
        x = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 40, n)).astype(np.float32)
        y = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 40, n)).astype(np.float32)
        r = np.float32(rng.choice([-1.0, 1.0]) * 2.0 ** int(rng.integers(-140, -100)))
        a = np.concatenate([x, x, [r]]).astype(np.float32)
        b = np.concatenate([y, -y, [np.float32(1.0)]]).astype(np.float32)
        perm = rng.permutation(len(a))
        a, b = a[perm], b[perm]
        assert sign_f32(lib, a, b) == (r >= 0) == fsum_nonneg(a, b)


def test_exact_zero_is_nonnegative(lib):
    rng = np.random.default_rng(3)
    for _ in range(50):
        x = rng.standard_normal(16).astype(np.float32)
        y = rng.standard_normal(16).astype(np.float32)
        a = np.concatenate([x, -x]).astype(np.float32)
        b = np.concatenate([y, y]).astype(np.float32)
        assert math.fsum(float(p) * float(q) for p, q in zip(a, b)) == 0.0
        assert sign_f32(lib, a, b) is True


def test_extreme_exponents(lib):
    tiny = np.float32(2.0 ** -149)  # smallest subnormal float32
    big = np.float32(np.finfo(np.float32).max)
    # the largest and smallest products together: big*big - big*big + tiny*tiny
    a = np.array([big, big, tiny], dtype=np.float32)
    b = np.array([big, -big, tiny], dtype=np.float32)
    assert sign_f32(lib, a, b) is True
    b[2] = -tiny
    assert sign_f32(lib, a, b) is False
    # many maximal products of one sign do not wrap the accumulator
    n = 4096
    assert sign_f32(lib, np.full(n, big), np.full(n, big)) is True
    assert sign_f32(lib, np.full(n, big), np.full(n, -big)) is False


def test_sums_that_need_many_partials(lib):
    # products +-m * 2^e with exponents spread over the whole float32 product
    # range, so that the exact sum has no short float64 expansion; each case
    # is checked to need more than 16 partials in Shewchuk's growing
    # expansion, then compared with fsum
    rng = np.random.default_rng(11)
    checked = 0
    for _ in range(400):
        n = 96
        e1 = rng.integers(-149, 104, n)
        e2 = rng.integers(-149, 104, n)
        m1 = rng.integers(1, 2 ** 24, n)
        m2 = rng.integers(1, 2 ** 24, n)
        s = rng.choice([-1.0, 1.0], n)
        a = np.array([np.float32(np.ldexp(float(m), int(e) - 23)) for m, e in zip(m1, e1)], dtype=np.float32)
        b = np.array([np.float32(sv * np.ldexp(float(m), int(e) - 23)) for m, e, sv in zip(m2, e2, s)],
                     dtype=np.float32)
        prods = [float(x) * float(y) for x, y in zip(a, b)]
        if grow_expansion_len(prods) <= 16:
            continue
        checked += 1
        assert sign_f32(lib, a, b) == fsum_nonneg(a, b)
    assert checked >= 50


def test_words_hold_the_exact_sum(lib):
    # the fixed-point words, read as one integer times 2^-320, equal the exact
    # sum (Python integers are exact)
    rng = np.random.default_rng(5)
    fp = ctypes.POINTER(ctypes.c_float)
    for _ in range(50):
        n = 40
        a = (rng.standard_normal(n) * 2.0 ** rng.integers(-60, 60, n)).astype(np.float32)
        b = (rng.standard_normal(n) * 2.0 ** rng.integers(-60, 60, n)).astype(np.float32)
        out = (ctypes.c_uint64 * 10)()
        lib.hst_check_dot_words_f32(a.ctypes.data_as(fp), b.ctypes.data_as(fp), n, out)
        v = 0
        for i in reversed(range(10)):
            v = (v << 64) | int(out[i])
        if v >= 1 << 639:
            v -= 1 << 640
        exact = sum(int(float(x).as_integer_ratio()[0]) * int(float(y).as_integer_ratio()[0])
                    * (2 ** 320) // (int(float(x).as_integer_ratio()[1]) * int(float(y).as_integer_ratio()[1]))
                    for x, y in zip(a, b))
        assert v == exact


def test_bf16_rows(lib):
    rng = np.random.default_rng(9)
    hp = ctypes.POINTER(ctypes.c_uint16)
    for _ in range(100):
        n = 128
        x = rng.standard_normal(n).astype(np.float32)
        y = rng.standard_normal(n).astype(np.float32)
        xb = (x.view(np.uint32) >> 16).astype(np.uint16)
        yb = (y.view(np.uint32) >> 16).astype(np.uint16)
        # cancel all but one pair, exactly
        xb = np.concatenate([xb, xb, xb[:1]])
        yb = np.concatenate([yb, yb ^ np.uint16(0x8000), yb[:1]])
        xf = (xb.astype(np.uint32) << 16).view(np.float32)
        yf = (yb.astype(np.uint32) << 16).view(np.float32)
        got = bool(lib.hst_check_dot_nonneg_bf16(np.ascontiguousarray(xb).ctypes.data_as(hp),
                                                 np.ascontiguousarray(yb).ctypes.data_as(hp), len(xb)))
        assert got == fsum_nonneg(xf, yf)
