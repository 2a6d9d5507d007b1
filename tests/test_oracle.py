"""Pins for the CPU oracle: each test checks it against something other than
itself -- a library routine on the same exact values, exact rational
arithmetic, closed forms, invariants of the matrix product, or values fixed
by the number formats.  CPU only."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from barrier_pipelined_tiled_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f16_bits(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float16).view(np.uint16)


def bf16_bits(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_bits(x, dtype):
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def test_golden_half_encodings():
    data = json.load(open(os.path.join(GOLDEN, "half_encodings.json")))
    for dtype in ("f16", "bf16"):
        for entry in data[dtype]:
            h = np.array([int(entry[0], 16)], dtype=np.uint16)
            want = float(entry[1])
            got = oracle.decode(h, dtype)[0]
            assert got == want and math.copysign(1, got) == math.copysign(1, want), entry
            if math.isfinite(want):
                back = oracle.encode(np.array([want], dtype=np.float32), dtype)[0]
                assert back == h[0], (entry, hex(back))


def test_decode_f16_exhaustive_vs_numpy():
    allbits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(allbits, "f16")
    want = allbits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_exhaustive_vs_torch():
    allbits = np.arange(65536, dtype=np.uint16)
    want = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode(allbits, "bf16")
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def _float32_probe_values(rng, n):
    raw = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return raw[np.isfinite(raw)]


def test_encode_f16_vs_numpy():
    rng = np.random.default_rng(7)
    vals = [_float32_probe_values(rng, 400_000)]
    finite16 = np.arange(65536, dtype=np.uint16).view(np.float16)
    finite16 = finite16[np.isfinite(finite16)].astype(np.float32)
    vals.append(finite16)
    # exact midpoints between neighbouring fp16 values (fp32 holds them exactly)
    pos = np.sort(np.unique(finite16[finite16 >= 0]).astype(np.float64))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals += [mids, -mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))]
    vals.append(np.array([65519.996, 65520.0, 65536.0, 1e-8, 2.98e-8, 2.9802322e-8, 3e-8], np.float32))
    x = np.concatenate(vals).astype(np.float32)
    got = oracle.encode(x, "f16")
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_bf16_vs_torch():
    rng = np.random.default_rng(8)
    x = _float32_probe_values(rng, 400_000)
    allbf = torch.from_numpy(np.arange(65536, dtype=np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    allbf = allbf.to(torch.float64).numpy()
    pos = np.sort(np.unique(allbf[np.isfinite(allbf) & (allbf >= 0)]))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.nextafter(mids, np.float32(np.inf))]).astype(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.encode(x, "bf16")
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


# ----------------------------------------------------------------------------
# the product: worked examples, exact arithmetic, closed forms
# ----------------------------------------------------------------------------

def test_golden_worked_products():
    data = json.load(open(os.path.join(GOLDEN, "worked_product.json")))
    for case in data["cases"]:
        dt = case["dtype"]
        A = to_bits([[float(v) for v in r] for r in case["A"]], dt)
        B = to_bits([[float(v) for v in r] for r in case["B"]], dt)
        want = np.array([[float(v) for v in r] for r in case["C"]], dtype=np.float32)
        got = oracle.gemm(A, B, dt)
        assert np.array_equal(got, want), (case["note"], got, want)


def _exact(A_vals, B_vals):
    """Exact rational product of two small float64 matrices."""
    M, K = A_vals.shape
    N = B_vals.shape[1]
    Af = [[Fraction(float(A_vals[i, k])) for k in range(K)] for i in range(M)]
    Bf = [[Fraction(float(B_vals[k, j])) for j in range(N)] for k in range(K)]
    return [[sum((Af[i][k] * Bf[k][j] for k in range(K)), Fraction(0)) for j in range(N)]
            for i in range(M)]


def _f32_of_fraction(fr: Fraction) -> np.float32:
    """Correctly rounded fp32 of an exact rational: round to double first
    only when that double is the exact value."""
    d = float(fr)
    assert Fraction(d) == fr
    return np.float32(d)


SHAPES_SMALL = [s for s in itertools.product(range(4, 17, 3), range(4, 17, 4), range(4, 17, 5))]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bruteforce_exact_sums(dtype):
    """Entries j/64 with |j| <= 64: every partial sum is an exact binary
    fraction well inside fp64, so the oracle's fp64 sum must equal the exact
    rational sum and its fp32 output the correctly rounded value."""
    rng = np.random.default_rng(11)
    for (M, N, K) in SHAPES_SMALL:
        A = rng.integers(-64, 65, size=(M, K)) / 64.0
        B = rng.integers(-64, 65, size=(K, N)) / 64.0
        Ab, Bb = to_bits(A, dtype), to_bits(B, dtype)
        c32, c64 = oracle.gemm(Ab, Bb, dtype, want64=True)
        ex = _exact(oracle.decode(Ab, dtype), oracle.decode(Bb, dtype))
        for i in range(M):
            for j in range(N):
                assert Fraction(float(c64[i, j])) == ex[i][j]
                assert c32[i, j] == _f32_of_fraction(ex[i][j])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_bruteforce_error_bound_random(dtype):
    """Full-range random inputs: recursive fp64 summation of K exact products
    is within gamma_K * sum|a_k b_k| of the exact sum, gamma_K = K u/(1-K u),
    u = 2^-53; the fp32 output adds at most half an fp32 ulp."""
    rng = np.random.default_rng(12)
    u = 2.0 ** -53
    for (M, N, K) in [(5, 7, 16), (16, 16, 16), (9, 4, 13), (4, 16, 11)]:
        A = rng.uniform(-1, 1, size=(M, K))
        B = rng.uniform(-1, 1, size=(K, N)) * (2.0 ** rng.integers(-20, 3, size=(K, N)))
        Ab, Bb = to_bits(A, dtype), to_bits(B, dtype)
        c32, c64 = oracle.gemm(Ab, Bb, dtype, want64=True)
        Ad, Bd = oracle.decode(Ab, dtype), oracle.decode(Bb, dtype)
        ex = _exact(Ad, Bd)
        gamma = K * u / (1 - K * u)
        absprod = np.abs(Ad) @ np.abs(Bd)
        for i in range(M):
            for j in range(N):
                err = abs(Fraction(float(c64[i, j])) - ex[i][j])
                assert err <= Fraction(gamma * absprod[i, j]) * (1 + Fraction(1, 2**40))
                e32 = abs(Fraction(float(c32[i, j])) - ex[i][j])
                ulp32 = np.spacing(np.float32(abs(float(ex[i][j])))) if ex[i][j] != 0 else np.float32(0)
                assert e32 <= err + Fraction(float(ulp32)) / 2 + Fraction(gamma * absprod[i, j])


def test_small_integers_exact_vs_int64_matmul():
    """Integer entries in [-2, 2]: every sum is an exact integer far below
    2^24, so the fp32 output must equal the int64 matrix product."""
    for (M, N, K, seed) in [(384, 512, 640, 1), (130, 70, 1030, 2), (64, 1024, 256, 3)]:
        A = inputs.small_integers((M, K), seed)
        B = inputs.small_integers((K, N), seed + 100)
        want = A.to(torch.int64).numpy() @ B.to(torch.int64).numpy()
        got = oracle.gemm(inputs.bits(A), inputs.bits(B), "f16")
        assert np.array_equal(got.astype(np.int64), want)
        assert np.array_equal(got, want.astype(np.float32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_cross_check_numpy_float64_matmul(dtype):
    """Same exact inputs through numpy's float64 matmul: only the summation
    order differs, so the two agree within 2 gamma_K |A||B|."""
    rng = np.random.default_rng(13)
    M, N, K = 192, 160, 256
    Ab = to_bits(rng.uniform(-1, 1, size=(M, K)), dtype)
    Bb = to_bits(rng.uniform(-1, 1, size=(K, N)), dtype)
    _, c64 = oracle.gemm(Ab, Bb, dtype, want64=True)
    Ad, Bd = oracle.decode(Ab, dtype), oracle.decode(Bb, dtype)
    ref = Ad @ Bd
    u = 2.0 ** -53
    bound = 2 * (K * u / (1 - K * u)) * (np.abs(Ad) @ np.abs(Bd))
    assert np.all(np.abs(c64 - ref) <= bound)


def test_identity_and_permutation():
    rng = np.random.default_rng(14)
    M = K = 48
    N = 33
    B = f16_bits(rng.uniform(-1, 1, size=(K, N)))
    I = f16_bits(np.eye(K))
    # A = I gives B exactly (every fp16 value is an fp32 value)
    assert np.array_equal(oracle.gemm(I, B), oracle.decode(B).astype(np.float32))
    A = f16_bits(rng.uniform(-1, 1, size=(M, K)))
    IN = f16_bits(np.eye(K))
    assert np.array_equal(oracle.gemm(A, IN), oracle.decode(A).astype(np.float32))
    # P * B permutes the rows of B; A * P permutes the columns of A
    perm = rng.permutation(K)
    P = np.zeros((K, K))
    P[np.arange(K), perm] = 1.0
    assert np.array_equal(oracle.gemm(f16_bits(P), B), oracle.decode(B)[perm].astype(np.float32))
    col_perm = np.argsort(perm)
    assert np.array_equal(oracle.gemm(A, f16_bits(P)),
                          oracle.decode(A)[:, col_perm].astype(np.float32))


def test_transpose_identity_bitwise():
    """(A B)^T = B^T A^T: the same products in the same k order, so the two
    results agree bit for bit."""
    rng = np.random.default_rng(15)
    for dtype in ("f16", "bf16"):
        A = to_bits(rng.uniform(-1, 1, size=(37, 53)), dtype)
        B = to_bits(rng.uniform(-1, 1, size=(53, 29)), dtype)
        c = oracle.gemm(A, B, dtype)
        ct = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), dtype)
        assert np.array_equal(c.T, ct)


def test_rank_one_closed_forms():
    rng = np.random.default_rng(16)
    u = f16_bits(rng.uniform(-1, 1, size=(23, 1)))
    v = f16_bits(rng.uniform(-1, 1, size=(1, 31)))
    # K = 1: C = u v^T, each product exact in fp32 (at most 22 significant bits)
    want = (oracle.decode(u) * oracle.decode(v)).astype(np.float32)
    assert np.array_equal(oracle.gemm(u, v), want)
    # A = u 1^T, B = 1 v^T with K a power of two: C = K u v^T exactly
    K = 64
    A = np.repeat(u, K, axis=1)
    B = np.repeat(v, K, axis=0)
    assert np.array_equal(oracle.gemm(A, B), (K * oracle.decode(u) * oracle.decode(v)).astype(np.float32))
    # all ones: C = K (exact in fp16, bf16 and fp32 for these K)
    for K in (4096, 16384):
        ones_a = f16_bits(np.ones((2, K)))
        ones_b = f16_bits(np.ones((K, 3)))
        assert np.array_equal(oracle.gemm(ones_a, ones_b), np.full((2, 3), K, np.float32))
        ones_a16 = bf16_bits(np.ones((2, K)))
        ones_b16 = bf16_bits(np.ones((K, 3)))
        assert np.array_equal(oracle.gemm(ones_a16, ones_b16, "bf16"), np.full((2, 3), K, np.float32))


def test_linearity_in_a():
    A1 = inputs.bits(inputs.small_integers((40, 96), 21))
    A2 = inputs.bits(inputs.small_integers((40, 96), 22))
    B = inputs.bits(inputs.small_integers((96, 50), 23))
    alpha, beta = 2.0, -4.0
    Acomb = f16_bits(alpha * oracle.decode(A1) + beta * oracle.decode(A2))
    lhs = oracle.gemm(Acomb, B)
    rhs = alpha * oracle.gemm(A1, B) + beta * oracle.gemm(A2, B)
    assert np.array_equal(lhs, rhs.astype(np.float32))


def test_leading_dimensions_and_subblocks():
    rng = np.random.default_rng(17)
    A = f16_bits(rng.uniform(-1, 1, size=(70, 90)))
    B = f16_bits(rng.uniform(-1, 1, size=(90, 110)))
    full = oracle.gemm(A, B)
    # a view with lda > K and ldb > N gives the same as its contiguous copy
    Av = A[5:47, 3:71]
    Bv = B[3:71, 9:100]
    got = oracle.gemm(Av, Bv)
    assert np.array_equal(got, oracle.gemm(np.ascontiguousarray(Av), np.ascontiguousarray(Bv)))
    # rows of A and columns of B select the matching block of the full product
    assert np.array_equal(oracle.gemm(A[10:30], B[:, 40:77]), full[10:30, 40:77])


def test_batched_equals_single_calls():
    rng = np.random.default_rng(18)
    A = f16_bits(rng.uniform(-1, 1, size=(5, 19, 24)))
    B = f16_bits(rng.uniform(-1, 1, size=(5, 24, 13)))
    c = oracle.gemm(A, B)
    for b in range(5):
        assert np.array_equal(c[b], oracle.gemm(A[b], B[b]))


def test_thread_count_changes_nothing():
    """One thread and all of them give the same bits (each output element
    is one thread's ascending-k sum), and the setter takes effect."""
    rng = np.random.default_rng(20)
    A = f16_bits(rng.uniform(-1, 1, size=(2, 70, 130)))
    B = f16_bits(rng.uniform(-1, 1, size=(2, 130, 45)))
    n0 = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        assert oracle.num_threads() == 1
        one32, one64 = oracle.gemm(A, B, want64=True)
    finally:
        oracle.set_num_threads(n0)
    assert oracle.num_threads() == n0
    all32, all64 = oracle.gemm(A, B, want64=True)
    assert np.array_equal(one32, all32) and np.array_equal(one64, all64)


def test_gemm_at_equals_full_product():
    rng = np.random.default_rng(19)
    for dtype in ("f16", "bf16"):
        A = to_bits(rng.uniform(-1, 1, size=(3, 40, 300)), dtype)
        B = to_bits(rng.uniform(-1, 1, size=(3, 300, 50)), dtype)
        c32, c64 = oracle.gemm(A, B, dtype, want64=True)
        n = 200
        bi, ri, ci = rng.integers(0, 3, n), rng.integers(0, 40, n), rng.integers(0, 50, n)
        g32, g64 = oracle.gemm_at(A, B, bi, ri, ci, dtype, want64=True)
        assert np.array_equal(g32, c32[bi, ri, ci])
        assert np.array_equal(g64, c64[bi, ri, ci])


def test_empty_and_zero_k():
    A = np.zeros((4, 0), np.uint16)
    B = np.zeros((0, 5), np.uint16)
    assert np.array_equal(oracle.gemm(A, B), np.zeros((4, 5), np.float32))
    assert oracle.gemm(np.zeros((0, 3), np.uint16), np.zeros((3, 2), np.uint16)).shape == (0, 2)


# ----------------------------------------------------------------------------
# comparison metrics
# ----------------------------------------------------------------------------

def test_metrics_hand_computed():
    r = np.array([[3.0, 4.0], [0.0, 0.0]])         # ||R|| = 5
    g = r * (1 + 1e-3)
    m = oracle.compare(g, r, K=256)
    assert m["ok"] and abs(m["rel_rms"] - 1e-3) < 1e-12
    assert abs(m["max_abs"] - 4e-3) < 1e-12
    assert abs(m["max_abs_tol"] - 2e-2 * 4.0) < 1e-12
    g2 = r.copy()
    g2[0, 0] = 3.1                                  # diff 0.1 -> rel_rms 0.02
    m2 = oracle.compare(g2, r, K=256)
    assert not m2["ok"] and abs(m2["rel_rms"] - 0.02) < 1e-12
    g3 = r.copy()
    g3[1, 1] = np.nan
    m3 = oracle.compare(g3, r, K=256)
    assert not m3["ok"] and m3["nonfinite"] == 1
    z = np.zeros((3, 3))
    assert oracle.compare(z, z, K=0)["ok"]
    zz = z.copy()
    zz[0, 0] = 1e-30
    assert not oracle.compare(zz, z, K=0)["ok"]
    # max-abs bound scales with sqrt(K / 256) from K = 256 up
    assert abs(oracle.max_abs_tol(1024, 1.0) - 4e-2) < 1e-15
    assert oracle.max_abs_tol(1, 1.0) == oracle.max_abs_tol(256, 1.0) == 2e-2
    # a K = 1 product rounded to bf16 (relative error up to 2^-9) passes
    r = np.array([[1.0 + 2.0 ** -8]])
    g = np.array([[1.0]])
    assert oracle.compare(g, r, K=1)["ok"]


# ----------------------------------------------------------------------------
# the input recipe (shared by both sides; no product arithmetic in it)
# ----------------------------------------------------------------------------

def test_input_recipes():
    a = inputs.uniform((300, 200), 5, nonzero=True)
    b = inputs.uniform((300, 200), 5, nonzero=True)
    assert torch.equal(a, b)                       # seeded: same bits every time
    assert a.dtype == torch.float16 and not bool((a == 0).any())
    assert float(a.min()) >= -1.0 and float(a.max()) <= 1.0
    n = inputs.normal((512, 512), 9, std=1 / 128)
    assert n.dtype == torch.bfloat16
    assert abs(float(n.float().std()) - 1 / 128) < 1e-4
    w = inputs.WORKLOADS["f16_skinny_64x8192x8192"]
    assert w.flops == 2 * 64 * 8192 * 8192
    assert w.compulsory_bytes == 2 * 64 * 8192 + 2 * 8192 * 8192 + 2 * 64 * 8192
