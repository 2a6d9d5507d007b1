"""Seeded random GEMM calls through the automatic variant choice.

Each case draws a batch count, M, N and K (among them few-row, 8-aligned and
ragged shapes), fp16 or bf16, 16-bit or fp32 output, row-padded operands
(leading dimensions past K and N, some not a multiple of 8) and B given as
K x N or transposed, and compares the whole C with the oracle: bitwise for
small-integer inputs, within the tolerance for random ones.  The fixed shape
lists of the other tests pick their combinations by hand; these are drawn.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import barrier_pipelined_tiled_amd as pkg
import oracle
from barrier_pipelined_tiled_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkg.lib()


def _cases(n=160, seed=20261203):
    """Families, each drawn so that the automatic choice reaches its kernels:
    ragged shapes (guarded kernel, repack route), 8-aligned shapes (the
    pipelined tiles), few rows of A (skinny kernels), long K over few output
    tiles (split-K), and two short-K batches of 2048 tiles (persistent)."""
    rng = np.random.default_rng(seed)
    out = []
    a8 = lambda lo, hi: 8 * int(rng.integers(lo // 8, hi // 8 + 1))
    for i in range(n):
        fam = i % 5
        batch = int(rng.choice([1, 1, 1, 2, 3]))
        pad = int(rng.choice([0, 0, 8, 16]))
        if fam == 0:                       # ragged
            M, N, K = int(rng.integers(1, 520)), int(rng.integers(1, 520)), int(rng.integers(1, 1100))
            pad = int(rng.choice([0, 5, 8]))
        elif fam == 1:                     # 8-aligned
            M, N, K = a8(8, 640), a8(8, 640), a8(8, 1280)
        elif fam == 2:                     # few rows of A
            M, N, K = int(rng.integers(1, 129)), a8(64, 1024), 256 * int(rng.integers(2, 17))
        elif fam == 3:                     # long K, few output tiles
            batch = 1
            M, N, K = a8(136, 320), a8(64, 512), 64 * int(rng.integers(32, 129))
        else:                              # aligned, larger
            M, N, K = a8(256, 1024), a8(256, 1024), a8(64, 512)
        dtype = str(rng.choice(["f16", "bf16"]))
        out_fp32 = bool(rng.integers(0, 2))
        bt = bool(rng.random() < 0.25)
        exact = bool(rng.random() < 0.3)
        out.append((i, batch, M, N, K, dtype, out_fp32, pad, bt, exact))
    for j, K in enumerate((128, 256)):     # 16 x 8 x 16 = 2048 tiles of 256 x 128
        out.append((n + j, 16, 2048, 2048, K, "f16", False, 0, False, j == 0))
    return out


def _operand(shape, seed, dtype, exact, pad):
    rows, cols = shape[-2], shape[-1]
    full = shape[:-1] + (cols + pad,)
    t = inputs.small_integers(full, seed, dtype=dtype) if exact else inputs.uniform(full, seed, dtype=dtype,
                                                                                    nonzero=True)
    return t[..., :cols]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}")
def test_random_call_matches_the_oracle(case):
    i, batch, M, N, K, dtype, out_fp32, pad, bt, exact = case
    print(f"[fuzz] case {i}: batch={batch} M={M} N={N} K={K} {dtype} out_fp32={out_fp32} pad={pad} "
          f"bt={bt} exact={exact}", flush=True)
    lead = (batch,) if batch > 1 else ()
    A = _operand(lead + (M, K), 9700 + 3 * i, dtype, exact, pad)
    if bt:
        Bt = _operand(lead + (N, K), 9701 + 3 * i, dtype, exact, pad)
        B = Bt.transpose(-1, -2)
        C = pkg.gemm_ex_bt(A.to(DEV), Bt.to(DEV), dtype=dtype, out_fp32=out_fp32)
    else:
        B = _operand(lead + (K, N), 9701 + 3 * i, dtype, exact, pad)
        C = pkg.gemm_ex(A.to(DEV), B.to(DEV), dtype=dtype, out_fp32=out_fp32)
    torch.cuda.synchronize()
    got = C.cpu()
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B), dtype)
    if exact:
        if out_fp32:
            assert np.array_equal(got.numpy(), ref)
        else:
            assert np.array_equal(got.contiguous().view(torch.int16).numpy().view(np.uint16), oracle.encode(ref, dtype))
    else:
        m = oracle.compare(got.float().numpy(), ref, K)
        assert m["ok"], m
