"""gemm_ex_noalloc (no device allocation in the call; split partials and
repack copies in the library's fixed device array) against gemm_ex on the
same inputs: the same kernels and split counts run, so the outputs must be
identical bit for bit, and both meet the oracle.  Two calls in a row on one
stream, the second with a smaller input, reuse the array."""
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


# (expected variant, first shape, second smaller shape); the first three
# need scratch (skinny split-K: 4 and 16 splits; split-K for few tiles: 4
# and 4 splits; repack copies), the last none
CASES = [
    ("skinny_64x128_ring_k32_s4_splitk", (64, 8192, 8192), (64, 2048, 4096)),
    ("splitk_pipelined", (1024, 1024, 8192), (300, 520, 2048)),
    ("repack_pipelined", (512, 201, 256), (300, 201, 384)),
    ("pipelined_128x128x32_s4", (512, 384, 320), (256, 256, 256)),
]


@pytest.mark.parametrize("vname,big,small", CASES)
@pytest.mark.parametrize("out_fp32", [False, True])
def test_noalloc_matches_gemm_ex(vname, big, small, out_fp32):
    v = pkg.variants()[vname]
    data = []
    for i, (M, N, K) in enumerate((big, small)):
        print(f"noalloc {vname} M={M} N={N} K={K} out_fp32={out_fp32}", flush=True)
        assert pkg.select_variant("f16", 1, M, N, K, K, N, out_fp32) == v
        A = inputs.uniform((M, K), 9101 + 2 * i, nonzero=True)
        B = inputs.uniform((K, N), 9102 + 2 * i, nonzero=True)
        data.append((A, B, A.to(DEV), B.to(DEV)))
    out_t = torch.float32 if out_fp32 else torch.float16
    refs = []
    for A, B, Ad, Bd in data:
        refs.append(pkg.gemm_ex(Ad, Bd, out_fp32=out_fp32))
    torch.cuda.synchronize()
    # two calls in a row, no synchronisation between them
    outs = []
    for A, B, Ad, Bd in data:
        C = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=out_t, device=DEV)
        pkg.gemm_ex_noalloc(Ad, Bd, C, out_fp32=out_fp32)
        outs.append(C)
    torch.cuda.synchronize()
    for (A, B, _, _), ref, got in zip(data, refs, outs):
        assert torch.equal(got.cpu().view(torch.int16 if not out_fp32 else torch.int32),
                           ref.cpu().view(torch.int16 if not out_fp32 else torch.int32))
        m = oracle.compare(got.cpu().float().numpy(), oracle.gemm(inputs.bits(A), inputs.bits(B), "f16"),
                           A.shape[1])
        assert m["ok"], m


def test_noalloc_exact_integers_repeated():
    """Integer inputs (every partial sum exact): 6 calls in a row alternating
    a large and a small skinny split-K shape on the shared array, each equal
    to the oracle bit for bit."""
    shapes = [(64, 8192, 8192), (48, 1024, 2048)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A = inputs.small_integers((M, K), 9201 + i)
        B = inputs.small_integers((K, N), 9211 + i)
        data.append((A.to(DEV), B.to(DEV), oracle.gemm(inputs.bits(A), inputs.bits(B), "f16")))
    outs = []
    for rep in range(6):
        Ad, Bd, ref = data[rep % 2]
        C = torch.empty((Ad.shape[0], Bd.shape[1]), dtype=torch.float32, device=DEV)
        pkg.gemm_ex_noalloc(Ad, Bd, C, out_fp32=True)
        outs.append((rep % 2, C))
    torch.cuda.synchronize()
    for j, C in outs:
        assert np.array_equal(C.cpu().numpy(), data[j][2])


@pytest.mark.parametrize("M,N,K,vname", [(64, 8192, 8192, "skinny_64x128_ring_k32_s4_splitk"),
                                         (1024, 1024, 8192, "splitk_pipelined")])
def test_noalloc_under_graph_capture_keeps_its_splits(M, N, K, vname):
    """Captured into a graph, gemm_ex_noalloc still runs its split paths
    (gemm_ex, which takes no pool buffer under capture, runs unsplit): the
    same kernels and split counts as the eager gemm_ex call, so each of three
    replays -- with eager calls and synchronisations between them -- equals
    that call bit for bit, and (integer inputs) the oracle exactly."""
    assert pkg.select_variant("f16", 1, M, N, K, K, N, True) == pkg.variants()[vname]
    print(f"noalloc capture {vname} M={M} N={N} K={K}", flush=True)
    A = inputs.small_integers((M, K), 9301)
    B = inputs.small_integers((K, N), 9302)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B), "f16")
    Ad, Bd = A.to(DEV), B.to(DEV)
    eager = pkg.gemm_ex(Ad, Bd, out_fp32=True)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up on a side stream, as torch advises
        pkg.gemm_ex_noalloc(Ad, Bd, C, out_fp32=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(eager.cpu().numpy(), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkg.gemm_ex_noalloc(Ad, Bd, C, out_fp32=True)
    for rep in range(3):
        C.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, eager), rep
        again = pkg.gemm_ex(Ad, Bd, out_fp32=True)
        torch.cuda.synchronize()
        assert torch.equal(again, eager), rep
    assert np.array_equal(C.cpu().numpy(), ref)
