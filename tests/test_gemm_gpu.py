"""GPU parity: the HIP kernels (called through the C ABI) against the CPU
oracle on the same seeded inputs.

* random inputs: rel-RMS <= 5e-3 and max|err| <= 2e-2 sqrt(K/256) max|C_ref|
  after a non-finite check (the oracle's ``compare``);
* small-integer inputs: every partial sum is an exact integer in fp32, so any
  summation order gives the same fp32 result -- the GPU must match the
  oracle bit for bit (fp32 output) or match the oracle's round-to-nearest-
  even 16-bit encoding of it bit for bit (16-bit output);
* full workload sizes run the automatic choice (what the benchmark times)
  and compare sampled outputs computed one by one by the oracle.
"""
import os

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


def say(msg):
    print(msg, flush=True)


def run(A, B, dtype="f16", out_fp32=False, variant=0, C=None):
    """GEMM of CPU tensors on the GPU; returns the CPU result."""
    Ad, Bd = A.to(DEV), B.to(DEV)
    Cd = pkg.gemm_ex(Ad, Bd, C, dtype=dtype, out_fp32=out_fp32, variant=variant)
    torch.cuda.synchronize()
    return Cd.cpu()


def as_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def check_random(A, B, dtype, out_fp32, variant=0):
    got = run(A, B, dtype, out_fp32, variant)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B), dtype)
    m = oracle.compare(got.float().numpy(), ref, A.shape[-1])
    assert m["ok"], m
    return m


def check_exact(A, B, dtype, out_fp32, variant=0):
    got = run(A, B, dtype, out_fp32, variant)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B), dtype)
    if out_fp32:
        assert np.array_equal(got.numpy(), ref)
    else:
        assert np.array_equal(as_bits(got), oracle.encode(ref, dtype))


VARIANTS = ["generic_64x64x16", "pipelined_256x256x64_s2", "pipelined_128x128x64_s2",
            "pipelined_256x256x32_s4", "pipelined_256x256x32_s5", "pipelined_128x128x32_s4",
            "skinny_64x32_w4_k64_s4", "skinny_64x128_w4_k32_s4_splitk", "repack_pipelined",
            "pipelined_256x256x32_s4_apair", "skinny_64x128_ring_k32_s4_splitk"]
# the pipelined variants need K to be a multiple of the K-tile spanning at
# least as many tiles as ring stages (K >= 160 covers every variant), 16-byte
# aligned rows (ld % 8 == 0) and N % 8 == 0; M is free and N may end inside
# a tile (200, 520, 136 below)
SHAPES_PIPE = [(256, 256, 256), (512, 384, 320), (300, 200, 192), (1, 8, 256), (33, 520, 192),
               (129, 136, 256), (640, 768, 512), (256, 512, 1024)]
SHAPES_GENERIC_ONLY = [(100, 70, 50), (5, 3, 1), (257, 65, 129), (129, 129, 64), (64, 64, 64), (96, 201, 256)]
# K % BK != 0 with K % 8 == 0: the variants whose ring leaves room for a tail
# stage copy the partial last K-tile first and consume it last.  K = 136 has
# exactly as many full 32-wide tiles as the 4-stage ring (and two 64-wide
# ones); 200, 248 and 1032 leave tails of 8, 24 and 8 (64-wide: 8, 56, 8)
TAIL_VARIANTS = ["pipelined_128x128x64_s2", "pipelined_256x256x32_s4", "pipelined_128x128x32_s4"]
SHAPES_KTAIL = [(256, 256, 136), (300, 264, 200), (129, 520, 248), (384, 512, 1032), (1, 8, 136)]


# the skinny variant splits K over 4 waves in 64-deep chunks, 4 per wave at
# least: K a multiple of 256 and >= 1024; any M (64-row tiles); N % 8 == 0 with
# a ragged last 32-column tile; chunk counts per wave at the ring depth (K =
# 1024) and above it so stages are reused
SHAPES_SKINNY = [(64, 1024, 2048), (37, 320, 2560), (100, 256, 2048), (1, 512, 4096), (64, 2048, 3072),
                 (64, 200, 1024), (70, 264, 1280), (64, 256, 8192)]
# the wide skinny variant: 128-column blocks, K split over S workgroups with
# S*128 | K and K/(S*128) >= 4.  Above, S comes out as 4, 4, 4, 8, 4, 2, 2, 8
# (the fewest splits reaching 256 workgroups, else the most that K allows);
# these two allow S = 1 only (no workspace, no second kernel)
SHAPES_WIDE_ONLY = [(64, 1024, 512), (3, 136, 640)]
# the shared-ring skinny variant takes any K that is a multiple of 64 per
# split: one chunk, and fewer chunks than the ring has stages (the copies
# past the last chunk read zeros)
SHAPES_RING_ONLY = [(64, 256, 64), (5, 136, 192), (64, 512, 320)]


# the repack route copies A and B zero-padded to K, N rounded up to 8 with
# aligned rows, then runs a pipelined kernel: odd N (201, 65, 1000, 7), odd
# K (129 -> 136 gives four 32-wide tiles and a tail; 250 -> 256), tight
# (odd) leading dimensions throughout
SHAPES_REPACK = [(300, 201, 256), (257, 65, 129), (129, 129, 250), (64, 1000, 1000), (1, 7, 130),
                 (96, 201, 256), (512, 512, 512)]


def _shapes(vname):
    if vname == "repack_pipelined":
        return SHAPES_REPACK
    if vname == "skinny_64x128_ring_k32_s4_splitk":
        return SHAPES_SKINNY + SHAPES_WIDE_ONLY + SHAPES_RING_ONLY
    if vname.startswith("skinny_64x128"):
        return SHAPES_SKINNY + SHAPES_WIDE_ONLY
    if vname.startswith("skinny"):
        return SHAPES_SKINNY
    extra = SHAPES_GENERIC_ONLY if vname.startswith("generic") else []
    if vname in TAIL_VARIANTS or vname.startswith("generic"):
        extra = extra + SHAPES_KTAIL
    return SHAPES_PIPE + extra


@pytest.mark.parametrize("vname", VARIANTS)
@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("f16", True), ("bf16", True), ("bf16", False)])
def test_variant_parity_random(vname, dtype, out_fp32):
    v = pkg.variants()[vname]
    for i, (M, N, K) in enumerate(_shapes(vname)):
        say(f"[random] {vname} {dtype} out_fp32={out_fp32} M={M} N={N} K={K}")
        A = inputs.uniform((M, K), 1000 + i, dtype=dtype, nonzero=True)
        B = inputs.uniform((K, N), 2000 + i, dtype=dtype, nonzero=True)
        check_random(A, B, dtype, out_fp32, v)


@pytest.mark.parametrize("vname", VARIANTS)
@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("f16", True), ("bf16", True)])
def test_variant_parity_exact_integers(vname, dtype, out_fp32):
    v = pkg.variants()[vname]
    for i, (M, N, K) in enumerate(_shapes(vname)):
        say(f"[exact] {vname} {dtype} out_fp32={out_fp32} M={M} N={N} K={K}")
        A = inputs.small_integers((M, K), 3000 + i, dtype=dtype)
        B = inputs.small_integers((K, N), 4000 + i, dtype=dtype)
        check_exact(A, B, dtype, out_fp32, v)


def test_small_workload_all_rotating_sets():
    w = inputs.WORKLOADS["f16_256"]
    for j in range(w.rotating):
        say(f"[f16_256] set {j}")
        A, B = w.make_a(j), w.make_b(j)
        m = check_random(A, B, "f16", False)
        assert m["rel_rms"] < 1e-3


def test_identity_and_permutation_exact():
    K = 512
    B = inputs.uniform((K, 384), 5001, nonzero=True)
    I = torch.eye(K, dtype=torch.float16)
    assert torch.equal(run(I, B), B)                       # A = I gives B exactly
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(5))
    P = torch.zeros(K, K, dtype=torch.float16)
    P[torch.arange(K), perm] = 1
    assert torch.equal(run(P, B), B[perm])                 # P B permutes rows


PADDED_CASES = [(v, 70, 200, 2048) if v.startswith("skinny") else (v, 300, 200, 192) for v in VARIANTS] + \
    [("generic_64x64x16", 300, 201, 200)] + [(v, 300, 200, 200) for v in TAIL_VARIANTS] + \
    [("repack_pipelined", 300, 201, 250)]


@pytest.mark.parametrize("vname,M,N,K", PADDED_CASES)
def test_padded_leading_dimensions_nan_padding(vname, M, N, K):
    """lda > K, ldb > N, ldc > N with NaN in every padding element: the
    result must be finite and correct, and C's padding must be untouched.
    N = 200 ends inside the last column tile of every fast variant; the
    guarded kernel also takes N = 201 and K = 200."""
    v = pkg.variants()[vname]
    say(f"[padded] {vname} M={M} N={N} K={K}")
    A = inputs.uniform((M, K), 6001, nonzero=True)
    B = inputs.uniform((K, N), 6002, nonzero=True)
    Ap = torch.full((M, K + 8), float("nan"), dtype=torch.float16)
    Ap[:, :K] = A
    Bp = torch.full((K, N + 24), float("nan"), dtype=torch.float16)
    Bp[:, :N] = B
    Cp = torch.full((M, N + 8), 7.0, dtype=torch.float16, device=DEV)
    pkg.gemm_ex(Ap.to(DEV)[:, :K], Bp.to(DEV)[:, :N], Cp[:, :N], variant=v)
    torch.cuda.synchronize()
    Cp = Cp.cpu()
    assert torch.all(Cp[:, N:] == 7.0)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B))
    m = oracle.compare(Cp[:, :N].float().numpy(), ref, K)
    assert m["ok"], (vname, m)


def test_k_zero_writes_zeros_and_empty_is_noop():
    C = torch.full((40, 24), 3.0, dtype=torch.float16, device=DEV)
    A = torch.empty((40, 0), dtype=torch.float16, device=DEV)
    B = torch.empty((0, 24), dtype=torch.float16, device=DEV)
    pkg.gemm_ex(A, B, C)
    torch.cuda.synchronize()
    assert torch.all(C == 0)
    C2 = torch.full((0, 24), 3.0, dtype=torch.float16, device=DEV)
    pkg.gemm_ex(torch.empty((0, 8), dtype=torch.float16, device=DEV),
                torch.ones((8, 24), dtype=torch.float16, device=DEV), C2)


@pytest.mark.parametrize("vname", VARIANTS)
def test_batched_small(vname):
    v = pkg.variants()[vname]
    b, M, N, K = (3, 64, 256, 2048) if vname.startswith("skinny") else (3, 160, 192, 192)
    say(f"[batched] {vname}")
    A = inputs.uniform((b, M, K), 7001, lo=-0.5, hi=0.5)
    B = inputs.uniform((b, K, N), 7002, lo=-0.5, hi=0.5)
    got = run(A, B, "f16", False, v)
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B))
    m = oracle.compare(got.float().numpy(), ref, K)
    assert m["ok"], m
    Ai = inputs.small_integers((b, M, K), 7003)
    Bi = inputs.small_integers((b, K, N), 7004)
    gi = run(Ai, Bi, "f16", True, v)
    assert np.array_equal(gi.numpy(), oracle.gemm(inputs.bits(Ai), inputs.bits(Bi)))


# the persistent short-K kernel: whole 256 x 128 tiles, K = 128 or 256,
# 16-bit C, at least 256 tiles.  Tile counts 256, 384 (some workgroups walk
# two tiles, some one), 512, and 512 over 32 batch entries; 400 tiles of 5
# row blocks, which the A-resident kernel walks as 100 groups of 4 on a grid
# of 100 (not a multiple of 8: the plain round-robin walk).
PERSIST_SHAPES = [("f16", 4, 1024, 2048, 256), ("f16", 6, 2048, 1024, 256), ("bf16", 1, 4096, 4096, 256),
                  ("f16", 32, 512, 1024, 256), ("f16", 6, 2048, 1024, 128), ("bf16", 4, 1024, 2048, 128),
                  ("f16", 5, 1280, 2048, 256)]


PERSIST_VARIANTS = ["persistent_256x128x32_shortk", "persistent_256x128x32_shortk_apair",
                    "persistent_256x128x32_shortk_aresident"]


@pytest.mark.parametrize("vname", PERSIST_VARIANTS)
@pytest.mark.parametrize("dtype,batch,M,N,K", PERSIST_SHAPES)
def test_persistent_parity(dtype, batch, M, N, K, vname):
    v = pkg.variants()[vname]
    say(f"[persistent] {vname} {dtype} batch={batch} M={M} N={N} K={K}")
    A = inputs.uniform((batch, M, K), 7701 + M + N, dtype=dtype, nonzero=True)
    B = inputs.uniform((batch, K, N), 7702 + M + N, dtype=dtype, nonzero=True)
    check_random(A, B, dtype, False, v)
    Ai = inputs.small_integers((batch, M, K), 7703, dtype=dtype)
    Bi = inputs.small_integers((batch, K, N), 7704, dtype=dtype)
    got = run(Ai, Bi, dtype, False, v)
    assert np.array_equal(as_bits(got), oracle.encode(oracle.gemm(inputs.bits(Ai), inputs.bits(Bi), dtype), dtype))


@pytest.mark.parametrize("vname", PERSIST_VARIANTS)
@pytest.mark.parametrize("K", [256, 128])
def test_persistent_padded_views_nan_padding(K, vname):
    """lda > K, ldb > N, ldc > N and batch strides from padded tensors, NaN
    in every padding element of A and B: the result must be correct and C's
    padding untouched."""
    v = pkg.variants()[vname]
    b, M, N = 4, 1024, 2048                       # 256 tiles of 256 x 128
    say(f"[persistent padded] b={b} M={M} N={N} K={K}")
    A = inputs.uniform((b, M, K), 7721 + K, nonzero=True)
    B = inputs.uniform((b, K, N), 7722 + K, nonzero=True)
    Ap = torch.full((b, M, K + 8), float("nan"), dtype=torch.float16)
    Ap[:, :, :K] = A
    Bp = torch.full((b, K, N + 24), float("nan"), dtype=torch.float16)
    Bp[:, :, :N] = B
    Cp = torch.full((b, M, N + 8), 7.0, dtype=torch.float16, device=DEV)
    pkg.gemm_ex(Ap.to(DEV)[:, :, :K], Bp.to(DEV)[:, :, :N], Cp[:, :, :N], variant=v)
    torch.cuda.synchronize()
    Cp = Cp.cpu()
    assert torch.all(Cp[:, :, N:] == 7.0)
    m = oracle.compare(Cp[:, :, :N].float().numpy(), oracle.gemm(inputs.bits(A), inputs.bits(B)), K)
    assert m["ok"], m


@pytest.mark.parametrize("vname", PERSIST_VARIANTS)
def test_persistent_repeated_calls(vname):
    """Back-to-back calls on one stream, the second into a C that the first
    filled: every call writes every tile once, bit-identical each time."""
    v = pkg.variants()[vname]
    A = inputs.uniform((6, 2048, 256), 7711, nonzero=True).to(DEV)
    B = inputs.uniform((6, 256, 1024), 7712, nonzero=True).to(DEV)
    outs = [pkg.gemm_ex(A, B, variant=v) for _ in range(4)]
    C = torch.full((6, 2048, 1024), float("nan"), dtype=torch.float16, device=DEV)
    pkg.gemm_ex(A, B, C, variant=v)
    torch.cuda.synchronize()
    for o in outs[1:] + [C]:
        assert torch.equal(o, outs[0])


# the persistent kernel with wave roles: whole 128 x 256 tiles, K = 128 or
# 256, 16-bit C, at least 256 row blocks.  256 row blocks (one per
# workgroup), 320 (some workgroups walk two, reloading the A panel mid-walk),
# 3 column tiles per row, and 1 (a new panel every tile).
ROLES = "persistent_128x256x32_shortk_roles"
ROLES_SHAPES = [("f16", 8, 4096, 1024, 256), ("f16", 10, 4096, 512, 256), ("bf16", 16, 2048, 768, 256),
                ("f16", 9, 4096, 256, 128), ("bf16", 64, 512, 512, 128)]


@pytest.mark.parametrize("dtype,batch,M,N,K", ROLES_SHAPES)
def test_roles_parity(dtype, batch, M, N, K):
    v = pkg.variants()[ROLES]
    say(f"[roles] {dtype} batch={batch} M={M} N={N} K={K}")
    A = inputs.uniform((batch, M, K), 7801 + M + N, dtype=dtype, nonzero=True)
    B = inputs.uniform((batch, K, N), 7802 + M + N, dtype=dtype, nonzero=True)
    check_random(A, B, dtype, False, v)
    # into a NaN-filled C: each workgroup walks its row blocks' column tiles
    # in a rotated order, and every tile must be written exactly once
    Ai = inputs.small_integers((batch, M, K), 7803, dtype=dtype)
    Bi = inputs.small_integers((batch, K, N), 7804, dtype=dtype)
    C = torch.full((batch, M, N), float("nan"), dtype=torch.float16 if dtype == "f16" else torch.bfloat16, device=DEV)
    got = run(Ai, Bi, dtype, False, v, C=C)
    assert np.array_equal(as_bits(got), oracle.encode(oracle.gemm(inputs.bits(Ai), inputs.bits(Bi), dtype), dtype))


@pytest.mark.parametrize("K", [256, 128])
def test_roles_match_the_pair_kernel_bitwise(K):
    """The wave-role kernel and the A-pair persistent kernel run the same
    products in the same order: bitwise equal C on random inputs."""
    V = pkg.variants()
    b, M, N = 12, 4096, 1024                      # 384 row blocks: uneven walks
    say(f"[roles vs pair] b={b} M={M} N={N} K={K}")
    A = inputs.uniform((b, M, K), 7811 + K, nonzero=True).to(DEV)
    B = inputs.uniform((b, K, N), 7812 + K, nonzero=True).to(DEV)
    r = pkg.gemm_ex(A, B, variant=V[ROLES])
    q = pkg.gemm_ex(A, B, variant=V["persistent_256x128x32_shortk_apair"])
    torch.cuda.synchronize()
    assert torch.equal(r.view(torch.int16), q.view(torch.int16))


@pytest.mark.parametrize("K", [256, 128])
def test_roles_padded_views_nan_padding(K):
    """lda > K, ldb > N, ldc > N and batch strides from padded tensors, NaN in
    every padding element of A and B: correct, and C's padding untouched."""
    v = pkg.variants()[ROLES]
    b, M, N = 8, 4096, 512
    say(f"[roles padded] b={b} M={M} N={N} K={K}")
    A = inputs.uniform((b, M, K), 7821 + K, nonzero=True)
    B = inputs.uniform((b, K, N), 7822 + K, nonzero=True)
    Ap = torch.full((b, M, K + 8), float("nan"), dtype=torch.float16)
    Ap[:, :, :K] = A
    Bp = torch.full((b, K, N + 24), float("nan"), dtype=torch.float16)
    Bp[:, :, :N] = B
    Cp = torch.full((b, M, N + 8), 7.0, dtype=torch.float16, device=DEV)
    pkg.gemm_ex(Ap.to(DEV)[:, :, :K], Bp.to(DEV)[:, :, :N], Cp[:, :, :N], variant=v)
    torch.cuda.synchronize()
    Cp = Cp.cpu()
    assert torch.all(Cp[:, :, N:] == 7.0)
    m = oracle.compare(Cp[:, :, :N].float().numpy(), oracle.gemm(inputs.bits(A), inputs.bits(B)), K)
    assert m["ok"], m


def test_roles_repeated_calls():
    """Back-to-back calls on one stream, the last into a NaN-filled C: every
    call writes every tile once, bit-identical each time."""
    v = pkg.variants()[ROLES]
    A = inputs.uniform((10, 4096, 256), 7831, nonzero=True).to(DEV)
    B = inputs.uniform((10, 256, 512), 7832, nonzero=True).to(DEV)
    outs = [pkg.gemm_ex(A, B, variant=v) for _ in range(4)]
    C = torch.full((10, 4096, 512), float("nan"), dtype=torch.float16, device=DEV)
    pkg.gemm_ex(A, B, C, variant=v)
    torch.cuda.synchronize()
    for o in outs[1:] + [C]:
        assert torch.equal(o, outs[0])


def test_batched_entry_point():
    b, M, N, K = 4, 256, 256, 256
    A = inputs.uniform((b, M, K), 7101, lo=-0.5, hi=0.5)
    B = inputs.uniform((b, K, N), 7102, lo=-0.5, hi=0.5)
    C = pkg.gemm_batched_f16(A.to(DEV), B.to(DEV))
    torch.cuda.synchronize()
    m = oracle.compare(C.cpu().float().numpy(), oracle.gemm(inputs.bits(A), inputs.bits(B)), K)
    assert m["ok"], m


def test_repeat_runs_bitwise_identical():
    w = inputs.WORKLOADS["f16_256"]
    A, B = w.make_a(0).to(DEV), w.make_b(0).to(DEV)
    outs = [pkg.gemm_f16(A, B).cpu() for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


@pytest.mark.parametrize("M,N,K,vname", [(64, 2048, 4096, "skinny_64x128_ring_k32_s4_splitk"),   # 16 splits eager
                                         (256, 2048, 4096, "splitk_pipelined")])                # 8 splits eager
def test_graph_capture_of_a_split_k_call(M, N, K, vname):
    """A call captured into a graph takes no buffer from the workspace pool (a
    graph would keep its address): captured, the split-K paths run unsplit.
    Exact-integer inputs make the split (eager) and unsplit (captured) sums
    bit-identical, so every replay -- with eager calls and synchronisations
    between replays -- must equal the oracle exactly."""
    assert pkg.select_variant("f16", 1, M, N, K, K, N, True) == pkg.variants()[vname]
    A = inputs.small_integers((M, K), 7501)
    B = inputs.small_integers((K, N), 7502)
    ref = torch.from_numpy(oracle.gemm(inputs.bits(A), inputs.bits(B), "f16"))
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    pkg.gemm_f16(Ad, Bd, C, out_fp32=True)
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                 # warm-up on a side stream, as torch advises
        pkg.gemm_f16(Ad, Bd, C, out_fp32=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkg.gemm_f16(Ad, Bd, C, out_fp32=True)
    for rep in range(3):
        C.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.cpu(), ref), rep
        eager = pkg.gemm_f16(Ad, Bd, out_fp32=True)
        torch.cuda.synchronize()
        assert torch.equal(eager.cpu(), ref), rep


@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("bf16", True)])
def test_repack_unaligned_bases(dtype, out_fp32):
    """Views that start one element into their storage (2-byte aligned bases)
    and have odd row strides: the automatic choice copies them into aligned,
    zero-padded buffers and runs the pipelined kernel; C is a view too."""
    M, N, K = 384, 263, 520
    Af = inputs.uniform((M, K + 3), 7601, dtype=dtype, nonzero=True)
    Bf = inputs.uniform((K, N + 5), 7602, dtype=dtype, nonzero=True)
    A, B = Af[:, 1:K + 1], Bf[:, 3:N + 3]
    assert pkg.select_variant(dtype, 1, M, N, K, K + 3, N + 5, out_fp32, A_ptr=(1 << 20) + 2) == \
        pkg.variants()["repack_pipelined"]
    out_t = torch.float32 if out_fp32 else (torch.float16 if dtype == "f16" else torch.bfloat16)
    Cf = torch.full((M, N + 1), 5.0, dtype=out_t, device=DEV)
    pkg.gemm_ex(Af.to(DEV)[:, 1:K + 1], Bf.to(DEV)[:, 3:N + 3], Cf[:, 1:], dtype=dtype, out_fp32=out_fp32)
    torch.cuda.synchronize()
    Cf = Cf.cpu()
    assert torch.all(Cf[:, 0] == 5.0)
    ref = oracle.gemm(inputs.bits(A.contiguous()), inputs.bits(B.contiguous()), dtype)
    m = oracle.compare(Cf[:, 1:].float().numpy(), ref, K)
    assert m["ok"], m


def test_repack_full_size_odd_shape():
    """4000 x 4095 x 4090 (odd N and K, tight leading dimensions) through the
    automatic choice: sampled against the oracle, random and exact-integer."""
    M, N, K = 4000, 4095, 4090
    assert pkg.select_variant("f16", 1, M, N, K, K, N) == pkg.variants()["repack_pipelined"]
    b, r, c = _sample_positions(1, M, N, 2048, 23)
    for kind in ("random", "exact"):
        if kind == "random":
            A = inputs.uniform((M, K), 7701, nonzero=True)
            B = inputs.uniform((K, N), 7702, nonzero=True)
        else:
            A = inputs.small_integers((M, K), 7703)
            B = inputs.small_integers((K, N), 7704)
        say(f"[repack full] {kind}")
        C = pkg.gemm_f16(A.to(DEV), B.to(DEV), out_fp32=(kind == "exact"))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(C).all().item())
        got = C[torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV)].cpu()
        ref = oracle.gemm_at(inputs.bits(A), inputs.bits(B), b, r, c, "f16")
        if kind == "random":
            m = oracle.compare(got.float().numpy(), ref, K)
            assert m["ok"], m
        else:
            assert np.array_equal(got.numpy(), ref)


def test_graph_of_a_pass_over_rotating_sets():
    """The launch-bound 256^3 shape as bench.py --graph runs it: one graph
    holding the calls on several rotating (A, B, C) sets, captured on a
    non-default stream.  Exact-integer inputs; every replay, with eager
    calls and synchronisations between replays, gives each C the oracle's
    RNE encoding bit for bit."""
    M = N = K = 256
    sets = []
    for j in range(4):
        A = inputs.small_integers((M, K), 7601 + 2 * j)
        B = inputs.small_integers((K, N), 7602 + 2 * j)
        ref = oracle.encode(oracle.gemm(inputs.bits(A), inputs.bits(B), "f16"), "f16")
        sets.append((A.to(DEV), B.to(DEV), torch.empty((M, N), dtype=torch.float16, device=DEV), ref))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        for A, B, C, _ in sets:                    # one eager pass first
            pkg.gemm_f16(A, B, C, stream=s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for A, B, C, _ in sets:
                pkg.gemm_f16(A, B, C, stream=s)
        for rep in range(3):
            for _, _, C, _ in sets:
                C.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for j, (A, B, C, ref) in enumerate(sets):
                assert np.array_equal(as_bits(C.cpu()), ref), (rep, j)
            eager = pkg.gemm_f16(sets[0][0], sets[0][1], stream=s)
            torch.cuda.synchronize()
            assert np.array_equal(as_bits(eager.cpu()), sets[0][3]), rep


def test_graph_capture_of_a_repack_call():
    """Under graph capture the repack route may not use its workspace, so the
    guarded kernel takes the call; every replay must still be exact."""
    M, N, K = 512, 511, 520
    assert pkg.select_variant("f16", 1, M, N, K, K, N, True) == pkg.variants()["repack_pipelined"]
    A = inputs.small_integers((M, K), 7801)
    B = inputs.small_integers((K, N), 7802)
    ref = torch.from_numpy(oracle.gemm(inputs.bits(A), inputs.bits(B), "f16"))
    Ad, Bd = A.to(DEV), B.to(DEV)
    C = torch.empty((M, N), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pkg.gemm_f16(Ad, Bd, C, out_fp32=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkg.gemm_f16(Ad, Bd, C, out_fp32=True)
    for rep_i in range(3):
        C.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.cpu(), ref), rep_i
        eager = pkg.gemm_f16(Ad, Bd, out_fp32=True)
        torch.cuda.synchronize()
        assert torch.equal(eager.cpu(), ref), rep_i


SPLIT_VARIANTS = ["skinny_64x128_w4_k32_s4_splitk", "skinny_64x128_ring_k32_s4_splitk"]


@pytest.mark.parametrize("vname", SPLIT_VARIANTS)
def test_split_k_workspace_streams_and_growth(vname):
    """The split-K path takes its partials' buffer from a per-device pool
    whose buffers are ordered by events: calls on two streams in flight
    together, and a call that needs a larger buffer after a smaller one, must
    each give the result of a lone call, bit for bit (the split sums run in a
    fixed order)."""
    v = pkg.variants()[vname]
    shapes = [(64, 256, 2048), (64, 2048, 4096), (32, 1024, 8192)]     # 4-8 splits; growing
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A = inputs.uniform((M, K), 7201 + i, nonzero=True).to(DEV)
        B = inputs.uniform((K, N), 7301 + i, nonzero=True).to(DEV)
        data.append((A, B))
    lone = [run(A.cpu(), B.cpu(), "f16", True, v) for A, B in data]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for rep in range(3):
        for i, (A, B) in enumerate(data):
            st = s1 if (i + rep) % 2 == 0 else s2
            C = torch.empty((A.shape[0], B.shape[1]), dtype=torch.float32, device=DEV)
            with torch.cuda.stream(st):
                pkg.gemm_ex(A, B, C, out_fp32=True, variant=v, stream=st)
            outs.append((i, C))
    torch.cuda.synchronize()
    for i, C in outs:
        assert torch.equal(C.cpu(), lone[i]), i


@pytest.mark.parametrize("vname", SPLIT_VARIANTS)
def test_split_k_repeated_and_interleaved(vname):
    """Many split-K calls in a row on one stream -- 2 to 64 splits, with
    repack calls that reuse the pooled buffers in between -- must each give
    the lone call's result bit for bit (the partials are added in split
    order, in groups of 8 above 8 splits), and that result meets the
    oracle."""
    v = pkg.variants()[vname]
    # wide kernel: S = 2, 4, 8, 32, 64 (one 64 x 128 block over K = 16384
    # and 32768: the most splits K allows); the ring kernel takes S = 1 .. 64
    # by its own rule
    shapes = [(64, 200, 1024), (64, 1024, 2048), (64, 2048, 4096), (64, 128, 16384), (64, 128, 32768)]
    rp_A = inputs.uniform((257, 129), 7601, nonzero=True).to(DEV)
    rp_B = inputs.uniform((129, 201), 7602, nonzero=True).to(DEV)
    rp_ref = run(rp_A.cpu(), rp_B.cpu(), "f16", True, pkg.variants()["repack_pipelined"])
    for i, (M, N, K) in enumerate(shapes):
        say(f"split-K repeated M={M} N={N} K={K}")
        A = inputs.uniform((M, K), 7611 + i, nonzero=True)
        B = inputs.uniform((K, N), 7621 + i, nonzero=True)
        lone = run(A, B, "f16", True, v)
        m = oracle.compare(lone.numpy(), oracle.gemm(inputs.bits(A), inputs.bits(B), "f16"), K)
        assert m["ok"], m
        Ad, Bd = A.to(DEV), B.to(DEV)
        outs, rps = [], []
        for rep in range(24):
            C = torch.empty((M, N), dtype=torch.float32, device=DEV)
            pkg.gemm_ex(Ad, Bd, C, out_fp32=True, variant=v)
            outs.append(C)
            if rep % 5 == 2:
                rps.append(pkg.gemm_ex(rp_A, rp_B, out_fp32=True, variant=pkg.variants()["repack_pipelined"]))
        torch.cuda.synchronize()
        for rep, C in enumerate(outs):
            assert torch.equal(C.cpu(), lone), (M, N, K, rep)
        for C in rps:
            assert torch.equal(C.cpu(), rp_ref)


class _RawStream:
    """A bare HIP stream handle in the shape the binding takes (.cuda_stream)."""
    def __init__(self, handle):
        self.cuda_stream = handle


def _hip_runtime():
    import ctypes
    path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
    hip = ctypes.CDLL(path)          # the runtime this process already uses
    hip.hipStreamCreate.argtypes = [ctypes.c_void_p]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return hip


def test_workspace_streams_created_and_destroyed():
    """Split-K calls (the skinny workload shape, 4 splits through the
    automatic choice) each on a new stream destroyed right after the call,
    while its kernels may still run: a later stream can receive the same
    handle, and the pool's events must keep its call off the buffer until the
    earlier kernels are done.  Every result must equal a lone call's bit for
    bit; the first mismatch fails."""
    import ctypes
    hip = _hip_runtime()
    M, N, K = 64, 8192, 8192
    A = inputs.uniform((M, K), 7701, nonzero=True)
    Bs = [inputs.uniform((K, N), 7702 + j, nonzero=True) for j in range(2)]
    lone = [run(A, B, "f16", False) for B in Bs]
    Ad, Bds = A.to(DEV), [B.to(DEV) for B in Bs]
    outs, handles = [], []
    for rep in range(32):
        h = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(h)) == 0
        handles.append(h.value)
        C = torch.empty((M, N), dtype=torch.float16, device=DEV)
        pkg.gemm_f16(Ad, Bds[rep % 2], C, stream=_RawStream(h.value))
        assert hip.hipStreamDestroy(h) == 0
        outs.append((rep % 2, C))
    torch.cuda.synchronize()
    say(f"distinct stream handles over 32 streams: {len(set(handles))}")
    for rep, (j, C) in enumerate(outs):
        assert torch.equal(C.cpu(), lone[j]), rep
    m = oracle.compare(lone[0].float().numpy(), oracle.gemm(inputs.bits(A), inputs.bits(Bs[0]), "f16"), K)
    assert m["ok"], m


def test_workspace_per_thread_streams_from_two_threads():
    """hipStreamPerThread is one handle that names a different stream on
    each host thread.  Two threads issue split-K calls on it at the same
    time, with different inputs: every result must equal a lone call's bit
    for bit."""
    import threading
    per_thread = _RawStream(2)                 # hipStreamPerThread
    M, N, K = 64, 4096, 8192
    data = []
    for t in range(2):
        A = inputs.uniform((M, K), 7711 + t, nonzero=True)
        B = inputs.uniform((K, N), 7721 + t, nonzero=True)
        data.append((A, B, run(A, B, "f16", True)))
    dev_data = [(A.to(DEV), B.to(DEV)) for A, B, _ in data]
    outs = [[], []]
    errors = []

    def worker(t):
        try:
            Ad, Bd = dev_data[t]
            for rep in range(40):
                C = torch.empty((M, N), dtype=torch.float32, device=DEV)
                pkg.gemm_ex(Ad, Bd, C, out_fp32=True, stream=per_thread)
                outs[t].append(C)
        except Exception as exc:               # reported below, in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        assert len(outs[t]) == 40
        for rep, C in enumerate(outs[t]):
            assert torch.equal(C.cpu(), data[t][2]), (t, rep)


# split-K over the pipelined kernel's batch: M > 128, at most 128 tiles of
# 128 x 128, K a multiple of 64 * S with K / S >= 256.  Ragged M and N;
# S = 4, 8, 2, 8, 2, 4, 32 and 64 below
SHAPES_SPLITK = [(256, 1024, 1024), (300, 520, 2048), (129, 136, 512), (640, 768, 4096), (200, 8192, 1024),
                 (1024, 1024, 8192), (256, 512, 32768), (256, 256, 16384)]     # ... and 64


@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("f16", True), ("bf16", True), ("bf16", False)])
def test_splitk_parity(dtype, out_fp32):
    """Random inputs within tolerance, integer inputs bitwise (the partials
    and their sum are exact), each through the automatic choice."""
    v = pkg.variants()["splitk_pipelined"]
    for i, (M, N, K) in enumerate(SHAPES_SPLITK):
        say(f"[split-K] M={M} N={N} K={K} {dtype} out_fp32={out_fp32}")
        assert pkg.select_variant(dtype, 1, M, N, K, K, N, out_fp32) == v
        A = inputs.uniform((M, K), 7901 + i, nonzero=True, dtype=dtype)
        B = inputs.uniform((K, N), 7911 + i, nonzero=True, dtype=dtype)
        check_random(A, B, dtype, out_fp32)
        A = inputs.small_integers((M, K), 7921 + i, dtype=dtype)
        B = inputs.small_integers((K, N), 7931 + i, dtype=dtype)
        check_exact(A, B, dtype, out_fp32)


@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("bf16", True)])
def test_splitk_bt_parity(dtype, out_fp32):
    """B given transposed (N x K): each K range reads its columns of Bt.
    Random inputs within tolerance, integer inputs bitwise."""
    v = pkg.variants()["splitk_pipelined"]
    for i, (M, N, K) in enumerate(SHAPES_SPLITK[:4]):
        say(f"[split-K bt] M={M} N={N} K={K} {dtype} out_fp32={out_fp32}")
        assert pkg.select_variant(dtype, 1, M, N, K, K, K, out_fp32, bt=True) == v
        for kind in ("random", "exact"):
            if kind == "random":
                A = inputs.uniform((M, K), 7981 + i, nonzero=True, dtype=dtype)
                Bt = inputs.uniform((N, K), 7991 + i, nonzero=True, dtype=dtype)
            else:
                A = inputs.small_integers((M, K), 7985 + i, dtype=dtype)
                Bt = inputs.small_integers((N, K), 7995 + i, dtype=dtype)
            got = pkg.gemm_ex_bt(A.to(DEV), Bt.to(DEV), dtype=dtype, out_fp32=out_fp32).cpu()
            ref = oracle.gemm(inputs.bits(A), inputs.bits(Bt.t().contiguous()), dtype)
            if kind == "random":
                m = oracle.compare(got.float().numpy(), ref, K)
                assert m["ok"], m
            elif out_fp32:
                assert np.array_equal(got.numpy(), ref)
            else:
                assert np.array_equal(as_bits(got), oracle.encode(ref, dtype))


@pytest.mark.parametrize("out_fp32", [False, True])
def test_splitk_padded_views(out_fp32):
    """Views with padded leading dimensions; C rows of odd length (element
    stores from the sum kernel).  The padding, NaN, stays untouched."""
    M, N, K = 300, 520, 2048
    A0 = inputs.small_integers((M, K + 64), 7941)
    B0 = inputs.small_integers((K, N + 8), 7942)
    A, B = A0[:, :K], B0[:, :N]
    ref = oracle.gemm(inputs.bits(A.contiguous()), inputs.bits(B.contiguous()), "f16")
    out_t = torch.float32 if out_fp32 else torch.float16
    Cbuf = torch.full((M, N + 3), float("nan"), dtype=out_t, device=DEV)
    C = Cbuf[:, :N]
    Ad, Bd = A0.to(DEV)[:, :K], B0.to(DEV)[:, :N]
    assert pkg.select_variant("f16", 1, M, N, K, K + 64, N + 8, out_fp32) == pkg.variants()["splitk_pipelined"]
    pkg.gemm_ex(Ad, Bd, C, out_fp32=out_fp32)
    torch.cuda.synchronize()
    got = C.cpu()
    if out_fp32:
        assert np.array_equal(got.numpy(), ref)
    else:
        assert np.array_equal(as_bits(got), oracle.encode(ref, "f16"))
    assert torch.isnan(Cbuf[:, N:].float()).all()


def test_splitk_repeated_with_other_workspace_users():
    """Split-K calls of different split counts in a row on one stream, with
    skinny split-K calls (the same workspace) in between: each equals the
    lone call bit for bit."""
    v = pkg.variants()["splitk_pipelined"]
    shapes = [(256, 1024, 1024), (200, 8192, 1024), (640, 768, 4096)]
    sk_A = inputs.uniform((64, 4096), 7951, nonzero=True).to(DEV)
    sk_B = inputs.uniform((4096, 2048), 7952, nonzero=True).to(DEV)
    sk_ref = pkg.gemm_ex(sk_A, sk_B, out_fp32=True).cpu()
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A = inputs.uniform((M, K), 7961 + i, nonzero=True)
        B = inputs.uniform((K, N), 7971 + i, nonzero=True)
        data.append((A.to(DEV), B.to(DEV), run(A, B, "f16", True, v)))
    outs, sks = [], []
    for rep in range(4):
        for i, (Ad, Bd, _) in enumerate(data):
            outs.append((i, pkg.gemm_ex(Ad, Bd, out_fp32=True, variant=v)))
            sks.append(pkg.gemm_ex(sk_A, sk_B, out_fp32=True))
    torch.cuda.synchronize()
    for i, C in outs:
        assert torch.equal(C.cpu(), data[i][2]), i
    for C in sks:
        assert torch.equal(C.cpu(), sk_ref)


# ----------------------------------------------------------------------------
# full workload sizes, automatic variant choice (the benchmark's launches)
# ----------------------------------------------------------------------------

def _sample_positions(batch, M, N, n, seed):
    rng = np.random.default_rng(seed)
    b = rng.integers(0, batch, n)
    r = rng.integers(0, M, n)
    c = rng.integers(0, N, n)
    # corners of the first and last batch entry
    b = np.concatenate([b, [0, 0, batch - 1, batch - 1]])
    r = np.concatenate([r, [0, M - 1, 0, M - 1]])
    c = np.concatenate([c, [N - 1, 0, 0, N - 1]])
    return b, r, c


def _full_size(w, A, B):
    """Run workload w on the GPU; return (all-finite flag, sampled GPU values
    as float64, sample positions)."""
    Ad, Bd = A.to(DEV), B.to(DEV)
    if w.batch > 1:
        C = pkg.gemm_batched_f16(Ad, Bd, out_fp32=w.out_fp32)
    elif w.dtype == "f16":
        C = pkg.gemm_f16(Ad, Bd, out_fp32=w.out_fp32)
    else:
        C = pkg.gemm_bf16(Ad, Bd, out_fp32=w.out_fp32)
    torch.cuda.synchronize()
    finite = bool(torch.isfinite(C).all().item())
    C3 = C if C.dim() == 3 else C.unsqueeze(0)
    b, r, c = _sample_positions(w.batch, w.M, w.N, 4096, 17)
    idx = torch.from_numpy(np.stack([b, r, c])).to(DEV)
    vals = C3[idx[0], idx[1], idx[2]]
    return finite, vals, (b, r, c)


FULL = ["f16_4096", "bf16_4096x4096x16384", "f16_batched_64x4096x4096x256", "f16_skinny_64x8192x8192"]


@pytest.mark.parametrize("which", ["first", "last"])
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name, which):
    """The benchmark's first and last rotating input set at full size."""
    w = inputs.WORKLOADS[name]
    j = 0 if which == "first" else w.rotating - 1
    say(f"[full] {name} set {j}")
    A, B = w.make_a(j), w.make_b(j)
    assert pkg.select_variant(w.dtype, w.batch, w.M, w.N, w.K, w.K, w.N, w.out_fp32) != \
        pkg.variants()["generic_64x64x16"]
    finite, vals, (b, r, c) = _full_size(w, A, B)
    assert finite, "non-finite values in the output"
    ref = oracle.gemm_at(inputs.bits(A), inputs.bits(B), b, r, c, w.dtype)
    m = oracle.compare(vals.float().cpu().numpy(), ref, w.K)
    say(f"[full] {name} set {j} rel_rms={m['rel_rms']:.3e} max_abs={m['max_abs']:.3e}")
    assert m["ok"], m


@pytest.mark.parametrize("name", FULL)
def test_full_size_exact_integers(name):
    """Integer inputs in [-2, 2] at the full shape: sampled outputs must match
    the oracle bit for bit (|C| <= 4K stays inside fp16 for K <= 8192)."""
    w = inputs.WORKLOADS[name]
    say(f"[full-exact] {name}")
    A = inputs.small_integers(w.a_shape(), 8001, dtype=w.dtype)
    B = inputs.small_integers(w.b_shape(), 8002, dtype=w.dtype)
    finite, vals, (b, r, c) = _full_size(w, A, B)
    assert finite
    ref = oracle.gemm_at(inputs.bits(A), inputs.bits(B), b, r, c, w.dtype)
    got = vals.cpu()
    if w.out_fp32:
        assert np.array_equal(got.numpy(), ref)
    else:
        assert np.array_equal(as_bits(got), oracle.encode(ref, w.dtype))


@pytest.mark.parametrize("name,kind", [("f16_skinny_64x8192x8192", "random"), ("f16_skinny_64x8192x8192", "exact"),
                                       ("f16_4096", "random"), ("f16_4096", "exact")])
def test_full_size_whole_output(name, kind):
    """Every output of a full-size workload against the oracle's whole
    product, where the oracle finishes in seconds to half a minute on the
    host: the skinny workload (last rotating set) and one 4096^3 set.
    Random inputs: the tolerance; integer inputs in [-2, 2]: bitwise (fp16
    RNE encoding of the exact sums)."""
    w = inputs.WORKLOADS[name]
    j = w.rotating - 1
    say(f"[whole] {name} set {j} {kind}")
    if kind == "random":
        A, B = w.make_a(j), w.make_b(j)
    else:
        A = inputs.small_integers(w.a_shape(), 8101, dtype=w.dtype)
        B = inputs.small_integers(w.b_shape(), 8102, dtype=w.dtype)
    got = pkg.gemm_f16(A.to(DEV), B.to(DEV), out_fp32=w.out_fp32)
    torch.cuda.synchronize()
    got = got.cpu()
    ref = oracle.gemm(inputs.bits(A), inputs.bits(B), w.dtype)
    if kind == "random":
        m = oracle.compare(got.float().numpy(), ref, w.K)
        say(f"[whole] {name} rel_rms={m['rel_rms']:.3e} max_abs={m['max_abs']:.3e} nonfinite={m['nonfinite']}")
        assert m["ok"], m
    else:
        assert np.array_equal(as_bits(got), oracle.encode(ref, w.dtype))


# The pipelined variants differ only in ring depth, K-tile width, tile size,
# whether A is staged in pairs and the layout B arrives in.  Each output is
# still the same sequence of 32x32x16 MFMAs over ascending 16-wide k-steps,
# so on the same random inputs they must agree bit for bit: a race (a stage
# read before it was published, or overwritten while still read) would show
# as a difference between schedules.
SCHED_FAMILY = ["pipelined_256x256x64_s2", "pipelined_128x128x64_s2", "pipelined_256x256x32_s4",
                "pipelined_256x256x32_s5", "pipelined_128x128x32_s4", "pipelined_256x256x32_s4_apair"]
SCHED_FAMILY_BT = ["pipelined_bt_256x256x32_s4", "pipelined_bt_128x128x32_s4", "pipelined_bt_256x256x64_s2",
                   "pipelined_bt_256x256x32_s4_apair"]


@pytest.mark.parametrize("M,N,K", [(512, 512, 512), (640, 768, 1024), (4096, 4096, 4096)])
@pytest.mark.parametrize("out_fp32", [False, True])
def test_schedules_give_bitwise_identical_results(M, N, K, out_fp32):
    say(f"[schedules] M={M} N={N} K={K} out_fp32={out_fp32}")
    A = inputs.uniform((M, K), 8401 + K, nonzero=True).to(DEV)
    B = inputs.uniform((K, N), 8402 + K, nonzero=True).to(DEV)
    Bt = B.t().contiguous()
    V = pkg.variants()
    outs = {}
    for vname in SCHED_FAMILY:
        outs[vname] = pkg.gemm_ex(A, B, out_fp32=out_fp32, variant=V[vname])
    for vname in SCHED_FAMILY_BT:
        outs[vname] = pkg.gemm_ex_bt(A, Bt, out_fp32=out_fp32, variant=V[vname])
    torch.cuda.synchronize()
    view = torch.int32 if out_fp32 else torch.int16
    ref_name = "pipelined_256x256x32_s4"
    ref = outs[ref_name].cpu().view(view)
    for vname, C in outs.items():
        diff = (C.cpu().view(view) != ref).sum().item()
        assert diff == 0, f"{vname} differs from {ref_name} in {diff} outputs"
    m = oracle.compare(outs[ref_name].float().cpu().numpy()[:64], oracle.gemm(
        inputs.bits(A[:64].cpu()), inputs.bits(B.cpu()), "f16"), K)
    assert m["ok"], m


def test_persistent_schedule_matches_the_pipelined_kernel_bitwise():
    """The persistent short-K kernel (a ring running across tiles, C of a
    tile stored during the next) against the pipelined kernel on the same
    batched inputs: bitwise identical."""
    V = pkg.variants()
    batch, M, N, K = 32, 512, 512, 256
    A = inputs.uniform((batch, M, K), 8501, nonzero=True).to(DEV)
    B = inputs.uniform((batch, K, N), 8502, nonzero=True).to(DEV)
    p = pkg.gemm_ex(A, B, variant=V["persistent_256x128x32_shortk"])
    pa = pkg.gemm_ex(A, B, variant=V["persistent_256x128x32_shortk_apair"])
    q = pkg.gemm_ex(A, B, variant=V["pipelined_256x256x32_s4"])
    r = pkg.gemm_ex(A, B, variant=V["pipelined_128x128x32_s4"])
    torch.cuda.synchronize()
    assert torch.equal(p.cpu().view(torch.int16), q.cpu().view(torch.int16))
    assert torch.equal(p.cpu().view(torch.int16), r.cpu().view(torch.int16))
    assert torch.equal(pa.cpu().view(torch.int16), q.cpu().view(torch.int16))


@pytest.mark.parametrize("K", [256, 128])
def test_resident_panel_kernel_over_several_groups(K):
    """The A-resident persistent kernel where each workgroup walks two row
    blocks' groups of 4 column tiles (16 x 2048 x 2048: 8 row blocks, the
    16 column tiles split in 4 ranges, 512 groups on 256 workgroups), so the
    panel is reloaded mid-walk: bitwise equal to the A-pair persistent
    kernel (same products in the same order), sampled outputs within the
    oracle's bound, and integer inputs exact everywhere sampled."""
    V = pkg.variants()
    b, M, N = 16, 2048, 2048
    say(f"[persistent groups] b={b} M={M} N={N} K={K}")
    A = inputs.uniform((b, M, K), 8601 + K, nonzero=True)
    B = inputs.uniform((b, K, N), 8602 + K, nonzero=True)
    Ad, Bd = A.to(DEV), B.to(DEV)
    r = pkg.gemm_ex(Ad, Bd, variant=V["persistent_256x128x32_shortk_aresident"])
    q = pkg.gemm_ex(Ad, Bd, variant=V["persistent_256x128x32_shortk_apair"])
    torch.cuda.synchronize()
    assert torch.equal(r.view(torch.int16), q.view(torch.int16))
    for e in (0, 7, 15):
        got, ref = _sampled_block(A[e], B[e], r[e], 8603 + e)
        m = oracle.compare(got.float().numpy(), ref, K)
        assert m["ok"], (e, m)
    Ai = inputs.small_integers((b, M, K), 8611)
    Bi = inputs.small_integers((b, K, N), 8612)
    ri = pkg.gemm_ex(Ai.to(DEV), Bi.to(DEV), variant=V["persistent_256x128x32_shortk_aresident"])
    torch.cuda.synchronize()
    for e in (0, 9):
        got, ref = _sampled_block(Ai[e], Bi[e], ri[e], 8613 + e)
        assert np.array_equal(as_bits(got), oracle.encode(ref, "f16")), e


@pytest.mark.parametrize("M,N,K", [(128, 4096, 4096), (96, 8192, 2048), (65, 1000, 1024), (64, 512, 65536),
                                   (64, 256, 8192)])
def test_mid_rows_take_the_ring_kernel_exactly(M, N, K):
    """65 to 128 rows with few 128 x 128 tiles, or narrow outputs over long K:
    the automatic choice runs the shared-ring skinny kernel (two row blocks,
    the second ragged below 128 rows, for the former), split over K.
    Integer inputs: equal to the oracle bitwise."""
    say(f"[mid rows] M={M} N={N} K={K}")
    assert pkg.select_variant("f16", 1, M, N, K, K, N, True) == pkg.variants()["skinny_64x128_ring_k32_s4_splitk"]
    A = inputs.small_integers((M, K), 8301 + M)
    B = inputs.small_integers((K, N), 8302 + N)
    got = run(A, B, "f16", True)
    assert np.array_equal(got.numpy(), oracle.gemm(inputs.bits(A), inputs.bits(B), "f16"))


def _sampled_block(A, B, C, seed, n=16):
    """Rows and columns of C (random ones plus the first and last) and the
    oracle's fp32 values of that block, from the CPU operands A (M,K), B (K,N)."""
    M, N = C.shape
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.integers(0, M, n), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.integers(0, N, n), [0, N - 1]]))
    ref = oracle.gemm(inputs.bits(A[torch.from_numpy(rows)]), inputs.bits(B[:, torch.from_numpy(cols)]), "f16")
    got = C[torch.from_numpy(rows).to(DEV)][:, torch.from_numpy(cols).to(DEV)].cpu()
    return got, ref


def test_operand_over_2gib_runs_on_64bit_offsets():
    """B of 2^20 x 1024 fp16 spans 2 GiB, past the 32-bit byte offsets of the
    buffer descriptors: every fast variant must refuse the call and the
    automatic choice must take the guarded kernel, whose offsets are 64-bit.
    Integer inputs make the sampled outputs exact."""
    M, N, K = 96, 1024, 1 << 20
    say(f"[max-size] B extent {K * N * 2} bytes, M={M} N={N} K={K}")
    assert pkg.select_variant("f16", 1, M, N, K, K, N, True) == pkg.variants()["generic_64x64x16"]
    A = inputs.small_integers((M, K), 8101)
    B = inputs.small_integers((K, N), 8102)
    Ad, Bd = A.to(DEV), B.to(DEV)
    for vname in ("pipelined_256x256x32_s4_apair", "pipelined_256x256x32_s4", "skinny_64x128_ring_k32_s4_splitk",
                  "repack_pipelined"):
        with pytest.raises(pkg.GemmError) as e:
            pkg.gemm_ex(Ad, Bd, out_fp32=True, variant=pkg.variants()[vname])
        assert e.value.status == pkg.BPT_ERR_UNSUPPORTED, vname
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    pkg.gemm_ex(Ad, Bd, C, out_fp32=True)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any().item()
    got, ref = _sampled_block(A, B, C, 8103)
    assert np.array_equal(got.numpy(), ref)
    del Ad, Bd, C
    torch.cuda.empty_cache()


@pytest.mark.parametrize("out_fp32,vname", [(False, "persistent_128x256x32_shortk_roles"),
                                            (True, "pipelined_256x256x32_s4_apair")])
def test_single_output_over_2gib(out_fp32, vname):
    """One C of 32768 x 32768 (2 GiB in fp16, 4 GiB in fp32) from the fast
    kernels: their C addresses are 64-bit, so every element is written (C is
    filled with NaN first) and sampled outputs equal the oracle bit for bit
    (integer inputs, |C| <= 1024)."""
    M = N = 32768
    K = 256
    say(f"[max-size] C {M}x{N} out_fp32={out_fp32} ({vname})")
    assert pkg.select_variant("f16", 1, M, N, K, K, N, out_fp32) == pkg.variants()[vname]
    A = inputs.small_integers((M, K), 8201)
    B = inputs.small_integers((K, N), 8202)
    C = torch.full((M, N), float("nan"), dtype=torch.float32 if out_fp32 else torch.float16, device=DEV)
    pkg.gemm_ex(A.to(DEV), B.to(DEV), C, out_fp32=out_fp32)
    torch.cuda.synchronize()
    assert not torch.isnan(C).any().item()
    got, ref = _sampled_block(A, B, C, 8203)
    if out_fp32:
        assert np.array_equal(got.numpy(), ref)
    else:
        assert np.array_equal(as_bits(got), oracle.encode(ref, "f16"))
    del C
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# B given transposed (gemm_ex_bt): C = A * Bt^T, Bt N x K row-major.  The
# oracle takes B = Bt^T, transposed on the host (16-bit patterns, exact).
# ----------------------------------------------------------------------------

BT_VARIANTS = ["pipelined_bt_256x256x32_s4", "pipelined_bt_128x128x32_s4", "generic_bt_64x64x16",
               "pipelined_bt_256x256x64_s2", "pipelined_bt_256x256x32_s4_apair"]
# any N (rows of Bt past N read as zero): 201, 7 and 520 are not multiples
# of 8; K tails of 8 (136 = 4 x 32 + 8, 1032) as on the other layout
SHAPES_BT = [(256, 256, 256), (300, 201, 192), (33, 520, 136), (129, 136, 256), (512, 384, 1032), (1, 7, 128)]
SHAPES_BT_GENERIC_ONLY = [(5, 3, 1), (257, 65, 129), (100, 70, 50)]


def _bt_shapes(vname):
    if vname.startswith("generic"):
        return SHAPES_BT + SHAPES_BT_GENERIC_ONLY
    if "x64_s2" in vname:                 # 64-wide K-tiles, no tail stage: K % 64 == 0, K >= 128
        return [(M, N, K) for (M, N, K) in SHAPES_BT if K % 64 == 0] + [(200, 264, 1088)]
    if "apair" in vname:                  # A in K-tile pairs: K % 64 == 0, K >= 192, no tail
        return [(M, N, K) for (M, N, K) in SHAPES_BT if K % 64 == 0 and K >= 192] + [(200, 264, 1088), (257, 1000, 384)]
    return SHAPES_BT


def _bt_bits(Bt):
    """16-bit patterns of B = Bt^T for the oracle."""
    b = inputs.bits(Bt)
    return np.ascontiguousarray(np.swapaxes(b, -1, -2))


def run_bt(A, Bt, dtype="f16", out_fp32=False, variant=0):
    C = pkg.gemm_ex_bt(A.to(DEV), Bt.to(DEV), None, dtype=dtype, out_fp32=out_fp32, variant=variant)
    torch.cuda.synchronize()
    return C.cpu()


@pytest.mark.parametrize("vname", BT_VARIANTS)
@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("f16", True), ("bf16", True), ("bf16", False)])
def test_bt_parity_random(vname, dtype, out_fp32):
    v = pkg.variants()[vname]
    for i, (M, N, K) in enumerate(_bt_shapes(vname)):
        say(f"[bt random] {vname} {dtype} out_fp32={out_fp32} M={M} N={N} K={K}")
        A = inputs.uniform((M, K), 9000 + i, dtype=dtype, nonzero=True)
        Bt = inputs.uniform((N, K), 9100 + i, dtype=dtype, nonzero=True)
        got = run_bt(A, Bt, dtype, out_fp32, v)
        ref = oracle.gemm(inputs.bits(A), _bt_bits(Bt), dtype)
        m = oracle.compare(got.float().numpy(), ref, K)
        assert m["ok"], (M, N, K, m)


@pytest.mark.parametrize("vname", BT_VARIANTS)
@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("f16", True), ("bf16", True)])
def test_bt_parity_exact_integers(vname, dtype, out_fp32):
    v = pkg.variants()[vname]
    for i, (M, N, K) in enumerate(_bt_shapes(vname)):
        say(f"[bt exact] {vname} {dtype} out_fp32={out_fp32} M={M} N={N} K={K}")
        A = inputs.small_integers((M, K), 9200 + i, dtype=dtype)
        Bt = inputs.small_integers((N, K), 9300 + i, dtype=dtype)
        got = run_bt(A, Bt, dtype, out_fp32, v)
        ref = oracle.gemm(inputs.bits(A), _bt_bits(Bt), dtype)
        if out_fp32:
            assert np.array_equal(got.numpy(), ref), (M, N, K)
        else:
            assert np.array_equal(as_bits(got), oracle.encode(ref, dtype)), (M, N, K)


@pytest.mark.parametrize("vname", BT_VARIANTS)
def test_bt_batched_and_padded(vname):
    """Batched, and leading dimensions with NaN in every padding element
    (Bt's rows padded past K, C's rows past N)."""
    v = pkg.variants()[vname]
    b, M, N, K = 3, 160, 200, 192
    A = inputs.uniform((b, M, K), 9401, lo=-0.5, hi=0.5)
    Bt = inputs.uniform((b, N, K), 9402, lo=-0.5, hi=0.5)
    got = run_bt(A, Bt, "f16", False, v)
    m = oracle.compare(got.float().numpy(), oracle.gemm(inputs.bits(A), _bt_bits(Bt)), K)
    assert m["ok"], m
    A2 = inputs.uniform((M, K), 9403, nonzero=True)
    Bt2 = inputs.uniform((N, K), 9404, nonzero=True)
    Ap = torch.full((M, K + 8), float("nan"), dtype=torch.float16)
    Ap[:, :K] = A2
    Btp = torch.full((N, K + 16), float("nan"), dtype=torch.float16)
    Btp[:, :K] = Bt2
    Cp = torch.full((M, N + 8), 7.0, dtype=torch.float16, device=DEV)
    pkg.gemm_ex_bt(Ap.to(DEV)[:, :K], Btp.to(DEV)[:, :K], Cp[:, :N], variant=v)
    torch.cuda.synchronize()
    Cp = Cp.cpu()
    assert torch.all(Cp[:, N:] == 7.0)
    m = oracle.compare(Cp[:, :N].float().numpy(), oracle.gemm(inputs.bits(A2), _bt_bits(Bt2)), K)
    assert m["ok"], m


def test_bt_full_size_sampled_and_exact():
    """4096^3 with B given transposed (the automatic choice), sampled against
    the oracle: random inputs by tolerance, small integers bit for bit."""
    M = N = K = 4096
    assert pkg.select_variant("f16", 1, M, N, K, K, K, bt=True) == pkg.variants()["pipelined_bt_256x256x32_s4_apair"]
    b, r, c = _sample_positions(1, M, N, 2048, 29)
    for kind in ("random", "exact"):
        if kind == "random":
            A = inputs.uniform((M, K), 9501, nonzero=True)
            Bt = inputs.uniform((N, K), 9502, nonzero=True)
        else:
            A = inputs.small_integers((M, K), 9503)
            Bt = inputs.small_integers((N, K), 9504)
        say(f"[bt full] {kind}")
        C = pkg.gemm_ex_bt(A.to(DEV), Bt.to(DEV), out_fp32=(kind == "exact"))
        torch.cuda.synchronize()
        assert bool(torch.isfinite(C).all().item())
        got = C[torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV)].cpu()
        ref = oracle.gemm_at(inputs.bits(A), _bt_bits(Bt), b, r, c, "f16")
        if kind == "random":
            m = oracle.compare(got.float().numpy(), ref, K)
            assert m["ok"], m
        else:
            assert np.array_equal(got.numpy(), ref)
