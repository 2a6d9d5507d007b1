"""Race detection with the LDS-poison build (libbpt_gemm_poison.so).

That build fills every LDS-DMA copy's destination with a pattern that is NaN
as fp16 and as bf16 right before issuing the copy ("Xe2 Nbarrier Pipelining",
Checklist for Adding Split Barriers: a stage may be read only after its copy
has landed and every wave's arrival, and refilled only after every wave is
done reading it).  A fragment read that is not ordered after the copy it
needs, or a copy issued while some wave still reads the stage's older
contents, then puts NaN into C.  Every kernel family that stages through LDS
runs here on the same inputs through both builds: the results must be finite
and bitwise equal to the normal build's (same instructions, same order of
products).  The guarded kernel stages nothing through LDS-DMA and is not run.
"""
from __future__ import annotations

import pytest
import torch

import barrier_pipelined_tiled_amd as pkg
from barrier_pipelined_tiled_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pkg.lib()
    with pkg.library(pkg.POISON_LIB_PATH):
        pass


def say(msg):
    print(msg, flush=True)


def both(fn):
    """fn() with the normal build, then with the poison build."""
    ref = fn()
    torch.cuda.synchronize()
    with pkg.library(pkg.POISON_LIB_PATH):
        got = fn()
        torch.cuda.synchronize()
    return ref, got


def same_and_finite(ref, got):
    assert torch.isfinite(got.float()).all(), f"{(~torch.isfinite(got.float())).sum().item()} non-finite outputs"
    view = torch.int32 if ref.dtype == torch.float32 else torch.int16
    diff = (ref.view(view) != got.view(view)).sum().item()
    assert diff == 0, f"{diff} outputs differ from the normal build"


PIPELINED = ["pipelined_256x256x64_s2", "pipelined_128x128x64_s2", "pipelined_256x256x32_s4",
             "pipelined_256x256x32_s5", "pipelined_128x128x32_s4", "pipelined_256x256x32_s4_apair"]
BT = ["pipelined_bt_256x256x32_s4", "pipelined_bt_128x128x32_s4", "pipelined_bt_256x256x64_s2",
      "pipelined_bt_256x256x32_s4_apair"]
# (variant, M, N, K): K tails, the three skinny kernels (one with 16 splits),
# the repack route and split-K
SINGLE = [("pipelined_128x128x32_s4", 384, 512, 1032), ("pipelined_256x256x32_s4", 300, 264, 200),
          ("skinny_64x32_w4_k64_s4", 64, 1024, 2048), ("skinny_64x128_w4_k32_s4_splitk", 64, 1024, 2048),
          ("skinny_64x128_ring_k32_s4_splitk", 64, 2048, 3072), ("skinny_64x128_ring_k32_s4_splitk", 64, 2048, 4096),
          ("skinny_64x128_ring_k32_s4_splitk", 37, 320, 2560), ("repack_pipelined", 300, 201, 256),
          ("splitk_pipelined", 256, 1024, 1024), ("splitk_pipelined", 300, 520, 2048)]
PERSIST = ["persistent_256x128x32_shortk", "persistent_256x128x32_shortk_apair",
           "persistent_256x128x32_shortk_aresident"]


@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("bf16", True)])
@pytest.mark.parametrize("vname", PIPELINED + BT)
def test_pipelined_family_poison(vname, dtype, out_fp32):
    M, N, K = 640, 768, 1024
    say(f"[poison] {vname} {M}x{N}x{K} {dtype} out_fp32={out_fp32}")
    A = inputs.uniform((M, K), 9101, dtype=dtype, nonzero=True).to(DEV)
    B = inputs.uniform((K, N), 9102, dtype=dtype, nonzero=True).to(DEV)
    v = pkg.variants()[vname]
    if vname in BT:
        Bt = B.t().contiguous()
        ref, got = both(lambda: pkg.gemm_ex_bt(A, Bt, dtype=dtype, out_fp32=out_fp32, variant=v))
    else:
        ref, got = both(lambda: pkg.gemm_ex(A, B, dtype=dtype, out_fp32=out_fp32, variant=v))
    same_and_finite(ref, got)


@pytest.mark.parametrize("vname,M,N,K", SINGLE)
def test_single_matrix_kernels_poison(vname, M, N, K):
    say(f"[poison] {vname} {M}x{N}x{K}")
    A = inputs.uniform((M, K), 9201 + K, nonzero=True).to(DEV)
    B = inputs.uniform((K, N), 9202 + K, nonzero=True).to(DEV)
    v = pkg.variants()[vname]
    ref, got = both(lambda: pkg.gemm_ex(A, B, variant=v))
    same_and_finite(ref, got)


# several tiles (and, for the A-resident kernel, several groups) per
# workgroup, so the ring runs across tile boundaries
@pytest.mark.parametrize("batch,M,N,K", [(6, 2048, 1024, 256), (6, 2048, 1024, 128), (5, 1280, 2048, 256),
                                         (16, 2048, 2048, 128), (16, 2048, 2048, 256)])
@pytest.mark.parametrize("vname", PERSIST)
def test_persistent_kernels_poison(vname, batch, M, N, K):
    say(f"[poison] {vname} {batch}x{M}x{N}x{K}")
    A = inputs.uniform((batch, M, K), 9301 + K, nonzero=True).to(DEV)
    B = inputs.uniform((batch, K, N), 9302 + K, nonzero=True).to(DEV)
    v = pkg.variants()[vname]
    ref, got = both(lambda: pkg.gemm_ex(A, B, variant=v))
    same_and_finite(ref, got)


# the wave-role kernel: copy waves fill the B ring and the A panel, store
# waves read the C slots; 320 row blocks (panels reloaded mid-walk), and one
# column tile per row block (a new panel every tile)
@pytest.mark.parametrize("batch,M,N,K", [(10, 4096, 512, 256), (9, 4096, 256, 128), (10, 4096, 512, 128)])
def test_roles_kernel_poison(batch, M, N, K):
    say(f"[poison] roles {batch}x{M}x{N}x{K}")
    A = inputs.uniform((batch, M, K), 9351 + K, nonzero=True).to(DEV)
    B = inputs.uniform((batch, K, N), 9352 + K, nonzero=True).to(DEV)
    v = pkg.variants()["persistent_128x256x32_shortk_roles"]
    ref, got = both(lambda: pkg.gemm_ex(A, B, variant=v))
    same_and_finite(ref, got)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("BH,Sq,Skv,D", [(2, 300, 257, 256), (2, 512, 4096, 256), (3, 256, 96, 128),
                                         (2, 512, 4000, 128), (1, 100, 31, 256)])
def test_attention_poison(BH, Sq, Skv, D, dtype):
    say(f"[poison] attention BH={BH} Sq={Sq} Skv={Skv} D={D} {dtype}")
    Q = inputs.uniform((BH, Sq, D), 9401 + Skv, dtype=dtype).to(DEV)
    K = inputs.uniform((BH, Skv, D), 9402 + Skv, dtype=dtype).to(DEV)
    V = inputs.uniform((BH, Skv, D), 9403 + Skv, dtype=dtype).to(DEV)
    ref, got = both(lambda: pkg.attention_fwd(Q, K, V, dtype=dtype))
    same_and_finite(ref, got)


# the benchmark workloads at full size, in the launch configuration the
# benchmark times (its automatic kernel choice), on its first input set
@pytest.mark.parametrize("name", ["f16_4096", "bf16_4096x4096x16384", "f16_batched_64x4096x4096x256",
                                  "f16_skinny_64x8192x8192"])
def test_full_size_workloads_poison(name):
    w = inputs.WORKLOADS[name]
    say(f"[poison] full size {name}")
    A = w.make_a(0).to(DEV)
    B = w.make_b(0).to(DEV)
    ref, got = both(lambda: pkg.gemm_ex(A, B, dtype=w.dtype, out_fp32=w.out_fp32))
    same_and_finite(ref, got)


@pytest.mark.parametrize("name", ["attn_f16_64x4096x4096x256", "attn_f16_64x4096x4096x128"])
def test_full_size_attention_poison(name):
    w = inputs.ATTENTION[name]
    say(f"[poison] full size {w.name}")
    q, k, v = w.make_q(0).to(DEV), w.make_k(0).to(DEV), w.make_v(0).to(DEV)
    ref, got = both(lambda: pkg.attention_fwd(q, k, v, scale=w.scale, dtype=w.dtype, out_fp32=w.out_fp32))
    same_and_finite(ref, got)
