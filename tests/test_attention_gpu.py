"""GPU parity of the fused attention kernel (attention_fwd) against the
oracle's plain fp64 softmax(scale Q K^T) V, through the C ABI.

Random inputs are judged by oracle.compare_attention (rel_rms <= 5e-3 and
max|err| <= 1e-2 max|O_ref|).  Inputs whose weights are exact -- all logits
equal, or one key ahead of the rest by more than the fp32 range of exp2 --
must give the oracle's value rounded once, bit for bit.
"""
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


def _dt(dtype):
    return torch.float16 if dtype == "f16" else torch.bfloat16


def run_attention(q, k, v, scale, dtype="f16", out_fp32=False):
    O = pkg.attention_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, dtype=dtype, out_fp32=out_fp32)
    torch.cuda.synchronize()
    return O.cpu()


def check_random(q, k, v, scale, dtype, out_fp32):
    got = run_attention(q, k, v, scale, dtype, out_fp32)
    ref = oracle.attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), scale, dtype)
    m = oracle.compare_attention(got.float().numpy(), ref)
    assert m["ok"], m
    return m


# (BH, Sq, Skv, D): whole and ragged query tiles (256 rows) and key blocks
# (32 keys at D = 256, 64 at D = 128), one query or key, exactly one whole
# key block (the second half of the waves runs only its first, peeled
# block), several key blocks with a ragged tail
SHAPES = [(1, 128, 64, 256), (2, 300, 200, 256), (1, 1, 1, 256), (3, 129, 1000, 128), (2, 257, 63, 128),
          (1, 64, 4096, 256), (4, 128, 130, 256), (2, 256, 32, 256), (1, 300, 64, 128)]


@pytest.mark.parametrize("BH,Sq,Skv,D", SHAPES)
@pytest.mark.parametrize("dtype,out_fp32", [("f16", False), ("f16", True), ("bf16", False), ("bf16", True)])
def test_parity_random(BH, Sq, Skv, D, dtype, out_fp32):
    say(f"attention BH={BH} Sq={Sq} Skv={Skv} D={D} {dtype} out_fp32={out_fp32}")
    seed = 1000 + BH * 7 + Sq + Skv + D
    q = inputs.uniform((BH, Sq, D), seed, lo=-0.5, hi=0.5, dtype=dtype)
    k = inputs.uniform((BH, Skv, D), seed + 1, lo=-0.5, hi=0.5, dtype=dtype)
    v = inputs.uniform((BH, Skv, D), seed + 2, dtype=dtype)
    check_random(q, k, v, 1.0 / D ** 0.5, dtype, out_fp32)


@pytest.mark.parametrize("scale", [1.0, 4.0])
def test_parity_sharp_logits(scale):
    """Logits of tens: the running maximum moves by more than 2^8 between
    key blocks, so the lazy rescale of O and of the row sums runs."""
    say(f"attention sharp logits scale={scale}")
    BH, Sq, Skv, D = 2, 200, 700, 256
    q = inputs.uniform((BH, Sq, D), 2001)
    k = inputs.uniform((BH, Skv, D), 2002)
    v = inputs.uniform((BH, Skv, D), 2003)
    check_random(q, k, v, scale, "f16", True)


@pytest.mark.parametrize("D,Skv", [(256, 300), (128, 1024)])
def test_parity_negative_scale(D, Skv):
    """A negative scale turns the row maximum of the logits into the minimum
    of the raw products (its own code path); ragged Skv masks the tail."""
    say(f"attention negative scale D={D} Skv={Skv}")
    q = inputs.uniform((2, 150, D), 2051, lo=-0.5, hi=0.5)
    k = inputs.uniform((2, Skv, D), 2052, lo=-0.5, hi=0.5)
    v = inputs.uniform((2, Skv, D), 2053)
    check_random(q, k, v, -0.75, "f16", True)


def test_zero_scale_exact():
    """scale 0: every logit is 0 whatever Q and K are, so O is the mean of
    the values, exactly for integers over a power-of-two key count."""
    say("attention zero scale")
    BH, Sq, Skv, D = 2, 70, 512, 256
    q = inputs.uniform((BH, Sq, D), 2061)
    k = inputs.uniform((BH, Skv, D), 2062)
    v = inputs.small_integers((BH, Skv, D), 2063, -3, 3)
    ref = oracle.attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), 0.0)
    got = run_attention(q, k, v, 0.0, "f16", True)
    assert np.array_equal(got.numpy(), ref)


@pytest.mark.parametrize("D,Skv", [(256, 16), (128, 8)])
def test_zero_scale_ragged_exact(D, Skv):
    """scale 0 with fewer keys than one key block: the masked keys must get
    weight 0 (not NaN), the rest weight 1, so O is the exact mean of the
    integer values over a power-of-two count."""
    say(f"attention zero scale ragged D={D} Skv={Skv}")
    q = inputs.uniform((2, 40, D), 2071)
    k = inputs.uniform((2, Skv, D), 2072)
    v = inputs.small_integers((2, Skv, D), 2073, -3, 3)
    ref = oracle.attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), 0.0)
    got = run_attention(q, k, v, 0.0, "f16", True)
    assert np.array_equal(got.numpy(), ref)


def test_zero_scale_ragged_tail():
    say("attention zero scale, ragged tail of several blocks")
    q = inputs.uniform((2, 70, 256), 2081)
    k = inputs.uniform((2, 300, 256), 2082)
    v = inputs.uniform((2, 300, 256), 2083)
    check_random(q, k, v, 0.0, "f16", True)


def test_rising_maximum_across_blocks():
    """Keys whose logits grow block by block (key j scaled by j/Skv): every
    block raises each row's maximum, many times over 2^8."""
    say("attention rising maximum")
    BH, Sq, Skv, D = 1, 128, 640, 128
    q = inputs.uniform((BH, Sq, D), 2101)
    ramp = (torch.arange(Skv, dtype=torch.float32) / Skv * 8.0).view(1, Skv, 1)
    k = (inputs.uniform((BH, Skv, D), 2102).float() * ramp).to(torch.float16)
    v = inputs.uniform((BH, Skv, D), 2103)
    check_random(q, k, v, 1.0, "f16", True)


@pytest.mark.parametrize("D", [128, 256])
def test_equal_logits_exact(D):
    """Q = 0: every weight is exp2(0) = 1, the row sum is Skv and O the mean
    of the values.  Integer values over a power-of-two key count make every
    step exact, so O equals the oracle bit for bit (fp32 and fp16 out)."""
    say(f"attention equal logits D={D}")
    BH, Sq, Skv = 2, 130, 1024
    q = torch.zeros((BH, Sq, D), dtype=torch.float16)
    k = inputs.uniform((BH, Skv, D), 2201)
    v = inputs.small_integers((BH, Skv, D), 2202, -3, 3)
    ref = oracle.attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), 0.5)
    got32 = run_attention(q, k, v, 0.5, "f16", True)
    assert np.array_equal(got32.numpy(), ref)
    got16 = run_attention(q, k, v, 0.5, "f16", False)
    assert np.array_equal(inputs.bits(got16), oracle.encode(ref, "f16"))


def test_dominant_key_exact():
    """Row i's query matches key i only, with a logit 512 above every other
    (2^-512 underflows fp32): the weights are exactly one-hot and O row i is
    value row i, bit for bit."""
    say("attention dominant key")
    Sq = Skv = 192
    D = 256
    qv = torch.zeros((1, Sq, D))
    kv = torch.zeros((1, Skv, D))
    for i in range(Sq):
        qv[0, i, i % D] = 16.0
        kv[0, i, i % D] = 32.0
    q, k = qv.to(torch.float16), kv.to(torch.float16)
    v = inputs.uniform((1, Skv, D), 2301)
    got = run_attention(q, k, v, 1.0, "f16", False)
    assert torch.equal(got, v)


def test_no_keys_and_empty_calls():
    q = inputs.uniform((2, 100, 128), 2401).to(DEV)
    k = torch.empty((2, 0, 128), dtype=torch.float16, device=DEV)
    v = torch.empty((2, 0, 128), dtype=torch.float16, device=DEV)
    O = torch.full((2, 100, 128), 7.0, dtype=torch.float16, device=DEV)
    pkg.attention_fwd(q, k, v, O)
    torch.cuda.synchronize()
    assert torch.count_nonzero(O).item() == 0
    qe = torch.empty((0, 5, 128), dtype=torch.float16, device=DEV)
    pkg.attention_fwd(qe, qe, qe)                                  # nothing to do
    torch.cuda.synchronize()


def test_strided_views_and_batch_strides():
    """Q, K, V and O as column slices of wider rows (ld > D) with padded batch
    strides; the padding of O must be left alone."""
    say("attention strided views")
    BH, Sq, Skv, D = 3, 150, 333, 128
    qf = inputs.uniform((BH, Sq + 8, D + 64), 2501).to(DEV)
    kf = inputs.uniform((BH, Skv, D + 16), 2502).to(DEV)
    vf = inputs.uniform((BH, Skv + 40, D + 8), 2503).to(DEV)
    q, k, v = qf[:, 3:3 + Sq, 32:32 + D], kf[:, :, 8:8 + D], vf[:, 40:, :D]
    Of = torch.full((BH, Sq, D + 24), float("nan"), dtype=torch.float32, device=DEV)
    O = Of[:, :, 8:8 + D]
    pkg.attention_fwd(q, k, v, O, scale=0.2, out_fp32=True)
    torch.cuda.synchronize()
    ref = oracle.attention(inputs.bits(q.cpu()), inputs.bits(k.cpu()), inputs.bits(v.cpu()), 0.2)
    m = oracle.compare_attention(O.cpu().numpy(), ref)
    assert m["ok"], m
    assert torch.isnan(Of[:, :, :8]).all() and torch.isnan(Of[:, :, 8 + D:]).all()


def test_repeat_runs_bitwise_identical():
    w = inputs.ATTENTION["attn_f16_2x512x512x256"]
    q, k, v = (x.to(DEV) for x in (w.make_q(), w.make_k(), w.make_v()))
    outs = [pkg.attention_fwd(q, k, v, scale=w.scale).cpu() for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])


def test_small_workload_whole():
    w = inputs.ATTENTION["attn_f16_2x512x512x256"]
    for j in range(w.rotating):
        say(f"attention workload {w.name} set {j}")
        check_random(w.make_q(j), w.make_k(j), w.make_v(j), w.scale, w.dtype, w.out_fp32)


def test_key_extent_near_2gib():
    """Two heads of 4,194,000 keys at D = 256.  Each head's K and V, plus
    the block of rows a ragged tail may read past the end, span just under
    2^31 bytes, the most the 32-bit buffer offsets take (4,194,240 keys are
    refused).  The second head starts more than 2^31 bytes past the base,
    and the last block holds 16 keys.  Sampled rows against the oracle."""
    BH, Sq, Skv, D = 2, 64, 4194000, 256
    assert (Skv + 64) * D * 2 < 2**31 - 1 and (4194240 + 64) * D * 2 > 2**31 - 1
    say(f"attention BH={BH} Sq={Sq} Skv={Skv} D={D} (K, V {BH * Skv * D * 2} bytes each)")
    q = inputs.uniform((BH, Sq, D), 2701, lo=-0.5, hi=0.5)
    k = inputs.uniform((BH, Skv, D), 2702, lo=-0.5, hi=0.5)
    v = inputs.uniform((BH, Skv, D), 2703)
    scale = 1.0 / 16
    got = run_attention(q, k, v, scale, "f16", True)
    assert torch.isfinite(got).all()
    bi = np.array([0, 0, 1, 1], dtype=np.int64)
    ri = np.array([0, Sq - 1, 0, 37], dtype=np.int64)
    ref = oracle.attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), scale, "f16", rows=(bi, ri))
    m = oracle.compare_attention(got[bi, ri].numpy(), ref)
    assert m["ok"], m


def test_full_size_sampled():
    """The benchmark's shape (64 heads x 4096 queries x 4096 keys, D = 256):
    every output finite, and 64 sampled rows (each head's first or last row
    among them) against the oracle."""
    w = inputs.ATTENTION["attn_f16_64x4096x4096x256"]
    say(f"attention workload {w.name}")
    q, k, v = w.make_q(0), w.make_k(0), w.make_v(0)
    got = run_attention(q, k, v, w.scale, w.dtype, w.out_fp32)
    assert torch.isfinite(got.float()).all()
    rng = np.random.default_rng(2601)
    bi = np.concatenate([np.arange(w.BH), rng.integers(0, w.BH, 32)])[:64]
    ri = np.concatenate([np.where(np.arange(w.BH) % 2 == 0, 0, w.Sq - 1), rng.integers(0, w.Sq, 32)])[:64]
    ref = oracle.attention(inputs.bits(q), inputs.bits(k), inputs.bits(v), w.scale, w.dtype, rows=(bi, ri))
    m = oracle.compare_attention(got[bi, ri].float().numpy(), ref)
    assert m["ok"], m
