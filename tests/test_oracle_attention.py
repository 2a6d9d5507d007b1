"""Pins of the attention oracle (oracle.attention, oracle.c
oracle_attention) against facts fixed by the mathematics of
O = softmax(scale * Q K^T) V, not against itself:

* closed forms: equal logits give the plain mean of the value rows; one key
  gives its value row; a key far ahead of the rest gives its value row (and
  an unshifted exp would overflow there);
* invariances: a constant added to every key of a row's logits, a joint
  permutation of keys and values, a power-of-two moved between Q and scale;
* a library routine: scipy.special.softmax followed by numpy's matmul in
  fp64, on shapes up to the head dimension 256 of the pages' SDP kernel;
* layout: sampled rows, strided views and batches equal the whole.
CPU only.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from barrier_pipelined_tiled_amd import inputs


def _bits(t):
    return inputs.bits(t)


def _f16(x):
    """16-bit patterns of an array of values exactly representable in fp16."""
    t = torch.tensor(np.asarray(x, dtype=np.float64), dtype=torch.float64).to(torch.float16)
    assert np.array_equal(t.double().numpy(), np.asarray(x, dtype=np.float64))
    return _bits(t)


def _library(q, k, v, scale, dtype="f16"):
    Q, K, V = (oracle.decode(x, dtype) for x in (q, k, v))
    logits = np.float64(np.float32(scale)) * (Q @ np.swapaxes(K, -1, -2))
    return scipy.special.softmax(logits, axis=-1) @ V


@pytest.mark.parametrize("BH,Sq,Skv,D,scale", [(1, 5, 7, 8, 0.35), (2, 33, 65, 64, 0.125),
                                               (3, 17, 100, 256, 1 / 16), (1, 4, 300, 256, 1.0),
                                               (2, 9, 31, 128, 2.0)])
def test_matches_library_softmax(BH, Sq, Skv, D, scale):
    q = _bits(inputs.uniform((BH, Sq, D), 11 + D, lo=-0.5, hi=0.5))
    k = _bits(inputs.uniform((BH, Skv, D), 12 + D, lo=-0.5, hi=0.5))
    v = _bits(inputs.uniform((BH, Skv, D), 13 + D))
    _, o64 = oracle.attention(q, k, v, scale, want64=True)
    ref = _library(q, k, v, scale)
    assert np.max(np.abs(o64 - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_bf16_matches_library_softmax():
    q = _bits(inputs.uniform((2, 20, 64), 21, dtype="bf16"))
    k = _bits(inputs.uniform((2, 50, 64), 22, dtype="bf16"))
    v = _bits(inputs.uniform((2, 50, 64), 23, dtype="bf16"))
    _, o64 = oracle.attention(q, k, v, 0.125, dtype="bf16", want64=True)
    ref = _library(q, k, v, 0.125, "bf16")
    assert np.max(np.abs(o64 - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_equal_logits_give_the_mean_of_the_values_exactly():
    """Q = 0: every logit is 0, every weight exp(0) = 1, so O is the mean of
    the value rows.  Integer values over a power-of-two key count make the
    mean exact in fp64 and fp32."""
    Skv, D = 64, 16
    q = _f16(np.zeros((3, D)))
    k = _bits(inputs.uniform((Skv, D), 31))
    vi = inputs.small_integers((Skv, D), 32, -7, 7)
    o32, o64 = oracle.attention(q, k, _bits(vi), 0.5, want64=True)
    mean = vi.double().numpy().sum(axis=0) / Skv
    assert np.array_equal(o64, np.broadcast_to(mean, o64.shape))
    assert np.array_equal(o32, np.broadcast_to(mean.astype(np.float32), o32.shape))


def test_identical_keys_give_the_mean_whatever_the_queries():
    Skv, D = 40, 32
    krow = inputs.uniform((1, D), 41)
    k = _bits(krow.expand(Skv, D).contiguous())
    v = _bits(inputs.uniform((Skv, D), 42))
    q = _bits(inputs.uniform((6, D), 43))
    _, o64 = oracle.attention(q, k, v, 0.7, want64=True)
    V = oracle.decode(v)
    mean = np.array([math.fsum(V[:, d]) for d in range(D)]) / Skv
    assert np.max(np.abs(o64 - mean)) <= 4e-16 * Skv


def test_one_key_returns_its_value_row():
    q = _bits(inputs.uniform((2, 9, 24), 51))
    k = _bits(inputs.uniform((2, 1, 24), 52))
    v = _bits(inputs.uniform((2, 1, 24), 53))
    o32, o64 = oracle.attention(q, k, v, 3.0, want64=True)
    V = oracle.decode(v)
    assert np.array_equal(o64, np.broadcast_to(V, o64.shape))


def test_dominant_key_returns_its_value_row_without_overflow():
    """Logit 1024 for one key, 0 for the rest: exp(1024) overflows fp64, so
    only a max-shifted softmax survives; the others' weights underflow to 0
    and O is that key's value row exactly."""
    Skv, D, hit = 50, 8, 17
    qv = np.zeros((1, D)); qv[0, 3] = 32.0
    kv = np.zeros((Skv, D)); kv[hit, 3] = 32.0
    v = _bits(inputs.uniform((Skv, D), 61))
    o32, o64 = oracle.attention(_f16(qv), _f16(kv), v, 1.0, want64=True)
    assert np.all(np.isfinite(o64))
    assert np.array_equal(o64[0], oracle.decode(v)[hit])


def test_constant_logit_shift_changes_nothing():
    """Adding the same row c to every key adds Q.c to every logit of a query
    row: softmax is unchanged.  Small integers keep K + c exact in fp16."""
    Skv, D = 30, 16
    ki = inputs.small_integers((Skv, D), 71)
    c = inputs.small_integers((1, D), 72, -3, 3)
    q = _bits(inputs.uniform((5, D), 73, lo=-0.25, hi=0.25))
    v = _bits(inputs.uniform((Skv, D), 74))
    _, a = oracle.attention(q, _bits(ki), v, 0.5, want64=True)
    _, b = oracle.attention(q, _bits((ki + c).to(torch.float16)), v, 0.5, want64=True)
    assert np.max(np.abs(a - b)) <= 1e-13 * np.max(np.abs(a))


def test_joint_permutation_of_keys_and_values_changes_nothing():
    Skv, D = 45, 32
    q = _bits(inputs.uniform((4, D), 81))
    k = _bits(inputs.uniform((Skv, D), 82))
    v = _bits(inputs.uniform((Skv, D), 83))
    perm = np.random.default_rng(84).permutation(Skv)
    _, a = oracle.attention(q, k, v, 0.3, want64=True)
    _, b = oracle.attention(q, np.ascontiguousarray(k[perm]), np.ascontiguousarray(v[perm]), 0.3, want64=True)
    assert np.max(np.abs(a - b)) <= 1e-14 * np.max(np.abs(a))


def test_power_of_two_moves_between_queries_and_scale_bitwise():
    """(2Q) . k times scale/2 is Q . k times scale exactly (power-of-two
    factors commute with rounding), so the logits and everything after
    them are bit-identical."""
    D = 64
    qt = inputs.uniform((7, D), 91, lo=-0.5, hi=0.5)
    k = _bits(inputs.uniform((33, D), 92))
    v = _bits(inputs.uniform((33, D), 93))
    _, a = oracle.attention(_bits(qt), k, v, 0.25, want64=True)
    _, b = oracle.attention(_bits(qt * 2), k, v, 0.125, want64=True)
    assert np.array_equal(a, b)


def test_sampled_rows_strided_views_and_batches_equal_the_whole():
    BH, Sq, Skv, D = 3, 20, 37, 32
    qf = _bits(inputs.uniform((BH, Sq, D + 8), 101))
    kf = _bits(inputs.uniform((BH, Skv, D + 16), 102))
    vf = _bits(inputs.uniform((BH, Skv, D + 24), 103))
    q, k, v = qf[:, :, :D], kf[:, :, 4:D + 4], vf[:, :, 8:D + 8]           # ld > D
    whole = oracle.attention(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v), 0.2)
    assert np.array_equal(oracle.attention(q, k, v, 0.2), whole)
    bi, ri = np.array([2, 0, 1, 2]), np.array([19, 0, 7, 3])
    assert np.array_equal(oracle.attention(q, k, v, 0.2, rows=(bi, ri)), whole[bi, ri])
    for b in range(BH):
        assert np.array_equal(oracle.attention(q[b], k[b], v[b], 0.2), whole[b])


def test_no_keys_give_zeros():
    q = _bits(inputs.uniform((2, 4, 8), 111))
    k = np.zeros((2, 0, 8), dtype=np.uint16)
    v = np.zeros((2, 0, 8), dtype=np.uint16)
    assert np.array_equal(oracle.attention(q, k, v, 1.0), np.zeros((2, 4, 8), np.float32))


def test_attention_metrics():
    r = np.linspace(-1.0, 1.0, 64).reshape(8, 8)
    m = oracle.compare_attention(r * (1 + 1e-3), r)
    assert m["ok"] and abs(m["rel_rms"] - 1e-3) < 1e-9
    g = r.copy(); g[3, 3] += 0.011
    assert not oracle.compare_attention(g, r)["ok"]                     # over 1e-2 * max|R|
    g = r.copy(); g[0, 0] = np.nan
    assert oracle.compare_attention(g, r)["nonfinite"] == 1 and not oracle.compare_attention(g, r)["ok"]
    z = np.zeros((4, 4))
    assert oracle.compare_attention(z, z)["ok"] and not oracle.compare_attention(z + 1e-30, z)["ok"]
