"""Pins for the oracle's forward (O, LSE) against facts that do not come from
the oracle's own code: hand-worked values, a page's worked example, closed
forms, invariants, a second algorithm (the scalar online recurrence of the
vyre-libs page) and library routines (torch SDPA, scipy logsumexp).

A plausible slip in the oracle (a dropped scale, max or log term, a sign, a
swapped operand or index) fails at least one of these: the hand 2x2 case and
the library comparisons use unequal nq/nk/d/dv so a transposed operand or a
wrong stride cannot pass.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def test_hand_worked_2x2():
    # Q = K = I, V = [[1,2],[3,4]], scale 1: the scores are the identity, so
    # row 0 has weights (sigma(1), sigma(-1)) and row 1 the mirror image.
    q = np.eye(2)[None]
    k = np.eye(2)[None]
    v = np.array([[1.0, 2.0], [3.0, 4.0]])[None]
    o, lse = oracle.attention_fwd(q, k, v, 1.0)
    a = 1.0 / (1.0 + math.exp(-1.0))
    b = 1.0 - a
    want = np.array([[a * 1 + b * 3, a * 2 + b * 4], [b * 1 + a * 3, b * 2 + a * 4]])
    np.testing.assert_allclose(o[0], want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0], [[1.5378828427, 2.5378828427], [2.4621171573, 3.4621171573]],
                               atol=1e-10)
    np.testing.assert_allclose(lse[0], [math.log(1 + math.e)] * 2, atol=1e-14)
    np.testing.assert_allclose(lse[0], [1.3132616875] * 2, atol=1e-10)


def test_page_seq_len_one_example():
    g = json.load(open(os.path.join(GOLDEN, "seq_len_one.json")))
    d = g["head_dim"]
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    o, lse = oracle.attention_fwd(q, k, v, 1.0 / math.sqrt(d))
    np.testing.assert_array_equal(o[0, 0], g["expected_o"])
    assert abs(lse[0, 0] - g["expected_lse"]) < 1e-12


@pytest.mark.parametrize("bh,nq,nk,d,dv", [(1, 1, 1, 1, 1), (2, 3, 5, 4, 6), (3, 17, 9, 8, 3),
                                           (2, 64, 64, 32, 32), (1, 33, 130, 16, 64)])
def test_matches_torch_sdpa_fp64(bh, nq, nk, d, dv):
    q, k, v = _rand((bh, nq, d), 1), _rand((bh, nk, d), 2), _rand((bh, nk, dv), 3)
    scale = 0.37
    o, lse = oracle.attention_fwd(q, k, v, scale)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale)
    np.testing.assert_allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    want_lse = scipy.special.logsumexp(scale * np.einsum("bid,bjd->bij", q, k), axis=-1)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-12)


def test_identity_values_expose_probabilities():
    # With V = I (nk x nk) the output row is the probability row itself.
    bh, nq, nk, d = 2, 7, 11, 5
    q, k = _rand((bh, nq, d), 4), _rand((bh, nk, d), 5)
    v = np.broadcast_to(np.eye(nk), (bh, nk, nk)).copy()
    scale = 0.8
    p, lse = oracle.attention_fwd(q, k, v, scale)
    assert np.all(p >= 0) and np.all(p <= 1)
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-14)
    s = scale * np.einsum("bid,bjd->bij", q, k)
    np.testing.assert_allclose(p, np.exp(s - lse[..., None]), atol=1e-14)
    # the largest score gets the largest weight
    assert np.array_equal(p.argmax(-1), s.argmax(-1))


def test_invariants():
    bh, nq, nk, d = 2, 9, 13, 6
    q, k, v = _rand((bh, nq, d), 6), _rand((bh, nk, d), 7), _rand((bh, nk, d), 8)
    scale = 1 / math.sqrt(d)
    o, lse = oracle.attention_fwd(q, k, v, scale)
    # constant V rows -> O equals that row
    c = _rand((d,), 9)
    oc, _ = oracle.attention_fwd(q, k, np.broadcast_to(c, v.shape).copy(), scale)
    np.testing.assert_allclose(oc, np.broadcast_to(c, oc.shape), atol=1e-14)
    # Q = 0 -> uniform weights: O = mean of V, LSE = ln nk
    oz, lz = oracle.attention_fwd(np.zeros_like(q), k, v, scale)
    np.testing.assert_allclose(oz, np.broadcast_to(v.mean(1, keepdims=True), oz.shape), atol=1e-14)
    np.testing.assert_allclose(lz, math.log(nk), atol=1e-14)
    # adding a vector to every V row adds it to every O row
    os_, _ = oracle.attention_fwd(q, k, v + c, scale)
    np.testing.assert_allclose(os_, o + c, atol=1e-13)
    # adding a vector u to every K row leaves O unchanged, shifts LSE by scale q.u
    u = _rand((d,), 10)
    ok, lk = oracle.attention_fwd(q, k + u, v, scale)
    np.testing.assert_allclose(ok, o, atol=1e-13)
    np.testing.assert_allclose(lk, lse + scale * q @ u, atol=1e-12)
    # LSE bounds: max score <= LSE <= max score + ln nk
    smax = (scale * np.einsum("bid,bjd->bij", q, k)).max(-1)
    assert np.all(lse >= smax - 1e-13) and np.all(lse <= smax + math.log(nk) + 1e-13)
    # permuting the keys (with their values) changes nothing
    perm = np.random.default_rng(11).permutation(nk)
    op, lp = oracle.attention_fwd(q, k[:, perm], v[:, perm], scale)
    np.testing.assert_allclose(op, o, atol=1e-13)
    np.testing.assert_allclose(lp, lse, atol=1e-13)


def test_large_scores_do_not_overflow():
    # scores around +-1000: exp without the max shift would overflow
    q = np.array([[[30.0, -20.0]]])
    k = np.array([[[40.0, 10.0], [39.0, 10.0], [-40.0, 0.0]]])
    v = np.array([[[1.0], [2.0], [3.0]]])
    o, lse = oracle.attention_fwd(q, k, v, 1.0)
    s = np.array([1000.0, 970.0, -1200.0])
    w = np.exp(s - s.max())
    w /= w.sum()
    np.testing.assert_allclose(o[0, 0, 0], w @ [1.0, 2.0, 3.0], atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 1000.0 + math.log1p(math.exp(-30.0)), atol=1e-12)


def _online_recurrence(q, k, v, scale, tile):
    """The vyre-libs page's recurrence: one query row, keys taken in tiles of
    ``tile`` (tile 1 is the scalar key-by-key reference), running max m,
    running sum l and a rescaled accumulator; m starts at the most negative
    finite float as on that page."""
    nq, d = q.shape
    nk = k.shape[0]
    out = np.zeros((nq, v.shape[1]))
    lse = np.zeros(nq)
    for i in range(nq):
        m, l, acc = -np.finfo(np.float64).max, 0.0, np.zeros(v.shape[1])
        for t0 in range(0, nk, tile):
            scores = [scale * float(q[i] @ k[j]) for j in range(t0, min(t0 + tile, nk))]
            m_new = max(m, max(scores))
            rescale = math.exp(m - m_new)
            l *= rescale
            acc *= rescale
            for jj, s in enumerate(scores):
                p = math.exp(s - m_new)
                l += p
                acc += p * v[t0 + jj]
            m = m_new
        out[i] = acc / l
        lse[i] = m + math.log(l)
    return out, lse


@pytest.mark.parametrize("seq,hd,tile", [(8, 16, 4), (1, 4, 1), (4, 8, 4), (5, 8, 4), (8, 16, 1)])
def test_agrees_with_online_recurrence(seq, hd, tile):
    # the vyre-libs tests' shapes: seq 8 / hd 16 / tile 4, seq 1, seq == tile, seq == tile + 1
    q, k, v = _rand((seq, hd), 12), _rand((seq, hd), 13), _rand((seq, hd), 14)
    scale = 1 / math.sqrt(hd)
    o, lse = oracle.attention_fwd(q[None], k[None], v[None], scale)
    o2, l2 = _online_recurrence(q, k, v, scale, tile)
    np.testing.assert_allclose(o[0], o2, atol=1e-12)
    np.testing.assert_allclose(lse[0], l2, atol=1e-12)


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.attention_fwd(np.zeros((1, 2, 3)), np.zeros((1, 2, 4)), np.zeros((1, 2, 3)), 1.0)
