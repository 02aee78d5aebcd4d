"""Pins for the oracle's backward (dQ, dK, dV): central finite differences of
L = sum(O * dO) through the (separately pinned) forward, a hand-worked 2x2
case, torch fp64 autograd through SDPA (a library routine), and identities
that hold for any inputs."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_2x2():
    # Q = K = I, V = [[1,2],[3,4]], scale 1, dO = [[1,0],[0,0]].
    # Row 0 weights (a, b) = (sigma(1), sigma(-1)); dP_0 = (1, 3);
    # D_0 = a + 3b; dS_0 = (-2ab, 2ab); row 1 has dO = 0 so it contributes 0.
    q = np.eye(2)[None]
    k = np.eye(2)[None]
    v = np.array([[1.0, 2.0], [3.0, 4.0]])[None]
    do = np.array([[1.0, 0.0], [0.0, 0.0]])[None]
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, 1.0)
    a = 1.0 / (1.0 + math.exp(-1.0))
    b = 1.0 - a
    g = 2 * a * b
    assert abs(g - 0.3932238665) < 1e-10
    np.testing.assert_allclose(dq[0], [[-g, g], [0, 0]], atol=1e-14)
    np.testing.assert_allclose(dk[0], [[-g, 0], [g, 0]], atol=1e-14)
    np.testing.assert_allclose(dv[0], [[a, 0], [b, 0]], atol=1e-14)


@pytest.mark.parametrize("nq,nk,d,dv", [(1, 1, 1, 1), (3, 5, 4, 2), (5, 3, 2, 4)])
def test_finite_differences(nq, nk, d, dv):
    q, k, v, do = _rand((1, nq, d), 1), _rand((1, nk, d), 2), _rand((1, nk, dv), 3), _rand((1, nq, dv), 4)
    scale = 0.7
    dq, dk, dvv = oracle.attention_bwd(q, k, v, do, scale)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_fwd(q_, k_, v_, scale, threads=1)
        return float((o * do).sum())

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dvv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"])
                        - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("bh,nq,nk,d,dv", [(2, 7, 5, 4, 3), (1, 33, 70, 16, 16), (3, 64, 64, 32, 32)])
def test_matches_torch_autograd_fp64(bh, nq, nk, d, dv):
    q, k, v, do = _rand((bh, nq, d), 5), _rand((bh, nk, d), 6), _rand((bh, nk, dv), 7), _rand((bh, nq, dv), 8)
    scale = 1 / math.sqrt(d)
    dq, dk, dvv = oracle.attention_bwd(q, k, v, do, scale)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dvv, tv.grad.numpy(), atol=1e-12)


def test_identities():
    bh, nq, nk, d = 2, 11, 9, 6
    q, k, v, do = _rand((bh, nq, d), 9), _rand((bh, nk, d), 10), _rand((bh, nk, d), 11), _rand((bh, nq, d), 12)
    scale = 0.45
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale)
    # each row of dS sums to zero, so the key gradients sum to zero
    np.testing.assert_allclose(dk.sum(1), 0.0, atol=1e-12)
    # each probability row sums to one, so the value gradients sum to sum(dO)
    np.testing.assert_allclose(dv.sum(1), do.sum(1), atol=1e-12)
    # both sides equal scale * sum_ij dS_ij (q_i . k_j)
    np.testing.assert_allclose((q * dq).sum((1, 2)), (k * dk).sum((1, 2)), atol=1e-12)
    # dO = 0 gives zero gradients
    z = oracle.attention_bwd(q, k, v, np.zeros_like(do), scale)
    for g in z:
        assert np.all(g == 0)
