"""Pins for the oracle's PSA rearrangements, block and block gradient: torch
view/permute (a different formulation of the same index maps, forward and
inverse), a tiny case readable by eye, the pack/merge consistency on the V
channels, the V-split trick checked against one attention with the full value
width, and the block gradient against torch fp64 autograd of the block written
with torch ops and against central finite differences."""
import numpy as np
import pytest
import torch

import oracle


def _qkv(b, nh, kd, h, w, dtype=torch.float16, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(b, nh * 4 * kd, h, w, generator=g).to(dtype)


def _bits(t):
    if isinstance(t, np.ndarray):
        return t.view(np.int16)
    return t.contiguous().view(torch.int16).numpy()


@pytest.mark.parametrize("b,nh,kd,h,w", [(1, 1, 1, 1, 2), (2, 3, 4, 5, 3), (16, 4, 32, 20, 20)])
def test_pack_matches_torch_permute(b, nh, kd, h, w):
    x = _qkv(b, nh, kd, h, w)
    got = oracle.psa_pack(x, nh, kd)
    want = x.view(b, nh, 4, kd, h * w).permute(2, 0, 1, 4, 3).reshape(4, b * nh, h * w, kd)
    assert np.array_equal(_bits(got), _bits(want))


def test_pack_tiny_by_eye():
    # one batch, one head, key_dim 1, two pixels: channels are (Q, K, V_lo, V_hi)
    x = torch.tensor([[[[1.0, 2.0]], [[3.0, 4.0]], [[5.0, 6.0]], [[7.0, 8.0]]]], dtype=torch.float16)
    got = oracle.psa_pack(x, 1, 1)
    want = torch.tensor([[[[1.0], [2.0]]], [[[3.0], [4.0]]], [[[5.0], [6.0]]], [[[7.0], [8.0]]]],
                        dtype=torch.float16)
    assert got.shape == (4, 1, 2, 1)
    assert np.array_equal(_bits(got), _bits(want))


@pytest.mark.parametrize("b,nh,kd,h,w", [(1, 1, 2, 1, 3), (2, 3, 4, 5, 3), (16, 4, 32, 20, 20)])
def test_merge_matches_torch_permute(b, nh, kd, h, w):
    g = torch.Generator().manual_seed(1)
    lo = torch.randn(b * nh, h * w, kd, generator=g).to(torch.bfloat16)
    hi = torch.randn(b * nh, h * w, kd, generator=g).to(torch.bfloat16)
    got = oracle.psa_merge(lo, hi, b, nh, kd, h, w)
    both = torch.stack([lo, hi], 0).view(2, b, nh, h * w, kd)  # [2, B, nh, N, kd]
    want = both.permute(1, 2, 0, 4, 3).reshape(b, nh * 2 * kd, h, w)
    assert np.array_equal(_bits(got), _bits(want))


def test_pack_then_merge_recovers_value_channels():
    b, nh, kd, h, w = 2, 3, 4, 3, 5
    x = _qkv(b, nh, kd, h, w, seed=3)
    packed = oracle.psa_pack(x, nh, kd)
    merged = oracle.psa_merge(packed[2], packed[3], b, nh, kd, h, w)
    xb = _bits(x).reshape(b, nh, 4 * kd, h, w)
    want = xb[:, :, 2 * kd:, :, :].reshape(b, nh * 2 * kd, h, w)
    assert np.array_equal(_bits(merged), want)


def test_split_trick_equals_full_value_width():
    b, nh, kd, h, w = 2, 2, 4, 3, 4
    x = _qkv(b, nh, kd, h, w, seed=4).double()
    out = oracle.psa_block(x, nh, kd)
    packed = oracle.psa_pack(x, nh, kd)
    v_full = np.concatenate([packed[2], packed[3]], axis=-1)  # dv = 2*kd
    o_full, _ = oracle.attention_fwd(packed[0], packed[1], v_full, 1 / np.sqrt(kd))
    ref = oracle.psa_merge(np.ascontiguousarray(o_full[..., :kd]), np.ascontiguousarray(o_full[..., kd:]),
                           b, nh, kd, h, w)
    np.testing.assert_allclose(out, ref, atol=1e-14)


def test_block_matches_torch_composite():
    b, nh, kd, h, w = 2, 2, 8, 4, 5
    x = _qkv(b, nh, kd, h, w, seed=5).double()
    out = oracle.psa_block(x, nh, kd)
    t = x.view(b, nh, 4, kd, h * w).transpose(-1, -2)  # [B, nh, 4, N, kd]
    qt, kt = t[:, :, 0], t[:, :, 1]
    vt = torch.cat([t[:, :, 2], t[:, :, 3]], dim=-1)    # [B, nh, N, 2kd]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=kd ** -0.5)
    want = o.transpose(-1, -2).reshape(b, nh * 2 * kd, h, w)
    np.testing.assert_allclose(out, want.numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Backward: the inverse index maps and the block gradient


@pytest.mark.parametrize("b,nh,kd,h,w", [(1, 1, 2, 1, 3), (2, 3, 4, 5, 3), (16, 4, 32, 20, 20)])
def test_merge_backward_matches_torch_permute(b, nh, kd, h, w):
    g = torch.Generator().manual_seed(2)
    d_out = torch.randn(b, nh * 2 * kd, h, w, generator=g).to(torch.bfloat16)
    lo, hi = oracle.psa_merge_backward(d_out, nh, kd)
    want = d_out.view(b, nh, 2, kd, h * w).permute(2, 0, 1, 4, 3).reshape(2, b * nh, h * w, kd)
    assert np.array_equal(_bits(lo), _bits(want[0])) and np.array_equal(_bits(hi), _bits(want[1]))


@pytest.mark.parametrize("b,nh,kd,h,w", [(1, 1, 1, 1, 2), (2, 3, 4, 5, 3), (16, 4, 32, 20, 20)])
def test_pack_backward_matches_torch_permute(b, nh, kd, h, w):
    g = torch.Generator().manual_seed(3)
    d_packed = torch.randn(4, b * nh, h * w, kd, generator=g).to(torch.float16)
    got = oracle.psa_pack_backward(d_packed, b, nh, h, w)
    want = d_packed.view(4, b, nh, h * w, kd).permute(1, 2, 0, 4, 3).reshape(b, nh * 4 * kd, h, w)
    assert np.array_equal(_bits(got), _bits(want))


def test_backward_maps_invert_forward_maps():
    b, nh, kd, h, w = 2, 3, 4, 3, 5
    x = _qkv(b, nh, kd, h, w, seed=6)
    assert np.array_equal(_bits(oracle.psa_pack_backward(oracle.psa_pack(x, nh, kd), b, nh, h, w)), _bits(x))
    g = torch.Generator().manual_seed(7)
    lo = torch.randn(b * nh, h * w, kd, generator=g).to(torch.float16)
    hi = torch.randn(b * nh, h * w, kd, generator=g).to(torch.float16)
    lo2, hi2 = oracle.psa_merge_backward(oracle.psa_merge(lo, hi, b, nh, kd, h, w), nh, kd)
    assert np.array_equal(_bits(lo2), _bits(lo)) and np.array_equal(_bits(hi2), _bits(hi))


def _torch_block(x, nh, kd):
    """The block written with torch ops (pack by view/permute, softmax
    attention per value half, merge by permute), fp64."""
    b, _, h, w = x.shape
    t = x.view(b, nh, 4, kd, h * w).transpose(-1, -2)  # [B, nh, 4, N, kd]
    q, k, v_lo, v_hi = t[:, :, 0], t[:, :, 1], t[:, :, 2], t[:, :, 3]
    p = torch.softmax(q @ k.transpose(-1, -2).contiguous() * kd ** -0.5, dim=-1)
    o = torch.stack([p @ v_lo, p @ v_hi], dim=2)        # [B, nh, 2, N, kd]
    return o.transpose(-1, -2).reshape(b, nh * 2 * kd, h, w)


@pytest.mark.parametrize("b,nh,kd,h,w", [(1, 1, 2, 2, 3), (2, 2, 8, 4, 5), (1, 3, 4, 1, 7)])
def test_block_backward_matches_torch_autograd(b, nh, kd, h, w):
    x = _qkv(b, nh, kd, h, w, seed=8).double()
    g = torch.Generator().manual_seed(9)
    d_out = torch.randn(b, nh * 2 * kd, h, w, generator=g, dtype=torch.float64)
    got = oracle.psa_block_backward(x, nh, kd, d_out)
    xr = x.clone().requires_grad_(True)
    (_torch_block(xr, nh, kd) * d_out).sum().backward()
    np.testing.assert_allclose(got, xr.grad.numpy(), atol=1e-11)


def test_block_backward_finite_differences():
    b, nh, kd, h, w = 1, 2, 2, 2, 2
    x = _qkv(b, nh, kd, h, w, seed=10).double()
    g = torch.Generator().manual_seed(11)
    d_out = torch.randn(b, nh * 2 * kd, h, w, generator=g, dtype=torch.float64).numpy()
    grad = oracle.psa_block_backward(x, nh, kd, d_out)
    xn = x.numpy()
    eps = 1e-6
    for idx in [(0, 0, 0, 0), (0, 3, 1, 0), (0, 5, 0, 1), (0, 10, 1, 1), (0, 15, 0, 0)]:
        xp, xm = xn.copy(), xn.copy()
        xp[idx] += eps
        xm[idx] -= eps
        fd = ((oracle.psa_block(xp, nh, kd) * d_out).sum() - (oracle.psa_block(xm, nh, kd) * d_out).sum()) / (2 * eps)
        assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, grad[idx])


@pytest.mark.parametrize("b,nh,kd,h,w", [(1, 1, 1, 1, 2), (2, 3, 4, 5, 3), (16, 4, 32, 20, 20)])
def test_extract_v_matches_torch_narrow(b, nh, kd, h, w):
    x = _qkv(b, nh, kd, h, w, seed=12)
    got = oracle.psa_extract_v(x, nh, kd)
    want = x.view(b, nh, 4 * kd, h, w)[:, :, 2 * kd:].reshape(b, nh * 2 * kd, h, w)
    assert np.array_equal(_bits(got), _bits(want))


def test_extract_v_backward_matches_torch_autograd():
    b, nh, kd, h, w = 2, 3, 4, 3, 5
    x = _qkv(b, nh, kd, h, w, seed=13).double().requires_grad_(True)
    g = torch.Generator().manual_seed(14)
    d_v = torch.randn(b, nh * 2 * kd, h, w, generator=g, dtype=torch.float64)
    v = x.view(b, nh, 4 * kd, h, w)[:, :, 2 * kd:].reshape(b, nh * 2 * kd, h, w)
    (v * d_v).sum().backward()
    got = oracle.psa_extract_v_backward(d_v, nh, kd)
    assert np.array_equal(got, x.grad.numpy())


def test_extract_v_equals_merge_of_packed_v_sections():
    b, nh, kd, h, w = 2, 2, 4, 3, 3
    x = _qkv(b, nh, kd, h, w, seed=15)
    packed = oracle.psa_pack(x, nh, kd)
    merged = oracle.psa_merge(packed[2], packed[3], b, nh, kd, h, w)
    assert np.array_equal(_bits(oracle.psa_extract_v(x, nh, kd)), _bits(merged))
