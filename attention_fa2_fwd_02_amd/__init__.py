"""MI355X-native exact attention (FlashAttention-2 style) and the PSA
pack/merge rearrangements, behind the C ABI of ``libfa2mi.so``
(``include/fa2mi.h``).

This module only marshals arguments: it checks tensors, allocates outputs with
torch on the inputs' device, and calls the C entry point of the same name with
raw device pointers and the current torch stream. Every step of the
computation runs in the HIP kernels; there is no fallback of any kind, and
every function raises if the library is missing or the tensors are not on a
GPU.

Entry points (same names as the C ABI):
  fa2_fwd, fa2_fwd_splitkv_plan, fa2_fwd_splitkv, fa2_fwd_splitkv_noalloc,
  fa2_fwd_splitkv_noalloc_max_bytes, fa2_pad_cols, fa2_bwd_delta,
  fa2_bwd_dq, fa2_bwd_dkdv, psa_pack_qkv, psa_merge_attn, psa_attn_fused,
  psa_attn_fused_backward, psa_merge_attn_backward, psa_pack_qkv_backward,
  psa_extract_v_nchw, psa_extract_v_backward
Compositions of them:
  attention_fwd (fa2_fwd, or fa2_fwd_splitkv when its plan splits the keys;
  other head dims up to 128 through zero padding with fa2_pad_cols),
  attention_bwd (delta -> dkdv -> dq, padded likewise),
  psa_block (pack -> fa2_fwd on V_lo -> fa2_fwd on V_hi -> merge),
  psa_block_backward (merge backward -> the attention backward of both calls
  -> pack backward, adding the two calls' dQ and dK)
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import FA2_BF16, FA2_F16, FA2_F32, Fa2Error, library_path, load  # noqa: F401

__all__ = [
    "fa2_fwd", "fa2_fwd_splitkv_plan", "fa2_fwd_splitkv", "fa2_fwd_splitkv_noalloc",
    "fa2_fwd_splitkv_noalloc_max_bytes", "fa2_pad_cols", "fa2_bwd_delta", "fa2_bwd_dq",
    "fa2_bwd_dkdv", "psa_pack_qkv", "psa_merge_attn", "psa_attn_fused", "psa_attn_fused_backward",
    "psa_merge_attn_backward", "psa_pack_qkv_backward", "psa_extract_v_nchw", "psa_extract_v_backward",
    "attention_fwd", "attention_bwd", "psa_block", "psa_block_backward", "Fa2Error", "load", "library_path",
]

_DT = {torch.float32: FA2_F32, torch.float16: FA2_F16, torch.bfloat16: FA2_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16") from None


def _check(name: str, t: torch.Tensor, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _scale(scale, head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim) if scale is None else float(scale)


def fa2_fwd(q, k, v, scale=None, o=None, lse=None):
    """Forward: returns (o [bh,n_q,d] in q's dtype, lse [bh,n_q] float32)."""
    _check("q", q)
    bh, n_q, d = q.shape
    n_k = k.shape[1]
    dev = q.device
    _check("k", k, q.dtype, (bh, n_k, d), dev)
    _check("v", v, q.dtype, (bh, n_k, d), dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((bh, n_q), dtype=torch.float32, device=dev)
    _check("o", o, q.dtype, q.shape, dev)
    _check("lse", lse, torch.float32, (bh, n_q), dev)
    _lib.call("fa2_fwd", _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
              lse.data_ptr(), bh, n_q, n_k, d, _scale(scale, d), _stream(dev))
    return o, lse


def fa2_fwd_splitkv_plan(dtype, bh, n_q, n_k, head_dim, num_splits=0):
    """(splits used, workspace bytes) of fa2_fwd_splitkv for these sizes.

    Host-only: needs the library but no GPU. num_splits 0 lets the library
    choose; a request is clamped to one range per 64 keys.
    """
    try:
        code = _DT[dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {dtype}; use float32, float16 or bfloat16") from None
    splits = ctypes.c_int32()
    nbytes = ctypes.c_int64()
    _lib.call("fa2_fwd_splitkv_plan", code, bh, n_q, n_k, head_dim, num_splits, ctypes.addressof(splits),
              ctypes.addressof(nbytes))
    return splits.value, nbytes.value


def fa2_fwd_splitkv(q, k, v, scale=None, num_splits=0, workspace=None, o=None, lse=None):
    """Key-split forward: the same (o, lse) as fa2_fwd, with each head's keys
    cut into ranges processed by separate workgroups and merged by their
    log-sum-exp. For few query rows per head (decoding). `workspace` is an
    optional uint8 GPU tensor of at least fa2_fwd_splitkv_plan's size
    (allocated here when omitted)."""
    _check("q", q)
    bh, n_q, d = q.shape
    n_k = k.shape[1]
    dev = q.device
    _check("k", k, q.dtype, (bh, n_k, d), dev)
    _check("v", v, q.dtype, (bh, n_k, d), dev)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((bh, n_q), dtype=torch.float32, device=dev)
    _check("o", o, q.dtype, q.shape, dev)
    _check("lse", lse, torch.float32, (bh, n_q), dev)
    _, need = fa2_fwd_splitkv_plan(q.dtype, bh, n_q, n_k, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check("workspace", workspace, torch.uint8, None, dev)
    _lib.call("fa2_fwd_splitkv", _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
              lse.data_ptr(), workspace.data_ptr(), workspace.numel(), bh, n_q, n_k, d, _scale(scale, d),
              num_splits, _stream(dev))
    return o, lse


def fa2_fwd_splitkv_noalloc_max_bytes() -> int:
    """Size in bytes of the static device scratch of fa2_fwd_splitkv_noalloc."""
    return int(load().fa2_fwd_splitkv_noalloc_max_bytes())


def fa2_fwd_splitkv_noalloc(q, k, v, o, lse, scale=None, num_splits=0):
    """Key-split forward into caller-provided o and lse with the library's
    static device scratch in place of a workspace (no device allocation in
    the call). Calls overlapping on one device share that scratch and race:
    keep them on one stream. Partials larger than the scratch raise Fa2Error."""
    _check("q", q)
    bh, n_q, d = q.shape
    n_k = k.shape[1]
    dev = q.device
    _check("k", k, q.dtype, (bh, n_k, d), dev)
    _check("v", v, q.dtype, (bh, n_k, d), dev)
    _check("o", o, q.dtype, q.shape, dev)
    _check("lse", lse, torch.float32, (bh, n_q), dev)
    _lib.call("fa2_fwd_splitkv_noalloc", _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
              lse.data_ptr(), bh, n_q, n_k, d, _scale(scale, d), num_splits, _stream(dev))
    return o, lse


def fa2_bwd_delta(o, do, delta=None):
    """delta [bh,n_q] float32 = rowsum(o * do)."""
    _check("o", o)
    bh, n_q, d = o.shape
    _check("do", do, o.dtype, o.shape, o.device)
    if delta is None:
        delta = torch.empty((bh, n_q), dtype=torch.float32, device=o.device)
    _check("delta", delta, torch.float32, (bh, n_q), o.device)
    _lib.call("fa2_bwd_delta", _dtype_code(o), o.data_ptr(), do.data_ptr(), delta.data_ptr(), bh, n_q, d,
              _stream(o.device))
    return delta


def _bwd_checks(q, k, v, do, lse, delta):
    _check("q", q)
    bh, n_q, d = q.shape
    n_k = k.shape[1]
    dev = q.device
    _check("k", k, q.dtype, (bh, n_k, d), dev)
    _check("v", v, q.dtype, (bh, n_k, d), dev)
    _check("do", do, q.dtype, q.shape, dev)
    _check("lse", lse, torch.float32, (bh, n_q), dev)
    _check("delta", delta, torch.float32, (bh, n_q), dev)
    return bh, n_q, n_k, d, dev


def fa2_bwd_dq(q, k, v, do, lse, delta, scale=None, dq=None):
    """dq [bh,n_q,d] from the saved lse and delta."""
    bh, n_q, n_k, d, dev = _bwd_checks(q, k, v, do, lse, delta)
    if dq is None:
        dq = torch.empty_like(q)
    _check("dq", dq, q.dtype, q.shape, dev)
    _lib.call("fa2_bwd_dq", _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
              lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), bh, n_q, n_k, d, _scale(scale, d), _stream(dev))
    return dq


def fa2_bwd_dkdv(q, k, v, do, lse, delta, scale=None, dk=None, dv=None):
    """(dk, dv) [bh,n_k,d] from the saved lse and delta."""
    bh, n_q, n_k, d, dev = _bwd_checks(q, k, v, do, lse, delta)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check("dk", dk, q.dtype, k.shape, dev)
    _check("dv", dv, q.dtype, v.shape, dev)
    _lib.call("fa2_bwd_dkdv", _dtype_code(q), q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
              lse.data_ptr(), delta.data_ptr(), dk.data_ptr(), dv.data_ptr(), bh, n_q, n_k, d,
              _scale(scale, d), _stream(dev))
    return dk, dv


NATIVE_HEAD_DIMS = (32, 64, 128)


def fa2_pad_cols(x, d_out, out=None):
    """x [..., d] -> [..., d_out]: the first min(d, d_out) columns of every
    row, zeros after them (pads when d_out > d, crops when d_out < d)."""
    _check("x", x)
    d = x.shape[-1]
    shape = tuple(x.shape[:-1]) + (d_out,)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    _check("out", out, x.dtype, shape, x.device)
    rows = x.numel() // d
    _lib.call("fa2_pad_cols", _dtype_code(x), x.data_ptr(), out.data_ptr(), rows, d, d_out, _stream(x.device))
    return out


def _padded_dim(d: int) -> int:
    for n in NATIVE_HEAD_DIMS:
        if d <= n:
            return n
    raise ValueError(f"head_dim {d} > {NATIVE_HEAD_DIMS[-1]} is not supported")


def _fwd_auto(q, k, v, scale):
    """fa2_fwd, or the key-split forward when the split plan uses more than
    one key range (few query rows per head: the plain grid would leave most
    CUs idle)."""
    bh, n_q, d = q.shape
    splits, _ = fa2_fwd_splitkv_plan(q.dtype, bh, n_q, k.shape[1], d, 0)
    if splits > 1:
        return fa2_fwd_splitkv(q, k, v, scale)
    return fa2_fwd(q, k, v, scale)


def attention_fwd(q, k, v, scale=None):
    """(o, lse) of softmax(scale q k^T) v. Shapes with few query rows per head
    take the key-split forward; head dims other than 32, 64 and 128 (up to
    128) run on zero-padded copies; scale defaults to 1/sqrt of the original
    head dim."""
    d = q.shape[-1]
    if d in NATIVE_HEAD_DIMS:
        return _fwd_auto(q, k, v, scale)
    dp = _padded_dim(d)
    o, lse = _fwd_auto(fa2_pad_cols(q, dp), fa2_pad_cols(k, dp), fa2_pad_cols(v, dp), _scale(scale, d))
    return fa2_pad_cols(o, d), lse


def attention_bwd(q, k, v, o, do, lse, scale=None):
    """(dq, dk, dv) given the forward's o and lse and the output gradient do
    (other head dims up to 128 through zero padding, as attention_fwd)."""
    d = q.shape[-1]
    if d not in NATIVE_HEAD_DIMS:
        dp = _padded_dim(d)
        dq, dk, dv = attention_bwd(*(fa2_pad_cols(t, dp) for t in (q, k, v, o, do)), lse, _scale(scale, d))
        return fa2_pad_cols(dq, d), fa2_pad_cols(dk, d), fa2_pad_cols(dv, d)
    delta = fa2_bwd_delta(o, do)
    dk, dv = fa2_bwd_dkdv(q, k, v, do, lse, delta, scale)
    dq = fa2_bwd_dq(q, k, v, do, lse, delta, scale)
    return dq, dk, dv


def psa_pack_qkv(qkv, num_heads: int, key_dim: int, packed=None):
    """qkv [B, nh*4*kd, H, W] -> packed [4, B*nh, H*W, kd] (Q, K, V_lo, V_hi)."""
    _check("qkv", qkv)
    b, ch, h, w = qkv.shape
    if ch != num_heads * 4 * key_dim:
        raise ValueError(f"qkv has {ch} channels, expected num_heads*4*key_dim = {num_heads * 4 * key_dim}")
    if packed is None:
        packed = torch.empty((4, b * num_heads, h * w, key_dim), dtype=qkv.dtype, device=qkv.device)
    _check("packed", packed, qkv.dtype, (4, b * num_heads, h * w, key_dim), qkv.device)
    _lib.call("psa_pack_qkv", _dtype_code(qkv), qkv.data_ptr(), packed.data_ptr(), b, num_heads, key_dim, h, w,
              _stream(qkv.device))
    return packed


def psa_merge_attn(o_lo, o_hi, batch: int, num_heads: int, h: int, w: int, out=None):
    """o_lo, o_hi [B*nh, H*W, kd] -> out [B, nh*2*kd, H, W]."""
    _check("o_lo", o_lo)
    bh, n, kd = o_lo.shape
    if bh != batch * num_heads or n != h * w:
        raise ValueError("o_lo shape does not match batch*num_heads x h*w")
    _check("o_hi", o_hi, o_lo.dtype, o_lo.shape, o_lo.device)
    if out is None:
        out = torch.empty((batch, num_heads * 2 * kd, h, w), dtype=o_lo.dtype, device=o_lo.device)
    _check("out", out, o_lo.dtype, (batch, num_heads * 2 * kd, h, w), o_lo.device)
    _lib.call("psa_merge_attn", _dtype_code(o_lo), o_lo.data_ptr(), o_hi.data_ptr(), out.data_ptr(), batch,
              num_heads, kd, h, w, _stream(o_lo.device))
    return out


def psa_block(qkv, num_heads: int, key_dim: int, workspace: dict | None = None):
    """PSA attention block: pack -> fa2_fwd(Q, K, V_lo) -> fa2_fwd(Q, K, V_hi)
    -> merge, at scale 1/sqrt(key_dim). ``workspace`` (optional dict) keeps
    the intermediate buffers between calls of the same shape. With a
    workspace the returned tensor is ``workspace["out"]``: it belongs to the
    workspace and the next call with the same workspace overwrites it (clone
    it to keep it); without one every call returns a fresh tensor."""
    b, _, h, w = qkv.shape
    ws = workspace if workspace is not None else {}
    shape_key = (tuple(qkv.shape), qkv.dtype, qkv.device, num_heads, key_dim)
    if ws.get("key") != shape_key:
        bh, n = b * num_heads, h * w
        ws.clear()
        ws["key"] = shape_key
        ws["packed"] = torch.empty((4, bh, n, key_dim), dtype=qkv.dtype, device=qkv.device)
        ws["o"] = torch.empty((2, bh, n, key_dim), dtype=qkv.dtype, device=qkv.device)
        ws["lse"] = torch.empty((bh, n), dtype=torch.float32, device=qkv.device)
        ws["out"] = torch.empty((b, num_heads * 2 * key_dim, h, w), dtype=qkv.dtype, device=qkv.device)
    packed, o, lse = ws["packed"], ws["o"], ws["lse"]
    psa_pack_qkv(qkv, num_heads, key_dim, packed)
    scale = 1.0 / math.sqrt(key_dim)
    fa2_fwd(packed[0], packed[1], packed[2], scale, o[0], lse)
    fa2_fwd(packed[0], packed[1], packed[3], scale, o[1], lse)
    return psa_merge_attn(o[0], o[1], b, num_heads, h, w, ws["out"])


def psa_attn_fused(qkv, num_heads: int, key_dim: int, out=None, lse=None):
    """The PSA attention block in one kernel: qkv [B, nh*4*kd, H, W] ->
    out [B, nh*2*kd, H, W] (scale 1/sqrt(kd)). Pass lse ([B*nh, H*W] float32)
    to receive the log-sum-exp. Returns out."""
    _check("qkv", qkv)
    b, ch, h, w = qkv.shape
    if ch != num_heads * 4 * key_dim:
        raise ValueError(f"qkv has {ch} channels, expected num_heads*4*key_dim = {num_heads * 4 * key_dim}")
    if out is None:
        out = torch.empty((b, num_heads * 2 * key_dim, h, w), dtype=qkv.dtype, device=qkv.device)
    _check("out", out, qkv.dtype, (b, num_heads * 2 * key_dim, h, w), qkv.device)
    lse_ptr = None
    if lse is not None:
        _check("lse", lse, torch.float32, (b * num_heads, h * w), qkv.device)
        lse_ptr = lse.data_ptr()
    _lib.call("psa_attn_fused", _dtype_code(qkv), qkv.data_ptr(), out.data_ptr(), lse_ptr, b, num_heads, key_dim,
              h, w, _stream(qkv.device))
    return out


def psa_attn_fused_backward(qkv, out, lse, d_out, num_heads: int, key_dim: int, d_qkv=None, delta=None):
    """Gradient of the PSA attention block with respect to qkv, from qkv, the
    block output `out` and its `lse` (psa_attn_fused with lse) and d_out.
    Returns d_qkv [B, nh*4*kd, H, W] (key_dim 32 with H*W <= 512, or key_dim
    64 with H*W <= 128; f16/bf16).
    `delta` ([B*nh, H*W] float32) receives rowsum(out * d_out) per pixel."""
    _check("qkv", qkv)
    b, ch, h, w = qkv.shape
    if ch != num_heads * 4 * key_dim:
        raise ValueError(f"qkv has {ch} channels, expected num_heads*4*key_dim = {num_heads * 4 * key_dim}")
    dev = qkv.device
    oshape = (b, num_heads * 2 * key_dim, h, w)
    _check("out", out, qkv.dtype, oshape, dev)
    _check("d_out", d_out, qkv.dtype, oshape, dev)
    _check("lse", lse, torch.float32, (b * num_heads, h * w), dev)
    if d_qkv is None:
        d_qkv = torch.empty_like(qkv)
    _check("d_qkv", d_qkv, qkv.dtype, qkv.shape, dev)
    if delta is None:
        delta = torch.empty((b * num_heads, h * w), dtype=torch.float32, device=dev)
    _check("delta", delta, torch.float32, (b * num_heads, h * w), dev)
    _lib.call("psa_attn_fused_backward", _dtype_code(qkv), qkv.data_ptr(), out.data_ptr(), lse.data_ptr(),
              d_out.data_ptr(), d_qkv.data_ptr(), delta.data_ptr(), b, num_heads, key_dim, h, w, _stream(dev))
    return d_qkv


def psa_merge_attn_backward(d_out, num_heads: int, key_dim: int, d_o_lo=None, d_o_hi=None):
    """d_out [B, nh*2*kd, H, W] -> (d_o_lo, d_o_hi) [B*nh, H*W, kd]."""
    _check("d_out", d_out)
    b, ch, h, w = d_out.shape
    if ch != num_heads * 2 * key_dim:
        raise ValueError(f"d_out has {ch} channels, expected num_heads*2*key_dim = {num_heads * 2 * key_dim}")
    shape = (b * num_heads, h * w, key_dim)
    if d_o_lo is None:
        d_o_lo = torch.empty(shape, dtype=d_out.dtype, device=d_out.device)
    if d_o_hi is None:
        d_o_hi = torch.empty(shape, dtype=d_out.dtype, device=d_out.device)
    _check("d_o_lo", d_o_lo, d_out.dtype, shape, d_out.device)
    _check("d_o_hi", d_o_hi, d_out.dtype, shape, d_out.device)
    _lib.call("psa_merge_attn_backward", _dtype_code(d_out), d_out.data_ptr(), d_o_lo.data_ptr(), d_o_hi.data_ptr(),
              b, num_heads, key_dim, h, w, _stream(d_out.device))
    return d_o_lo, d_o_hi


def psa_pack_qkv_backward(d_packed, batch: int, num_heads: int, h: int, w: int, d_qk_extra=None, d_qkv=None):
    """d_packed [4, B*nh, H*W, kd] (+ d_qk_extra [2, B*nh, H*W, kd] added to the
    dQ and dK sections) -> d_qkv [B, nh*4*kd, H, W]."""
    _check("d_packed", d_packed)
    if d_packed.dim() != 4 or d_packed.shape[0] != 4 or d_packed.shape[1] != batch * num_heads \
            or d_packed.shape[2] != h * w:
        raise ValueError(f"d_packed has shape {tuple(d_packed.shape)}, expected [4, batch*num_heads, h*w, key_dim]")
    kd = d_packed.shape[3]
    extra_ptr = None
    if d_qk_extra is not None:
        _check("d_qk_extra", d_qk_extra, d_packed.dtype, (2, batch * num_heads, h * w, kd), d_packed.device)
        extra_ptr = d_qk_extra.data_ptr()
    if d_qkv is None:
        d_qkv = torch.empty((batch, num_heads * 4 * kd, h, w), dtype=d_packed.dtype, device=d_packed.device)
    _check("d_qkv", d_qkv, d_packed.dtype, (batch, num_heads * 4 * kd, h, w), d_packed.device)
    _lib.call("psa_pack_qkv_backward", _dtype_code(d_packed), d_packed.data_ptr(), extra_ptr, d_qkv.data_ptr(),
              batch, num_heads, kd, h, w, _stream(d_packed.device))
    return d_qkv


def psa_block_backward(d_out, num_heads: int, key_dim: int, workspace: dict):
    """Gradient of psa_block with respect to qkv. ``workspace`` is the dict of
    the forward psa_block call on the same shapes (it holds the packed
    operands, both attention outputs and the LSE); the backward's own buffers
    are kept in it too. Steps: merge backward -> for V_lo and V_hi: delta,
    dK/dV, dQ on the packed sections -> pack backward, which adds the second
    call's dQ and dK to the first's. Returns d_qkv [B, nh*4*kd, H, W], which
    is ``workspace["d_qkv"]``: it belongs to the workspace and the next
    backward call with the same workspace overwrites it (clone it to keep
    it)."""
    ws = workspace
    _check("d_out", d_out)
    b, ch, h, w = d_out.shape
    key = ws.get("key")
    if key is None or key[0][0] != b or key[0][2:] != (h, w) or key[1] != d_out.dtype or key[3:] != (num_heads, key_dim):
        raise ValueError("workspace does not come from a psa_block forward on these shapes")
    bh, n = b * num_heads, h * w
    bkey = ("bwd",) + key
    if ws.get("bwd_key") != bkey:
        ws["bwd_key"] = bkey
        ws["d_o"] = torch.empty((2, bh, n, key_dim), dtype=d_out.dtype, device=d_out.device)
        ws["d_packed"] = torch.empty((4, bh, n, key_dim), dtype=d_out.dtype, device=d_out.device)
        ws["d_qk_extra"] = torch.empty((2, bh, n, key_dim), dtype=d_out.dtype, device=d_out.device)
        ws["delta"] = torch.empty((bh, n), dtype=torch.float32, device=d_out.device)
        ws["d_qkv"] = torch.empty((b, num_heads * 4 * key_dim, h, w), dtype=d_out.dtype, device=d_out.device)
    packed, o, lse = ws["packed"], ws["o"], ws["lse"]
    d_o, d_packed, extra, delta = ws["d_o"], ws["d_packed"], ws["d_qk_extra"], ws["delta"]
    psa_merge_attn_backward(d_out, num_heads, key_dim, d_o[0], d_o[1])
    scale = 1.0 / math.sqrt(key_dim)
    for half in (0, 1):
        dq_dst, dk_dst = (d_packed[0], d_packed[1]) if half == 0 else (extra[0], extra[1])
        fa2_bwd_delta(o[half], d_o[half], delta)
        fa2_bwd_dkdv(packed[0], packed[1], packed[2 + half], d_o[half], lse, delta, scale, dk_dst, d_packed[2 + half])
        fa2_bwd_dq(packed[0], packed[1], packed[2 + half], d_o[half], lse, delta, scale, dq_dst)
    return psa_pack_qkv_backward(d_packed, b, num_heads, h, w, extra, ws["d_qkv"])


def psa_extract_v_nchw(qkv, num_heads: int, key_dim: int, v=None):
    """qkv [B, nh*4*kd, H, W] -> v [B, nh*2*kd, H, W] (each head's V_lo, V_hi channels)."""
    _check("qkv", qkv)
    b, ch, h, w = qkv.shape
    if ch != num_heads * 4 * key_dim:
        raise ValueError(f"qkv has {ch} channels, expected num_heads*4*key_dim = {num_heads * 4 * key_dim}")
    if v is None:
        v = torch.empty((b, num_heads * 2 * key_dim, h, w), dtype=qkv.dtype, device=qkv.device)
    _check("v", v, qkv.dtype, (b, num_heads * 2 * key_dim, h, w), qkv.device)
    _lib.call("psa_extract_v_nchw", _dtype_code(qkv), qkv.data_ptr(), v.data_ptr(), b, num_heads, key_dim, h, w,
              _stream(qkv.device))
    return v


def psa_extract_v_backward(d_v, d_qkv, num_heads: int, key_dim: int):
    """Adds d_v [B, nh*2*kd, H, W] into the V channels of d_qkv [B, nh*4*kd, H, W]
    (in place; call it after psa_pack_qkv_backward). Returns d_qkv."""
    _check("d_v", d_v)
    b, ch, h, w = d_v.shape
    if ch != num_heads * 2 * key_dim:
        raise ValueError(f"d_v has {ch} channels, expected num_heads*2*key_dim = {num_heads * 2 * key_dim}")
    _check("d_qkv", d_qkv, d_v.dtype, (b, num_heads * 4 * key_dim, h, w), d_v.device)
    _lib.call("psa_extract_v_backward", _dtype_code(d_v), d_v.data_ptr(), d_qkv.data_ptr(), b, num_heads, key_dim,
              h, w, _stream(d_v.device))
    return d_qkv

