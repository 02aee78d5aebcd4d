"""CPU fp64 oracle for exact attention and the PSA rearrangements.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The library (the HIP path and its
Python binding) never imports it, and it imports nothing from the library.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, OpenMP over rows or
heads). This module only marshals arrays: it upcasts the dtype-rounded inputs
exactly to fp64, calls the C routine and returns fp64 numpy arrays.

What each routine follows:
  * ``attention_fwd``  - the definition softmax(scale * Q K^T) V with the
    natural-log LSE (vision-rs flash_attn2.rs, "Forward").
  * ``attention_bwd``  - its analytic gradients (same page, "Backward - dQ",
    "Backward - dK / dV").
  * ``psa_pack`` / ``psa_merge`` - the index maps of vision_rs psa.rs,
    "psa_pack_qkv" and "psa_merge_attn_nchw".
  * ``psa_block`` - pack, attention on (Q, K, V_lo) and (Q, K, V_hi) at
    scale 1/sqrt(key_dim), merge (psa.rs module doc, the V-split trick, and
    "FlashAttn2PsaRuntimeOp").
  * ``psa_merge_backward`` / ``psa_pack_backward`` - the inverse index maps
    (psa.rs "psa_merge_attn_backward", "psa_pack_qkv_backward").
  * ``psa_extract_v`` / ``psa_extract_v_backward`` - the V-channel gather of
    psa.rs "psa_extract_v_nchw" and its adjoint, the scatter of d_v into the
    V channels of a zero d_qkv ("psa_extract_v_backward").
  * ``psa_block_backward`` - the block's gradient by the chain rule in the
    order of psa.rs's backward: merge backward, the attention gradients of
    both calls (dQ and dK summed over the two calls, as that page's combined
    backward adds them), pack backward.

Every routine is pinned by the CPU tests in tests/test_oracle_*.py against
values and facts that do not come from this code (hand-worked cases, a page's
worked example, closed forms, invariants, finite differences and library
routines). The stability guards one page applies to scores and exponents
(bounded_score, bounded_exp_arg, flush_tiny, positive_denominator) are not
defined on the pages and are not modelled: parity unpinned for them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "attn_oracle.c"
_LIB = _HERE / "liboracle.so"
_lib = None

_i64 = ctypes.c_int64
_dptr = ctypes.POINTER(ctypes.c_double)


def build(force: bool = True) -> Path:
    """Compile attn_oracle.c into liboracle.so with gcc + OpenMP."""
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build()
        lib = ctypes.CDLL(str(_LIB))
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_fwd.argtypes = [_dptr] * 5 + [_i64] * 5 + [ctypes.c_double, ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [_dptr] * 7 + [_i64] * 5 + [ctypes.c_double, ctypes.c_int]
        lib.oracle_psa_pack.restype = ctypes.c_int
        lib.oracle_psa_pack.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int] + [_i64] * 4
        lib.oracle_psa_merge.restype = ctypes.c_int
        lib.oracle_psa_merge.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] + [_i64] * 4
        lib.oracle_psa_merge_backward.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] + [_i64] * 4
        lib.oracle_psa_pack_backward.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int] + [_i64] * 4
        lib.oracle_psa_extract_v.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int] + [_i64] * 4
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads the oracle uses: OMP_NUM_THREADS if set, else the cores this
    process may run on."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (any float dtype) or array to a
    C-contiguous fp64 numpy array."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dptr)


def attention_fwd(q, k, v, scale: float, threads: int | None = None):
    """O [bh, nq, dv] and LSE [bh, nq] (natural log), fp64.

    q [bh, nq, d], k [bh, nk, d], v [bh, nk, dv]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, nq, d = q.shape
    nk, dv = k.shape[1], v.shape[2]
    if k.shape != (bh, nk, d) or v.shape != (bh, nk, dv):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    o = np.empty((bh, nq, dv), np.float64)
    lse = np.empty((bh, nq), np.float64)
    rc = _load().oracle_attn_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse), bh, nq, nk, d, dv,
                                 float(scale), threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_attn_fwd failed")
    return o, lse


def attention_bwd(q, k, v, do, scale: float, threads: int | None = None):
    """dQ, dK, dV (fp64) of L = sum(O * dO) for O = attention(q, k, v)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    bh, nq, d = q.shape
    nk, dv = k.shape[1], v.shape[2]
    if do.shape != (bh, nq, dv):
        raise ValueError("dO shape mismatch")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dvv = np.empty_like(v)
    rc = _load().oracle_attn_bwd(_p(q), _p(k), _p(v), _p(do), _p(dq), _p(dk), _p(dvv),
                                 bh, nq, nk, d, dv, float(scale), threads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_attn_bwd failed")
    return dq, dk, dvv


def _raw(x) -> np.ndarray:
    """A tensor/array as a contiguous numpy array holding the same element
    bits: numpy's own dtype where it has one, the int16 bit view for bfloat16."""
    if hasattr(x, "detach"):
        import torch

        t = x.detach().to("cpu").contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy()
        return t.numpy()
    return np.ascontiguousarray(x)


def psa_pack(qkv, num_heads: int, key_dim: int) -> np.ndarray:
    """qkv [B, nh*4*kd, H, W] -> packed [4, B*nh, H*W, kd], bit-exact copy
    (numpy dtype of the input; bfloat16 comes back as its int16 bit view)."""
    src = _raw(qkv)
    b, ch, h, w = src.shape
    if ch != num_heads * 4 * key_dim:
        raise ValueError("channel count is not num_heads*4*key_dim")
    out = np.empty((4, b * num_heads, h * w, key_dim), src.dtype)
    rc = _load().oracle_psa_pack(src.ctypes.data, out.ctypes.data, src.itemsize,
                                 b, num_heads, key_dim, h * w)
    if rc != 0:
        raise RuntimeError("oracle_psa_pack failed")
    return out


def psa_merge(lo, hi, batch: int, num_heads: int, key_dim: int, h: int, w: int) -> np.ndarray:
    """lo, hi [B*nh, H*W, kd] -> out [B, nh*2*kd, H, W], bit-exact copy."""
    a, b_ = _raw(lo), _raw(hi)
    if a.shape != (batch * num_heads, h * w, key_dim) or b_.shape != a.shape or a.dtype != b_.dtype:
        raise ValueError("lo/hi shape mismatch")
    out = np.empty((batch, num_heads * 2 * key_dim, h, w), a.dtype)
    rc = _load().oracle_psa_merge(a.ctypes.data, b_.ctypes.data, out.ctypes.data, a.itemsize,
                                  batch, num_heads, key_dim, h * w)
    if rc != 0:
        raise RuntimeError("oracle_psa_merge failed")
    return out


def psa_block(qkv, num_heads: int, key_dim: int, threads: int | None = None) -> np.ndarray:
    """The PSA attention block in fp64: pack, attention with V_lo and with
    V_hi at scale 1/sqrt(key_dim), merge. Returns out [B, nh*2*kd, H, W] fp64."""
    x = _f64(qkv)
    b, _, h, w = x.shape
    packed = psa_pack(x, num_heads, key_dim)
    scale = 1.0 / np.sqrt(key_dim)
    o_lo, _ = attention_fwd(packed[0], packed[1], packed[2], scale, threads)
    o_hi, _ = attention_fwd(packed[0], packed[1], packed[3], scale, threads)
    return psa_merge(o_lo, o_hi, b, num_heads, key_dim, h, w)


def psa_merge_backward(d_out, num_heads: int, key_dim: int):
    """d_out [B, nh*2*kd, H, W] -> (d_lo, d_hi) [B*nh, H*W, kd], bit-exact copy."""
    src = _raw(d_out)
    b, ch, h, w = src.shape
    if ch != num_heads * 2 * key_dim:
        raise ValueError("channel count is not num_heads*2*key_dim")
    lo = np.empty((b * num_heads, h * w, key_dim), src.dtype)
    hi = np.empty_like(lo)
    rc = _load().oracle_psa_merge_backward(src.ctypes.data, lo.ctypes.data, hi.ctypes.data, src.itemsize,
                                           b, num_heads, key_dim, h * w)
    if rc != 0:
        raise RuntimeError("oracle_psa_merge_backward failed")
    return lo, hi


def psa_pack_backward(d_packed, batch: int, num_heads: int, h: int, w: int) -> np.ndarray:
    """d_packed [4, B*nh, H*W, kd] -> d_qkv [B, nh*4*kd, H, W], bit-exact copy."""
    src = _raw(d_packed)
    if src.ndim != 4 or src.shape[0] != 4 or src.shape[1] != batch * num_heads or src.shape[2] != h * w:
        raise ValueError("d_packed shape mismatch")
    kd = src.shape[3]
    out = np.empty((batch, num_heads * 4 * kd, h, w), src.dtype)
    rc = _load().oracle_psa_pack_backward(src.ctypes.data, out.ctypes.data, src.itemsize,
                                          batch, num_heads, kd, h * w)
    if rc != 0:
        raise RuntimeError("oracle_psa_pack_backward failed")
    return out


def psa_block_backward(qkv, num_heads: int, key_dim: int, d_out, threads: int | None = None) -> np.ndarray:
    """Gradient of sum(psa_block(qkv) * d_out) with respect to qkv, fp64.
    Returns d_qkv [B, nh*4*kd, H, W]."""
    x, g = _f64(qkv), _f64(d_out)
    b, _, h, w = x.shape
    packed = psa_pack(x, num_heads, key_dim)
    d_lo, d_hi = psa_merge_backward(g, num_heads, key_dim)
    scale = 1.0 / np.sqrt(key_dim)
    dq_lo, dk_lo, dv_lo = attention_bwd(packed[0], packed[1], packed[2], d_lo, scale, threads)
    dq_hi, dk_hi, dv_hi = attention_bwd(packed[0], packed[1], packed[3], d_hi, scale, threads)
    d_packed = np.stack([dq_lo + dq_hi, dk_lo + dk_hi, dv_lo, dv_hi])
    return psa_pack_backward(d_packed, b, num_heads, h, w)


def psa_extract_v(qkv, num_heads: int, key_dim: int) -> np.ndarray:
    """qkv [B, nh*4*kd, H, W] -> v [B, nh*2*kd, H, W], bit-exact copy."""
    src = _raw(qkv)
    b, ch, h, w = src.shape
    if ch != num_heads * 4 * key_dim:
        raise ValueError("channel count is not num_heads*4*key_dim")
    out = np.empty((b, num_heads * 2 * key_dim, h, w), src.dtype)
    rc = _load().oracle_psa_extract_v(src.ctypes.data, out.ctypes.data, src.itemsize, b, num_heads, key_dim, h * w)
    if rc != 0:
        raise RuntimeError("oracle_psa_extract_v failed")
    return out


def psa_extract_v_backward(d_v, num_heads: int, key_dim: int) -> np.ndarray:
    """The gradient of psa_extract_v with respect to qkv for output gradient
    d_v [B, nh*2*kd, H, W]: d_v in each head's V channels, zero in its Q and K
    channels. fp64 [B, nh*4*kd, H, W]."""
    g = _f64(d_v)
    b, ch, h, w = g.shape
    if ch != num_heads * 2 * key_dim:
        raise ValueError("channel count is not num_heads*2*key_dim")
    out = np.zeros((b, num_heads, 4 * key_dim, h, w), np.float64)
    out[:, :, 2 * key_dim:] = g.reshape(b, num_heads, 2 * key_dim, h, w)
    return out.reshape(b, num_heads * 4 * key_dim, h, w)


if __name__ == "__main__":  # pragma: no cover
    print(build(), file=sys.stderr)
