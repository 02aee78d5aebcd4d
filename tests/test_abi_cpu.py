"""CPU checks of the C-ABI boundary: the built library loads, exports every
function include/fa2mi.h declares, and rejects invalid arguments with the
documented status codes before anything is enqueued (these calls never reach
the HIP runtime, so they run without a GPU). The Python binding refuses CPU
tensors instead of computing anything on the host."""
import ctypes
import os
import re

import pytest
import torch

import attention_fa2_fwd_02_amd as fa2
from attention_fa2_fwd_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2mi.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
A = 0x10000        # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10008      # misaligned


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:fa2|psa)_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = fa2.load()
    names = _declared()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = fa2.load()
    assert lib.fa2_abi_version() == 1
    assert lib.fa2_status_str(0) == b"ok"
    assert lib.fa2_status_str(2) == b"unsupported size"


def _fwd(**kw):
    a = dict(dt=2, q=A, k=A, v=A, o=A, lse=A, bh=2, n_q=64, n_k=64, d=64, scale=0.125, stream=None)
    a.update(kw)
    lib = fa2.load()
    return lib.fa2_fwd(a["dt"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["bh"], a["n_q"], a["n_k"], a["d"],
                       a["scale"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    ({"q": None}, INVALID), ({"lse": None}, INVALID), ({"v": MIS}, INVALID),
    ({"bh": 0}, INVALID), ({"n_q": 0}, INVALID), ({"n_k": -3}, INVALID), ({"dt": 7}, INVALID),
    ({"d": 48}, UNSUPPORTED), ({"d": 256}, UNSUPPORTED), ({"d": 0}, INVALID),
    ({"scale": float("nan")}, INVALID), ({"scale": float("inf")}, INVALID),
    ({"scale": 0.0}, INVALID), ({"scale": -0.125}, INVALID),
    ({"n_q": 1 << 25, "d": 128}, INVALID),          # one head's rows over 2 GiB
    ({"n_k": (1 << 23) + 1, "d": 128}, INVALID),    # bf16 keys: 2 GiB + 256 B
    ({"dt": 0, "n_q": (1 << 22) + 1, "d": 128}, INVALID),  # f32: 2 GiB + 512 B
    ({"bh": 1 << 40, "n_q": 1 << 20}, INVALID),     # grid over 2^31-1 workgroups
    ({"n_q": 1 << 60}, INVALID),                    # length beyond int (its byte count would overflow int64)
    ({"n_k": (1 << 62) + 1}, INVALID),
])
def test_fwd_rejects_invalid_arguments(kw, code):
    assert _fwd(**kw) == code
    assert fa2.load().fa2_last_error().startswith(b"fa2_fwd: ")


def test_bwd_and_psa_reject_invalid_arguments():
    lib = fa2.load()
    assert lib.fa2_bwd_delta(2, A, None, A, 2, 64, 64, None) == INVALID
    assert lib.fa2_bwd_delta(2, A, A, A, 2, 64, 96, None) == UNSUPPORTED
    assert lib.fa2_bwd_dq(2, A, A, A, A, A, None, A, 2, 64, 64, 64, 0.1, None) == INVALID
    assert lib.fa2_bwd_dq(2, A, A, A, A, A, A, A, 2, 64, 64, 16, 0.1, None) == UNSUPPORTED
    assert lib.fa2_bwd_dkdv(2, A, A, A, A, A, A, A, MIS, 2, 64, 64, 64, 0.1, None) == INVALID
    assert lib.fa2_bwd_dkdv(1, A, A, A, A, A, A, A, A, 2, 64, 0, 64, 0.1, None) == INVALID
    assert lib.psa_pack_qkv(1, A, None, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_pack_qkv(1, A, A, 16, 4, 40, 20, 20, None) == UNSUPPORTED
    assert lib.psa_pack_qkv(1, A, A, 16, 0, 32, 20, 20, None) == INVALID
    assert lib.psa_merge_attn(1, A, A, MIS, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_merge_attn(5, A, A, A, 16, 4, 32, 20, 20, None) == INVALID
    assert b"psa_merge_attn" in lib.fa2_last_error()
    assert lib.psa_attn_fused(0, A, A, None, 16, 4, 32, 20, 20, None) == UNSUPPORTED   # f32
    assert lib.psa_attn_fused(1, A, A, None, 16, 4, 128, 20, 20, None) == UNSUPPORTED  # key_dim 128
    assert lib.psa_attn_fused(1, A, None, None, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_attn_fused(2, A, A, A + 2, 16, 4, 32, 20, 20, None) == INVALID     # lse misaligned
    assert lib.psa_attn_fused(2, A, A, A, 16, 4, 32, 0, 20, None) == INVALID
    assert lib.psa_merge_attn_backward(1, A, A, None, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_merge_attn_backward(1, A, A, A, 16, 4, 48, 20, 20, None) == UNSUPPORTED
    assert lib.psa_merge_attn_backward(1, A, MIS, A, 16, 4, 32, 20, 20, None) == INVALID
    assert b"psa_merge_attn_backward" in lib.fa2_last_error()
    assert lib.psa_pack_qkv_backward(2, None, None, A, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_pack_qkv_backward(2, A, MIS, A, 16, 4, 32, 20, 20, None) == INVALID    # extra misaligned
    assert lib.psa_pack_qkv_backward(2, A, None, A, 0, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_pack_qkv_backward(9, A, None, A, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_extract_v_nchw(1, A, None, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_extract_v_nchw(1, A, A, 16, 4, 16, 20, 20, None) == UNSUPPORTED
    assert lib.psa_extract_v_backward(2, MIS, A, 16, 4, 32, 20, 20, None) == INVALID
    assert lib.psa_extract_v_backward(2, A, A, 16, 4, 32, -1, 20, None) == INVALID
    fb = lib.psa_attn_fused_backward
    assert fb(0, A, A, A, A, A, A, 16, 4, 32, 20, 20, None) == UNSUPPORTED      # f32
    assert fb(1, A, A, A, A, A, A, 16, 4, 128, 4, 4, None) == UNSUPPORTED      # key_dim 128
    assert b"key_dim must be 32 or 64" in lib.fa2_last_error()
    assert fb(1, A, A, A, A, A, A, 16, 4, 64, 20, 20, None) == UNSUPPORTED      # key_dim 64, 400 pixels
    assert b"<= 128 at key_dim 64" in lib.fa2_last_error()
    assert fb(1, A, A, A, A, A, A, 16, 4, 32, 16, 33, None) == UNSUPPORTED      # key_dim 32, 528 pixels
    assert b"<= 512 at key_dim 32" in lib.fa2_last_error()
    assert fb(1, A, A, None, A, A, A, 16, 4, 32, 20, 20, None) == INVALID       # lse
    assert fb(2, A, A, A, A, A, A + 2, 16, 4, 32, 20, 20, None) == INVALID      # delta misaligned
    assert fb(2, A, MIS, A, A, A, A, 16, 4, 32, 20, 20, None) == INVALID        # out misaligned
    assert fb(2, A, A, A, A, None, A, 16, 4, 32, 20, 20, None) == INVALID       # d_qkv
    assert fb(2, A, A, A, A, A, A, 0, 4, 32, 20, 20, None) == INVALID
    assert b"psa_attn_fused_backward" in lib.fa2_last_error()


def _plan(dt, bh, n_q, n_k, d, splits):
    lib = fa2.load()
    used, nbytes = ctypes.c_int32(-7), ctypes.c_int64(-7)
    st = lib.fa2_fwd_splitkv_plan(dt, bh, n_q, n_k, d, splits, ctypes.addressof(used), ctypes.addressof(nbytes))
    return st, used.value, nbytes.value


@pytest.mark.parametrize("bh,n_q,n_k,d,req", [
    (32, 1, 32768, 128, 0), (32, 1, 32768, 128, 5), (3, 5, 1000, 64, 0), (2, 70, 333, 32, 0),
    (1, 130, 5000, 128, 1000), (8, 1, 100, 128, 0), (512, 4096, 4096, 128, 0), (1, 1, 65, 32, 7),
    (1, 1, 1, 64, 4), (7, 300, 9000, 64, 0),
])
def test_splitkv_plan(bh, n_q, n_k, d, req):
    """The plan is host-only: split count and workspace size follow the
    documented rule (ranges of a multiple of 64 keys covering n_k with no
    empty range; one float32 output row plus one log-sum-exp per range and
    query row; no workspace for a single range)."""
    st, used, nbytes = _plan(2, bh, n_q, n_k, d, req)
    assert st == OK
    tiles = -(-n_k // 64)
    assert 1 <= used <= tiles
    if req > 0:
        want = min(req, tiles)
        length = -(-(-(-n_k // want)) // 64) * 64
        assert used == -(-n_k // length)
    length = -(-(-(-n_k // used)) // 64) * 64
    assert (used - 1) * length < n_k <= used * length    # every range non-empty
    assert nbytes == (0 if used == 1 else used * bh * n_q * (d + 1) * 4)


def test_splitkv_plan_auto_fills_the_device():
    # one query row, 32 heads, 32768 keys: 32 workgroups without the split
    st, used, _ = _plan(2, 32, 1, 32768, 128, 0)
    assert st == OK and used * 32 >= 256 and 32768 / used >= 256
    # already one workgroup per CU or more: no split
    assert _plan(2, 512, 4096, 4096, 128, 0)[1] == 1
    # short key lengths are not cut below 256 keys per range
    assert _plan(2, 1, 1, 600, 128, 0)[1] == 3


def test_splitkv_rejects_invalid_arguments():
    lib = fa2.load()
    assert _plan(2, 32, 1, 4096, 128, -1)[0] == INVALID
    assert _plan(2, 32, 1, 4096, 96, 0)[0] == UNSUPPORTED
    assert _plan(2, 0, 1, 4096, 128, 0)[0] == INVALID
    assert _plan(6, 1, 1, 4096, 128, 0)[0] == INVALID
    assert lib.fa2_fwd_splitkv_plan(2, 32, 1, 4096, 128, 0, None, None) == INVALID
    assert b"fa2_fwd_splitkv_plan" in lib.fa2_last_error()
    _, used, need = _plan(2, 32, 1, 32768, 128, 0)
    assert used > 1

    def call(ws=A, nbytes=need, splits=0, **kw):
        a = dict(dt=2, q=A, k=A, v=A, o=A, lse=A, bh=32, n_q=1, n_k=32768, d=128, scale=0.1)
        a.update(kw)
        return lib.fa2_fwd_splitkv(a["dt"], a["q"], a["k"], a["v"], a["o"], a["lse"], ws, nbytes, a["bh"],
                                   a["n_q"], a["n_k"], a["d"], a["scale"], splits, None)

    assert call(nbytes=need - 1) == INVALID                  # workspace too small
    assert b"workspace_bytes" in lib.fa2_last_error()
    assert call(ws=None) == INVALID
    assert call(ws=MIS) == INVALID
    assert call(splits=-2) == INVALID
    assert call(q=None) == INVALID
    assert call(d=16) == UNSUPPORTED
    assert call(scale=0.0) == INVALID
    assert b"fa2_fwd_splitkv" in lib.fa2_last_error()


def test_pad_cols_rejects_invalid_arguments():
    lib = fa2.load()
    assert lib.fa2_pad_cols(1, A, A, 0, 7, 32, None) == INVALID
    assert lib.fa2_pad_cols(1, A, A, 10, 0, 32, None) == INVALID
    assert lib.fa2_pad_cols(1, A, A, 10, 7, -1, None) == INVALID
    assert lib.fa2_pad_cols(4, A, A, 10, 7, 32, None) == INVALID
    assert lib.fa2_pad_cols(2, None, A, 10, 7, 32, None) == INVALID
    assert lib.fa2_pad_cols(2, A, MIS, 10, 7, 32, None) == INVALID
    assert lib.fa2_pad_cols(2, A, A, 1 << 40, 7, 32, None) == INVALID   # grid
    assert b"fa2_pad_cols" in lib.fa2_last_error()


def test_binding_pads_only_unsupported_head_dims():
    assert [fa2._padded_dim(d) for d in (1, 4, 7, 8, 16, 32, 33, 64, 100, 128)] == \
        [32, 32, 32, 32, 32, 32, 64, 64, 128, 128]
    with pytest.raises(ValueError, match="not supported"):
        fa2._padded_dim(129)


def test_binding_refuses_host_tensors():
    q = torch.zeros(1, 8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa2.fa2_fwd(q, q, q)
    x = torch.zeros(1, 4 * 32, 2, 2, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa2.psa_pack_qkv(x, 1, 32)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_LIB_PATH", tmp_path / "libfa2mi.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()


def test_splitkv_noalloc_rejects_partials_above_its_scratch():
    """The allocation-free key-split forward refuses, on the host and before
    any HIP call, a plan whose float32 partials exceed its static scratch."""
    lib = fa2.load()
    cap = lib.fa2_fwd_splitkv_noalloc_max_bytes()
    assert cap == 32 << 20
    # 8 ranges x 256 heads x 256 rows x 129 floats = 270 MB
    assert lib.fa2_fwd_splitkv_noalloc(2, A, A, A, A, A, 256, 256, 4096, 128, 0.088, 8, None) == INVALID
    assert b"scratch" in lib.fa2_last_error()
    assert lib.fa2_fwd_splitkv_noalloc(2, A, A, A, A, None, 2, 1, 4096, 128, 0.088, 0, None) == INVALID
    assert lib.fa2_fwd_splitkv_noalloc(2, A, A, A, A, A, 2, 1, 4096, 48, 0.088, 0, None) == UNSUPPORTED
    assert lib.fa2_fwd_splitkv_noalloc(2, A, A, A, A, A, 2, 1, 4096, 128, 0.088, -1, None) == INVALID
