"""ctypes loader for libfa2mi.so and the signatures of include/fa2mi.h."""
from __future__ import annotations

import ctypes
from pathlib import Path

FA2_F32, FA2_F16, FA2_BF16 = 0, 1, 2
FA2_OK = 0

_LIB_PATH = Path(__file__).resolve().parent / "libfa2mi.so"
_lib = None

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_int = ctypes.c_int

# name -> argtypes, in the order of include/fa2mi.h
SIGNATURES = {
    "fa2_abi_version": [],
    "fa2_status_str": [_int],
    "fa2_last_error": [],
    "fa2_fwd": [_int, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _f32, _p],
    "fa2_fwd_splitkv_plan": [_int, _i64, _i64, _i64, _i32, _i32, _p, _p],
    "fa2_fwd_splitkv": [_int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _f32, _i32, _p],
    "fa2_fwd_splitkv_noalloc_max_bytes": [],
    "fa2_fwd_splitkv_noalloc": [_int, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _f32, _i32, _p],
    "fa2_bwd_delta": [_int, _p, _p, _p, _i64, _i64, _i32, _p],
    "fa2_bwd_dq": [_int, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _f32, _p],
    "fa2_bwd_dkdv": [_int, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i32, _f32, _p],
    "fa2_pad_cols": [_int, _p, _p, _i64, _i32, _i32, _p],
    "psa_pack_qkv": [_int, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_merge_attn": [_int, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_attn_fused": [_int, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_attn_fused_backward": [_int, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_merge_attn_backward": [_int, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_pack_qkv_backward": [_int, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_extract_v_nchw": [_int, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
    "psa_extract_v_backward": [_int, _p, _p, _i32, _i32, _i32, _i32, _i32, _p],
}
_RESTYPES = {"fa2_abi_version": _i32, "fa2_fwd_splitkv_noalloc_max_bytes": _i64,
             "fa2_status_str": ctypes.c_char_p, "fa2_last_error": ctypes.c_char_p}


class Fa2Error(RuntimeError):
    """A C entry point returned a non-zero fa2_status."""

    def __init__(self, name: str, status: int, detail: str):
        super().__init__(f"{name} failed with status {status}: {detail}")
        self.status = status


def library_path() -> Path:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Loads the built library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python attention_fa2_fwd_02_amd/build.py` (there is no fallback path)")
        lib = ctypes.CDLL(str(_LIB_PATH))
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = _RESTYPES.get(name, _int)
        _lib = lib
    return _lib


def call(name: str, *args) -> None:
    lib = load()
    st = getattr(lib, name)(*args)
    if st != FA2_OK:
        raise Fa2Error(name, st, lib.fa2_last_error().decode())
