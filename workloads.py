"""Seeded synthetic inputs for the attention hot path.

This module holds shapes, seeds and random-number draws only: none of the
attention arithmetic lives here. Both the HIP path's tests/bench and the CPU
oracle's tests take their inputs from it, so the two sides always see the same
tensors.

Recipe: values are drawn i.i.d. N(0, 1) in float32 with a seeded
``torch.Generator`` and rounded once to the workload dtype. Draw order per
workload is Q, K, V, dO (each a separate tensor). Where a key tensor is
"scaled by 3" the float32 draw is multiplied by 3 before the single rounding.
Small workloads draw on the CPU; workloads whose tensors exceed
``_CPU_DRAW_LIMIT`` elements draw on the target device with a device generator
seeded the same way (a different stream of numbers from the CPU one, still
seeded and reproducible on one device type).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
_CPU_DRAW_LIMIT = 1 << 24


@dataclass(frozen=True)
class AttnWorkload:
    """One attention problem over the flat [BH, N, D] layout."""

    name: str
    bh: int
    n_q: int
    n_k: int
    head_dim: int
    dtype: str
    seed: int
    k_mult: float = 1.0
    backward: bool = False
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    def fwd_flops(self) -> float:
        return 4.0 * self.bh * self.n_q * self.n_k * self.head_dim

    def bwd_flops(self) -> float:
        return 2.5 * self.fwd_flops()


@dataclass(frozen=True)
class PsaWorkload:
    """A YOLO C2PSA-shaped attention block: NCHW qkv [B, nh*4*kd, H, W]."""

    name: str
    batch: int
    num_heads: int
    key_dim: int
    h: int
    w: int
    dtype: str
    seed: int
    note: str = ""

    @property
    def n(self) -> int:
        return self.h * self.w

    @property
    def bh(self) -> int:
        return self.batch * self.num_heads

    @property
    def qkv_channels(self) -> int:
        return self.num_heads * 4 * self.key_dim

    @property
    def out_channels(self) -> int:
        return self.num_heads * 2 * self.key_dim

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.key_dim)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    def attn_flops(self) -> float:
        """Two attention calls at head_dim = key_dim (V split into halves)."""
        return 2 * 4.0 * self.bh * self.n * self.n * self.key_dim

    def algorithmic_bytes(self) -> dict:
        """Each tensor read or written once, per stage of the block."""
        es = torch.finfo(self.torch_dtype).bits // 8
        qkv = self.batch * self.qkv_channels * self.n * es
        sec = self.bh * self.n * self.key_dim * es
        lse = self.bh * self.n * 4
        out = self.batch * self.out_channels * self.n * es
        return {
            "pack": 2 * qkv,
            "attn_each": 4 * sec + lse,
            "merge": 2 * sec + out,
            "fused": qkv + out,
        }


C1 = AttnWorkload("c1_tiny_f32", bh=2, n_q=64, n_k=64, head_dim=32, dtype="f32", seed=1,
                  note="tiny fp32 forward, outputs O and LSE")
C2 = PsaWorkload("c2_psa_f16", batch=16, num_heads=4, key_dim=32, h=20, w=20, dtype="f16", seed=2,
                 note="C2PSA block: pack -> attention(V_lo) -> attention(V_hi) -> merge")
C3 = AttnWorkload("c3_llm_bf16", bh=512, n_q=4096, n_k=4096, head_dim=128, dtype="bf16", seed=3,
                  note="LLM-shaped forward, BH=16*32")
C4 = AttnWorkload("c4_xattn_bf16", bh=1024, n_q=1024, n_k=8192, head_dim=64, dtype="bf16", seed=4,
                  k_mult=3.0, note="cross-attention, unequal lengths, K scaled by 3")
C5 = AttnWorkload("c5_bwd_bf16", bh=256, n_q=2048, n_k=2048, head_dim=128, dtype="bf16", seed=5,
                  backward=True, note="backward from the forward's O and fp32 LSE")

# Not one of the five configurations: a decoding-shaped forward (one query
# row per head against a long key cache) for the key-split forward.
DECODE = AttnWorkload("decode_bf16", bh=32, n_q=1, n_k=32768, head_dim=128, dtype="bf16", seed=6,
                      note="decoding: 32 heads, 1 query row, 32768 keys")

ATTN_WORKLOADS = {w.name: w for w in (C1, C3, C4, C5, DECODE)}
PSA_WORKLOADS = {C2.name: C2}


def _draw(gen: torch.Generator, shape, dtype: torch.dtype, device, mult: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32, device=gen.device)
    if mult != 1.0:
        x.mul_(mult)
    return x.to(device=device, dtype=dtype)


def _generator(seed: int, numel: int, device) -> torch.Generator:
    dev = torch.device(device)
    if dev.type == "cuda" and numel > _CPU_DRAW_LIMIT:
        g = torch.Generator(device=dev)
    else:
        g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def attn_inputs(w: AttnWorkload, device="cpu", bh: int | None = None, n_q: int | None = None,
                n_k: int | None = None, with_do: bool | None = None, dtype: str | None = None,
                seed: int | None = None) -> dict:
    """Q, K, V (and dO when the workload is a backward one) for workload ``w``.

    ``bh``/``n_q``/``n_k``/``dtype``/``seed`` override the workload's sizes
    for reduced-size parity cases; the recipe is unchanged.
    """
    bh = w.bh if bh is None else bh
    n_q = w.n_q if n_q is None else n_q
    n_k = w.n_k if n_k is None else n_k
    dt = _DTYPES[dtype] if dtype is not None else w.torch_dtype
    seed = w.seed if seed is None else seed
    with_do = w.backward if with_do is None else with_do
    d = w.head_dim
    g = _generator(seed, bh * max(n_q, n_k) * d, device)
    out = {
        "q": _draw(g, (bh, n_q, d), dt, device),
        "k": _draw(g, (bh, n_k, d), dt, device, w.k_mult),
        "v": _draw(g, (bh, n_k, d), dt, device),
    }
    if with_do:
        out["do"] = _draw(g, (bh, n_q, d), dt, device)
    return out


def psa_inputs(w: PsaWorkload, device="cpu", batch: int | None = None, seed: int | None = None) -> torch.Tensor:
    """The NCHW qkv activation [B, nh*4*kd, H, W] for workload ``w``."""
    b = w.batch if batch is None else batch
    seed = w.seed if seed is None else seed
    shape = (b, w.qkv_channels, w.h, w.w)
    g = _generator(seed, b * w.qkv_channels * w.n, device)
    return _draw(g, shape, w.torch_dtype, device)
