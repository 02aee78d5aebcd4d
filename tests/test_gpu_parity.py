"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle
on the same seeded inputs.

Bars (written here, applied to every output): max-abs error <= 1e-4 for
float32 inputs, <= 2e-2 for float16 / bfloat16 inputs; PSA pack/merge are
bit-exact. Small cases span several tiles and ragged tails (key tiles are 64,
query blocks 128, dkdv key blocks 128, PSA pixel tiles 64); full-size
configurations are checked on sampled heads and rows the oracle computes one
by one, plus properties that hold at any size.
"""
import math

import numpy as np
import pytest
import torch

import attention_fa2_fwd_02_amd as fa2
import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-4, torch.float16: 2e-2, torch.bfloat16: 2e-2}
DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    fa2.load()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _err(name, got, want, tol, case):
    got = np.asarray(got, np.float64)
    e = float(np.abs(got - want).max()) if want.size else 0.0
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    rel = float(np.sqrt(np.mean((got - want) ** 2)) / rms) if rms > 0 else 0.0
    print(f"  {case} {name}: max_abs={e:.3e} rel_rms={rel:.3e} (tol {tol:g})", flush=True)
    assert np.all(np.isfinite(got)), f"{case} {name}: non-finite values"
    assert e <= tol, f"{case} {name}: max-abs {e:.3e} > {tol:g}"


def _err_bound(name, got, want, tol, mag, dtype, lse_err, case):
    """Bar for a gradient from the rounding its arithmetic prescribes. The
    backward recomputes p = exp(s - LSE) from the stored LSE, so every p
    carries a relative error of up to lse_err (the stored LSE's measured
    error, itself held to the forward's bar). For 16-bit inputs the method
    also stores O in the input type (delta = rowsum(O dO) is formed from it)
    and rounds P and dS to that type before the products dV = P^T dO,
    dQ = dS K and dK = dS^T Q (fp32 accumulation), so each term carries a
    relative error of up to u, the type's unit roundoff (2^-24 for float32).
    Hence |got - exact| <= tol + (2u + lse_err) sum|terms| + half a unit in
    the last place of the output, with `mag` that sum of term magnitudes per
    element (see _grad_term_magnitudes; 2u leaves a factor of two for the
    fp32 steps)."""
    got = np.asarray(got, np.float64)
    mant = {torch.bfloat16: 7, torch.float16: 10, torch.float32: 23}[dtype]
    u = 2.0 ** -(mant + 1)
    amag = np.maximum(np.abs(want), np.finfo(np.float64).tiny)
    half_ulp = np.exp2(np.floor(np.log2(amag)) - mant) / 2
    bar = tol + (2 * u + lse_err) * mag + half_ulp
    e = np.abs(got - want)
    worst = float((e / bar).max()) if want.size else 0.0
    print(f"  {case} {name}: max_abs={float(e.max()):.3e} max|ref|={float(np.abs(want).max()):.3g} "
          f"worst err/bar={worst:.3f} (bar {tol:g} + (2u + {lse_err:.2g}) sum|terms| + ulp/2)", flush=True)
    assert np.all(np.isfinite(got)), f"{case} {name}: non-finite values"
    assert worst <= 1.0, f"{case} {name}: error {worst:.3f} x the bar"


def _grad_term_magnitudes(q, k, v, do, o, lse, scale):
    """Per element of dQ, dK, dV, the sum of the magnitudes of the terms the
    gradient adds (fp64, from the inputs and the exact O and LSE). A dS term
    also counts p_ij sum_d |O_id dO_id|: delta_i comes from O as stored in the
    16-bit type, whose rounding moves delta_i by up to u times that sum."""
    q, k, v, do = (_np(t) for t in (q, k, v, do))
    p = np.exp(scale * np.einsum("bid,bjd->bij", q, k) - lse[:, :, None])
    dp = np.einsum("bid,bjd->bij", do, v)
    delta = np.sum(o * do, axis=-1)
    ds = np.abs(p * (dp - delta[:, :, None])) + p * np.sum(np.abs(o * do), axis=-1)[:, :, None]
    mq = scale * np.einsum("bij,bjd->bid", ds, np.abs(k))
    mk = scale * np.einsum("bij,bid->bjd", ds, np.abs(q))
    mv = np.einsum("bij,bid->bjd", p, np.abs(do))
    return mq, mk, mv


def _inputs(dt, bh, nq, nk, d, seed, k_mult=1.0, with_do=False):
    w = workloads.AttnWorkload("case", bh, nq, nk, d, dt, seed, k_mult=k_mult)
    return workloads.attn_inputs(w, device=DEV, with_do=with_do)


# n_k 64 and 128: one and two full key tiles with no ragged tail (the first tile
# runs outside the tile loop); 1 and 7: no full tile
FWD_SHAPES = [(2, 64, 64), (3, 200, 333), (2, 1, 1), (1, 129, 65), (2, 400, 400), (1, 7, 300), (1, 300, 7),
              (2, 96, 128)]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("shape", FWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_small(dt, d, shape):
    bh, nq, nk = shape
    case = f"fwd {dt} d={d} bh={bh} nq={nq} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=100 + nq + nk + d)
    scale = 1 / math.sqrt(d)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], scale)
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("shape", [(256, 100, 150), (512, 90, 130)], ids=["4waves", "8waves"])
def test_fwd_workgroup_sizes(dt, d, shape):
    """Shapes whose head count selects 4-wave (128-row) and 8-wave (256-row)
    workgroups in the plain forward, every output against the oracle (the
    small shapes above run 2-wave workgroups)."""
    bh, nq, nk = shape
    case = f"fwd {dt} d={d} bh={bh} nq={nq} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=500 + bh + d)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d))
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)


@pytest.mark.parametrize("dt,mult", [("f16", 6.0), ("bf16", 16.0), ("bf16", 1.0), ("f16", 1.0)])
def test_fwd_many_blocks_and_rerun(dt, mult):
    """The 8-wave forward (three LDS stages, K/V fetched two tiles ahead) over
    600 heads x 2 query blocks = 1200 workgroups, an uneven share per XCD,
    with 200 keys (a ragged fourth tile). With mult > 1, every 7th head has
    keys from 128 on equal to mult x its query 0, so that row's scores sit far
    above the first tile's max: f16 overflows its probabilities at mult 6,
    bf16 leaves range at mult 16, and the workgroups holding those rows redo
    their block with the exact pass. Every output against the oracle."""
    bh, nq, nk, d = 600, 300, 200, 64
    case = f"many-block fwd {dt} x{mult}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=77)
    k = x["k"].clone()
    if mult != 1.0:
        k[::7, 128:, :] = (mult * x["q"][::7, :1, :].float()).to(k.dtype)
    o, lse = fa2.fa2_fwd(x["q"], k, x["v"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], k, x["v"], 1 / math.sqrt(d))
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)


@pytest.mark.parametrize("dt,mult,nk", [("f16", 6.0, 256), ("bf16", 16.0, 256), ("bf16", 1.0, 1280),
                                        ("f16", 1.0, 512), ("bf16", 16.0, 1280)])
def test_fwd_persistent_many_blocks_and_rerun(dt, mult, nk):
    """The persistent forward (head_dim 128, 16-bit, key length a multiple of
    256, at least 512 query blocks of 256 rows): 264 heads x 2 query blocks
    (the second ragged, 44 rows) = 528 blocks over 256 workgroups, so the
    blocks per workgroup differ; 256 keys (the block's first tile and its
    last three steps only) or 1280 (the four-tile loop as well). With
    mult > 1, every 7th head has its last 64 keys equal to mult x its query
    0, far above the first tile's max: those blocks redo their rows with the
    exact pass and the block after each starts from scratch. Every output
    against the oracle."""
    bh, nq, d = 264, 300, 128
    case = f"persistent fwd {dt} x{mult} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=91 + nk)
    k = x["k"].clone()
    if mult != 1.0:
        k[::7, nk - 64:, :] = (mult * x["q"][::7, :1, :].float()).to(k.dtype)
    o, lse = fa2.fa2_fwd(x["q"], k, x["v"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], k, x["v"], 1 / math.sqrt(d))
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)


def test_fwd_c1_tiny_f32():
    w = workloads.C1
    x = workloads.attn_inputs(w, device=DEV)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], w.scale)
    _err("O", _np(o), o_ref, 1e-4, w.name)
    _err("LSE", _np(lse), lse_ref, 1e-4, w.name)


def test_fwd_single_key_passes_values_through():
    # one key: the softmax is [1], so O = V (vyre-libs tests, seq_len 1). In
    # float32 the kernel's P = 2^e with |e| an fp32 rounding error, so O = V up
    # to a few fp32 ulps; bfloat16 output rounds that back to V exactly.
    for dt in ("f32", "bf16"):
        x = _inputs(dt, 3, 77, 1, 64, seed=5)
        o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"])
        torch.cuda.synchronize()
        want = x["v"].expand(-1, 77, -1)
        if dt == "bf16":
            assert torch.equal(o, want), dt
        else:
            assert torch.allclose(o, want, rtol=1e-6, atol=0), dt
        want = (x["q"].double() @ x["k"].double().transpose(1, 2)).squeeze(-1) / 8.0
        assert torch.allclose(lse.double(), want, atol=1e-4), dt


def test_fwd_canaries_untouched():
    bh, nq, nk, d = 2, 131, 70, 64
    x = _inputs("bf16", bh, nq, nk, d, seed=7)
    pad = 4096
    obuf = torch.full((bh * nq * d + pad,), float("nan"), dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((bh * nq + pad,), float("nan"), dtype=torch.float32, device=DEV)
    o = obuf[: bh * nq * d].view(bh, nq, d)
    lse = lbuf[: bh * nq].view(bh, nq)
    fa2.fa2_fwd(x["q"], x["k"], x["v"], None, o, lse)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[bh * nq * d:]).all() and torch.isnan(lbuf[bh * nq:]).all()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("shape", [(4, 300, 500), (264, 300, 512)], ids=["per-block", "persistent"])
def test_fwd_deterministic(shape):
    # the second shape selects the persistent forward (528 query blocks)
    bh, nq, nk = shape
    x = _inputs("bf16", bh, nq, nk, 128, seed=8)
    a = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    b = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _sampled_fwd_check(w, heads, nrows, seed):
    x = workloads.attn_inputs(w, device=DEV)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    g = np.random.default_rng(seed)
    tol = TOL[w.torch_dtype]
    for hd in heads:
        rows = np.unique(np.concatenate([g.choice(w.n_q, nrows, replace=False), [0, w.n_q - 1]]))
        ridx = torch.as_tensor(rows, device=DEV)
        q = x["q"][hd].index_select(0, ridx)[None]
        o_ref, lse_ref = oracle.attention_fwd(q, x["k"][hd][None], x["v"][hd][None], w.scale)
        case = f"{w.name} head {hd} ({len(rows)} rows)"
        _err("O", _np(o[hd].index_select(0, ridx))[None], o_ref, tol, case)
        _err("LSE", _np(lse[hd].index_select(0, ridx))[None], lse_ref, tol, case)
    # properties over every row: finite, LSE >= max score is not cheap here, so
    # check the bound LSE <= log(n_k) + max_j |scale q.k_j| via Cauchy-Schwarz
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    qn = x["q"].float().norm(dim=-1)
    kn = x["k"].float().norm(dim=-1).amax(dim=-1, keepdim=True)
    assert (lse <= math.log(w.n_k) + w.scale * qn * kn + 1e-3).all()
    # |O| is bounded by the largest |V| entry of the head (convex combination)
    vmax = x["v"].float().abs().amax(dim=(1, 2))
    assert (o.float().abs().amax(dim=(1, 2)) <= vmax * (1 + 1e-2)).all()


def test_fwd_c3_llm_sampled():
    _sampled_fwd_check(workloads.C3, heads=[0, 137, 511], nrows=48, seed=3)


def test_fwd_c4_cross_attention_sampled():
    _sampled_fwd_check(workloads.C4, heads=[0, 601, 1023], nrows=48, seed=4)


# ---------------------------------------------------------------------------
# Head dims outside {32, 64, 128}: zero padding through fa2_pad_cols


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_pad_cols_bitexact(dt):
    """Padding and cropping are bit copies: the padded tensor is torch's
    zero-padded tensor, and cropping it back returns the input."""
    g = torch.Generator(device="cpu").manual_seed(61)
    x = torch.randn(3, 37, 7, generator=g).to(DTYPES[dt]).to(DEV)
    for d_out in (7, 8, 32, 100, 128):
        y = fa2.fa2_pad_cols(x, d_out)
        back = fa2.fa2_pad_cols(y, 7)
        torch.cuda.synchronize()
        want = torch.nn.functional.pad(x.cpu(), (0, max(0, d_out - 7)))[..., :d_out]
        assert torch.equal(y.cpu(), want), d_out
        assert torch.equal(back.cpu(), x.cpu()), d_out
    # crop below the input width
    z = fa2.fa2_pad_cols(x, 3)
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), x.cpu()[..., :3])


ANY_DIM_SHAPES = [(2, 64, 64), (1, 129, 70), (2, 1, 200)]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [4, 7, 8, 16, 40, 100])
@pytest.mark.parametrize("shape", ANY_DIM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_bwd_any_head_dim(dt, d, shape):
    """Head dims the kernels are not built for (the vyre-libs tests use 4, 7,
    8 and 16) through zero padding to 32 / 64 / 128: forward and backward
    against the oracle at the original head dim and scale."""
    bh, nq, nk = shape
    case = f"any-dim {dt} d={d} bh={bh} nq={nq} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=400 + nq + nk + d, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = fa2.attention_fwd(x["q"], x["k"], x["v"])
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse)
    torch.cuda.synchronize()
    assert o.shape == x["q"].shape and dk.shape == x["k"].shape
    tol = TOL[DTYPES[dt]]
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], scale)
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _err(name, _np(got), want, tol, case)


def test_vyre_trig_fixture_head_dim_16():
    """The vyre-libs tiled-versus-reference test case (tests section of
    flash_attention_2.rs): one head, 8 rows, head_dim 16, float32, inputs
    given by sines and cosines of the flat element index, scale 1/sqrt(16).
    Head_dim 16 runs padded to 32; forward and backward against the oracle
    (bar 1e-4; the page's own bar between its two implementations is 1e-3)."""
    n, d = 8, 16
    i = torch.arange(n * d, dtype=torch.float64)
    q = (torch.sin(0.13 * i) - 0.5).float().view(1, n, d)
    k = (torch.cos(0.07 * i) + 0.25).float().view(1, n, d)
    v = (2.0 * torch.sin(0.19 * i)).float().view(1, n, d)
    do = torch.cos(0.11 * i).float().view(1, n, d)
    o, lse = fa2.attention_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    dq, dk, dv = fa2.attention_bwd(q.to(DEV), k.to(DEV), v.to(DEV), o, do.to(DEV), lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(q, k, v, 0.25)
    _err("O", _np(o), o_ref, 1e-4, "vyre trig fixture")
    _err("LSE", _np(lse), lse_ref, 1e-4, "vyre trig fixture")
    ref = oracle.attention_bwd(q, k, v, do, 0.25)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _err(name, _np(got), want, 1e-4, "vyre trig fixture")


def test_vyre_constant_fixture_head_dim_7():
    """The vyre-libs output-shape test case: 5 rows, head_dim 7, q = 1,
    k = 0.5, v = 2 everywhere. All scores are equal, so O = v = 2 exactly and
    lse = scale * 7 * 0.5 + ln 5 with scale = 1/sqrt(7)."""
    n, d = 5, 7
    q = torch.full((1, n, d), 1.0, device=DEV)
    k = torch.full((1, n, d), 0.5, device=DEV)
    v = torch.full((1, n, d), 2.0, device=DEV)
    o, lse = fa2.attention_fwd(q, k, v)
    torch.cuda.synchronize()
    assert o.shape == (1, n, d)
    assert torch.allclose(o.cpu(), torch.full((1, n, d), 2.0), rtol=0, atol=1e-6)
    want = 3.5 / math.sqrt(7.0) + math.log(5.0)
    assert torch.allclose(lse.cpu().double(), torch.full((1, n), want, dtype=torch.float64), atol=1e-5)


# ---------------------------------------------------------------------------
# Key-split forward (few query rows per head)

SPLIT_SHAPES = [(4, 1, 3000), (3, 5, 1000), (2, 70, 333), (1, 130, 700), (2, 64, 64), (1, 1, 65), (2, 257, 129)]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("splits", [0, 3])
@pytest.mark.parametrize("shape", SPLIT_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fwd_splitkv_small(dt, d, splits, shape):
    bh, nq, nk = shape
    used, nbytes = fa2.fa2_fwd_splitkv_plan(DTYPES[dt], bh, nq, nk, d, splits)
    case = f"splitkv {dt} d={d} bh={bh} nq={nq} nk={nk} splits={splits}->{used}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=300 + nq + nk + d)
    scale = 1 / math.sqrt(d)
    # workspace and outputs with NaN canaries past their ends
    ws = torch.full((nbytes + 4096,), 0xFF, dtype=torch.uint8, device=DEV)
    obuf = torch.full((bh * nq * d + 256,), float("nan"), dtype=x["q"].dtype, device=DEV)
    lbuf = torch.full((bh * nq + 256,), float("nan"), dtype=torch.float32, device=DEV)
    o = obuf[: bh * nq * d].view(bh, nq, d)
    lse = lbuf[: bh * nq].view(bh, nq)
    fa2.fa2_fwd_splitkv(x["q"], x["k"], x["v"], scale, splits, ws[:max(nbytes, 16)], o, lse)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[bh * nq * d:]).all() and torch.isnan(lbuf[bh * nq:]).all()
    assert (ws[max(nbytes, 16):] == 0xFF).all()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], scale)
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)


def test_fwd_splitkv_decode_full():
    """Decoding shape at full size: 32 heads, one query row, 32768 keys,
    head_dim 128, bfloat16; every output against the oracle, and the split
    count the plan picks actually spreads the keys."""
    bh, nq, nk, d = 32, 1, 32768, 128
    used, _ = fa2.fa2_fwd_splitkv_plan(torch.bfloat16, bh, nq, nk, d, 0)
    assert used >= 8
    x = _inputs("bf16", bh, nq, nk, d, seed=31)
    o, lse = fa2.fa2_fwd_splitkv(x["q"], x["k"], x["v"])
    o1, lse1 = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(d))
    case = f"decode bh={bh} nk={nk} splits={used}"
    _err("O", _np(o), o_ref, 2e-2, case)
    _err("LSE", _np(lse), lse_ref, 2e-2, case)
    _err("O (fa2_fwd)", _np(o1), o_ref, 2e-2, case)


def test_attention_fwd_takes_the_key_split_path_for_decoding():
    """attention_fwd routes a decoding shape through the key-split forward
    (same result as fa2_fwd_splitkv, bit for bit) and a large shape through
    fa2_fwd."""
    x = _inputs("bf16", 4, 2, 9000, 128, seed=43)
    assert fa2.fa2_fwd_splitkv_plan(torch.bfloat16, 4, 2, 9000, 128, 0)[0] > 1
    o, lse = fa2.attention_fwd(x["q"], x["k"], x["v"])
    o2, lse2 = fa2.fa2_fwd_splitkv(x["q"], x["k"], x["v"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], 1 / math.sqrt(128))
    _err("O", _np(o), o_ref, 2e-2, "attention_fwd decode")
    _err("LSE", _np(lse), lse_ref, 2e-2, "attention_fwd decode")
    y = _inputs("bf16", 256, 256, 256, 64, seed=44)
    assert fa2.fa2_fwd_splitkv_plan(torch.bfloat16, 256, 256, 256, 64, 0)[0] == 1
    o, lse = fa2.attention_fwd(y["q"], y["k"], y["v"])
    o2, lse2 = fa2.fa2_fwd(y["q"], y["k"], y["v"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_fwd_splitkv_workspace_reuse():
    """Two calls in a row on one workspace, the second smaller: the second
    result does not depend on what the first left behind."""
    x = _inputs("bf16", 8, 3, 5000, 64, seed=41)
    y = _inputs("bf16", 2, 1, 700, 64, seed=42)
    ws = torch.empty(fa2.fa2_fwd_splitkv_plan(torch.bfloat16, 8, 3, 5000, 64, 0)[1], dtype=torch.uint8,
                     device=DEV)
    fa2.fa2_fwd_splitkv(x["q"], x["k"], x["v"], workspace=ws)
    o, lse = fa2.fa2_fwd_splitkv(y["q"], y["k"], y["v"], workspace=ws)
    o2, lse2 = fa2.fa2_fwd_splitkv(y["q"], y["k"], y["v"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    o_ref, lse_ref = oracle.attention_fwd(y["q"], y["k"], y["v"], 1 / 8.0)
    _err("O", _np(o), o_ref, 2e-2, "reuse")
    _err("LSE", _np(lse), lse_ref, 2e-2, "reuse")


# ---------------------------------------------------------------------------
# PSA


def test_psa_pack_merge_bitexact_c2():
    w = workloads.C2
    qkv = workloads.psa_inputs(w, device=DEV)
    packed = fa2.psa_pack_qkv(qkv, w.num_heads, w.key_dim)
    torch.cuda.synchronize()
    want = oracle.psa_pack(qkv, w.num_heads, w.key_dim)
    assert np.array_equal(packed.cpu().numpy().view(np.int16), want.view(np.int16))
    g = torch.Generator(device="cpu").manual_seed(9)
    lo = torch.randn(w.bh, w.n, w.key_dim, generator=g).to(DEV, torch.float16)
    hi = torch.randn(w.bh, w.n, w.key_dim, generator=g).to(DEV, torch.float16)
    out = fa2.psa_merge_attn(lo, hi, w.batch, w.num_heads, w.h, w.w)
    torch.cuda.synchronize()
    want = oracle.psa_merge(lo, hi, w.batch, w.num_heads, w.key_dim, w.h, w.w)
    assert np.array_equal(out.cpu().numpy().view(np.int16), want.view(np.int16))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", [(32, 2, 3, 5, 7), (64, 1, 2, 9, 9), (128, 2, 1, 4, 6), (32, 3, 2, 8, 8)])
def test_psa_pack_merge_bitexact_shapes(dt, kd, b, nh, h, w):
    dtype = DTYPES[dt]
    g = torch.Generator(device="cpu").manual_seed(kd + h * w)
    qkv = torch.randn(b, nh * 4 * kd, h, w, generator=g).to(DEV, dtype)
    packed = fa2.psa_pack_qkv(qkv, nh, kd)
    out = fa2.psa_merge_attn(packed[2], packed[3], b, nh, h, w)
    torch.cuda.synchronize()
    bits = (lambda a: a.view(np.int32)) if dt == "f32" else (lambda a: a.view(np.int16))
    cpu = lambda t: t.cpu().view(torch.int32 if dt == "f32" else torch.int16).numpy()
    assert np.array_equal(cpu(packed), bits(oracle.psa_pack(qkv, nh, kd)))
    assert np.array_equal(cpu(out), bits(oracle.psa_merge(packed[2], packed[3], b, nh, kd, h, w)))


def test_psa_block_c2():
    w = workloads.C2
    qkv = workloads.psa_inputs(w, device=DEV)
    out = fa2.psa_block(qkv, w.num_heads, w.key_dim)
    torch.cuda.synchronize()
    want = oracle.psa_block(qkv, w.num_heads, w.key_dim)
    _err("out", _np(out), want, 2e-2, w.name)


# ---------------------------------------------------------------------------
# Backward

BWD_SHAPES = [(2, 64, 64), (2, 200, 150), (1, 1, 1), (1, 129, 257), (1, 33, 31), (2, 300, 130)]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small(dt, d, shape):
    bh, nq, nk = shape
    case = f"bwd {dt} d={d} bh={bh} nq={nq} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=200 + nq + nk + d, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], scale)
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    tol = TOL[DTYPES[dt]]
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _err(name, _np(got), want, tol, case)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("shape", [(256, 100, 150), (512, 90, 130), (64, 300, 520)],
                         ids=["4waves", "8waves", "2waves-multi"])
def test_bwd_workgroup_sizes(dt, d, shape):
    """Shapes whose head count selects 4-wave (128-row) and 8-wave (256-row)
    workgroups in both dq (query rows) and dkdv (key rows), and a 2-wave
    launch with several query and key tiles per workgroup; every dQ, dK and
    dV element against the oracle (the small shapes above run 2-wave
    workgroups with one or two tiles)."""
    bh, nq, nk = shape
    case = f"bwd {dt} d={d} bh={bh} nq={nq} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=600 + bh + d, with_do=True)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], 1 / math.sqrt(d))
    tol = TOL[DTYPES[dt]]
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _err(name, _np(got), want, tol, case)


@pytest.mark.parametrize("dt,nk", [("bf16", 256), ("f16", 1280), ("bf16", 1280)])
def test_bwd_persistent_dq(dt, nk):
    """The persistent dQ (head_dim 128, 16-bit, key length a multiple of
    256, at least 512 query blocks of 256 rows): 264 heads x 2 query blocks
    (the second ragged, 44 rows) = 528 blocks over 256 workgroups, so the
    blocks per workgroup differ and the next block's rows, loaded during the
    last tile, come from another head or past the last block; 256 keys (the
    last four-step group only) or 1280 (the four-step loop as well). Every
    dQ, dK and dV element against the oracle."""
    bh, nq, d = 264, 300, 128
    case = f"persistent dq {dt} nk={nk}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=700 + nk, with_do=True)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], 1 / math.sqrt(d))
    tol = TOL[DTYPES[dt]]
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _err(name, _np(got), want, tol, case)


def test_bwd_delta_matches_rowsum():
    x = _inputs("bf16", 3, 130, 10, 128, seed=12, with_do=True)
    o = x["v"].new_empty(0)
    o = torch.randn(3, 130, 128, device=DEV).to(torch.bfloat16)
    delta = fa2.fa2_bwd_delta(o, x["do"])
    torch.cuda.synchronize()
    want = (o.double() * x["do"].double()).sum(-1)
    assert torch.allclose(delta.double(), want, atol=1e-4, rtol=1e-5)


def test_bwd_c5_sampled():
    w = workloads.C5
    x = workloads.attn_inputs(w, device=DEV)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], w.scale)
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale)
    torch.cuda.synchronize()
    heads = [0, 77, 255]
    tol = TOL[w.torch_dtype]
    for hd in heads:
        sl = slice(hd, hd + 1)
        ref = oracle.attention_bwd(x["q"][sl], x["k"][sl], x["v"][sl], x["do"][sl], w.scale)
        case = f"{w.name} head {hd}"
        for name, got, want in zip(("dQ", "dK", "dV"), (dq[sl], dk[sl], dv[sl]), ref):
            _err(name, _np(got), want, tol, case)
    # properties over every head: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
    assert dk.float().sum(1).abs().max().item() < 5e-2
    assert (dv.float().sum(1) - x["do"].float().sum(1)).abs().max().item() < 5e-2


@pytest.mark.parametrize("shape", [(2, 300, 260), (264, 300, 512)], ids=["per-block", "persistent"])
def test_bwd_deterministic(shape):
    # the second shape selects the persistent dQ (528 query blocks)
    bh, nq, nk = shape
    x = _inputs("bf16", bh, nq, nk, 128, seed=13, with_do=True)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"])
    a = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse)
    b = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse)
    torch.cuda.synchronize()
    for u, v_ in zip(a, b):
        assert torch.equal(u, v_)


# ---------------------------------------------------------------------------
# Edge cases: extreme scores, degenerate inputs at full size, maximum sizes


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_fwd_bwd_peaked_softmax(dt, d):
    """scale 8/sqrt(d): scaled scores with a spread of ~8, nearly one-hot rows;
    the reference max moves often and most probabilities underflow. dO is
    drawn like every other input, and the gradients reach ~30, where an
    absolute 2e-2 is finer than the 16-bit output can hold. O and LSE keep
    the plain bars; the gradients are held to the rounding bound of their
    arithmetic (_err_bound): for float32 that is the stored LSE's error
    carried into every p, for the 16-bit types also the rounding of O, P and
    dS to the input type."""
    bh, nq, nk = 2, 150, 333
    case = f"peaked {dt} d={d}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=300 + d, with_do=True)
    scale = 8 / math.sqrt(d)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], scale)
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], scale)
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], scale)
    mags = _grad_term_magnitudes(x["q"], x["k"], x["v"], x["do"], o_ref, lse_ref, scale)
    lse_err = float(np.abs(_np(lse) - lse_ref).max())
    for name, got, want, mag in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref, mags):
        _err_bound(name, _np(got), want, tol, mag, DTYPES[dt], lse_err, case)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("mult", [6.0, 16.0])
def test_fwd_scores_far_above_first_tile(dt, mult):
    """Keys from 128 on are mult x query 0, so query 0's scores there exceed
    the first key tile's max by about 70 (mult 6) or 190 (mult 16) in log2
    units. The forward takes the first tile's max as the reference and only
    reruns a workgroup with the per-tile max when l leaves range (always at
    mult 16; at mult 6 only where the element type cannot hold the
    probabilities, f16). Either way the result is the softmax."""
    bh, nq, nk, d = 2, 70, 300, 64
    case = f"far scores {dt} x{mult}"
    print(case, flush=True)
    x = _inputs(dt, bh, nq, nk, d, seed=91)
    k = x["k"].clone()
    k[:, 128:, :] = (mult * x["q"][:, :1, :].float()).to(k.dtype)
    o, lse = fa2.fa2_fwd(x["q"], k, x["v"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], k, x["v"], 1 / 8.0)
    tol = TOL[DTYPES[dt]]
    _err("O", _np(o), o_ref, tol, case)
    _err("LSE", _np(lse), lse_ref, tol, case)


def test_fwd_degenerate_inputs_full_length():
    """At the LLM sequence length with the 8-wave launch: Q = 0 and identical
    keys both make every row uniform, so O is the mean of V over the keys and
    LSE = scale q.k_0 + ln n_k (checked on every row, no oracle needed)."""
    bh, n, d = 32, 4096, 128
    x = _inputs("bf16", bh, n, n, d, seed=17)
    vmean = x["v"].double().mean(dim=1, keepdim=True)          # [bh, 1, d]
    # Q = 0
    q0 = torch.zeros_like(x["q"])
    o, lse = fa2.fa2_fwd(q0, x["k"], x["v"])
    torch.cuda.synchronize()
    assert (o.double() - vmean).abs().max().item() <= 2e-2
    assert (lse.double() - math.log(n)).abs().max().item() <= 1e-4
    # every key equal to key 0 of its head
    k0 = x["k"][:, :1, :].expand(-1, n, -1).contiguous()
    o, lse = fa2.fa2_fwd(x["q"], k0, x["v"])
    torch.cuda.synchronize()
    assert (o.double() - vmean).abs().max().item() <= 2e-2
    want = (x["q"].double() @ k0[:, :1, :].double().transpose(1, 2)).squeeze(-1) / math.sqrt(d) + math.log(n)
    assert (lse.double() - want).abs().max().item() <= 2e-3


def test_fwd_max_head_size():
    """One head whose K and V are just under the 2 GiB per-tensor limit of the
    ABI (n_k = 2^23 - 5 rows of 128 bf16): buffer offsets reach the top of
    their 32-bit range and the last key tile is ragged."""
    w = workloads.AttnWorkload("maxhead", 1, 4, (1 << 23) - 5, 128, "bf16", seed=19)
    x = workloads.attn_inputs(w, device=DEV)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_fwd(x["q"], x["k"], x["v"], w.scale)
    _err("O", _np(o), o_ref, 2e-2, w.name)
    _err("LSE", _np(lse), lse_ref, 2e-2, w.name)


def test_bwd_long_keys():
    """Backward over a million keys per head (ragged last tile)."""
    w = workloads.AttnWorkload("longkeys", 2, 4, (1 << 20) + 3, 64, "bf16", seed=23, backward=True)
    x = workloads.attn_inputs(w, device=DEV)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], w.scale)
    dq, dk, dv = fa2.attention_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, w.scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], w.scale)
    for name, got, want in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        _err(name, _np(got), want, 2e-2, w.name)


# ---------------------------------------------------------------------------
# Fused PSA forward (one kernel, NCHW in and out)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", [(32, 16, 4, 20, 20), (32, 2, 3, 5, 7), (64, 2, 2, 9, 9),
                                         (32, 1, 1, 1, 1), (64, 3, 1, 16, 24), (32, 2, 2, 13, 11),
                                         # whole-head kernel capacity (448 / 256 pixels) and one past it
                                         (32, 1, 2, 16, 28), (32, 1, 1, 1, 449),
                                         # whole-head kernel at 7 key blocks per head (256 < h*w <= 448):
                                         # ragged last key block, 3 and 4 workgroups per head
                                         (32, 3, 5, 12, 22), (32, 2, 3, 16, 20), (32, 4, 2, 14, 28),
                                         (32, 1, 3, 8, 55),
                                         (64, 1, 2, 16, 16), (64, 1, 1, 1, 257),
                                         # tiled kernel with 16-byte vector access (h*w % 8 == 0)
                                         (32, 1, 1, 16, 32), (64, 1, 2, 16, 24),
                                         # tiled kernel, 4-wave launch (many workgroups), aligned and not
                                         (32, 64, 4, 16, 32), (64, 64, 4, 15, 35)])
def test_psa_attn_fused(dt, kd, b, nh, h, w):
    dtype = DTYPES[dt]
    case = f"psa fused {dt} kd={kd} b={b} nh={nh} h={h} w={w}"
    print(case, flush=True)
    wl = workloads.PsaWorkload("case", b, nh, kd, h, w, dt, seed=kd + b + h * w)
    qkv = workloads.psa_inputs(wl, device=DEV)
    lse = torch.empty((b * nh, h * w), dtype=torch.float32, device=DEV)
    out = fa2.psa_attn_fused(qkv, nh, kd, lse=lse)
    torch.cuda.synchronize()
    want = oracle.psa_block(qkv, nh, kd)
    _err("out", _np(out), want, 2e-2, case)
    packed = oracle.psa_pack(qkv, nh, kd)
    pk = torch.from_numpy(packed.view(np.int16)).view(dtype)
    _, lse_ref = oracle.attention_fwd(pk[0], pk[1], pk[2], 1 / math.sqrt(kd))
    _err("LSE", _np(lse), lse_ref, 2e-2, case)
    # the four-launch block computes the same thing
    blk = fa2.psa_block(qkv, nh, kd)
    torch.cuda.synchronize()
    _err("vs block", _np(out), _np(blk), 2e-2, case)


def test_psa_attn_fused_no_lse_and_canary():
    wl = workloads.C2
    qkv = workloads.psa_inputs(wl, device=DEV)
    n = wl.batch * wl.out_channels * wl.n
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.float16, device=DEV)
    out = buf[:n].view(wl.batch, wl.out_channels, wl.h, wl.w)
    fa2.psa_attn_fused(qkv, wl.num_heads, wl.key_dim, out=out)
    torch.cuda.synchronize()
    assert torch.isnan(buf[n:]).all() and torch.isfinite(out).all()


# ---------------------------------------------------------------------------
# PSA backward: merge backward, pack backward, the composed block gradient


def _bitsof(t, dt):
    return t.cpu().view(torch.int32 if dt == "f32" else torch.int16).numpy()


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", [(32, 16, 4, 20, 20), (32, 2, 3, 5, 7), (64, 1, 2, 9, 9),
                                         (128, 2, 1, 4, 6), (32, 1, 1, 1, 1)])
def test_psa_merge_pack_backward_bitexact(dt, kd, b, nh, h, w):
    dtype = DTYPES[dt]
    case = f"psa bwd maps {dt} kd={kd} b={b} nh={nh} h={h} w={w}"
    print(case, flush=True)
    g = torch.Generator(device="cpu").manual_seed(31 + kd + h * w)
    d_out = torch.randn(b, nh * 2 * kd, h, w, generator=g).to(DEV, dtype)
    d_packed = torch.randn(4, b * nh, h * w, kd, generator=g).to(DEV, dtype)
    lo, hi = fa2.psa_merge_attn_backward(d_out, nh, kd)
    d_qkv = fa2.psa_pack_qkv_backward(d_packed, b, nh, h, w)
    torch.cuda.synchronize()
    bits = (lambda a: a.view(np.int32)) if dt == "f32" else (lambda a: a.view(np.int16))
    want_lo, want_hi = oracle.psa_merge_backward(d_out, nh, kd)
    assert np.array_equal(_bitsof(lo, dt), bits(want_lo)) and np.array_equal(_bitsof(hi, dt), bits(want_hi))
    assert np.array_equal(_bitsof(d_qkv, dt), bits(oracle.psa_pack_backward(d_packed, b, nh, h, w)))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", [(32, 2, 3, 5, 7), (64, 1, 2, 9, 9), (32, 16, 4, 20, 20)])
def test_psa_pack_backward_adds_second_qk(dt, kd, b, nh, h, w):
    """With d_qk_extra, sections 0 and 1 are the sum (in fp32, one rounding)
    of the two Q/K gradients; V sections stay a bit-exact copy."""
    dtype = DTYPES[dt]
    case = f"psa pack bwd + extra {dt} kd={kd} b={b} nh={nh} h={h} w={w}"
    print(case, flush=True)
    g = torch.Generator(device="cpu").manual_seed(41 + kd + h * w)
    d_packed = torch.randn(4, b * nh, h * w, kd, generator=g).to(DEV, dtype)
    extra = torch.randn(2, b * nh, h * w, kd, generator=g).to(DEV, dtype)
    got = fa2.psa_pack_qkv_backward(d_packed, b, nh, h, w, d_qk_extra=extra)
    torch.cuda.synchronize()
    summed = _np(d_packed).copy()
    summed[:2] += _np(extra)
    want = oracle.psa_pack_backward(summed, b, nh, h, w)
    # one rounding of the exact sum to the element type: at most half an ulp
    ulp = {torch.float32: 2.0 ** -23, torch.float16: 2.0 ** -10, torch.bfloat16: 2.0 ** -7}[dtype]
    bound = ulp * np.maximum(np.abs(want), 2.0 ** -14)
    assert np.all(np.abs(_np(got) - want) <= bound), case
    v_sec = _np(got).reshape(b, nh, 4, kd, h * w)[:, :, 2:]
    v_want = want.reshape(b, nh, 4, kd, h * w)[:, :, 2:]
    assert np.array_equal(v_sec, v_want)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", [(32, 16, 4, 20, 20), (32, 2, 3, 5, 7), (64, 1, 2, 9, 9),
                                         (32, 1, 2, 13, 11)])
def test_psa_block_backward(dt, kd, b, nh, h, w):
    dtype = DTYPES[dt]
    case = f"psa block bwd {dt} kd={kd} b={b} nh={nh} h={h} w={w}"
    print(case, flush=True)
    wl = workloads.PsaWorkload("case", b, nh, kd, h, w, dt, seed=51 + kd + h * w)
    qkv = workloads.psa_inputs(wl, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(52 + kd + h * w)
    d_out = torch.randn(b, nh * 2 * kd, h, w, generator=g).to(DEV, dtype)
    ws = {}
    fa2.psa_block(qkv, nh, kd, ws)
    d_qkv = fa2.psa_block_backward(d_out, nh, kd, ws)
    torch.cuda.synchronize()
    want = oracle.psa_block_backward(qkv, nh, kd, d_out)
    _err("d_qkv", _np(d_qkv), want, TOL[dtype], case)
    # the workspace is reused on a second call with the same shapes: same bits
    first = d_qkv.clone()
    d_qkv2 = fa2.psa_block_backward(d_out, nh, kd, ws)
    torch.cuda.synchronize()
    assert torch.equal(first, d_qkv2)


PSA_FUSED_BWD_SHAPES = [(16, 4, 20, 20), (2, 3, 5, 7), (1, 2, 8, 8), (1, 2, 5, 13), (2, 1, 16, 16),
                        (1, 1, 1, 257), (1, 2, 16, 28), (1, 1, 16, 32)]


# key_dim 64: whole-map capacities 64 and 128, aligned and not
PSA_FUSED_BWD_CASES = [(32,) + sh for sh in PSA_FUSED_BWD_SHAPES] + [
    (64, 2, 1, 5, 7), (64, 1, 3, 8, 8), (64, 2, 2, 9, 9), (64, 3, 2, 4, 30), (64, 1, 2, 8, 16)]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", PSA_FUSED_BWD_CASES, ids=lambda v: str(v))
def test_psa_attn_fused_backward(dt, kd, b, nh, h, w):
    """The fused block backward (three kernels, NCHW in and out) against the
    oracle's fp64 chain rule of the block; at key_dim 32 maps from 35 to 512
    pixels cover every whole-map capacity (64, 128, 256, 512), at key_dim 64
    maps from 35 to 128 pixels the capacities 64 and 128, each with and
    without 16-byte aligned rows. Also: delta is rowsum(out * d_out), and a
    second call gives the same bits."""
    dtype = DTYPES[dt]
    case = f"psa fused bwd {dt} kd={kd} b={b} nh={nh} h={h} w={w}"
    print(case, flush=True)
    wl = workloads.PsaWorkload("case", b, nh, kd, h, w, dt, seed=71 + h * w)
    qkv = workloads.psa_inputs(wl, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(72 + h * w)
    d_out = torch.randn(b, nh * 2 * kd, h, w, generator=g).to(DEV, dtype)
    lse = torch.empty(b * nh, h * w, dtype=torch.float32, device=DEV)
    out = fa2.psa_attn_fused(qkv, nh, kd, lse=lse)
    delta = torch.full((b * nh, h * w), float("nan"), dtype=torch.float32, device=DEV)
    d_qkv = torch.full_like(qkv, float("nan"))
    fa2.psa_attn_fused_backward(qkv, out, lse, d_out, nh, kd, d_qkv=d_qkv, delta=delta)
    torch.cuda.synchronize()
    want = oracle.psa_block_backward(qkv, nh, kd, d_out)
    _err("d_qkv", _np(d_qkv), want, TOL[dtype], case)
    rows = (out.double() * d_out.double()).view(b, nh, 2 * kd, h * w).sum(2).reshape(b * nh, h * w)
    assert torch.allclose(delta.double(), rows, atol=1e-3, rtol=1e-4), case
    again = fa2.psa_attn_fused_backward(qkv, out, lse, d_out, nh, kd)
    torch.cuda.synchronize()
    assert torch.equal(again, d_qkv), case


def test_psa_attn_fused_backward_matches_composed_path():
    """At C2, the fused backward and psa_block_backward (eight launches on the
    pages' V-split) agree within the bar."""
    w2 = workloads.C2
    qkv = workloads.psa_inputs(w2, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(81)
    d_out = torch.randn(w2.batch, w2.out_channels, w2.h, w2.w, generator=g).to(DEV, w2.torch_dtype)
    lse = torch.empty(w2.bh, w2.n, dtype=torch.float32, device=DEV)
    out = fa2.psa_attn_fused(qkv, w2.num_heads, w2.key_dim, lse=lse)
    fused = fa2.psa_attn_fused_backward(qkv, out, lse, d_out, w2.num_heads, w2.key_dim)
    ws = {}
    fa2.psa_block(qkv, w2.num_heads, w2.key_dim, ws)
    composed = fa2.psa_block_backward(d_out, w2.num_heads, w2.key_dim, ws)
    torch.cuda.synchronize()
    _err("d_qkv fused vs composed", _np(fused), _np(composed), 2e-2, "C2")


def test_psa_attn_fused_backward_rejects_unsupported():
    qkv = torch.zeros(1, 4 * 64, 4, 4, dtype=torch.float16, device=DEV)
    out = torch.zeros(1, 2 * 64, 4, 4, dtype=torch.float16, device=DEV)
    lse = torch.zeros(1, 16, dtype=torch.float32, device=DEV)
    qkv128 = torch.zeros(1, 4 * 128, 4, 4, dtype=torch.float16, device=DEV)
    out128 = torch.zeros(1, 2 * 128, 4, 4, dtype=torch.float16, device=DEV)
    with pytest.raises(fa2.Fa2Error, match="key_dim must be 32 or 64"):
        fa2.psa_attn_fused_backward(qkv128, out128, lse, out128, 1, 128)
    qkv64 = torch.zeros(1, 4 * 64, 1, 129, dtype=torch.float16, device=DEV)
    out64 = torch.zeros(1, 2 * 64, 1, 129, dtype=torch.float16, device=DEV)
    lse64 = torch.zeros(1, 129, dtype=torch.float32, device=DEV)
    with pytest.raises(fa2.Fa2Error, match="128 at key_dim 64"):
        fa2.psa_attn_fused_backward(qkv64, out64, lse64, out64, 1, 64)
    qkv = torch.zeros(1, 4 * 32, 1, 513, dtype=torch.float16, device=DEV)
    out = torch.zeros(1, 2 * 32, 1, 513, dtype=torch.float16, device=DEV)
    lse = torch.zeros(1, 513, dtype=torch.float32, device=DEV)
    with pytest.raises(fa2.Fa2Error, match="512"):
        fa2.psa_attn_fused_backward(qkv, out, lse, out, 1, 32)


def test_psa_block_backward_needs_forward_workspace():
    with pytest.raises(ValueError, match="workspace"):
        fa2.psa_block_backward(torch.zeros(1, 64, 2, 2, dtype=torch.float16, device=DEV), 1, 32, {})


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("kd,b,nh,h,w", [(32, 16, 4, 20, 20), (32, 2, 3, 5, 7), (64, 1, 2, 9, 9),
                                         (128, 2, 1, 4, 6), (32, 1, 1, 1, 1)])
def test_psa_extract_v_and_backward(dt, kd, b, nh, h, w):
    dtype = DTYPES[dt]
    case = f"psa extract_v {dt} kd={kd} b={b} nh={nh} h={h} w={w}"
    print(case, flush=True)
    g = torch.Generator(device="cpu").manual_seed(61 + kd + h * w)
    qkv = torch.randn(b, nh * 4 * kd, h, w, generator=g).to(DEV, dtype)
    v = fa2.psa_extract_v_nchw(qkv, nh, kd)
    torch.cuda.synchronize()
    bits = (lambda a: a.view(np.int32)) if dt == "f32" else (lambda a: a.view(np.int16))
    assert np.array_equal(_bitsof(v, dt), bits(oracle.psa_extract_v(qkv, nh, kd)))
    # backward adds into the V channels of an existing d_qkv, Q/K untouched
    d_v = torch.randn(b, nh * 2 * kd, h, w, generator=g).to(DEV, dtype)
    d_qkv = torch.randn(b, nh * 4 * kd, h, w, generator=g).to(DEV, dtype)
    before = _np(d_qkv)
    fa2.psa_extract_v_backward(d_v, d_qkv, nh, kd)
    torch.cuda.synchronize()
    want = before + oracle.psa_extract_v_backward(d_v, nh, kd)
    ulp = {torch.float32: 2.0 ** -23, torch.float16: 2.0 ** -10, torch.bfloat16: 2.0 ** -7}[dtype]
    got = _np(d_qkv)
    assert np.all(np.abs(got - want) <= ulp * np.maximum(np.abs(want), 2.0 ** -14)), case
    qk = lambda a: a.reshape(b, nh, 4 * kd, h * w)[:, :, :2 * kd]
    assert np.array_equal(qk(got), qk(before))
