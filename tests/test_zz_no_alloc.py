"""The allocation-free key-split forward (fa2_fwd_splitkv_noalloc, static
device scratch) against the workspace entry point fa2_fwd_splitkv on the same
inputs: two calls in a row on one stream, the second smaller, each compared
element by element (same kernels and split plan, so the results must be
identical) and the smaller one also against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import attention_fa2_fwd_02_amd as fa2
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _inputs(dt, bh, nq, nk, d, seed):
    w = workloads.AttnWorkload("noalloc", bh, nq, nk, d, dt, seed)
    return workloads.attn_inputs(w, device=DEV)


def _with_workspace(x, d, splits):
    return fa2.fa2_fwd_splitkv(x["q"], x["k"], x["v"], 1 / math.sqrt(d), num_splits=splits)


def test_noalloc_matches_workspace_entry_point_two_calls():
    assert torch.cuda.is_available()
    fa2.load()
    # first call: 4 key ranges of 2048 keys, 8.5 MB of partials in the scratch
    big = dict(dt="bf16", bh=64, nq=64, nk=8192, d=128)
    # second call: smaller, another dtype and head dim, ragged ranges
    small = dict(dt="f16", bh=6, nq=3, nk=1000, d=64)
    xb = _inputs(big["dt"], big["bh"], big["nq"], big["nk"], big["d"], seed=41)
    xs = _inputs(small["dt"], small["bh"], small["nq"], small["nk"], small["d"], seed=42)
    sb, nb = fa2.fa2_fwd_splitkv_plan(xb["q"].dtype, big["bh"], big["nq"], big["nk"], big["d"])
    ss, ns = fa2.fa2_fwd_splitkv_plan(xs["q"].dtype, small["bh"], small["nq"], small["nk"], small["d"])
    print(f"plans: big {sb} splits {nb} B, small {ss} splits {ns} B, "
          f"scratch {fa2.fa2_fwd_splitkv_noalloc_max_bytes()} B", flush=True)
    assert sb > 1 and ss > 1 and 0 < ns < nb <= fa2.fa2_fwd_splitkv_noalloc_max_bytes()

    ob, lb = torch.empty_like(xb["q"]), torch.empty(big["bh"], big["nq"], device=DEV)
    os_, ls = torch.empty_like(xs["q"]), torch.empty(small["bh"], small["nq"], device=DEV)
    ob.fill_(float("nan")), lb.fill_(float("nan")), os_.fill_(float("nan")), ls.fill_(float("nan"))
    fa2.fa2_fwd_splitkv_noalloc(xb["q"], xb["k"], xb["v"], ob, lb, 1 / math.sqrt(big["d"]))
    fa2.fa2_fwd_splitkv_noalloc(xs["q"], xs["k"], xs["v"], os_, ls, 1 / math.sqrt(small["d"]))
    wb_o, wb_l = _with_workspace(xb, big["d"], 0)
    ws_o, ws_l = _with_workspace(xs, small["d"], 0)
    torch.cuda.synchronize()
    assert torch.equal(ob, wb_o) and torch.equal(lb, wb_l), "first call differs from fa2_fwd_splitkv"
    assert torch.equal(os_, ws_o) and torch.equal(ls, ws_l), "second call differs from fa2_fwd_splitkv"

    o_ref, lse_ref = oracle.attention_fwd(xs["q"], xs["k"], xs["v"], 1 / math.sqrt(small["d"]))
    e_o = np.abs(os_.float().cpu().numpy() - o_ref).max()
    e_l = np.abs(ls.cpu().numpy() - lse_ref).max()
    print(f"small call vs oracle: O {e_o:.3e} LSE {e_l:.3e}", flush=True)
    assert e_o <= 2e-2 and e_l <= 2e-2
    # two heads of the first call against the oracle as well
    for hd in (0, 63):
        sl = slice(hd, hd + 1)
        o_ref, lse_ref = oracle.attention_fwd(xb["q"][sl], xb["k"][sl], xb["v"][sl], 1 / math.sqrt(big["d"]))
        assert np.abs(ob[sl].float().cpu().numpy() - o_ref).max() <= 2e-2
        assert np.abs(lb[sl].cpu().numpy() - lse_ref).max() <= 2e-2
