"""Entry points replayed from a captured HIP graph.

The attention and PSA entry points launch kernels on the caller's stream and
allocate nothing when the caller passes the outputs, so a serving loop can
capture them. Each graph is replayed several times with eager work and
synchronisations in between; before every replay the outputs are cleared, and
after it they must equal the eager results bit for bit (same kernels, same
inputs).
"""
import pytest
import torch

import attention_fa2_fwd_02_amd as fa2
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _capture(fn, calls):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, outputs, expected, eager_between):
    for rep in range(3):
        for t in outputs:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(outputs, expected)):
            assert torch.equal(got, want), f"replay {rep}: output {i} differs from the eager call"
        eager_between()
        torch.cuda.synchronize()


def test_psa_attn_fused_graph_replay():
    w = workloads.C2
    qkv = workloads.psa_inputs(w, device=DEV)
    out = torch.empty((w.batch, w.out_channels, w.h, w.w), dtype=w.torch_dtype, device=DEV)
    lse = torch.empty((w.bh, w.n), dtype=torch.float32, device=DEV)
    print(f"graph psa_attn_fused {tuple(qkv.shape)}", flush=True)
    fa2.psa_attn_fused(qkv, w.num_heads, w.key_dim, out, lse)
    torch.cuda.synchronize()
    expected = [out.clone(), lse.clone()]
    g = _capture(lambda: fa2.psa_attn_fused(qkv, w.num_heads, w.key_dim, out, lse), calls=4)
    other = torch.empty_like(out)
    _replay_and_check(g, [out, lse], expected, lambda: fa2.psa_attn_fused(qkv, w.num_heads, w.key_dim, other))


@pytest.mark.parametrize("bh,n_q,n_k,d", [(4, 300, 333, 64), (264, 300, 256, 128)],
                         ids=["per-block", "persistent"])
def test_attention_fwd_bwd_graph_replay(bh, n_q, n_k, d):
    """The small shape runs one workgroup per query (or key) block; the
    second (528 query blocks of 256 rows at head_dim 128, keys a multiple of
    256) selects the persistent forward and dQ, whose workgroups walk blocks
    and keep nothing between launches."""
    print(f"graph fa2_fwd + backward bf16 bh={bh} n_q={n_q} n_k={n_k} d={d}", flush=True)
    w = workloads.AttnWorkload("graph", bh, n_q, n_k, d, "bf16", 61)
    x = workloads.attn_inputs(w, device=DEV, with_do=True)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((bh, n_q), dtype=torch.float32, device=DEV)
    delta = torch.empty_like(lse)

    def step():
        fa2.fa2_fwd(q, k, v, None, o, lse)
        fa2.fa2_bwd_delta(o, do, delta)
        fa2.fa2_bwd_dkdv(q, k, v, do, lse, delta, None, dk, dv)
        fa2.fa2_bwd_dq(q, k, v, do, lse, delta, None, dq)

    step()
    torch.cuda.synchronize()
    outputs = [o, lse, delta, dq, dk, dv]
    expected = [t.clone() for t in outputs]
    g = _capture(step, calls=2)
    o2 = torch.empty_like(o)
    _replay_and_check(g, outputs, expected, lambda: fa2.fa2_fwd(q, k, v, None, o2))
