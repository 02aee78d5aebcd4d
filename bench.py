"""Benchmark of the attention hot path on one MI355X.

A step is one pass of the whole path over resident synthetic inputs at the
LLM shape (BH 512 = 16 x 32 heads, N_q = N_k = 4096, head_dim 128, bf16):
forward (fa2_fwd: O and LSE), then backward from that O and LSE with a
synthetic dO (fa2_bwd_delta, fa2_bwd_dkdv, fa2_bwd_dq). `value` is the step's
algorithmic throughput by the FLOP convention fwd = 4 BH Nq Nk D, bwd = 2.5 x
fwd. Per-kernel durations come from HIP events recorded around every launch
on the launch stream inside the timed region.

Legs measured in the same run (not part of `value`): the tiny float32
forward (BH 2, N 64, D 32), the forward alone at the LLM shape,
cross-attention (BH 1024, Nq 1024, Nk 8192, D 64, K x 3), the
backward-config step (BH 256, N 2048, D 128), the C2PSA block (pack,
attention twice, merge, and the fused kernel) warm and with L2/MALL flushed
before each call, and its backward (composed and fused), a decoding shape
(32 heads, 1 query row, 32768 keys, D 128) through the key-split forward and
the plain forward, and a reference bf16 GEMM (random and constant operands)
that shows the chip's practical dense-MFMA ceiling on random data.

Per-kernel work is reported two ways: executed MFMA work (the products a
kernel runs: forward S and P V, 4 units of BH Nq Nk D; dkdv S, dP, dV, dK, 8
units; dq S, dP, dQ, 6 units) and algorithmic work (what the FLOP convention
counts once: forward 4 units, dkdv 8, dq 2 -- its S and dP products repeat
dkdv's and are the price of the atomic-free split).

The CPU baseline times the fp64 oracle on a bounded sample of the same
workload (a few heads at full sequence length) on the host cores, and each
configuration's oracle (C1 and C2 on their full inputs, C3, C4 and C5 on a
few full-length heads) beside the GPU time of the same configuration.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention fwd/bwd TFLOP/s + % bf16 MFMA peak; PSA block fwd us/call"


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    # ten untimed steps (~0.16 s): the chip's clock under this load settles
    # only after about 0.15 s of work
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-legs", action="store_true", help="skip the other-shape legs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=0, help="oracle sample heads (0: three per thread)")
    ap.add_argument("--only", choices=["main", "c1", "c3_fwd", "c4", "c5", "c2", "decode", "gemm_ref"], default=None,
                    help="run just the main step or just one leg (for profiling one workload); prints no JSON "
                         "line unless it is the main step")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="no GPU: read the rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE outputs (run_counter_collection.csv "
                         "of a run with --calibrate-copy) and write profiles/traffic.json")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy three times (reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


class KernelTimer:
    """HIP events around each launch on the launch stream; sums per name."""

    def __init__(self, torch):
        self.torch = torch
        self.pending = []
        self.total = {}
        self.count = {}

    def run(self, name, fn, *a, **kw):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        out = fn(*a, **kw)
        e.record()
        self.pending.append((name, s, e))
        return out

    def collect(self):
        for name, s, e in self.pending:
            self.total[name] = self.total.get(name, 0.0) + s.elapsed_time(e)
            self.count[name] = self.count.get(name, 0) + 1
        self.pending.clear()

    def avg_ms(self, name):
        return self.total[name] / self.count[name]


def _traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        data = json.loads(f.read_text())
        ent = data["kernels"][kernel]
        h = hashlib.sha256()
        for src in ent["source"]:
            h.update((ROOT / src).read_bytes())
        if h.hexdigest() != ent["source_sha256"]:
            return None
        return ent["fetch_bytes"] + ent["write_bytes"]
    except (KeyError, ValueError, OSError):
        return None


def _flush_buffer(torch):
    return torch.empty(1 << 30, dtype=torch.uint8, device="cuda")


# kernels of the step (rocprofv3 kernel names, template arguments as printed)
# and the sources their code comes from
TRAFFIC_KERNELS = {
    "fwd": ("fwd_stream_kernel<(fa2mi::Dt)2, 128>", ["attention_fa2_fwd_02_amd/csrc/fa2_fwd.hip"]),
    "dkdv": ("dkdv_kernel<(fa2mi::Dt)2, 128, 32, 8>", ["attention_fa2_fwd_02_amd/csrc/fa2_bwd.hip"]),
    "dq": ("dq_stream_kernel<(fa2mi::Dt)2, 128>", ["attention_fa2_fwd_02_amd/csrc/fa2_bwd.hip"]),
    "delta": ("delta_kernel<(fa2mi::Dt)2, 128>", ["attention_fa2_fwd_02_amd/csrc/fa2_bwd.hip"]),
}


def _write_traffic(fetch_dir: str, write_dir: str):
    """profiles/traffic.json from two rocprofv3 counter runs of the step with
    --calibrate-copy: each counter's KiB per dispatch, scaled by what the same
    counter reads for the plain 1 GiB device copy of the same program."""
    import csv
    from collections import defaultdict

    def per_kernel(d):
        f = next(Path(d).rglob("*counter_collection.csv"))
        agg = defaultdict(list)
        for r in csv.DictReader(open(f)):
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    copy = [k for k in fetch if "copyBuffer" in k or "__amd_rocclr_copy" in k]
    if not copy:
        raise SystemExit("no device copy kernel in the counter run (was it taken with --calibrate-copy?)")
    ck = max(copy, key=lambda k: fetch[k])
    sf, sw = 1048576.0 / fetch[ck], 1048576.0 / write[ck]
    out = {"what": "HBM bytes per launch of each kernel of the LLM-shape step (BH 512, N 4096, D 128, bf16), from "
                   "rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the factor that maps the same "
                   "counter on a plain 1 GiB device copy to 1 GiB",
           "command_fetch": "rocprofv3 --pmc FETCH_SIZE -d <fetch_dir> -o run --output-format csv -- python3 bench.py "
                            "--steps 3 --warmup 1 --no-legs --no-cpu-baseline --calibrate-copy",
           "command_write": "rocprofv3 --pmc WRITE_SIZE -d <write_dir> -o run --output-format csv -- python3 bench.py "
                            "--steps 3 --warmup 1 --no-legs --no-cpu-baseline --calibrate-copy",
           "command_summary": "python3 bench.py --write-traffic <fetch_dir> <write_dir>",
           "copy_reference_kib": {"FETCH_SIZE": round(fetch[ck], 4), "WRITE_SIZE": round(write[ck], 4),
                                  "bytes": 1 << 30},
           "scale": {"fetch": round(sf, 4), "write": round(sw, 4)}, "kernels": {}}
    for key, (name, srcs) in TRAFFIC_KERNELS.items():
        srcs = srcs + ["attention_fa2_fwd_02_amd/csrc/fa2_device.h"]
        fk = [k for k in fetch if k.startswith("fa2mi::" + name) or name in k]
        wk = [k for k in write if k.startswith("fa2mi::" + name) or name in k]
        if not fk or not wk:
            raise SystemExit(f"kernel {name} not found in the counter runs")
        fr, wr = fetch[fk[0]], write[wk[0]]
        h = hashlib.sha256()
        for src in srcs:
            h.update((ROOT / src).read_bytes())
        out["kernels"][key] = {"kernel": name, "fetch_kib_raw": round(fr, 1), "write_kib_raw": round(wr, 1),
                               "fetch_bytes": int(fr * 1024 * sf), "write_bytes": int(wr * 1024 * sw),
                               "source": srcs, "source_sha256": h.hexdigest()}
    (ROOT / "profiles" / "traffic.json").write_text(json.dumps(out, indent=1) + "\n")
    for key, ent in out["kernels"].items():
        print(key, ent["fetch_bytes"] / 1e9, ent["write_bytes"] / 1e9)


def main():
    args = _parse()
    if args.write_traffic:
        _write_traffic(*args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards over heads with no "
              "exchange, so per-GPU throughput is the N=1 figure. Nothing was run.", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_fa2_fwd_02_amd as fa2
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa2.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    if args.only not in (None, "main"):
        print(json.dumps({"leg": args.only, **_legs(torch, fa2, workloads, dev, only=args.only)[args.only]}))
        return

    w3, w5 = workloads.C3, workloads.C5
    x = workloads.attn_inputs(w3, device=dev, with_do=True)
    q, k, v, do = x["q"], x["k"], x["v"], x["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w3.bh, w3.n_q), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sc = w3.scale

    timer = KernelTimer(torch)

    def step():
        timer.run("fwd", fa2.fa2_fwd, q, k, v, sc, o, lse)
        timer.run("delta", fa2.fa2_bwd_delta, o, do, delta)
        timer.run("dkdv", fa2.fa2_bwd_dkdv, q, k, v, do, lse, delta, sc, dk, dv)
        timer.run("dq", fa2.fa2_bwd_dq, q, k, v, do, lse, delta, sc, dq)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.pending.clear()
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timer.collect()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    fwd_fl = w3.fwd_flops()
    step_fl = fwd_fl + w3.bwd_flops()
    value = step_fl / (ms_step * 1e-3) / 1e12

    # per-kernel work per launch, in units of BH Nq Nk D flops: executed MFMA
    # work and the algorithmic share (the backward's 10 units counted once:
    # dkdv's S, dP, dV, dK products are all required, dq adds only dQ)
    nqnkd = w3.bh * w3.n_q * w3.n_k * w3.head_dim
    exec_units = {"fwd": 4.0, "dkdv": 8.0, "dq": 6.0}
    algo_units = {"fwd": 4.0, "dkdv": 8.0, "dq": 2.0}
    es = 2
    kern_bytes = {"delta": 2 * w3.bh * w3.n_q * w3.head_dim * es + w3.bh * w3.n_q * 4}
    kernels = {}
    for name in ("fwd", "delta", "dkdv", "dq"):
        ms = timer.avg_ms(name)
        ent = {"avg_ms": round(ms, 4)}
        if name in exec_units:
            tf_a = algo_units[name] * nqnkd / (ms * 1e-3) / 1e12
            tf_x = exec_units[name] * nqnkd / (ms * 1e-3) / 1e12
            ent.update({"tflops_algorithmic": round(tf_a, 1), "frac_bf16_peak_algorithmic": round(tf_a / PEAK_BF16_TFLOPS, 4),
                        "tflops_executed": round(tf_x, 1), "frac_bf16_peak_executed": round(tf_x / PEAK_BF16_TFLOPS, 4)})
        else:
            gbs = kern_bytes[name] / (ms * 1e-3) / 1e9
            ent.update({"gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)})
        kernels[name] = ent
    dom = max(("fwd", "dkdv", "dq", "delta"), key=lambda n: timer.avg_ms(n))
    dom_ms = timer.avg_ms(dom)
    if dom in exec_units:
        ach = algo_units[dom] * nqnkd / (dom_ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": _traffic(dom)}
    else:
        ach = kern_bytes[dom] / (dom_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": _traffic(dom)}
    print(f"[bench] main step {ms_step:.3f} ms, {value:.1f} TFLOP/s; kernels {kernels}", file=sys.stderr, flush=True)

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    legs = {}
    if not args.no_legs and args.only is None:
        del x, q, k, v, do, o, lse, delta, dq, dk, dv
        torch.cuda.empty_cache()
        legs = _legs(torch, fa2, workloads, dev)

    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = _cpu_baseline(w3, args.cpu_heads)
        cpu["per_config"] = _cpu_per_config(workloads, legs)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) bf16 Q, K, V, dO drawn on the device from seeded generators",
        "config": {"workload": "llm_fwd_bwd: fa2_fwd + fa2_bwd_delta + fa2_bwd_dkdv + fa2_bwd_dq",
                   "bh": w3.bh, "n_q": w3.n_q, "n_k": w3.n_k, "head_dim": w3.head_dim,
                   "scale": w3.scale, "causal": False, "parallelism": "single GPU"},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": cpu,
        "legs": legs,
        "device": {"name": props.name, "cus": props.multi_processor_count, "gcn_arch": getattr(props, "gcnArchName", "")},
    }
    print(json.dumps(out))


def _warm(torch, fn, warm_s=0.25, min_calls=3):
    """Untimed calls until about warm_s seconds of them have run. Under a
    sustained load the chip's clock settles only after about 0.15 s: the LLM
    forward took 3.66, 3.56 and 3.52 ms (medians of ten synchronized calls)
    in three consecutive rounds after three warm-up calls, and back-to-back
    calls converge to the same 3.52 ms, so a few warm-up calls time a clock
    that is still ramping."""
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _time_fn(torch, fn, reps, flush=None):
    _warm(torch, fn)
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(1)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e))
    ts.sort()
    return ts[len(ts) // 2]


def _time_batch(torch, fn, calls):
    """Average time per call of `calls` back-to-back calls between two events
    (launch latency overlapped, as in a stream of blocks)."""
    _warm(torch, fn)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(calls):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / calls


def _time_stream(torch, fn, calls, reps=3):
    """Kernel throughput of a long launch: median over `reps` batches of the
    average time per call of `calls` back-to-back calls between two events.
    The host queues each call while the previous one runs, as in the step; the
    median single call between two events is reported next to it as
    `single_call_ms`."""
    _warm(torch, fn)
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(calls):
            fn()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) / calls)
    ts.sort()
    return ts[len(ts) // 2]


def _time_graph(torch, fn, calls, reps=5):
    """Average time per call of `calls` calls captured in one HIP graph,
    median over `reps` replays (launch work done at capture, as in a
    graph-captured serving loop)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) / calls)
    ts.sort()
    del g
    return ts[len(ts) // 2]


def _legs(torch, fa2, workloads, dev, only=None):
    legs = {}
    if only in (None, "c1"):
        _leg_c1(torch, fa2, workloads, dev, legs)
    if only in (None, "c3_fwd"):
        _leg_c3(torch, fa2, workloads, dev, legs)
    if only in (None, "c4"):
        _leg_c4(torch, fa2, workloads, dev, legs)
    if only in (None, "c5"):
        _leg_c5(torch, fa2, workloads, dev, legs)
    if only in (None, "c2"):
        _leg_c2(torch, fa2, workloads, dev, legs)
    if only in (None, "decode"):
        _leg_decode(torch, fa2, workloads, dev, legs)
    if only in (None, "gemm_ref"):
        _leg_gemm_ref(torch, dev, legs)
    return legs


def _leg_decode(torch, fa2, workloads, dev, legs):
    """Decoding shape (32 heads, 1 query row, 32768 keys, D 128, bf16): the
    key-split forward against the plain forward. HBM-bound: the algorithmic
    bytes are Q, K, V, O and LSE once; K and V (537 MB) exceed the MALL, so
    back-to-back calls stream them from HBM."""
    w = workloads.DECODE
    x = workloads.attn_inputs(w, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((w.bh, w.n_q), dtype=torch.float32, device=dev)
    splits, nbytes = fa2.fa2_fwd_splitkv_plan(w.torch_dtype, w.bh, w.n_q, w.n_k, w.head_dim, 0)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    es = 2
    algo = w.bh * (2 * w.n_q * w.head_dim * es + 2 * w.n_k * w.head_dim * es + 4 * w.n_q)
    ms_split = _time_fn(torch, lambda: fa2.fa2_fwd_splitkv(x["q"], x["k"], x["v"], w.scale, 0, ws, o, lse), 20)
    ms_plain = _time_fn(torch, lambda: fa2.fa2_fwd(x["q"], x["k"], x["v"], w.scale, o, lse), 20)
    gbs = algo / (ms_split * 1e-3) / 1e9
    legs["decode"] = {"shape": [w.bh, w.n_q, w.n_k, w.head_dim], "splits": splits,
                      "splitkv_us": round(ms_split * 1e3, 2), "fa2_fwd_us": round(ms_plain * 1e3, 2),
                      "algorithmic_mb": round(algo / 1e6, 1), "splitkv_gbs": round(gbs, 1),
                      "splitkv_frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
    del x, o, lse, ws
    torch.cuda.empty_cache()
    print(f"[bench] leg decode {legs['decode']}", file=sys.stderr, flush=True)


def _leg_gemm_ref(torch, dev, legs):
    """Practical dense bf16 ceiling on this chip: the vendor GEMM (torch.matmul,
    hipBLASLt) at 8192^3 with random N(0,1) operands and with constant ones.
    Data-dependent power draw lowers the clock for random operands, so the
    random-operand rate is the one attention kernels on real data can approach."""
    n = 8192
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    a = torch.randn(n, n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    flops = 2.0 * n * n * n
    ms_rand = _time_fn(torch, lambda: torch.matmul(a, b, out=c), 10)
    a.fill_(1.0)
    b.fill_(1.0)
    ms_const = _time_fn(torch, lambda: torch.matmul(a, b, out=c), 10)
    tf_rand = flops / (ms_rand * 1e-3) / 1e12
    tf_const = flops / (ms_const * 1e-3) / 1e12
    legs["gemm_ref"] = {"shape": [n, n, n], "random_tflops": round(tf_rand, 1),
                        "random_frac_bf16_peak": round(tf_rand / PEAK_BF16_TFLOPS, 4),
                        "constant_tflops": round(tf_const, 1),
                        "constant_frac_bf16_peak": round(tf_const / PEAK_BF16_TFLOPS, 4)}
    del a, b, c
    torch.cuda.empty_cache()
    print(f"[bench] leg gemm_ref {legs['gemm_ref']}", file=sys.stderr, flush=True)


def _leg_c1(torch, fa2, workloads, dev, legs):
    """Tiny float32 forward (BH 2, N 64, D 32): launch-bound; per call alone
    (events around one call) and back to back (200 calls between two
    events)."""
    w1 = workloads.C1
    x = workloads.attn_inputs(w1, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((w1.bh, w1.n_q), dtype=torch.float32, device=dev)
    ms = _time_fn(torch, lambda: fa2.fa2_fwd(x["q"], x["k"], x["v"], w1.scale, o, lse), 50)
    ms_stream = _time_batch(torch, lambda: fa2.fa2_fwd(x["q"], x["k"], x["v"], w1.scale, o, lse), 200)
    legs["c1"] = {"us_per_call": round(ms * 1e3, 2), "us_per_call_stream": round(ms_stream * 1e3, 2),
                  "gflops_stream": round(w1.fwd_flops() / (ms_stream * 1e-3) / 1e9, 2)}
    del x, o, lse
    print(f"[bench] leg c1 {legs['c1']}", file=sys.stderr, flush=True)


def _leg_c3(torch, fa2, workloads, dev, legs):
    # forward alone at the LLM shape
    w3 = workloads.C3
    x = workloads.attn_inputs(w3, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((w3.bh, w3.n_q), dtype=torch.float32, device=dev)
    fwd3 = lambda: fa2.fa2_fwd(x["q"], x["k"], x["v"], w3.scale, o, lse)
    ms = _time_stream(torch, fwd3, 10)
    ms_single = _time_fn(torch, fwd3, 5)
    tf = w3.fwd_flops() / (ms * 1e-3) / 1e12
    legs["c3_fwd"] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "single_call_ms": round(ms_single, 4)}
    # Context, not a result: the same launch on constant inputs (Q = K =
    # 0.25, V = 0.5). The kernel runs the same instructions in the same
    # number of cycles whatever the data; what changes is the clock the chip
    # holds, which drops with the switching power of random operands. The
    # ratio of the two times is that clock ratio.
    for t, val in ((x["q"], 0.25), (x["k"], 0.25), (x["v"], 0.5)):
        t.fill_(val)
    ms_c = _time_stream(torch, fwd3, 10)
    tf_c = w3.fwd_flops() / (ms_c * 1e-3) / 1e12
    legs["c3_fwd"].update({"const_inputs_ms": round(ms_c, 4), "const_inputs_tflops": round(tf_c, 1),
                           "const_inputs_frac_bf16_peak": round(tf_c / PEAK_BF16_TFLOPS, 4),
                           "clock_ratio_const_over_random": round(ms / ms_c, 3)})
    del x, o, lse
    torch.cuda.empty_cache()
    print(f"[bench] leg c3_fwd {legs['c3_fwd']}", file=sys.stderr, flush=True)


def _leg_c4(torch, fa2, workloads, dev, legs):
    w4 = workloads.C4
    x = workloads.attn_inputs(w4, device=dev)
    o = torch.empty_like(x["q"])
    lse = torch.empty((w4.bh, w4.n_q), dtype=torch.float32, device=dev)
    fwd4 = lambda: fa2.fa2_fwd(x["q"], x["k"], x["v"], w4.scale, o, lse)
    ms = _time_stream(torch, fwd4, 10)
    ms_single = _time_fn(torch, fwd4, 5)
    tf = w4.fwd_flops() / (ms * 1e-3) / 1e12
    legs["c4"] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                  "single_call_ms": round(ms_single, 4)}
    del x, o, lse
    torch.cuda.empty_cache()
    print(f"[bench] leg c4 {legs['c4']}", file=sys.stderr, flush=True)


def _leg_c5(torch, fa2, workloads, dev, legs):
    w5 = workloads.C5
    x = workloads.attn_inputs(w5, device=dev)
    o, lse = fa2.fa2_fwd(x["q"], x["k"], x["v"], w5.scale)
    delta = torch.empty_like(lse)
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))

    def bwd():
        fa2.fa2_bwd_delta(o, x["do"], delta)
        fa2.fa2_bwd_dkdv(x["q"], x["k"], x["v"], x["do"], lse, delta, w5.scale, dk, dv)
        fa2.fa2_bwd_dq(x["q"], x["k"], x["v"], x["do"], lse, delta, w5.scale, dq)

    ms = _time_stream(torch, bwd, 10)
    ms_single = _time_fn(torch, bwd, 5)
    tf = w5.bwd_flops() / (ms * 1e-3) / 1e12
    legs["c5"] = {"ms": round(ms, 4), "tflops_counted": round(tf, 1), "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                  "single_call_ms": round(ms_single, 4)}
    del x, o, lse, delta, dq, dk, dv
    torch.cuda.empty_cache()
    print(f"[bench] leg c5 {legs['c5']}", file=sys.stderr, flush=True)


def _leg_c2(torch, fa2, workloads, dev, legs):
    w2 = workloads.C2
    qkv = workloads.psa_inputs(w2, device=dev)
    ws = {}
    fa2.psa_block(qkv, w2.num_heads, w2.key_dim, ws)
    byts = w2.algorithmic_bytes()
    total_bytes = byts["pack"] + 2 * byts["attn_each"] + byts["merge"]
    warm = _time_fn(torch, lambda: fa2.psa_block(qkv, w2.num_heads, w2.key_dim, ws), 50)
    flush = _flush_buffer(torch)
    cold = _time_fn(torch, lambda: fa2.psa_block(qkv, w2.num_heads, w2.key_dim, ws), 20, flush=flush)
    del flush
    out_f = torch.empty((w2.batch, w2.out_channels, w2.h, w2.w), dtype=w2.torch_dtype, device=dev)
    fused_warm = _time_fn(torch, lambda: fa2.psa_attn_fused(qkv, w2.num_heads, w2.key_dim, out_f), 50)
    flush = _flush_buffer(torch)
    fused_cold = _time_fn(torch, lambda: fa2.psa_attn_fused(qkv, w2.num_heads, w2.key_dim, out_f), 20, flush=flush)
    del flush
    fused_bytes = byts["fused"]  # qkv read once, out written once
    fused_stream = _time_batch(torch, lambda: fa2.psa_attn_fused(qkv, w2.num_heads, w2.key_dim, out_f), 200)
    fused_graph = _time_graph(torch, lambda: fa2.psa_attn_fused(qkv, w2.num_heads, w2.key_dim, out_f), 100)
    block_stream = _time_batch(torch, lambda: fa2.psa_block(qkv, w2.num_heads, w2.key_dim, ws), 200)
    # backward of the block (merge backward, attention backward of both
    # calls, pack backward) from the forward's workspace
    fa2.psa_block(qkv, w2.num_heads, w2.key_dim, ws)
    g = torch.Generator(device=dev)
    g.manual_seed(w2.seed + 1000)
    d_out = torch.randn((w2.batch, w2.out_channels, w2.h, w2.w), generator=g, device=dev).to(w2.torch_dtype)
    bwd_warm = _time_fn(torch, lambda: fa2.psa_block_backward(d_out, w2.num_heads, w2.key_dim, ws), 50)
    bwd_stream = _time_batch(torch, lambda: fa2.psa_block_backward(d_out, w2.num_heads, w2.key_dim, ws), 200)
    # fused backward (three kernels, NCHW in and out) from the fused forward
    lse_f = torch.empty((w2.bh, w2.n), dtype=torch.float32, device=dev)
    fa2.psa_attn_fused(qkv, w2.num_heads, w2.key_dim, out_f, lse_f)
    d_qkv = torch.empty_like(qkv)
    delta = torch.empty((w2.bh, w2.n), dtype=torch.float32, device=dev)

    def fbwd():
        fa2.psa_attn_fused_backward(qkv, out_f, lse_f, d_out, w2.num_heads, w2.key_dim, d_qkv, delta)

    fbwd_warm = _time_fn(torch, fbwd, 50)
    fbwd_stream = _time_batch(torch, fbwd, 200)
    # pack and merge alone, beside a plain device copy moving the same bytes
    # (the floor of a launch that reads and writes them once); each is timed
    # as 100 calls in one HIP graph, since a few-microsecond launch issued
    # call by call from Python is bound by the host
    packed, o2 = ws["packed"], ws["o"]
    out_m = torch.empty_like(out_f)
    pack_g = _time_graph(torch, lambda: fa2.psa_pack_qkv(qkv, w2.num_heads, w2.key_dim, packed), 100)
    merge_g = _time_graph(torch, lambda: fa2.psa_merge_attn(o2[0], o2[1], w2.batch, w2.num_heads, w2.h, w2.w,
                                                            out_m), 100)
    src_p, dst_p = torch.empty_like(qkv), torch.empty_like(qkv)
    src_m, dst_m = torch.empty_like(out_m), torch.empty_like(out_m)
    copy_pack = _time_graph(torch, lambda: dst_p.copy_(src_p), 100)
    copy_merge = _time_graph(torch, lambda: dst_m.copy_(src_m), 100)
    del src_p, dst_p, src_m, dst_m

    def gbs(nbytes, ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 1)

    rearr = {"pack_us_graph": round(pack_g * 1e3, 2), "pack_gbs": gbs(byts["pack"], pack_g),
             "pack_frac_hbm": round(byts["pack"] / (pack_g * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "copy_same_bytes_as_pack_us_graph": round(copy_pack * 1e3, 2),
             "merge_us_graph": round(merge_g * 1e3, 2), "merge_gbs": gbs(byts["merge"], merge_g),
             "merge_frac_hbm": round(byts["merge"] / (merge_g * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
             "copy_same_bytes_as_merge_us_graph": round(copy_merge * 1e3, 2)}
    legs["c2"] = {
        **rearr,
        "fused_us_per_call_stream": round(fused_stream * 1e3, 2),
        "fused_us_per_call_graph": round(fused_graph * 1e3, 2),
        "block_us_per_call_stream": round(block_stream * 1e3, 2),
        "fused_gbs_stream": round(fused_bytes / (fused_stream * 1e-3) / 1e9, 1),
        "fused_us_per_call_warm": round(fused_warm * 1e3, 2), "fused_us_per_call_cold": round(fused_cold * 1e3, 2),
        "fused_bytes": fused_bytes,
        "fused_gbs_cold": round(fused_bytes / (fused_cold * 1e-3) / 1e9, 1),
        "fused_frac_hbm_cold": round(fused_bytes / (fused_cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "us_per_call_warm": round(warm * 1e3, 2), "us_per_call_cold": round(cold * 1e3, 2),
        "bytes": total_bytes,
        "gbs_warm": round(total_bytes / (warm * 1e-3) / 1e9, 1),
        "gbs_cold": round(total_bytes / (cold * 1e-3) / 1e9, 1),
        "frac_hbm_cold": round(total_bytes / (cold * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "attn_tflops_warm": round(w2.attn_flops() / (warm * 1e-3) / 1e12, 2),
        "bwd_us_per_call_warm": round(bwd_warm * 1e3, 2),
        "bwd_us_per_call_stream": round(bwd_stream * 1e3, 2),
        "fused_bwd_us_per_call_warm": round(fbwd_warm * 1e3, 2),
        "fused_bwd_us_per_call_stream": round(fbwd_stream * 1e3, 2),
    }
    print(f"[bench] leg c2 {legs['c2']}", file=sys.stderr, flush=True)


def _cpu_baseline(w, heads_arg):
    import numpy as np
    import torch

    import oracle
    import workloads

    threads = oracle.default_threads()
    heads = heads_arg or 3 * threads  # three full-length heads per thread: ~10-20 s
    x = workloads.attn_inputs(w, device="cpu", bh=heads, with_do=True, seed=w.seed)
    print(f"[bench] cpu baseline: oracle fwd+bwd on {heads} heads, {threads} threads", file=sys.stderr, flush=True)
    q, k, v, do = (oracle._f64(x[n]) for n in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    oracle.attention_fwd(q, k, v, w.scale, threads)
    oracle.attention_bwd(q, k, v, do, w.scale, threads)
    secs = time.perf_counter() - t0
    fl = 3.5 * 4.0 * heads * w.n_q * w.n_k * w.head_dim
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(fl / secs / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle forward + backward of {heads} of the {w.bh} heads at full length "
                      f"(n_q = n_k = {w.n_q}, head_dim {w.head_dim}), bf16-rounded inputs upcast to fp64; "
                      f"{secs:.1f} s",
            "seconds": round(secs, 2), "cpu_model": cpu_model, "host": platform.node()}


def _cpu_per_config(workloads, legs):
    """The fp64 oracle per configuration on the host cores, beside the same
    configuration's GPU time from the legs: C1 and C2 on their full inputs,
    C3, C4 (forward) and C5 (backward) on the first few heads at full
    length. Speed-up = oracle seconds per head / GPU seconds per head."""
    import oracle

    threads = oracle.default_threads()
    out = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    w = workloads.C1
    x = workloads.attn_inputs(w, device="cpu")
    secs = timed(lambda: oracle.attention_fwd(x["q"], x["k"], x["v"], w.scale, threads))
    gpu_ms = legs.get("c1", {}).get("us_per_call", 0) / 1e3
    out["c1"] = {"sample": "full input", "oracle_s": round(secs, 5), "gpu_ms": gpu_ms or None,
                 "speedup": round(secs / (gpu_ms * 1e-3), 1) if gpu_ms else None}
    w = workloads.C2
    qkv = workloads.psa_inputs(w, device="cpu")
    secs = timed(lambda: oracle.psa_block(qkv, w.num_heads, w.key_dim, threads))
    gpu_ms = legs.get("c2", {}).get("us_per_call_warm", 0) / 1e3
    gpu_fused = legs.get("c2", {}).get("fused_us_per_call_warm", 0) / 1e3
    out["c2"] = {"sample": "full input (pack, attention on V_lo and V_hi, merge)", "oracle_s": round(secs, 4),
                 "gpu_ms_block": gpu_ms or None, "gpu_ms_fused": gpu_fused or None,
                 "speedup_block": round(secs / (gpu_ms * 1e-3), 1) if gpu_ms else None,
                 "speedup_fused": round(secs / (gpu_fused * 1e-3), 1) if gpu_fused else None}
    for name, w, heads, bwd, leg, key in (("c3", workloads.C3, 8, False, "c3_fwd", "ms"),
                                          ("c4", workloads.C4, 16, False, "c4", "ms"),
                                          ("c5", workloads.C5, 8, True, "c5", "ms")):
        x = workloads.attn_inputs(w, device="cpu", bh=heads, with_do=bwd, seed=w.seed)
        if bwd:  # the oracle's backward recomputes P from Q, K, V itself
            secs = timed(lambda: oracle.attention_bwd(x["q"], x["k"], x["v"], x["do"], w.scale, threads))
        else:
            secs = timed(lambda: oracle.attention_fwd(x["q"], x["k"], x["v"], w.scale, threads))
        gpu_ms = legs.get(leg, {}).get(key)
        per_head_gpu = gpu_ms * 1e-3 / w.bh if gpu_ms else None
        fl = (w.bwd_flops() if bwd else w.fwd_flops()) * heads / w.bh
        out[name] = {"sample": f"{heads} of {w.bh} heads at full length" + (" (backward)" if bwd else " (forward)"),
                     "oracle_s": round(secs, 3), "oracle_gflops": round(fl / secs / 1e9, 2),
                     "gpu_ms_all_heads": gpu_ms,
                     "speedup": round((secs / heads) / per_head_gpu, 1) if per_head_gpu else None}
    out["threads"] = threads
    print(f"[bench] oracle per config {out}", file=sys.stderr, flush=True)
    return out


if __name__ == "__main__":
    main()
