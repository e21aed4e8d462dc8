"""Benchmark of the DSpark ancestral draft block on one MI355X.

One step = one replay of the hipGraph that holds the whole K-position block
(for B <= 128 one persistent kernel for all K positions and the proposal
kernel; other plans K fused per-position kernels, their pick launches and the
proposal kernel) over one batch of synthetic inputs already resident in HBM.

Default workload: single-request decode, B=1, K=7, V=200064, r=256, bf16
base logits -- the drafting-alone setup of the pages ("brb-nv/TensorRT-LLM
pull 27", section "Commits 1-2: fixed-shape decode", drafting-alone table).

MALL ("cold", the default): before every timed replay a 1 GiB buffer is
read, outside the timed region, so W (102 MB) does not start in the 256 MB
Infinity Cache -- as after a target-model forward, which mostly reads
weights. (A flush that writes would leave dirty lines whose write-back the
next kernel pays for.) "warm" replays back to back. A step's time is the
HIP-event time of its replay.

Prints ONE JSON line (rank 0, N=1).
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

# The HIP runtime launches a graph either from AQL packets it captured when
# the graph was instantiated (this ROCm's default) or node by node. On MI355X
# here the second is ~3.7 us faster per replay: a one-kernel graph 10.3
# against 14.0 us, the B=1 block 82 against 86 us, with the same kernels. The
# benchmark takes it unless the caller chose; it must be set before HIP starts.
os.environ.setdefault("DEBUG_CLR_GRAPH_PACKET_CAPTURE", "0")

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, AMD published peak
PAGES_B1_US = 148.0           # the pages' drafting-alone time at B=1 (GB300), context only
METRIC = "µs per K=7 draft block (V=200064) at B=1/8/44/88; % of HBM roofline"


def algorithmic_bytes(w, resident):
    """HBM bytes a block must move, in two models (both in the design notes).

    compulsory (this design): the base logits of the real rows read once, W
    read once per block by the resident plans (once per position otherwise),
    the float32 logits written, the embedding rows gathered, the tokens
    written; the proposal re-reads the logits and writes q. A kernel cannot
    move fewer bytes than these, so their rate is at most the HBM peak.

    method (the method's own model): the same with W read once per position, as
    the method defines the bias of each position. The resident plans keep W
    on chip for the whole block, so their rate under this model can exceed
    the HBM peak; it is reported, labelled, and never used as the fraction.
    """
    s_base = 2 if w.base_dtype == "bf16" else 4
    B, K, V, r = w.B, w.K, w.V, w.r
    base = w.n_real_rows * K * V * s_base
    wb = r * V * 2
    logits = B * K * V * 4
    extra = B * K * r * 2 + B * K * 4
    prop = B * K * V * (4 + 4)
    w_reads = 1 if resident else K
    if resident:    # one launch runs all K positions
        dom = base + w_reads * wb + logits + extra
    else:           # one launch per position
        dom = (base + K * wb + logits + extra) // K
    method_dom = (base + K * wb + logits + extra) // (1 if resident else K)
    return {"dominant_per_launch": dom, "proposal_per_launch": prop,
            "block": base + w_reads * wb + logits + extra + prop,
            "method_dominant_per_launch": method_dom,
            "method_block": base + K * wb + logits + extra + prop}


class Bench:
    def __init__(self, w, mall="cold", packed=True):
        import torch
        from ancestral_draft_token_amd.device import DeviceProblem
        self.torch = torch
        self.w = w
        self.mall = mall
        # W packed once for the resident kernels (dspark_pack_w), outside the
        # timed region: a weight, laid out at load time
        self.p = DeviceProblem(w, packed=packed)
        self.stream = torch.cuda.Stream()
        self.flush_buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda:0")
        self.flush_out = torch.empty((), dtype=torch.float32, device="cuda:0")
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        self.stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.stream):
            self.p.enqueue()                      # eager call before capture
            self.graph.capture_begin()
            self.p.enqueue()
            self.graph.capture_end()
        torch.cuda.synchronize()

    def flush(self):
        if self.mall == "cold":
            torch = self.torch
            torch.amax(self.flush_buf, dim=0, out=self.flush_out)   # reads 1 GiB

    def steps(self, n):
        """n timed replays; returns per-replay microseconds (HIP events on the replay stream)."""
        torch = self.torch
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        with torch.cuda.stream(self.stream):
            for i in range(n):
                self.flush()
                starts[i].record(self.stream)
                self.graph.replay()
                ends[i].record(self.stream)
        torch.cuda.synchronize()
        return [s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)]

    def kernel_times(self, reps):
        """Eager blocks with an event after every launch: mean us per launch of each kernel."""
        torch = self.torch
        from ancestral_draft_token_amd.hip_events import EventSet
        from ancestral_draft_token_amd import LAUNCH_KINDS, dspark_launch_plan
        w = self.w
        plan = dspark_launch_plan(w.B, w.K, w.V, w.r)
        names = [LAUNCH_KINDS[kind] for kind in plan]
        self.plan = plan
        times = {n: [] for n in names}
        ev = EventSet(len(names) + 1)
        try:
            for _ in range(reps):
                with torch.cuda.stream(self.stream):
                    self.flush()
                    self.p.enqueue(stream=self.stream, events=ev.handles, chunk_cols=None)
                ev.synchronize()
                for i, n in enumerate(names):
                    times[n].append(ev.elapsed_ms(i, i + 1) * 1e3)
        finally:
            torch.cuda.synchronize()
            ev.close()
        return {n: statistics.mean(v) for n, v in times.items()}


def measure_verify(w, reps=10, mall="cold"):
    """Both verification rules after one draft block of ``w``: the block's own
    tokens and proposals against targets p_k = 0.7 q_k + 0.3 softmax(noise)
    (p_K = softmax(noise)), synthetic. Mean us per call over ``reps`` calls
    (two launches each, events on the launch stream, the MALL flushed before
    each). Algorithmic bytes per row:
    - standard: the distribution the emitted token is drawn from, read once
      (p_j and q_j after a rejection, p_K after all K accepted), plus the
      2 (n + 1) probes of the acceptance tests and the K + 1 tokens written;
    - block: every p_0..p_K and q_0..q_{K-1} read once (every residual mass is
      needed before the stop is known), plus the 2 K probes and the tokens."""
    import numpy as np
    import torch
    from ancestral_draft_token_amd import (dspark_verify_block, dspark_verify_block_workspace_bytes,
                                           dspark_verify_standard, dspark_verify_workspace_bytes)
    from ancestral_draft_token_amd.device import DeviceProblem
    prob = DeviceProblem(w)
    prob.enqueue()
    torch.cuda.synchronize()
    B, K, V = w.B, w.K, w.V
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(11)
    p = torch.softmax(torch.randn((B, K + 1, V), device=dev, generator=g) * 2.0, dim=-1)
    p[:, :K] = 0.7 * prob.q + 0.3 * p[:, :K]
    p = p.contiguous()
    flush_buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    targets = "p_k = 0.7 q_k + 0.3 softmax(2 N(0,1)), p_K = softmax(2 N(0,1)), synthetic"
    res = {}
    for rule, fn, wsb in (("standard", dspark_verify_standard, dspark_verify_workspace_bytes),
                          ("block", dspark_verify_block, dspark_verify_block_workspace_bytes)):
        n = torch.empty(B, dtype=torch.int32, device=dev)
        out = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
        wb = wsb(B, K, V)
        ws = torch.empty(wb, dtype=torch.uint8, device=dev)
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            for i in range(reps + 2):
                if mall == "cold":
                    torch.amax(flush_buf, dim=0, out=flush_out)
                starts[i].record(stream)
                fn(prob.tokens, prob.q, p, prob.seed, prob.offset, B, K, V, n, out, ws, wb, stream=stream)
                ends[i].record(stream)
        torch.cuda.synchronize()
        us = [s_.elapsed_time(e) * 1e3 for s_, e in zip(starts[2:], ends[2:])]
        acc = n.cpu().numpy().astype(np.int64)
        if rule == "standard":
            row_bytes = np.where(acc < K, 8 * V, 4 * V) + 8 * (np.minimum(acc, K - 1) + 1 if K else 0) + 4 * (K + 1)
        else:
            row_bytes = np.full(B, 8 * K * V + 4 * V + 8 * K + 4 * (K + 1), dtype=np.int64)
        algo = int(row_bytes.sum())
        mean_us = statistics.mean(us)
        res[rule] = {"workload": w.name, "us": round(mean_us, 2), "accepted_mean": round(float(acc.mean()), 3),
                     "bytes": algo, "achieved_gbs": round(algo / (mean_us * 1e-6) / 1e9, 1),
                     "roofline_frac": round(algo / (mean_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "targets": targets}
    del prob, p, flush_buf
    torch.cuda.empty_cache()
    return res


ATTN_SHAPES = {
    # the drafter's windowed GQA layer at the sampler's batch sizes: 64 query /
    # 4 key-value heads of 128, a 4096-token window, K=7, a full window of
    # context (P = 8192) for every row
    "b1": dict(B=1, K=7, Hq=64, Hkv=4, W=4096, P=8192),
    "b88": dict(B=88, K=7, Hq=64, Hkv=4, W=4096, P=8192),
}


def measure_attention(name, reps=20, mall="cold", layout="bhld"):
    """The drafter's non-causal windowed block attention (one layer) on
    synthetic bf16 Q/K/V of the ``ATTN_SHAPES`` shape. Mean us per call (one
    launch from 256 (row, key/value head) pairs, two below; events on the
    launch stream, MALL flushed before each), and the mean over calls run
    back to back between one pair of events.
    Algorithmic bytes: per (row, key/value head) the K and V rows of the
    window's key range (W - 1 + K keys), plus Q read and o, lse written.
    ``layout``: the cache layout, "bhld" ([B, Hkv, L, D], each head's keys
    contiguous: the library's streaming layout) or "blhd" ([B, L, Hkv, D])."""
    import math
    import torch
    from ancestral_draft_token_amd import (DSPARK_KV_LAYOUT_BHLD, DSPARK_KV_LAYOUT_BLHD,
                                           dspark_window_attention_workspace_bytes, dspark_window_block_attention)
    c = ATTN_SHAPES[name]
    B, K, Hq, Hkv, W, P = c["B"], c["K"], c["Hq"], c["Hkv"], c["W"], c["P"]
    D, L = 128, c["P"] + c["K"]
    dev = "cuda:0"
    g = torch.Generator(device=dev).manual_seed(5)
    q = torch.randn((B, K, Hq, D), device=dev, generator=g).to(torch.bfloat16)
    shape = (B, Hkv, L, D) if layout == "bhld" else (B, L, Hkv, D)
    kc = torch.randn(shape, device=dev, generator=g).to(torch.bfloat16)
    vc = torch.randn(shape, device=dev, generator=g).to(torch.bfloat16)
    code = DSPARK_KV_LAYOUT_BHLD if layout == "bhld" else DSPARK_KV_LAYOUT_BLHD
    ctx = torch.full((B,), P, dtype=torch.int32, device=dev)
    out = torch.empty((B, K, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, K, Hq), dtype=torch.float32, device=dev)
    wb = dspark_window_attention_workspace_bytes(B, K, Hq, Hkv, D, L, W)
    ws = torch.empty(wb, dtype=torch.uint8, device=dev)
    flush_buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 2)]
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for i in range(reps + 2):
            if mall == "cold":
                torch.amax(flush_buf, dim=0, out=flush_out)
            starts[i].record(stream)
            dspark_window_block_attention(q, kc, vc, ctx, B, K, Hq, Hkv, D, L, W, 1.0 / math.sqrt(D), out, lse, ws,
                                          wb, stream=stream, layout=code)
            ends[i].record(stream)
    torch.cuda.synchronize()
    us = statistics.mean(s_.elapsed_time(e) * 1e3 for s_, e in zip(starts[2:], ends[2:]))
    # back to back: one pair of events around `reps` calls, so the ~5 us an
    # event pair costs is spread over them (the 770 MB a B=88 call reads is
    # three times the MALL, so consecutive calls still stream from HBM)
    b2b0, b2b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        b2b0.record(stream)
        for _ in range(reps):
            dspark_window_block_attention(q, kc, vc, ctx, B, K, Hq, Hkv, D, L, W, 1.0 / math.sqrt(D), out, lse, ws,
                                          wb, stream=stream, layout=code)
        b2b1.record(stream)
    torch.cuda.synchronize()
    us_b2b = b2b0.elapsed_time(b2b1) * 1e3 / reps
    keys = min(P + K, W - 1 + K)
    algo = B * Hkv * keys * D * 2 * 2 + B * K * Hq * D * 2 + B * K * Hq * (D + 1) * 4
    flops = 4 * B * K * Hq * D * keys
    del q, kc, vc, flush_buf
    torch.cuda.empty_cache()
    res = {"shape": dict(c, D=D), "cache_layout": layout, "us": round(us, 2), "bytes": algo,
           "achieved_gbs": round(algo / (us * 1e-6) / 1e9, 1),
           "roofline_frac": round(algo / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "tflops": round(flops / (us * 1e-6) / 1e12, 1), "data": "synthetic bf16 N(0,1)",
           "us_back_to_back": round(us_b2b, 2),
           "roofline_frac_back_to_back": round(algo / (us_b2b * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    # measured HBM bytes of the kernel from the committed counter summary, if
    # it was taken on the current source
    tr = attention_traffic(name, layout, mall)
    if tr is not None:
        res["traffic"] = tr
        res["traffic_frac"] = round(tr / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    return res


def attention_workload(name, layout):
    return f"window_attention_{name}_w4096_{layout}"


def attention_traffic(name, layout, mall):
    """Counter bytes per call of the single-launch attention kernel (wa_block)
    from profiles/traffic_<workload>_<mall>.json, or None (no summary, or the
    kernel source changed since it was taken)."""
    from ancestral_draft_token_amd.profiling import source_hash
    path = os.path.join(ROOT, "profiles", f"traffic_{attention_workload(name, layout)}_{mall}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_hash("window_attn.hip"):
        return None
    return int(rec["bytes_per_launch"])


def traffic_for(w, args):
    """Measured HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 counter summary for this workload (profiles/), scaled by the
    copy-kernel calibration recorded there; None if there is none."""
    from ancestral_draft_token_amd.profiling import source_hash
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}_{args.mall}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_hash():
        return None          # the kernel changed since the counters were taken
    return round(rec["bytes_per_launch"])


def cpu_baseline(w, budget_s=12.0, max_reps=50):
    """The CPU oracle, as it stands, on the same workload: whole blocks, repeated.
    It parallelises over rows (OpenMP), so it uses min(B, host threads) threads."""
    import oracle
    threads = min(w.B, oracle.max_threads())
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.draft_block(w, num_threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    return {"value": round(el / reps * 1e6, 1), "unit": "us/block", "cores": threads, "kind": "oracle",
            "host_threads": oracle.max_threads(),
            "sample": f"{reps} full block(s) of {w.name} (all {w.K} positions, V={w.V}), "
                      f"{el:.1f} s of CPU work"}


def copy_bandwidth(nbytes=512 << 20, reps=10):
    """A plain device-to-device copy of nbytes (torch), MALL flushed before each:
    (read + write bytes) / mean event time, in GB/s."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    flush_buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda:0")
    flush_out = torch.empty((), dtype=torch.float32, device="cuda:0")
    dst.copy_(src)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
    for i in range(reps):
        torch.amax(flush_buf, dim=0, out=flush_out)
        starts[i].record()
        dst.copy_(src)
        ends[i].record()
    torch.cuda.synchronize()
    us = statistics.mean(s_.elapsed_time(e) * 1e3 for s_, e in zip(starts, ends))
    del src, dst, flush_buf
    torch.cuda.empty_cache()
    return {"bytes": 2 * nbytes, "us": round(us, 2), "gbs": round(2 * nbytes / (us * 1e-6) / 1e9, 1),
            "what": f"torch copy_ of {nbytes >> 20} MiB (read + write), MALL flushed"}


def kernel_roofline(w, r, args):
    """The dominant kernel's rate against the HBM peak: compulsory bytes per
    launch over its event-timed mean duration, the counter-measured traffic
    over the same time, and the method's byte model (labelled, may exceed 1)."""
    dom_us = r["kernels_us"]["markov_bias_gumbel_argmax"]
    ab = r["bytes"]
    achieved = ab["dominant_per_launch"] / (dom_us * 1e-6) / 1e9
    traffic = traffic_for(w, args)
    method = ab["method_dominant_per_launch"] / (dom_us * 1e-6) / 1e9
    out = {"bound": "hbm", "kernel": "markov_bias_gumbel_argmax", "workload": w.name,
           "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
           "traffic_frac": (round(traffic / (dom_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                            if traffic is not None else None),
           "kernel_us": round(dom_us, 2), "bytes_per_launch": ab["dominant_per_launch"],
           "positions_per_launch": w.K if r["resident"] else 1,
           "bytes_model": ("base logits of the real rows + W once per launch + float32 logits "
                           "written + embedding rows + tokens"),
           "method_model": {"bytes_per_launch": ab["method_dominant_per_launch"],
                            "achieved": round(method, 1), "frac": round(method / HBM_PEAK_GBS, 4),
                            "note": "W counted once per position, as the method defines the bias; "
                                    "the resident plans read it once per block, so this may exceed 1"}}
    for key in ("frac", "traffic_frac"):
        if out[key] is not None and out[key] > 1.0:
            print(f"[bench] WARNING: {key} {out[key]} of {w.name} exceeds 1", file=sys.stderr, flush=True)
    return out


def measure(w, steps, warmup, mall, kernel_reps=5, packed=True):
    b = Bench(w, mall=mall, packed=packed)
    b.steps(warmup)
    torch = b.torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    us = b.steps(steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kt = b.kernel_times(kernel_reps)
    resident = 4 in b.plan
    ab = algorithmic_bytes(w, resident)
    med = statistics.median(us)
    res = {
        "us_per_block": statistics.mean(us),
        "us_median": med,
        "us_p10": sorted(us)[len(us) // 10],
        "us_p90": sorted(us)[(len(us) * 9) // 10],
        "wall_s": wall,
        "kernels_us": kt,
        "plan": b.plan,
        "resident": resident,
        "bytes": ab,
        "block_gbs": ab["block"] / (statistics.mean(us) * 1e-6) / 1e9,
        "method_block_gbs": ab["method_block"] / (statistics.mean(us) * 1e-6) / 1e9,
    }
    del b
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="b1", choices=["tiny", "b1", "b8", "b44", "b88"])
    ap.add_argument("--mall", default="cold", choices=["cold", "warm"])
    ap.add_argument("--no-sweep", action="store_true", help="skip the B=8/44/88 lines in 'also'")
    ap.add_argument("--w-layout", default="packed", choices=["packed", "plain"],
                    help="W as packed once by dspark_pack_w (default) or read from [r, V] itself")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--pmc-run", action="store_true",
                    help="for rocprofv3 --pmc: a calibration copy of known size, then a few replays")
    ap.add_argument("--attention-run", metavar="SHAPE:LAYOUT",
                    help="for rocprofv3: a calibration copy of known size, then --steps calls of the window "
                         "attention alone (SHAPE b1 or b88, LAYOUT bhld or blhd); prints their timing")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the draft-block sampler is built and measured on "
              "a single GPU (its multi-GPU sharding is a design, not code); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from ancestral_draft_token_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    w = inputs.WORKLOADS[args.workload]()
    packed = args.w_layout == "packed"
    if args.pmc_run or args.attention_run:
        from ancestral_draft_token_amd.profiling import COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        if args.attention_run:
            shape, layout = args.attention_run.split(":")
            r = measure_attention(shape, reps=max(3, args.steps), mall=args.mall, layout=layout)
            print(json.dumps({"attention": attention_workload(shape, layout), **r}), flush=True)
            return
        b = Bench(w, mall=args.mall, packed=packed)
        b.steps(max(3, args.steps))
        torch.cuda.synchronize()
        print(f"[bench] pmc run done: {w.name}", file=sys.stderr, flush=True)
        return
    print(f"[bench] {w.name}: warmup {args.warmup}, steps {args.steps}, MALL {args.mall}",
          file=sys.stderr, flush=True)
    r = measure(w, args.steps, args.warmup, args.mall, packed=packed)
    copy = copy_bandwidth()
    line = {
        "metric": METRIC,
        "value": round(r["us_per_block"], 2),
        "unit": "us/block",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["us_per_block"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": (round(r["us_per_block"] / PAGES_B1_US, 4) if args.workload == "b1" else None),
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "B_real": w.n_real_rows, "K": w.K, "V": w.V,
                   "r": w.r, "base": w.base_dtype, "mall": args.mall,
                   "graph": "one hipGraph per block", "launches": r["plan"],
                   "w_layout": args.w_layout,
                   "hip_graph_packet_capture": os.environ.get("DEBUG_CLR_GRAPH_PACKET_CAPTURE")},
        "us_median": round(r["us_median"], 2),
        "us_p10": round(r["us_p10"], 2),
        "us_p90": round(r["us_p90"], 2),
        "block_roofline_frac": round(r["block_gbs"] / HBM_PEAK_GBS, 4),
        "block_copy_frac": round(r["block_gbs"] / copy["gbs"], 4),
        "block_bytes": r["bytes"]["block"],
        "block_method_model_frac": round(r["method_block_gbs"] / HBM_PEAK_GBS, 4),
        "kernels_us": {k: round(v, 2) for k, v in r["kernels_us"].items()},
        "roofline": kernel_roofline(w, r, args),
        "copy": copy,
    }
    if not args.no_sweep:
        also = {}
        for name in ("b8", "b44", "b88"):
            if name == args.workload:
                continue
            wo = inputs.WORKLOADS[name]()
            print(f"[bench] also {wo.name}", file=sys.stderr, flush=True)
            ro = measure(wo, max(20, args.steps), max(5, args.warmup), args.mall, packed=packed)
            also[name] = {"workload": wo.name, "us_per_block": round(ro["us_per_block"], 2),
                          "us_median": round(ro["us_median"], 2),
                          "block_roofline_frac": round(ro["block_gbs"] / HBM_PEAK_GBS, 4),
                          "block_copy_frac": round(ro["block_gbs"] / copy["gbs"], 4),
                          "block_method_model_frac": round(ro["method_block_gbs"] / HBM_PEAK_GBS, 4),
                          "kernels_us": {k: round(v, 2) for k, v in ro["kernels_us"].items()},
                          "roofline": kernel_roofline(wo, ro, args)}
            del wo
        line["also"] = also
        if "b88" in also:
            line["roofline_b88"] = also["b88"]["roofline"]
        if args.mall == "cold":
            print(f"[bench] warm MALL {w.name}", file=sys.stderr, flush=True)
            rw = measure(w, max(10, args.steps // 2), 3, "warm", packed=packed)
            line["warm"] = {"workload": w.name, "mall": "warm", "us_per_block": round(rw["us_per_block"], 2),
                            "block_roofline_frac": round(rw["block_gbs"] / HBM_PEAK_GBS, 4),
                            "kernels_us": {k: round(v, 2) for k, v in rw["kernels_us"].items()}}
    # the step after the block: verification of its drafts (standard token-level
    # and block verification; each entry holds both)
    print(f"[bench] verify {w.name}", file=sys.stderr, flush=True)
    line["verify"] = {args.workload: measure_verify(w, mall=args.mall)}
    if not args.no_sweep:
        for name in ("b88",):
            if name != args.workload:
                print(f"[bench] verify {name}", file=sys.stderr, flush=True)
                line["verify"][name] = measure_verify(inputs.WORKLOADS[name](), mall=args.mall)
    # the drafter's windowed block attention (a second workload of the pages)
    # (head-major caches, the library's streaming layout; B=88 also with the
    # position-major [B, L, Hkv, D] layout)
    line["attention"] = {}
    for name in (("b1", "b88") if not args.no_sweep else ("b88",)):
        print(f"[bench] window attention {name}", file=sys.stderr, flush=True)
        line["attention"][name] = measure_attention(name, mall=args.mall)
    print("[bench] window attention b88, [B, L, Hkv, D] caches", file=sys.stderr, flush=True)
    line["attention"]["b88_blhd"] = measure_attention("b88", mall=args.mall, layout="blhd")
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
        if not args.no_sweep and args.workload != "b88":
            print("[bench] cpu baseline (oracle) b88, all host threads", file=sys.stderr, flush=True)
            line["cpu_baseline_b88"] = cpu_baseline(inputs.WORKLOADS["b88"](), budget_s=10.0, max_reps=3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
