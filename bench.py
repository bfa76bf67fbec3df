"""Benchmark of the paged KV attention path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]

A step is one pass of the whole hot path over one batch: per-batch metadata,
the cache write of the new tokens (save_kv) and attention (split kernel +
merge), through the one-call entry point pka_forward_with_metadata (the
decode launch builds the metadata itself).  The headline workload is the
largest single-GPU decode batch, Qwen3-235B-shaped (one layer on one GPU:
batch 128, 64 query / 4 KV heads, head_dim 128, bf16, page size 1, seq_lens
log-uniform in [2048, 32768], 1.42 M cached tokens); --workload picks another
decode batch for the same measurement (profiling).  Inputs are resident in
HBM before timing starts.  The JSON line reports KV bytes read per step /
step time, the dominant launch against the HBM roofline (HIP events on the
stream the kernels run on), the oracle timed on the host cores, and the
other decode workloads, extend, verify and a graph-replayed step as extras.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published
METRIC = "paged decode KV-read GB/s (% HBM peak); extend TFLOP/s (% MFMA peak)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kv_bytes(layout) -> int:
    """K and V bytes of every cached token (key width + value width per head)."""
    spec = layout.spec
    eb = {"f32": 4, "bf16": 2, "fp8": 1}[spec.kv_dtype]
    return int(layout.total_tokens) * spec.num_kv_heads * (spec.head_dim + spec.value_dim) * eb


def decode_algorithmic_bytes(layout) -> int:
    """KV read + Q read + O write + index buffers (kv_indices, indptr, last_page_len)."""
    spec = layout.spec
    qb = {"f32": 4, "bf16": 2}[spec.q_dtype]
    qo = layout.batch * spec.num_q_heads * (spec.head_dim + spec.value_dim) * qb
    idx = 4 * (layout.kv_pages + 2 * layout.batch + 1)
    return kv_bytes(layout) + qo + idx


def extend_flops(layout) -> float:
    """2 * (Dk + Dv) * Hq * (causally valid query/key pairs): q.k over the key
    width and p.v over the value width, 2 flops per MAC."""
    spec = layout.spec
    pairs = 0
    for L, n in zip(layout.seq_lens.tolist(), layout.extend_lens.tolist()):
        p = L - n
        pairs += n * p + n * (n + 1) // 2
    return 2.0 * (spec.head_dim + spec.value_dim) * spec.num_q_heads * pairs


def code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed: a
    change to comments or layout alone leaves the kernel, and this, the same."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            k = text.find("*/", i + 2)
            i = n if k < 0 else k + 2
            out.append(" ")
        elif c in "\"'":
            k = i + 1
            while k < n and text[k] != c:
                k += 2 if text[k] == "\\" else 1
            out.append(text[i:k + 1])
            i = k + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(*names) -> str:
    """Hash of the kernel sources' code (comments and layout aside) plus the
    build flags: what decides the compiled kernels."""
    from paged_kv_attention_02_amd import build as pkb
    h = hashlib.sha256(" ".join(pkb.HIPCC_FLAGS).encode())
    for n in names:
        with open(os.path.join(ROOT, "paged_kv_attention_02_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str, src_hash: str):
    """Counter-derived HBM bytes per launch, if measured on the current source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def time_events(fn, iters: int, warm: int = 2):
    """Average ms per call of fn() from HIP events on the current stream."""
    import torch
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(iters):
        fn(i)
    stop.record()
    stop.synchronize()
    return start.elapsed_time(stop) / iters


def time_per_call(fn, iters: int, warm: int = 2):
    """Median and min ms per call from one HIP event pair around each call."""
    import torch
    for _ in range(warm):
        fn(0)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": round(ms[len(ms) // 2], 4), "min": round(ms[0], 4)}


def _smi_sample():
    """(mean gfx clock MHz over the XCDs, socket power W) from amd-smi, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"], capture_output=True,
                           text=True, timeout=20)
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = [v["clk"]["value"] for k, v in g["clock"].items()
               if k.startswith("gfx") and isinstance(v.get("clk", {}).get("value"), (int, float))]
        pw = g["power"]["socket_power"]["value"]
        return (sum(clk) / len(clk), float(pw)) if clk else None
    except Exception:
        return None


def gpu_state_under(fn, seconds: float = 1.5):
    """Run fn(i) back to back for about `seconds` while amd-smi (a child
    process) samples the gfx clock and socket power; medians of the samples."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        time.sleep(0.25)
        while not stop.is_set():
            s_ = _smi_sample()
            if s_ is None:
                return
            samples.append(s_)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    if not samples:
        return None
    clk = sorted(c for c, _ in samples)
    pw = sorted(p for _, p in samples)
    return {"gfx_clock_MHz": round(clk[len(clk) // 2]), "socket_power_W": round(pw[len(pw) // 2]),
            "samples": len(samples)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layout, values, budget_s: float = 20.0):
    """The oracle (fp64, OpenMP) on whole requests of the same workload until
    about budget_s of work; reported in the same unit as the GPU value."""
    import numpy as np
    from tests.oracle_ref import oracle_requests
    import oracle
    threads = len(os.sched_getaffinity(0))
    order = list(range(layout.batch))
    done, kv, t_total = [], 0, 0.0
    spec = layout.spec
    eb = {"f32": 4, "bf16": 2, "fp8": 1}[spec.kv_dtype]
    for b in order:
        t0 = time.perf_counter()
        oracle_requests(layout, values, [b], threads=threads)
        t_total += time.perf_counter() - t0
        done.append(b)
        kv += int(layout.seq_lens[b]) * spec.num_kv_heads * (spec.head_dim + spec.value_dim) * eb
        if t_total >= budget_s:
            break
    return {"value": round(kv / t_total / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(done)} of {layout.batch} requests ({sum(int(layout.seq_lens[b]) for b in done)} "
                      f"cached tokens), all {spec.num_q_heads} heads, fp64 C oracle, "
                      f"{oracle.max_threads()} OpenMP threads, wall {t_total:.2f} s incl. "
                      f"per-request cache repacking",
            "cpu": cpu_model()}


def cpu_baseline_extend(layout, values, budget_s: float = 10.0, stride: int = 8):
    """The oracle on a bounded sample of the extend workload: every stride-th
    new token of whole requests, all heads, until about budget_s of work;
    GFLOP/s with the same causal flop count as the GPU figure."""
    from tests.oracle_ref import oracle_requests
    import oracle
    threads = len(os.sched_getaffinity(0))
    spec = layout.spec
    flops, t_total, toks, reqs = 0.0, 0.0, 0, 0
    for b in range(layout.batch):
        L, n = int(layout.seq_lens[b]), int(layout.extend_lens[b])
        p = L - n
        ts = list(range(0, n, stride))
        t0 = time.perf_counter()
        oracle_requests(layout, values, [b], tokens=lambda nb, ts=ts: ts, threads=threads)
        t_total += time.perf_counter() - t0
        flops += sum(2.0 * (spec.head_dim + spec.value_dim) * spec.num_q_heads * (p + i + 1) for i in ts)
        toks += len(ts)
        reqs += 1
        if t_total >= budget_s:
            break
    return {"value": round(flops / t_total / 1e9, 3), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"every {stride}th new token of {reqs} of {layout.batch} requests ({toks} query tokens, "
                      f"all {spec.num_q_heads} heads), fp64 C oracle, {oracle.max_threads()} OpenMP threads, "
                      f"wall {t_total:.2f} s incl. per-request cache repacking",
            "cpu": cpu_model()}


def bench_decode_kernel(spec, iters: int, warm: int = 10):
    """Decode figures for one workload on two copies of pools and metadata
    used alternately (as for the headline batch): attn_decode alone on
    prebuilt metadata, and the whole step as one call and as two."""
    import torch
    import workloads
    from tests.gpu_problem import GpuProblem
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    probs = [GpuProblem(layout, values), GpuProblem(layout, values)]
    for p in probs:
        p.attention_step(save=True)
    torch.cuda.synchronize()
    ms = time_events(lambda i: probs[i % 2].attention_step(save=False, lse=False), iters, warm=warm)
    # the whole step (metadata, cache write, decode, merge) as one call and
    # as two (init_metadata, then forward)
    ms_step = time_events(lambda i: probs[i % 2].fused_step(), iters, warm=warm)
    ms_two = time_events(lambda i: probs[i % 2].step(), iters, warm=warm)
    for p in probs:
        assert p.md.status() == 0, "device status flags set"
    nbytes = decode_algorithmic_bytes(layout)
    kvb = kv_bytes(layout)
    out = {"workload": layout.spec.name, "kv_tokens": layout.total_tokens,
           "ms": round(ms, 4), "kv_read_GBps": round(kvb / ms / 1e6, 1),
           "algorithmic_GBps": round(nbytes / ms / 1e6, 1),
           "frac_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
           "step_ms": round(ms_step, 4), "step_kv_read_GBps": round(kvb / ms_step / 1e6, 1),
           "two_call_step_ms": round(ms_two, 4)}
    del probs
    torch.cuda.empty_cache()
    return out


def bench_verify(spec, iters: int, warm: int = 10):
    """Speculative verify (target_verify batches, n chained draft tokens per
    request) through both paths the dispatch can take: the decode path
    (speculative attention mode decode: the split-K multi-query decode kernel
    + merge) and the extend path (mode prefill).  Two copies of pools and
    metadata are used alternately.  The context is created for the batch's
    draft count (max_q_per_request = n, as a server configures its number of
    speculative tokens), which sizes the partial workspace and the merge.
    GB/s counts each cached token's K and V once."""
    import torch
    import workloads
    import paged_kv_attention_02_amd as pka
    from tests.gpu_problem import GpuProblem
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    probs = []
    max_q = int(max(layout.extend_lens))
    for _ in range(2):
        p = GpuProblem(layout, values, max_q_per_request=max_q)
        p.mode = "target_verify"
        p.md = pka.Batch(p.ctx, "target_verify", layout.batch, layout.num_q_tokens, layout.kv_pages)
        p.metadata_step()
        probs.append(p)
    torch.cuda.synchronize()
    kvb = kv_bytes(layout)
    n = sorted(set(int(x) for x in layout.extend_lens))
    out = {"workload": spec.name, "kv_tokens": layout.total_tokens, "q_tokens": layout.num_q_tokens,
           "draft_tokens_per_request": n[0] if len(n) == 1 else n, "max_q_per_request": max_q}
    for path, mode in (("decode_path", "decode"), ("extend_path", "prefill")):
        call = lambda i, m=mode: probs[i % 2].attention_step(save=False, spec_mode=m, lse=False)
        ms = time_events(call, iters, warm=warm)
        out[path] = {"ms": round(ms, 4), "kv_read_GBps": round(kvb / ms / 1e6, 1),
                     "frac_hbm_peak": round(kvb / ms / 1e6 / HBM_PEAK_GBS, 4)}
    out["extend_path"]["variant"] = probs[0].ctx.describe("target_verify", layout.batch, layout.num_q_tokens)
    out["metadata_ms"] = round(time_events(lambda i: probs[i % 2].metadata_step(), iters, warm=warm), 4)
    for p in probs:
        assert p.md.status() == 0, "device status flags set"
    del probs
    torch.cuda.empty_cache()
    return out


def bench_verify_drafts(iters: int):
    """bench_verify on the Llama-shaped verify batch with 4 and 8 chained
    draft tokens per request (contexts of 512-4096 tokens)."""
    import workloads
    out = {}
    for n_draft in (4, 8):
        vs = workloads.EXTRA["llama3_8b_verify"]
        vs = vs.replace(name=vs.name.replace("_n4", f"_n{n_draft}"), new_len_args=(n_draft, n_draft),
                        prefix_len_args=(512 - n_draft, 4096 - n_draft))
        out[f"n{n_draft}"] = bench_verify(vs, iters)
        log(f"verify, {n_draft} draft tokens: {out[f'n{n_draft}']}")
    # a small batch (4 requests of 8,192 tokens, 8 drafts): too few extend
    # items to fill the chip, so the extend path cuts their key ranges
    vs = workloads.EXTRA["llama3_8b_verify"]
    vs = vs.replace(name=vs.name.replace("_b64", "_b4").replace("_n4", "_n8"), batch=4, new_len_args=(8, 8),
                    prefix_len_args=(8184, 8184))
    out["small_b4_n8"] = bench_verify(vs, iters)
    log(f"verify, 4 requests x 8 draft tokens: {out['small_b4_n8']}")
    return out


def bench_graph_step(spec, iters: int, per_graph: int = 8):
    """The Llama-shaped step (one forward_with_metadata call with the cache
    write) captured in HIP graphs and replayed, against the same steps
    launched eagerly: one graph per copy of pools and metadata holding one
    step, replayed alternately, and one graph holding `per_graph` steps
    (alternating the copies, as one captured decode step holds the attention
    of many layers).  Replays of a graph start ~9 us after the previous one
    ends (kernel trace), so the per-step figure of the many-step graph shows
    how that launch cost amortises."""
    import torch
    import workloads
    from tests.gpu_problem import GpuProblem
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    probs = [GpuProblem(layout, values), GpuProblem(layout, values)]

    def capture(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    graphs = [capture(lambda p=p: p.fused_step()) for p in probs]
    multi = capture(lambda: [probs[i % 2].fused_step() for i in range(per_graph)])
    torch.cuda.synchronize()
    ms_graph = time_events(lambda i: graphs[i % 2].replay(), iters, warm=10)
    ms_multi = time_events(lambda i: multi.replay(), max(2, iters // per_graph), warm=2) / per_graph
    ms_eager = time_events(lambda i: probs[i % 2].fused_step(), iters, warm=10)
    for p in probs:
        assert p.md.status() == 0, "device status flags set"
    kvb = kv_bytes(layout)
    out = {"workload": spec.name, "ms_per_step_graph": round(ms_graph, 4),
           "ms_per_step_eager": round(ms_eager, 4),
           f"ms_per_step_graph_of_{per_graph}_steps": round(ms_multi, 4),
           "kv_read_GBps_graph": round(kvb / ms_graph / 1e6, 1),
           "kv_read_GBps_eager": round(kvb / ms_eager / 1e6, 1),
           f"kv_read_GBps_graph_of_{per_graph}_steps": round(kvb / ms_multi / 1e6, 1)}
    del graphs, multi, probs
    torch.cuda.empty_cache()
    return out


# Untimed extend calls before timing: the matrix cores' clock takes ~10 ms of
# sustained MFMA load to settle (the first 20 calls run ~12% slower).
EXTEND_WARM = 20


def bench_extend(iters: int, gpu_state: bool = True, kv_dtype: str = "bf16", spec=None,
                 warm: int = EXTEND_WARM, constant: bool = False):
    """Extend TFLOP/s on one workload.  constant: Q, K and V all 1/16 instead
    of N(0,1) -- the same instruction stream with operand bits that barely
    toggle, so the clock is not held down by the power limit (a diagnostic
    beside the bf16 GEMM reference, never the headline figure)."""
    import torch
    import workloads
    from tests.gpu_problem import GpuProblem
    spec = workloads.WORKLOADS["llama3_8b_extend"] if spec is None else spec
    if kv_dtype != spec.kv_dtype:
        spec = spec.replace(name=spec.name.replace("extend_bf16", f"extend_{kv_dtype}kv"), kv_dtype=kv_dtype)
    layout = workloads.make_layout(spec)
    values = workloads.make_values(layout, device="cuda")
    if constant:
        for t in (values.q, values.k_all, values.v_all):
            t.fill_(0.0625)
    prob = GpuProblem(layout, values)
    prob.attention_step(save=True)
    torch.cuda.synchronize()
    call = lambda i: prob.attention_step(save=False, lse=False)
    ms = time_events(call, iters, warm=warm)
    fl = extend_flops(layout)
    tf = fl / ms / 1e9
    spec = layout.spec
    out = {"workload": spec.name, "q_tokens": layout.num_q_tokens,
           "kv_tokens": layout.total_tokens, "gflop": round(fl / 1e9, 2), "ms": round(ms, 4),
           "TFLOPs": round(tf, 1), "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
           "frac_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
           "ms_per_call": time_per_call(call, iters), "warmup_calls": warm,
           "metadata_ms": round(time_events(lambda i: prob.metadata_step(), iters), 4),
           "variant": f"extend_mfma_kernel<Dk {spec.head_dim}, Dv {spec.value_dim}, scale>0, "
                      f"page {spec.page_size}{' >= 64' if spec.page_size >= 64 else ' < 64'}, "
                      f"{spec.kv_dtype} cache>"}
    if gpu_state:
        out["gpu_state"] = gpu_state_under(call)
    del prob
    torch.cuda.empty_cache()
    return out


def bench_gemm(iters: int, n: int = 8192):
    """A square bf16 GEMM through the vendor library (torch.matmul), on
    N(0,1) operands and on constant operands: what the matrix cores sustain
    on this chip with data like the attention operands (the sustained clock
    under MFMA load depends on the operand bits)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(7)
    out = {"workload": f"bf16 GEMM {n}x{n}x{n} (torch.matmul)", "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS}
    for kind in ("random", "constant"):
        if kind == "random":
            a = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16).contiguous()
            b = torch.randn((n, n), generator=g, device="cuda").to(torch.bfloat16).contiguous()
        else:
            a = torch.ones((n, n), device="cuda", dtype=torch.bfloat16)
            b = torch.ones((n, n), device="cuda", dtype=torch.bfloat16)
        c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
        ms = time_events(lambda i: torch.matmul(a, b, out=c), iters)
        out[f"{kind}_TFLOPs"] = round(2.0 * n ** 3 / ms / 1e9, 1)
        del a, b, c
    torch.cuda.empty_cache()
    return out


def bench_copy(iters: int, nbytes: int = 1 << 30):
    """A plain device copy of known size: the reference for scaling HBM
    traffic counters (FETCH_SIZE / WRITE_SIZE) into bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    ms = time_events(lambda i: dst.copy_(src), iters)
    return {"workload": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
            "ms": round(ms, 4), "GBps_read_plus_write": round(2 * nbytes / ms / 1e6, 1)}


# Untimed run of a step before its warm-up steps (seconds).
SETTLE_S = 0.25

# The workload the headline line is quoted on: the largest single-GPU decode
# batch (Qwen3-235B-shaped, one layer on one GPU, 1.42 M cached tokens).
HEADLINE = "qwen3_235b_decode"


def traffic_key(spec_name: str) -> str:
    """Key of a decode workload's step launch in profiles/traffic.json."""
    return "decode_step:" + spec_name


def bench_decode_step(spec, steps: int, warmup: int, extras: bool) -> dict:
    """The whole step on one decode workload: per-batch metadata, the cache
    write of the new tokens and attention (split kernel + merge), through the
    one-call entry point pka_forward_with_metadata, on two copies of pools
    and metadata used alternately (so the 256 MB Infinity Cache cannot serve
    one step's KV from the previous step).  Returns the step time, the same
    step as two calls, and the roofline record of the dominant launch."""
    import torch
    import workloads
    from tests.gpu_problem import GpuProblem
    layout = workloads.make_layout(spec)
    log(f"workload {spec.name}: B={layout.batch} tokens={layout.total_tokens} pages={layout.kv_pages}")
    values = workloads.make_values(layout, device="cuda")
    probs = [GpuProblem(layout, values), GpuProblem(layout, values)]
    torch.cuda.synchronize()

    def timed_steps(step):
        # settle: the first ~50 ms of launches after the inputs are generated
        # run up to 15% slower (the GPU leaving its idle state); run the step
        # untimed for SETTLE_S, then the warm-up steps, then the timed ones
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 < SETTLE_S:
            step(i)
            i += 1
            if i % 16 == 0:
                torch.cuda.synchronize()
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    ms_step = timed_steps(lambda i: probs[i % 2].fused_step())
    kvb = kv_bytes(layout)
    for p in probs:
        assert p.md.status() == 0, "device status flags set"
    log(f"{spec.name}: step {ms_step:.4f} ms -> {kvb / ms_step / 1e6:.1f} GB/s KV read")
    # the same step as two calls: the metadata kernel, then the forward
    ms_two = timed_steps(lambda i: probs[i % 2].step())
    for p in probs:
        assert p.md.status() == 0, "device status flags set"
    # dominant kernel: the step's decode launch (metadata built in the kernel)
    # + the merge, HIP events on the stream they run on
    attn_call = lambda i: probs[i % 2].fused_step(save=False, lse=False)
    ms_attn = time_events(attn_call, steps)
    attn_dist = time_per_call(attn_call, steps)
    attn_state = gpu_state_under(attn_call) if extras else None
    # the plain attn_decode call on metadata built beforehand, and the
    # metadata kernel alone
    ms_plain = time_events(lambda i: probs[i % 2].attention_step(save=False, lse=False), steps)
    ms_meta = time_events(lambda i: probs[i % 2].metadata_step(), steps)
    nbytes = decode_algorithmic_bytes(layout)
    achieved = nbytes / (ms_attn * 1e-3) / 1e9
    src = source_hash("decode.hip", "pka_internal.h", "fp8.h")
    ctx = probs[0].ctx
    variant = ctx.describe("decode", layout.batch, layout.num_q_tokens, with_metadata=True)
    roof = {"bound": "hbm",
            "kernel": "decode_mfma_kernel (metadata built in-kernel) + decode_merge_kernel "
                      "(one forward_with_metadata call, no cache write)",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profiles(traffic_key(spec.name), src),
            "bytes_per_launch": nbytes, "ms_per_launch": round(ms_attn, 4),
            "ms_per_launch_per_call": attn_dist,
            "variant": variant,
            "gpu_state": attn_state,
            "source_hash": src}
    if roof["traffic"]:
        roof["traffic_over_algorithmic"] = round(roof["traffic"] / nbytes, 4)
    log(f"{spec.name}: forward_with_metadata {ms_attn:.4f} ms -> {achieved:.1f} GB/s "
        f"({100 * achieved / HBM_PEAK_GBS:.1f}% of peak); attn_decode {ms_plain:.4f} ms; metadata {ms_meta:.4f} ms")
    log(f"{spec.name}: resolved variant: {variant}")
    out = {"layout": layout, "values": values, "ms_step": ms_step, "kv_bytes": kvb,
           "value": kvb / (ms_step * 1e-3) / 1e9,
           "config": {"workload": spec.name, "batch": layout.batch, "num_q_heads": spec.num_q_heads,
                      "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
                      "page_size": spec.page_size, "kv_dtype": spec.kv_dtype,
                      "kv_tokens": layout.total_tokens, "kv_bytes_per_step": kvb, "seed": spec.seed,
                      "step": "forward_with_metadata(save_kv_cache=True): one decode launch builds the "
                              "metadata, writes the new tokens and attends, then the merge",
                      "two_call_step_ms": round(ms_two, 4),
                      "two_call_step_GBps": round(kvb / ms_two / 1e6, 1),
                      "attn_decode_ms": round(ms_plain, 4),
                      "metadata_ms": round(ms_meta, 4)},
           "roofline": roof}
    del probs
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=["qwen3_235b_decode", "llama3_8b_decode", "long_fp8_decode", "l4_log_decode"],
                    help="decode workload of the headline step (default: the Qwen3-235B-shaped batch)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extend / other decode figures and the clock and power sampling")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work")
    ap.add_argument("--only", choices=["extend", "extend_fp8", "qwen3_235b_decode", "llama3_8b_decode",
                                       "long_fp8_decode", "l4_log_decode", "copy", "gemm",
                                       "asym_extend", "asym_decode", "verify", "graph"], default=None,
                    help="run one extra leg alone (for profiling) and print its figures")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the attention path here is "
              "a single-GPU kernel library and no multi-GPU figure is produced.", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    import paged_kv_attention_02_amd as pka
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pka.lib()  # fail loudly if the library is missing
    all_specs = dict(workloads.WORKLOADS, **workloads.EXTRA)
    if args.only:
        if args.only == "copy":
            res = bench_copy(args.steps)
        elif args.only == "gemm":
            res = bench_gemm(args.steps)
        elif args.only == "extend":
            res = bench_extend(args.steps, gpu_state=False)
        elif args.only == "extend_fp8":
            res = bench_extend(args.steps, gpu_state=False, kv_dtype="fp8")
        elif args.only == "asym_extend":
            res = bench_extend(args.steps, gpu_state=False, spec=workloads.EXTRA["asym_extend"])
        elif args.only == "asym_decode":
            res = bench_decode_kernel(workloads.EXTRA["asym_decode"], args.steps)
        elif args.only == "verify":
            res = bench_verify_drafts(args.steps)
        elif args.only == "graph":
            res = bench_graph_step(workloads.WORKLOADS["llama3_8b_decode"], args.steps)
        else:
            res = bench_decode_kernel(all_specs[args.only], args.steps)
        print(json.dumps(res), flush=True)
        return

    spec = all_specs[args.workload]
    head = bench_decode_step(spec, args.steps, args.warmup, extras=not args.no_extras)
    layout, values = head.pop("layout"), head.pop("values")
    result = {
        "metric": METRIC, "value": round(head["value"], 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["ms_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
    }

    if not args.no_extras:
        # the other decode workloads, each as the headline step is measured
        result["decode_workloads"] = {}
        for wl in ("llama3_8b_decode", "long_fp8_decode", "qwen3_235b_decode", "l4_log_decode"):
            if wl == args.workload:
                continue
            r = bench_decode_step(all_specs[wl], args.steps, args.warmup, extras=False)
            r.pop("layout"), r.pop("values")
            result["decode_workloads"][wl] = {
                "step_ms": round(r["ms_step"], 4), "step_kv_read_GBps": round(r["value"], 1),
                "step_frac_hbm_peak": round(r["value"] / HBM_PEAK_GBS, 4),
                "config": r["config"], "roofline": r["roofline"]}
            log(f"decode {wl}: {result['decode_workloads'][wl]}")
        result["extend"] = bench_extend(args.steps)
        result["mfma_reference"] = bench_gemm(min(args.steps, 20))
        result["extend"]["frac_of_random_gemm"] = round(
            result["extend"]["TFLOPs"] / result["mfma_reference"]["random_TFLOPs"], 4)
        log(f"extend: {result['extend']}")
        c = bench_extend(args.steps, constant=True)
        result["extend_constant_operands"] = {k: c[k] for k in ("TFLOPs", "frac_mfma_peak", "ms", "gpu_state")}
        log(f"extend on constant operands (power diagnostic): {result['extend_constant_operands']}")
        result["extend_fp8kv"] = bench_extend(args.steps, gpu_state=False, kv_dtype="fp8")
        log(f"extend over an fp8 cache: {result['extend_fp8kv']}")
        log(f"bf16 GEMM reference: {result['mfma_reference']}")
        # key / value heads of different widths (192 / 128)
        result["asym_extend"] = bench_extend(args.steps, gpu_state=False,
                                             spec=workloads.EXTRA["asym_extend"])
        log(f"extend, 192/128 widths: {result['asym_extend']}")
        result["asym_decode"] = bench_decode_kernel(workloads.EXTRA["asym_decode"], args.steps)
        log(f"decode, 192/128 widths: {result['asym_decode']}")
        # speculative verify through the decode path and the extend path
        result["verify"] = bench_verify_drafts(args.steps)
        # the Llama-shaped step replayed from a HIP graph
        result["graph_step"] = bench_graph_step(workloads.WORKLOADS["llama3_8b_decode"], args.steps)
        log(f"step from a HIP graph: {result['graph_step']}")

    if not args.no_cpu_baseline:
        log("timing the oracle on the host cores ...")
        result["cpu_baseline"] = cpu_baseline(layout, values, args.cpu_budget)
        result["cpu_baseline"]["gpu_speedup"] = round(result["value"] / result["cpu_baseline"]["value"], 1)
        if not args.no_extras:
            elayout = workloads.make_layout(workloads.WORKLOADS["llama3_8b_extend"])
            evalues = workloads.make_values(elayout, device="cuda")
            cb = cpu_baseline_extend(elayout, evalues, min(args.cpu_budget, 10.0))
            cb["gpu_speedup"] = round(result["extend"]["TFLOPs"] * 1e3 / cb["value"], 1)
            result["extend"]["cpu_baseline"] = cb
            log(f"extend oracle: {cb}")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
