#!/usr/bin/env python3
"""Benchmark of the fused Kronecker-factored transform + per-token INT4 quantization.

One step = one kq_transform_quant over one batch of synthetic tokens already resident in
HBM (the whole hot path: load, optional channel scale, both contractions, absmax, clip,
round, clamp, pack, store). The throughput (`value`, tokens/s) is timed over K
back-to-back steps bracketed by device synchronizations; the kernel's average duration
(for the roofline) is the span of HIP events recorded on the launch stream around the
same K launches, divided by K. Default workload: hidden size 8192 with factors 64 x 128,
16384 bf16 tokens (Student-t activations with outlier channels, orthogonal factors,
clip logit 3).

Prints ONE JSON line on stdout. Algorithmic work per token: 2*n*(n1+n2) FLOP and
2.5*n bytes (bf16 in + packed int4 out; 4.5*n for fp32 input; 3*n with --bits 8). Input/output buffer sets are rotated so that consecutive steps never hit data left in
the 256 MB last-level (Infinity) cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# every source that decides what a launch reads and writes: the kernels, the device helpers
# (DMA and its cache policy), and the host code that picks the kernel and sizes its grid
KERNEL_SOURCES = ("kq_api.hip", "kq_internal.h", "kq_device.h", "kq_common.h", "kq_fused.hip",
                  "kq_generic.hip", "kq_large.hip", "kq_f32.hip")


def _code_text(src: str) -> str:
    """A source without its comments and blank lines: edits to comments leave what a launch
    reads and writes unchanged, so they do not invalidate a traffic profile."""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        path = os.path.join(ROOT, "kronecker_factored_transforms_amd", "csrc", f)
        if os.path.exists(path):
            with open(path, encoding="utf-8") as fh:
                h.update(f.encode() + b"\0" + _code_text(fh.read()).encode())
    return h.hexdigest()


def traffic_from_profile(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    there is none for this workload/kernel or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", txt)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_sha and m_b) or m_sha.group(1) != kernel_source_sha256():
        return None
    return float(m_b.group(1))


def hbm_probe(torch, dev, achieved_gbs, small_kernel_us=None):
    """What library kernels reach on this machine's HBM, measured beside the transform: a plain
    device-to-device copy (1 byte written per byte read), and a 4:1 read:write stream, the
    transform's own ratio (the sum of four 256 MiB quarters of a bf16 tensor into a fifth:
    1 GiB in, 256 MiB out). 1 GiB source, beyond the 256 MB Infinity Cache; 3 untimed and
    10 timed runs each. The transform's achieved rate is reported as a fraction of both.
    Then the 4:1 stream at the byte volume of the 2048-token attention-input workload, whose
    time per call is set beside that workload's (small_kernel_us)."""
    src = torch.empty(2 ** 29, dtype=torch.bfloat16, device=dev).uniform_(-1, 1)
    dst = torch.empty_like(src)
    red = torch.empty(2 ** 27, dtype=torch.bfloat16, device=dev)
    ops = {"copy": (lambda: dst.copy_(src), 2 * src.numel() * 2),
           "read4_write1": (lambda: torch.sum(src.view(4, -1), dim=0, out=red),
                            src.numel() * 2 + red.numel() * 2)}
    res = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name + "_GBps"] = round(nbytes * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    del src, dst, red
    # the same 4:1 stream at the volume of 2048 tokens of n = 4096 (16 MiB in, 4 MiB out),
    # where launch and ramp costs weigh: 80 buffer sets (1.6 GiB) rotated past the Infinity
    # Cache, 100 untimed and 1000 timed launches, like the workloads' own timing
    nsets = 80
    srcs = [torch.empty(2 ** 23, dtype=torch.bfloat16, device=dev).uniform_(-1, 1) for _ in range(nsets)]
    reds = [torch.empty(2 ** 21, dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    for i in range(100):
        torch.sum(srcs[i % nsets].view(4, -1), dim=0, out=reds[i % nsets])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(1000):
        torch.sum(srcs[i % nsets].view(4, -1), dim=0, out=reds[i % nsets])
    e1.record()
    torch.cuda.synchronize()
    res["read4_write1_16MiB_us"] = round(e0.elapsed_time(e1), 3)  # ms per 1000 = us per call
    del srcs, reds
    if small_kernel_us:
        res["attn_n4096_us_over_small_stream"] = round(small_kernel_us / res["read4_write1_16MiB_us"], 3)
    res["kernel_frac_of_copy"] = round(achieved_gbs / res["copy_GBps"], 3)
    res["kernel_frac_of_read4_write1"] = round(achieved_gbs / res["read4_write1_GBps"], 3)
    res["kind"] = "torch copy_ and a sum over the outer dimension of 4 (library kernels), same box"
    log(f"[bench] HBM probe: copy {res['copy_GBps']:.0f} GB/s, 4:1 stream {res['read4_write1_GBps']:.0f} GB/s; "
        f"the transform reaches {res['kernel_frac_of_copy']:.2f} and {res['kernel_frac_of_read4_write1']:.2f} of them; "
        f"4:1 stream of 16 MiB in + 4 MiB out: {res['read4_write1_16MiB_us']:.2f} us per call")
    return res


def cpu_baseline(inp, seconds: float, bits: int = 4):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload's tokens."""
    import numpy as np
    from oracle import kq_oracle as O

    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:  # pragma: no cover
        blas = []

    from kronecker_factored_transforms_amd import synth as S

    wl = inp.wl
    if wl.per_row:  # identity left factor, one step per row of n2 values
        P1 = S.to_bf16_bits(np.eye(wl.n1)) if wl.dtype == "bf16" else np.eye(wl.n1, dtype=np.float32)
    else:
        P1 = inp.P1

    def run(X):
        Y = O.transform(X, P1, inp.P2, inp.c, wl.dtype).astype(np.float32)
        if wl.per_row:
            Y = Y.reshape(-1, wl.n2)
        q, s = O.quantize_per_token(Y, O.clip_ratio(inp.alpha), wl.scale_dtype, bits=bits)
        return (O.pack_int4(q) if bits == 4 else O.pack_int8(q)), s

    T = inp.X.shape[0]
    k = min(T, 64)
    run(inp.X[:k])  # warm
    t0 = time.perf_counter()
    run(inp.X[:k])
    dt = max(time.perf_counter() - t0, 1e-6)
    k = int(min(T, max(k, seconds / dt * k)))
    # whole passes over the first k tokens until about `seconds` of wall time
    passes, done = 0, 0
    w0, c0 = time.perf_counter(), os.times()
    while True:
        run(inp.X[:k])
        passes += 1
        done += k
        if time.perf_counter() - w0 >= seconds:
            break
    w1, c1 = time.perf_counter(), os.times()
    wall = w1 - w0
    cpu = (c1.user - c0.user) + (c1.system - c0.system)
    return {
        "value": done / wall,
        "unit": "tokens/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": (f"first {k} of {T} tokens of the same workload, {passes} pass(es); float64 "
                   f"factored transform (numpy.matmul) + fp32 quantizer + packing, {wall:.1f} s "
                   f"wall, {cpu:.1f} s CPU; BLAS {blas}; host cpu_count {os.cpu_count()}, "
                   f"affinity {len(os.sched_getaffinity(0))}"),
    }


PEAK_INT8_TOPS = 5000.0        # MI355X dense int8 MFMA, TOP/s


def bench_int4_gemm(args, torch, B, dev):
    """kq_int4_gemm on random codes: [T x K] x [N x K]^T -> [T x N] bf16, rotated buffers."""
    T, N, K = args.int4_gemm
    set_bytes = (T + N) * K // 2 + T * N * 2
    nsets = max(2, math.ceil(args.rotate_mib * 2 ** 20 / set_bytes))
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    sets = []
    for _ in range(nsets):
        xq = torch.randint(0, 256, (T, K // 2), dtype=torch.uint8, device=dev, generator=g)
        wq = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g)
        sx = torch.rand(T, device=dev, generator=g).to(torch.float16)
        sw = torch.rand(N, device=dev, generator=g).to(torch.float16)
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        sets.append((xq, sx, wq, sw, out))
    stream = torch.cuda.current_stream()
    sh = int(stream.cuda_stream)

    def step(i):
        xq, sx, wq, sw, out = sets[i % nsets]
        B.kq_int4_gemm(xq, K // 2, sx, T, wq, K // 2, sw, N, K, "fp16", "bf16", out, N, sh)

    K_steps = args.steps
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    span[0].record(stream)
    for i in range(K_steps):
        step(i)
    span[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    us = span[0].elapsed_time(span[1]) / K_steps * 1e3
    ops = 2.0 * T * N * K
    byts = (T + N) * K / 2 + T * N * 2
    tops = ops / us / 1e6
    log(f"[bench] int4 gemm T={T} N={N} K={K}: {us:.2f} us/launch, {tops:.0f} TOP/s, "
        f"{byts / us / 1e3:.0f} GB/s of operands+output")
    del sets
    ref = int8_library_gemm(torch, dev, T, N, K, args.steps, args.warmup)
    log(f"[bench] library reference: torch._int_mm (int8 x int8 -> int32, one code per byte) "
        f"{ref['us']:.2f} us, {ref['tops']:.0f} TOP/s; kq_int4_gemm is {ref['us'] / us:.2f}x as fast")
    print(json.dumps({
        "metric": "INT4 x INT4 GEMM (kq_int4_gemm) TOP/s", "value": tops, "unit": "TOP/s",
        "n_gpus": 1, "steps": K_steps, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / K_steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4 (int8 MFMA)", "data": "synthetic",
        "config": {"workload": "int4_gemm", "T": T, "N": N, "K": K, "out_dtype": "bf16",
                   "buffer_sets": nsets},
        "roofline": {"bound": "mfma", "achieved": tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": tops / PEAK_INT8_TOPS, "traffic": None, "kernel_avg_us": us},
        "library_reference": {"op": "torch._int_mm (hipBLASLt int8)", "us": ref["us"],
                              "value": ref["tops"], "unit": "TOP/s",
                              "frac": ref["tops"] / PEAK_INT8_TOPS},
    }), flush=True)


def int8_library_gemm(torch, dev, T, N, K, steps, warmup):
    """The vendor library's int8 GEMM on the same shape, operands already one int8 per byte
    (what an INT4 GEMM would multiply after unpacking), timed like kq_int4_gemm."""
    g = torch.Generator(device=dev)
    g.manual_seed(1)
    a = torch.randint(-128, 128, (T, K), dtype=torch.int8, device=dev, generator=g)
    w = torch.randint(-128, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
    wt = w.t()
    stream = torch.cuda.current_stream()
    for _ in range(max(1, warmup // 4)):
        c = torch._int_mm(a, wt)
    n = max(5, steps // 4)
    e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    e[0].record(stream)
    for _ in range(n):
        c = torch._int_mm(a, wt)
    e[1].record(stream)
    torch.cuda.synchronize()
    del c
    us = e[0].elapsed_time(e[1]) / n * 1e3
    return {"us": us, "tops": 2.0 * T * N * K / us / 1e6}


# Workloads timed beside the headline in the default run: the other gated and reported
# configurations (the 65536-token prefill carries the second 60 % gate; the with-c
# down-projection and attention inputs; the 64-token decode batch, eager and replayed from a
# HIP graph).
EXTRA_WORKLOADS = ("prefill_n8192_t65536", "down_proj_n14336", "attn_n4096", "decode_n8192_t64")
GRAPH_CALLS = 100  # calls captured per graph for the decode timing


def measure(torch, B, S, dev, name, args, tokens=None, split_flags=0, bits=4, min_warm_ms=0.0,
            graph=False, keep_inputs=False):
    """Time one workload: `args.warmup` untimed steps (more, up to `min_warm_ms` of GPU time,
    when asked), then exactly `args.steps` steps bracketed by device synchronizations; the
    kernel's average duration is the HIP event span on the launch stream over those steps."""
    import numpy as np

    wl = S.WORKLOADS[name]
    t_gen = time.perf_counter()
    inp = S.make(wl, T=tokens)
    if tokens is not None:
        wl = S.with_tokens(wl, tokens)
    log(f"[bench] generated {wl.name}: T={wl.T} n={wl.n} ({wl.n1}x{wl.n2}) {wl.dtype} "
        f"in {time.perf_counter() - t_gen:.1f}s")

    def dev_tensor(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    sha = {k: (hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest() if v is not None
               else None) for k, v in (("X", inp.X), ("P1", inp.P1), ("P2", inp.P2), ("c", inp.c))}
    X0 = dev_tensor(inp.X)
    c = torch.from_numpy(inp.c).to(dev) if inp.c is not None else None
    if wl.per_row:  # identity left factor, one step per row of V
        plan = B.Plan(None, dev_tensor(inp.P2), None, inp.alpha, wl.scale_dtype, flags=split_flags,
                      n1=wl.n1, bits=bits)
    else:
        plan = B.Plan(dev_tensor(inp.P1), dev_tensor(inp.P2), c, inp.alpha, wl.scale_dtype,
                      flags=split_flags, bits=bits)
    T, n = wl.T, wl.n
    nscales = T * wl.n1 if wl.per_row else T
    esize = 2 if wl.dtype == "bf16" else 4
    code_bytes = n * bits // 8  # per token
    ws_bytes = plan.workspace_bytes(T)
    set_bytes = T * n * esize + T * code_bytes + nscales * 2
    nsets = max(2, math.ceil(args.rotate_mib * 2 ** 20 / set_bytes))
    Xs = [X0] + [X0.clone() for _ in range(nsets - 1)]
    outs = [(torch.empty((T, code_bytes), dtype=torch.uint8, device=dev),
             torch.empty((nscales,), dtype=plan.scale_dtype, device=dev)) for _ in range(nsets)]
    # the intermediate of the two-kernel designs for large factors: allocated once, outside
    # the timed region (the library itself never allocates in a call)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.current_stream()
    handle, sh = plan.handle, int(stream.cuda_stream)
    kname = plan.kernel_for(T)
    log(f"[bench] {wl.name}: kernel={kname} clip={plan.clip:.6f} buffer sets={nsets} "
        f"({nsets * set_bytes / 2**20:.0f} MiB)" + (f", workspace {ws_bytes / 2**20:.1f} MiB" if ws_bytes else ""))

    def step(i, sh=sh):
        X = Xs[i % nsets]
        codes, scales = outs[i % nsets]
        B.kq_transform_quant_ws(handle, X, T, n, codes, scales, None, ws, ws_bytes, sh)

    K = args.steps
    # events are created before the warmup: creating them between the warmup and the
    # timed region would leave the GPU idle for milliseconds, and the launches right
    # after such a pause run measurably slower while the clocks ramp back up
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K if args.per_launch_events else 0)]
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    w0 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    nwarm = 0
    for _ in range(args.warmup):
        step(nwarm)
        nwarm += 1
    span[0].record(stream)
    torch.cuda.synchronize()
    while min_warm_ms > 0 and w0.elapsed_time(span[0]) < min_warm_ms:
        for _ in range(16):
            step(nwarm)
            nwarm += 1
        span[0].record(stream)
        torch.cuda.synchronize()

    # timed region: K back-to-back steps, bracketed by synchronizations (the throughput)
    t0 = time.perf_counter()
    span[0].record(stream)
    for i in range(K):
        step(i)
    span[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    gpu_span_ms = span[0].elapsed_time(span[1]) / K
    k_avg_s = gpu_span_ms / 1e3
    per_launch = None
    if args.per_launch_events:
        # diagnostic only: an event pair around every launch; the event packets add a few
        # microseconds to each measured interval and space the launches apart
        for i in range(K):
            ev[i][0].record(stream)
            step(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        kernel_ms = sorted(a.elapsed_time(b) for a, b in ev)
        per_launch = {"mean_us": sum(kernel_ms) / K * 1e3, "median_us": kernel_ms[K // 2] * 1e3,
                      "p10_us": kernel_ms[K // 10] * 1e3, "p90_us": kernel_ms[(9 * K) // 10] * 1e3,
                      "min_us": kernel_ms[0] * 1e3, "max_us": kernel_ms[-1] * 1e3}
    graph_us = None
    if graph:
        # the same calls captured once in a HIP graph and replayed: no host enqueue cost per
        # call (what a serving loop that captures its decode step sees)
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            with torch.cuda.graph(g, stream=cap):
                csh = int(torch.cuda.current_stream().cuda_stream)
                for i in range(GRAPH_CALLS):
                    step(i, csh)
        torch.cuda.synchronize()
        reps = max(4, K // GRAPH_CALLS + 1)
        for _ in range(2):
            g.replay()
        gs = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        torch.cuda.synchronize()
        gs[0].record(stream)
        for _ in range(reps):
            g.replay()
        gs[1].record(stream)
        torch.cuda.synchronize()
        graph_us = gs[0].elapsed_time(gs[1]) * 1e3 / (reps * GRAPH_CALLS)
        del g

    flop_tok = 2 * n * (wl.n1 + wl.n2)
    byte_tok = esize * n + code_bytes
    tokens_per_s = T / (ms_per_step / 1e3)
    achieved_gbs = T * byte_tok / k_avg_s / 1e9
    achieved_tflops = T * flop_tok / k_avg_s / 1e12
    traffic = traffic_from_profile(wl.name, kname)
    log(f"[bench] {wl.name}: {K} steps: {ms_per_step * 1e3:.2f} us/step wall, {gpu_span_ms * 1e3:.2f} "
        f"us/launch on the stream: {achieved_gbs:.0f} GB/s ({achieved_gbs / PEAK_HBM_GBS:.3f} of HBM), "
        f"{achieved_tflops:.1f} TFLOP/s" + (f"; graph replay {graph_us:.2f} us/call" if graph else "")
        + (f"; per-launch events: {per_launch}" if per_launch else ""))
    res = {
        "workload": wl.name, "T": T, "n": n, "n1": wl.n1, "n2": wl.n2, "x_dtype": wl.dtype,
        "scale_dtype": wl.scale_dtype, "per_channel_c": inp.c is not None, "alpha": inp.alpha,
        "kernel": kname, "buffer_sets": nsets, "scales_per_token": wl.n1 if wl.per_row else 1,
        "code_bits": bits, "workspace_bytes": ws_bytes, "warmup_steps_run": nwarm,
        "tokens_per_s": tokens_per_s, "ms_per_step": ms_per_step,
        "roofline": {
            "bound": "hbm", "achieved": achieved_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved_gbs / PEAK_HBM_GBS, "traffic": traffic,
            "kernel_avg_us": k_avg_s * 1e6,
            "kernel_avg_source": "HIP event span of the timed region on the launch stream / steps",
            "algorithmic_bytes_per_launch": T * byte_tok,
        },
        "mfma": {"achieved": achieved_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                 "frac": achieved_tflops / PEAK_BF16_TFLOPS,
                 "algorithmic_flop_per_launch": T * flop_tok},
        "inputs_sha256": sha,
    }
    if graph_us is not None:
        res["graph_replay_us_per_call"] = graph_us
        res["eager_us_per_call"] = ms_per_step * 1e3
    if per_launch:
        res["per_launch_events_us"] = per_launch
    plan.close()
    if not keep_inputs:
        del Xs, outs, X0, ws
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        inp = None
    return res, inp


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="hidden_n8192")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count (sweeps; the JSON names it)")
    ap.add_argument("--rotate-mib", type=int, default=1536,
                    help="minimum total size of the rotated input+output buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only --workload (the default run also times " + ", ".join(EXTRA_WORKLOADS) + ")")
    ap.add_argument("--split", choices=["default", "reg1", "reg2", "cols", "deep", "stream", "pair",
                                        "generic", "twostage", "ptile", "rsplit"],
                    default="default", help="work split of the fused kernel (default: the plan's)")
    ap.add_argument("--per-launch-events", action="store_true",
                    help="also time every launch with its own event pair (diagnostic)")
    ap.add_argument("--graph", action="store_true",
                    help="also replay the calls from a captured HIP graph (per-call time)")
    ap.add_argument("--bits", type=int, choices=[4, 8], default=4,
                    help="code width: 4 (packed nibbles, the default) or 8 (one byte per value)")
    ap.add_argument("--int4-gemm", type=int, nargs=3, metavar=("T", "N", "K"), default=None,
                    help="time kq_int4_gemm on random codes instead (tokens, out channels, K)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}). Tokens are independent, "
              f"so N GPUs would each run the same kernel on T/N tokens with no communication.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from kronecker_factored_transforms_amd import binding as B
    from kronecker_factored_transforms_amd import synth as S

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.int4_gemm:
        bench_int4_gemm(args, torch, B, dev)
        return
    flags = {"default": 0, "reg1": B.KQ_FLAG_SPLIT_REG1, "reg2": B.KQ_FLAG_SPLIT_REG2,
             "cols": B.KQ_FLAG_SPLIT_COLS, "deep": B.KQ_FLAG_SPLIT_DEEP,
             "stream": B.KQ_FLAG_SPLIT_STREAM, "pair": B.KQ_FLAG_SPLIT_PAIR,
             "generic": B.KQ_FLAG_FORCE_GENERIC, "twostage": B.KQ_FLAG_SPLIT_TWOSTAGE,
             "ptile": B.KQ_FLAG_SPLIT_PTILE, "rsplit": B.KQ_FLAG_SPLIT_RSPLIT}[args.split]

    if args.copy_probe:
        a = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        log("[bench] copy probe: 3 x 512 MiB device-to-device copies")

    # like every workload below, the headline follows a pause (input generation, buffer
    # rotation set-up): its timed region starts after at least 20 ms of launches, so that it
    # does not run in the clock ramp after that idle gap (the --warmup steps are the minimum)
    head, inp = measure(torch, B, S, dev, args.workload, args, tokens=args.tokens,
                        split_flags=flags, bits=args.bits, graph=args.graph, keep_inputs=True,
                        min_warm_ms=20.0)

    extras = {}
    run_extra = (not args.no_extra and args.workload == "hidden_n8192" and args.tokens is None
                 and args.split == "default" and args.bits == 4)
    if run_extra:
        for name in EXTRA_WORKLOADS:
            # these follow a pause for input generation: warm the clocks for at least 20 ms of
            # launches (beyond the --warmup steps) before their timed region
            extras[name], _ = measure(torch, B, S, dev, name, args, min_warm_ms=20.0,
                                      graph=name.startswith("decode"))

    probe = None
    if run_extra:
        small = extras.get("attn_n4096", {}).get("roofline", {}).get("kernel_avg_us")
        probe = hbm_probe(torch, dev, head["roofline"]["achieved"], small)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds, args.bits)
        log(f"[bench] cpu oracle: {cpu['value']:.0f} tokens/s on {cpu['cores']} cores")

    cfg = {k: head[k] for k in ("workload", "T", "n", "n1", "n2", "x_dtype", "scale_dtype",
                                "per_channel_c", "alpha", "kernel", "buffer_sets",
                                "scales_per_token", "code_bits")}
    out = {
        "metric": "tokens/s + % of roofline (HBM GB/s or MFMA TFLOP/s), n=8192 64x128 transform+INT4",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": head["warmup_steps_run"],
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["x_dtype"],
        "data": "synthetic",
        "config": cfg,
        "inputs_sha256": head["inputs_sha256"],
        "roofline": head["roofline"],
        "hbm_probe": probe,
        "mfma": head["mfma"],
        "cpu_baseline": cpu,
    }
    if "per_launch_events_us" in head:
        out["per_launch_events_us"] = head["per_launch_events_us"]
    if "graph_replay_us_per_call" in head:
        out["graph_replay_us_per_call"] = head["graph_replay_us_per_call"]
    if extras:
        out["configs"] = extras
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
