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


def kernel_source_sha256() -> str:
    h = hashlib.sha256()
    for f in ("kq_fused.hip", "kq_generic.hip"):
        with open(os.path.join(ROOT, "kronecker_factored_transforms_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
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
    print(json.dumps({
        "metric": "INT4 x INT4 GEMM (kq_int4_gemm) TOP/s", "value": tops, "unit": "TOP/s",
        "n_gpus": 1, "steps": K_steps, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / K_steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4 (int8 MFMA)", "data": "synthetic",
        "config": {"workload": "int4_gemm", "T": T, "N": N, "K": K, "out_dtype": "bf16",
                   "buffer_sets": nsets},
        "roofline": {"bound": "mfma", "achieved": tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                     "frac": tops / PEAK_INT8_TOPS, "traffic": None, "kernel_avg_us": us},
    }), flush=True)


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
    ap.add_argument("--split", choices=["default", "reg1", "reg2", "cols", "deep", "stream", "pair", "generic"],
                    default="default", help="work split of the fused kernel (default: the plan's)")
    ap.add_argument("--per-launch-events", action="store_true",
                    help="also time every launch with its own event pair (diagnostic)")
    ap.add_argument("--bits", type=int, choices=[4, 8], default=4,
                    help="code width: 4 (packed nibbles, the default) or 8 (one byte per value)")
    ap.add_argument("--int4-gemm", type=int, nargs=3, metavar=("T", "N", "K"), default=None,
                    help="time kq_int4_gemm on random codes instead (tokens, out channels, K)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}). Tokens are independent, "
              f"so N GPUs would each run the same kernel on T/N tokens with no communication.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
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
    wl = S.WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    inp = S.make(wl, T=args.tokens)
    if args.tokens is not None:
        wl = S.with_tokens(wl, args.tokens)
    log(f"[bench] generated {wl.name}: T={wl.T} n={wl.n} ({wl.n1}x{wl.n2}) {wl.dtype} "
        f"in {time.perf_counter() - t_gen:.1f}s")

    def dev_tensor(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # fingerprints of the synthetic inputs, so that runs can be matched to the same data
    sha = {k: (hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest() if v is not None
               else None) for k, v in (("X", inp.X), ("P1", inp.P1), ("P2", inp.P2), ("c", inp.c))}
    X0 = dev_tensor(inp.X)
    c = torch.from_numpy(inp.c).to(dev) if inp.c is not None else None
    flags = {"default": 0, "reg1": B.KQ_FLAG_SPLIT_REG1, "reg2": B.KQ_FLAG_SPLIT_REG2,
             "cols": B.KQ_FLAG_SPLIT_COLS, "deep": B.KQ_FLAG_SPLIT_DEEP,
             "stream": B.KQ_FLAG_SPLIT_STREAM, "pair": B.KQ_FLAG_SPLIT_PAIR,
             "generic": B.KQ_FLAG_FORCE_GENERIC}[args.split]
    if wl.per_row:  # identity left factor, one step per row of V
        plan = B.Plan(None, dev_tensor(inp.P2), None, inp.alpha, wl.scale_dtype, flags=flags,
                      n1=wl.n1, bits=args.bits)
    else:
        plan = B.Plan(dev_tensor(inp.P1), dev_tensor(inp.P2), c, inp.alpha, wl.scale_dtype,
                      flags=flags, bits=args.bits)
    T, n = wl.T, wl.n
    nscales = T * wl.n1 if wl.per_row else T
    esize = 2 if wl.dtype == "bf16" else 4
    code_bytes = n * args.bits // 8  # per token
    set_bytes = T * n * esize + T * code_bytes + nscales * 2
    nsets = max(2, math.ceil(args.rotate_mib * 2 ** 20 / set_bytes))
    Xs = [X0] + [X0.clone() for _ in range(nsets - 1)]
    outs = [(torch.empty((T, code_bytes), dtype=torch.uint8, device=dev),
             torch.empty((nscales,), dtype=plan.scale_dtype, device=dev)) for _ in range(nsets)]
    stream = torch.cuda.current_stream()
    handle, sh = plan.handle, int(stream.cuda_stream)
    kname = plan.kernel_for(T)
    log(f"[bench] kernel={kname} clip={plan.clip:.6f} buffer sets={nsets} "
        f"({nsets * set_bytes / 2**20:.0f} MiB)")

    if args.copy_probe:
        a = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("[bench] copy probe: 3 x 512 MiB device-to-device copies")

    def step(i):
        X = Xs[i % nsets]
        codes, scales = outs[i % nsets]
        B.kq_transform_quant(handle, X, T, n, codes, scales, None, sh)

    K = args.steps
    # events are created before the warmup: creating them between the warmup and the
    # timed region would leave the GPU idle for milliseconds, and the launches right
    # after such a pause run measurably slower while the clocks ramp back up
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K if args.per_launch_events else 0)]
    span = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: K back-to-back steps, bracketed by synchronizations (the throughput)
    t0 = time.perf_counter()
    span[0].record(stream)
    for i in range(K):
        step(i)
    span[1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    gpu_span_ms = span[0].elapsed_time(span[1]) / K
    # average launch duration: the HIP event span of the timed region on the launch stream
    # over K back-to-back launches (each launch waits for the previous one)
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

    flop_tok = 2 * n * (wl.n1 + wl.n2)
    byte_tok = esize * n + code_bytes
    tokens_per_s = T / (ms_per_step / 1e3)
    achieved_gbs = T * byte_tok / k_avg_s / 1e9
    achieved_tflops = T * flop_tok / k_avg_s / 1e12
    traffic = traffic_from_profile(wl.name, kname)
    log(f"[bench] {K} steps: {ms_per_step * 1e3:.2f} us/step wall, {gpu_span_ms * 1e3:.2f} us/launch "
        f"on the stream: {achieved_gbs:.0f} GB/s, {achieved_tflops:.1f} TFLOP/s"
        + (f"; per-launch events: {per_launch}" if per_launch else ""))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds, args.bits)
        log(f"[bench] cpu oracle: {cpu['value']:.0f} tokens/s on {cpu['cores']} cores")

    out = {
        "metric": "tokens/s + % of roofline (HBM GB/s or MFMA TFLOP/s), n=8192 64x128 transform+INT4",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.name, "T": T, "n": n, "n1": wl.n1, "n2": wl.n2, "x_dtype": wl.dtype,
            "scale_dtype": wl.scale_dtype, "per_channel_c": inp.c is not None,
            "alpha": inp.alpha, "kernel": kname, "buffer_sets": nsets,
            "scales_per_token": wl.n1 if wl.per_row else 1, "code_bits": args.bits,
        },
        "inputs_sha256": sha,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / PEAK_HBM_GBS,
            "traffic": traffic,
            "kernel_avg_us": k_avg_s * 1e6,
            "kernel_avg_source": "HIP event span of the timed region on the launch stream / steps",
            "algorithmic_bytes_per_launch": T * byte_tok,
        },
        "mfma": {
            "achieved": achieved_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS,
            "algorithmic_flop_per_launch": T * flop_tok,
        },
        "cpu_baseline": cpu,
    }
    if per_launch:  # diagnostic: an event pair around every launch (adds a few us each)
        out["per_launch_events_us"] = per_launch
    print(json.dumps(out), flush=True)
    plan.close()


if __name__ == "__main__":
    main()
