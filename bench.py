#!/usr/bin/env python
"""KDA hot-path benchmark on one MI355X.

Headline (``value``): packed-decode state bandwidth in GB/s on the batched
decode workload (32 single-token requests, H=32, K=V=128, fp32 state pool of
512 slots = 1 GiB, slot indices at stride 8, lower bound -5). A step is one
kda_decode_packed call; consecutive steps rotate through 16 disjoint sets of
32 slots (1 GiB in total) so the 256 MB Infinity Cache cannot hold the state
between visits. Inputs are resident in HBM before timing starts.

The same JSON line carries the other legs of the hot path, each timed the same
way: spec-verify (8 rows), chunked prefill (one 8192-token sequence, and 64
varlen sequences), and the mixed 4096-token batch.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
METRIC = "KDA decode state GB/s (% HBM peak) + chunked prefill tokens/s (MFMA %)"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--legs", default="decode,spec,prefill,mixed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    return ap.parse_args()


def timed_launches(fn, steps: int, warmup: int):
    """Runs ``fn(i)`` warmup + steps times on the current stream. Returns
    (ms per step over the whole timed region, mean per-launch ms from event
    pairs around each call)."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        starts[i].record()
        fn(warmup + i)
        ends[i].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1) / steps
    per = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps
    return total, per


def _device_token_inputs(rows, H, K, V, seed, dev):
    import workloads as W

    return {k: v.to(dev) for k, v in W.make_token_inputs(rows, H, K, V, seed).items()}


def _device_pool(slots, H, K, V, std, seed, dev):
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn(slots, H, K, V, generator=g, device=dev).mul_(std)


def decode_io_bytes(rows, H, K, V):
    # q, k, v, raw_g (bf16) + raw_beta (bf16) + out (bf16) per row
    return rows * H * (2 * K * 2 + V * 2 + K * 2 + 2 + V * 2)


def leg_decode(steps, warmup):
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V, N, STRIDE, SETS = 32, 128, 128, 32, 8, 16
    pool = _device_pool(N * SETS, H, K, V, 0.05, 1999, dev)
    inp = _device_token_inputs(N, H, K, V, 1020, dev)
    perm = torch.randperm(N * SETS, generator=W._gen(1021)).to(torch.int32)
    tables = []
    for s in range(SETS):
        t = torch.full((N, STRIDE), -7, dtype=torch.int32)
        t[:, 0] = perm[s * N:(s + 1) * N]
        tables.append(t.to(dev))
    out = torch.empty(N, H, V, dtype=torch.bfloat16, device=dev)

    def step(i):
        kda.kda_decode_packed(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                              inp["dt_bias"], -5.0, pool, tables[i % SETS][:, 0], out=out)

    total_ms, launch_ms = timed_launches(step, steps, warmup)
    state_bytes = 2 * N * H * K * V * 4
    alg_bytes = state_bytes + decode_io_bytes(N, H, K, V)
    return {
        "workload": "batched_decode_h32_k128_n32_stride8_lb-5",
        "ms_per_step": total_ms,
        "launch_ms": launch_ms,
        "state_gbs": state_bytes / (total_ms * 1e-3) / 1e9,
        "alg_bytes_per_launch": alg_bytes,
        "achieved_gbs": alg_bytes / (launch_ms * 1e-3) / 1e9,
    }


def leg_spec(steps, warmup):
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V = 32, 128, 128
    res = {}
    pool = _device_pool(512, H, K, V, 0.05, 2999, dev)
    for name, (real, tps, nulls) in W.SPEC_LAYOUTS.items():
        n = real + nulls
        inp = _device_token_inputs(n * tps, H, K, V, 2100, dev)
        # rotate the requests over disjoint slots so no state is cache-resident
        perm = torch.randperm(512, generator=W._gen(2101)).to(torch.int32)
        sets = 512 // n
        tables = []
        for s in range(sets):
            t = torch.full((n, 8), -7, dtype=torch.int32)
            t[:, 0] = perm[s * n:(s + 1) * n]
            t[real:, 0] = -1
            tables.append(t.to(dev))
        out = torch.empty(n * tps, H, V, dtype=torch.bfloat16, device=dev)

        def step(i):
            kda.kda_decode_packed(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                                  inp["dt_bias"], -5.0, pool, tables[i % sets][:, 0],
                                  tokens_per_seq=tps, out=out)

        total_ms, launch_ms = timed_launches(step, steps, warmup)
        state_bytes = 2 * real * H * K * V * 4
        res[name] = {"us_per_step": total_ms * 1e3, "launch_us": launch_ms * 1e3,
                     "state_gbs": state_bytes / (launch_ms * 1e-3) / 1e9}
    return res


PREFILL_FLOP_PER_TOKEN_HEAD_USEFUL = None  # set in prefill_flops()


def prefill_flops(lens, H, K, V, C=64):
    """Useful MFMA-form flops of the chunked algorithm (causal triangles
    counted once): per chunk of n tokens and head,
      A and P (n^2/2 pairs x K each, x2 flop) ............ 2 * n*n*K
      W = T(beta K e^g), U = T(beta V) (triangular) ....... n*n*(K+V)
      V' = U - W S, (Q e^g) S ............................ 2 * 2*n*K*V
      P V' (triangular) .................................. n*n*V
      S += (K e^{g_n-g})^T V' ............................ 2*n*K*V
    """
    total = 0
    for L in lens:
        full, rem = divmod(L, C)
        for n in [C] * full + ([rem] if rem else []):
            total += 2 * n * n * K + n * n * (K + V) + 4 * n * K * V + n * n * V + 2 * n * K * V
    return total * H


def prefill_io_bytes(T, H, K, V, seqs):
    return T * H * (2 * K * 2 + V * 2 + K * 2 + 2 + V * 2) + 2 * seqs * H * K * V * 4


def leg_prefill(steps, warmup, lens, name, seed):
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V = 32, 128, 128
    T = sum(lens)
    n = len(lens)
    copies = 2  # two input copies, alternated, so inputs are not cache-resident
    inps = [_device_token_inputs(T, H, K, V, seed + c, dev) for c in range(copies)]
    pool = _device_pool(max(2 * n, 4), H, K, V, 0.05, seed + 10, dev)
    idx = [torch.arange(c * n, (c + 1) * n, dtype=torch.int32, device=dev) for c in range(2)]
    cu = W.cu_from_lengths(lens).to(dev)
    out = torch.empty(T, H, V, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(n, T, H, K, V), dtype=torch.uint8, device=dev)

    def step(i):
        inp = inps[i % copies]
        kda.kda_chunk_prefill(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                              inp["dt_bias"], -5.0, pool, idx[i % 2], cu, out=out, workspace=ws)

    total_ms, launch_ms = timed_launches(step, steps, warmup)
    flops = prefill_flops(lens, H, K, V)
    io = prefill_io_bytes(T, H, K, V, n)
    return {
        "workload": name,
        "ms_per_step": total_ms,
        "tokens_per_s": T / (total_ms * 1e-3),
        "useful_tflops": flops / (total_ms * 1e-3) / 1e12,
        "mfma_frac": flops / (total_ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS,
        "io_gbs": io / (total_ms * 1e-3) / 1e9,
        "hbm_frac": io / (total_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "useful_flops_per_step": flops,
        "io_bytes_per_step": io,
    }


def leg_mixed(steps, warmup):
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V, D = 32, 128, 128, 96
    lens = W.split_total(4000, 5, 4000)
    T = D + sum(lens)
    inp = _device_token_inputs(T, H, K, V, 4001, dev)
    pool = _device_pool(1024, H, K, V, 0.05, 4011, dev)
    perm = torch.randperm(1024, generator=W._gen(4012)).to(torch.int32)
    sets = 1024 // (D + 5)
    tables = []
    for s in range(sets):
        t = torch.full((D + 5, 8), -7, dtype=torch.int32)
        t[:, 0] = perm[s * (D + 5):(s + 1) * (D + 5)]
        tables.append(t.to(dev))
    cu = W.cu_from_lengths(lens).to(dev)
    out = torch.empty(T, H, V, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(kda.kda_mixed_batch_workspace_size(D, 5, T - D, H, K, V), dtype=torch.uint8,
                     device=dev)

    def step(i):
        kda.kda_mixed_batch(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                            inp["dt_bias"], -5.0, pool, tables[i % sets][:, 0], D, cu, out=out,
                            workspace=ws)

    total_ms, _ = timed_launches(step, steps, warmup)
    return {"workload": "mixed_d96_p4000_h32_k128", "ms_per_step": total_ms,
            "tokens_per_s": T / (total_ms * 1e-3)}


def cpu_baseline(seconds: float):
    """The fp64 oracle (recurrent form, as it stands) on a bounded sample of
    the decode workload: the same 32 requests on a compact 32-slot pool,
    repeated until about ``seconds`` of wall time has passed."""
    import torch

    import workloads as W
    from oracle import oracle as O

    H, K, V, N = 32, 128, 128, 32
    case = W.decode_case("cpu_sample", H, K, V, N, 1, N, 8, -5.0, seed=1020, pool_seed=77)
    threads = os.cpu_count() or 1
    O.set_threads(threads)
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.decode_packed(case.inputs, case.pool, case.state_indices, H, K, V, 1, -5.0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    state_bytes = 2 * N * H * K * V * 4 * reps
    return {"value": state_bytes / el / 1e9, "unit": "GB/s", "cores": O.max_threads(),
            "kind": "oracle",
            "sample": f"{reps} repeats of the 32-request batched decode (H=32, K=V=128) on a "
                      f"32-slot pool, {el:.1f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    legs = set(args.legs.split(","))
    torch.cuda.synchronize()

    dec = leg_decode(args.steps, args.warmup)
    extra = {}
    if "spec" in legs:
        extra["spec_verify"] = leg_spec(args.steps, args.warmup)
    if "prefill" in legs:
        for nm, fn in (("prefill_t8192", lambda: leg_prefill(max(args.steps // 10, 5), 3, [8192],
                                                            "prefill_t8192_h32_k128", 3000)),
                       ("prefill_varlen64", lambda: leg_prefill(
                           max(args.steps // 10, 5), 3,
                           __import__("workloads").random_lengths(64, 1, 256, 3001, force_ones=2),
                           "prefill_varlen64_h32_k128", 3002))):
            try:
                extra[nm] = fn()
            except Exception as e:  # report, do not hide
                extra[nm] = {"error": str(e)[:300]}
    if "mixed" in legs:
        try:
            extra["mixed_4096"] = leg_mixed(max(args.steps // 10, 5), 3)
        except Exception as e:
            extra["mixed_4096"] = {"error": str(e)[:300]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(dec["state_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": dec["workload"], "heads": 32, "head_dim_k": 128, "head_dim_v": 128,
                   "requests": 32, "pool_slots": 512, "index_stride": 8, "lower_bound": -5.0,
                   "slot_sets_rotated": 16},
        "roofline": {"bound": "hbm", "achieved": round(dec["achieved_gbs"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec["achieved_gbs"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel<128,32>", "launch_us": round(dec["launch_ms"] * 1e3, 3),
                     "alg_bytes_per_launch": dec["alg_bytes_per_launch"]},
        "cpu_baseline": cpu,
        "legs": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
