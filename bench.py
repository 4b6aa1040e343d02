#!/usr/bin/env python
"""KDA hot-path benchmark on one MI355X.

Headline (``value``): packed-decode state bandwidth in GB/s on the batched
decode workload: 32 single-token requests, H=32, K=V=128, fp32 state pool of
512 slots (1 GiB), slot indices at stride 8 (column 0 of a block table),
lower bound -5. A step is one kda_decode_packed call; consecutive steps rotate
through 16 disjoint sets of 32 slots (1 GiB in total) so the 256 MB Infinity
Cache cannot hold a request's state between visits. Inputs are resident in
HBM before timing starts.

Timing: the calls are captured once in a HIP graph (they allocate nothing
and never synchronise) and the graph is replayed; HIP events on the replay
stream bracket the timed region. Eager (Python-launched) times are reported
next to them. The same JSON line carries the other legs of the hot path:
spec-verify (8 rows), chunked prefill (one 8192-token sequence; 64 varlen
sequences; one 65536-token sequence), the mixed 4096-token batch, spec
decode with a state per token, the gated RMSNorm output epilogue and the
short-conv input prologue.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
METRIC = "KDA decode state GB/s (% HBM peak) + chunked prefill tokens/s (MFMA %)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_batched_decode_h32_k128_n32_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--legs", default="decode,spec,prefill,mixed,norm,conv")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of a known size, run a few times, used to
    scale the FETCH_SIZE / WRITE_SIZE counters against known bytes."""
    import torch

    n = mib * 2**20 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "bytes_read": n * 4, "bytes_written": n * 4}))


def graph_time(fn, n_calls: int, steps: int, warmup: int):
    """Captures fn(0..n_calls-1) in one HIP graph and replays it until at
    least ``steps`` calls are timed. Returns (ms per call, calls timed)."""
    import torch

    for i in range(n_calls):  # eager warm-up (also JIT-free: everything is prebuilt)
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n_calls):
                fn(i)
    torch.cuda.synchronize()
    reps = max(1, (steps + n_calls - 1) // n_calls)
    wreps = max(1, (warmup + n_calls - 1) // n_calls)
    for _ in range(wreps):
        g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (reps * n_calls), reps * n_calls


def eager_time(fn, steps: int, warmup: int):
    """Python-launched calls on the current stream; events bracket the region."""
    import torch

    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        fn(warmup + i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def _device_token_inputs(rows, H, K, V, seed, dev):
    import workloads as W

    return {k: v.to(dev) for k, v in W.make_token_inputs(rows, H, K, V, seed).items()}


def _device_pool(slots, H, K, V, std, seed, dev):
    import torch

    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return torch.randn(slots, H, K, V, generator=g, device=dev).mul_(std)


def token_io_bytes(rows, H, K, V):
    """q, k, v, raw_g, raw_beta read and out written, all bf16, per call."""
    return rows * H * (2 * K * 2 + V * 2 + K * 2 + 2 + V * 2)


DECODE_SOURCES = ("kda_decode.hip", "kda_device.h", "kda_internal.h")


def source_code(text: str) -> str:
    """The code of a C++/HIP source without its comments, trailing blanks and
    blank lines (string and character literals kept as they are), so that a
    counter summary stays valid across edits that change no code."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def sources_hash(names) -> str:
    """Hash of the code of the named sources and of the compiler flags each
    is built with (the same code under another schedule is another kernel)."""
    from gated_delta_rule_45_amd import build as kb

    h = hashlib.sha256()
    for name in names:
        text = open(os.path.join(ROOT, "gated_delta_rule_45_amd", "csrc", name), encoding="utf-8").read()
        h.update(source_code(text).encode())
        h.update(" ".join(kb.FLAGS + kb.SOURCE_FLAGS.get(name, [])).encode())
    return h.hexdigest()[:16]


def decode_kernel_hash() -> str:
    """Hash of the code of every source the decode kernel is compiled from."""
    return sources_hash(DECODE_SOURCES)


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, only if it was taken on the current decode kernel source."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != decode_kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _lb(lower_bound) -> str:
    return "None" if lower_bound is None else f"{lower_bound:g}"


def leg_decode(steps, warmup, with_norm=False, stride=8, lower_bound=-5.0):
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V, N, STRIDE, SETS = 32, 128, 128, 32, stride, 16
    pool = _device_pool(N * SETS, H, K, V, 0.05, 1999, dev)
    inp = _device_token_inputs(N, H, K, V, 1020, dev)
    perm = torch.randperm(N * SETS, generator=W._gen(1021)).to(torch.int32)
    tables = []
    for s in range(SETS):
        t = torch.full((N, STRIDE), -7, dtype=torch.int32)
        t[:, 0] = perm[s * N:(s + 1) * N]
        tables.append(t.to(dev))
    out = torch.empty(N, H, V, dtype=torch.bfloat16, device=dev)
    norm = None
    if with_norm:
        nm = W.make_norm(N, H, V, 1022)
        norm = kda.GatedRMSNorm(nm["gate"].to(dev), nm["weight"].to(dev), nm["eps"])

    def step(i):
        kda.kda_decode_packed(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                              inp["dt_bias"], lower_bound, pool, tables[i % SETS][:, 0], out=out, norm=norm)

    eager_ms = eager_time(step, steps, warmup)
    ms, timed = graph_time(step, SETS, steps, warmup)
    state_bytes = 2 * N * H * K * V * 4
    alg_bytes = state_bytes + token_io_bytes(N, H, K, V) + (N * H * V * 2 if with_norm else 0)
    return {
        "workload": f"batched_decode_h32_k128_n32_stride{stride}_lb{_lb(lower_bound)}" +
                    ("_gated_rmsnorm" if with_norm else ""),
        "ms_per_step": ms, "eager_ms_per_step": eager_ms, "steps_timed": timed,
        "state_gbs": state_bytes / (ms * 1e-3) / 1e9,
        "alg_bytes_per_launch": alg_bytes,
        "achieved_gbs": alg_bytes / (ms * 1e-3) / 1e9,
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
        perm = torch.randperm(512, generator=W._gen(2101)).to(torch.int32)
        sets = 512 // n  # disjoint slot sets: 1 GiB of state in rotation
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

        ms, _ = graph_time(step, sets, steps, warmup)
        state_bytes = 2 * real * H * K * V * 4
        res[name] = {"us_per_step": round(ms * 1e3, 3),
                     "state_gbs": round(state_bytes / (ms * 1e-3) / 1e9, 1)}
    return res


def leg_spec_states(steps, warmup):
    """Spec decode with a state per token (kda_spec_decode): each request
    reads one state and writes one per token; a random accepted count picks
    the column the state is read from."""
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V = 32, 128, 128
    res = {}
    pool = _device_pool(512, H, K, V, 0.05, 2999, dev)
    for name, (real, tps, nulls) in W.SPEC_LAYOUTS.items():
        n = real + nulls
        inp = _device_token_inputs(n * tps, H, K, V, 2200, dev)
        perm = torch.randperm(512, generator=W._gen(2201)).to(torch.int32)
        sets = 512 // (n * 8)  # disjoint tables of 8 columns per request
        tables, accs = [], []
        for s_ in range(sets):
            t = perm[s_ * n * 8:(s_ + 1) * n * 8].view(n, 8).clone()
            t[real:, :] = -1
            tables.append(t.to(dev))
            a = torch.randint(1, tps + 1, (n,), generator=W._gen(2202 + s_)).to(torch.int32)
            a[real:] = 1
            accs.append(a.to(dev))
        out = torch.empty(n * tps, H, V, dtype=torch.bfloat16, device=dev)

        def step(i):
            kda.kda_spec_decode(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                                inp["dt_bias"], -5.0, pool, tables[i % sets], accs[i % sets],
                                tokens_per_seq=tps, out=out)

        ms, _ = graph_time(step, sets, steps, warmup)
        state_bytes = (1 + tps) * real * H * K * V * 4
        res[name] = {"us_per_step": round(ms * 1e3, 3),
                     "state_gbs": round(state_bytes / (ms * 1e-3) / 1e9, 1)}
    return res


def prefill_flops(lens, H, K, V, C=64):
    """Useful flops of the chunked algorithm, causal triangles counted once.
    Per chunk of n tokens and head:
      A and P (n^2/2 pairs, K each, 2 flop) ............ 2 n^2 K
      W = T(beta K e^g), U = T(beta V) (T triangular) .. n^2 (K + V)
      V' = U - W S and (Q e^g) S ....................... 4 n K V
      P V' (triangular) ................................ n^2 V
      S += (K e^{g_n - g})^T V' ........................ 2 n K V
    (140 k flop per token-head at n = 64, K = V = 128)."""
    total = 0
    for L in lens:
        full, rem = divmod(L, C)
        for n in [C] * full + ([rem] if rem else []):
            total += 2 * n * n * K + n * n * (K + V) + 4 * n * K * V + n * n * V + 2 * n * K * V
    return total * H


def prefill_io_bytes(T, H, K, V, seqs):
    """Mandatory HBM traffic: token inputs/outputs plus one state read and write."""
    return token_io_bytes(T, H, K, V) + 2 * seqs * H * K * V * 4


def leg_prefill(steps, warmup, lens, name, seed, with_norm=False, lower_bound=-5.0, min_workspace=False):
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V = 32, 128, 128
    T = sum(lens)
    n = len(lens)
    copies = 2  # two input copies alternate, so no call finds its inputs cached
    inps = [_device_token_inputs(T, H, K, V, seed + c, dev) for c in range(copies)]
    pool = _device_pool(2 * n, H, K, V, 0.05, seed + 10, dev)
    idx = [torch.arange(c * n, (c + 1) * n, dtype=torch.int32, device=dev) for c in range(2)]
    cu = W.cu_from_lengths(lens).to(dev)
    out = torch.empty(T, H, V, dtype=torch.bfloat16, device=dev)
    # The full workspace runs long sequences with chunk records; the smallest
    # accepted one without (both launches build every chunk's operands).
    size = (kda.kda_chunk_prefill_workspace_min_size if min_workspace else kda.kda_chunk_prefill_workspace_size)
    ws = torch.empty(size(n, T, H, K, V), dtype=torch.uint8, device=dev)
    norm = None
    if with_norm:
        nm = W.make_norm(T, H, V, seed + 20)
        norm = kda.GatedRMSNorm(nm["gate"].to(dev), nm["weight"].to(dev), nm["eps"])

    def step(i):
        inp = inps[i % copies]
        kda.kda_chunk_prefill(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                              inp["dt_bias"], lower_bound, pool, idx[i % 2], cu, out=out, workspace=ws,
                              norm=norm)

    ms, _ = graph_time(step, copies, steps, warmup)
    flops = prefill_flops(lens, H, K, V)
    io = prefill_io_bytes(T, H, K, V, n)
    return {
        "workload": name,
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "useful_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
        "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 5),
        "io_gbs": round(io / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(io / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
        "useful_flops_per_step": flops,
        "io_bytes_per_step": io,
    }


PREFILL_COUNTERS_FILE = os.path.join(ROOT, "profiles", "chunk_prefill_kernels_counters.json")
PREFILL_SOURCES = ("kda_chunk.hip", "kda_chunk_exact.hip", "kda_device.h", "kda_internal.h")


def prefill_kernel_hash() -> str:
    """Hash of the code of every source the chunked-prefill kernels are compiled from."""
    return sources_hash(PREFILL_SOURCES)


def prefill_counters(workload: str):
    """The committed rocprofv3 counter summary of one prefill workload (per
    kernel: mean duration, HBM bytes from FETCH_SIZE x 2 / WRITE_SIZE x 1, MFMA
    busy and executed MFMA flops), only if it was taken on the current
    prefill kernel sources."""
    try:
        d = json.load(open(PREFILL_COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != prefill_kernel_hash():
        return None
    return d.get("workloads", {}).get(workload)


def prefill_roofline(leg: dict):
    """Roofline of a prefill call: co-bound by bf16 MFMA (useful flops of the
    chunked algorithm) and HBM (mandatory I/O), with the measured traffic and
    the per-kernel counters when a matching summary is committed."""
    ms = leg["ms_per_step"]
    r = {"bound": "co-bound",
         "mfma_frac": leg["mfma_frac"], "mfma_achieved_tflops": leg["useful_tflops"],
         "mfma_peak_tflops": BF16_DENSE_TFLOPS,
         "hbm_frac": leg["hbm_frac"], "hbm_achieved_gbs": leg["io_gbs"], "hbm_peak_gbs": HBM_PEAK_GBS,
         "alg_flops_per_call": leg["useful_flops_per_step"], "alg_bytes_per_call": leg["io_bytes_per_step"],
         "traffic": None}
    c = prefill_counters(leg["workload"])
    if c is not None:
        kernels = c["kernels"]
        dom = max(kernels, key=lambda k: kernels[k]["us"])
        traffic = sum(k["hbm_bytes"] for k in kernels.values())
        mops = sum(k.get("mfma_flops", 0) for k in kernels.values())
        r.update({
            "traffic": traffic,
            "traffic_over_algorithmic": round(traffic / leg["io_bytes_per_step"], 3),
            "dominant_kernel": dom, "dominant_kernel_us": kernels[dom]["us"],
            "dominant_kernel_mfma_busy": kernels[dom].get("mfma_busy"),
            "counter_mfma_tflops": round(mops / (ms * 1e-3) / 1e12, 2),
            "counter_mfma_frac": round(mops / (ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 5),
            "kernels": kernels, "counters_from": os.path.relpath(PREFILL_COUNTERS_FILE, ROOT),
        })
    return r


def _cpu_threads() -> int:
    """Cores the oracle may use: the OpenMP allowance if one is set (the
    box's CPU share), else every core the process sees."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    return int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)


def cpu_prefill_baseline(lens, full_tokens: int, seconds: float):
    """The fp64 oracle (recurrent form, as it stands) on head samples of a
    prefill config, single-threaded (one head) and on every core (one head
    per core, OpenMP over (sequence, head) pairs), each repeated for about
    ``seconds``; tokens/s scaled to the config's 32 heads and full_tokens
    (heads are independent and the recurrence's cost is linear in tokens)."""
    import workloads as W
    from oracle import oracle as O

    H, K, V = 32, 128, 128
    T = sum(lens)
    res = {}
    for key, threads in (("single_thread", 1), ("all_core", _cpu_threads())):
        heads = min(max(threads, 1), H)
        case = W.prefill_case("cpu_sample", heads, K, V, lens, len(lens), -5.0, seed=3900)
        O.set_threads(threads)
        cu = case.cu_seqlens.tolist()
        reps, t0 = 0, time.perf_counter()
        while True:
            O.prefill(case.inputs, case.pool, case.state_indices, cu, heads, K, V, lower_bound=-5.0,
                      return_pool=False)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
        per_call = el / reps * (H / heads) * (full_tokens / T)
        res[key] = {"value": round(full_tokens / per_call, 1), "unit": "tokens/s", "cores": O.max_threads(),
                    "kind": "oracle",
                    "sample": f"{reps} x {heads} head(s) of {len(lens)} sequence(s), {T} tokens, K=V=128, "
                              f"fp64 recurrent oracle, {el:.1f} s wall; scaled to 32 heads and "
                              f"{full_tokens} tokens"}
    return res


def leg_conv(steps, warmup, lens, name, seed):
    """Short causal conv prologue (width 4) producing mixed_qkv for a batch:
    reads x and the conv states, writes mixed_qkv and the new conv states."""
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V, Wd = 32, 128, 128, 4
    D = 2 * H * K + H * V
    rows, n = sum(lens), len(lens)
    ci = W.make_conv(rows, H, K, V, Wd, 2 * n, seed)
    x, w, b = ci["x"].to(dev), ci["weight"].to(dev), ci["bias"].to(dev)
    state = ci["conv_state"].to(dev)
    idx = [torch.arange(c * n, (c + 1) * n, dtype=torch.int32, device=dev) for c in range(2)]
    cu = W.cu_from_lengths(lens).to(dev)
    out = torch.empty(rows, D, dtype=torch.bfloat16, device=dev)

    def step(i):
        kda.kda_short_conv(x, w, b, state, idx[i % 2], cu, H=H, K=K, V=V, out=out)

    ms, _ = graph_time(step, 2, steps, warmup)
    io = rows * D * 2 * 2 + 2 * n * (Wd - 1) * D * 2
    return {"workload": name, "ms_per_step": round(ms, 5), "rows_per_s": round(rows / (ms * 1e-3), 1),
            "io_gbs": round(io / (ms * 1e-3) / 1e9, 1), "io_bytes_per_step": io}


def leg_conv_decode(steps, warmup, n=32):
    """Decode of n one-token requests (H=32, K=V=128) with the width-4 conv
    prologue fused (kda_conv_decode_packed), against the two-pass pipeline
    (kda_short_conv, then kda_decode_packed) on the same inputs; 2 GiB of state
    in rotation, as in the decode leg."""
    import torch

    import gated_delta_rule_45_amd as kda
    import workloads as W

    dev = torch.device("cuda")
    H, K, V, Wd = 32, 128, 128, 4
    slots = 1024
    pool = _device_pool(slots, H, K, V, 0.05, 3200, dev)
    inp = _device_token_inputs(n, H, K, V, 3201, dev)
    ci = W.make_conv(n, H, K, V, Wd, slots, 3202)
    x, w, b, cs = ci["x"].to(dev), ci["weight"].to(dev), ci["bias"].to(dev), ci["conv_state"].to(dev)
    perm = torch.randperm(slots, generator=W._gen(3203)).to(torch.int32)
    sets = slots // n
    idx = [perm[i * n:(i + 1) * n].to(dev) for i in range(sets)]
    cu = torch.arange(0, n + 1, dtype=torch.int32, device=dev)
    out = torch.empty(n, H, V, dtype=torch.bfloat16, device=dev)
    mixed = torch.empty(n, 2 * H * K + H * V, dtype=torch.bfloat16, device=dev)

    def fused(i):
        kda.kda_conv_decode_packed(x, w, b, cs, inp["raw_g"], inp["raw_beta"], inp["A_log"], inp["dt_bias"],
                                   -5.0, pool, idx[i % sets], out=out)

    def two_pass(i):
        kda.kda_short_conv(x, w, b, cs, idx[i % sets], cu, H=H, K=K, V=V, out=mixed)
        kda.kda_decode_packed(mixed, inp["raw_g"], inp["raw_beta"], inp["A_log"], inp["dt_bias"], -5.0,
                              pool, idx[i % sets], out=out)

    ms_f, _ = graph_time(fused, sets, steps, warmup)
    ms_t, _ = graph_time(two_pass, sets, steps, warmup)
    state_bytes = 2 * n * H * K * V * 4
    return {"workload": f"conv_decode_h32_k128_n{n}_w4", "us_per_step_fused": round(ms_f * 1e3, 3),
            "us_per_step_two_pass": round(ms_t * 1e3, 3),
            "state_gbs_fused": round(state_bytes / (ms_f * 1e-3) / 1e9, 1)}


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
    ov = kda.Overlap()  # decode rows on a caller-owned side stream beside the prefill

    def step(i):
        kda.kda_mixed_batch(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                            inp["dt_bias"], -5.0, pool, tables[i % sets][:, 0], D, cu, out=out,
                            workspace=ws, overlap=ov)

    ms, _ = graph_time(step, sets, steps, warmup)
    return {"workload": "mixed_d96_p4000_h32_k128", "ms_per_step": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1)}


def cpu_baseline(seconds: float):
    """The fp64 oracle (recurrent form, as it stands) on a bounded sample of
    the decode workload: the same 32 requests on a compact 32-slot pool,
    repeated until about ``seconds`` of wall time have passed."""
    import workloads as W
    from oracle import oracle as O

    H, K, V, N = 32, 128, 128, 32
    case = W.decode_case("cpu_sample", H, K, V, N, 1, N, 8, -5.0, seed=1020, pool_seed=77)

    def run(threads, secs):
        O.set_threads(threads)
        O.decode_packed(case.inputs, case.pool, case.state_indices, H, K, V, 1, -5.0)  # load, warm
        reps = 0
        t0 = time.perf_counter()
        while True:
            O.decode_packed(case.inputs, case.pool, case.state_indices, H, K, V, 1, -5.0)
            reps += 1
            el = time.perf_counter() - t0
            if el >= secs:
                break
        state_bytes = 2 * N * H * K * V * 4 * reps
        return {"value": round(state_bytes / el / 1e9, 3), "unit": "GB/s", "cores": O.max_threads(),
                "kind": "oracle",
                "sample": f"{reps} repeats of the 32-request batched decode (H=32, K=V=128) through "
                          f"the fp64 recurrent oracle on a 32-slot pool, {el:.1f} s wall"}

    single = run(1, seconds / 4)
    res = run(_cpu_threads(), seconds)
    res["single_thread"] = single
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the KDA library runs on one GPU per process (heads and sequences shard across GPUs with no exchange); --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    import gated_delta_rule_45_amd as kda

    kda.lib()  # fail loudly here if the HIP library is missing
    legs = set(args.legs.split(","))

    dec = leg_decode(args.steps, args.warmup)
    extra = {}
    if "decode" in legs:
        # The other decode variants of the configuration: stride 1, and no lower bound.
        for key, kw in (("decode_stride1", {"stride": 1}), ("decode_lbNone", {"lower_bound": None})):
            d = leg_decode(args.steps, args.warmup, **kw)
            extra[key] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in d.items()
                          if k != "steps_timed"}
            extra[key]["hbm_frac"] = round(d["achieved_gbs"] / HBM_PEAK_GBS, 4)
    if "spec" in legs:
        extra["spec_verify"] = leg_spec(max(args.steps // 4, 64), 16)
        extra["spec_decode_per_token_states"] = leg_spec_states(max(args.steps // 4, 64), 16)
    import workloads as W

    pf_steps = max(args.steps // 32, 6)
    vl = W.random_lengths(64, 1, 256, 3001, force_ones=2)
    # name -> (lengths, workload, seed, steps, warmup, lower bound, CPU sample lengths, full tokens,
    # smallest workspace); "--legs prefill" runs them all, "--legs prefill_t8192" (etc.) one of them.
    prefill_legs = {
        "prefill_t8192": ([8192], "prefill_t8192_h32_k128", 3000, pf_steps, 2, -5.0, [8192], 8192, False),
        "prefill_varlen64": (vl, "prefill_varlen64_h32_k128", 3002, pf_steps, 2, -5.0, vl, sum(vl), False),
        "prefill_t65536": ([65536], "prefill_t65536_h32_k128", 3004, max(pf_steps // 2, 4), 1, -5.0,
                           [8192], 65536, False),
        "prefill_t8192_lbNone": ([8192], "prefill_t8192_h32_k128_lbNone", 3000, pf_steps, 2, None, None, 0,
                                 False),
        # The same 8192-token call with the smallest accepted workspace (no chunk records).
        "prefill_t8192_min_workspace": ([8192], "prefill_t8192_h32_k128_min_workspace", 3000, pf_steps, 2,
                                        -5.0, None, 0, True),
    }
    for key, (lens, wl, seed, st, wu, lb, lens_s, full, minws) in prefill_legs.items():
        if "prefill" not in legs and key not in legs:
            continue
        leg = leg_prefill(st, wu, lens, wl, seed, lower_bound=lb, min_workspace=minws)
        leg["roofline"] = prefill_roofline(leg)
        if lens_s is not None and not args.no_cpu_baseline:
            leg["cpu_baseline"] = cpu_prefill_baseline(lens_s, full, args.cpu_seconds / 5)
        extra[key] = leg
    if "mixed" in legs:
        extra["mixed_4096"] = leg_mixed(max(args.steps // 16, 9), 9)
    if "conv" in legs:
        # Short causal conv prologue: the decode batch and one 8192-token sequence.
        extra["conv_prologue_decode_n32"] = leg_conv(args.steps, args.warmup, [1] * 32,
                                                     "conv_prologue_decode_h32_k128_n32_w4", 3100)
        extra["conv_prologue_t8192"] = leg_conv(max(args.steps // 8, 16), 4, [8192],
                                                "conv_prologue_t8192_h32_k128_w4", 3101)
        extra["conv_decode_fused_n32"] = leg_conv_decode(args.steps, args.warmup)
    if "norm" in legs:
        # Gated RMSNorm output epilogue: inside the decode kernel (whole-row
        # tiles) and inside the prefill state pass.
        d = leg_decode(args.steps, args.warmup, with_norm=True)
        extra["decode_gated_rmsnorm"] = {k: (round(v, 5) if isinstance(v, float) else v)
                                         for k, v in d.items() if k != "steps_timed"}
        extra["prefill_t8192_gated_rmsnorm"] = leg_prefill(max(args.steps // 32, 6), 2, [8192],
                                                           "prefill_t8192_h32_k128_gated_rmsnorm",
                                                           3000, with_norm=True)

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
                   "slot_sets_rotated": 16, "timing": "hip graph replay of 16 calls",
                   "eager_ms_per_step": round(dec["eager_ms_per_step"], 5),
                   "hbm_frac_state_only": round(dec["state_gbs"] / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(dec["achieved_gbs"], 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec["achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "decode_kernel<128,128,128>",
                     "launch_us": round(dec["ms_per_step"] * 1e3, 3),
                     "alg_bytes_per_launch": dec["alg_bytes_per_launch"]},
        "cpu_baseline": cpu,
        "legs": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
