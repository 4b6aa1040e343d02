"""Race evidence for the MFMA, LDS and LDS-DMA kernels. A racy
recompute_w_u configuration once produced ~1e38 garbage (vLLM PR #50649,
Purpose), and graph replays are checked in the hundreds there (vLLM PR
#60683, Test plan). Each check below repeats a call from the same starting
state and requires every repeat to be bit-identical to the first, stopping
at the first mismatch; the workspace scan looks for non-finite or
garbage-sized values in the only intermediate data that goes through HBM,
the segment maps (M and B) of a cut sequence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import log, run_gpu, to_device

pytestmark = pytest.mark.gpu

REPEATS = 100


def _repeat_identical(case, repeats=REPEATS, **kw):
    dc = to_device(case)
    start = dc.pool.clone()
    ref = run_gpu(dc, **kw).clone()
    pool_ref = dc.pool.clone()
    for rep in range(1, repeats):
        dc.pool.copy_(start)
        out = run_gpu(dc, **kw)
        assert torch.equal(out, ref), f"{case.name}: repeat {rep} output differs from the first call"
        assert torch.equal(dc.pool, pool_ref), f"{case.name}: repeat {rep} state differs from the first call"
    assert torch.isfinite(ref.float()).all() and float(ref.float().abs().max()) < 1e30
    log(f"[case] {case.name}: {repeats} calls bit-identical")


def test_prefill_8192_repeats_bit_identical():
    _repeat_identical(W.prefill_8192())


def test_prefill_varlen64_repeats_bit_identical():
    _repeat_identical(W.prefill_varlen())


def test_prefill_cut_sequence_repeats_bit_identical():
    # A 3000-token sequence at H = 8 is cut into segments (maps and scan)
    # beside short uncut ones; no lower bound, so exact-path chunks can occur.
    case = W.prefill_case("race_cut_h8", 8, 128, 128, [3000, 70, 1, 200], 16, None, seed=811)
    _repeat_identical(case)


@pytest.mark.parametrize("layout", ["1x8", "2x4"])
def test_spec_verify_repeats_bit_identical(layout):
    _repeat_identical(W.spec_verify(layout))


def _graph_replays(case, call, replays=REPEATS):
    dc = to_device(case)
    start = dc.pool.clone()
    out_e = call(dc)
    torch.cuda.synchronize()
    pool_e = dc.pool.clone()
    dc.pool.copy_(start)
    out_g = torch.empty_like(out_e)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(dc, out_g)
    torch.cuda.synchronize()
    for rep in range(replays):
        dc.pool.copy_(start)
        if rep % 10 == 0:  # eager work between some replays
            torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"{case.name}: replay {rep} output differs from eager"
        assert torch.equal(dc.pool, pool_e), f"{case.name}: replay {rep} state differs from eager"
    log(f"[case] graph {case.name}: {replays} replays bit-identical to eager")


def test_graph_prefill_cut_sequence_100_replays():
    case = W.prefill_case("race_graph_cut_h8", 8, 128, 128, [2500, 33, 400], 8, -5.0, seed=812)
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(3, 2933, 8, 128, 128), dtype=torch.uint8,
                     device="cuda")

    def call(dc, out=None):
        i = dc.inputs
        o, _ = kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                     i["dt_bias"], -5.0, dc.pool, dc.state_indices, dc.cu_seqlens,
                                     out=out, workspace=ws)
        return o

    _graph_replays(case, call)


def test_graph_spec_verify_100_replays():
    case = W.spec_verify("2x4")

    def call(dc, out=None):
        i = dc.inputs
        o, _ = kda.kda_decode_packed(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                     i["dt_bias"], -5.0, dc.pool, dc.state_indices,
                                     tokens_per_seq=4, out=out)
        return o

    _graph_replays(case, call)


@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_workspace_maps_finite_after_prefill(lower_bound):
    """Every segment map item a cut prefill writes (M as bf16 hi/lo MFMA
    fragments, B as fp32) is finite and below 1e30, and at least one item was
    written. The workspace starts zeroed, so items the call does not plan
    stay zero."""
    case = W.prefill_8192(lower_bound)
    dc = to_device(case)
    T, H, K, V = 8192, 32, 128, 128
    ws = torch.zeros(kda.kda_chunk_prefill_workspace_size(1, T, H, K, V), dtype=torch.uint8, device="cuda")
    i = dc.inputs
    kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"],
                          lower_bound, dc.pool, dc.state_indices, dc.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    assert kda.prefill_status(ws) == 0
    off, item, n = kda.kda_chunk_prefill_workspace_maps(1, T, H, K, V)
    assert n > 0 and off + n * item <= ws.numel()
    area = ws[off:off + n * item].view(n, item)
    m = area[:, :K * K * 4].contiguous().view(torch.bfloat16).float()
    b = area[:, K * K * 4:].contiguous().view(torch.float32)
    for name, x in (("M", m), ("B", b)):
        assert torch.isfinite(x).all(), f"non-finite {name} in the workspace maps"
        big = float(x.abs().max())
        assert big < 1e30, f"garbage-sized {name} in the workspace maps: {big:.3e}"
    written = int((b.abs().amax(dim=1) > 0).sum())
    assert written > 0
    log(f"[case] workspace maps lb={lower_bound}: {n} items, {written} written, "
        f"max|M|={float(m.abs().max()):.3e} max|B|={float(b.abs().max()):.3e}")


@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_workspace_records_finite_after_prefill(lower_bound):
    """Every chunk record a cut prefill writes with a full workspace (the
    state step's operand tiles -W, scale Q o e^gam, scale P and
    (K o e^{gam_last - gam})^T in bf16, then e^{gam_last} and U in fp32) is
    finite and below 1e30. The workspace starts zeroed, so slots the call
    does not fill stay zero; at 8192 tokens every head has records."""
    case = W.prefill_8192(lower_bound)
    dc = to_device(case)
    T, H, K, V, C = 8192, 32, 128, 128, 64
    full = kda.kda_chunk_prefill_workspace_size(1, T, H, K, V)
    ws = torch.zeros(full, dtype=torch.uint8, device="cuda")
    i = dc.inputs
    kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"],
                          lower_bound, dc.pool, dc.state_indices, dc.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    assert kda.prefill_status(ws) == 0
    # Records follow the rest of the workspace at the next 256-byte boundary,
    # one per (head, chunk slot), T / C + num_seqs slots per head.
    start = (kda.kda_chunk_prefill_workspace_min_size(1, T, H, K, V) + 255) // 256 * 256
    tiles = (2 * C * K + C * C + K * C) * 2
    rec = tiles + K * 4 + C * V * 4
    slots = T // C + 1
    assert start + H * slots * rec == full
    area = ws[start:].view(H * slots, rec)
    bf = area[:, :tiles].contiguous().view(torch.bfloat16).float()
    f32 = area[:, tiles:].contiguous().view(torch.float32)
    for name, x in (("operand tiles", bf), ("e^gam_last and U", f32)):
        assert torch.isfinite(x).all(), f"non-finite {name} in the chunk records"
        big = float(x.abs().max())
        assert big < 1e30, f"garbage-sized {name} in the chunk records: {big:.3e}"
    written = (area.view(H, slots, rec) != 0).any(dim=2).sum(dim=1)
    assert int(written.min()) > 0, "a head without records"
    log(f"[case] chunk records lb={lower_bound}: {int(written.sum())} of {H * slots} slots written, "
        f"max|tiles|={float(bf.abs().max()):.3e} max|U|={float(f32.abs().max()):.3e}")
