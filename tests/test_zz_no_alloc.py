"""The no-alloc chunked prefill (kda_chunk_prefill_noalloc) against the
workspace entry point (kda_chunk_prefill) it mirrors: two calls in a row on
the library's static scratch, the second with a smaller input, each
bit-identical to the workspace call from the same starting state and within
the prefill bar of the fp64 oracle; a size whose chunk records do not fit
the scratch, bit-identical to the workspace call with the smallest accepted
workspace (no records). Sizes beyond the scratch are rejected before
anything is launched."""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import PREFILL_TOL_O, PREFILL_TOL_S, log, rel_err, run_oracle, to_device

pytestmark = pytest.mark.gpu


def _call(fn, dc, **kw):
    c = dc.case
    i = dc.inputs
    out, _ = fn(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"], c.lower_bound,
                dc.pool, dc.state_indices, dc.cu_seqlens, has_initial_state=dc.has_initial_state,
                scale=c.scale, **kw)
    torch.cuda.synchronize()
    return out


def _check(case):
    need = kda.kda_chunk_prefill_workspace_size(len(case.cu_seqlens) - 1, case.rows, case.H, case.K, case.V)
    log(f"[case] no-alloc {case.name}: rows={case.rows} workspace={need} B")
    assert need <= kda.NOALLOC_SCRATCH_BYTES
    dc_ws = to_device(case)
    out_ws = _call(kda.kda_chunk_prefill, dc_ws)
    dc_na = to_device(case)
    out_na = _call(kda.kda_chunk_prefill_noalloc, dc_na)
    assert torch.equal(out_na, out_ws), "output differs from kda_chunk_prefill"
    assert torch.equal(dc_na.pool, dc_ws.pool), "state pool differs from kda_chunk_prefill"
    ref_out, ref_fs = run_oracle(case)
    got = out_na.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    e_o = rel_err(got, ref_out)
    idx = case.state_indices.tolist()
    e_s = max(rel_err(dc_na.pool[s].cpu().numpy().astype(np.float64), ref_fs[i])
              for i, s in enumerate(idx) if s >= 0)
    log(f"[case] no-alloc {case.name}: bit-identical to the workspace call; e_o={e_o:.3e} e_S={e_s:.3e}")
    assert e_o <= PREFILL_TOL_O and e_s <= PREFILL_TOL_S


def test_noalloc_prefill_matches_workspace_prefill_twice():
    # First call: a long sequence that the plan cuts into segments, beside
    # short ones (4 heads, K = V = 128).
    big = W.prefill_case("noalloc_big", 4, 128, 128, [2100, 1, 70, 130], 12, -5.0, seed=801,
                         std=0.1, scale=1.0 / math.sqrt(128))
    _check(big)
    # Second call, smaller: the scratch still holds the first call's words.
    small = W.prefill_case("noalloc_small", 4, 128, 128, [1, 5, 63, 64, 65], 12, None, seed=802,
                           std=0.1, has_initial=[1, 0, 1, 1, 0])
    _check(small)


def test_noalloc_prefill_without_records_matches_min_workspace_prefill():
    # One 8192-token sequence at H = 8: the plan and maps fit the scratch,
    # the chunk records (93 MB) do not, so the no-alloc call runs the
    # schedule without records, as kda_chunk_prefill does with the smallest
    # accepted workspace: bit-identical to that, and at the prefill bars.
    case = W.prefill_case("noalloc_norec", 8, 128, 128, [8192], 4, -5.0, seed=803, std=0.1,
                          scale=1.0 / math.sqrt(128))
    N, T = 1, 8192
    small = kda.kda_chunk_prefill_workspace_min_size(N, T, 8, 128, 128)
    assert small <= kda.NOALLOC_SCRATCH_BYTES < kda.kda_chunk_prefill_workspace_size(N, T, 8, 128, 128)
    log(f"[case] no-alloc noalloc_norec: rows={T} min workspace={small} B")
    dc_ws = to_device(case)
    ws = torch.empty(small, dtype=torch.uint8, device="cuda")
    out_ws = _call(kda.kda_chunk_prefill, dc_ws, workspace=ws)
    dc_na = to_device(case)
    out_na = _call(kda.kda_chunk_prefill_noalloc, dc_na)
    assert torch.equal(out_na, out_ws), "output differs from kda_chunk_prefill without records"
    assert torch.equal(dc_na.pool, dc_ws.pool), "state pool differs from kda_chunk_prefill without records"
    ref_out, ref_fs = run_oracle(case)
    got = out_na.float().cpu().numpy().astype(np.float64)
    e_o = rel_err(got, ref_out)
    s = int(case.state_indices[0])
    e_s = rel_err(dc_na.pool[s].cpu().numpy().astype(np.float64), ref_fs[0])
    log(f"[case] no-alloc noalloc_norec: bit-identical to the smallest-workspace call; e_o={e_o:.3e} e_S={e_s:.3e}")
    assert e_o <= PREFILL_TOL_O and e_s <= PREFILL_TOL_S


def test_noalloc_prefill_rejects_sizes_beyond_the_scratch():
    # Two 8192-token sequences at H = 32 need more segment maps than the
    # scratch holds; the call is refused on the host, so the inputs' values
    # do not matter.
    H, K, V, T = 32, 128, 128, 16384
    need = kda.kda_chunk_prefill_workspace_size(2, T, H, K, V)
    assert need > kda.NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda")
    qkv = torch.zeros(T, 2 * H * K + H * V, dtype=torch.bfloat16, device=dev)
    raw_g = torch.zeros(T, H * K, dtype=torch.bfloat16, device=dev)
    raw_beta = torch.zeros(T, H, dtype=torch.bfloat16, device=dev)
    A_log = torch.zeros(H, device=dev)
    dt_bias = torch.zeros(H * K, device=dev)
    pool = torch.ones(2, H, K, V, device=dev)
    idx = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    cu = torch.tensor([0, 8192, T], dtype=torch.int32, device=dev)
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_chunk_prefill_noalloc(qkv, raw_g, raw_beta, A_log, dt_bias, -5.0, pool, idx, cu)
    torch.cuda.synchronize()
    assert ei.value.status == 3 and any("static scratch" in r for r in ei.value.reasons)
    assert bool((pool == 1).all())
    log(f"[case] no-alloc: two 8192-token sequences at H=32 ({need} B of workspace) are rejected before any launch")
