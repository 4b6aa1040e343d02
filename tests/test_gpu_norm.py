"""GPU parity of the gated RMSNorm output epilogue against the fp64 oracle.

vLLM PR #60683 (Purpose) names a gated RMSNorm after the KDA recurrence in its
decode kernels without a formula; the reading (per row and head over V:
o / sqrt(mean(o^2) + eps) * weight * act(gate)) is the oracle's. Decode
applies it inside the kernel when a workgroup holds a head's whole row of V
channels (batches of >= 512 (request, head) pairs at V = 128, >= 256 at
V = 64) and as a pass over the output otherwise; prefill and the prefill
rows of a mixed batch always take the pass. Every path is compared here,
with null slots (zero rows), gate rows inside a wider buffer and both
activations.
"""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import (DECODE_TOL_O, DECODE_TOL_S, PREFILL_TOL_O, PREFILL_TOL_S, cast_aware_err,
                         check_case, log, rel_err)
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _with_norm(case: W.Case, seed: int, activation="sigmoid", row_pad=0) -> W.Case:
    case.norm = W.make_norm(case.rows, case.H, case.V, seed, activation=activation, row_pad=row_pad)
    return case


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("activation", ["sigmoid", "silu"])
def test_decode_norm_fused_whole_rows(K, V, activation):
    # 16 requests x 32 heads = 512 pairs: whole-row tiles, the in-kernel epilogue.
    case = W.decode_case(f"norm_fused_k{K}_v{V}_{activation}", 32, K, V, 16, 1, 64, 8, -5.0,
                         seed=7000 + K + V, std=0.1)
    case.block_table[3, 0] = -1
    _with_norm(case, 7100 + K + V, activation, row_pad=8)
    check_case(case, DECODE_TOL_O, DECODE_TOL_S, cast_aware=True)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64)])
@pytest.mark.parametrize("tps", [1, 4])
def test_decode_norm_separate_pass(K, V, tps):
    # 4 requests x 4 heads: 16-column tiles, the epilogue runs as a pass.
    case = W.decode_case(f"norm_pass_k{K}_v{V}_t{tps}", 4, K, V, 4, tps, 16, 3, None,
                         seed=7200 + K + tps, std=0.1)
    case.block_table[1, 0] = -1
    _with_norm(case, 7300 + K + tps, "silu" if tps == 4 else "sigmoid")
    check_case(case, DECODE_TOL_O, DECODE_TOL_S, cast_aware=True)


def test_decode_norm_paths_agree():
    """The in-kernel epilogue (one call over 16 requests) and the pass (the
    same requests in four calls of 4) give the same outputs to within the
    bf16 rounding of o that the pass starts from."""
    case = W.decode_case("norm_agree", 32, 128, 128, 16, 1, 64, 1, -5.0, seed=7400, std=0.1)
    _with_norm(case, 7401)
    dev = torch.device("cuda")
    inp = {k: v.to(dev) for k, v in case.inputs.items()}
    gate, weight = case.norm["gate"].to(dev), case.norm["weight"].to(dev)
    idx = case.state_indices.to(dev)
    pool_a, pool_b = case.pool.to(dev), case.pool.to(dev)
    whole, _ = kda.kda_decode_packed(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                                     inp["dt_bias"], -5.0, pool_a, idx,
                                     norm=kda.GatedRMSNorm(gate, weight, 1e-6))
    parts = []
    for i in range(4):
        r = slice(4 * i, 4 * i + 4)
        o, _ = kda.kda_decode_packed(inp["mixed_qkv"][r], inp["raw_g"][r], inp["raw_beta"][r],
                                     inp["A_log"], inp["dt_bias"], -5.0, pool_b, idx[r],
                                     norm=kda.GatedRMSNorm(gate[r], weight, 1e-6))
        parts.append(o)
    torch.cuda.synchronize()
    a = whole.float().cpu().numpy()
    b = torch.cat(parts).float().cpu().numpy()
    e = rel_err(a.astype(np.float64), b.astype(np.float64))
    log(f"[case] norm fused vs pass: max diff / max = {e:.3e}")
    assert e <= 8e-3
    # The states agree to fp32 summation order (the tile widths differ).
    assert rel_err(pool_a.cpu().numpy().astype(np.float64), pool_b.cpu().numpy().astype(np.float64)) < 1e-5


@pytest.mark.parametrize("layout", ["1x8", "4x2", "3x2+1null"])
def test_spec_decode_norm(layout):
    real, tps, nulls = W.SPEC_LAYOUTS[layout]
    n = real + nulls
    case = W.spec_decode_case(f"spec_norm_{layout}", 32, 128, 128, n, tps, num_slots=64,
                              lower_bound=-5.0, seed=7500 + tps, null_rows=tuple(range(real, n)))
    norm = W.make_norm(n * tps, 32, 128, 7600 + tps, activation="silu", row_pad=16)
    dev = torch.device("cuda")
    inp = {k: v.to(dev) for k, v in case.inputs.items()}
    pool = case.pool.to(dev)
    gate = norm["gate"]
    gate_d = gate.as_strided((gate.shape[0], gate.stride(0)), (gate.stride(0), 1)).to(dev)[:, :gate.shape[1]]
    out, _ = kda.kda_spec_decode(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                                 inp["dt_bias"], -5.0, pool, case.block_table.to(dev),
                                 case.num_accepted.to(dev), tokens_per_seq=tps,
                                 norm=kda.GatedRMSNorm(gate_d, norm["weight"].to(dev), norm["eps"], "silu"))
    torch.cuda.synchronize()
    ref, _, _ = O.spec_decode(case.inputs, case.pool, case.block_table, case.num_accepted, 32, 128, 128,
                              tps, lower_bound=-5.0, return_pool=False)
    ref = O.gated_rmsnorm(ref, gate, norm["weight"], norm["eps"], "silu")
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    for r in range(real, n):
        assert np.all(got[r * tps:(r + 1) * tps] == 0.0), "padded request rows not zero"
    e_o, e_oc = rel_err(got, ref), cast_aware_err(got, ref)
    log(f"[case] {case.name}: e_o={e_o:.3e} e_o_cast={e_oc:.3e}")
    assert e_oc <= DECODE_TOL_O


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64)])
def test_prefill_norm(K, V):
    lens = [1, 70, 0, 130, 2100, 64]
    case = W.prefill_case(f"prefill_norm_k{K}_v{V}", 3, K, V, lens, 16, -5.0, seed=7700 + K,
                          std=0.1, scale=1.0 / math.sqrt(K), has_initial=[1, 1, 1, 0, 1, 1])
    case.block_table[1, 0] = -1
    _with_norm(case, 7800 + K, "sigmoid", row_pad=8)
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


def test_mixed_batch_norm():
    """Decode rows (in-kernel epilogue: 512 pairs) and prefill rows (pass on
    the shifted gate rows) in one call."""
    case = W.mixed_case("mixed_norm", 32, 128, 128, 16, [40, 1, 300], 64, -5.0, seed=7900)
    _with_norm(case, 7901, "silu", row_pad=8)
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)
