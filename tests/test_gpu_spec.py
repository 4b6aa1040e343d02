"""GPU parity of speculative decoding with a state per token against the
fp64 oracle: the initial state comes from block-table column
num_accepted-1, the state after every token goes to its own column (vLLM
PR #51682 report, Purpose: the state slot is column 0 of a block table of
1 + num_speculative_blocks columns; vLLM PR #60683, Refusal and steps:
padded requests carry a null slot and one accepted token)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import DECODE_TOL_O, DECODE_TOL_S, cast_aware_err, log, rel_err
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _run(case: W.Case, table: torch.Tensor):
    dev = torch.device("cuda")
    inp = {k: v.to(dev) for k, v in case.inputs.items()}
    pool = case.pool.to(dev)
    acc = case.num_accepted.to(dev)
    out, _ = kda.kda_spec_decode(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                                 inp["dt_bias"], case.lower_bound, pool, table.to(dev), acc,
                                 tokens_per_seq=case.tokens_per_seq, scale=case.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), pool.cpu()


def _check(case: W.Case, table: torch.Tensor | None = None):
    table = case.block_table if table is None else table
    got, pool_after = _run(case, table)
    H, K, V, T = case.H, case.K, case.V, case.tokens_per_seq
    ref, states, _ = O.spec_decode(case.inputs, case.pool, table, case.num_accepted, H, K, V, T,
                                   lower_bound=case.lower_bound, scale=case.scale, return_pool=False)
    assert np.all(np.isfinite(got))
    e_o, e_oc = rel_err(got, ref), cast_aware_err(got, ref)
    tab = table[:, :T].tolist()
    acc = case.num_accepted.tolist()
    written, e_s = set(), 0.0
    for n in range(len(tab)):
        if tab[n][acc[n] - 1] < 0:
            assert np.all(got[n * T:(n + 1) * T] == 0.0), "padded request rows not zero"
            continue
        for t in range(T):
            sl = tab[n][t]
            if sl < 0:
                continue
            written.add(sl)
            e_s = max(e_s, rel_err(pool_after[sl].numpy().astype(np.float64), states[n, t]))
    untouched = [s for s in range(case.pool.shape[0]) if s not in written]
    assert torch.equal(pool_after[untouched], case.pool[untouched]), "an unwritten slot changed"
    log(f"[case] {case.name}: e_o={e_o:.3e} e_o_cast={e_oc:.3e} e_S(all tokens)={e_s:.3e} "
        f"slots written={len(written)}")
    assert e_oc <= DECODE_TOL_O and e_s <= DECODE_TOL_S


@pytest.mark.parametrize("layout", sorted(W.SPEC_LAYOUTS))
@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_spec_decode_per_token_states(layout, lower_bound):
    real, tps, nulls = W.SPEC_LAYOUTS[layout]
    n = real + nulls
    case = W.spec_decode_case(f"spec_states_{layout}_lb{lower_bound}", 32, 128, 128, n, tps,
                              num_slots=512, lower_bound=lower_bound, seed=5100 + tps,
                              null_rows=tuple(range(real, n)), pool_seed=2999)
    _check(case)


def test_spec_decode_per_token_states_seven_tokens():
    # 128 (request, head) pairs (32-column tiles), 7 of 8 token places, a
    # padded request.
    case = W.spec_decode_case("spec_states_4x7_h32", 32, 128, 128, 4, 7, num_slots=64,
                              lower_bound=-5.0, seed=5400, null_rows=(3,), pool_seed=2999)
    _check(case)


def test_spec_decode_null_columns_strided_table_and_small_heads():
    # Every other column of a wider table (column stride 2), some null entries,
    # K = V = 64.
    case = W.spec_decode_case("spec_strided_k64", 4, 64, 64, 3, 4, num_slots=64, lower_bound=-5.0,
                              seed=5200, width=8, std=0.1, null_cols=((0, 2), (2, 3)),
                              accepted=[4, 2, 1])
    wide = case.block_table.to("cuda")     # [3, 8], distinct slots
    table = wide[:, ::2]                   # a strided [3, 4] view on the device
    assert table.stride() == (8, 2)
    case.block_table = table.cpu()
    _check(case, table)


@pytest.mark.parametrize("tps", [1, 4, 8])
def test_one_accepted_token_matches_plain_decode(tps):
    """With one accepted token the initial state is column 0's, as in plain
    decode; the outputs agree bit for bit (same kernel arithmetic), and the
    state stored after the last token equals plain decode's final state: bit
    for bit with one token, and up to fp32 rounding with several (plain
    decode applies a block of tokens as one rank-T update, the per-token path
    token by token, and e^{G} of a running sum G carries a relative error
    of about |G| 2^-24 where the per-token products round eight times)."""
    n = 8 // tps
    case = W.spec_decode_case(f"spec_vs_decode_{tps}", 32, 128, 128, n, tps, num_slots=512,
                              lower_bound=-5.0, seed=5300 + tps, accepted=[1] * n, pool_seed=2999)
    dev = torch.device("cuda")
    got, pool_spec = _run(case, case.block_table)
    inp = {k: v.to(dev) for k, v in case.inputs.items()}
    pool = case.pool.to(dev)
    out, _ = kda.kda_decode_packed(inp["mixed_qkv"], inp["raw_g"], inp["raw_beta"], inp["A_log"],
                                   inp["dt_bias"], -5.0, pool, case.block_table[:, 0].to(dev),
                                   tokens_per_seq=tps)
    torch.cuda.synchronize()
    assert np.array_equal(got, out.float().cpu().numpy().astype(np.float64))
    worst = 0.0
    for r in range(n):
        a = pool_spec[int(case.block_table[r, tps - 1])]
        b = pool.cpu()[int(case.block_table[r, 0])]
        if tps == 1:
            assert torch.equal(a, b)
        else:
            worst = max(worst, float((a - b).abs().max() / b.abs().max()))
    assert worst <= 1e-5, worst
    log(f"[case] spec vs plain decode, {n} x {tps}: outputs bit-identical, final states rel diff {worst:.2e}")
