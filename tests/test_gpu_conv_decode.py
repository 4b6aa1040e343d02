"""GPU parity of the decode entry with the short conv prologue fused
(kda_conv_decode_packed).

vLLM PR #60683 (Purpose) runs the conv step, the KDA recurrence and the norm
in one decode kernel. The fused entry is checked two ways:
  - against this library's two-pass pipeline (kda_short_conv writing
    mixed_qkv, then kda_decode_packed), bit for bit in outputs, KDA states
    and conv states, wherever the two-pass decode runs the same per-token
    kernel (one token per request, or at least 256 (request, head) pairs);
  - against the fp64 oracle (its conv, the conv output rounded to bf16 as
    mixed_qkv is, then its recurrence) for spec-verify-sized requests, at the
    decode bars, with the new conv states bit for bit.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import DECODE_TOL_O, DECODE_TOL_S, cast_aware_err, log, rel_err
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _inputs(num_seqs, tps, H, K, V, width, seed, null=()):
    rows = num_seqs * tps
    slots = max(64, 2 * num_seqs + 8)
    ti = W.make_token_inputs(rows, H, K, V, seed)  # raw_g, raw_beta, A_log, dt_bias (mixed_qkv unused)
    ci = W.make_conv(rows, H, K, V, width, slots, seed + 1, bias=width != 3)
    pool = W.make_pool(slots, H, K, V, 0.05, seed + 2).clone()
    table = W.make_block_table(num_seqs, 2, slots, seed + 3, null_rows=null)
    return ti, ci, pool, table


def _dev(t):
    return None if t is None else t.to("cuda")


def _fused(ti, ci, pool, table, tps, lb):
    pool_d, cs = pool.to("cuda"), ci["conv_state"].to("cuda")
    out, _, _ = kda.kda_conv_decode_packed(_dev(ci["x"]), _dev(ci["weight"]), _dev(ci["bias"]), cs,
                                           _dev(ti["raw_g"]), _dev(ti["raw_beta"]), _dev(ti["A_log"]),
                                           _dev(ti["dt_bias"]), lb, pool_d, table.to("cuda")[:, 0],
                                           tokens_per_seq=tps)
    torch.cuda.synchronize()
    return out.cpu(), pool_d.cpu(), cs.cpu()


def _two_pass(ti, ci, pool, table, tps, lb, H, K, V):
    pool_d, cs = pool.to("cuda"), ci["conv_state"].to("cuda")
    idx = table.to("cuda")[:, 0]
    rows = ci["x"].shape[0]
    cu = torch.arange(0, rows + 1, tps, dtype=torch.int32, device="cuda")
    mixed, _ = kda.kda_short_conv(_dev(ci["x"]), _dev(ci["weight"]), _dev(ci["bias"]), cs, idx, cu,
                                  H=H, K=K, V=V)
    out, _ = kda.kda_decode_packed(mixed, _dev(ti["raw_g"]), _dev(ti["raw_beta"]), _dev(ti["A_log"]),
                                   _dev(ti["dt_bias"]), lb, pool_d, idx, tokens_per_seq=tps)
    torch.cuda.synchronize()
    return out.cpu(), pool_d.cpu(), cs.cpu()


@pytest.mark.parametrize("num_seqs,tps,H,K,V,width,lb", [
    (32, 1, 32, 128, 128, 4, -5.0),   # 1024 pairs: whole heads, the conv state written in-kernel
    (8, 1, 32, 128, 128, 3, None),    # 256 pairs: 64-column tiles, then the conv-state pass
    (2, 1, 32, 128, 128, 2, -5.0),    # 64 pairs: 16-column tiles
    (64, 2, 8, 64, 128, 4, -5.0),     # 512 pairs, 2 tokens: whole heads
    (40, 3, 8, 128, 64, 4, None),     # 320 pairs, 3 tokens, V = 64: whole heads
    (16, 1, 16, 64, 64, 4, -5.0),     # K = V = 64
])
def test_fused_conv_decode_matches_two_pass(num_seqs, tps, H, K, V, width, lb):
    ti, ci, pool, table = _inputs(num_seqs, tps, H, K, V, width, seed=9100 + num_seqs + tps + width,
                                  null=(1,))
    fo, fp, fc = _fused(ti, ci, pool, table, tps, lb)
    to, tp, tc = _two_pass(ti, ci, pool, table, tps, lb, H, K, V)
    assert torch.equal(fo, to), "outputs differ from the two-pass pipeline"
    assert torch.equal(fp, tp), "KDA states differ from the two-pass pipeline"
    assert torch.equal(fc, tc), "conv states differ from the two-pass pipeline"
    null = int(table[1, 0])
    assert null < 0 and torch.all(fo[tps:2 * tps] == 0)
    log(f"[case] conv_decode {num_seqs}x{tps} h{H} k{K} v{V} w{width}: bit-identical to two passes")


@pytest.mark.parametrize("num_seqs,tps,width,lb", [(2, 4, 4, -5.0), (1, 8, 3, None), (3, 5, 2, -5.0)])
def test_fused_conv_decode_vs_oracle(num_seqs, tps, width, lb):
    H, K, V = 32, 128, 128
    null = (2,) if num_seqs > 2 else ()
    ti, ci, pool, table = _inputs(num_seqs, tps, H, K, V, width, seed=9300 + tps, null=null)
    fo, fp, fc = _fused(ti, ci, pool, table, tps, lb)
    rows = num_seqs * tps
    idx = table[:, 0]
    cu = list(range(0, rows + 1, tps))
    y, st_ref = O.short_conv(ci["x"], ci["weight"], ci["bias"], ci["conv_state"], idx, cu, H, K, V)
    inp = dict(ti)
    inp["mixed_qkv"] = torch.from_numpy(y).to(torch.bfloat16)  # mixed_qkv is bf16 between the passes
    ref, fs, _ = O.decode_packed(inp, pool, idx, H, K, V, tokens_per_seq=tps, lower_bound=lb,
                                 return_pool=False)
    got = fo.float().numpy().astype(np.float64)
    e_o, e_oc = rel_err(got, ref), cast_aware_err(got, ref)
    live = [n for n in range(num_seqs) if int(idx[n]) >= 0]
    fin = np.stack([fp[int(idx[n])].double().numpy() for n in live])
    e_s = rel_err(fin, fs[live])
    for n in live:
        s = int(idx[n])
        assert np.array_equal(fc[s].double().numpy(), st_ref[s]), f"conv state of slot {s}"
    log(f"[case] conv_decode {num_seqs}x{tps} w{width} lb={lb}: e_o={e_o:.3e} e_o_cast={e_oc:.3e} e_S={e_s:.3e}")
    assert e_oc <= DECODE_TOL_O and e_s <= DECODE_TOL_S
