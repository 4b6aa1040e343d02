"""GPU parity of the short causal conv prologue against the fp64 oracle.

vLLM PR #60683 (Purpose) names a conv step before the KDA recurrence in its
decode kernels without a formula; the reading (depthwise causal conv of
width W per [q | k | v] channel with a per-slot conv state, silu, per-head
L2 norm of q and k) is the oracle's. Outputs are compared to the bar of the
decode path (each element's bf16 cast allowed, e_o_cast <= 2e-3); the
new conv states are copies of bf16 inputs and must match bit for bit, and
every other slot must be untouched.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import DECODE_TOL_O, cast_aware_err, log, rel_err
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _run_conv(lens, H, K, V, width, seed, slots=16, index_stride=3, null=(), no_init=(), bias=True,
              x_row_pad=0, out_row_pad=0):
    dev = torch.device("cuda")
    rows = sum(lens)
    ci = W.make_conv(rows, H, K, V, width, slots, seed, bias=bias, x_row_pad=x_row_pad)
    D = 2 * H * K + H * V
    table = W.make_block_table(len(lens), index_stride, slots, seed + 5, null_rows=null)
    idx = table[:, 0]
    cu = W.cu_from_lengths(lens)
    hs = None
    if no_init:
        hs = torch.ones(len(lens), dtype=torch.uint8)
        for i in no_init:
            hs[i] = 0
    x = ci["x"]
    xd = x.as_strided((rows, x.stride(0)), (x.stride(0), 1)).to(dev)[:, :D] if rows else x.to(dev)
    state_d = ci["conv_state"].to(dev)
    out = None
    if out_row_pad:
        out = torch.zeros(rows, D + out_row_pad, dtype=torch.bfloat16, device=dev)[:, :D]
    got, _ = kda.kda_short_conv(xd, ci["weight"].to(dev), None if ci["bias"] is None else ci["bias"].to(dev),
                                state_d, table.to(dev)[:, 0], cu.to(dev), H=H, K=K, V=V,
                                has_initial_state=None if hs is None else hs.to(dev), out=out)
    torch.cuda.synchronize()
    ref, ref_state = O.short_conv(x, ci["weight"], ci["bias"], ci["conv_state"], idx, cu.tolist(), H, K, V,
                                  has_initial_state=None if hs is None else hs.tolist())
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(g))
    e_o, e_oc = rel_err(g, ref), cast_aware_err(g, ref)
    st_after = state_d.cpu()
    written = [int(idx[i]) for i in range(len(lens)) if int(idx[i]) >= 0 and lens[i] > 0]
    for s in written:   # copies of bf16 inputs: bit for bit
        assert np.array_equal(st_after[s].double().numpy(), ref_state[s]), f"conv state of slot {s}"
    others = [s for s in range(slots) if s not in written]
    assert torch.equal(st_after[others], ci["conv_state"][others]), "an unwritten conv-state slot changed"
    return e_o, e_oc, len(written)


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("width", [2, 3, 4])
def test_short_conv_varlen(K, V, width):
    # Sequences shorter than the history (1, 2 rows), an empty one, a null
    # slot, one without an initial state, padded input and output rows and a
    # strided slot view.
    lens = [1, 2, 5, 70, 0, 3, 130]
    e_o, e_oc, nw = _run_conv(lens, 3, K, V, width, seed=8000 + K + V + width, null=(2,), no_init=(3,),
                              bias=width != 3, x_row_pad=8, out_row_pad=16)
    log(f"[case] short_conv k{K} v{V} w{width}: e_o={e_o:.3e} e_o_cast={e_oc:.3e} states written={nw}")
    assert e_oc <= DECODE_TOL_O


@pytest.mark.parametrize("K,V,width", [(128, 128, 4), (64, 64, 3), (64, 128, 2)])
def test_short_conv_row_blocks_cross_sequences(K, V, width):
    """About 2000 rows: each workgroup takes a block of 7 rows, so blocks
    start mid-sequence and cross sequence boundaries (the input window is
    refilled at every sequence start), short sequences included."""
    lens = [300, 1, 2, 700, 5, 0, 64, 3, 900]
    e_o, e_oc, nw = _run_conv(lens, 2, K, V, width, seed=8300 + K + width, slots=24, null=(3,),
                              no_init=(4, 6))
    log(f"[case] short_conv row blocks k{K} v{V} w{width}: e_o={e_o:.3e} e_o_cast={e_oc:.3e} "
        f"states written={nw}")
    assert e_oc <= DECODE_TOL_O


def test_short_conv_decode_batch():
    """The decode shape: 32 one-row sequences, H = 32, K = V = 128, width 4."""
    e_o, e_oc, nw = _run_conv([1] * 32, 32, 128, 128, 4, seed=8100, slots=64, index_stride=8)
    log(f"[case] short_conv decode batch: e_o={e_o:.3e} e_o_cast={e_oc:.3e} states written={nw}")
    assert e_oc <= DECODE_TOL_O and nw == 32


def test_prologue_recurrence_epilogue_chain():
    """conv prologue -> packed decode (4 tokens per request) -> gated RMSNorm,
    against the oracle's chain. Each side rounds the prologue's output to
    bf16 itself, so a last-bit difference in mixed_qkv can move o by about
    2^-8 relative; the bar is the prefill one (1e-2)."""
    dev = torch.device("cuda")
    H, K, V, Wd, n, tps = 4, 128, 128, 4, 6, 4
    rows = n * tps
    ci = W.make_conv(rows, H, K, V, Wd, 16, 8200)
    case = W.decode_case("chain", H, K, V, n, tps, 16, 2, -5.0, seed=8201, std=0.1)
    nm = W.make_norm(rows, H, V, 8202)
    cu = torch.arange(0, rows + 1, tps, dtype=torch.int32)
    idx = case.state_indices
    # GPU chain
    mixed, _ = kda.kda_short_conv(ci["x"].to(dev), ci["weight"].to(dev), ci["bias"].to(dev),
                                  ci["conv_state"].to(dev), idx.to(dev), cu.to(dev), H=H, K=K, V=V)
    inp = {k: v.to(dev) for k, v in case.inputs.items()}
    out, _ = kda.kda_decode_packed(mixed, inp["raw_g"], inp["raw_beta"], inp["A_log"], inp["dt_bias"], -5.0,
                                   case.pool.to(dev), idx.to(dev), tokens_per_seq=tps,
                                   norm=kda.GatedRMSNorm(nm["gate"].to(dev), nm["weight"].to(dev), nm["eps"]))
    torch.cuda.synchronize()
    # Oracle chain
    y, _ = O.short_conv(ci["x"], ci["weight"], ci["bias"], ci["conv_state"], idx, cu.tolist(), H, K, V)
    oinp = dict(case.inputs, mixed_qkv=torch.from_numpy(y).float().to(torch.bfloat16))
    ref, _, _ = O.decode_packed(oinp, case.pool, idx, H, K, V, tokens_per_seq=tps, lower_bound=-5.0)
    ref = O.gated_rmsnorm(ref, nm["gate"], nm["weight"], nm["eps"])
    got = out.float().cpu().numpy().astype(np.float64)
    e = rel_err(got, ref)
    log(f"[case] conv -> decode -> norm chain: e_o={e:.3e}")
    assert np.all(np.isfinite(got)) and e <= 1e-2
