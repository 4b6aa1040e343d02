"""GPU parity of the chunked prefill (chunk 64) and the mixed-batch router
against the fp64 oracle.

Chunked prefill with the WY recompute_w_u step and the rule that decode rows
of a mixed batch go to the recurrent kernel come from vLLM PR #50649
(Purpose); the length-1 cases target the NaN that page describes for
length-1 sequences in the chunk kernel, and every output is scanned for
non-finite or garbage-sized values (the ~1e38 values of its racy config).
"""
import math

import numpy as np
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import (DECODE_TOL_O, DECODE_TOL_S, PREFILL_TOL_O, PREFILL_TOL_S, cast_aware_err,
                         check_case, log, rel_err, run_gpu, run_oracle, to_device)
from oracle import oracle as O

pytestmark = pytest.mark.gpu

RAGGED = [1, 5, 63, 64, 65, 130, 200, 1]


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_ragged_prefill(K, V, lower_bound):
    case = W.prefill_case(f"ragged_k{K}_v{V}_lb{lower_bound}", 3, K, V, RAGGED, 16, lower_bound,
                          seed=601 + K + V, std=0.1, scale=1.0 / math.sqrt(K))
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


@pytest.mark.parametrize("lower_bound", [-5.3, -12.0])
def test_prefill_steep_lower_bound(lower_bound):
    """A bound steep enough that a 16-row block can decay by more than the
    factored path allows (15 |lb| > 79): the host must still launch the
    exact-path kernel for the chunks the factored one hands over."""
    case = W.prefill_case(f"steep_lb{lower_bound}", 3, 128, 128, RAGGED, 16, lower_bound,
                          seed=607, std=0.1, scale=1.0 / math.sqrt(128))
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


def test_prefill_initial_state_flags_null_slot_and_empty_sequence():
    lens = [70, 0, 33, 1, 128]
    case = W.prefill_case("flags", 4, 128, 128, lens, 12, -5.0, seed=611, std=0.2,
                          has_initial=[1, 1, 0, 1, 0], index_stride=3)
    case.block_table[3, 0] = -1   # a padded request on the null slot
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


def test_prefill_single_long_sequence_8192():
    check_case(W.prefill_8192(), PREFILL_TOL_O, PREFILL_TOL_S)


def test_prefill_varlen_64_sequences():
    check_case(W.prefill_varlen(), PREFILL_TOL_O, PREFILL_TOL_S)


def test_prefill_varlen_no_lower_bound():
    case = W.prefill_varlen(None)
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


# Long sequences are cut into segments whose states are composed
# (S_out = M S_in + B per segment) before every later segment runs in
# parallel. At H=3 the sequences of more than 12 chunks (2100, 1100, 4200 and
# 2500 tokens: 33, 18, 66 and 40 chunks) are cut into 6, 3, 11 and 7
# segments of balanced lengths (the last chunks ragged); the short ones stay
# whole.
CUT = [2100, 5, 1100, 1, 4200, 64, 2500]


@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_prefill_cut_sequences(K, V, lower_bound):
    case = W.prefill_case(f"cut_k{K}_v{V}_lb{lower_bound}", 3, K, V, CUT, 16, lower_bound,
                          seed=651 + K + V, std=0.1, scale=1.0 / math.sqrt(K))
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


def test_prefill_cut_sequences_with_flags_and_null_slot():
    """Cut sequences without an initial state and on the null slot (zero
    output, no state traffic), beside an uncut one, at index stride 3."""
    lens = [1500, 2500, 2200, 70, 3000]
    case = W.prefill_case("cut_flags", 4, 128, 128, lens, 12, -5.0, seed=661, std=0.2,
                          has_initial=[1, 1, 0, 1, 0], index_stride=3)
    case.block_table[1, 0] = -1
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


def test_prefill_many_sequences_with_a_cut_one():
    """Sixteen sequences at H = 16, one of them long enough (47 chunks) to
    be cut (into 8 segments), beside short uncut ones."""
    lens = [3000, 1, 64, 65, 17, 130, 2, 90, 33, 127, 5, 64, 200, 1, 48, 77]
    case = W.prefill_case("one_buffer_cut", 16, 128, 128, lens, 24, -5.0, seed=681, std=0.1)
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


def _round256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("K,V,lower_bound", [(128, 128, -5.0), (128, 64, None), (64, 128, -5.0)])
def test_prefill_records_and_min_workspace(K, V, lower_bound):
    """Long sequences with chunk records (a full workspace: the first launch
    keeps every chunk's state-step operands for the second) and without
    them (the smallest accepted workspace: both launches build them), each
    at the prefill bars. With records exactly the chunks of the cut
    sequences' later segments get a record: at H = 8 the 3100-, 700- and
    900-token sequences (49, 11 and 15 chunks) are cut into 9, 2 and 3
    segments, the others stay whole."""
    H = 8
    lens = [3100, 64, 700, 1, 900]
    case = W.prefill_case(f"records_k{K}_v{V}_lb{lower_bound}", H, K, V, lens, 8, lower_bound,
                          seed=841 + K + V, std=0.1, scale=1.0 / math.sqrt(K))
    N, T = len(lens), sum(lens)
    full = kda.kda_chunk_prefill_workspace_size(N, T, H, K, V)
    small = kda.kda_chunk_prefill_workspace_min_size(N, T, H, K, V)
    assert 0 < small < full
    ref = run_oracle(case)
    ws = torch.full((full,), 0xA5, dtype=torch.uint8, device="cuda")
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S, oracle=ref, workspace=ws)
    # Chunk slots of the call (sequence by sequence) and the ones of
    # segments 1 .. n - 1 of the cut sequences (balanced split).
    rec = 64 * K * 2 * 2 + 64 * 64 * 2 + K * 64 * 2 + K * 4 + 64 * V * 4
    rec_bound = T // 64 + N
    base = _round256(small)
    assert base + H * rec_bound * rec == full
    segs = {0: 9, 2: 2, 4: 3}
    expect, c0 = set(), 0
    for i, n in enumerate(lens):
        nch = (n + 63) // 64
        if i in segs:
            expect.update(range(c0 + nch // segs[i], c0 + nch))  # segment 0 is chunks [0, nch / ns)
        c0 += nch
    recs = ws[base:].view(H, rec_bound, rec).cpu()
    written = (recs != 0xA5).any(dim=2)
    got = {c for c in range(rec_bound) if bool(written[:, c].all())}
    untouched = {c for c in range(rec_bound) if not bool(written[:, c].any())}
    assert got == expect and untouched == set(range(rec_bound)) - expect, (sorted(got), sorted(expect))
    ws_min = torch.full((small,), 0xA5, dtype=torch.uint8, device="cuda")
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S, oracle=ref, workspace=ws_min)
    log(f"[case] records k{K} v{V} lb={lower_bound}: {len(expect)} records per head written; "
        f"both schedules at the prefill bars")


def test_prefill_cut_sequence_is_deterministic():
    case = W.prefill_case("det_cut", 2, 128, 128, [4000, 40], 4, -5.0, seed=671)
    results = []
    for _ in range(3):
        dc = to_device(case)
        out = run_gpu(dc).cpu()
        results.append((out, dc.pool.cpu()))
    for out, pool in results[1:]:
        assert torch.equal(out, results[0][0]) and torch.equal(pool, results[0][1])
    log("[case] cut-sequence prefill determinism: 3 runs bit-identical")


def test_prefill_is_deterministic():
    case = W.prefill_case("det", 8, 128, 128, [300, 77, 1], 8, -5.0, seed=621)
    results = []
    for _ in range(3):
        dc = to_device(case)
        out = run_gpu(dc).cpu()
        results.append((out, dc.pool.cpu()))
    for out, pool in results[1:]:
        assert torch.equal(out, results[0][0]) and torch.equal(pool, results[0][1])
    log("[case] prefill determinism: 3 runs bit-identical")


def test_mixed_batch_4096():
    """cfg4 at full size: the batch at the prefill bars, and its 96 decode
    rows (recurrent kernel, 128-column tiles) also at the decode bars
    (cast-aware output error <= 2e-3, state <= 1e-3) and bit-identical to a
    plain decode call on the same rows."""
    case = W.mixed_4096()
    ref_out, ref_fs = run_oracle(case)
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S, oracle=(ref_out, ref_fs))
    D = case.num_decodes
    dc = to_device(case)
    out = run_gpu(dc)
    got = out[:D].float().cpu().numpy().astype(np.float64)
    e_oc = cast_aware_err(got, ref_out[:D])
    slots = case.state_indices[:D].tolist()
    got_s = dc.pool[torch.tensor(slots, device=dc.pool.device)].cpu().numpy().astype(np.float64)
    e_s = rel_err(got_s, np.stack([ref_fs[i] for i in range(D)]))
    log(f"[case] mixed_4096 decode rows: e_o_cast={e_oc:.3e} e_S={e_s:.3e}")
    assert e_oc <= DECODE_TOL_O and e_s <= DECODE_TOL_S
    dc2 = to_device(case)
    i = dc2.inputs
    out_dec, _ = kda.kda_decode_packed(i["mixed_qkv"][:D], i["raw_g"][:D], i["raw_beta"][:D], i["A_log"],
                                       i["dt_bias"], case.lower_bound, dc2.pool, dc2.state_indices[:D])
    assert torch.equal(out[:D], out_dec)


def test_mixed_batch_decode_rows_match_decode_kernel():
    """The decode rows of a mixed batch are bit-identical to a plain decode
    call on the same rows (they take the recurrent kernel, not the chunk path)."""
    case = W.mixed_case("mixed_vs_decode", 4, 128, 128, 9, [40, 1, 90], 40, -5.0, seed=631)
    dc = to_device(case)
    out_mixed = run_gpu(dc)
    D = case.num_decodes
    dc2 = to_device(case)
    i = dc2.inputs
    out_dec, _ = kda.kda_decode_packed(i["mixed_qkv"][:D], i["raw_g"][:D], i["raw_beta"][:D],
                                       i["A_log"], i["dt_bias"], -5.0, dc2.pool,
                                       dc2.state_indices[:D])
    assert torch.equal(out_mixed[:D], out_dec)


def _head_slice(case: W.Case, heads):
    """The same case restricted to a subset of heads (heads are independent)."""
    H, K, V = case.H, case.K, case.V
    qkv = case.inputs["mixed_qkv"]
    cols = ([h * K + i for h in heads for i in range(K)] +
            [H * K + h * K + i for h in heads for i in range(K)] +
            [2 * H * K + h * V + j for h in heads for j in range(V)])
    inp = {
        "mixed_qkv": qkv[:, cols].contiguous(),
        "raw_g": case.inputs["raw_g"].view(-1, H, K)[:, heads].reshape(qkv.shape[0], -1).contiguous(),
        "raw_beta": case.inputs["raw_beta"][:, heads].contiguous(),
        "A_log": case.inputs["A_log"][heads].contiguous(),
        "dt_bias": case.inputs["dt_bias"].view(H, K)[heads].reshape(-1).contiguous(),
    }
    return inp, case.pool[:, heads].contiguous()


def test_prefill_65536_sampled_heads():
    """One 65 536-token sequence at full size (all 32 heads on the GPU, as the
    benchmark launches it); the oracle checks a sample of heads."""
    case = W.prefill_65536()
    dc = to_device(case)
    out = run_gpu(dc)
    heads = [0, 21]
    inp, pool = _head_slice(case, heads)
    ref_out, ref_fs, _ = O.prefill(inp, pool, case.state_indices, case.cu_seqlens.tolist(), len(heads),
                                   case.K, case.V, lower_bound=case.lower_bound, return_pool=False)
    got = out[:, heads].float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    e_o = rel_err(got, ref_out)
    slot = int(case.state_indices[0])
    got_s = dc.pool[slot, heads].cpu().numpy().astype(np.float64)
    e_s = rel_err(got_s, ref_fs[0])
    log(f"[case] prefill_t65536 heads {heads}: e_o={e_o:.3e} e_S={e_s:.3e}")
    assert e_o <= PREFILL_TOL_O and e_s <= PREFILL_TOL_S


@pytest.mark.parametrize("spread", ["uniform", "heavy"])
def test_prefill_exact_path_extreme_decays(spread):
    """Gates far past the factored limit, without a lower bound: e^{A_log} =
    16 on every head and raw_g around 3 ("uniform": about 49 per token, so
    every 16-row block and most 4-row sub-blocks decay by more than 80), or
    raw_g with a heavy spread ("heavy": a mix of tiny and huge per-token
    decays inside one block). Ragged lengths, one long enough to be cut."""
    lens = [1, 37, 64, 130, 300, 1500]
    case = W.prefill_case(f"extreme_{spread}", 4, 128, 128, lens, 8, None, seed=701, std=0.1,
                          scale=1.0 / math.sqrt(128))
    g = torch.Generator().manual_seed(702)
    rows = case.inputs["raw_g"].shape[0]
    if spread == "uniform":
        raw = 3.0 + 0.3 * torch.randn(rows, 4 * 128, generator=g)
    else:
        raw = 4.0 * torch.randn(rows, 4 * 128, generator=g)
    case.inputs["raw_g"] = raw.to(torch.bfloat16)
    case.inputs["A_log"] = torch.full((4,), math.log(16.0), dtype=torch.float32)
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)


@pytest.mark.parametrize("records", [True, False])
def test_prefill_two_cut_sequences_h32_sampled_heads(records):
    """Two sequences cut into at least three segments each at H = 32 and
    K = V = 128: the scan has 2 x 32 x 8 = 512 items on a grid of at most one
    workgroup per CU, so each workgroup takes two (the second sequence's on
    its second pass). With and without chunk records; the oracle checks a
    sample of heads, outputs and both final states."""
    lens = [2000, 2500, 300]
    case = W.prefill_case(f"two_cut_h32_rec{records}", 32, 128, 128, lens, 8, -5.0, seed=691, std=0.1)
    dc = to_device(case)
    T, H, K, V, N = sum(lens), 32, 128, 128, len(lens)
    size = (kda.kda_chunk_prefill_workspace_size if records else kda.kda_chunk_prefill_workspace_min_size)(
        N, T, H, K, V)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    i = dc.inputs
    out, _ = kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"],
                                   case.lower_bound, dc.pool, dc.state_indices, dc.cu_seqlens,
                                   scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    plan = ws[:16 + 2 * (N + 1) * 4].view(torch.int32).cpu().tolist()
    assert plan[0] == 0 and plan[3] == 2, f"expected two cut sequences, plan counts {plan[:4]}"
    seg_start = plan[4 + N + 1:4 + 2 * (N + 1)]
    nseg = [seg_start[k + 1] - seg_start[k] for k in range(N)]
    assert nseg[0] >= 3 and nseg[1] >= 3 and nseg[2] == 1, nseg
    heads = [0, 13, 31]
    inp, pool = _head_slice(case, heads)
    ref_out, ref_fs, _ = O.prefill(inp, pool, case.state_indices, case.cu_seqlens.tolist(), len(heads),
                                   K, V, lower_bound=case.lower_bound, scale=case.scale, return_pool=False)
    got = out[:, heads].float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    e_o = rel_err(got, ref_out)
    e_s = max(rel_err(dc.pool[int(case.state_indices[k]), heads].cpu().numpy().astype(np.float64), ref_fs[k])
              for k in range(N))
    log(f"[case] two cut sequences H=32 records={records} segments {nseg} heads {heads}: "
        f"e_o={e_o:.3e} e_S={e_s:.3e}")
    assert e_o <= PREFILL_TOL_O and e_s <= PREFILL_TOL_S


@pytest.mark.parametrize("T", [1, 3, 8])
def test_cross_path_decodes_prefill_spec_verify(T):
    """T single-token decodes = one prefill of T = one spec-verify call of T
    tokens (each against the oracle, and against each other)."""
    case = W.prefill_case(f"cross_{T}", 8, 128, 128, [T], 4, -5.0, seed=641 + T, std=0.1)
    dc = to_device(case)
    out_pre = run_gpu(dc)
    pool_pre = dc.pool.clone()
    dc2 = to_device(case)
    i = dc2.inputs
    out_spec, _ = kda.kda_decode_packed(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                        i["dt_bias"], -5.0, dc2.pool, dc2.state_indices,
                                        tokens_per_seq=T)
    dc3 = to_device(case)
    i = dc3.inputs
    outs = []
    for t in range(T):
        o, _ = kda.kda_decode_packed(i["mixed_qkv"][t:t + 1], i["raw_g"][t:t + 1],
                                     i["raw_beta"][t:t + 1], i["A_log"], i["dt_bias"], -5.0,
                                     dc3.pool, dc3.state_indices)
        outs.append(o)
    out_dec = torch.cat(outs)
    torch.cuda.synchronize()
    ref, ref_fs, _ = O.prefill(case.inputs, case.pool, case.state_indices, [0, T], 8, 128, 128,
                               lower_bound=-5.0, return_pool=False)
    slot = int(case.state_indices[0])
    for name, o, pool, tol in (("prefill", out_pre, pool_pre, PREFILL_TOL_O),
                               ("spec", out_spec, dc2.pool, DECODE_TOL_O * 2),
                               ("decodes", out_dec, dc3.pool, DECODE_TOL_O * 2)):
        e = rel_err(o.float().cpu().numpy(), ref)
        es = rel_err(pool[slot].cpu().numpy().astype(np.float64), ref_fs[0])
        log(f"[case] cross T={T} {name}: e_o={e:.3e} e_S={es:.3e}")
        assert e <= tol and es <= PREFILL_TOL_S
    # Spec-verify and T single decodes run the same recurrence in fp32.
    e = rel_err(out_spec.float().cpu().numpy(), out_dec.float().cpu().numpy().astype(np.float64))
    assert e <= DECODE_TOL_O * 2


def test_prefill_split_equals_whole():
    T1, T2 = 100, 93
    case = W.prefill_case("split", 4, 128, 128, [T1 + T2], 4, -5.0, seed=651)
    dc = to_device(case)
    out_whole = run_gpu(dc)
    pool_whole = dc.pool.clone()
    dc2 = to_device(case)
    i = dc2.inputs
    cu1 = torch.tensor([0, T1], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, T2], dtype=torch.int32, device="cuda")
    o1, _ = kda.kda_chunk_prefill(i["mixed_qkv"][:T1], i["raw_g"][:T1], i["raw_beta"][:T1],
                                  i["A_log"], i["dt_bias"], -5.0, dc2.pool, dc2.state_indices, cu1)
    o2, _ = kda.kda_chunk_prefill(i["mixed_qkv"][T1:].contiguous(), i["raw_g"][T1:].contiguous(),
                                  i["raw_beta"][T1:].contiguous(), i["A_log"], i["dt_bias"], -5.0,
                                  dc2.pool, dc2.state_indices, cu2)
    torch.cuda.synchronize()
    e = rel_err(torch.cat([o1, o2]).float().cpu().numpy(), out_whole.float().cpu().numpy().astype(np.float64))
    slot = int(case.state_indices[0])
    es = rel_err(dc2.pool[slot].cpu().numpy(), pool_whole[slot].cpu().numpy().astype(np.float64))
    log(f"[case] split vs whole: e_o={e:.3e} e_S={es:.3e}")
    assert e <= PREFILL_TOL_O and es <= PREFILL_TOL_S


def test_mixed_batches_from_two_host_threads():
    """With an overlap handle the router runs a batch's decode rows on the
    handle's side stream, forked from the caller's stream after the plan and
    joined back. Two host threads, each on its own stream with its own pool
    and its own handle, call it repeatedly at the same time; every output and
    final state must still match the oracle."""
    import threading

    cases = [W.mixed_case(f"threads_{n}", 4, 128, 128, 7, [90, 1, 40], 16, -5.0, seed=671 + n)
             for n in range(2)]
    refs = [run_oracle(c) for c in cases]
    results = [None, None]
    errors = []

    def worker(n):
        try:
            c = cases[n]
            s = torch.cuda.Stream()
            ov = kda.Overlap()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(4):
                    dc = to_device(c)
                    i = dc.inputs
                    o, _ = kda.kda_mixed_batch(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                               i["dt_bias"], -5.0, dc.pool, dc.state_indices,
                                               c.num_decodes, dc.cu_seqlens, overlap=ov)
                    outs.append((o, dc))
                s.synchronize()
            ov.close()
            results[n] = outs
        except Exception as exc:  # reported on the main thread
            errors.append(repr(exc))

    threads = [threading.Thread(target=worker, args=(n,)) for n in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    for n, c in enumerate(cases):
        ref_out, ref_fs = refs[n]
        idx = c.state_indices.tolist()
        for o, dc in results[n]:
            e = rel_err(o.float().cpu().numpy().astype(np.float64), ref_out)
            es = max(rel_err(dc.pool[s].cpu().numpy().astype(np.float64), ref_fs[i])
                     for i, s in enumerate(idx) if s >= 0)
            log(f"[case] thread {n}: e_o={e:.3e} e_S={es:.3e}")
            assert e <= PREFILL_TOL_O and es <= PREFILL_TOL_S


@pytest.mark.parametrize("cu", [[0, 100, 50, 200], [0, 100, 150, 190], [5, 100, 150, 200]],
                         ids=["decreasing", "short_of_num_tokens", "not_from_zero"])
def test_prefill_bad_cu_seqlens_sets_status_and_nan_rows(cu):
    """cu_seqlens outside the contract (the host never reads them, so the
    call itself succeeds): the workspace's status word becomes
    KDA_PREFILL_BAD_CU_SEQLENS, every output row is NaN and no slot changes.
    A valid call on the same workspace then clears the status."""
    case = W.prefill_case("bad_cu", 4, 128, 128, [100, 50, 50], 8, -5.0, seed=641)
    dc = to_device(case)
    i = dc.inputs
    snapshot = dc.pool.clone()
    T = 200
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(3, T, 4, 128, 128), dtype=torch.uint8,
                     device="cuda")
    bad = torch.tensor(cu, dtype=torch.int32, device="cuda")
    out, _ = kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"],
                                   -5.0, dc.pool, dc.state_indices, bad, workspace=ws)
    torch.cuda.synchronize()
    assert kda.prefill_status(ws) == kda.PREFILL_BAD_CU_SEQLENS
    assert torch.isnan(out.float()).all()
    assert torch.equal(dc.pool, snapshot)
    out2, _ = kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"],
                                    -5.0, dc.pool, dc.state_indices, dc.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    assert kda.prefill_status(ws) == 0
    assert torch.isfinite(out2.float()).all()
    log(f"[case] bad cu_seqlens {cu}: status word set, {out.numel()} NaN outputs, slots untouched")


@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_prefill_cut_sequence_weak_decay(lower_bound):
    """With dt_bias shifted down by 10 the per-token decay is close to 1
    (|g| ~ 1e-4), so a segment's map M stays far from zero and the scan's
    composition S_{j+1} = M_j S_j + B_j carries real weight (with the pages'
    gate inputs M underflows to zero over a segment). A 4096-token sequence
    at H = 8 is cut into segments; parity at the prefill bars, and the
    workspace maps must hold a sizeable M."""
    case = W.prefill_case("cut_weak_decay", 8, 128, 128, [4096, 300], 8, lower_bound, seed=821)
    case.inputs["dt_bias"] = case.inputs["dt_bias"] - 10.0
    check_case(case, PREFILL_TOL_O, PREFILL_TOL_S)
    dc = to_device(case)
    T, H, K, V = 4396, 8, 128, 128
    ws = torch.zeros(kda.kda_chunk_prefill_workspace_size(2, T, H, K, V), dtype=torch.uint8, device="cuda")
    i = dc.inputs
    kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"], i["dt_bias"],
                          lower_bound, dc.pool, dc.state_indices, dc.cu_seqlens, workspace=ws)
    torch.cuda.synchronize()
    off, item, n = kda.kda_chunk_prefill_workspace_maps(2, T, H, K, V)
    m = ws[off:off + n * item].view(n, item)[:, :K * K * 4].contiguous().view(torch.bfloat16).float()
    m_max = float(m.abs().max())
    log(f"[case] cut_weak_decay lb={lower_bound}: max|M| = {m_max:.3e}")
    assert m_max > 0.05
