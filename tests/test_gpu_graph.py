"""The entry points allocate nothing and never synchronise, so they can be
captured in a HIP graph (padded graph replays are how the spec-verify path is
served, vLLM PR #60683, Refusal and steps). Each graph is replayed several
times with eager work and synchronisations in between, and every replay must
match an eager call from the same starting state bit for bit."""
import pytest
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from kda_testlib import log, to_device

pytestmark = pytest.mark.gpu


def _capture(call, dc, out_g):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(dc, out_g)
    torch.cuda.synchronize()
    return g


def _check_graph(case, call, capture_first=False, out_shape=None):
    """``capture_first``: the graph is captured before any eager call of this
    case (the capture itself does not execute the kernels); the eager
    reference follows from the same starting state."""
    dc = to_device(case)
    start = dc.pool.clone()
    if capture_first:
        out_g = torch.empty(out_shape, dtype=torch.bfloat16, device="cuda")
        g = _capture(call, dc, out_g)
        dc.pool.copy_(start)
        out_e = call(dc)
        torch.cuda.synchronize()
        pool_e = dc.pool.clone()
    else:
        # Eager reference from the starting state, then the capture.
        out_e = call(dc)
        torch.cuda.synchronize()
        pool_e = dc.pool.clone()
        dc.pool.copy_(start)
        out_g = torch.empty_like(out_e)
        g = _capture(call, dc, out_g)
    for rep in range(3):
        dc.pool.copy_(start)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: output differs from eager"
        assert torch.equal(dc.pool, pool_e), f"replay {rep}: state differs from eager"
        del junk
    log(f"[case] graph {case.name}: 3 replays bit-identical to eager")


def test_graph_decode_and_spec_verify():
    case = W.decode_case("graph_spec", 8, 128, 128, 4, 2, 16, 4, -5.0, seed=701, null_rows=(3,))

    def call(dc, out=None):
        i = dc.inputs
        o, _ = kda.kda_decode_packed(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                     i["dt_bias"], -5.0, dc.pool, dc.state_indices,
                                     tokens_per_seq=2, out=out)
        return o

    _check_graph(case, call)


def test_graph_prefill():
    case = W.prefill_case("graph_prefill", 8, 128, 128, [1, 100, 200], 8, -5.0, seed=702)
    ws = torch.empty(kda.kda_chunk_prefill_workspace_size(3, 301, 8, 128, 128), dtype=torch.uint8,
                     device="cuda")

    def call(dc, out=None):
        i = dc.inputs
        o, _ = kda.kda_chunk_prefill(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                     i["dt_bias"], -5.0, dc.pool, dc.state_indices, dc.cu_seqlens,
                                     out=out, workspace=ws)
        return o

    _check_graph(case, call)


@pytest.mark.parametrize("overlap", [False, True])
def test_graph_mixed_batch(overlap):
    """With an overlap handle the capture records a fork onto the handle's
    side stream (decode rows) and a join back (the handle is made outside the
    capture)."""
    case = W.mixed_case("graph_mixed", 8, 128, 128, 6, [70, 1, 33], 16, None, seed=703)
    ws = torch.empty(kda.kda_mixed_batch_workspace_size(6, 3, 104, 8, 128, 128), dtype=torch.uint8,
                     device="cuda")
    ov = kda.Overlap() if overlap else None

    def call(dc, out=None):
        i = dc.inputs
        o, _ = kda.kda_mixed_batch(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                   i["dt_bias"], None, dc.pool, dc.state_indices, 6, dc.cu_seqlens,
                                   out=out, workspace=ws, overlap=ov)
        return o

    _check_graph(case, call)
    if ov is not None:
        ov.close()


def test_graph_mixed_batch_capture_first():
    """The first call of a fresh overlap handle, and of this case, is made
    under capture; replays must match the eager call that follows."""
    case = W.mixed_case("graph_mixed_first", 8, 128, 128, 5, [1, 130, 64], 16, -5.0, seed=704)
    ws = torch.empty(kda.kda_mixed_batch_workspace_size(5, 3, 195, 8, 128, 128), dtype=torch.uint8,
                     device="cuda")
    ov = kda.Overlap()

    def call(dc, out=None):
        i = dc.inputs
        o, _ = kda.kda_mixed_batch(i["mixed_qkv"], i["raw_g"], i["raw_beta"], i["A_log"],
                                   i["dt_bias"], -5.0, dc.pool, dc.state_indices, 5, dc.cu_seqlens,
                                   out=out, workspace=ws, overlap=ov)
        return o

    _check_graph(case, call, capture_first=True, out_shape=(200, 8, 128))
    ov.close()
