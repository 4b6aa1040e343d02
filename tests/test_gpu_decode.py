"""GPU parity of packed decode and spec-verify against the fp64 oracle.

The decode matrix follows the test described on the prhub report of vLLM PR
#51682 (section Implementation breakdown): num_seqs {1, 8, 32} x lower_bound
{-5, None} x state_indices stride {1, 8}, on the batched-decode shape (H=32,
K=V=128, 512-slot pool). Spec-verify layouts follow vLLM PR #60683 (Refusal
and steps): whole requests of k+1 rows, at most 8 rows, padded requests on a
null slot.
"""
import math

import pytest
import torch

import workloads as W
from kda_testlib import DECODE_TOL_O, DECODE_TOL_S, check_case, log, run_gpu, to_device

pytestmark = pytest.mark.gpu


def test_tiny_decode():
    check_case(W.tiny_decode(), DECODE_TOL_O, DECODE_TOL_S)


@pytest.mark.parametrize("num_seqs", [1, 8, 32])
@pytest.mark.parametrize("lower_bound", [-5.0, None])
@pytest.mark.parametrize("index_stride", [1, 8])
def test_batched_decode_matrix(num_seqs, lower_bound, index_stride):
    check_case(W.batched_decode(index_stride, lower_bound, num_seqs), DECODE_TOL_O, DECODE_TOL_S)


@pytest.mark.parametrize("layout", list(W.SPEC_LAYOUTS))
@pytest.mark.parametrize("lower_bound", [-5.0, None])
def test_spec_verify(layout, lower_bound):
    check_case(W.spec_verify(layout, lower_bound), DECODE_TOL_O, DECODE_TOL_S)


@pytest.mark.parametrize("H,K,V,n,tps,lower_bound", [
    (32, 128, 128, 5, 6, -5.0),  # 160 (request, head) pairs: 32-column tiles, 6 of 8 token places
    (32, 128, 128, 2, 5, None),  # 16-column tiles, 5 of 8 token places
    (16, 64, 128, 3, 7, -5.0),
    (8, 128, 64, 4, 3, None),    # 3 of 4 token places
])
def test_spec_verify_ragged_token_blocks(H, K, V, n, tps, lower_bound):
    """Requests of 2..8 tokens on tiles of at most 32 columns, which take the
    block form of the token chain, with token counts that leave places of
    the 4- or 8-token block empty, and a padded request on a null slot."""
    case = W.decode_case(f"block_h{H}_k{K}_v{V}_{n}x{tps}", H, K, V, n, tps, 64, 2, lower_bound,
                         seed=560 + tps, std=0.1, null_rows=(1,))
    check_case(case, DECODE_TOL_O, DECODE_TOL_S)


@pytest.mark.parametrize("lower_bound", [-7.5, -12.0])
def test_spec_verify_steep_lower_bounds(lower_bound):
    """One request of 8 tokens on 16-column tiles: at lb = -7.5 the factored
    form of the token-pair tables runs at its bound (running decays down to
    e^-60), at lb = -12 the per-channel form takes over."""
    case = W.decode_case(f"block_lb{lower_bound}", 32, 128, 128, 1, 8, 64, 2, lower_bound,
                         seed=590, std=0.1)
    check_case(case, DECODE_TOL_O, DECODE_TOL_S)


@pytest.mark.parametrize("K,V", [(64, 128), (128, 64), (64, 64)])
def test_other_head_dims(K, V):
    case = W.decode_case(f"dims_k{K}_v{V}", 3, K, V, 5, 3, 17, 2, None, seed=501, std=0.2,
                         null_rows=(1,), scale=1.0 / math.sqrt(K))
    check_case(case, DECODE_TOL_O, DECODE_TOL_S)


def test_padded_slot_stride_and_wide_qkv_rows():
    case = W.decode_case("padded_slot", 4, 128, 128, 6, 2, 9, 3, -5.0, seed=502, slot_pad=36)
    assert case.pool.stride(0) == 4 * 128 * 128 + 36
    # Rows of mixed_qkv also live in a wider buffer (row stride > 2*H*K + H*V).
    check_case(case, DECODE_TOL_O, DECODE_TOL_S, qkv_row_pad=64)


def test_decode_is_deterministic():
    """Repeated calls from the same state give bit-identical results."""
    case = W.batched_decode(8, -5.0, 8)
    outs, states = [], []
    for rep in range(3):
        dc = to_device(case)
        outs.append(run_gpu(dc).cpu())
        states.append(dc.pool[case.state_indices.long().cuda()].cpu())
    for rep in range(1, 3):
        assert torch.equal(outs[0], outs[rep])
        assert torch.equal(states[0], states[rep])
    log("[case] decode determinism: 3 runs bit-identical")
