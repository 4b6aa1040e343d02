"""The oracle against the hand-worked fixtures in tests/golden/.

The source pages print no KDA values, so each fixture is an example worked
by hand in exact arithmetic (its derivation is in the file). These tests fix
the oracle's recurrence, chunked form, gate, beta, packed-row layout, strided
slot addressing and in-place pool update to those closed forms.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["hand_worked_k2_v1.json", "hand_worked_scalar.json"])
def test_pregated_recurrence_and_chunked_form(name):
    fx = _load(name)
    i, e = fx["inputs"], fx["expected"]
    g = np.log(np.array(i["alpha"], dtype=np.float64))
    args = (np.array(i["q"], float), np.array(i["k"], float), np.array(i["v"], float), g,
            np.array(i["beta"], float), np.array(i["S0"], float))
    o, S = O.recurrent_pregated(*args, scale=i["scale"])
    np.testing.assert_allclose(o, e["o"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(S, e["S"], rtol=1e-14, atol=1e-15)
    for C in (1, 2, 3):
        oc, Sc = O.chunked_pregated(*args, C, scale=i["scale"])
        np.testing.assert_allclose(oc, e["o"], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(Sc, e["S"], rtol=1e-13, atol=1e-14)


def test_gate_and_beta_closed_forms():
    fx = _load("gate_closed_forms.json")
    for c in fx["gate"]:
        got = O.gate(c["raw_g"], c["A_log"], c["dt_bias"], c["lower_bound"])
        assert got == pytest.approx(c["g"], rel=1e-13), c["closed_form"]
    for c in fx["beta"]:
        assert O.beta(c["raw_beta"]) == pytest.approx(c["beta"], rel=1e-13), c["closed_form"]


def _decode_inputs(i):
    bf = torch.bfloat16
    return {
        "mixed_qkv": torch.tensor(i["mixed_qkv"], dtype=torch.float32).to(bf),
        "raw_g": torch.tensor(i["raw_g"], dtype=torch.float32).to(bf),
        "raw_beta": torch.tensor(i["raw_beta"], dtype=torch.float32).to(bf),
        "A_log": torch.tensor(i["A_log"], dtype=torch.float32),
        "dt_bias": torch.tensor(i["dt_bias"], dtype=torch.float32),
    }


@pytest.mark.parametrize("variant", ["no_lower_bound", "lower_bound_-2"])
def test_packed_decode_through_the_gated_entry(variant):
    fx = _load("packed_decode_h2.json")
    i, e = fx["inputs"], fx["expected"][variant]
    H, K, V = i["H"], i["K"], i["V"]
    pool = torch.tensor(i["pool"], dtype=torch.float32).reshape(-1, H, K, V)
    bt = torch.tensor(i["block_table"], dtype=torch.int32)
    idx = bt[:, 0]
    assert idx.stride(0) == bt.shape[1]
    out, _, pool_after = O.decode_packed(_decode_inputs(i), pool, idx, H, K, V, 1,
                                         e.get("lower_bound"), i["scale"])
    np.testing.assert_allclose(out.reshape(len(e["out"]), H), e["out"], rtol=1e-6)
    np.testing.assert_allclose(pool_after.reshape(-1, H), e["pool"], rtol=1e-6)
    # The untouched slot is bit-identical.
    assert np.array_equal(pool_after.reshape(-1, H)[1], np.array(i["pool"][1], dtype=np.float32))


def test_prefill_of_the_same_rows_as_one_sequence():
    fx = _load("packed_decode_h2.json")
    i, e = fx["inputs"], fx["expected"]["prefill_both_rows_on_slot_2"]
    H, K, V = i["H"], i["K"], i["V"]
    pool = torch.tensor(i["pool"], dtype=torch.float32).reshape(-1, H, K, V)
    out, _, pool_after = O.prefill(_decode_inputs(i), pool, torch.tensor([2], dtype=torch.int32),
                                   e["cu_seqlens"], H, K, V, lower_bound=None, scale=i["scale"])
    np.testing.assert_allclose(out.reshape(2, H), e["out"], rtol=1e-6)
    np.testing.assert_allclose(pool_after.reshape(-1, H)[2], e["slot_2"], rtol=1e-6)
