"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before launching anything
(every failed check is reported at once). No call here reaches a kernel."""
import ctypes
import os
import re

import pytest
import torch

import gated_delta_rule_45_amd as kda
from gated_delta_rule_45_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("kda_decode_packed", "kda_chunk_prefill", "kda_mixed_batch"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = kda.lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, f"not exported: {missing}"


def test_status_strings_and_version():
    L = kda.lib()
    assert L.kda_status_string(0) == b"KDA_OK"
    assert L.kda_status_string(3) == b"KDA_ERR_WORKSPACE"
    assert b"gfx950" in L.kda_version()


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def _gate(**kw):
    d = dict(A_log=FAKE, dt_bias=FAKE, has_lower_bound=1, lower_bound=-5.0, scale=1.0)
    d.update(kw)
    return B.KdaGate(**d)


def _state(**kw):
    d = dict(pool=FAKE, slot_stride=32 * 128 * 128, num_slots=4, indices=FAKE, index_stride=8)
    d.update(kw)
    return B.KdaState(**d)


def _decode(num_seqs=4, tps=1, H=32, K=128, V=128, qkv=FAKE, stride=3 * 32 * 128, g=None, s=None,
            out=FAKE, norm=None):
    L = kda.lib()
    g = g or _gate()
    s = s or _state()
    st = L.kda_decode_packed(num_seqs, tps, H, K, V, qkv, stride, FAKE, FAKE, ctypes.byref(g),
                             ctypes.byref(s), ctypes.byref(norm) if norm is not None else None, out, None)
    return st, L.kda_last_error().decode()


def test_decode_rejects_and_lists_every_reason():
    st, msg = _decode(tps=9, K=96, s=_state(index_stride=0, pool=None), out=None)
    assert st == 1
    for frag in ("tokens_per_seq must be in 1..8", "K must be 64 or 128",
                 "index_stride must be >= 1", "pool must not be NULL", "out must not be NULL"):
        assert frag in msg, msg


def test_spec_decode_rejects_and_lists_every_reason():
    L = kda.lib()
    g, s = _gate(), _state()
    st = L.kda_spec_decode(4, 9, 32, 128, 128, FAKE, 3 * 32 * 128, FAKE, FAKE, ctypes.byref(g),
                           ctypes.byref(s), 0, None, None, FAKE, None)
    msg = L.kda_last_error().decode()
    assert st == 1
    for frag in ("tokens_per_seq must be in 1..8", "index_col_stride must be >= 1",
                 "num_accepted_tokens must not be NULL"):
        assert frag in msg, msg


def test_output_norm_rejects_and_lists_every_reason():
    bad = B.KdaOutNorm(gate=None, gate_row_stride=100, weight=FAKE + 4, eps=0.0, activation=7)
    st, msg = _decode(norm=bad)
    assert st == 1
    for frag in ("norm->activation", "norm->eps must be finite and > 0", "norm->gate must not be NULL",
                 "norm->gate_row_stride must be >= H*V", "norm->weight must be 16-byte aligned"):
        assert frag in msg, msg
    ok = B.KdaOutNorm(gate=FAKE, gate_row_stride=32 * 128 + 8, weight=FAKE, eps=1e-6, activation=1)
    st, msg = _decode(norm=ok, out=None)
    assert st == 1 and "norm" not in msg and "out must not be NULL" in msg


def test_short_conv_rejects_and_lists_every_reason():
    L = kda.lib()
    cv = B.KdaShortConv(weight=None, bias=FAKE + 4, width=5, l2_eps=float("nan"), conv_state=FAKE,
                        conv_slot_stride=10, num_slots=0)
    st = L.kda_short_conv(2, 10, None, None, 32, 96, 128, FAKE, 100, ctypes.byref(cv), FAKE, 0,
                          FAKE, 3 * 32 * 128, None)
    msg = L.kda_last_error().decode()
    assert st == 1
    for frag in ("cu_seqlens must not be NULL", "K must be 64 or 128", "index_stride must be >= 1",
                 "conv->width must be 2, 3 or 4", "conv->l2_eps", "conv->weight must not be NULL",
                 "conv->bias must be 16-byte aligned", "conv->num_slots", "x_row_stride must be >="):
        assert frag in msg, msg
    # Output overlapping the input is refused.
    cv = B.KdaShortConv(weight=FAKE, bias=None, width=4, l2_eps=1e-6, conv_state=FAKE,
                        conv_slot_stride=3 * 3 * 32 * 128, num_slots=4)
    st = L.kda_short_conv(2, 10, FAKE, None, 32, 128, 128, FAKE, 3 * 32 * 128, ctypes.byref(cv), FAKE, 1,
                          FAKE + 3 * 32 * 128 * 2, 3 * 32 * 128, None)
    assert st == 1 and "must not overlap x" in L.kda_last_error().decode()


def test_conv_decode_rejects_and_lists_every_reason():
    L = kda.lib()
    g, s_ = _gate(), _state()
    cv = B.KdaShortConv(weight=None, bias=FAKE, width=5, l2_eps=1e-6, conv_state=FAKE,
                        conv_slot_stride=3 * 3 * 32 * 128, num_slots=2)
    st = L.kda_conv_decode_packed(4, 1, 32, 128, 128, FAKE + 2, 3 * 32 * 128 + 4, ctypes.byref(cv), FAKE,
                                  FAKE, ctypes.byref(g), ctypes.byref(s_), None, FAKE, None)
    msg = L.kda_last_error().decode()
    assert st == 1
    for frag in ("conv->width must be 2, 3 or 4", "conv->weight must not be NULL",
                 "conv->num_slots must be >= state->num_slots", "x must be 16-byte aligned",
                 "x_row_stride must be a multiple of 8"):
        assert frag in msg, msg
    st = L.kda_conv_decode_packed(4, 1, 32, 128, 128, FAKE, 3 * 32 * 128, None, FAKE, FAKE,
                                  ctypes.byref(g), ctypes.byref(s_), None, FAKE, None)
    assert st == 1 and "conv must not be NULL" in L.kda_last_error().decode()


def test_negative_index_stride_rejected():
    st, msg = _decode(s=_state(index_stride=-8))
    assert st == 1 and "index_stride" in msg


def test_bad_gate_values_rejected():
    st, msg = _decode(g=_gate(lower_bound=float("nan")))
    assert st == 1 and "lower_bound" in msg
    st, msg = _decode(g=_gate(lower_bound=0.5))
    assert st == 1 and "lower_bound" in msg
    st, msg = _decode(g=_gate(scale=float("inf")))
    assert st == 1 and "scale" in msg
    st, msg = _decode(g=_gate(A_log=None))
    assert st == 1 and "A_log" in msg


def test_alignment_and_strides_are_unsupported_not_invalid():
    st, msg = _decode(qkv=FAKE + 2)
    assert st == 2 and "mixed_qkv must be 16-byte aligned" in msg
    st, msg = _decode(stride=3 * 32 * 128 + 4)
    assert st == 2 and "multiple of 8" in msg
    st, msg = _decode(stride=100)
    assert st == 1 and "qkv_row_stride" in msg
    st, msg = _decode(stride=(1 << 24) + 8)
    assert st == 2 and "qkv_row_stride must be <= 2^24" in msg


def test_slot_stride_too_small():
    st, msg = _decode(s=_state(slot_stride=100))
    assert st == 1 and "slot_stride" in msg


def test_empty_decode_is_a_no_op():
    st, msg = _decode(num_seqs=0)
    assert st == 0 and msg == ""


def test_workspace_size_query():
    L = kda.lib()
    a = L.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128)
    b = L.kda_chunk_prefill_workspace_size(64, 8192, 32, 128, 128)
    c = L.kda_chunk_prefill_workspace_size(1, 65536, 32, 128, 128)
    assert 0 < a < b and a <= c  # a sequence has at most 8 map items at H=32
    assert L.kda_chunk_prefill_workspace_size(1, 10, 32, 96, 128) == 0
    assert L.kda_chunk_prefill_workspace_size(-1, 10, 32, 128, 128) == 0
    assert L.kda_mixed_batch_workspace_size(96, 5, 4000, 32, 128, 128) == \
        L.kda_chunk_prefill_workspace_size(5, 4000, 32, 128, 128)
    # The smallest accepted workspace leaves out the chunk records: one fp32
    # U tile and the bf16/fp32 operand tiles per chunk slot and head.
    lo = L.kda_chunk_prefill_workspace_min_size(1, 8192, 32, 128, 128)
    rec = 64 * 128 * 2 * 2 + 64 * 64 * 2 + 128 * 64 * 2 + 128 * 4 + 64 * 128 * 4
    assert 0 < lo < a and a - lo >= (8192 // 64 + 1) * 32 * rec
    assert L.kda_chunk_prefill_workspace_min_size(1, 10, 32, 96, 128) == 0


def test_prefill_rejects_missing_workspace_and_cu_seqlens():
    L = kda.lib()
    g, s = _gate(), _state(index_stride=1)
    st = L.kda_chunk_prefill(2, 100, None, None, 32, 128, 128, FAKE, 3 * 32 * 128, FAKE, FAKE,
                             ctypes.byref(g), ctypes.byref(s), None, FAKE, None, 0, None)
    msg = L.kda_last_error().decode()
    assert st == 1
    assert "cu_seqlens must not be NULL" in msg and "workspace" in msg
    need = L.kda_chunk_prefill_workspace_min_size(2, 100, 32, 128, 128)
    st = L.kda_chunk_prefill(2, 100, FAKE, None, 32, 128, 128, FAKE, 3 * 32 * 128, FAKE, FAKE,
                             ctypes.byref(g), ctypes.byref(s), None, FAKE, FAKE, need - 1, None)
    assert st == 3 and "workspace" in L.kda_last_error().decode()


def test_noalloc_prefill_rejects_sizes_beyond_its_scratch():
    """The no-alloc prefill has no workspace argument; a call whose workspace
    would exceed the static scratch is refused on the host, with every
    other failed check listed beside it."""
    L = kda.lib()
    g, s = _gate(), _state(index_stride=1)
    assert L.kda_chunk_prefill_workspace_size(2, 16384, 32, 128, 128) > B.NOALLOC_SCRATCH_BYTES
    st = L.kda_chunk_prefill_noalloc(2, 16384, FAKE, None, 32, 128, 128, FAKE, 3 * 32 * 128, FAKE,
                                     FAKE, ctypes.byref(g), ctypes.byref(s), None, FAKE, None)
    msg = L.kda_last_error().decode()
    assert st == 3 and "static scratch" in msg, msg
    st = L.kda_chunk_prefill_noalloc(2, 100, None, None, 32, 128, 128, FAKE, 3 * 32 * 128, FAKE,
                                     FAKE, ctypes.byref(g), ctypes.byref(s), None, None, None)
    msg = L.kda_last_error().decode()
    assert st == 1 and "cu_seqlens must not be NULL" in msg and "out must not be NULL" in msg


def test_mixed_rejects_negative_decodes():
    L = kda.lib()
    g, s = _gate(), _state()
    st = L.kda_mixed_batch(-1, 0, 0, None, None, 32, 128, 128, FAKE, 3 * 32 * 128, FAKE, FAKE,
                           ctypes.byref(g), ctypes.byref(s), None, FAKE, None, 0, None, None)
    assert st == 1 and "num_decodes" in L.kda_last_error().decode()


def test_binding_refuses_host_tensors_listing_each():
    t = torch.zeros(4, 3 * 4 * 64, dtype=torch.bfloat16)
    with pytest.raises(kda.KdaError) as ei:
        kda.kda_decode_packed(t, torch.zeros(4, 256, dtype=torch.bfloat16),
                              torch.zeros(4, 4, dtype=torch.bfloat16), torch.zeros(4),
                              torch.zeros(256), -5.0, torch.zeros(8, 4, 64, 64),
                              torch.zeros(4, dtype=torch.int32))
    reasons = ei.value.reasons
    assert sum("must be on a GPU" in r for r in reasons) == 7


def test_workspace_maps_query():
    """The segment-map area lies inside the workspace; one item is M (K*K*4
    bytes of bf16 hi/lo fragments) plus B (fp32 K*V); an 8192-token sequence
    at H = 32 has 8 map items per head."""
    off, item, n = kda.kda_chunk_prefill_workspace_maps(1, 8192, 32, 128, 128)
    assert item == (128 * 128 + 128 * 128) * 4 and n == 8 * 32
    assert off % 256 == 0 and off + n * item <= kda.kda_chunk_prefill_workspace_size(1, 8192, 32, 128, 128)
    off2, item2, n2 = kda.kda_chunk_prefill_workspace_maps(64, 8192, 32, 64, 128)
    assert item2 == (64 * 64 + 64 * 128) * 4 and off2 + n2 * item2 <= \
        kda.kda_chunk_prefill_workspace_size(64, 8192, 32, 64, 128)
    with pytest.raises(kda.KdaError):
        kda.kda_chunk_prefill_workspace_maps(1, 8192, 32, 96, 128)
