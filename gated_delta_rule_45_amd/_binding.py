"""Python binding of the KDA C ABI (``libkda.so``): argument marshalling only.

Every step of the computation runs in the HIP kernels behind the C ABI. This
module turns torch tensors into device pointers, strides and sizes, passes the
caller's current HIP stream, and turns a non-zero status into an exception
that lists every failed check. There is no fallback: if the library is not
built, or the tensors are not on a GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkda.so")

KDA_OK = 0
NOALLOC_SCRATCH_BYTES = 64 << 20  # KDA_NOALLOC_SCRATCH_BYTES in kda.h
PREFILL_BAD_CU_SEQLENS = 1        # KDA_PREFILL_BAD_CU_SEQLENS in kda.h


def prefill_status(workspace) -> int:
    """The status word a prefill (or mixed) call left at offset 0 of its
    workspace: 0, or PREFILL_BAD_CU_SEQLENS when its cu_seqlens broke the
    contract (then its output rows are NaN and no slot was touched). Reads
    device memory, so it waits for the workspace's stream."""
    return int(workspace[:4].view(torch.int32).item())
STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
                3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_HIP"}


class KdaGate(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("has_lower_bound", ctypes.c_int32), ("lower_bound", ctypes.c_float),
                ("scale", ctypes.c_float)]


class KdaState(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("slot_stride", ctypes.c_int64),
                ("num_slots", ctypes.c_int64), ("indices", ctypes.c_void_p),
                ("index_stride", ctypes.c_int64)]


class KdaOutNorm(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("gate_row_stride", ctypes.c_int64),
                ("weight", ctypes.c_void_p), ("eps", ctypes.c_float), ("activation", ctypes.c_int32)]


NORM_ACTIVATIONS = {"sigmoid": 0, "silu": 1}


class GatedRMSNorm:
    """Optional output epilogue of every entry point: per row and head,
    y = o / sqrt(mean(o^2) + eps) * weight * act(gate) over the head's V
    channels, act = sigmoid or z*sigmoid(z). ``gate`` is bf16 [rows, >= H*V]
    (unit-stride rows, head h at h*V), ``weight`` fp32 [V]."""

    def __init__(self, gate, weight, eps: float = 1e-6, activation: str = "sigmoid"):
        self.gate, self.weight, self.eps, self.activation = gate, weight, float(eps), activation


class KdaShortConv(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("width", ctypes.c_int32),
                ("l2_eps", ctypes.c_float), ("conv_state", ctypes.c_void_p),
                ("conv_slot_stride", ctypes.c_int64), ("num_slots", ctypes.c_int64)]


class Overlap:
    """Caller-owned overlap resources of ``kda_mixed_batch`` (a side stream
    and two events on the current device, kda_overlap_create). Create it once,
    outside graph capture, and pass it as ``overlap=`` so that the decode rows
    of a mixed batch run beside the prefill's chunk passes. One handle serves
    one call at a time; concurrent callers need their own."""

    def __init__(self):
        h = ctypes.c_void_p()
        _raise_if(lib().kda_overlap_create(ctypes.byref(h)))
        self.handle = h

    def close(self):
        if self.handle is not None and self.handle.value:
            _raise_if(lib().kda_overlap_destroy(self.handle))
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


class KdaError(ValueError):
    """A call was rejected. ``status`` is the C status code, ``reasons`` the
    list of every failed check."""

    def __init__(self, status: int, reasons: list[str]):
        self.status = status
        self.reasons = reasons
        super().__init__(f"{STATUS_NAMES.get(status, status)}: " + "; ".join(reasons))


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libkda.so from the package directory (built by ``build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"KDA HIP library not built: {LIB_PATH} is missing "
                               "(run gated_delta_rule_45_amd.build.build())")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        gp, spn, npn = ctypes.POINTER(KdaGate), ctypes.POINTER(KdaState), ctypes.POINTER(KdaOutNorm)
        L.kda_decode_packed.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, vp, gp, spn, npn, vp, vp]
        L.kda_decode_packed.restype = i32
        L.kda_spec_decode.argtypes = [i32, i32, i32, i32, i32, vp, i64, vp, vp, gp, spn, i64, vp, npn,
                                      vp, vp]
        L.kda_spec_decode.restype = i32
        L.kda_chunk_prefill_workspace_size.argtypes = [i32, i64, i32, i32, i32]
        L.kda_chunk_prefill_workspace_size.restype = sz
        L.kda_chunk_prefill_workspace_min_size.argtypes = [i32, i64, i32, i32, i32]
        L.kda_chunk_prefill_workspace_min_size.restype = sz
        L.kda_chunk_prefill_workspace_maps.argtypes = [i32, i64, i32, i32, i32, ctypes.POINTER(sz),
                                                       ctypes.POINTER(sz), ctypes.POINTER(i64)]
        L.kda_chunk_prefill_workspace_maps.restype = i32
        L.kda_chunk_prefill.argtypes = [i32, i64, vp, vp, i32, i32, i32, vp, i64, vp, vp, gp, spn,
                                        npn, vp, vp, sz, vp]
        L.kda_chunk_prefill.restype = i32
        L.kda_chunk_prefill_noalloc.argtypes = [i32, i64, vp, vp, i32, i32, i32, vp, i64, vp, vp, gp,
                                                spn, npn, vp, vp]
        L.kda_chunk_prefill_noalloc.restype = i32
        L.kda_mixed_batch_workspace_size.argtypes = [i32, i32, i64, i32, i32, i32]
        L.kda_mixed_batch_workspace_size.restype = sz
        L.kda_mixed_batch.argtypes = [i32, i32, i64, vp, vp, i32, i32, i32, vp, i64, vp, vp, gp,
                                      spn, npn, vp, vp, sz, vp, vp]
        L.kda_mixed_batch.restype = i32
        L.kda_overlap_create.argtypes = [ctypes.POINTER(vp)]
        L.kda_overlap_create.restype = i32
        L.kda_overlap_destroy.argtypes = [vp]
        L.kda_overlap_destroy.restype = i32
        L.kda_short_conv.argtypes = [i32, i64, vp, vp, i32, i32, i32, vp, i64,
                                     ctypes.POINTER(KdaShortConv), vp, i64, vp, i64, vp]
        L.kda_short_conv.restype = i32
        L.kda_conv_decode_packed.argtypes = [i32, i32, i32, i32, i32, vp, i64,
                                             ctypes.POINTER(KdaShortConv), vp, vp, gp, spn, npn, vp,
                                             vp]
        L.kda_conv_decode_packed.restype = i32
        L.kda_status_string.argtypes = [i32]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_error.argtypes = []
        L.kda_last_error.restype = ctypes.c_char_p
        L.kda_version.argtypes = []
        L.kda_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _raise_if(status: int) -> None:
    if status != KDA_OK:
        detail = lib().kda_last_error().decode()
        raise KdaError(status, [r for r in detail.split("; ") if r] or [STATUS_NAMES.get(status, "")])


# ------------------------------------------------------------ marshalling

class _Marshal:
    """Collects every marshalling problem before raising once."""

    def __init__(self):
        self.reasons: list[str] = []
        self.device = None

    def tensor(self, name, t, dtype, ndim=None, optional=False):
        if t is None:
            if not optional:
                self.reasons.append(f"{name} is required")
            return
        if not isinstance(t, torch.Tensor):
            self.reasons.append(f"{name} must be a torch.Tensor")
            return
        if not t.is_cuda:
            self.reasons.append(f"{name} must be on a GPU (got {t.device})")
        elif self.device is None:
            self.device = t.device
        elif t.device != self.device:
            self.reasons.append(f"{name} is on {t.device}, expected {self.device}")
        if t.dtype != dtype:
            self.reasons.append(f"{name} must be {dtype} (got {t.dtype})")
        if ndim is not None and t.dim() != ndim:
            self.reasons.append(f"{name} must be {ndim}-D (got {t.dim()}-D)")

    def check(self, ok, msg):
        if not ok:
            self.reasons.append(msg)

    def raise_if_any(self):
        if self.reasons:
            raise KdaError(1, self.reasons)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _common(m: _Marshal, mixed_qkv, raw_g, raw_beta, A_log, dt_bias, initial_state, state_indices,
            qkv_name: str = "mixed_qkv"):
    m.tensor(qkv_name, mixed_qkv, torch.bfloat16, 2)
    m.tensor("raw_g", raw_g, torch.bfloat16, 2)
    m.tensor("raw_beta", raw_beta, torch.bfloat16, 2)
    m.tensor("A_log", A_log, torch.float32, 1)
    m.tensor("dt_bias", dt_bias, torch.float32, 1)
    m.tensor("initial_state", initial_state, torch.float32, 4)
    m.tensor("state_indices", state_indices, torch.int32, 1)
    if m.reasons:
        m.raise_if_any()
    slots, H, K, V = initial_state.shape
    st = initial_state.stride()
    m.check(st[1:] == (K * V, V, 1), "initial_state must be contiguous within a slot ([H][K][V])")
    m.check(mixed_qkv.stride(1) == 1, f"{qkv_name} rows must be unit-stride")
    m.check(raw_g.is_contiguous(), "raw_g must be contiguous")
    m.check(raw_beta.is_contiguous(), "raw_beta must be contiguous")
    m.check(A_log.is_contiguous() and dt_bias.is_contiguous(), "A_log and dt_bias must be contiguous")
    m.check(raw_g.shape[1] == H * K, f"raw_g must have H*K = {H * K} columns")
    m.check(raw_beta.shape[1] == H, f"raw_beta must have H = {H} columns")
    m.check(A_log.shape[0] == H, f"A_log must have H = {H} entries")
    m.check(dt_bias.shape[0] == H * K, f"dt_bias must have H*K = {H * K} entries")
    m.check(raw_g.shape[0] == mixed_qkv.shape[0] and raw_beta.shape[0] == mixed_qkv.shape[0],
            f"{qkv_name}, raw_g and raw_beta must have the same number of rows")
    m.raise_if_any()
    return H, K, V


def _gate(A_log, dt_bias, lower_bound, scale) -> KdaGate:
    has = lower_bound is not None
    return KdaGate(A_log=A_log.data_ptr(), dt_bias=dt_bias.data_ptr(), has_lower_bound=int(has),
                   lower_bound=float(lower_bound) if has else 0.0, scale=float(scale))


def _state(initial_state, state_indices) -> KdaState:
    return KdaState(pool=initial_state.data_ptr(), slot_stride=initial_state.stride(0),
                    num_slots=initial_state.shape[0], indices=state_indices.data_ptr(),
                    index_stride=state_indices.stride(0))


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _out(out, rows, H, V, device, m: _Marshal):
    if out is None:
        return torch.empty(rows, H, V, dtype=torch.bfloat16, device=device)
    m.tensor("out", out, torch.bfloat16, 3)
    m.check(tuple(out.shape) == (rows, H, V) and out.is_contiguous(),
            f"out must be a contiguous [{rows}, {H}, {V}] tensor")
    m.raise_if_any()
    return out


def _norm(norm, rows, H, V, m: _Marshal):
    """The optional epilogue as a C struct (None when absent)."""
    if norm is None:
        return None
    if not isinstance(norm, GatedRMSNorm):
        m.check(False, "norm must be a GatedRMSNorm or None")
        m.raise_if_any()
    m.tensor("norm.gate", norm.gate, torch.bfloat16, 2)
    m.tensor("norm.weight", norm.weight, torch.float32, 1)
    m.raise_if_any()
    m.check(norm.activation in NORM_ACTIVATIONS,
            f"norm.activation must be one of {sorted(NORM_ACTIVATIONS)}")
    m.check(norm.gate.shape[0] == rows and norm.gate.shape[1] >= H * V and norm.gate.stride(1) == 1,
            f"norm.gate must be [{rows}, >= {H * V}] with unit-stride rows")
    m.check(norm.weight.shape[0] == V and norm.weight.is_contiguous(),
            f"norm.weight must be a contiguous [{V}] tensor")
    m.raise_if_any()
    return KdaOutNorm(gate=norm.gate.data_ptr(), gate_row_stride=norm.gate.stride(0),
                      weight=norm.weight.data_ptr(), eps=norm.eps,
                      activation=NORM_ACTIVATIONS[norm.activation])


def _byref(x):
    return ctypes.byref(x) if x is not None else None


# ----------------------------------------------------------------- entries

def kda_decode_packed(mixed_qkv, raw_g, raw_beta, A_log, dt_bias, lower_bound, initial_state,
                      state_indices, *, tokens_per_seq: int = 1, scale: float = 1.0, out=None,
                      norm: GatedRMSNorm | None = None):
    """Packed decode / spec-verify. ``initial_state`` (fp32 [slots, H, K, V])
    is updated in place; ``state_indices`` is a 1-D int32 view, possibly
    strided, with one entry per request; ``norm`` an optional output
    epilogue. Returns ``(out, initial_state)``."""
    m = _Marshal()
    H, K, V = _common(m, mixed_qkv, raw_g, raw_beta, A_log, dt_bias, initial_state, state_indices)
    num_seqs = state_indices.shape[0]
    rows = num_seqs * int(tokens_per_seq)
    m.check(mixed_qkv.shape[0] == rows,
            f"mixed_qkv has {mixed_qkv.shape[0]} rows, expected num_seqs*tokens_per_seq = {rows}")
    m.raise_if_any()
    out = _out(out, rows, H, V, mixed_qkv.device, m)
    nm = _norm(norm, rows, H, V, m)
    g, s = _gate(A_log, dt_bias, lower_bound, scale), _state(initial_state, state_indices)
    st = lib().kda_decode_packed(num_seqs, int(tokens_per_seq), H, K, V, _ptr(mixed_qkv),
                                 mixed_qkv.stride(0), _ptr(raw_g), _ptr(raw_beta),
                                 ctypes.byref(g), ctypes.byref(s), _byref(nm), _ptr(out),
                                 _stream(mixed_qkv.device))
    _raise_if(st)
    return out, initial_state


def kda_spec_decode(mixed_qkv, raw_g, raw_beta, A_log, dt_bias, lower_bound, initial_state,
                    block_table, num_accepted_tokens, *, tokens_per_seq: int, scale: float = 1.0,
                    out=None, norm: GatedRMSNorm | None = None):
    """Speculative decoding with a state per token. ``block_table`` is an
    int32 [num_seqs, >= tokens_per_seq] view (any strides): request n starts
    from the slot in column num_accepted_tokens[n] - 1 and the state after
    its token t is written to the slot in column t (null entries skipped).
    ``initial_state`` (fp32 [slots, H, K, V]) is updated in place. Returns
    ``(out, initial_state)``."""
    m = _Marshal()
    m.tensor("block_table", block_table, torch.int32, 2)
    m.tensor("num_accepted_tokens", num_accepted_tokens, torch.int32, 1)
    m.raise_if_any()
    tps = int(tokens_per_seq)
    num_seqs = block_table.shape[0]
    m.check(block_table.shape[1] >= tps,
            f"block_table has {block_table.shape[1]} columns, needs tokens_per_seq = {tps}")
    m.raise_if_any()
    col0 = block_table[:, 0]
    H, K, V = _common(m, mixed_qkv, raw_g, raw_beta, A_log, dt_bias, initial_state, col0)
    rows = num_seqs * tps
    m.check(mixed_qkv.shape[0] == rows,
            f"mixed_qkv has {mixed_qkv.shape[0]} rows, expected num_seqs*tokens_per_seq = {rows}")
    m.check(num_accepted_tokens.shape[0] == num_seqs and num_accepted_tokens.is_contiguous(),
            f"num_accepted_tokens must be a contiguous [{num_seqs}] tensor")
    m.raise_if_any()
    out = _out(out, rows, H, V, mixed_qkv.device, m)
    nm = _norm(norm, rows, H, V, m)
    g, s = _gate(A_log, dt_bias, lower_bound, scale), _state(initial_state, col0)
    st = lib().kda_spec_decode(num_seqs, tps, H, K, V, _ptr(mixed_qkv), mixed_qkv.stride(0),
                               _ptr(raw_g), _ptr(raw_beta), ctypes.byref(g), ctypes.byref(s),
                               block_table.stride(1), _ptr(num_accepted_tokens), _byref(nm),
                               _ptr(out), _stream(mixed_qkv.device))
    _raise_if(st)
    return out, initial_state


def kda_chunk_prefill_workspace_size(num_seqs: int, num_tokens: int, H: int, K: int, V: int) -> int:
    return int(lib().kda_chunk_prefill_workspace_size(num_seqs, num_tokens, H, K, V))


def kda_chunk_prefill_workspace_min_size(num_seqs: int, num_tokens: int, H: int, K: int, V: int) -> int:
    """The smallest workspace kda_chunk_prefill accepts (no chunk records)."""
    return int(lib().kda_chunk_prefill_workspace_min_size(num_seqs, num_tokens, H, K, V))


def kda_chunk_prefill_workspace_maps(num_seqs: int, num_tokens: int, H: int, K: int, V: int):
    """(offset, item_bytes, items) of the segment-map area of a prefill
    workspace of these sizes (kda_chunk_prefill_workspace_maps)."""
    off, item, n = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_int64()
    _raise_if(lib().kda_chunk_prefill_workspace_maps(num_seqs, num_tokens, H, K, V, ctypes.byref(off),
                                                     ctypes.byref(item), ctypes.byref(n)))
    return int(off.value), int(item.value), int(n.value)


def kda_mixed_batch_workspace_size(num_decodes: int, num_prefills: int, num_prefill_tokens: int,
                                   H: int, K: int, V: int) -> int:
    return int(lib().kda_mixed_batch_workspace_size(num_decodes, num_prefills, num_prefill_tokens,
                                                    H, K, V))


def _workspace(workspace, need, device, m: _Marshal):
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    m.tensor("workspace", workspace, torch.uint8, 1)
    m.raise_if_any()
    return workspace


def kda_chunk_prefill(mixed_qkv, raw_g, raw_beta, A_log, dt_bias, lower_bound, initial_state,
                      state_indices, cu_seqlens, *, has_initial_state=None, scale: float = 1.0,
                      out=None, workspace=None, norm: GatedRMSNorm | None = None):
    """Varlen chunked prefill (chunk 64). ``cu_seqlens`` is device int32
    [num_seqs+1]; the token count is taken from ``mixed_qkv.shape[0]`` (the
    host never reads ``cu_seqlens``). Without ``workspace`` a scratch tensor of
    the required size is allocated with torch. Returns ``(out, initial_state)``."""
    m = _Marshal()
    H, K, V = _common(m, mixed_qkv, raw_g, raw_beta, A_log, dt_bias, initial_state, state_indices)
    m.tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    m.tensor("has_initial_state", has_initial_state, torch.uint8, 1, optional=True)
    m.raise_if_any()
    num_seqs = cu_seqlens.shape[0] - 1
    num_tokens = mixed_qkv.shape[0]
    m.check(cu_seqlens.is_contiguous(), "cu_seqlens must be contiguous")
    m.check(state_indices.shape[0] == num_seqs, "state_indices needs one entry per sequence")
    if has_initial_state is not None:
        m.check(has_initial_state.shape[0] == num_seqs and has_initial_state.is_contiguous(),
                "has_initial_state must be contiguous with one entry per sequence")
    m.raise_if_any()
    out = _out(out, num_tokens, H, V, mixed_qkv.device, m)
    need = kda_chunk_prefill_workspace_size(max(num_seqs, 0), num_tokens, H, K, V)
    ws = _workspace(workspace, need, mixed_qkv.device, m)
    nm = _norm(norm, num_tokens, H, V, m)
    g, s = _gate(A_log, dt_bias, lower_bound, scale), _state(initial_state, state_indices)
    st = lib().kda_chunk_prefill(num_seqs, num_tokens, _ptr(cu_seqlens), _ptr(has_initial_state),
                                 H, K, V, _ptr(mixed_qkv), mixed_qkv.stride(0), _ptr(raw_g),
                                 _ptr(raw_beta), ctypes.byref(g), ctypes.byref(s), _byref(nm),
                                 _ptr(out), _ptr(ws), ws.numel(), _stream(mixed_qkv.device))
    _raise_if(st)
    return out, initial_state


def kda_chunk_prefill_noalloc(mixed_qkv, raw_g, raw_beta, A_log, dt_bias, lower_bound, initial_state,
                              state_indices, cu_seqlens, *, has_initial_state=None, scale: float = 1.0,
                              out=None, norm: GatedRMSNorm | None = None):
    """kda_chunk_prefill on the library's static per-GPU scratch instead of a
    workspace (no device allocation in the library; ``out`` is allocated
    here only when not given). Sizes whose workspace would exceed
    ``NOALLOC_SCRATCH_BYTES`` are rejected. Returns ``(out, initial_state)``."""
    m = _Marshal()
    H, K, V = _common(m, mixed_qkv, raw_g, raw_beta, A_log, dt_bias, initial_state, state_indices)
    m.tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    m.tensor("has_initial_state", has_initial_state, torch.uint8, 1, optional=True)
    m.raise_if_any()
    num_seqs = cu_seqlens.shape[0] - 1
    num_tokens = mixed_qkv.shape[0]
    m.check(cu_seqlens.is_contiguous(), "cu_seqlens must be contiguous")
    m.check(state_indices.shape[0] == num_seqs, "state_indices needs one entry per sequence")
    if has_initial_state is not None:
        m.check(has_initial_state.shape[0] == num_seqs and has_initial_state.is_contiguous(),
                "has_initial_state must be contiguous with one entry per sequence")
    m.raise_if_any()
    out = _out(out, num_tokens, H, V, mixed_qkv.device, m)
    nm = _norm(norm, num_tokens, H, V, m)
    g, s = _gate(A_log, dt_bias, lower_bound, scale), _state(initial_state, state_indices)
    st = lib().kda_chunk_prefill_noalloc(num_seqs, num_tokens, _ptr(cu_seqlens),
                                         _ptr(has_initial_state), H, K, V, _ptr(mixed_qkv),
                                         mixed_qkv.stride(0), _ptr(raw_g), _ptr(raw_beta),
                                         ctypes.byref(g), ctypes.byref(s), _byref(nm), _ptr(out),
                                         _stream(mixed_qkv.device))
    _raise_if(st)
    return out, initial_state


def kda_mixed_batch(mixed_qkv, raw_g, raw_beta, A_log, dt_bias, lower_bound, initial_state,
                    state_indices, num_decodes: int, prefill_cu_seqlens, *, has_initial_state=None,
                    scale: float = 1.0, out=None, workspace=None, norm: GatedRMSNorm | None = None,
                    overlap: Overlap | None = None):
    """Mixed batch: rows [0, num_decodes) are single-token decodes (recurrent
    kernel), the rest are prefill sequences given by ``prefill_cu_seqlens``
    (relative to ``num_decodes``; chunk pipeline). ``state_indices`` has the
    decodes' entries first, then the prefills'. With ``overlap`` (an
    ``Overlap``) the decode rows run on its side stream beside the prefill.
    Returns ``(out, initial_state)``."""
    m = _Marshal()
    H, K, V = _common(m, mixed_qkv, raw_g, raw_beta, A_log, dt_bias, initial_state, state_indices)
    m.tensor("prefill_cu_seqlens", prefill_cu_seqlens, torch.int32, 1)
    m.tensor("has_initial_state", has_initial_state, torch.uint8, 1, optional=True)
    m.raise_if_any()
    num_prefills = prefill_cu_seqlens.shape[0] - 1
    rows = mixed_qkv.shape[0]
    num_prefill_tokens = rows - int(num_decodes)
    m.check(prefill_cu_seqlens.is_contiguous(), "prefill_cu_seqlens must be contiguous")
    m.check(num_prefill_tokens >= 0, "num_decodes exceeds the number of rows")
    m.check(state_indices.shape[0] == int(num_decodes) + num_prefills,
            "state_indices needs one entry per decode and per prefill sequence")
    m.raise_if_any()
    out = _out(out, rows, H, V, mixed_qkv.device, m)
    need = kda_mixed_batch_workspace_size(int(num_decodes), max(num_prefills, 0),
                                          num_prefill_tokens, H, K, V)
    ws = _workspace(workspace, need, mixed_qkv.device, m)
    nm = _norm(norm, rows, H, V, m)
    g, s = _gate(A_log, dt_bias, lower_bound, scale), _state(initial_state, state_indices)
    st = lib().kda_mixed_batch(int(num_decodes), num_prefills, num_prefill_tokens,
                               _ptr(prefill_cu_seqlens), _ptr(has_initial_state), H, K, V,
                               _ptr(mixed_qkv), mixed_qkv.stride(0), _ptr(raw_g), _ptr(raw_beta),
                               ctypes.byref(g), ctypes.byref(s), _byref(nm), _ptr(out), _ptr(ws),
                               ws.numel(), overlap.handle if overlap is not None else None,
                               _stream(mixed_qkv.device))
    _raise_if(st)
    return out, initial_state


def kda_short_conv(x, weight, bias, conv_state, state_indices, cu_seqlens, *, H: int, K: int, V: int,
                   has_initial_state=None, l2_eps: float = 1e-6, out=None):
    """Short causal conv prologue: mixed_qkv from the [q | k | v]
    pre-activations ``x`` (bf16 [rows, >= D], D = 2*H*K + H*V, unit-stride
    rows). ``weight`` fp32 [D, width], ``bias`` fp32 [D] or None,
    ``conv_state`` bf16 [slots, width-1, D] (updated in place; rows of a slot
    contiguous), ``state_indices`` int32 1-D (possibly strided),
    ``cu_seqlens`` device int32 [num_seqs+1]. Returns ``(out, conv_state)``
    with ``out`` bf16 [rows, D] (or the given ``out``, any unit-stride rows)."""
    m = _Marshal()
    m.tensor("x", x, torch.bfloat16, 2)
    m.tensor("weight", weight, torch.float32, 2)
    m.tensor("bias", bias, torch.float32, 1, optional=True)
    m.tensor("conv_state", conv_state, torch.bfloat16, 3)
    m.tensor("state_indices", state_indices, torch.int32, 1)
    m.tensor("cu_seqlens", cu_seqlens, torch.int32, 1)
    m.tensor("has_initial_state", has_initial_state, torch.uint8, 1, optional=True)
    m.raise_if_any()
    D = 2 * H * K + H * V
    width = weight.shape[1]
    num_seqs = cu_seqlens.shape[0] - 1
    rows = x.shape[0]
    m.check(x.shape[1] >= D and x.stride(1) == 1, f"x must be [rows, >= {D}] with unit-stride rows")
    m.check(tuple(weight.shape) == (D, width) and weight.is_contiguous(),
            f"weight must be a contiguous [{D}, width] tensor")
    if bias is not None:
        m.check(tuple(bias.shape) == (D,) and bias.is_contiguous(), f"bias must be a contiguous [{D}] tensor")
    m.check(conv_state.shape[1:] == (width - 1, D) and conv_state.stride(1) == D and conv_state.stride(2) == 1,
            f"conv_state must be [slots, {width - 1}, {D}] with contiguous slots")
    m.check(cu_seqlens.is_contiguous(), "cu_seqlens must be contiguous")
    m.check(state_indices.shape[0] == num_seqs, "state_indices needs one entry per sequence")
    if has_initial_state is not None:
        m.check(has_initial_state.shape[0] == num_seqs and has_initial_state.is_contiguous(),
                "has_initial_state must be contiguous with one entry per sequence")
    m.raise_if_any()
    if out is None:
        out = torch.empty(rows, D, dtype=torch.bfloat16, device=x.device)
    else:
        m.tensor("out", out, torch.bfloat16, 2)
        m.raise_if_any()
        m.check(out.shape[0] == rows and out.shape[1] >= D and out.stride(1) == 1,
                f"out must be [{rows}, >= {D}] with unit-stride rows")
        m.raise_if_any()
    cv = KdaShortConv(weight=weight.data_ptr(), bias=bias.data_ptr() if bias is not None else None,
                      width=int(width), l2_eps=float(l2_eps), conv_state=conv_state.data_ptr(),
                      conv_slot_stride=conv_state.stride(0), num_slots=conv_state.shape[0])
    st = lib().kda_short_conv(num_seqs, rows, _ptr(cu_seqlens), _ptr(has_initial_state), H, K, V,
                              _ptr(x), x.stride(0), ctypes.byref(cv), _ptr(state_indices),
                              state_indices.stride(0), _ptr(out), out.stride(0), _stream(x.device))
    _raise_if(st)
    return out, conv_state


def kda_conv_decode_packed(x, weight, bias, conv_state, raw_g, raw_beta, A_log, dt_bias, lower_bound,
                           initial_state, state_indices, *, tokens_per_seq: int = 1, scale: float = 1.0,
                           l2_eps: float = 1e-6, out=None, norm: GatedRMSNorm | None = None):
    """Packed decode with the short conv prologue fused: q, k and v come from
    the pre-activations ``x`` (bf16 [num_seqs*tokens_per_seq, >= D], unit-stride
    rows) through the conv (``weight`` fp32 [D, width], ``bias`` fp32 [D] or
    None, ``conv_state`` bf16 [slots, width-1, D], updated in place on the
    KDA state's slot numbers). ``initial_state`` is updated in place as for
    kda_decode_packed. Returns ``(out, initial_state, conv_state)``."""
    m = _Marshal()
    m.tensor("x", x, torch.bfloat16, 2)
    m.tensor("weight", weight, torch.float32, 2)
    m.tensor("bias", bias, torch.float32, 1, optional=True)
    m.tensor("conv_state", conv_state, torch.bfloat16, 3)
    m.raise_if_any()
    H, K, V = _common(m, x, raw_g, raw_beta, A_log, dt_bias, initial_state, state_indices, "x")
    D = 2 * H * K + H * V
    width = weight.shape[1]
    num_seqs = state_indices.shape[0]
    rows = num_seqs * int(tokens_per_seq)
    m.check(x.shape[0] == rows, f"x has {x.shape[0]} rows, expected num_seqs*tokens_per_seq = {rows}")
    m.check(x.shape[1] >= D, f"x must have >= {D} columns")
    m.check(tuple(weight.shape) == (D, width) and weight.is_contiguous(),
            f"weight must be a contiguous [{D}, width] tensor")
    if bias is not None:
        m.check(tuple(bias.shape) == (D,) and bias.is_contiguous(), f"bias must be a contiguous [{D}] tensor")
    m.check(conv_state.shape[1:] == (width - 1, D) and conv_state.stride(1) == D and conv_state.stride(2) == 1,
            f"conv_state must be [slots, {width - 1}, {D}] with contiguous slots")
    m.raise_if_any()
    out = _out(out, rows, H, V, x.device, m)
    nm = _norm(norm, rows, H, V, m)
    cv = KdaShortConv(weight=weight.data_ptr(), bias=bias.data_ptr() if bias is not None else None,
                      width=int(width), l2_eps=float(l2_eps), conv_state=conv_state.data_ptr(),
                      conv_slot_stride=conv_state.stride(0), num_slots=conv_state.shape[0])
    g, s = _gate(A_log, dt_bias, lower_bound, scale), _state(initial_state, state_indices)
    st = lib().kda_conv_decode_packed(num_seqs, int(tokens_per_seq), H, K, V, _ptr(x), x.stride(0),
                                      ctypes.byref(cv), _ptr(raw_g), _ptr(raw_beta), ctypes.byref(g),
                                      ctypes.byref(s), _byref(nm), _ptr(out), _stream(x.device))
    _raise_if(st)
    return out, initial_state, conv_state
