"""ctypes front end of the fp64 KDA oracle (``kda_oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module. It never imports the HIP
package, and the HIP package never imports it.

Functions take host (CPU) torch tensors in the same formats the HIP path takes
(bf16 ``mixed_qkv``/``raw_g``/``raw_beta``, fp32 ``A_log``/``dt_bias``/pool,
int32 slot indices, possibly a strided 1-D view) and return fp64 numpy arrays.
The pool passed in is never modified: the oracle works on a copy and returns it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
# A planted-mistake copy of the oracle can be loaded instead (mutation tests).
_LIB_OVERRIDE = os.environ.get("KDA_ORACLE_LIB_OVERRIDE")


def build() -> str:
    """Compiles the oracle with gcc (plain C, OpenMP over independent pairs)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Args(ctypes.Structure):
    _fields_ = [
        ("mixed_qkv", ctypes.c_void_p),
        ("qkv_row_stride", ctypes.c_int64),
        ("raw_g", ctypes.c_void_p),
        ("raw_beta", ctypes.c_void_p),
        ("A_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
        ("has_lower_bound", ctypes.c_int32),
        ("lower_bound", ctypes.c_double),
        ("scale", ctypes.c_double),
        ("pool", ctypes.c_void_p),
        ("slot_stride", ctypes.c_int64),
        ("state_indices", ctypes.c_void_p),
        ("index_stride", ctypes.c_int64),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
        d, i32, i64, vp = ctypes.c_double, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.kda_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.kda_oracle_bf16_to_double.restype = d
        L.kda_oracle_gate.argtypes = [d, d, d, i32, d]
        L.kda_oracle_gate.restype = d
        L.kda_oracle_beta.argtypes = [d]
        L.kda_oracle_beta.restype = d
        L.kda_oracle_recurrent_pregated.argtypes = [i32, i32, i32] + [vp] * 5 + [d, vp, vp]
        L.kda_oracle_recurrent_pregated.restype = None
        L.kda_oracle_chunked_pregated.argtypes = [i32, i32, i32, i32] + [vp] * 5 + [d, vp, vp]
        L.kda_oracle_chunked_pregated.restype = None
        L.kda_oracle_set_threads.argtypes = [i32]
        L.kda_oracle_set_threads.restype = None
        L.kda_oracle_max_threads.argtypes = []
        L.kda_oracle_max_threads.restype = i32
        L.kda_oracle_decode_packed.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(_Args), i32, vp, vp]
        L.kda_oracle_decode_packed.restype = i32
        L.kda_oracle_prefill.argtypes = [i32, vp, vp, i32, i32, i32, ctypes.POINTER(_Args), i32, vp, vp]
        L.kda_oracle_spec_decode.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(_Args), ctypes.c_int64,
                                             vp, vp, vp]
        L.kda_oracle_spec_decode.restype = i32
        L.kda_oracle_prefill.restype = i32
        L.kda_oracle_gated_rmsnorm.argtypes = [ctypes.c_int64, i32, i32, vp, vp, ctypes.c_int64, vp, d, i32]
        L.kda_oracle_gated_rmsnorm.restype = None
        L.kda_oracle_short_conv.argtypes = [i32, vp, vp, i32, i32, i32, i32, vp, vp, vp, d, vp, vp,
                                            ctypes.c_int64, vp]
        L.kda_oracle_short_conv.restype = None
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    lib().kda_oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().kda_oracle_max_threads())


# ------------------------------------------------------------- scalar pieces

def bf16_to_double(bits: int) -> float:
    return float(lib().kda_oracle_bf16_to_double(int(bits) & 0xFFFF))


def gate(raw_g: float, A_log: float, dt_bias: float, lower_bound: float | None) -> float:
    has = lower_bound is not None
    return float(lib().kda_oracle_gate(raw_g, A_log, dt_bias, int(has),
                                       float(lower_bound) if has else 0.0))


def beta(raw_beta: float) -> float:
    return float(lib().kda_oracle_beta(raw_beta))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def recurrent_pregated(q, k, v, g, beta_, S0, scale: float = 1.0):
    """Recurrence on one (sequence, head) from per-token g and beta.
    q,k,g: [T,K]; v: [T,V]; beta_: [T]; S0: [K,V]. Returns (o [T,V], S [K,V])."""
    q, k, v, g, b = map(_f64, (q, k, v, g, beta_))
    S = _f64(S0).copy()
    T, K = q.shape
    V = v.shape[1]
    o = np.zeros((T, V), dtype=np.float64)
    lib().kda_oracle_recurrent_pregated(T, K, V, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                        _ptr(b), float(scale), _ptr(S), _ptr(o))
    return o, S


def chunked_pregated(q, k, v, g, beta_, S0, chunk: int, scale: float = 1.0):
    """Chunked (WY) form of the same recurrence, chunk size ``chunk``."""
    q, k, v, g, b = map(_f64, (q, k, v, g, beta_))
    S = _f64(S0).copy()
    T, K = q.shape
    V = v.shape[1]
    o = np.zeros((T, V), dtype=np.float64)
    lib().kda_oracle_chunked_pregated(T, K, V, int(chunk), _ptr(q), _ptr(k), _ptr(v),
                                      _ptr(g), _ptr(b), float(scale), _ptr(S), _ptr(o))
    return o, S


# ------------------------------------------------------------ batch entries

def _bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return np.ascontiguousarray(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def _args(inp: dict, pool: np.ndarray, idx: np.ndarray, index_stride: int,
          lower_bound, scale: float, keep: list) -> _Args:
    qkv = inp["mixed_qkv"].cpu()
    qkv_bits = _bits(qkv)
    raw_g = _bits(inp["raw_g"].cpu())
    raw_beta = _bits(inp["raw_beta"].cpu())
    A_log = np.ascontiguousarray(inp["A_log"].cpu().numpy().astype(np.float32))
    dt_bias = np.ascontiguousarray(inp["dt_bias"].cpu().numpy().astype(np.float32))
    keep += [qkv_bits, raw_g, raw_beta, A_log, dt_bias, pool, idx]
    has = lower_bound is not None
    return _Args(
        mixed_qkv=qkv_bits.ctypes.data, qkv_row_stride=qkv_bits.shape[1],
        raw_g=raw_g.ctypes.data, raw_beta=raw_beta.ctypes.data,
        A_log=A_log.ctypes.data, dt_bias=dt_bias.ctypes.data,
        has_lower_bound=int(has), lower_bound=float(lower_bound) if has else 0.0,
        scale=float(scale), pool=pool.ctypes.data, slot_stride=pool.shape[1],
        state_indices=idx.ctypes.data, index_stride=int(index_stride))


def _indices(state_indices: torch.Tensor):
    """A 1-D (possibly strided) int32 view -> its base buffer and element stride."""
    assert state_indices.dim() == 1 and state_indices.dtype == torch.int32
    st = state_indices.stride(0)
    n = state_indices.shape[0]
    if n == 0:
        return np.zeros(1, dtype=np.int32), 1
    base = torch.as_strided(state_indices, ((n - 1) * st + 1,), (1,))
    return np.ascontiguousarray(base.cpu().numpy()), st


def _pool2d(pool: torch.Tensor) -> np.ndarray:
    """Copy of the pool as [slots, slot_stride] fp32, keeping a padded slot
    stride (slots whose stride exceeds H*K*V) as it is in the caller's buffer."""
    pool = pool.detach().cpu()
    per = int(np.prod(pool.shape[1:]))
    st = pool.stride(0)
    inner_dense = pool[0].is_contiguous() if pool.shape[0] else True
    if pool.shape[0] and st > per and inner_dense:
        flat = torch.as_strided(pool, (pool.shape[0], st), (st, 1))
        return np.array(flat.numpy(), dtype=np.float32, copy=True)
    return np.array(pool.reshape(pool.shape[0], -1).numpy(), dtype=np.float32, copy=True)


def _compact(pool: torch.Tensor, idx: np.ndarray):
    """Gathers the slots the call references into a small pool and remaps the
    index buffer to it (plumbing only: the oracle sees the same slot contents,
    and untouched slots cannot change). Returns (pool2d, idx_remapped)."""
    refs = sorted({int(x) for x in np.unique(idx) if x >= 0})
    pool = pool.detach().cpu()
    if not refs:
        return np.zeros((1, int(np.prod(pool.shape[1:]))), dtype=np.float32), idx
    sel = pool[torch.tensor(refs, dtype=torch.long)]
    comp = np.array(sel.reshape(len(refs), -1).numpy(), dtype=np.float32, copy=True)
    remap = {s: i for i, s in enumerate(refs)}
    idx2 = np.array([remap.get(int(x), int(x)) if x >= 0 else int(x) for x in idx], dtype=np.int32)
    return comp, idx2


def decode_packed(inp: dict, pool: torch.Tensor, state_indices: torch.Tensor,
                  H: int, K: int, V: int, tokens_per_seq: int = 1,
                  lower_bound=None, scale: float = 1.0, form: int = 0,
                  return_pool: bool = True):
    """Packed decode / spec-verify. Returns (out [rows,H,V], final_state
    [seqs,H,K,V] (zeros for null slots), pool_after [slots, slot_stride]).
    With ``return_pool=False`` only the referenced slots are copied and
    pool_after is None (much faster on GiB-sized pools)."""
    idx, ist = _indices(state_indices)
    num_seqs = state_indices.shape[0]
    if return_pool:
        P = _pool2d(pool)
    else:
        P, idx = _compact(pool, idx)
    keep: list = []
    a = _args(inp, P, idx, ist, lower_bound, scale, keep)
    rows = num_seqs * tokens_per_seq
    out = np.zeros((rows, H, V), dtype=np.float64)
    fs = np.zeros((num_seqs, H, K, V), dtype=np.float64)
    rc = lib().kda_oracle_decode_packed(num_seqs, tokens_per_seq, H, K, V, ctypes.byref(a),
                                        int(form), _ptr(out), _ptr(fs))
    if rc != 0:
        raise ValueError("oracle rejected the decode arguments")
    return out, fs, (P if return_pool else None)


def spec_decode(inp: dict, pool: torch.Tensor, block_table: torch.Tensor, num_accepted,
                H: int, K: int, V: int, tokens_per_seq: int, lower_bound=None,
                scale: float = 1.0, return_pool: bool = True):
    """Speculative decoding with a state per token: request n reads its
    initial state from block-table column num_accepted[n] - 1 and stores the
    state after its token t into column t (entries < 0 are skipped; a request
    whose initial entry is < 0 touches nothing and outputs zeros).
    ``block_table``: int32 [num_seqs, >= tokens_per_seq] (any strides; the
    oracle gets the same entries, packed). Returns (out [rows,H,V],
    states [seqs,tokens,H,K,V], pool_after)."""
    num_seqs = block_table.shape[0]
    T = int(tokens_per_seq)
    tab = np.ascontiguousarray(block_table[:, :T].cpu().numpy().astype(np.int32))
    acc = np.ascontiguousarray(np.asarray(num_accepted, dtype=np.int32))
    if return_pool:
        P = _pool2d(pool)
        flat = tab.reshape(-1)
    else:
        P, flat = _compact(pool, tab.reshape(-1))
    flat = np.ascontiguousarray(flat.astype(np.int32))
    keep: list = []
    a = _args(inp, P, flat, T, lower_bound, scale, keep)
    out = np.zeros((num_seqs * T, H, V), dtype=np.float64)
    states = np.zeros((num_seqs, T, H, K, V), dtype=np.float64)
    rc = lib().kda_oracle_spec_decode(num_seqs, T, H, K, V, ctypes.byref(a), 1, _ptr(acc),
                                      _ptr(out), _ptr(states))
    if rc != 0:
        raise ValueError("oracle rejected the spec-decode arguments")
    return out, states, (P if return_pool else None)


def prefill(inp: dict, pool: torch.Tensor, state_indices: torch.Tensor,
            cu_seqlens, H: int, K: int, V: int, has_initial_state=None,
            lower_bound=None, scale: float = 1.0, form: int = 0,
            return_pool: bool = True):
    """Varlen prefill over rows 0..cu_seqlens[-1]-1 of ``inp``.
    Returns (out [rows,H,V], final_state [seqs,H,K,V], pool_after)."""
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    num_seqs = cu.shape[0] - 1
    hs = None
    if has_initial_state is not None:
        hs = np.ascontiguousarray(np.asarray(has_initial_state, dtype=np.uint8))
    idx, ist = _indices(state_indices)
    if return_pool:
        P = _pool2d(pool)
    else:
        P, idx = _compact(pool, idx)
    keep: list = []
    a = _args(inp, P, idx, ist, lower_bound, scale, keep)
    rows = int(cu[-1]) if num_seqs >= 0 else 0
    out = np.zeros((rows, H, V), dtype=np.float64)
    fs = np.zeros((num_seqs, H, K, V), dtype=np.float64)
    rc = lib().kda_oracle_prefill(num_seqs, _ptr(cu), _ptr(hs) if hs is not None else None,
                                  H, K, V, ctypes.byref(a), int(form), _ptr(out), _ptr(fs))
    if rc != 0:
        raise ValueError("oracle rejected the prefill arguments")
    return out, fs, (P if return_pool else None)


def mixed_batch(inp: dict, pool: torch.Tensor, state_indices: torch.Tensor,
                num_decodes: int, prefill_cu_seqlens, H: int, K: int, V: int,
                has_initial_state=None, lower_bound=None, scale: float = 1.0,
                form: int = 0, return_pool: bool = True):
    """Decode rows [0, D) then prefill sequences over rows D.. (cu_seqlens
    relative to D); slot entries: the D decodes first, then the prefills.
    Every sequence is independent, so this is one call over all of them with
    cu_seqlens [0, 1, ..., D, D + c_1, ...]."""
    cu_p = np.asarray(prefill_cu_seqlens, dtype=np.int64)
    cu = np.concatenate([np.arange(num_decodes + 1, dtype=np.int64), num_decodes + cu_p[1:]])
    hs = None
    if has_initial_state is not None:
        hs = np.concatenate([np.ones(num_decodes, dtype=np.uint8),
                             np.asarray(has_initial_state, dtype=np.uint8)])
    return prefill(inp, pool, state_indices, cu, H, K, V, has_initial_state=hs,
                   lower_bound=lower_bound, scale=scale, form=form, return_pool=return_pool)


# ---------------------------------------------------------- output epilogue

ACTIVATIONS = {"sigmoid": 0, "silu": 1}


def gated_rmsnorm(out: np.ndarray, gate: torch.Tensor, weight: torch.Tensor, eps: float,
                  activation: str = "sigmoid") -> np.ndarray:
    """Gated RMSNorm of KDA outputs (reading R20 of the design notes; the
    pages name the step after the recurrence, vLLM PR #60683 Purpose, but
    print no formula): per row and head, over the head's V channels,
    y = o / sqrt(mean(o^2) + eps) * w * act(z), act = sigmoid or z*sigmoid(z).
    out: fp64 [rows, H, V] (not modified); gate: bf16 [rows, >= H*V] (its
    first H*V columns are the gate input); weight: fp32 [V]. Returns a new
    fp64 array."""
    y = np.ascontiguousarray(np.array(out, dtype=np.float64))
    rows, H, V = y.shape
    g = gate.detach().cpu()
    assert g.dtype == torch.bfloat16 and g.dim() == 2 and g.shape[0] == rows and g.shape[1] >= H * V
    bits = _bits(g[:, :H * V].contiguous()) if rows else np.zeros(1, dtype=np.uint16)
    w = np.ascontiguousarray(weight.detach().cpu().float().numpy())
    assert w.shape == (V,)
    lib().kda_oracle_gated_rmsnorm(rows, H, V, _ptr(y), _ptr(bits), H * V, _ptr(w), float(eps),
                                   ACTIVATIONS[activation])
    return y


# --------------------------------------------------------- input prologue

def short_conv(x: torch.Tensor, weight: torch.Tensor, bias, conv_state: torch.Tensor,
               state_indices: torch.Tensor, cu_seqlens, H: int, K: int, V: int,
               has_initial_state=None, l2_eps: float = 1e-6):
    """Short causal conv prologue (reading R22 of the design notes; vLLM PR
    #60683 Purpose names a conv step before the recurrence but prints no
    formula): per sequence and channel of the [q | k | v] pre-activations,
    a = bias + sum_i w[c][i] x[t - (W-1) + i] with earlier inputs from the
    conv state, y = silu(a), then q and k of each head L2-normalised.
    x: bf16 [rows, >= D]; weight: fp32 [D, W]; bias: fp32 [D] or None;
    conv_state: [slots, W-1, D] (any float dtype; read as given);
    state_indices: int32 1-D (strides honoured). Returns (y fp64 [rows, D],
    new conv state fp64 [slots, W-1, D])."""
    D = 2 * H * K + H * V
    Wd = int(weight.shape[1])
    rows = x.shape[0]
    xb = _bits(x[:, :D].contiguous()) if rows else np.zeros(1, dtype=np.uint16)
    w = np.ascontiguousarray(weight.detach().cpu().float().numpy())
    assert w.shape == (D, Wd)
    b = None if bias is None else np.ascontiguousarray(bias.detach().cpu().float().numpy())
    st = np.array(conv_state.detach().cpu().double().numpy(), dtype=np.float64, copy=True)  # never the caller's buffer
    assert st.shape[1:] == (Wd - 1, D)
    idx, stride = _indices(state_indices)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    hs = None if has_initial_state is None else np.ascontiguousarray(np.asarray(has_initial_state, dtype=np.uint8))
    y = np.zeros((max(rows, 1), D), dtype=np.float64)
    lib().kda_oracle_short_conv(len(cu) - 1, _ptr(cu), _ptr(hs) if hs is not None else None, H, K, V, Wd,
                                _ptr(xb), _ptr(w), _ptr(b) if b is not None else None, float(l2_eps),
                                _ptr(st), _ptr(idx), stride, _ptr(y))
    return y[:rows], st
