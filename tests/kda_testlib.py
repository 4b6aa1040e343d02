"""Helpers shared by the GPU parity tests: run a seeded case through the HIP
path (C ABI via the binding) and through the fp64 oracle, and compare them.

Comparison metrics (max-normalised, as in the tolerances the tests assert):
  e_o      = max|o_gpu - o_ref| / max|o_ref|        over the whole output
  e_o_cast = max(|o_gpu - o_ref| - h(o)) / max|o_ref|
             the error left after allowing each element the rounding of the
             bf16 output cast: h(o) = 2^(floor(log2 max(|o_ref|, |o_gpu|)) - 8)
             is half a bf16 ulp in the binade of the element (bf16 keeps 8
             significant bits, so round-to-nearest-even is off by at most
             that); the decode tolerance applies to this, the computation's
             own error
  e_S      = max|S_gpu - S_ref| / max|S_ref|        over the touched slots
Untouched and null slots must be bit-identical to the pre-call snapshot.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import gated_delta_rule_45_amd as kda
import workloads as W
from oracle import oracle as O

DECODE_TOL_O = 2e-3   # output: max abs error <= 2e-3 * max|ref|
DECODE_TOL_S = 1e-3   # final state relative error
PREFILL_TOL_O = 1e-2  # chunked prefill output: <= 1e-2 * max|ref|
PREFILL_TOL_S = 1e-2  # chunked prefill final state (reported bar)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class DeviceCase:
    case: W.Case
    inputs: dict
    pool: torch.Tensor
    block_table: torch.Tensor
    cu_seqlens: torch.Tensor | None
    has_initial_state: torch.Tensor | None

    @property
    def state_indices(self):
        return self.block_table[:, 0]


def to_device(case: W.Case, device="cuda", qkv_row_pad: int = 0) -> DeviceCase:
    inputs = {k: v.to(device) for k, v in case.inputs.items()}
    if qkv_row_pad:
        # mixed_qkv rows inside a wider buffer: row stride > 2*H*K + H*V.
        qkv = inputs["mixed_qkv"]
        wide = torch.zeros(qkv.shape[0], qkv.shape[1] + qkv_row_pad, dtype=qkv.dtype, device=device)
        wide[:, :qkv.shape[1]] = qkv
        inputs["mixed_qkv"] = wide[:, :qkv.shape[1]]
    if case.pool.is_contiguous():
        pool = case.pool.to(device)
    else:  # keep a padded slot stride on the device too
        st = case.pool.stride(0)
        base = torch.empty(case.pool.shape[0] * st, dtype=torch.float32, device=device)
        pool = torch.as_strided(base, case.pool.shape, case.pool.stride())
        pool.copy_(case.pool)
    return DeviceCase(case, inputs, pool, case.block_table.to(device),
                      None if case.cu_seqlens is None else case.cu_seqlens.to(device),
                      None if case.has_initial_state is None else case.has_initial_state.to(device))


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp in the binade of |x|: 2^(floor(log2|x|) - 8), 0 at 0
    (times 1 + 1e-6, for the fp32 rounding that precedes the cast)."""
    _, ex = np.frexp(np.abs(x))  # |x| = f 2^ex with f in [0.5, 1): floor(log2|x|) = ex - 1
    return np.where(x != 0, np.ldexp(1.0, ex - 9) * (1 + 1e-6), 0.0)


def cast_aware_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.abs(ref).max())
    allow = bf16_half_ulp(np.maximum(np.abs(ref), np.abs(got)))
    excess = np.abs(got - ref) - allow
    return max(float(excess.max()), 0.0) / (den if den > 0 else 1.0)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = float(np.abs(ref).max())
    if den == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max()) / den


def device_norm(case: W.Case, device="cuda"):
    """The case's output epilogue on the device (the gate keeps its row stride)."""
    if case.norm is None:
        return None
    gate = case.norm["gate"]
    base = gate.as_strided((gate.shape[0], gate.stride(0)), (gate.stride(0), 1)) if gate.shape[0] else gate
    gate_d = base.to(device)[:, :gate.shape[1]]
    return kda.GatedRMSNorm(gate_d, case.norm["weight"].to(device), case.norm["eps"],
                            case.norm["activation"])


def run_gpu(dc: DeviceCase, **kw):
    c = dc.case
    if c.norm is not None and "norm" not in kw:
        kw = dict(kw, norm=device_norm(c))
    args = (dc.inputs["mixed_qkv"], dc.inputs["raw_g"], dc.inputs["raw_beta"], dc.inputs["A_log"],
            dc.inputs["dt_bias"], c.lower_bound, dc.pool, dc.state_indices)
    if c.kind == "decode":
        out, _ = kda.kda_decode_packed(*args, tokens_per_seq=c.tokens_per_seq, scale=c.scale, **kw)
    elif c.kind == "prefill":
        out, _ = kda.kda_chunk_prefill(*args, dc.cu_seqlens, has_initial_state=dc.has_initial_state,
                                       scale=c.scale, **kw)
    else:
        out, _ = kda.kda_mixed_batch(*args, c.num_decodes, dc.cu_seqlens,
                                     has_initial_state=dc.has_initial_state, scale=c.scale, **kw)
    torch.cuda.synchronize()
    return out


def run_oracle(case: W.Case):
    """Returns (out [rows,H,V] fp64, final_state [seqs,H,K,V] fp64)."""
    c = case
    if c.kind == "decode":
        out, fs, _ = O.decode_packed(c.inputs, c.pool, c.state_indices, c.H, c.K, c.V,
                                     tokens_per_seq=c.tokens_per_seq, lower_bound=c.lower_bound,
                                     scale=c.scale, return_pool=False)
    elif c.kind == "prefill":
        hs = None if c.has_initial_state is None else c.has_initial_state.tolist()
        out, fs, _ = O.prefill(c.inputs, c.pool, c.state_indices, c.cu_seqlens.tolist(), c.H, c.K,
                               c.V, has_initial_state=hs, lower_bound=c.lower_bound, scale=c.scale,
                               return_pool=False)
    else:
        hs = None if c.has_initial_state is None else c.has_initial_state.tolist()
        out, fs, _ = O.mixed_batch(c.inputs, c.pool, c.state_indices, c.num_decodes,
                                   c.cu_seqlens.tolist(), c.H, c.K, c.V, has_initial_state=hs,
                                   lower_bound=c.lower_bound, scale=c.scale, return_pool=False)
    if c.norm is not None:
        out = O.gated_rmsnorm(out, c.norm["gate"], c.norm["weight"], c.norm["eps"], c.norm["activation"])
    return out, fs


def norm_bar_ratio(got: np.ndarray, ref_y: np.ndarray, ref_o: np.ndarray, norm: dict,
                   tol_o: float) -> float:
    """The output bar carried through the gated RMSNorm epilogue. The bar
    allows every output element an error of d = tol_o * max|o_ref|. To first
    order that moves y_j = o_j w_j act_j / r (r = sqrt(mean(o^2) + eps) of the
    row) by at most |w_j act_j| d (1 + |o_j| / r) / r (the change of r is at
    most d, by Cauchy-Schwarz); the bf16 cast of y adds half a bf16 ulp of
    y_j's binade (bf16_half_ulp, of the larger of |y_ref| and |y_gpu|). Returns
    max |y_gpu - y_ref| / that bound (at most 1 passes)."""
    rows, H, V = ref_o.shape
    w = norm["weight"].double().numpy()
    z = norm["gate"][:, :H * V].double().numpy().reshape(rows, H, V)
    sg = 1.0 / (1.0 + np.exp(-z))
    act = z * sg if norm["activation"] == "silu" else sg
    r = np.sqrt((ref_o ** 2).mean(axis=-1, keepdims=True) + norm["eps"])
    d = tol_o * float(np.abs(ref_o).max())
    bound = np.abs(w * act) * d * (1.0 + np.abs(ref_o) / r) / r + \
        bf16_half_ulp(np.maximum(np.abs(ref_y), np.abs(got)))
    return float((np.abs(got - ref_y) / np.maximum(bound, 1e-30)).max())


def seq_lengths(case: W.Case) -> list[int]:
    if case.kind == "decode":
        return [case.tokens_per_seq] * case.state_indices.shape[0]
    cu = case.cu_seqlens.tolist()
    lens = [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]
    if case.kind == "mixed":
        return [1] * case.num_decodes + lens
    return lens


def check_case(case: W.Case, tol_o: float, tol_s: float, oracle=None, qkv_row_pad: int = 0,
               cast_aware: bool | None = None, **kw) -> dict:
    """Runs the case on the GPU and in the oracle; asserts parity and slot
    bit-exactness; returns the measured errors."""
    log(f"[case] {case.name} kind={case.kind} rows={case.rows} H={case.H} K={case.K} V={case.V}")
    dc = to_device(case, qkv_row_pad=qkv_row_pad)
    snapshot = dc.pool.clone()
    out = run_gpu(dc, **kw)
    ref_out, ref_fs = oracle if oracle is not None else run_oracle(case)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), "non-finite output"
    assert np.abs(got).max() < 1e30, "garbage-sized output"
    e_o = rel_err(got, ref_out)
    e_oc = cast_aware_err(got, ref_out)
    if cast_aware is None:
        cast_aware = case.kind == "decode"
    idx = case.state_indices.tolist()
    lens = seq_lengths(case)
    touched = [(i, s) for i, s in enumerate(idx) if s >= 0 and lens[i] > 0]
    e_s = 0.0
    if touched:
        slots = torch.tensor([s for _, s in touched], device=dc.pool.device)
        got_s = dc.pool[slots].cpu().numpy().astype(np.float64)
        ref_s = np.stack([ref_fs[i] for i, _ in touched])
        assert np.all(np.isfinite(got_s)), "non-finite state"
        e_s = rel_err(got_s, ref_s)
    # Untouched and null slots: bit-identical to the snapshot.
    mask = torch.ones(dc.pool.shape[0], dtype=torch.bool, device=dc.pool.device)
    for _, s in touched:
        mask[s] = False
    assert torch.equal(dc.pool[mask], snapshot[mask]), "an untouched or null slot changed"
    # Null-slot rows are exactly zero.
    row = 0
    for i, s in enumerate(idx):
        if s < 0:
            assert torch.count_nonzero(out[row:row + lens[i]]).item() == 0, "null-slot rows not zero"
        row += lens[i]
    if case.norm is not None and case.kind != "decode" and oracle is None:
        # Prefill rows: the output bar is max-normalised, so it is carried
        # through the per-row normalisation rather than applied to y directly.
        ref_o = dataclasses.replace(case, norm=None)
        ratio = norm_bar_ratio(got, ref_out, run_oracle(ref_o)[0], case.norm, tol_o)
        log(f"[case] {case.name}: e_o={e_o:.3e} e_S={e_s:.3e} norm-bar ratio={ratio:.3e}")
        assert ratio <= 1.0, f"output error exceeds the carried bar ({ratio:.3e})"
        assert e_s <= tol_s, f"state error {e_s:.3e} > {tol_s}"
        return {"e_o": e_o, "e_o_cast": e_oc, "e_S": e_s}
    log(f"[case] {case.name}: e_o={e_o:.3e} e_o_cast={e_oc:.3e} e_S={e_s:.3e}")
    gate = e_oc if cast_aware else e_o
    assert gate <= tol_o, f"output error {gate:.3e} > {tol_o} (raw e_o {e_o:.3e})"
    assert e_s <= tol_s, f"state error {e_s:.3e} > {tol_s}"
    return {"e_o": e_o, "e_o_cast": e_oc, "e_S": e_s}
