"""Seeded synthetic inputs for KDA decode, spec-verify, prefill and mixed batches.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic, imports neither the oracle nor the HIP package, and is the
one piece of code both sides share. Everything is drawn on the CPU with a
seeded ``torch.Generator`` in fp32 and then cast, so every consumer sees the
same bytes. Seeds follow ``1000 * workload + variant``.

Input recipe (shapes from the workloads the pages describe; value
distributions are this project's choice, since the pages give none):
  mixed_qkv  bf16 [rows, 2*H*K + H*V]: randn, q and k L2-normalised per head
             (in fp32, before the cast); v plain randn.
  raw_g      bf16 [rows, H*K] randn;   raw_beta bf16 [rows, H] randn.
  A_log      fp32 [H] = log(U[1, 16]); dt_bias fp32 [H*K] = 0.1 * randn.
  pool       fp32 [slots, H, K, V] = std * randn (optionally padded slots).
  state_indices: column 0 of an int32 block table [seqs, width] of unique
             random slots; the other columns hold other slots (never read).
  output-norm epilogue: gate bf16 [rows, H*V (+ pad)] randn, weight fp32 [V]
             = 1 + 0.1 * randn, eps 1e-6.
  conv prologue: x bf16 [rows, D (+ pad)] randn (D = 2*H*K + H*V); weight
             fp32 [D, W] = 0.5 * randn; bias fp32 [D] = 0.1 * randn; conv
             state bf16 [slots, W-1, D] randn.
"""
from __future__ import annotations

import dataclasses
import functools

import torch


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def make_token_inputs(rows: int, H: int, K: int, V: int, seed: int) -> dict:
    """Per-row tensors (CPU): mixed_qkv, raw_g, raw_beta, plus A_log, dt_bias."""
    g = _gen(seed)
    q = torch.randn(rows, H, K, generator=g)
    k = torch.randn(rows, H, K, generator=g)
    v = torch.randn(rows, H, V, generator=g)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    mixed = torch.cat([q.reshape(rows, H * K), k.reshape(rows, H * K), v.reshape(rows, H * V)], dim=1)
    raw_g = torch.randn(rows, H * K, generator=g)
    raw_beta = torch.randn(rows, H, generator=g)
    A_log = torch.log(torch.empty(H).uniform_(1.0, 16.0, generator=g))
    dt_bias = 0.1 * torch.randn(H * K, generator=g)
    return {
        "mixed_qkv": mixed.to(torch.bfloat16),
        "raw_g": raw_g.to(torch.bfloat16),
        "raw_beta": raw_beta.to(torch.bfloat16),
        "A_log": A_log.float(),
        "dt_bias": dt_bias.float(),
    }


@functools.lru_cache(maxsize=2)
def make_pool(num_slots: int, H: int, K: int, V: int, std: float, seed: int,
              slot_pad: int = 0) -> torch.Tensor:
    """fp32 state pool [slots, H, K, V] (CPU). With ``slot_pad`` > 0 the
    result is a view of a larger buffer whose slot stride is H*K*V + slot_pad.
    The result is cached (pools reach 2 GiB): callers must not modify it."""
    g = _gen(seed)
    per = H * K * V
    buf = torch.randn(num_slots, per + slot_pad, generator=g).mul_(std)
    return buf[:, :per].view(num_slots, H, K, V) if slot_pad == 0 else \
        torch.as_strided(buf, (num_slots, H, K, V), (per + slot_pad, K * V, V, 1))


def make_block_table(num_seqs: int, width: int, num_slots: int, seed: int,
                     null_rows=()) -> torch.Tensor:
    """int32 [num_seqs, width]. Column 0 holds unique random slots (-1 on the
    rows listed in ``null_rows``); other columns hold further distinct slots
    when the pool is large enough, else -7 (a value the kernels never read)."""
    g = _gen(seed)
    need = num_seqs * width
    perm = torch.randperm(num_slots, generator=g)
    if need <= num_slots:
        table = perm[:need].view(num_seqs, width).to(torch.int32).clone()
    else:
        table = torch.full((num_seqs, width), -7, dtype=torch.int32)
        table[:, 0] = perm[:num_seqs].to(torch.int32)
    for r in null_rows:
        table[r, 0] = -1
    return table


def random_lengths(num_seqs: int, lo: int, hi: int, seed: int, force_ones: int = 0) -> list[int]:
    g = _gen(seed)
    lens = torch.randint(lo, hi + 1, (num_seqs,), generator=g).tolist()
    for i in range(min(force_ones, num_seqs)):
        lens[(i * 7 + 3) % num_seqs] = 1
    return lens


def split_total(total: int, parts: int, seed: int) -> list[int]:
    """``parts`` positive lengths summing to ``total`` (distinct random cuts)."""
    g = _gen(seed)
    cuts = sorted((torch.randperm(total - 1, generator=g)[: parts - 1] + 1).tolist())
    bounds = [0] + cuts + [total]
    return [bounds[i + 1] - bounds[i] for i in range(parts)]


def make_norm(rows: int, H: int, V: int, seed: int, activation: str = "sigmoid",
              row_pad: int = 0, eps: float = 1e-6) -> dict:
    """Gate input and weight of the output epilogue. With ``row_pad`` the gate
    rows sit inside a wider buffer (row stride H*V + row_pad)."""
    g = _gen(seed)
    wide = torch.randn(rows, H * V + row_pad, generator=g).to(torch.bfloat16)
    weight = 1.0 + 0.1 * torch.randn(V, generator=g)
    return {"gate": wide[:, :H * V], "weight": weight, "eps": eps, "activation": activation}


def make_conv(rows: int, H: int, K: int, V: int, width: int, num_slots: int, seed: int,
              bias: bool = True, x_row_pad: int = 0) -> dict:
    """Inputs of the conv prologue; x rows sit inside a wider buffer when
    ``x_row_pad`` > 0."""
    g = _gen(seed)
    D = 2 * H * K + H * V
    x = torch.randn(rows, D + x_row_pad, generator=g).to(torch.bfloat16)[:, :D]
    weight = 0.5 * torch.randn(D, width, generator=g)
    b = 0.1 * torch.randn(D, generator=g) if bias else None
    state = torch.randn(num_slots, width - 1, D, generator=g).to(torch.bfloat16)
    return {"x": x, "weight": weight, "bias": b, "conv_state": state}


def cu_from_lengths(lens) -> torch.Tensor:
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


@dataclasses.dataclass
class Case:
    """One synthetic call. ``kind`` is 'decode', 'prefill' or 'mixed'."""
    name: str
    kind: str
    H: int
    K: int
    V: int
    inputs: dict
    pool: torch.Tensor
    block_table: torch.Tensor
    tokens_per_seq: int = 1
    cu_seqlens: torch.Tensor | None = None
    num_decodes: int = 0
    has_initial_state: torch.Tensor | None = None
    lower_bound: float | None = -5.0
    scale: float = 1.0
    num_accepted: torch.Tensor | None = None  # spec decode with a state per token
    norm: dict | None = None  # output epilogue: gate, weight, eps, activation

    @property
    def state_indices(self) -> torch.Tensor:
        return self.block_table[:, 0]

    @property
    def rows(self) -> int:
        return self.inputs["mixed_qkv"].shape[0]


def decode_case(name, H, K, V, num_seqs, tokens_per_seq, num_slots, index_stride,
                lower_bound, seed, std=0.05, null_rows=(), slot_pad=0, scale=1.0,
                pool_seed=None) -> Case:
    rows = num_seqs * tokens_per_seq
    return Case(name=name, kind="decode", H=H, K=K, V=V,
                inputs=make_token_inputs(rows, H, K, V, seed),
                pool=make_pool(num_slots, H, K, V, std,
                               seed + 1 if pool_seed is None else pool_seed, slot_pad),
                block_table=make_block_table(num_seqs, index_stride, num_slots, seed + 2, null_rows),
                tokens_per_seq=tokens_per_seq, lower_bound=lower_bound, scale=scale)


def spec_decode_case(name, H, K, V, num_seqs, tokens_per_seq, num_slots, lower_bound, seed,
                     width=8, std=0.05, null_rows=(), null_cols=(), accepted=None,
                     pool_seed=None) -> Case:
    """Spec decode with a state per token: a [num_seqs, width] block table of
    distinct slots (width >= tokens_per_seq; needs num_slots >= num_seqs *
    width), requests in ``null_rows`` padded (null slot in every column they
    use, one accepted token), (row, col) pairs in ``null_cols`` set to -1,
    and num_accepted drawn uniformly from 1..tokens_per_seq unless given."""
    assert width >= tokens_per_seq and num_slots >= num_seqs * width
    rows = num_seqs * tokens_per_seq
    table = make_block_table(num_seqs, width, num_slots, seed + 2)
    g = _gen(seed + 3)
    acc = (torch.randint(1, tokens_per_seq + 1, (num_seqs,), generator=g).to(torch.int32)
           if accepted is None else torch.tensor(accepted, dtype=torch.int32))
    for r in null_rows:
        table[r, :] = -1
        acc[r] = 1
    for r, c in null_cols:
        table[r, c] = -1
    return Case(name=name, kind="spec", H=H, K=K, V=V,
                inputs=make_token_inputs(rows, H, K, V, seed),
                pool=make_pool(num_slots, H, K, V, std, seed + 1 if pool_seed is None else pool_seed),
                block_table=table, tokens_per_seq=tokens_per_seq, lower_bound=lower_bound,
                num_accepted=acc)


def prefill_case(name, H, K, V, lens, num_slots, lower_bound, seed, std=0.05,
                 index_stride=1, has_initial=None, scale=1.0) -> Case:
    T = int(sum(lens))
    return Case(name=name, kind="prefill", H=H, K=K, V=V,
                inputs=make_token_inputs(T, H, K, V, seed),
                pool=make_pool(num_slots, H, K, V, std, seed + 1),
                block_table=make_block_table(len(lens), index_stride, num_slots, seed + 2),
                cu_seqlens=cu_from_lengths(lens),
                has_initial_state=None if has_initial is None else torch.tensor(has_initial, dtype=torch.uint8),
                lower_bound=lower_bound, scale=scale)


def mixed_case(name, H, K, V, num_decodes, prefill_lens, num_slots, lower_bound, seed,
               std=0.05, index_stride=8, scale=1.0) -> Case:
    T = num_decodes + int(sum(prefill_lens))
    return Case(name=name, kind="mixed", H=H, K=K, V=V,
                inputs=make_token_inputs(T, H, K, V, seed),
                pool=make_pool(num_slots, H, K, V, std, seed + 1),
                block_table=make_block_table(num_decodes + len(prefill_lens), index_stride, num_slots, seed + 2),
                cu_seqlens=cu_from_lengths(prefill_lens), num_decodes=num_decodes,
                lower_bound=lower_bound, scale=scale)


# ------------------------------------------------- the pages' workload shapes

def tiny_decode() -> Case:
    """8 single-token sequences, H=4, K=V=64, 32-slot pool of 0.1*randn,
    slots as column 0 of an [8, 8] block table (stride 8), lower bound -5."""
    return decode_case("tiny_decode_h4_k64_n8", 4, 64, 64, 8, 1, 32, 8, -5.0, 0, std=0.1)


def batched_decode(index_stride: int = 8, lower_bound: float | None = -5.0,
                   num_seqs: int = 32) -> Case:
    """32 single-token sequences, H=32, K=V=128, 512-slot pool (1 GiB) of
    0.05*randn, unique random slots at index stride 1 or 8."""
    variant = (index_stride == 8) * 2 + (lower_bound is None) + 4 * (num_seqs != 32)
    return decode_case(f"batched_decode_h32_k128_n{num_seqs}_s{index_stride}_lb{lower_bound}",
                       32, 128, 128, num_seqs, 1, 512, index_stride, lower_bound,
                       1000 + 10 * variant + num_seqs % 10, pool_seed=1999)


SPEC_LAYOUTS = {  # name -> (real sequences, tokens per sequence, padded null requests)
    "1x8": (1, 8, 0),
    "2x4": (2, 4, 0),
    "4x2": (4, 2, 0),
    "3x2+1null": (3, 2, 1),
}


def spec_verify(layout: str, lower_bound: float | None = -5.0) -> Case:
    """8-row spec-verify step, H=32, K=V=128, 512-slot pool; the padded
    request (if any) sits on slot -1."""
    real, tps, nulls = SPEC_LAYOUTS[layout]
    variant = list(SPEC_LAYOUTS).index(layout)
    n = real + nulls
    return decode_case(f"spec_verify_{layout}_h32_k128", 32, 128, 128, n, tps, 512, 8,
                       lower_bound, 2000 + variant, null_rows=tuple(range(real, n)),
                       pool_seed=2999)


def prefill_8192(lower_bound: float | None = -5.0) -> Case:
    """One 8192-token sequence, H=32, K=V=128, initial state 0.05*randn."""
    return prefill_case("prefill_t8192_h32_k128", 32, 128, 128, [8192], 4, lower_bound, 3000)


def prefill_varlen(lower_bound: float | None = -5.0) -> Case:
    """64 sequences with lengths U{1..256} (two forced to length 1)."""
    lens = random_lengths(64, 1, 256, 3001, force_ones=2)
    return prefill_case("prefill_varlen64_h32_k128", 32, 128, 128, lens, 128, lower_bound, 3002)


def mixed_4096(lower_bound: float | None = -5.0) -> Case:
    """96 decode rows + 5 prefill sequences summing to 4000 tokens (random cut
    points), H=32, K=V=128, 1024-slot pool (2 GiB), block table [101, 8]."""
    lens = split_total(4000, 5, 4000)
    return mixed_case("mixed_d96_p4000_h32_k128", 32, 128, 128, 96, lens, 1024,
                      lower_bound, 4001)


def prefill_65536(lower_bound: float | None = -5.0) -> Case:
    """One 65 536-token prefill, H=32, K=V=128."""
    return prefill_case("prefill_t65536_h32_k128", 32, 128, 128, [65536], 4, lower_bound, 4002)
