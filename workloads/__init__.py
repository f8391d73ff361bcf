"""Seeded synthetic inputs for attention over a paged, block-table-indexed KV cache.

This module is shared by the CPU oracle's tests and by the GPU path's tests and benchmark. It holds
none of the method's arithmetic: only random draws, length draws, the deal of a shuffled block pool
to sequences, NaN fill of slack cache slots, and the slot address of each new token (the caller-side
input that the cache scatter consumes: slot = physical block * block_size + offset, as the vLLM
``PagedAttention.write_to_paged_cache`` page describes its ``slot_mapping``).

Recipe (one ``torch.Generator('cpu')`` per case, fixed draw order):
  lengths -> (prefix lengths) -> block permutation -> q -> k -> v (-> k_new, v_new)
Values are ``randn`` float32 rounded to bfloat16 (round-to-nearest-even, ``Tensor.to``). Lengths are
``randint(lo, hi + 1)``. Pools hold exactly the blocks the sequences need unless a pool size is
given; a seeded ``randperm`` of the pool is dealt to sequences in order. Cache slots that hold no
token (tail of a sequence's last block, and unused blocks) are NaN, so any read of them shows.

Cache layout (both K and V): ``[num_blocks, num_kv_heads, block_size, head_dim]`` bfloat16.
Block tables: int32 ``[batch, max_blocks_per_seq]``, padded with -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import torch

BLOCK_SIZE = 16
SEED_BASE = 232000
_CHUNK = 1 << 24  # randn is drawn in fixed chunks of this many values (part of the recipe)

__all__ = [
    "BLOCK_SIZE", "SEED_BASE", "DecodeInputs", "RaggedInputs", "ChunkedInputs",
    "paged_decode_inputs", "ragged_prefill_inputs", "chunked_prefill_inputs",
    "CONFIGS", "make_config", "config_seed",
]


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn_bf16(g: torch.Generator, shape: Sequence[int]) -> torch.Tensor:
    """N(0,1) float32 draws rounded to bfloat16, drawn in fixed-size chunks."""
    n = 1
    for s in shape:
        n *= int(s)
    out = torch.empty(n, dtype=torch.bfloat16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        out[s:e] = torch.randn(e - s, generator=g, dtype=torch.float32).to(torch.bfloat16)
    return out.view(*[int(s) for s in shape])


def _draw_lengths(g, lengths, length_range, batch) -> List[int]:
    if lengths is not None:
        return [int(x) for x in lengths]
    lo, hi = length_range
    return [int(x) for x in torch.randint(int(lo), int(hi) + 1, (int(batch),), generator=g)]


def _deal_blocks(g, kv_lens: List[int], bs: int, num_blocks: Optional[int]):
    """Shuffle the pool and deal blocks to sequences in order. Returns (tables, perm, used, NB)."""
    need = [(L + bs - 1) // bs for L in kv_lens]
    used = sum(need)
    nb = used if num_blocks is None else int(num_blocks)
    if nb < used:
        raise ValueError(f"pool of {nb} blocks cannot hold {used} needed blocks")
    perm = torch.randperm(max(nb, 1), generator=g)[:nb] if nb > 0 else torch.zeros(0, dtype=torch.long)
    width = max(max(need) if need else 0, 1)
    tables = torch.full((len(kv_lens), width), -1, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(need):
        if n:
            tables[b, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    return tables, perm, used, nb


def _nan_fill(cache: torch.Tensor, tables: torch.Tensor, valid_lens: List[int], perm, used: int, bs: int):
    """NaN every slot that holds no token: unused blocks and the tail of each last block."""
    nan = float("nan")
    if perm.numel() > used:
        cache[perm[used:]] = nan
    for b, L in enumerate(valid_lens):
        r = L % bs
        if L > 0 and r:
            blk = int(tables[b, (L - 1) // bs])
            cache[blk, :, r:, :] = nan


@dataclass
class DecodeInputs:
    q: torch.Tensor             # [B, Hq, D] bf16
    k_cache: torch.Tensor       # [NB, Hkv, BS, D] bf16
    v_cache: torch.Tensor       # [NB, Hkv, BS, D] bf16
    block_tables: torch.Tensor  # [B, max_blocks] int32, pad -1
    seq_lens: torch.Tensor      # [B] int32
    scale: float
    block_size: int
    meta: Dict = field(default_factory=dict)

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.numel() else 0


def paged_decode_inputs(seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                        seq_lens: Optional[Sequence[int]] = None, len_range=None, batch=None,
                        block_size: int = BLOCK_SIZE, num_blocks: Optional[int] = None,
                        scale: Optional[float] = None) -> DecodeInputs:
    g = _gen(seed)
    lens = _draw_lengths(g, seq_lens, len_range, batch)
    tables, perm, used, nb = _deal_blocks(g, lens, block_size, num_blocks)
    B = len(lens)
    q = randn_bf16(g, (B, num_q_heads, head_dim))
    k_cache = randn_bf16(g, (nb, num_kv_heads, block_size, head_dim))
    v_cache = randn_bf16(g, (nb, num_kv_heads, block_size, head_dim))
    _nan_fill(k_cache, tables, lens, perm, used, block_size)
    _nan_fill(v_cache, tables, lens, perm, used, block_size)
    return DecodeInputs(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
                        seq_lens=torch.tensor(lens, dtype=torch.int32),
                        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                        block_size=block_size, meta={"seed": seed, "num_blocks": nb, "used_blocks": used})


@dataclass
class RaggedInputs:
    q: torch.Tensor          # [Tq, Hq, D] bf16
    k: torch.Tensor          # [Tkv, Hkv, D] bf16
    v: torch.Tensor          # [Tkv, Hkv, D] bf16
    qo_indptr: torch.Tensor  # [B+1] int32
    kv_indptr: torch.Tensor  # [B+1] int32
    causal: bool
    scale: float
    meta: Dict = field(default_factory=dict)


def _indptr(lens: List[int]) -> torch.Tensor:
    out = [0]
    for L in lens:
        out.append(out[-1] + int(L))
    return torch.tensor(out, dtype=torch.int32)


def ragged_prefill_inputs(seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                          qo_lens: Optional[Sequence[int]] = None, kv_lens: Optional[Sequence[int]] = None,
                          len_range=None, batch=None, causal: bool = True,
                          scale: Optional[float] = None) -> RaggedInputs:
    """Ragged requests. With no ``kv_lens`` the kv lengths equal the q lengths (no cached prefix)."""
    g = _gen(seed)
    qo = _draw_lengths(g, qo_lens, len_range, batch)
    kv = list(qo) if kv_lens is None else [int(x) for x in kv_lens]
    if len(kv) != len(qo):
        raise ValueError("qo_lens and kv_lens differ in length")
    qi, ki = _indptr(qo), _indptr(kv)
    q = randn_bf16(g, (int(qi[-1]), num_q_heads, head_dim))
    k = randn_bf16(g, (int(ki[-1]), num_kv_heads, head_dim))
    v = randn_bf16(g, (int(ki[-1]), num_kv_heads, head_dim))
    return RaggedInputs(q=q, k=k, v=v, qo_indptr=qi, kv_indptr=ki, causal=bool(causal),
                        scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                        meta={"seed": seed})


@dataclass
class ChunkedInputs:
    q: torch.Tensor             # [Tc, Hq, D] bf16 (new chunk queries)
    k_new: torch.Tensor         # [Tc, Hkv, D] bf16 (new chunk keys, to be scattered)
    v_new: torch.Tensor         # [Tc, Hkv, D] bf16
    k_cache: torch.Tensor       # [NB, Hkv, BS, D] bf16, prefix filled, chunk slots NaN
    v_cache: torch.Tensor
    block_tables: torch.Tensor  # [B, max_blocks] int32
    slot_mapping: torch.Tensor  # [Tc] int64
    qo_indptr: torch.Tensor     # [B+1] int32 (chunk offsets)
    kv_lens: torch.Tensor       # [B] int32 (prefix + chunk)
    prefix_lens: torch.Tensor   # [B] int32
    causal: bool
    scale: float
    block_size: int
    meta: Dict = field(default_factory=dict)


def chunked_prefill_inputs(seed: int, *, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           chunk_lens: Optional[Sequence[int]] = None, prefix_lens: Optional[Sequence[int]] = None,
                           chunk_range=None, prefix_range=None, batch=None, block_size: int = BLOCK_SIZE,
                           num_blocks: Optional[int] = None, causal: bool = True,
                           scale: Optional[float] = None) -> ChunkedInputs:
    """A cached prefix in the paged pool plus a new chunk per request, still to be scattered."""
    g = _gen(seed)
    C = _draw_lengths(g, chunk_lens, chunk_range, batch)
    P = _draw_lengths(g, prefix_lens, prefix_range, len(C))
    if len(P) != len(C):
        raise ValueError("prefix_lens and chunk_lens differ in length")
    kv = [p + c for p, c in zip(P, C)]
    tables, perm, used, nb = _deal_blocks(g, kv, block_size, num_blocks)
    qi = _indptr(C)
    Tc = int(qi[-1])
    q = randn_bf16(g, (Tc, num_q_heads, head_dim))
    k_cache = randn_bf16(g, (nb, num_kv_heads, block_size, head_dim))
    v_cache = randn_bf16(g, (nb, num_kv_heads, block_size, head_dim))
    k_new = randn_bf16(g, (Tc, num_kv_heads, head_dim))
    v_new = randn_bf16(g, (Tc, num_kv_heads, head_dim))
    # Slots from the prefix end onward hold no token yet: NaN until the scatter writes the chunk.
    _nan_fill(k_cache, tables, P, perm, used, block_size)
    _nan_fill(v_cache, tables, P, perm, used, block_size)
    slots = torch.empty(Tc, dtype=torch.int64)
    nan = float("nan")
    for b in range(len(C)):
        first_chunk_block = P[b] // block_size
        n_blocks = (kv[b] + block_size - 1) // block_size
        for j in range(first_chunk_block, n_blocks):
            blk = int(tables[b, j])
            lo = max(P[b] - j * block_size, 0)
            k_cache[blk, :, lo:, :] = nan
            v_cache[blk, :, lo:, :] = nan
        for i in range(C[b]):
            pos = P[b] + i
            slots[int(qi[b]) + i] = int(tables[b, pos // block_size]) * block_size + pos % block_size
    return ChunkedInputs(q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache,
                         block_tables=tables, slot_mapping=slots, qo_indptr=qi,
                         kv_lens=torch.tensor(kv, dtype=torch.int32),
                         prefix_lens=torch.tensor(P, dtype=torch.int32), causal=bool(causal),
                         scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                         block_size=block_size, meta={"seed": seed, "num_blocks": nb, "used_blocks": used})


# The five workloads. Each is seeded SEED_BASE + id.
CONFIGS = {
    1: dict(kind="decode", name="tiny paged decode", num_q_heads=4, num_kv_heads=2, head_dim=64,
            seq_lens=[37, 100], num_blocks=16),
    2: dict(kind="ragged", name="ragged causal prefill", num_q_heads=32, num_kv_heads=8, head_dim=128,
            len_range=(128, 2048), batch=8, causal=True),
    3: dict(kind="decode", name="batched paged decode", num_q_heads=32, num_kv_heads=8, head_dim=128,
            len_range=(512, 8192), batch=64),
    4: dict(kind="decode", name="long-context split-KV decode", num_q_heads=64, num_kv_heads=8,
            head_dim=128, seq_lens=[131072] * 4),
    5: dict(kind="chunked", name="chunked prefill over paged prefix", num_q_heads=16, num_kv_heads=4,
            head_dim=256, chunk_range=(64, 1024), prefix_range=(0, 4096), batch=16, causal=True),
}


def config_seed(cid: int) -> int:
    return SEED_BASE + int(cid)


def make_config(cid: int):
    spec = dict(CONFIGS[int(cid)])
    kind = spec.pop("kind")
    spec.pop("name")
    seed = config_seed(cid)
    if kind == "decode":
        return paged_decode_inputs(seed, **spec)
    if kind == "ragged":
        return ragged_prefill_inputs(seed, **spec)
    return chunked_prefill_inputs(seed, **spec)
