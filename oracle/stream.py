"""Oracle for decode attention over part of a sequence: a sliding window of the last W tokens, and
attention streamed over several launches, each over a tile of resident blocks.

TEST INFRASTRUCTURE ONLY (tests, smoke check); never imported by the product path, and it shares no
code with the HIP library.

Sources, by page title and section:
  [Atlas-swap] spark_storage/high_speed_swap/impl_more.rs, ``attend_layer_on_stream_with_q_pos``:
               a step begins, each tile of at most ``resident_blocks`` blocks is attended by one
               launch through its own block table (the last block of the final tile consuming only
               ``last_block_valid_slots`` slots), and a final call normalises the output.
  [vLLM-PA]    paged_attn.py, ``forward_decode`` (``sliding_window``) and the libmir-cuda page's
               split plan (``captured_configs(token_count, window)``): attention restricted to the
               most recent tokens.

Readings where the pages leave a step open:
  * a window W keeps keys t with L - W <= t < L (all keys when W <= 0 or W >= L);
  * streamed attention over tiles is attention over the concatenation of every tile's tokens:
    softmax is invariant to the order of its terms, so the tiles may come in any order; a tile's
    tokens are its first ``tile_len`` logical slots read through the tile's table.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, _ints, attend_rows, gather_tokens, kv_head_of


def paged_decode_window(q, k_cache, v_cache, block_tables, seq_lens, scale: float, window: int,
                        return_lse: bool = False):
    """Decode attention of q[b, h] over keys [max(0, L_b - window), L_b) of sequence b."""
    qf = _f64(q)
    B, Hq, D = qf.shape
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    tables = _ints(block_tables)
    lens = _ints(seq_lens)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    heads = np.arange(Hq)
    for b in range(B):
        L = int(lens[b])
        lo = max(0, L - window) if window > 0 else 0
        if L == 0:
            continue
        for kh in range(Hkv):
            K = gather_tokens(k_cache, tables[b], L, kh, bs)[lo:]
            V = gather_tokens(v_cache, tables[b], L, kh, bs)[lo:]
            hs = heads[kv_head_of(heads, G) == kh]
            out[b, hs], lse[b, hs] = attend_rows(qf[b, hs], K, V, scale)
    return (out, lse) if return_lse else out


def streamed_decode(q, k_cache, v_cache, tiles, scale: float, return_lse: bool = False):
    """Attention of q[b, h] over the tokens of every tile: ``tiles`` is a list of
    (tile_tables [B, cap], tile_lens [B]) pairs; tile i contributes the first tile_lens[b] logical
    slots of its table row b."""
    qf = _f64(q)
    B, Hq, D = qf.shape
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    heads = np.arange(Hq)
    for b in range(B):
        for kh in range(Hkv):
            Ks, Vs = [], []
            for tables, lens in tiles:
                n = int(_ints(lens)[b])
                if n == 0:
                    continue
                row = _ints(tables)[b]
                Ks.append(gather_tokens(k_cache, row, n, kh, bs))
                Vs.append(gather_tokens(v_cache, row, n, kh, bs))
            if not Ks:
                continue
            hs = heads[kv_head_of(heads, G) == kh]
            out[b, hs], lse[b, hs] = attend_rows(qf[b, hs], np.concatenate(Ks), np.concatenate(Vs), scale)
    return (out, lse) if return_lse else out
