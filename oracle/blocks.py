"""Oracle for the block-management calls around the paged cache: copy_blocks and swap_blocks.

TEST INFRASTRUCTURE ONLY (tests, smoke check); never imported by the product path, and it shares no
code with the HIP library.

Source, by page title and section:
  [vLLM-PA] paged_attn.py (vLLM-derived fork ported to Iluvatar BI-V100), ``PagedAttention``:
            ``copy_blocks`` (for every layer's key and value cache, each (src, dst) pair of
            ``src_to_dists`` copies block src onto block dst) and ``swap_blocks`` (the same pairwise
            block copy from one cache to another, key cache then value cache, used to move blocks
            between device and host memory).

Readings where the page leaves a step open:
  * a block is the leading-index slice cache[b] of a cache [num_blocks, ...] (all kv heads, all
    slots of the block);
  * the mapping is an int64 array [n, 2] of (src, dst) block indices;
  * every pair reads the source cache as it was before the call (the pairs act at once); a mapping
    whose destinations repeat, or name another pair's source, has no single answer and is rejected;
  * copy_blocks skips pairs naming a block outside the cache (the kernel does the same); swap_blocks
    rejects them.
The copies are bit copies: values are handled as raw 16-bit patterns.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _bits(x) -> np.ndarray:
    if torch is not None and isinstance(x, torch.Tensor):
        t = x.detach().to("cpu").contiguous()
        return t.view(torch.int16).numpy().copy() if t.element_size() == 2 else t.numpy().copy()
    return np.array(x, copy=True)


def _pairs(mapping) -> np.ndarray:
    if torch is not None and isinstance(mapping, torch.Tensor):
        m = mapping.detach().to("cpu").to(torch.int64).numpy()
    else:
        m = np.asarray(mapping, dtype=np.int64)
    m = m.reshape(-1, 2)
    return m


def _check_simultaneous(m: np.ndarray) -> None:
    dst = m[:, 1]
    if np.unique(dst).size != dst.size:
        raise ValueError("a destination block repeats")
    moving = m[m[:, 0] != m[:, 1]]
    if np.intersect1d(moving[:, 0], moving[:, 1]).size:
        raise ValueError("a destination block is another pair's source")


def copy_blocks(k_caches: Sequence, v_caches: Sequence, mapping) -> Tuple[List[np.ndarray], List[np.ndarray]]:
    """[vLLM-PA] ``copy_blocks``: for every layer l and pair (s, d): K_l[d] = K_l[s], V_l[d] = V_l[s].
    Pairs naming a block outside [0, num_blocks) are skipped. Returns the new caches (bit patterns)."""
    m = _pairs(mapping)
    outs = []
    for caches in (k_caches, v_caches):
        layer_out = []
        for c in caches:
            src = _bits(c)
            nb = src.shape[0]
            ok = (m[:, 0] >= 0) & (m[:, 0] < nb) & (m[:, 1] >= 0) & (m[:, 1] < nb)
            live = m[ok]
            _check_simultaneous(live)
            dst = src.copy()
            for s, d in live:
                dst[d] = src[s]
            layer_out.append(dst)
        outs.append(layer_out)
    return outs[0], outs[1]


def swap_blocks(src_cache, dst_cache, mapping) -> np.ndarray:
    """[vLLM-PA] ``swap_blocks`` for one cache: dst[d] = src[s] for every pair (s, d); other blocks of
    dst keep their contents. Out-of-range pairs raise. Returns the new dst (bit patterns)."""
    m = _pairs(mapping)
    src = _bits(src_cache)
    dst = _bits(dst_cache)
    if ((m[:, 0] < 0) | (m[:, 0] >= src.shape[0]) | (m[:, 1] < 0) | (m[:, 1] >= dst.shape[0])).any():
        raise IndexError("block index outside the cache")
    if np.unique(m[:, 1]).size != m.shape[0]:
        raise ValueError("a destination block repeats")
    out = dst.copy()
    for s, d in m:
        out[d] = src[s]
    return out
