"""fp64 oracle: exact softmax attention read through a block table, plus the cache scatter.

TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline). The product path never imports
this module, and it shares no code with the HIP library.

Sources, by page title and section:
  [vLLM-PA]  paged_attn.py (vLLM-derived fork ported to Iluvatar BI-V100), ``PagedAttention``:
             ``_forward_decode_pytorch`` (tile loop with running max/sum and final divide),
             ``forward_decode`` (V1 single pass, V2 with 512-token partitions and their
             max-logit / exp-sum temporaries), ``_forward_prefix_pytorch`` (phase 1 prefix keys
             unmasked, phase 2 chunk keys with a causal mask), ``write_to_paged_cache``.
  [Atlas-FI] spark_runtime/flashinfer.rs, ``ragged_prefill_bf16_hd256`` (ragged rows from
             qo_indptr / kv_indptr) and its CPU-reference test (per-request causal GQA attention).
  [libmir]   libmir-cuda 0.3.0 src/backend/kv/attention/mod.rs, ``PagedAttentionBf16::validate_table``.

Readings where the pages leave a step open:
  * cache layout is [num_blocks, num_kv_heads, block_size, head_dim] for K and V;
  * block tables are int32 padded with -1; only the first ceil(L/block_size) entries are read;
  * slots past a sequence's length are excluded by length (never read), whatever they hold;
  * a sequence of length 0, and a causal row that sees no key, give an all-zero output row;
  * causal alignment is bottom-right: query i of a request sits at absolute key position
    kv_len - qo_len + i and sees keys j <= that position;
  * slot_mapping entries < 0 are skipped; duplicate or out-of-range slots are caller errors.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

try:  # torch is optional here: the oracle also takes plain numpy arrays
    import torch
except ImportError:  # pragma: no cover
    torch = None

# Status codes of the library contract, used by the host-side table validator below.
STATUS = {"OK": 0, "INVALID_ARGUMENT": 1, "UNSUPPORTED": 2, "BAD_TABLE": 3,
          "WORKSPACE_TOO_SMALL": 4, "HIP_ERROR": 5}


# ----------------------------------------------------------------------------------------------
# Conversions. bf16 -> f32 -> f64 widening is exact.
# ----------------------------------------------------------------------------------------------
def _is_torch(x) -> bool:
    return torch is not None and isinstance(x, torch.Tensor)


def _f64(x) -> np.ndarray:
    if _is_torch(x):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _ints(x) -> np.ndarray:
    if _is_torch(x):
        return x.detach().to("cpu").to(torch.int64).numpy()
    return np.asarray(x, dtype=np.int64)


def _bits16(x) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 tensor (or an int16/uint16 array) as int16."""
    if _is_torch(x):
        return x.detach().to("cpu").contiguous().view(torch.int16).numpy().copy()
    a = np.asarray(x)
    if a.dtype.itemsize != 2:
        raise TypeError("expected 16-bit data")
    return a.view(np.int16).copy()


# ----------------------------------------------------------------------------------------------
# The two index rules every path shares.
# ----------------------------------------------------------------------------------------------
def kv_head_of(q_head, group: int):
    """Grouped-query attention: consecutive q heads share one kv head, kh = h // (Hq / Hkv).

    [Atlas-FI] CPU-reference test (``kh = h / group``); [vLLM-PA] decode fallback views the query
    as (num_kv_heads, gqa_ratio, head_dim).
    """
    return q_head // group


def key_visible(i, j, qo_len: int, kv_len: int, causal: bool):
    """Whether key j is visible to query row i of a request (broadcasts over arrays).

    Causal rows are aligned bottom-right: row i sits at absolute position kv_len - qo_len + i.
    [Atlas-FI] CPU-reference test (qo == kv, keys 0..=qi); [vLLM-PA] ``_forward_prefix_pytorch``:
    prefix keys are all visible, chunk key k is visible to chunk row q iff k <= q.
    """
    i = np.asarray(i)
    j = np.asarray(j)
    if not causal:
        return np.ones(np.broadcast(i, j).shape, dtype=bool)
    return j <= i + (kv_len - qo_len)


# ----------------------------------------------------------------------------------------------
# Block-table read.
# ----------------------------------------------------------------------------------------------
def gather_tokens(cache, table_row, length: int, kv_head: int, block_size: int) -> np.ndarray:
    """Logical rows [0, length) of one sequence for one kv head, as float64 [length, D].

    Token t lives in physical block table_row[t // block_size] at offset t % block_size
    ([vLLM-PA] ``PagedAttentionMetadata.block_tables``: logical block -> physical block).
    """
    t = np.arange(int(length))
    row = _ints(table_row)
    blk = row[t // block_size]
    off = t % block_size
    if length and (blk.min() < 0 or blk.max() >= cache.shape[0]):
        raise IndexError("block table entry outside the pool")
    if _is_torch(cache):
        rows = cache[torch.from_numpy(blk), kv_head, torch.from_numpy(off)]
        return _f64(rows)
    return _f64(np.asarray(cache)[blk, kv_head, off])


# ----------------------------------------------------------------------------------------------
# The core definition: softmax(scale * Q K^T) V over the visible keys.
# ----------------------------------------------------------------------------------------------
def attend_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                visible: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """out[r] = sum_t w[r,t] V[t] / sum_t w[r,t],  w = exp(s - max s),  s = scale <Q[r], K[t]>.

    Also returns lse[r] = log sum_t exp(s[r,t]). A row with no visible key returns zeros and
    lse = -inf. ([vLLM-PA] ``_forward_decode_pytorch``: scores, max-shifted exponentials, running
    sum, final divide; [Atlas-FI] CPU-reference test: max, exp, denominator, weighted V.)
    """
    Q = np.asarray(Q, dtype=np.float64)
    nq, nk = Q.shape[0], K.shape[0]
    out = np.zeros((nq, V.shape[1]), dtype=np.float64)
    lse = np.full(nq, -np.inf)
    if nq == 0 or nk == 0:
        return out, lse
    s = scale * (Q @ K.T)
    if visible is not None:
        s = np.where(visible, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    w = np.exp(s[has] - m[has, None])
    l = w.sum(axis=1)
    out[has] = (w @ V) / l[:, None]
    lse[has] = m[has] + np.log(l)
    return out, lse


# ----------------------------------------------------------------------------------------------
# Decode: one query token per sequence.
# ----------------------------------------------------------------------------------------------
def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                 return_lse: bool = False):
    """out[b, h] = attention of q[b, h] over tokens [0, L_b) of sequence b, read through its table.

    A sequence of length 0 gives zeros ([vLLM-PA] ``_forward_decode_pytorch`` zeroes such rows).
    q: [B, Hq, D]; caches: [NB, Hkv, bs, D]; block_tables: [B, max_blocks]; seq_lens: [B].
    """
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
        if L == 0:
            continue
        for kh in range(Hkv):
            K = gather_tokens(k_cache, tables[b], L, kh, bs)
            V = gather_tokens(v_cache, tables[b], L, kh, bs)
            hs = heads[kv_head_of(heads, G) == kh]
            out[b, hs], lse[b, hs] = attend_rows(qf[b, hs], K, V, scale)
    return (out, lse) if return_lse else out


def paged_decode_pairs(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                       pairs: Iterable[Tuple[int, int]]) -> np.ndarray:
    """paged_decode restricted to the listed (b, h) pairs; returns [len(pairs), D]."""
    Hq = q.shape[1]
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    tables = _ints(block_tables)
    lens = _ints(seq_lens)
    pairs = list(pairs)
    out = np.zeros((len(pairs), q.shape[2]))
    for n, (b, h) in enumerate(pairs):
        L = int(lens[b])
        if L == 0:
            continue
        kh = kv_head_of(h, G)
        K = gather_tokens(k_cache, tables[b], L, kh, bs)
        V = gather_tokens(v_cache, tables[b], L, kh, bs)
        out[n], _ = attend_rows(_f64(q[b, h])[None, :], K, V, scale)
    return out


def decode_partials(q, k_cache, v_cache, block_tables, seq_lens, scale: float, partition_tokens: int):
    """Per-partition softmax statistics of decode, partitions of ``partition_tokens`` logical tokens.

    For partition p of sequence b (tokens [p*P, min((p+1)*P, L_b))), per q head:
      m_p = max s,  l_p = sum exp(s - m_p),  o_p = sum exp(s - m_p) V / l_p.
    Partitions with no token have m_p = -inf, l_p = 0, o_p = 0. ([vLLM-PA] ``forward_decode``:
    V2 cuts tokens into 512-token partitions with per-partition max logits and exp sums.)
    Returns o [B, Hq, Pmax, D], m [B, Hq, Pmax], l [B, Hq, Pmax].
    """
    qf = _f64(q)
    B, Hq, D = qf.shape
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    tables = _ints(block_tables)
    lens = _ints(seq_lens)
    P = max(1, max((int(L) + partition_tokens - 1) // partition_tokens for L in lens) if B else 1)
    o = np.zeros((B, Hq, P, D))
    m = np.full((B, Hq, P), -np.inf)
    l = np.zeros((B, Hq, P))
    heads = np.arange(Hq)
    for b in range(B):
        L = int(lens[b])
        for kh in range(Hkv):
            if L == 0:
                continue
            K = gather_tokens(k_cache, tables[b], L, kh, bs)
            V = gather_tokens(v_cache, tables[b], L, kh, bs)
            hs = heads[kv_head_of(heads, G) == kh]
            for p in range((L + partition_tokens - 1) // partition_tokens):
                t0, t1 = p * partition_tokens, min(L, (p + 1) * partition_tokens)
                s = scale * (qf[b, hs] @ K[t0:t1].T)
                mp = s.max(axis=1)
                w = np.exp(s - mp[:, None])
                lp = w.sum(axis=1)
                m[b, hs, p] = mp
                l[b, hs, p] = lp
                o[b, hs, p] = (w @ V[t0:t1]) / lp[:, None]
    return o, m, l


def merge_partials(o, m, l) -> Tuple[np.ndarray, np.ndarray]:
    """Log-sum-exp merge of partition statistics over the last-but-one axis of ``o``.

    Over partitions with l_p > 0: M = max m_p, w_p = l_p exp(m_p - M),
    out = sum w_p o_p / sum w_p, lse = M + log sum w_p. With no such partition: zeros, -inf.
    This is the running-max rescale of [vLLM-PA] ``_forward_decode_pytorch`` (corr = exp(m - m_new),
    l = l*corr + sum, o = o*corr + P V) applied once to whole partitions.
    """
    o = np.asarray(o, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    live = l > 0
    M = np.where(live, m, -np.inf).max(axis=-1)
    has = np.isfinite(M)
    Ms = np.where(has, M, 0.0)
    w = np.where(live, l * np.exp(np.where(live, m, 0.0) - Ms[..., None]), 0.0)
    den = w.sum(axis=-1)
    safe = np.where(has, den, 1.0)
    out = np.where(has[..., None], (w[..., None] * o).sum(axis=-2) / safe[..., None], 0.0)
    lse = np.where(has, Ms + np.log(safe), -np.inf)
    return out, lse


# ----------------------------------------------------------------------------------------------
# Prefill: ragged rows, contiguous or paged K/V.
# ----------------------------------------------------------------------------------------------
def _request_of(indptr: np.ndarray, t: int) -> int:
    b = int(np.searchsorted(indptr, t, side="right")) - 1
    if not (0 <= b < len(indptr) - 1 and indptr[b] <= t < indptr[b + 1]):
        raise IndexError("row outside every request")
    return b


def ragged_prefill(q, k, v, qo_indptr, kv_indptr, causal: bool, scale: float) -> np.ndarray:
    """Per request b: rows qo_indptr[b]..qo_indptr[b+1] of q attend to rows kv_indptr[b]..
    kv_indptr[b+1] of k/v, causal (bottom-right) if asked. ([Atlas-FI] ``ragged_prefill_bf16_hd256``
    and its CPU-reference test.) q: [Tq, Hq, D]; k, v: [Tkv, Hkv, D]; returns [Tq, Hq, D]."""
    qf, kf, vf = _f64(q), _f64(k), _f64(v)
    Tq, Hq, D = qf.shape
    Hkv = kf.shape[1]
    G = Hq // Hkv
    qi, ki = _ints(qo_indptr), _ints(kv_indptr)
    out = np.zeros((Tq, Hq, D))
    for b in range(len(qi) - 1):
        q0, q1, k0, k1 = int(qi[b]), int(qi[b + 1]), int(ki[b]), int(ki[b + 1])
        nq, nk = q1 - q0, k1 - k0
        if nq == 0:
            continue
        vis = key_visible(np.arange(nq)[:, None], np.arange(nk)[None, :], nq, nk, causal)
        for h in range(Hq):
            kh = kv_head_of(h, G)
            out[q0:q1, h], _ = attend_rows(qf[q0:q1, h], kf[k0:k1, kh], vf[k0:k1, kh], scale, vis)
    return out


def ragged_prefill_rows(q, k, v, qo_indptr, kv_indptr, causal: bool, scale: float,
                        rows: Iterable[Tuple[int, int]]) -> np.ndarray:
    """ragged_prefill restricted to the listed (q row, q head) pairs; returns [len(rows), D]."""
    Hq = q.shape[1]
    G = Hq // k.shape[1]
    qi, ki = _ints(qo_indptr), _ints(kv_indptr)
    rows = list(rows)
    out = np.zeros((len(rows), q.shape[2]))
    for n, (t, h) in enumerate(rows):
        b = _request_of(qi, int(t))
        i = int(t) - int(qi[b])
        nq, nk = int(qi[b + 1] - qi[b]), int(ki[b + 1] - ki[b])
        kh = kv_head_of(h, G)
        K = _f64(k[int(ki[b]):int(ki[b + 1]), kh])
        V = _f64(v[int(ki[b]):int(ki[b + 1]), kh])
        vis = key_visible(i, np.arange(nk), nq, nk, causal)[None, :]
        out[n], _ = attend_rows(_f64(q[int(t), h])[None, :], K, V, scale, vis)
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, qo_indptr, kv_lens, causal: bool,
                  scale: float) -> np.ndarray:
    """Prefill whose K/V come through the block table: request b's queries (rows of q given by
    qo_indptr) attend to its first kv_lens[b] cached tokens; query i sees keys
    j <= kv_lens[b] - qo_len + i when causal. ([vLLM-PA] ``_forward_prefix_pytorch``: the cached
    prefix is visible to every chunk row, the chunk itself is causal.)"""
    qf = _f64(q)
    Tq, Hq, D = qf.shape
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    tables = _ints(block_tables)
    qi, kl = _ints(qo_indptr), _ints(kv_lens)
    out = np.zeros((Tq, Hq, D))
    for b in range(len(qi) - 1):
        q0, q1, nk = int(qi[b]), int(qi[b + 1]), int(kl[b])
        nq = q1 - q0
        if nq == 0:
            continue
        vis = key_visible(np.arange(nq)[:, None], np.arange(nk)[None, :], nq, nk, causal)
        for kh in range(Hkv):
            K = gather_tokens(k_cache, tables[b], nk, kh, bs)
            V = gather_tokens(v_cache, tables[b], nk, kh, bs)
            for h in range(kh * G, (kh + 1) * G):
                out[q0:q1, h], _ = attend_rows(qf[q0:q1, h], K, V, scale, vis)
    return out


def paged_prefill_rows(q, k_cache, v_cache, block_tables, qo_indptr, kv_lens, causal: bool,
                       scale: float, rows: Iterable[Tuple[int, int]]) -> np.ndarray:
    """paged_prefill restricted to the listed (q row, q head) pairs; returns [len(rows), D]."""
    Hq = q.shape[1]
    Hkv, bs = k_cache.shape[1], k_cache.shape[2]
    G = Hq // Hkv
    tables = _ints(block_tables)
    qi, kl = _ints(qo_indptr), _ints(kv_lens)
    rows = list(rows)
    out = np.zeros((len(rows), q.shape[2]))
    for n, (t, h) in enumerate(rows):
        b = _request_of(qi, int(t))
        i = int(t) - int(qi[b])
        nq, nk = int(qi[b + 1] - qi[b]), int(kl[b])
        kh = kv_head_of(h, G)
        K = gather_tokens(k_cache, tables[b], nk, kh, bs)
        V = gather_tokens(v_cache, tables[b], nk, kh, bs)
        vis = key_visible(i, np.arange(nk), nq, nk, causal)[None, :]
        out[n], _ = attend_rows(_f64(q[int(t), h])[None, :], K, V, scale, vis)
    return out


# ----------------------------------------------------------------------------------------------
# Cache scatter (bit copy) and the host-side table check.
# ----------------------------------------------------------------------------------------------
def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping) -> Tuple[np.ndarray, np.ndarray]:
    """For each new token t with s = slot_mapping[t] >= 0 and every kv head h:
    k_cache[s // bs, h, s % bs, :] = k[t, h, :], the same for v. Returns new caches as int16 bit
    patterns. ([vLLM-PA] ``write_to_paged_cache``: key/value [T, Hkv, D] scattered by the flattened
    slot_mapping.) Duplicate or out-of-range slots raise."""
    kb, vb = _bits16(k), _bits16(v)
    kc, vc = _bits16(k_cache), _bits16(v_cache)
    nb, _, bs, _ = kc.shape
    slots = _ints(slot_mapping).reshape(-1)
    live = slots[slots >= 0]
    if live.size and (live.max() >= nb * bs):
        raise IndexError("slot outside the pool")
    if np.unique(live).size != live.size:
        raise ValueError("duplicate slot in slot_mapping")
    for t, s in enumerate(slots):
        if s < 0:
            continue
        kc[s // bs, :, s % bs, :] = kb[t]
        vc[s // bs, :, s % bs, :] = vb[t]
    return kc, vc


def validate_block_tables(block_tables, seq_lens, block_size: int, num_blocks: int) -> int:
    """Checked-mode table validation, returning a status code of the library contract.

    Rules ([libmir] ``validate_table``): the table must hold its declared tokens
    (ceil(L/bs) <= max_blocks_per_seq), and every entry a sequence reads must name a physical block
    that exists (0 <= id < num_blocks). Malformed sizes are an invalid argument.
    """
    if block_size <= 0 or num_blocks < 0:
        return STATUS["INVALID_ARGUMENT"]
    tables = _ints(block_tables)
    lens = _ints(seq_lens).reshape(-1)
    if tables.ndim != 2 or tables.shape[0] != lens.shape[0]:
        return STATUS["INVALID_ARGUMENT"]
    if (lens < 0).any():
        return STATUS["INVALID_ARGUMENT"]
    width = tables.shape[1]
    for b, L in enumerate(lens):
        need = (int(L) + block_size - 1) // block_size
        if need > width:
            return STATUS["BAD_TABLE"]
        used = tables[b, :need]
        if need and (used.min() < 0 or used.max() >= num_blocks):
            return STATUS["BAD_TABLE"]
    return STATUS["OK"]
