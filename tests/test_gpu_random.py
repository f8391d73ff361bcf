"""Seeded random parity sweep on the GPU, through the C ABI: each case draws a shape (batch, lengths,
head counts and GQA group, head_dim, block size, causal mode, decode path, window, cache dtype) and
compares the kernels with the fp64 oracle on the seeded inputs of that shape. The fixed edge lists in
the other GPU tests pin chosen corners; this sweep covers combinations nobody listed."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_232_amd as pkv
from parity import assert_parity
from test_gpu_stream import _tiles
from workloads import chunked_prefill_inputs, paged_decode_inputs, ragged_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

HEAD_DIMS = (64, 128, 256)
GROUPS = (1, 2, 3, 4, 6, 8, 12, 16)
KV_HEADS = (1, 2, 3, 4, 8)
BLOCK_SIZES = (16, 32, 64, 128, 256)


def _length(rng, hi: int, tile: int) -> int:
    """A length with the edges over-drawn: 0, 1, a tile multiple +-1, else uniform in [2, hi]."""
    u = rng.random()
    if u < 0.1:
        return 0
    if u < 0.2:
        return 1
    if u < 0.45:
        k = int(rng.integers(1, max(2, hi // tile) + 1))
        return max(0, min(hi, k * tile + int(rng.integers(-1, 2))))
    return int(rng.integers(2, hi + 1))


def _heads(rng, max_q_heads: int = 32):
    while True:
        hkv = int(rng.choice(KV_HEADS))
        g = int(rng.choice(GROUPS))
        if hkv * g <= max_q_heads:
            return hkv * g, hkv


def _draw_prefill(seed: int):
    rng = np.random.default_rng(seed)
    d = int(rng.choice(HEAD_DIMS))
    hq, hkv = _heads(rng, 24 if d == 256 else 32)
    batch = int(rng.integers(1, 6))
    cap = 300 if d == 256 else 400
    qo = [_length(rng, cap, 32) for _ in range(batch)]
    prefix = [0 if rng.random() < 0.3 else _length(rng, 600, 64) for _ in range(batch)]
    return dict(d=d, hq=hq, hkv=hkv, qo=qo, prefix=prefix, causal=bool(rng.random() < 0.75),
                bs=int(rng.choice(BLOCK_SIZES)))


def _draw_decode(seed: int):
    rng = np.random.default_rng(seed)
    d = int(rng.choice(HEAD_DIMS))
    hq, hkv = _heads(rng)
    batch = int(rng.integers(1, 9))
    lens = [_length(rng, 3000, 512) for _ in range(batch)]
    pt = int(rng.choice([0, -1, 32, 64, 96, 256, 512, 1024]))
    fp8 = bool(rng.random() < 0.35)
    window = 0 if fp8 or rng.random() < 0.5 else int(rng.integers(1, 2500))
    scales = (float(rng.choice([0.02, 0.125, 1.0])), float(rng.choice([0.03, 0.25, 1.0])))
    return dict(d=d, hq=hq, hkv=hkv, lens=lens, bs=int(rng.choice(BLOCK_SIZES)), pt=pt, fp8=fp8,
                window=window, scales=scales)


@pytest.mark.parametrize("seed", range(40))
def test_random_ragged_prefill(seed):
    c = _draw_prefill(7000 + seed)
    # kv = a prefix of cached keys followed by the request's own tokens; a quarter of the requests
    # keep fewer keys than queries (leading rows then see no key under causal masking)
    rng = np.random.default_rng(17000 + seed)
    kv = [p + q if rng.random() < 0.75 else int(rng.integers(0, q + 1)) for p, q in zip(c["prefix"], c["qo"])]
    ri = ragged_prefill_inputs(7000 + seed, num_q_heads=c["hq"], num_kv_heads=c["hkv"], head_dim=c["d"],
                               qo_lens=c["qo"], kv_lens=kv, causal=c["causal"])
    print(f"ragged seed {seed}: D={c['d']} Hq={c['hq']} Hkv={c['hkv']} qo={c['qo']} kv={kv} causal={c['causal']}",
          flush=True)
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, ri.causal, ri.scale)
    out = pkv.ragged_prefill(ri.q.to(DEV), ri.k.to(DEV), ri.v.to(DEV), ri.qo_indptr.to(DEV), ri.kv_indptr.to(DEV),
                             ri.causal, ri.scale, qo_indptr_h=ri.qo_indptr, kv_indptr_h=ri.kv_indptr)
    torch.cuda.synchronize()
    assert_parity(out.cpu(), ref, f"random ragged seed {seed}")


@pytest.mark.parametrize("seed", range(40))
def test_random_paged_prefill(seed):
    c = _draw_prefill(8000 + seed)
    # a pool two blocks larger than the requests use (never empty: the library refuses an empty pool)
    nb = sum((p + q + c["bs"] - 1) // c["bs"] for p, q in zip(c["prefix"], c["qo"])) + 2
    ci = chunked_prefill_inputs(8000 + seed, num_q_heads=c["hq"], num_kv_heads=c["hkv"], head_dim=c["d"],
                                chunk_lens=c["qo"], prefix_lens=c["prefix"], block_size=c["bs"],
                                num_blocks=nb, causal=c["causal"])
    print(f"paged seed {seed}: D={c['d']} Hq={c['hq']} Hkv={c['hkv']} chunk={c['qo']} prefix={c['prefix']} "
          f"BS={c['bs']} causal={c['causal']}", flush=True)
    kc, vc = ci.k_cache.to(DEV), ci.v_cache.to(DEV)
    pkv.reshape_and_cache(ci.k_new.to(DEV), ci.v_new.to(DEV), kc, vc, ci.slot_mapping.to(DEV))
    out = pkv.paged_prefill(ci.q.to(DEV), kc, vc, ci.block_tables.to(DEV), ci.qo_indptr.to(DEV),
                            ci.kv_lens.to(DEV), ci.causal, ci.scale, qo_indptr_h=ci.qo_indptr, kv_lens_h=ci.kv_lens)
    torch.cuda.synchronize()
    ek, ev = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    assert np.array_equal(kc.cpu().view(torch.int16).numpy(), ek)
    assert np.array_equal(vc.cpu().view(torch.int16).numpy(), ev)
    ref = oracle.paged_prefill(ci.q, torch.from_numpy(ek).view(torch.bfloat16), torch.from_numpy(ev).view(torch.bfloat16),
                               ci.block_tables, ci.qo_indptr, ci.kv_lens, ci.causal, ci.scale)
    assert_parity(out.cpu(), ref, f"random paged seed {seed}")


@pytest.mark.parametrize("seed", range(48))
def test_random_decode(seed):
    c = _draw_decode(9000 + seed)
    nb = sum((L + c["bs"] - 1) // c["bs"] for L in c["lens"]) + 2
    di = paged_decode_inputs(9000 + seed, num_q_heads=c["hq"], num_kv_heads=c["hkv"], head_dim=c["d"],
                             seq_lens=c["lens"], block_size=c["bs"], num_blocks=nb)
    print(f"decode seed {seed}: D={c['d']} Hq={c['hq']} Hkv={c['hkv']} lens={c['lens']} BS={c['bs']} "
          f"pt={c['pt']} fp8={c['fp8']} window={c['window']}", flush=True)
    B, Hq = di.q.shape[0], di.q.shape[1]
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    kw = dict(max_seq_len=di.max_seq_len, partition_tokens=c["pt"], lse=lse)
    if c["fp8"]:
        ks, vs = c["scales"]
        kq, vq = oracle.quantize(di.k_cache, ks), oracle.quantize(di.v_cache, vs)
        ref, rlse = oracle.paged_decode_fp8(di.q, kq, vq, di.block_tables, di.seq_lens, di.scale, ks, vs,
                                            return_lse=True)
        kc = torch.from_numpy(np.ascontiguousarray(kq)).view(torch.uint8).to(DEV)
        vc = torch.from_numpy(np.ascontiguousarray(vq)).view(torch.uint8).to(DEV)
        kw.update(k_scale=ks, v_scale=vs)
    else:
        if c["window"]:
            ref, rlse = oracle.paged_decode_window(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens,
                                                   di.scale, c["window"], return_lse=True)
            kw.update(window=c["window"])
        else:
            ref, rlse = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale,
                                            return_lse=True)
        kc, vc = di.k_cache.to(DEV), di.v_cache.to(DEV)
    out = pkv.paged_attn_decode(di.q.to(DEV), kc, vc, di.block_tables.to(DEV), di.seq_lens.to(DEV), di.scale, **kw)
    torch.cuda.synchronize()
    assert_parity(out.cpu(), ref, f"random decode seed {seed}")
    got = lse.cpu().double().numpy()
    empty = ~np.isfinite(rlse)
    assert np.array_equal(np.isneginf(got), empty), "an empty sequence's lse must be -inf, others finite"
    np.testing.assert_allclose(got[~empty], rlse[~empty], rtol=0, atol=2e-3)


@pytest.mark.parametrize("seed", range(16))
def test_random_streamed_decode(seed):
    """Decode streamed over tiles of resident blocks, the tiles in a drawn order, against the oracle's
    streamed fold (itself pinned to one-pass decode)."""
    rng = np.random.default_rng(11000 + seed)
    d = int(rng.choice(HEAD_DIMS))
    hq, hkv = _heads(rng)
    bs = int(rng.choice(BLOCK_SIZES))
    lens = [_length(rng, 2500, 256) for _ in range(int(rng.integers(1, 7)))]
    cap = int(rng.choice([1, 2, 3, 8, 64]))
    nb = sum((L + bs - 1) // bs for L in lens) + 2
    di = paged_decode_inputs(11000 + seed, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=lens,
                             block_size=bs, num_blocks=nb)
    tiles = _tiles(di.block_tables, lens, bs, cap)
    order = rng.permutation(len(tiles))
    tiles = [tiles[i] for i in order]
    print(f"streamed seed {seed}: D={d} Hq={hq} Hkv={hkv} lens={lens} BS={bs} cap={cap} tiles={len(tiles)}",
          flush=True)
    ref, rlse = oracle.streamed_decode(di.q, di.k_cache, di.v_cache, tiles, di.scale, return_lse=True)
    sd = pkv.StreamedDecode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.scale)
    sd.begin()
    for t_tab, t_len in tiles:
        sd.step(t_tab.to(DEV), t_len.to(DEV))
    lse = torch.empty(len(lens), hq, dtype=torch.float32, device=DEV)
    out = sd.finalize(lse=lse)
    torch.cuda.synchronize()
    assert_parity(out.cpu(), ref, f"random streamed seed {seed}")
    got = lse.cpu().double().numpy()
    empty = ~np.isfinite(rlse)
    assert np.array_equal(np.isneginf(got), empty)
    np.testing.assert_allclose(got[~empty], rlse[~empty], rtol=0, atol=2e-3)


@pytest.mark.parametrize("seed", range(16))
def test_random_scatter(seed):
    """reshape_and_cache into a bf16 or an fp8 cache, bit-exact: drawn head counts, head dims
    (including ones off the power-of-two path), block sizes (including non-powers of two), and slot
    maps with skipped (negative or past the pool) entries."""
    rng = np.random.default_rng(12000 + seed)
    fp8 = bool(rng.random() < 0.5)
    d = int(rng.choice([16, 32, 48, 64, 80, 128, 256] if fp8 else [8, 24, 64, 72, 128, 256]))
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    bs = int(rng.choice([1, 5, 12, 16, 32, 100, 256]))
    nb = int(rng.integers(1, 40))
    T = int(rng.integers(0, min(nb * bs, 300) + 1))
    slots = rng.choice(nb * bs, size=T, replace=False).astype(np.int64)
    skip = rng.random(T) < 0.1
    slots[skip] = np.where(rng.random(int(skip.sum())) < 0.5, -1, nb * bs + rng.integers(0, 50, int(skip.sum())))
    slots = torch.from_numpy(slots)
    # the library skips slots past the pool like negative ones (a caller error it tolerates); the
    # oracle refuses them, so it sees those entries as skipped
    ref_slots = torch.where(slots >= nb * bs, torch.full_like(slots, -1), slots)
    g = torch.Generator().manual_seed(12000 + seed)
    k = (torch.randn(T, hkv, d, generator=g) * 4).to(torch.bfloat16)
    v = (torch.randn(T, hkv, d, generator=g) * 4).to(torch.bfloat16)
    print(f"scatter seed {seed}: fp8={fp8} T={T} Hkv={hkv} D={d} BS={bs} NB={nb} skipped={int(skip.sum())}",
          flush=True)
    if fp8:
        kc0 = torch.randint(0, 256, (nb, hkv, bs, d), generator=g, dtype=torch.int32).to(torch.uint8)
        vc0 = torch.randint(0, 256, (nb, hkv, bs, d), generator=g, dtype=torch.int32).to(torch.uint8)
        ks, vs = float(rng.choice([0.01, 0.5, 2.0])), float(rng.choice([0.02, 1.0, 3.0]))
        ek, ev = oracle.reshape_and_cache_fp8(k, v, kc0, vc0, ref_slots, ks, vs)
        kc, vc = kc0.to(DEV), vc0.to(DEV)
        pkv.reshape_and_cache_fp8(k.to(DEV), v.to(DEV), kc, vc, slots.to(DEV), ks, vs)
        torch.cuda.synchronize()
        assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)
    else:
        bits = lambda: torch.randint(-32768, 32768, (nb, hkv, bs, d), generator=g,
                                     dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
        kc0, vc0 = bits(), bits()
        ek, ev = oracle.reshape_and_cache(k, v, kc0, vc0, ref_slots)
        kc, vc = kc0.to(DEV), vc0.to(DEV)
        pkv.reshape_and_cache(k.to(DEV), v.to(DEV), kc, vc, slots.to(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(kc.cpu().view(torch.int16).numpy(), ek)
        assert np.array_equal(vc.cpu().view(torch.int16).numpy(), ev)
