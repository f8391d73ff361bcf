"""Pins for the fp64 oracle: hand-derived golden values, an independent brute-force formulation,
closed forms and invariants. CPU only. Each test names what it pins."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from workloads import chunked_prefill_inputs, paged_decode_inputs, ragged_prefill_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    if isinstance(x, list):
        return [_num(v) for v in x]
    if isinstance(x, str):
        return float(x)  # "nan", "-inf"
    return float(x)


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        fx = json.load(f)
    assert fx["citation"] and fx["derivation"]
    return fx


# ------------------------------------------------------------------------------------------------
# Golden fixtures (values derived by hand from the definitions the fixtures cite)
# ------------------------------------------------------------------------------------------------
def test_golden_decode_gqa_shuffled_table():
    fx = load("decode_gqa_shuffled.json")
    kc, vc = np.array(_num(fx["k_cache"])), np.array(_num(fx["v_cache"]))
    out, lse = oracle.paged_decode(np.array(fx["q"]), kc, vc, np.array(fx["block_tables"]),
                                   np.array(fx["seq_lens"]), fx["scale"], return_lse=True)
    np.testing.assert_allclose(out, np.array(fx["expected_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(fx["expected_lse"]), rtol=0, atol=1e-12)


def test_golden_decode_pairs_match():
    fx = load("decode_gqa_shuffled.json")
    kc, vc = np.array(_num(fx["k_cache"])), np.array(_num(fx["v_cache"]))
    got = oracle.paged_decode_pairs(np.array(fx["q"]), kc, vc, np.array(fx["block_tables"]),
                                    np.array(fx["seq_lens"]), fx["scale"], [(0, h) for h in range(4)])
    np.testing.assert_allclose(got, np.array(fx["expected_out"])[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_golden_prefill_bottom_right(causal):
    fx = load("prefill_bottom_right.json")
    args = (np.array(fx["q"]), np.array(fx["k"]), np.array(fx["v"]), np.array(fx["qo_indptr"]),
            np.array(fx["kv_indptr"]), causal, fx["scale"])
    exp = np.array(fx["expected_causal" if causal else "expected_noncausal"])
    np.testing.assert_allclose(oracle.ragged_prefill(*args), exp, rtol=0, atol=1e-12)
    rows = [(t, 0) for t in range(3)]
    np.testing.assert_allclose(oracle.ragged_prefill_rows(*args, rows), exp[:, 0], rtol=0, atol=1e-12)


def test_golden_lse_merge():
    fx = load("lse_merge.json")
    out, lse = oracle.merge_partials(np.array(fx["o"]), np.array(_num(fx["m"])), np.array(fx["l"]))
    np.testing.assert_allclose(out, np.array(fx["expected_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(_num(fx["expected_lse"])), rtol=0, atol=1e-12)


def test_golden_scatter():
    fx = load("scatter.json")
    i16 = lambda x: np.array(x, dtype=np.int16)
    kc, vc = oracle.reshape_and_cache(i16(fx["k"]), i16(fx["v"]), i16(fx["k_cache"]), i16(fx["v_cache"]),
                                      np.array(fx["slot_mapping"]))
    assert np.array_equal(kc, i16(fx["expected_k_cache"]))
    assert np.array_equal(vc, i16(fx["expected_v_cache"]))


def test_golden_paged_prefill_prefix_offset():
    fx = load("paged_prefill_prefix.json")
    args = (np.array(fx["q"]), np.array(_num(fx["k_cache"])), np.array(_num(fx["v_cache"])),
            np.array(fx["block_tables"]), np.array(fx["qo_indptr"]), np.array(fx["kv_lens"]), True,
            fx["scale"])
    exp = np.array(fx["expected_causal"])
    np.testing.assert_allclose(oracle.paged_prefill(*args), exp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.paged_prefill_rows(*args, [(0, 0), (1, 0)]), exp[:, 0], atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Brute force: dense fp64 attention from torch's SDPA with an explicit mask, on K/V that never went
# through a block table. The paged cache is built by the test from the dense rows.
# ------------------------------------------------------------------------------------------------
def _sdpa(qrows, K, V, scale, mask):
    """qrows [H, n, D], K/V [H, m, D] float64; mask [n, m] bool (True = visible)."""
    return torch.nn.functional.scaled_dot_product_attention(
        qrows, K, V, attn_mask=mask, scale=scale).numpy()


@pytest.mark.parametrize("lens,bs,hq,hkv,d,seed", [
    ([1], 16, 1, 1, 8, 0), ([17, 5, 64], 16, 4, 2, 16, 1), ([33, 2], 4, 6, 3, 8, 2),
    ([64, 63, 1], 8, 8, 1, 32, 3),
])
def test_decode_matches_dense_sdpa(lens, bs, hq, hkv, d, seed):
    rng = np.random.default_rng(seed)
    B = len(lens)
    need = [(L + bs - 1) // bs for L in lens]
    nb = sum(need) + 3
    perm = rng.permutation(nb)
    tables = np.full((B, max(need)), -1)
    dense_k = [rng.standard_normal((L, hkv, d)) for L in lens]
    dense_v = [rng.standard_normal((L, hkv, d)) for L in lens]
    kc = np.full((nb, hkv, bs, d), np.nan)
    vc = np.full((nb, hkv, bs, d), np.nan)
    pos = 0
    for b, L in enumerate(lens):
        blocks = perm[pos:pos + need[b]]
        pos += need[b]
        tables[b, :need[b]] = blocks
        for t in range(L):
            kc[blocks[t // bs], :, t % bs] = dense_k[b][t]
            vc[blocks[t // bs], :, t % bs] = dense_v[b][t]
    q = rng.standard_normal((B, hq, d))
    scale = 0.7 / math.sqrt(d)
    got = oracle.paged_decode(q, kc, vc, tables, np.array(lens), scale)
    G = hq // hkv
    for b, L in enumerate(lens):
        Kd = torch.from_numpy(dense_k[b]).permute(1, 0, 2).repeat_interleave(G, 0)
        Vd = torch.from_numpy(dense_v[b]).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = _sdpa(torch.from_numpy(q[b])[:, None, :], Kd, Vd, scale, torch.ones(1, L, dtype=torch.bool))
        np.testing.assert_allclose(got[b], ref[:, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("qo,kv,hq,hkv,d,causal,seed", [
    ([5, 9], [5, 9], 4, 2, 16, True, 0), ([3, 1, 7], [10, 1, 7], 2, 1, 8, True, 1),
    ([4, 6], [7, 6], 6, 2, 8, False, 2), ([16], [40], 8, 8, 32, True, 3),
])
def test_ragged_prefill_matches_dense_sdpa(qo, kv, hq, hkv, d, causal, seed):
    rng = np.random.default_rng(seed)
    qi = np.concatenate([[0], np.cumsum(qo)])
    ki = np.concatenate([[0], np.cumsum(kv)])
    q = rng.standard_normal((qi[-1], hq, d))
    k = rng.standard_normal((ki[-1], hkv, d))
    v = rng.standard_normal((ki[-1], hkv, d))
    scale = 1.3 / math.sqrt(d)
    got = oracle.ragged_prefill(q, k, v, qi, ki, causal, scale)
    G = hq // hkv
    for b in range(len(qo)):
        nq, nk = qo[b], kv[b]
        mask = torch.ones(nq, nk, dtype=torch.bool)
        if causal:  # row i sits at absolute position nk - nq + i
            for i in range(nq):
                mask[i, nk - nq + i + 1:] = False
        Q = torch.from_numpy(q[qi[b]:qi[b + 1]]).permute(1, 0, 2)
        Kd = torch.from_numpy(k[ki[b]:ki[b + 1]]).permute(1, 0, 2).repeat_interleave(G, 0)
        Vd = torch.from_numpy(v[ki[b]:ki[b + 1]]).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = _sdpa(Q, Kd, Vd, scale, mask)
        np.testing.assert_allclose(got[qi[b]:qi[b + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_paged_prefill_matches_dense_sdpa():
    rng = np.random.default_rng(7)
    bs, hq, hkv, d = 4, 4, 2, 8
    P, C = [5, 0, 12], [3, 6, 1]
    kvl = [p + c for p, c in zip(P, C)]
    need = [(L + bs - 1) // bs for L in kvl]
    nb = sum(need) + 2
    perm = rng.permutation(nb)
    tables = np.full((3, max(need)), -1)
    kc = np.full((nb, hkv, bs, d), np.nan)
    vc = np.full((nb, hkv, bs, d), np.nan)
    dense = []
    pos = 0
    for b, L in enumerate(kvl):
        blocks = perm[pos:pos + need[b]]
        pos += need[b]
        tables[b, :need[b]] = blocks
        Kd, Vd = rng.standard_normal((L, hkv, d)), rng.standard_normal((L, hkv, d))
        dense.append((Kd, Vd))
        for t in range(L):
            kc[blocks[t // bs], :, t % bs] = Kd[t]
            vc[blocks[t // bs], :, t % bs] = Vd[t]
    qi = np.concatenate([[0], np.cumsum(C)])
    q = rng.standard_normal((qi[-1], hq, d))
    scale = 0.25
    got = oracle.paged_prefill(q, kc, vc, tables, qi, np.array(kvl), True, scale)
    for b in range(3):
        mask = torch.zeros(C[b], kvl[b], dtype=torch.bool)
        for i in range(C[b]):
            mask[i, :P[b] + i + 1] = True
        Q = torch.from_numpy(q[qi[b]:qi[b + 1]]).permute(1, 0, 2)
        Kd = torch.from_numpy(dense[b][0]).permute(1, 0, 2).repeat_interleave(2, 0)
        Vd = torch.from_numpy(dense[b][1]).permute(1, 0, 2).repeat_interleave(2, 0)
        if C[b]:
            ref = _sdpa(Q, Kd, Vd, scale, mask)
            np.testing.assert_allclose(got[qi[b]:qi[b + 1]], ref.transpose(1, 0, 2), rtol=0, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# Closed forms
# ------------------------------------------------------------------------------------------------
def test_single_key_returns_v_exactly():
    di = paged_decode_inputs(11, num_q_heads=4, num_kv_heads=2, head_dim=64, seq_lens=[1, 1, 1])
    out = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    for b in range(3):
        blk = int(di.block_tables[b, 0])
        for h in range(4):
            assert np.array_equal(out[b, h], di.v_cache[blk, h // 2, 0].double().numpy())


def test_identical_keys_and_zero_scale_give_mean_of_v():
    di = paged_decode_inputs(12, num_q_heads=2, num_kv_heads=1, head_dim=16, seq_lens=[50])
    blocks = di.block_tables[0, :4]
    kc = di.k_cache.clone()
    kc[blocks] = di.k_cache[blocks[0], :, 0:1, :]  # every valid key equal (slack keys too)
    Vd = oracle.gather_tokens(di.v_cache, di.block_tables[0], 50, 0, 16)
    for cache, scale in ((kc, di.scale), (di.k_cache, 0.0)):
        out = oracle.paged_decode(di.q, cache, di.v_cache, di.block_tables, di.seq_lens, scale)
        np.testing.assert_allclose(out[0], np.broadcast_to(Vd.mean(0), (2, 16)), rtol=0, atol=1e-12)


def test_position_probe_decode_ragged_paged():
    """K = 0 and V[t, 0] = t: the output's first column is the mean visible key position."""
    bs, d = 16, 8
    # decode: mean of 0..L-1
    lens = [1, 16, 17, 100]
    di = paged_decode_inputs(13, num_q_heads=2, num_kv_heads=1, head_dim=d, seq_lens=lens)
    kc = torch.zeros_like(di.k_cache)
    vc = torch.zeros_like(di.v_cache)
    for b, L in enumerate(lens):
        for t in range(L):
            vc[int(di.block_tables[b, t // bs]), 0, t % bs, 0] = float(t)
    out = oracle.paged_decode(di.q, kc, vc, di.block_tables, di.seq_lens, di.scale)
    for b, L in enumerate(lens):
        np.testing.assert_allclose(out[b, :, 0], (L - 1) / 2, atol=1e-12)
    # ragged causal, qo == kv: row i -> i/2; qo < kv: row i -> (kv - qo + i)/2
    qo, kv = [5, 9], [5, 12]
    ri = ragged_prefill_inputs(14, num_q_heads=2, num_kv_heads=1, head_dim=d, qo_lens=qo, kv_lens=kv)
    k = torch.zeros_like(ri.k)
    v = torch.zeros_like(ri.v)
    for b in range(2):
        for j in range(kv[b]):
            v[int(ri.kv_indptr[b]) + j, 0, 0] = float(j)
    out = oracle.ragged_prefill(ri.q, k, v, ri.qo_indptr, ri.kv_indptr, True, ri.scale)
    for b in range(2):
        for i in range(qo[b]):
            np.testing.assert_allclose(out[int(ri.qo_indptr[b]) + i, :, 0], (kv[b] - qo[b] + i) / 2, atol=1e-12)
    # paged prefill: row i of the chunk -> (P + i)/2
    ci = chunked_prefill_inputs(15, num_q_heads=2, num_kv_heads=1, head_dim=d, chunk_lens=[3, 20],
                                prefix_lens=[0, 37])
    kc = torch.zeros_like(ci.k_cache)
    vc = torch.zeros_like(ci.v_cache)
    kvl = ci.kv_lens.tolist()
    for b in range(2):
        for t in range(kvl[b]):
            vc[int(ci.block_tables[b, t // bs]), 0, t % bs, 0] = float(t)
    out = oracle.paged_prefill(ci.q, kc, vc, ci.block_tables, ci.qo_indptr, ci.kv_lens, True, ci.scale)
    for b, P in enumerate([0, 37]):
        for i in range(int(ci.qo_indptr[b + 1] - ci.qo_indptr[b])):
            np.testing.assert_allclose(out[int(ci.qo_indptr[b]) + i, :, 0], (P + i) / 2, atol=1e-12)


def test_causal_row_zero_returns_first_v():
    ri = ragged_prefill_inputs(16, num_q_heads=4, num_kv_heads=2, head_dim=16, qo_lens=[4, 1, 9])
    out = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, True, ri.scale)
    for b in range(3):
        r = int(ri.qo_indptr[b])
        for h in range(4):
            assert np.array_equal(out[r, h], ri.v[r, h // 2].double().numpy())


def test_gqa_constant_value_per_kv_head():
    di = paged_decode_inputs(17, num_q_heads=8, num_kv_heads=4, head_dim=16, seq_lens=[30, 7])
    vc = di.v_cache.clone()
    for kh in range(4):
        vc[:, kh] = float(kh + 1)
    out = oracle.paged_decode(di.q, di.k_cache, vc, di.block_tables, di.seq_lens, di.scale)
    for h in range(8):
        np.testing.assert_allclose(out[:, h], h // 2 + 1, atol=1e-12)


def test_zero_length_sequence_gives_zeros():
    di = paged_decode_inputs(18, num_q_heads=2, num_kv_heads=1, head_dim=16, seq_lens=[0, 5, 0])
    out = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    assert np.all(out[0] == 0) and np.all(out[2] == 0) and np.all(np.isfinite(out[1]))


def test_causal_row_without_keys_gives_zeros():
    ri = ragged_prefill_inputs(19, num_q_heads=1, num_kv_heads=1, head_dim=8, qo_lens=[4], kv_lens=[2])
    out = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, True, ri.scale)
    # rows 0, 1 sit at positions -2, -1: no key visible
    assert np.all(out[:2] == 0) and np.all(np.isfinite(out[2:])) and np.any(out[2:] != 0)


# ------------------------------------------------------------------------------------------------
# Invariants
# ------------------------------------------------------------------------------------------------
def _shuffle_pool(di, seed):
    g = torch.Generator().manual_seed(seed)
    nb = di.k_cache.shape[0]
    perm = torch.randperm(nb, generator=g)          # new position of old block i is perm[i]
    kc = torch.empty_like(di.k_cache)
    vc = torch.empty_like(di.v_cache)
    kc[perm] = di.k_cache
    vc[perm] = di.v_cache
    tables = di.block_tables.clone()
    live = tables >= 0
    tables[live] = perm[tables[live].long()].to(torch.int32)
    return kc, vc, tables


def test_block_shuffle_leaves_output_bit_identical():
    di = paged_decode_inputs(20, num_q_heads=8, num_kv_heads=2, head_dim=32, len_range=(1, 300), batch=5)
    base = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    kc, vc, tables = _shuffle_pool(di, 99)
    assert not torch.equal(tables, di.block_tables)
    out = oracle.paged_decode(di.q, kc, vc, tables, di.seq_lens, di.scale)
    assert np.array_equal(base, out)


@pytest.mark.parametrize("part", [16, 64, 512, 4096])
def test_split_merge_equals_unsplit(part):
    di = paged_decode_inputs(21, num_q_heads=4, num_kv_heads=2, head_dim=32, seq_lens=[1, 513, 1500, 0, 64])
    full, lse = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale,
                                    return_lse=True)
    o, m, l = oracle.decode_partials(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale, part)
    merged, mlse = oracle.merge_partials(o, m, l)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mlse[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=0, atol=1e-12)
    assert np.all(np.isneginf(mlse[~np.isfinite(lse)]))


def test_merge_is_order_invariant_and_idempotent_on_one_partition():
    di = paged_decode_inputs(22, num_q_heads=4, num_kv_heads=1, head_dim=16, seq_lens=[2000, 700])
    o, m, l = oracle.decode_partials(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale, 256)
    ref, _ = oracle.merge_partials(o, m, l)
    perm = np.random.default_rng(0).permutation(o.shape[2])
    out, _ = oracle.merge_partials(o[:, :, perm], m[:, :, perm], l[:, :, perm])
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)
    one, lse1 = oracle.merge_partials(o[:, :, :1], m[:, :, :1], l[:, :, :1])
    np.testing.assert_allclose(one, o[:, :, 0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse1, m[:, :, 0] + np.log(l[:, :, 0]), rtol=0, atol=1e-13)


def test_scatter_then_gather_round_trip():
    ci = chunked_prefill_inputs(23, num_q_heads=4, num_kv_heads=2, head_dim=16, chunk_lens=[5, 40, 1],
                                prefix_lens=[3, 0, 31])
    before_k = ci.k_cache.view(torch.int16).numpy()
    kc, vc = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    bs = ci.block_size
    slots = ci.slot_mapping.numpy()
    kn = ci.k_new.view(torch.int16).numpy()
    vn = ci.v_new.view(torch.int16).numpy()
    for t, s in enumerate(slots):
        assert np.array_equal(kc[s // bs, :, s % bs], kn[t]) and np.array_equal(vc[s // bs, :, s % bs], vn[t])
    touched = np.zeros(kc.shape[0] * bs, dtype=bool)
    touched[slots] = True
    touched = touched.reshape(kc.shape[0], bs)
    for blk in range(kc.shape[0]):
        for off in range(bs):
            if not touched[blk, off]:
                assert np.array_equal(kc[blk, :, off], before_k[blk, :, off])


def test_scatter_rejects_duplicates_and_out_of_range():
    ci = chunked_prefill_inputs(24, num_q_heads=2, num_kv_heads=1, head_dim=8, chunk_lens=[4], prefix_lens=[0])
    bad = ci.slot_mapping.clone()
    bad[1] = bad[0]
    with pytest.raises(ValueError):
        oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, bad)
    bad = ci.slot_mapping.clone()
    bad[0] = ci.k_cache.shape[0] * 16
    with pytest.raises(IndexError):
        oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, bad)


def test_chunked_paged_prefill_equals_ragged_over_prefix_plus_chunk():
    """After the scatter, prefill through the table equals ragged prefill over [prefix; chunk] rows."""
    ci = chunked_prefill_inputs(25, num_q_heads=4, num_kv_heads=2, head_dim=16, chunk_lens=[7, 1, 33],
                                prefix_lens=[20, 0, 16])
    kc, vc = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    kc = torch.from_numpy(kc).view(torch.bfloat16)
    vc = torch.from_numpy(vc).view(torch.bfloat16)
    got = oracle.paged_prefill(ci.q, kc, vc, ci.block_tables, ci.qo_indptr, ci.kv_lens, True, ci.scale)
    # contiguous K/V per request: the dense rows the test knows independently of any table read
    ks, vs, kvi = [], [], [0]
    P = ci.prefix_lens.tolist()
    for b in range(3):
        for t in range(P[b]):
            blk = int(ci.block_tables[b, t // 16])
            ks.append(ci.k_cache[blk, :, t % 16])
            vs.append(ci.v_cache[blk, :, t % 16])
        c0, c1 = int(ci.qo_indptr[b]), int(ci.qo_indptr[b + 1])
        ks.extend(ci.k_new[c0:c1])
        vs.extend(ci.v_new[c0:c1])
        kvi.append(kvi[-1] + P[b] + (c1 - c0))
    k = torch.stack(ks)
    v = torch.stack(vs)
    ref = oracle.ragged_prefill(ci.q, k, v, ci.qo_indptr, np.array(kvi), True, ci.scale)
    assert np.array_equal(got, ref)


def test_row_sampled_variants_equal_full():
    ri = ragged_prefill_inputs(26, num_q_heads=4, num_kv_heads=2, head_dim=16, qo_lens=[9, 3], kv_lens=[12, 3])
    full = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, True, ri.scale)
    rows = [(0, 0), (8, 3), (9, 1), (11, 2)]
    got = oracle.ragged_prefill_rows(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, True, ri.scale, rows)
    for n, (t, h) in enumerate(rows):
        np.testing.assert_allclose(got[n], full[t, h], rtol=0, atol=1e-14)
    di = paged_decode_inputs(27, num_q_heads=4, num_kv_heads=2, head_dim=16, seq_lens=[19, 0, 40])
    full = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    pairs = [(0, 1), (1, 3), (2, 2)]
    got = oracle.paged_decode_pairs(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale, pairs)
    for n, (b, h) in enumerate(pairs):
        np.testing.assert_allclose(got[n], full[b, h], rtol=0, atol=1e-14)


# ------------------------------------------------------------------------------------------------
# Table validation rules
# ------------------------------------------------------------------------------------------------
def test_validate_block_tables_rules():
    S = oracle.STATUS
    t = np.array([[3, 1, -1], [0, -1, -1]])
    assert oracle.validate_block_tables(t, [32, 16], 16, 4) == S["OK"]
    assert oracle.validate_block_tables(t, [1, 0], 16, 4) == S["OK"]
    assert oracle.validate_block_tables(t, [33, 16], 16, 4) == S["BAD_TABLE"]        # reads the -1 pad
    assert oracle.validate_block_tables(t, [16, 17], 16, 4) == S["BAD_TABLE"]        # reads the -1 pad
    assert oracle.validate_block_tables(t, [32, 16], 16, 3) == S["BAD_TABLE"]        # block 3 missing
    assert oracle.validate_block_tables(t, [64, 16], 16, 4) == S["BAD_TABLE"]        # 4 blocks > width 3
    assert oracle.validate_block_tables(t, [-1, 16], 16, 4) == S["INVALID_ARGUMENT"]
    assert oracle.validate_block_tables(t, [1, 1], 0, 4) == S["INVALID_ARGUMENT"]


# ------------------------------------------------------------------------------------------------
# The pins have teeth: plausible mistakes planted in the oracle (on the CPU) must fail a pin.
# ------------------------------------------------------------------------------------------------
def test_planted_gqa_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(A, "kv_head_of", lambda h, group: h % 2)  # interleaved instead of grouped
    with pytest.raises(AssertionError):
        test_golden_decode_gqa_shuffled_table()


def test_planted_causal_alignment_mistake_is_caught(monkeypatch):
    real = A.key_visible
    monkeypatch.setattr(A, "key_visible", lambda i, j, nq, nk, c: real(i, j, nk, nk, c))  # top-left
    with pytest.raises(AssertionError):
        test_golden_prefill_bottom_right(True)
    with pytest.raises(AssertionError):
        test_golden_paged_prefill_prefix_offset()


def test_planted_gather_mistake_is_caught(monkeypatch):
    real = A.gather_tokens

    def wrong(cache, row, length, kh, bs):  # reads the table in the wrong order
        return real(cache, np.asarray(row)[::-1].copy(), length, kh, bs)
    monkeypatch.setattr(A, "gather_tokens", wrong)
    with pytest.raises(AssertionError):
        test_golden_decode_gqa_shuffled_table()


# ----------------------------------------------------------------------------------------------
# Block management: copy_blocks / swap_blocks
# ----------------------------------------------------------------------------------------------
def _golden_blocks():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "copy_blocks.json")) as f:
        return json.load(f)


def test_golden_copy_and_swap_blocks():
    g = _golden_blocks()
    kc = np.array(g["k_cache"], dtype=np.int16)
    vc = np.array(g["v_cache"], dtype=np.int16)
    (k2,), (v2,) = oracle.copy_blocks([kc], [vc], g["mapping"])
    np.testing.assert_array_equal(k2, np.array(g["k_after"], dtype=np.int16))
    np.testing.assert_array_equal(v2, np.array(g["v_after"], dtype=np.int16))
    out = oracle.swap_blocks(kc, np.array(g["swap_dst"], dtype=np.int16), g["swap_mapping"])
    np.testing.assert_array_equal(out, np.array(g["swap_after"], dtype=np.int16))


def test_copy_blocks_invariants():
    rng = np.random.default_rng(7)
    layers = [rng.integers(-30000, 30000, size=(12, 2, 4, 8), dtype=np.int16) for _ in range(3)]
    vals = [rng.integers(-30000, 30000, size=(12, 2, 4, 8), dtype=np.int16) for _ in range(3)]
    m = np.array([[1, 5], [2, 7], [9, 0]])
    ks, vs = oracle.copy_blocks(layers, vals, m)
    for l in range(3):
        for s, d in m:
            np.testing.assert_array_equal(ks[l][d], layers[l][s])
            np.testing.assert_array_equal(vs[l][d], vals[l][s])
        untouched = [b for b in range(12) if b not in m[:, 1]]
        np.testing.assert_array_equal(ks[l][untouched], layers[l][untouched])
    # the pairs act at once: any order of the rows gives the same caches
    ks2, _ = oracle.copy_blocks(layers, vals, m[::-1])
    for a, b in zip(ks, ks2):
        np.testing.assert_array_equal(a, b)
    # out-of-range pairs are skipped, identity pairs change nothing
    ks3, _ = oracle.copy_blocks(layers, vals, [[3, 3], [40, 1], [-1, 2], [1, 99]])
    for a, b in zip(ks3, layers):
        np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.copy_blocks(layers, vals, [[1, 2], [3, 2]])
    with pytest.raises(ValueError):
        oracle.copy_blocks(layers, vals, [[1, 2], [2, 3]])


def test_swap_blocks_round_trip():
    rng = np.random.default_rng(8)
    dev = rng.integers(-30000, 30000, size=(10, 2, 16, 8), dtype=np.int16)
    host = np.zeros((6, 2, 16, 8), dtype=np.int16)
    out_map = np.array([[7, 0], [2, 1], [3, 2], [4, 3]])
    host2 = oracle.swap_blocks(dev, host, out_map)
    back = oracle.swap_blocks(host2, np.zeros_like(dev), out_map[:, ::-1])
    np.testing.assert_array_equal(back[out_map[:, 0]], dev[out_map[:, 0]])
    np.testing.assert_array_equal(host2[4:], host[4:])
    with pytest.raises(IndexError):
        oracle.swap_blocks(dev, host, [[10, 0]])


def test_planted_copy_direction_mistake_is_caught(monkeypatch):
    g = _golden_blocks()
    kc = np.array(g["k_cache"], dtype=np.int16)
    vc = np.array(g["v_cache"], dtype=np.int16)
    real = oracle.blocks._pairs
    monkeypatch.setattr(oracle.blocks, "_pairs", lambda m: real(m)[:, ::-1])
    (k2,), _ = oracle.copy_blocks([kc], [vc], g["mapping"])
    assert not np.array_equal(k2, np.array(g["k_after"], dtype=np.int16))


# ----------------------------------------------------------------------------------------------
# FP8 (e4m3) cache: the format's definition pinned by its special values, ties and error bound
# ----------------------------------------------------------------------------------------------
def test_e4m3_special_values():
    v = oracle.e4m3_value
    assert v(0x38) == 1.0 and v(0xB8) == -1.0
    assert v(0x7E) == 448.0 and v(0xFE) == -448.0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9 and v(0x08) == 2.0 ** -6
    assert v(0x00) == 0.0 and np.signbit(v(0x80))
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert v(0x3F) == 1.875 and v(0x40) == 2.0
    # exactly 254 finite codes, 126 distinct positive magnitudes
    finite = [c for c in range(256) if not np.isnan(v(c))]
    assert len(finite) == 254


def test_e4m3_round_trip_and_monotonic():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), codes)
    x = np.linspace(-500, 500, 20001, dtype=np.float32)
    dec = oracle.e4m3_decode(oracle.e4m3_encode(x))
    assert np.all(np.diff(dec) >= 0)


def test_e4m3_ties_saturation_and_nan():
    enc = oracle.e4m3_encode
    # midpoints go to the even code, anything off the midpoint to the nearer code
    pos = oracle.e4m3_decode(np.arange(0x7F))
    for c in range(0x7E):
        mid = (pos[c] + pos[c + 1]) / 2
        if np.float32(mid) != mid:
            continue
        want = c if c % 2 == 0 else c + 1
        assert enc(np.float32(mid))[()] == want, hex(c)
        assert enc(np.nextafter(np.float32(mid), np.float32(0)))[()] == c
        assert enc(np.nextafter(np.float32(mid), np.float32(1e9)))[()] == c + 1
    np.testing.assert_array_equal(enc(np.array([448, 449, 1e30, np.inf, -np.inf, -600], dtype=np.float32)),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE])
    np.testing.assert_array_equal(enc(np.array([np.nan, -np.nan], dtype=np.float32)), [0x7F, 0x7F])
    np.testing.assert_array_equal(enc(np.array([-0.0, 0.0], dtype=np.float32)), [0x80, 0x00])


def test_fp8_quantize_error_bound():
    # round to nearest: the error is at most half the spacing of the codes around x
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(50000) * 40).astype(np.float32)
    scale = 0.37
    y = (x / np.float32(scale)).astype(np.float64)
    back = oracle.e4m3_decode(oracle.quantize(x, scale))
    err = np.abs(back - np.clip(y, -448, 448))
    a = np.abs(np.clip(y, -448, 448))
    spacing = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(err <= spacing / 2 + 1e-12)


def test_fp8_decode_equals_bf16_decode_on_exact_values():
    # integer-valued K and V in [-8, 8] are exact in both formats: with unit scales the fp8 path is
    # the bf16 path
    import torch
    g = torch.Generator().manual_seed(3)
    B, Hq, Hkv, D, bs, nb = 2, 4, 2, 64, 16, 12
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    kc = torch.randint(-8, 9, (nb, Hkv, bs, D), generator=g).to(torch.bfloat16)
    vc = torch.randint(-8, 9, (nb, Hkv, bs, D), generator=g).to(torch.bfloat16)
    tables = torch.tensor([[3, 7, 1, 0], [5, 2, 9, 11]], dtype=torch.int32)
    lens = torch.tensor([50, 33], dtype=torch.int32)
    kq, vq = oracle.quantize(kc, 1.0), oracle.quantize(vc, 1.0)
    ref = oracle.paged_decode(q, kc, vc, tables, lens, 0.125)
    got = oracle.paged_decode_fp8(q, kq, vq, tables, lens, 0.125, 1.0, 1.0)
    np.testing.assert_array_equal(ref, got)
    # scales apply to the stored values: k_scale 2 with codes of kc/2 is the same cache
    kq2 = oracle.quantize(kc, 2.0)
    got2 = oracle.paged_decode_fp8(q, kq2, vq, tables, lens, 0.125, 2.0, 1.0)
    np.testing.assert_allclose(ref, got2, rtol=0, atol=1e-12)


def test_fp8_scatter_matches_quantized_bf16_scatter():
    import torch
    g = torch.Generator().manual_seed(4)
    T, Hkv, D, bs, nb = 9, 2, 64, 16, 4
    k = torch.randn(T, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(T, Hkv, D, generator=g).to(torch.bfloat16)
    slots = torch.tensor([0, 17, 5, -1, 63, 40, 41, 2, 30], dtype=torch.int64)
    kc0 = torch.zeros(nb, Hkv, bs, D, dtype=torch.uint8)
    vc0 = torch.zeros(nb, Hkv, bs, D, dtype=torch.uint8)
    kc, vc = oracle.reshape_and_cache_fp8(k, v, kc0, vc0, slots, 0.5, 0.25)
    for t, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        np.testing.assert_array_equal(kc[s // bs, :, s % bs], oracle.quantize(k[t], 0.5))
        np.testing.assert_array_equal(vc[s // bs, :, s % bs], oracle.quantize(v[t], 0.25))
    written = {s for s in slots.tolist() if s >= 0}
    for s in range(nb * bs):
        if s not in written:
            assert not kc[s // bs, :, s % bs].any()


# ----------------------------------------------------------------------------------------------
# Sliding window and streamed (multi-launch) decode attention
# ----------------------------------------------------------------------------------------------
def _small_decode(seed=21, lens=(50, 17, 33, 0), hq=4, hkv=2, d=16):
    import torch
    g = torch.Generator().manual_seed(seed)
    bs, nb = 8, 24
    q = torch.randn(len(lens), hq, d, generator=g, dtype=torch.float64)
    kc = torch.randn(nb, hkv, bs, d, generator=g, dtype=torch.float64)
    vc = torch.randn(nb, hkv, bs, d, generator=g, dtype=torch.float64)
    perm = torch.randperm(nb, generator=g)
    tables = torch.full((len(lens), 8), -1, dtype=torch.int64)
    k = 0
    for b, L in enumerate(lens):
        n = -(-L // bs)
        tables[b, :n] = perm[k:k + n]
        k += n
    return q, kc, vc, tables, torch.tensor(lens), bs


def test_window_matches_sdpa_with_a_window_mask():
    import torch
    q, kc, vc, tables, lens, bs = _small_decode()
    W = 13
    got = oracle.paged_decode_window(q, kc, vc, tables, lens, 0.3, W)
    for b, L in enumerate(lens.tolist()):
        if L == 0:
            assert not got[b].any()
            continue
        t = torch.arange(L)
        blk, off = tables[b, t // bs], t % bs
        for h in range(q.shape[1]):
            kh = h // 2
            K, V = kc[blk, kh, off], vc[blk, kh, off]
            mask = t >= L - W
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[b, h][None, None, None], K[None, None], V[None, None], attn_mask=mask[None, None, None],
                scale=0.3)[0, 0, 0]
            np.testing.assert_allclose(got[b, h], ref.numpy(), rtol=0, atol=1e-12)


def test_window_special_cases():
    q, kc, vc, tables, lens, bs = _small_decode()
    full = oracle.paged_decode(q, kc, vc, tables, lens, 0.3)
    np.testing.assert_array_equal(oracle.paged_decode_window(q, kc, vc, tables, lens, 0.3, 0), full)
    np.testing.assert_array_equal(oracle.paged_decode_window(q, kc, vc, tables, lens, 0.3, 1000), full)
    # a window of one token returns that token's value row exactly
    one = oracle.paged_decode_window(q, kc, vc, tables, lens, 0.3, 1)
    for b, L in enumerate(lens.tolist()):
        if L:
            t = L - 1
            np.testing.assert_array_equal(one[b, 0], vc[tables[b, t // bs], 0, t % bs].numpy())


def test_streamed_tiles_equal_one_pass_in_any_order():
    import torch
    q, kc, vc, tables, lens, bs = _small_decode(lens=(50, 17, 33, 40))
    full, flse = oracle.paged_decode(q, kc, vc, tables, lens, 0.3, return_lse=True)
    # split every table row into tiles of at most 3 blocks; the last block of a sequence's final
    # tile holds only its valid slots
    cap = 3
    tiles = []
    for i in range(0, 8, cap):
        t_tab = torch.full((4, cap), -1, dtype=torch.int64)
        t_len = torch.zeros(4, dtype=torch.int64)
        for b, L in enumerate(lens.tolist()):
            nblk = -(-L // bs)
            blocks = tables[b, i:min(i + cap, nblk)]
            t_tab[b, :len(blocks)] = blocks
            t_len[b] = max(0, min(L - i * bs, cap * bs))
        tiles.append((t_tab, t_len))
    got, glse = oracle.streamed_decode(q, kc, vc, tiles, 0.3, return_lse=True)
    np.testing.assert_allclose(got, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(glse, flse, rtol=0, atol=1e-12)
    got_rev = oracle.streamed_decode(q, kc, vc, tiles[::-1], 0.3)
    np.testing.assert_allclose(got_rev, full, rtol=0, atol=1e-12)
