"""GPU parity of ragged and paged prefill against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_232_amd as pkv
from parity import assert_parity
from workloads import chunked_prefill_inputs, make_config, ragged_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _ragged(ri):
    out = pkv.ragged_prefill(ri.q.to(DEV), ri.k.to(DEV), ri.v.to(DEV), ri.qo_indptr.to(DEV), ri.kv_indptr.to(DEV),
                             ri.causal, ri.scale, qo_indptr_h=ri.qo_indptr, kv_indptr_h=ri.kv_indptr)
    torch.cuda.synchronize()
    return out.cpu()


RAGGED_EDGE = [
    # qo_lens, kv_lens (None = same), Hq, Hkv, D, causal
    ([1], None, 1, 1, 64, True),
    ([5, 128, 129, 300], None, 4, 2, 128, True),   # G = 2: 2 heads x 64-row q tiles
    ([127, 1, 256], None, 8, 1, 64, True),
    ([200, 3], [450, 3], 4, 4, 128, True),          # qo < kv: bottom-right causal offset
    ([70, 9], [40, 9], 2, 1, 128, True),            # qo > kv: leading rows see no key
    ([100, 333], [180, 333], 6, 2, 128, False),     # non-causal, G = 3
    ([257, 64], None, 16, 4, 256, True),            # head_dim 256
    ([40, 0, 77], [60, 5, 77], 8, 2, 128, True),    # an empty request
    ([300], [0], 2, 1, 64, False),                  # no keys at all
    ([513, 255, 256], None, 4, 1, 128, True),       # 4 heads x 32-row q tiles, ragged tails
    ([700, 31], [1500, 31], 2, 2, 64, True),        # long prefix offset, head_dim 64
    ([600, 90], [600, 4000], 4, 2, 128, False),     # non-causal, kv much longer than q
    ([1] * 800, [37] * 800, 2, 1, 64, True),         # more q tiles than the launch arguments hold:
                                                    # schedule built on the device in the workspace
    # XCD placement of work-groups: heads of one kv head grouped on an XCD over 8 / Hkv schedule
    # rows (row counts not a multiple of the group pad the grid), and the per-XCD head mapping
    # when Hkv does not divide 8
    ([130, 70, 260], None, 16, 16, 128, True),      # Hkv = 16: per-XCD heads
    ([200, 17], None, 24, 3, 64, True),             # Hkv = 3: per-XCD heads, head_dim 64
    ([129, 5, 300], None, 8, 1, 128, True),         # group of 8 rows, 6 rows used
    ([129, 40, 1], [129, 90, 1], 16, 4, 256, True), # group of 2 rows, 4 rows, head_dim 256
    ([1] * 801, [37] * 801, 8, 2, 128, True),       # device-built schedule, 4 heads x 32 rows
    ([1] * 790, [50] * 790, 4, 2, 256, True),       # device-built schedule, 2 heads x 96-row q tiles
    ([400, 193, 192, 1], [600, 193, 300, 9], 8, 2, 256, True),  # 4 heads x 48-row q tiles, edges
    ([250, 97, 1], [400, 97, 30], 3, 3, 256, True), # one head per work-group: 192-row q tiles
    ([130, 61], [130, 200], 12, 2, 256, True),      # G = 6: 6 heads x 32-row q tiles
    # head_dim <= 128: a work-group takes gcd(G, 4) heads of one kv head over 128 / that rows
    ([129, 40, 1, 65], [129, 90, 1, 300], 32, 4, 128, True),  # G = 8: two head groups per kv
                                                    # head, XCD groups of 2 schedule rows
    ([100, 64, 65], [100, 64, 200], 12, 2, 64, True),  # G = 6: 2 heads x 64-row q tiles
    ([97, 33], [97, 150], 6, 2, 128, False),        # G = 3: one head, 128-row q tiles
    # schedules kept per XCD row class (a request's tiles on one XCD): 8 classes at 4 / 1 heads; a
    # request of 100 tiles would pad the class lists past the by-value schedule, so the plain
    # longest-first order runs instead
    ([3200, 40, 7], None, 4, 1, 64, True),
    ([300, 290, 40, 7, 100], [900, 290, 40, 60, 100], 8, 1, 64, True),  # 2 head groups, 4 classes
]


@pytest.mark.parametrize("case", range(len(RAGGED_EDGE)))
def test_ragged_prefill_edge_shapes(case):
    qo, kv, hq, hkv, d, causal = RAGGED_EDGE[case]
    ri = ragged_prefill_inputs(2000 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, qo_lens=qo,
                               kv_lens=kv, causal=causal)
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, ri.causal, ri.scale)
    out = _ragged(ri)
    assert_parity(out, ref, f"ragged edge {RAGGED_EDGE[case]}")


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 128), (8, 2, 64), (3, 3, 128), (16, 4, 256)])
@pytest.mark.parametrize("scale", [-0.3, 0.0])
def test_ragged_prefill_negative_and_zero_scale(hq, hkv, d, scale):
    """A negative scale (the kernels flip q's sign bits and keep a positive scale) and a zero one
    (uniform weights), at head_dim 64, 128 (even and odd GQA groups) and 256."""
    ri = ragged_prefill_inputs(2600 + hq + d, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, qo_lens=[150, 9, 300],
                               kv_lens=[200, 9, 300], causal=True)
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, True, scale)
    out = pkv.ragged_prefill(ri.q.to(DEV), ri.k.to(DEV), ri.v.to(DEV), ri.qo_indptr.to(DEV), ri.kv_indptr.to(DEV),
                             True, scale, qo_indptr_h=ri.qo_indptr, kv_indptr_h=ri.kv_indptr)
    torch.cuda.synchronize()
    assert_parity(out.cpu(), ref, f"ragged scale {scale} ({hq}/{hkv} heads, hd {d})")


def test_ragged_prefill_config_full():
    ri = make_config(2)
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, ri.causal, ri.scale)
    out = _ragged(ri)
    print("config2", assert_parity(out, ref, "config2 ragged prefill"))
    out2 = _ragged(ri)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "run-to-run difference"


def _chunked(ci):
    kc, vc = ci.k_cache.to(DEV), ci.v_cache.to(DEV)
    pkv.reshape_and_cache(ci.k_new.to(DEV), ci.v_new.to(DEV), kc, vc, ci.slot_mapping.to(DEV))
    out = pkv.paged_prefill(ci.q.to(DEV), kc, vc, ci.block_tables.to(DEV), ci.qo_indptr.to(DEV),
                            ci.kv_lens.to(DEV), ci.causal, ci.scale, qo_indptr_h=ci.qo_indptr, kv_lens_h=ci.kv_lens)
    torch.cuda.synchronize()
    return out.cpu(), kc.cpu(), vc.cpu()


PAGED_EDGE = [
    # chunk_lens, prefix_lens, Hq, Hkv, D, BS, causal
    ([1], [0], 1, 1, 64, 16, True),
    ([64, 1, 130], [0, 17, 31], 4, 2, 128, 16, True),
    ([9, 200], [300, 0], 8, 2, 256, 16, True),
    ([50, 129], [16, 100], 4, 1, 128, 32, True),
    ([33], [5000], 2, 2, 64, 64, True),
    ([600, 257], [700, 0], 4, 2, 128, 16, True),
    ([9, 200, 129], [300, 0, 2000], 16, 4, 256, 16, True),  # 5 schedule rows in groups of 2
    ([77, 1, 256], [33, 4000, 16], 8, 1, 64, 16, True),     # groups of 8, head_dim 64
    ([140, 60], [900, 45], 32, 8, 128, 32, True),           # one row per group
    ([129, 33, 1], [200, 64, 7], 32, 4, 64, 16, True),      # G = 8: 4 heads x 32 rows, XCD
                                                            # groups of 2 schedule rows
    # blocks larger than a kv tile (32 keys): a tile's rows sit in
    # one block at an offset, and the last blocks are partly filled
    ([130, 7], [300, 1000], 8, 2, 128, 128, True),
    ([66, 200], [129, 511], 4, 4, 64, 256, True),
    ([150, 40], [257, 1500], 16, 4, 256, 128, True),
    ([33, 140], [700, 3], 4, 1, 256, 256, True),
    ([200, 70, 1], [300, 0, 40], 8, 2, 128, 128, True),
    ([97, 64, 33], [64, 190, 1], 16, 4, 128, 64, True),    # blocks of two kv tiles at head_dim 128
    ([130, 31], [33, 96], 8, 2, 128, 32, True),            # blocks of exactly one kv tile
    # non-causal: every query row sees the whole prefix and chunk
    ([100, 140], [250, 33], 4, 2, 128, 16, False),
    ([60, 129], [1000, 0], 16, 4, 256, 16, False),
    ([31, 90], [64, 700], 8, 2, 64, 128, False),
]


@pytest.mark.parametrize("case", range(len(PAGED_EDGE)))
def test_paged_prefill_edge_shapes(case):
    C, P, hq, hkv, d, bs, causal = PAGED_EDGE[case]
    ci = chunked_prefill_inputs(3000 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, chunk_lens=C,
                                prefix_lens=P, block_size=bs, causal=causal)
    out, kc, vc = _chunked(ci)
    ek, ev = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    assert np.array_equal(kc.view(torch.int16).numpy(), ek) and np.array_equal(vc.view(torch.int16).numpy(), ev)
    ref = oracle.paged_prefill(ci.q, torch.from_numpy(ek).view(torch.bfloat16), torch.from_numpy(ev).view(torch.bfloat16),
                               ci.block_tables, ci.qo_indptr, ci.kv_lens, ci.causal, ci.scale)
    assert_parity(out, ref, f"paged edge {PAGED_EDGE[case]}")


def test_chunked_prefill_config_full():
    """16 requests, prefix up to 4096, head_dim 256, at the launch the benchmark times: the scatter
    bit-exact on the whole pool, every output row against the oracle, and a second run identical."""
    ci = make_config(5)
    out, kc, vc = _chunked(ci)
    ek, ev = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    assert np.array_equal(kc.view(torch.int16).numpy(), ek) and np.array_equal(vc.view(torch.int16).numpy(), ev)
    ref = oracle.paged_prefill(ci.q, torch.from_numpy(ek).view(torch.bfloat16),
                               torch.from_numpy(ev).view(torch.bfloat16), ci.block_tables, ci.qo_indptr,
                               ci.kv_lens, ci.causal, ci.scale)
    print("config5 full", assert_parity(out, ref, "config5 paged prefill"))
    out2, _, _ = _chunked(ci)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)), "run-to-run difference"


def test_paged_prefill_with_empty_prefix_equals_ragged():
    """With no cached prefix, prefill through the table must equal ragged prefill on the same rows."""
    ci = chunked_prefill_inputs(41, num_q_heads=8, num_kv_heads=2, head_dim=128, chunk_lens=[300, 45, 128],
                                prefix_lens=[0, 0, 0])
    out, _, _ = _chunked(ci)
    rag = pkv.ragged_prefill(ci.q.to(DEV), ci.k_new.to(DEV), ci.v_new.to(DEV), ci.qo_indptr.to(DEV),
                             ci.qo_indptr.to(DEV), True, ci.scale, qo_indptr_h=ci.qo_indptr, kv_indptr_h=ci.qo_indptr)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), rag.cpu().view(torch.int16))


def test_ragged_prefill_device_schedule_many_tiles():
    """9 767 (request, 32-row q tile) items of mixed lengths: the longest-first order is built on the device
    in the caller's workspace (items of one work bucket land in any order); every row matches the oracle
    and a second run (another order inside the buckets) is identical bit for bit."""
    g = torch.Generator().manual_seed(11)
    qo = [int(x) for x in torch.randint(1, 300, (1900,), generator=g)]
    ri = ragged_prefill_inputs(2100, num_q_heads=8, num_kv_heads=2, head_dim=64, qo_lens=qo, causal=True)
    need = pkv.prefill_workspace_bytes(ri.qo_indptr, 8, 2, 64)
    tiles = sum((n + 31) // 32 for n in qo)         # G = 4: 4 heads x 32 rows per work-group
    assert tiles > 768 and need >= 4 * tiles
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, ri.causal, ri.scale)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device=DEV)  # contents need no initialisation
    args = (ri.q.to(DEV), ri.k.to(DEV), ri.v.to(DEV), ri.qo_indptr.to(DEV), ri.kv_indptr.to(DEV), True, ri.scale)
    out = pkv.ragged_prefill(*args, qo_indptr_h=ri.qo_indptr, kv_indptr_h=ri.kv_indptr, workspace=ws)
    torch.cuda.synchronize()
    print("device schedule", assert_parity(out.cpu(), ref, "device-built schedule"))
    out2 = pkv.ragged_prefill(*args, qo_indptr_h=ri.qo_indptr, kv_indptr_h=ri.kv_indptr, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


GUARD = 512  # rows of sentinel before and after each buffer the kernels are told about


def _guarded(t: torch.Tensor):
    """t placed in a larger device buffer between GUARD sentinel rows; returns (buffer, view of t)."""
    buf = torch.full((t.shape[0] + 2 * GUARD,) + tuple(t.shape[1:]), 7.0, dtype=t.dtype)
    buf[GUARD:GUARD + t.shape[0]] = t
    buf = buf.to(DEV)
    return buf, buf[GUARD:GUARD + t.shape[0]]


def _guards_intact(buf: torch.Tensor):
    b = buf.cpu().float()
    return bool((b[:GUARD] == 7.0).all()) and bool((b[-GUARD:] == 7.0).all())


def test_ragged_prefill_device_offsets_clamped_to_host_sizes():
    """Device offsets that disagree with their host copies (the last ones past the buffers' ends) are
    clamped to the rows the host copies describe: the output equals the oracle over the clamped
    extents and no sentinel row around q, k, v or out changes."""
    qo_h, kv_h = [100, 150], [90, 210]
    ri = ragged_prefill_inputs(2200, num_q_heads=4, num_kv_heads=2, head_dim=128, qo_lens=qo_h, kv_lens=kv_h)
    qi_dev = torch.tensor([0, 120, 300], dtype=torch.int32)    # host: [0, 100, 250]
    ki_dev = torch.tensor([0, 95, 340], dtype=torch.int32)     # host: [0, 90, 300]
    qb, q = _guarded(ri.q)
    kb, k = _guarded(ri.k)
    vb, v = _guarded(ri.v)
    ob, out = _guarded(torch.zeros_like(ri.q))
    pkv.ragged_prefill(q, k, v, qi_dev.to(DEV), ki_dev.to(DEV), True, ri.scale, qo_indptr_h=ri.qo_indptr,
                       kv_indptr_h=ri.kv_indptr, out=out)
    torch.cuda.synchronize()
    for b_ in (qb, kb, vb, ob):
        assert _guards_intact(b_), "a sentinel row changed"
    qi_c = torch.tensor([0, 120, 250], dtype=torch.int32)
    ki_c = torch.tensor([0, 95, 300], dtype=torch.int32)
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, qi_c, ki_c, True, ri.scale)
    assert_parity(out.cpu(), ref, "clamped ragged offsets")


def test_paged_prefill_device_lengths_clamped():
    """A device kv length beyond its table row's capacity and a device q offset past the end of q are
    clamped: the output equals the oracle over the clamped extents, sentinel rows stay intact."""
    ci = chunked_prefill_inputs(2300, num_q_heads=8, num_kv_heads=2, head_dim=128, chunk_lens=[60, 100],
                                prefix_lens=[4, 28], block_size=16)
    # every table row full: kv lengths 64 and 128 fill 4 and 8 blocks of 16
    assert ci.kv_lens.tolist() == [64, 128] and ci.block_tables.shape[1] == 8
    kc, vc = ci.k_cache.to(DEV), ci.v_cache.to(DEV)
    pkv.reshape_and_cache(ci.k_new.to(DEV), ci.v_new.to(DEV), kc, vc, ci.slot_mapping.to(DEV))
    qb, q = _guarded(ci.q)
    ob, out = _guarded(torch.zeros_like(ci.q))
    qi_dev = torch.tensor([0, 60, 200], dtype=torch.int32)     # host: [0, 60, 160]
    kl_dev = torch.tensor([64, 5000], dtype=torch.int32)       # host: [64, 128]; capacity 8 * 16
    pkv.paged_prefill(q, kc, vc, ci.block_tables.to(DEV), qi_dev.to(DEV), kl_dev.to(DEV), True, ci.scale,
                      qo_indptr_h=ci.qo_indptr, kv_lens_h=ci.kv_lens, out=out)
    torch.cuda.synchronize()
    assert _guards_intact(qb) and _guards_intact(ob), "a sentinel row changed"
    ek, ev = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    ref = oracle.paged_prefill(ci.q, torch.from_numpy(ek).view(torch.bfloat16), torch.from_numpy(ev).view(torch.bfloat16),
                               ci.block_tables, ci.qo_indptr, ci.kv_lens, True, ci.scale)
    assert_parity(out.cpu(), ref, "clamped paged lengths")


def test_prefill_rejects_misshaped_outputs_and_workspaces():
    ri = ragged_prefill_inputs(2400, num_q_heads=4, num_kv_heads=2, head_dim=64, qo_lens=[10, 20])
    args = (ri.q.to(DEV), ri.k.to(DEV), ri.v.to(DEV), ri.qo_indptr.to(DEV), ri.kv_indptr.to(DEV), True, ri.scale)
    with pytest.raises(ValueError):
        pkv.ragged_prefill(*args, out=torch.empty(29, 4, 64, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        pkv.ragged_prefill(*args, out=torch.empty(30, 4, 32, dtype=torch.bfloat16, device=DEV))
    big = ragged_prefill_inputs(2401, num_q_heads=2, num_kv_heads=1, head_dim=64, qo_lens=[1] * 800)
    need = pkv.prefill_workspace_bytes(big.qo_indptr, 2, 1, 64)
    with pytest.raises(ValueError):
        pkv.ragged_prefill(big.q.to(DEV), big.k.to(DEV), big.v.to(DEV), big.qo_indptr.to(DEV),
                           big.kv_indptr.to(DEV), True, big.scale, workspace=torch.empty(need - 4, dtype=torch.uint8,
                                                                                         device=DEV))
