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
    ([5, 128, 129, 300], None, 4, 2, 128, True),
    ([127, 1, 256], None, 8, 1, 64, True),
    ([200, 3], [450, 3], 4, 4, 128, True),          # qo < kv: bottom-right causal offset
    ([70, 9], [40, 9], 2, 1, 128, True),            # qo > kv: leading rows see no key
    ([100, 333], [180, 333], 6, 2, 128, False),     # non-causal, G = 3
    ([257, 64], None, 16, 4, 256, True),            # head_dim 256
    ([40, 0, 77], [60, 5, 77], 8, 2, 128, True),    # an empty request
    ([300], [0], 2, 1, 64, False),                  # no keys at all
    ([513, 255, 256], None, 4, 1, 128, True),       # several 256-row q tiles, ragged tails
    ([700, 31], [1500, 31], 2, 2, 64, True),        # long prefix offset, head_dim 64
    ([600, 90], [600, 4000], 4, 2, 128, False),     # non-causal, kv much longer than q
    ([1] * 800, [37] * 800, 2, 1, 64, True),         # more q tiles than the launch schedule holds
    # XCD placement of work-groups: heads of one kv head grouped on an XCD over 8 / Hkv schedule
    # rows (row counts not a multiple of the group pad the grid), the per-XCD head mapping when
    # Hkv does not divide 8, and the plain grid
    ([130, 70, 260], None, 16, 16, 128, True),      # Hkv = 16: per-XCD heads
    ([200, 17], None, 24, 3, 64, True),             # Hkv = 3: per-XCD heads, head_dim 64
    ([129, 5, 300], None, 8, 1, 128, True),         # group of 8 rows, 6 rows used
    ([129, 40, 1], [129, 90, 1], 16, 4, 256, True), # group of 2 rows, 4 rows, head_dim 256
    ([1] * 801, [37] * 801, 8, 2, 128, True),       # plain grid (801 requests), group of 4
]


@pytest.mark.parametrize("case", range(len(RAGGED_EDGE)))
def test_ragged_prefill_edge_shapes(case):
    qo, kv, hq, hkv, d, causal = RAGGED_EDGE[case]
    ri = ragged_prefill_inputs(2000 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, qo_lens=qo,
                               kv_lens=kv, causal=causal)
    ref = oracle.ragged_prefill(ri.q, ri.k, ri.v, ri.qo_indptr, ri.kv_indptr, ri.causal, ri.scale)
    out = _ragged(ri)
    assert_parity(out, ref, f"ragged edge {RAGGED_EDGE[case]}")


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
    # chunk_lens, prefix_lens, Hq, Hkv, D, BS
    ([1], [0], 1, 1, 64, 16),
    ([64, 1, 130], [0, 17, 31], 4, 2, 128, 16),
    ([9, 200], [300, 0], 8, 2, 256, 16),
    ([50, 129], [16, 100], 4, 1, 128, 32),
    ([33], [5000], 2, 2, 64, 64),
    ([600, 257], [700, 0], 4, 2, 128, 16),
    ([9, 200, 129], [300, 0, 2000], 16, 4, 256, 16),  # 5 schedule rows in groups of 2
    ([77, 1, 256], [33, 4000, 16], 8, 1, 64, 16),     # groups of 8, head_dim 64
    ([140, 60], [900, 45], 32, 8, 128, 32),           # one row per group
]


@pytest.mark.parametrize("case", range(len(PAGED_EDGE)))
def test_paged_prefill_edge_shapes(case):
    C, P, hq, hkv, d, bs = PAGED_EDGE[case]
    ci = chunked_prefill_inputs(3000 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, chunk_lens=C,
                                prefix_lens=P, block_size=bs)
    out, kc, vc = _chunked(ci)
    ek, ev = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    assert np.array_equal(kc.view(torch.int16).numpy(), ek) and np.array_equal(vc.view(torch.int16).numpy(), ev)
    ref = oracle.paged_prefill(ci.q, torch.from_numpy(ek).view(torch.bfloat16), torch.from_numpy(ev).view(torch.bfloat16),
                               ci.block_tables, ci.qo_indptr, ci.kv_lens, True, ci.scale)
    assert_parity(out, ref, f"paged edge {PAGED_EDGE[case]}")


def test_chunked_prefill_config_sampled():
    """16 requests, prefix up to 4096, head_dim 256: scatter checked bit-exact on the whole pool, attention
    checked on sampled rows (every request's first and last row plus random rows)."""
    ci = make_config(5)
    out, kc, vc = _chunked(ci)
    ek, ev = oracle.reshape_and_cache(ci.k_new, ci.v_new, ci.k_cache, ci.v_cache, ci.slot_mapping)
    assert np.array_equal(kc.view(torch.int16).numpy(), ek) and np.array_equal(vc.view(torch.int16).numpy(), ev)
    rng = np.random.default_rng(5)
    qi = ci.qo_indptr.tolist()
    rows = []
    for b in range(len(qi) - 1):
        for t in (qi[b], qi[b + 1] - 1, int(rng.integers(qi[b], qi[b + 1]))):
            rows.append((t, int(rng.integers(0, 16))))
    ref = oracle.paged_prefill_rows(ci.q, torch.from_numpy(ek).view(torch.bfloat16),
                                    torch.from_numpy(ev).view(torch.bfloat16), ci.block_tables, ci.qo_indptr,
                                    ci.kv_lens, True, ci.scale, rows)
    got = torch.stack([out[t, h] for t, h in rows])
    print("config5 sampled", assert_parity(got, ref, "config5 sampled"))
    assert torch.isfinite(out.float()).all()


def test_paged_prefill_with_empty_prefix_equals_ragged():
    """With no cached prefix, prefill through the table must equal ragged prefill on the same rows."""
    ci = chunked_prefill_inputs(41, num_q_heads=8, num_kv_heads=2, head_dim=128, chunk_lens=[300, 45, 128],
                                prefix_lens=[0, 0, 0])
    out, _, _ = _chunked(ci)
    rag = pkv.ragged_prefill(ci.q.to(DEV), ci.k_new.to(DEV), ci.v_new.to(DEV), ci.qo_indptr.to(DEV),
                             ci.qo_indptr.to(DEV), True, ci.scale, qo_indptr_h=ci.qo_indptr, kv_indptr_h=ci.qo_indptr)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), rag.cpu().view(torch.int16))
