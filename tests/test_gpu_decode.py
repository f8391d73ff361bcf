"""GPU parity of paged decode (direct and split-KV + LSE merge) against the fp64 oracle, through the
C ABI. Inputs come from the seeded generators; the oracle never sees GPU output except to compare."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_232_amd as pkv
from parity import assert_parity
from workloads import make_config, paged_decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev(di):
    return (di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.block_tables.to(DEV),
            di.seq_lens.to(DEV))


def _run(di, pt, with_lse=False, dev_tensors=None):
    q, kc, vc, bt, sl = dev_tensors if dev_tensors is not None else _dev(di)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV) if with_lse else None
    out = pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, max_seq_len=di.max_seq_len,
                                partition_tokens=pt, lse=lse)
    torch.cuda.synchronize()
    return (out.cpu(), lse.cpu() if with_lse else None)


@pytest.mark.parametrize("pt", [0, 512, 32, -1])
def test_tiny_paged_decode_config(pt):
    di = make_config(1)
    ref, rlse = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale,
                                    return_lse=True)
    out, lse = _run(di, pt, with_lse=True)
    print(f"tiny decode pt={pt}", assert_parity(out, ref, f"tiny decode pt={pt}"))
    np.testing.assert_allclose(lse.double().numpy(), rlse, rtol=0, atol=2e-3)


EDGE = [
    # lens, Hq, Hkv, D, BS, NB extra
    ([1], 1, 1, 64, 16),
    ([15, 16, 17], 4, 2, 128, 16),
    ([31, 32, 33, 0], 8, 1, 128, 16),
    ([0, 0], 4, 4, 64, 16),
    ([1000, 1, 513, 512, 511], 8, 2, 128, 16),
    ([700, 64], 32, 2, 128, 16),       # G = 16: a full MFMA column tile
    ([300, 129], 32, 1, 64, 16),       # G = 32: two head groups
    ([257, 40], 6, 1, 128, 16),        # G = 6: partial column tile
    ([1500, 3], 16, 2, 256, 16),
    ([333, 77], 8, 4, 128, 32),        # block size 32
    ([600, 17], 4, 1, 64, 64),         # block size 64
    ([300, 129, 1], 8, 2, 128, 128),   # block size 128: partitions of 64 tokens start inside a block
    ([700, 5, 256], 4, 1, 64, 256),    # block size 256
    ([1000, 33], 16, 4, 256, 128),     # block size 128 at head_dim 256
    ([2100, 255, 257], 32, 8, 128, 256),
]


# Long sequences (64 or more partitions) at batch x heads large enough that a wave streams several
# consecutive partitions and parks the finished partials in LDS (the launch keeps at least 512
# waves): partial head groups, head_dim 256, a count capped by the LDS budget, ragged ends
LONG = [
    # lens, Hq, Hkv, D, pt
    ([65536 + 17, 60000], 16, 2, 64, 32),       # G = 8: 16 partitions per wave
    ([70000, 64 * 1000 + 1], 40, 2, 128, 64),   # G = 20: the second head group has 4 columns
    ([70000 + 5, 3000], 8, 4, 256, 64),         # head_dim 256
    ([20000, 19999], 32, 2, 256, 32),           # G = 16 at head_dim 256: 4 per wave (LDS cap)
]


@pytest.mark.parametrize("case", range(len(LONG)))
def test_decode_long_multi_partition(case):
    lens, hq, hkv, d, pt = LONG[case]
    di = paged_decode_inputs(1500 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=lens)
    ref, rlse = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale,
                                    return_lse=True)
    out, lse = _run(di, pt, with_lse=True)
    print(f"long decode {LONG[case]}", assert_parity(out, ref, f"long decode {LONG[case]}"))
    np.testing.assert_allclose(lse.double().numpy(), rlse, rtol=0, atol=2e-3)


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("pt", [0, 64, 512, 1024])
def test_decode_edge_shapes(case, pt):
    lens, hq, hkv, d, bs = EDGE[case]
    di = paged_decode_inputs(1000 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=lens,
                             block_size=bs, num_blocks=sum((L + bs - 1) // bs for L in lens) + 3)
    ref, rlse = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale,
                                    return_lse=True)
    out, lse = _run(di, pt, with_lse=True)
    assert_parity(out, ref, f"edge {EDGE[case]} pt={pt}")
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(lse.double().numpy()[fin], rlse[fin], rtol=0, atol=2e-3)
    assert np.all(np.isneginf(lse.double().numpy()[~fin]))


@pytest.fixture(scope="module")
def config3():
    di = make_config(3)
    return di, _dev(di)


@pytest.mark.parametrize("pt", [0, 512, 2048])
def test_batched_decode_config_full(config3, pt):
    di, dev = config3
    ref = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    out, _ = _run(di, pt, dev_tensors=dev)
    print(f"config3 pt={pt}", assert_parity(out, ref, f"config3 pt={pt}"))


def test_batched_decode_block_shuffle_and_determinism(config3):
    di, dev = config3
    out1, _ = _run(di, 512, dev_tensors=dev)
    out2, _ = _run(di, 512, dev_tensors=dev)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16)), "run-to-run difference"
    g = torch.Generator().manual_seed(5)
    nb = di.k_cache.shape[0]
    perm = torch.randperm(nb, generator=g)
    kc = torch.empty_like(di.k_cache)
    vc = torch.empty_like(di.v_cache)
    kc[perm] = di.k_cache
    vc[perm] = di.v_cache
    bt = di.block_tables.clone()
    live = bt >= 0
    bt[live] = perm[bt[live].long()].to(torch.int32)
    q, _, _, _, sl = dev
    out3, _ = _run(di, 512, dev_tensors=(q, kc.to(DEV), vc.to(DEV), bt.to(DEV), sl))
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16)), "block shuffle changed the output"


def test_long_context_split_decode_config_full():
    """131072-token sequences at the launch the benchmark times (split 512 + merge): every (sequence,
    head) row and its log-sum-exp against the oracle, and a property that holds at any size."""
    di = make_config(4)
    q, kc, vc, bt, sl = _dev(di)
    lse = torch.empty(4, 64, dtype=torch.float32, device=DEV)
    out = pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, max_seq_len=di.max_seq_len, partition_tokens=512,
                                lse=lse)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    # every output row is a convex combination of V rows, so it lies within the V value range
    vmax = max(float(vc[i:i + 4096].float().abs().amax()) for i in range(0, vc.shape[0], 4096))
    assert float(out.float().abs().max()) <= vmax + 1e-2
    del q, kc, vc
    torch.cuda.empty_cache()
    ref, rlse = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale,
                                    return_lse=True)
    print("config4 full", assert_parity(out, ref, "config4 full"))
    np.testing.assert_allclose(lse.double().numpy(), rlse, rtol=0, atol=2e-3)


def test_decode_rejects_misshaped_outputs():
    di = make_config(1)
    q, kc, vc, bt, sl = _dev(di)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, out=torch.empty(2, 4, 32, dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, lse=torch.empty(2, 3, dtype=torch.float32, device=DEV))
    with pytest.raises(TypeError):
        pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, lse=torch.empty(2, 4, dtype=torch.float16, device=DEV))
    need = pkv.decode_workspace_bytes(2, 4, 2, 64, di.max_seq_len, 32)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, partition_tokens=32,
                              workspace=torch.empty(need - 16, dtype=torch.uint8, device=DEV))


def test_split_and_direct_agree():
    di = paged_decode_inputs(77, num_q_heads=16, num_kv_heads=2, head_dim=128, len_range=(1, 3000), batch=9)
    a, la = _run(di, 0, with_lse=True)
    b, lb = _run(di, 512, with_lse=True)
    c, lc = _run(di, 96, with_lse=True)
    ref = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    for x, n in ((a, "direct"), (b, "split512"), (c, "split96")):
        assert_parity(x, ref, n)
    assert (a.float() - b.float()).abs().max() <= 2e-2
    assert (la - lb).abs().max() <= 2e-3 and (la - lc).abs().max() <= 2e-3


@pytest.mark.parametrize("pt", [32, 1024, -1])
@pytest.mark.parametrize("window", [40000, 2000])
def test_decode_long_multi_partition_window(window, pt):
    """A sliding window over long sequences: with 32-token partitions and 40000 keys visible a wave
    streams several partitions starting inside the window, with 2000 one partition per wave; with
    1024-token partitions a partition's first chunk may start inside the window."""
    di = paged_decode_inputs(1600, num_q_heads=16, num_kv_heads=2, head_dim=64, seq_lens=[65536 + 17, 60000])
    ref, rlse = oracle.paged_decode_window(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens,
                                           di.scale, window, return_lse=True)
    q, kc, vc, bt, sl = _dev(di)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=DEV)
    out = pkv.paged_attn_decode(q, kc, vc, bt, sl, di.scale, max_seq_len=di.max_seq_len, partition_tokens=pt,
                                lse=lse, window=window)
    torch.cuda.synchronize()
    print(f"long window decode {window} pt={pt}", assert_parity(out.cpu(), ref, f"long window decode {window} pt={pt}"))
    np.testing.assert_allclose(lse.cpu().double().numpy(), rlse, rtol=0, atol=2e-3)
