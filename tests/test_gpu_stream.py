"""GPU sliding-window decode and decode streamed over tiles of resident blocks, against the oracle,
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_232_amd as pkv
from parity import assert_parity
from workloads import paged_decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

WINDOW_SHAPES = [
    # lens, Hq, Hkv, D, BS
    ([1, 40, 0, 1000], 8, 2, 128, 16),
    ([1500, 513, 77], 32, 8, 128, 16),
    ([700, 64], 16, 2, 256, 16),
    ([333, 129], 8, 4, 64, 32),
]


@pytest.mark.parametrize("case", range(len(WINDOW_SHAPES)))
@pytest.mark.parametrize("window", [1, 17, 100, 512, 513, 4096])
@pytest.mark.parametrize("pt", [0, 96, 512, -1])
def test_window_decode(case, window, pt):
    lens, hq, hkv, d, bs = WINDOW_SHAPES[case]
    di = paged_decode_inputs(5000 + case, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seq_lens=lens,
                             block_size=bs)
    ref, rlse = oracle.paged_decode_window(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens,
                                           di.scale, window, return_lse=True)
    lse = torch.empty(len(lens), hq, dtype=torch.float32, device=DEV)
    out = pkv.paged_attn_decode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.block_tables.to(DEV),
                                di.seq_lens.to(DEV), di.scale, max_seq_len=di.max_seq_len, partition_tokens=pt,
                                lse=lse, window=window)
    torch.cuda.synchronize()
    assert_parity(out.cpu(), ref, f"window {window} case {case} pt {pt}")
    np.testing.assert_allclose(lse.cpu().double().numpy(), rlse, rtol=0, atol=2e-3)


def _tiles(tables, lens, bs, cap):
    """Split each table row into tiles of at most cap blocks (device int32 tensors)."""
    B = len(lens)
    nt = max(-(-int(L) // (bs * cap)) for L in lens) if B else 0
    out = []
    for i in range(nt):
        t_tab = torch.zeros((B, cap), dtype=torch.int32)
        t_len = torch.zeros(B, dtype=torch.int32)
        for b, L in enumerate(lens):
            nblk = -(-int(L) // bs)
            blocks = tables[b, i * cap:min((i + 1) * cap, nblk)]
            t_tab[b, :len(blocks)] = blocks
            t_len[b] = max(0, min(int(L) - i * cap * bs, cap * bs))
        out.append((t_tab, t_len))
    return out


@pytest.mark.parametrize("cap,reverse", [(4, False), (4, True), (64, False), (1, False)])
def test_streamed_decode_equals_one_pass(cap, reverse):
    lens = [1000, 33, 0, 517, 2048]
    di = paged_decode_inputs(5100, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=lens)
    tiles = _tiles(di.block_tables, lens, di.block_size, cap)
    if reverse:
        tiles = tiles[::-1]
    ref, rlse = oracle.streamed_decode(di.q, di.k_cache, di.v_cache, tiles, di.scale, return_lse=True)
    full = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    np.testing.assert_allclose(ref, full, rtol=0, atol=1e-12)
    sd = pkv.StreamedDecode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.scale)
    sd.begin()
    for t_tab, t_len in tiles:
        sd.step(t_tab.to(DEV), t_len.to(DEV))
    lse = torch.empty(len(lens), 32, dtype=torch.float32, device=DEV)
    out = sd.finalize(lse=lse)
    torch.cuda.synchronize()
    print(f"streamed cap={cap} reverse={reverse}", assert_parity(out.cpu(), ref, f"streamed cap {cap}"))
    np.testing.assert_allclose(lse.cpu().double().numpy(), rlse, rtol=0, atol=2e-3)


def test_streamed_decode_empty_tiles_and_restart():
    lens = [300, 40]
    di = paged_decode_inputs(5200, num_q_heads=8, num_kv_heads=2, head_dim=64, seq_lens=lens)
    sd = pkv.StreamedDecode(di.q.to(DEV), di.k_cache.to(DEV), di.v_cache.to(DEV), di.scale)
    # a state with no tile (or only empty tiles) finalises to zeros
    sd.begin()
    sd.step(torch.zeros(2, 4, dtype=torch.int32, device=DEV), torch.zeros(2, dtype=torch.int32, device=DEV))
    out = sd.finalize()
    torch.cuda.synchronize()
    assert not out.cpu().float().any()
    # begin resets: a second pass gives the one-pass result
    sd.begin()
    for t_tab, t_len in _tiles(di.block_tables, lens, di.block_size, 3):
        sd.step(t_tab.to(DEV), t_len.to(DEV))
    out = sd.finalize()
    torch.cuda.synchronize()
    ref = oracle.paged_decode(di.q, di.k_cache, di.v_cache, di.block_tables, di.seq_lens, di.scale)
    assert_parity(out.cpu(), ref, "streamed after restart")
