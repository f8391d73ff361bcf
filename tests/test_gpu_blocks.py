"""GPU copy_blocks / swap_blocks against the oracle's block copies: bit-exact, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_232_amd as pkv

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _random_cache(g, shape):
    # raw 16-bit patterns (NaN and Inf patterns included): the copy must move bits, not values
    bits = torch.randint(-32768, 32768, shape, generator=g, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16)


def _mapping(g, nb, n):
    perm = torch.randperm(nb, generator=g)
    return torch.stack([perm[:n], perm[n:2 * n]], dim=1).to(torch.int64)


@pytest.mark.parametrize("layers,nb,hkv,bs,d,npairs", [(3, 64, 8, 16, 128, 20), (1, 10, 2, 32, 64, 4),
                                                       (2, 40, 4, 16, 256, 1)])
def test_copy_blocks_bit_exact(layers, nb, hkv, bs, d, npairs):
    g = torch.Generator().manual_seed(1000 + nb)
    kcs = [_random_cache(g, (nb, hkv, bs, d)) for _ in range(layers)]
    vcs = [_random_cache(g, (nb, hkv, bs, d)) for _ in range(layers)]
    m = _mapping(g, nb, npairs)
    m = torch.cat([m, torch.tensor([[nb, 0], [-1, 1], [2, nb + 5]], dtype=torch.int64)])  # skipped
    ek, ev = oracle.copy_blocks(kcs, vcs, m)
    kd = [c.to(DEV) for c in kcs]
    vd = [c.to(DEV) for c in vcs]
    pkv.copy_blocks(kd, vd, m.to(DEV))
    torch.cuda.synchronize()
    for l in range(layers):
        assert np.array_equal(kd[l].cpu().view(torch.int16).numpy(), ek[l]), f"K layer {l}"
        assert np.array_equal(vd[l].cpu().view(torch.int16).numpy(), ev[l]), f"V layer {l}"


def test_copy_blocks_repeated_calls_over_changing_cache_sets():
    """A serving loop's pattern: the same layers called again with new mappings, interleaved with
    other cache sets, more sets than the binding keeps address arrays for, and a set whose tensors
    are freed and reallocated. Every call is checked bit-exact against the oracle."""
    g = torch.Generator().manual_seed(77)
    nb, shape = 24, (24, 2, 16, 64)
    sets = []
    for i in range(11):
        layers = 1 + i % 3
        sets.append(([_random_cache(g, shape).to(DEV) for _ in range(layers)],
                     [_random_cache(g, shape).to(DEV) for _ in range(layers)]))
    for step in range(30):
        i = (step * 7) % len(sets) if step % 3 else 0  # set 0 recurs; the others cycle past the limit
        kd, vd = sets[i]
        m = _mapping(g, nb, 5)
        ek, ev = oracle.copy_blocks([c.cpu() for c in kd], [c.cpu() for c in vd], m)
        pkv.copy_blocks(kd, vd, m.to(DEV))
        torch.cuda.synchronize()
        for l in range(len(kd)):
            assert np.array_equal(kd[l].cpu().view(torch.int16).numpy(), ek[l]), f"step {step} K layer {l}"
            assert np.array_equal(vd[l].cpu().view(torch.int16).numpy(), ev[l]), f"step {step} V layer {l}"
        if step == 10:
            # free set 1 and allocate new caches (possibly at the same addresses)
            sets[1] = ([_random_cache(g, shape).to(DEV)], [_random_cache(g, shape).to(DEV)])


def test_copy_blocks_empty_mapping_is_noop():
    g = torch.Generator().manual_seed(5)
    kc = _random_cache(g, (8, 2, 16, 64)).to(DEV)
    vc = _random_cache(g, (8, 2, 16, 64)).to(DEV)
    k0, v0 = kc.clone(), vc.clone()
    pkv.copy_blocks([kc], [vc], torch.empty(0, 2, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), v0.view(torch.int16))


def test_swap_out_and_in_through_pinned_host_memory():
    g = torch.Generator().manual_seed(6)
    nb, nh = 48, 20
    dev_cache = _random_cache(g, (nb, 4, 16, 128)).to(DEV)
    host = torch.empty((nh, 4, 16, 128), dtype=torch.bfloat16, pin_memory=True)
    host.view(torch.int16).fill_(-1)
    host_before = host.view(torch.int16).numpy().copy()
    # a run of consecutive pairs (moved as one copy) and scattered pairs
    out_map = torch.tensor([[10, 0], [11, 1], [12, 2], [30, 7], [3, 15], [47, 19]], dtype=torch.int64)
    pkv.swap_blocks(dev_cache, host, out_map)
    torch.cuda.synchronize()
    expect_host = oracle.swap_blocks(dev_cache.cpu(), host_before, out_map)
    assert np.array_equal(host.view(torch.int16).numpy(), expect_host)
    # swap back in to other device blocks
    in_map = torch.stack([out_map[:, 1], torch.tensor([40, 41, 42, 5, 6, 7])], dim=1)
    before = dev_cache.cpu()
    pkv.swap_blocks(host, dev_cache, in_map)
    torch.cuda.synchronize()
    expect_dev = oracle.swap_blocks(host, before, in_map)
    assert np.array_equal(dev_cache.cpu().view(torch.int16).numpy(), expect_dev)


def test_swap_between_device_caches():
    g = torch.Generator().manual_seed(7)
    a = _random_cache(g, (16, 2, 16, 64)).to(DEV)
    b = _random_cache(g, (12, 2, 16, 64)).to(DEV)
    m = torch.tensor([[0, 11], [15, 0], [4, 5], [5, 6]], dtype=torch.int64)
    expect = oracle.swap_blocks(a.cpu(), b.cpu(), m)
    pkv.swap_blocks(a, b, m)
    torch.cuda.synchronize()
    assert np.array_equal(b.cpu().view(torch.int16).numpy(), expect)
    with pytest.raises(pkv.PkvError):
        pkv.swap_blocks(a, b, torch.tensor([[16, 0]]))


def test_swap_out_to_pageable_host_memory():
    # pageable memory is not addressable by the GPU: the library falls back to HIP copies
    g = torch.Generator().manual_seed(9)
    dev_cache = _random_cache(g, (24, 2, 16, 64)).to(DEV)
    host = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16)
    m = torch.tensor([[3, 0], [4, 1], [5, 2], [20, 6], [0, 7]], dtype=torch.int64)
    expect = oracle.swap_blocks(dev_cache.cpu(), host.clone(), m)
    pkv.swap_blocks(dev_cache, host, m)
    torch.cuda.synchronize()
    assert np.array_equal(host.view(torch.int16).numpy(), expect)
