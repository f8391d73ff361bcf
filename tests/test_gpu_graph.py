"""A decode step (scatter of the new token's K/V, then decode over the grown cache) captured once in
a HIP graph and replayed with new inputs: every replay equals the eager step bit for bit and the
oracle within the parity gate. The launch is sized from the planner's real maximum length."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_232_amd as pkv
from parity import assert_parity
from workloads import paged_decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


@pytest.mark.parametrize("pt_req", [0, 512])
def test_decode_step_graph_replays(pt_req):
    Hq, Hkv, D = 32, 8, 128
    cap = [700, 1300, 64, 1025, 2000, 9]           # allocated tokens per sequence (table capacity)
    di = paged_decode_inputs(4100 + pt_req, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, seq_lens=cap)
    B, bs = len(cap), di.block_size
    max_len, pt, ws_bytes = pkv.decode_plan(cap, Hq, Hkv, D, pt_req)
    assert max_len == max(cap) and pt == pt_req
    kc, vc = di.k_cache.to(DEV), di.v_cache.to(DEV)
    bt = di.block_tables.to(DEV)
    q = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    k_new = torch.empty(B, Hkv, D, dtype=torch.bfloat16, device=DEV)
    v_new = torch.empty_like(k_new)
    slots = torch.empty(B, dtype=torch.int64, device=DEV)
    lens = torch.empty(B, dtype=torch.int32, device=DEV)
    out = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)

    def step(kc, vc, out):
        pkv.reshape_and_cache(k_new, v_new, kc, vc, slots)
        pkv.paged_attn_decode(q, kc, vc, bt, lens, di.scale, max_seq_len=max_len, partition_tokens=pt,
                              out=out, workspace=ws)

    g = torch.Generator().manual_seed(9)
    tables = di.block_tables

    def fill(step_lens):
        # the new token of sequence b goes to position step_lens[b] - 1
        q.copy_(torch.randn(B, Hq, D, generator=g).to(torch.bfloat16))
        k_new.copy_(torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16))
        v_new.copy_(torch.randn(B, Hkv, D, generator=g).to(torch.bfloat16))
        pos = [L - 1 for L in step_lens]
        slots.copy_(torch.tensor([int(tables[b, p // bs]) * bs + p % bs for b, p in enumerate(pos)]))
        lens.copy_(torch.tensor(step_lens, dtype=torch.int32))

    # warm up on a side stream, then capture
    fill([c - 5 if c > 5 else c for c in cap])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(kc.clone(), vc.clone(), torch.empty_like(out))
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(kc, vc, out)

    k_host, v_host = di.k_cache.clone(), di.v_cache.clone()
    for r, step_lens in enumerate([[c - 3 if c > 3 else c for c in cap], list(cap),
                                   [min(c, 1 + 97 * (i + 1)) for i, c in enumerate(cap)]]):
        fill(step_lens)
        torch.cuda.synchronize()
        # eager reference on copies of the caches as they are before this replay
        kc_e, vc_e, out_e = kc.clone(), vc.clone(), torch.empty_like(out)
        step(kc_e, vc_e, out_e)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), f"replay {r} differs from eager"
        assert torch.equal(kc.view(torch.int16), kc_e.view(torch.int16)), f"replay {r} cache differs"
        kb, vb = oracle.reshape_and_cache(k_new.cpu(), v_new.cpu(), k_host, v_host, slots.cpu())
        k_host = torch.from_numpy(kb).view(torch.bfloat16)
        v_host = torch.from_numpy(vb).view(torch.bfloat16)
        ref = oracle.paged_decode(q.cpu(), k_host, v_host, tables, lens.cpu(), di.scale)
        print(f"graph replay {r} pt={pt}", assert_parity(out.cpu(), ref, f"graph replay {r} pt={pt}"))
