#!/usr/bin/env python3
"""Benchmark of the paged-KV attention hot path on one MI355X (gfx950).

One step runs every call of the hot path once, on inputs already resident in HBM:
  1. reshape_and_cache + paged_prefill   chunked prefill over a paged prefix: 16 requests, prefix
                                          U[0,4096], chunk U[64,1024], 16 q / 4 kv heads, head_dim 256
  2. ragged_prefill                       8 requests, lengths U[128,2048], 32 q / 8 kv heads, hd 128, causal
  3. paged_attn_decode (library choice)   batch 64, lengths U[512,8192], 32 q / 8 kv heads, hd 128
  4. paged_attn_decode (split 512)        batch 4, 131072 tokens each, 64 q / 8 kv heads, hd 128
Each call is bracketed by HIP events on the stream it is launched on. The headline value is the
decode KV bandwidth (algorithmic bytes of calls 3 and 4 over their measured time); the ragged
prefill TFLOP/s is reported beside it. The direct and split decode paths of workload 3, decode of
workloads 3 and 4 over an fp8 (e4m3) cache, a sliding window over workload 4, workload 3 streamed
over tiles of resident blocks, a small decode step and the same step over 32 layers (each eager and
replayed from a HIP graph), and the
block-management calls (copy_blocks over 32 layers, swap_blocks to pinned host
memory) are timed separately, outside the step.

Besides rates and roofline fractions, every call reports tokens per second (decoded sequences and
KV tokens attended for decode, query rows for prefill); the decode steps are also timed host-inclusive
(wall clock over back-to-back calls), eager and replayed from a graph; a plain 1 GiB device copy is
timed for context; the batched and long-context decodes also run with a plan measured by
pkv_decode_tune.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --calibrate-copy     (times a plain 1 GiB device copy, for counter scaling)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import paged_kv_cache_232_amd as pkv  # noqa: E402
from workloads import CONFIGS, make_config  # noqa: E402

HBM_PEAK_GBS = 8000.0                          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 256 * 2.4e9 * 4096 / 1e12  # dense bf16 MFMA, 2516.6 TFLOP/s
PCIE_PEAK_GBS = 64.0                           # PCIe 5.0 x16, one direction
METRIC = "decode KV GB/s (% HBM peak); ragged-prefill bf16 TFLOP/s (% MFMA peak)"


# ----------------------------------------------------------------------------------------------
# Measured HBM traffic per call (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1, the factors a plain 1 GiB
# copy gives; profiles/hot_path_step_hbm_traffic.md). Each figure holds only while the kernel sources
# it was taken from are unchanged: the sha256 over those files is checked at run time, and a
# mismatch reports traffic as null.
CSRC = os.path.join(ROOT, "paged_kv_cache_232_amd", "csrc")
TRAFFIC = {
    "scatter5": (("cache.hip",), "ca92b19357222b29", 71235247),
    "paged5": (("prefill.hip", "common.h"), "f49de67e0e090139", 360248764),
    "ragged2": (("prefill.hip", "common.h"), "f49de67e0e090139", 190617705),
    # calls whose path the library chooses: the planner's source counts too
    "decode3": (("decode.hip", "common.h", "api.cpp"), "587cfab9b83cc238", 1019115770),
    "decode3_direct": (("decode.hip", "common.h"), "323c2aaa61f82093", 1019115770),
    "decode3_split": (("decode.hip", "common.h"), "323c2aaa61f82093", 1039502301),
    "decode4": (("decode.hip", "common.h"), "323c2aaa61f82093", 2220469594),
    "decode3_fp8": (("decode.hip", "common.h", "api.cpp"), "587cfab9b83cc238", 510425645),
    "decode4_fp8": (("decode.hip", "common.h", "api.cpp"), "587cfab9b83cc238", 1083848862),
    "copy_blocks": (("blocks.hip",), "e2f6aca7c6815576", 1073908547),
}


def sources_sha(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(call):
    if call not in TRAFFIC:
        return None
    files, sha, nbytes = TRAFFIC[call]
    return nbytes if sources_sha(files) == sha else None


# ----------------------------------------------------------------------------------------------
# Algorithmic work (what the method must move or compute; no padding, no masked work)
# ----------------------------------------------------------------------------------------------
def decode_bytes(lens, hq, hkv, d, bs) -> int:
    """K and V rows of every token + q in + out + the table entries read + seq_lens."""
    kv = sum(2 * L * hkv * d * 2 for L in lens)
    qo = 2 * len(lens) * hq * d * 2
    table = sum((L + bs - 1) // bs for L in lens) * 4 + 4 * len(lens)
    return kv + qo + table


def decode_bytes_fp8(lens, hq, hkv, d, bs) -> int:
    """As decode_bytes with one byte per cached K / V element (fp8 e4m3 codes)."""
    return decode_bytes(lens, hq, hkv, d, bs) - sum(2 * L * hkv * d for L in lens)


def decode_flops(lens, hq, d) -> int:
    return sum(4 * L * hq * d for L in lens)


def prefill_pairs(qo, kv, causal) -> int:
    if not causal:
        return qo * kv
    off = kv - qo
    # row i sees keys 0..min(kv-1, i+off)
    total = 0
    for i in range(qo):
        total += max(0, min(kv, i + off + 1))
    return total


def prefill_flops(qo_lens, kv_lens, hq, d, causal) -> int:
    return sum(4 * d * hq * prefill_pairs(q, k, causal) for q, k in zip(qo_lens, kv_lens))


def scatter_bytes(T, hkv, d) -> int:
    return 2 * (2 * T * hkv * d * 2) + 8 * T  # read k,v + write k,v rows + slots


# ----------------------------------------------------------------------------------------------
class Case:
    def __init__(self, name, fn, kind, work, unit, tokens=None):
        self.name, self.fn, self.kind, self.work, self.unit = name, fn, kind, work, unit
        # tokens: {label: count} per call, reported as count / time (e.g. decoded sequences,
        # KV tokens attended, prefill query rows)
        self.tokens = tokens or {}
        self.ms = []

    def rate(self, ms):
        return self.work / (ms * 1e-3) / (1e12 if self.kind == "mfma" else 1e9)


def build_cases(dev, tune=True):
    cases = {}
    # workload 5: scatter + paged prefill
    ci = make_config(5)
    spec = CONFIGS[5]
    c5 = dict(q=ci.q.to(dev), k_new=ci.k_new.to(dev), v_new=ci.v_new.to(dev), kc=ci.k_cache.to(dev),
              vc=ci.v_cache.to(dev), bt=ci.block_tables.to(dev), slots=ci.slot_mapping.to(dev),
              qi=ci.qo_indptr.to(dev), kl=ci.kv_lens.to(dev), qi_h=ci.qo_indptr, kl_h=ci.kv_lens,
              scale=ci.scale)
    c5["out"] = torch.empty_like(c5["q"])
    c5["ws"] = torch.empty(max(pkv.prefill_workspace_bytes(ci.qo_indptr, spec["num_q_heads"], spec["num_kv_heads"],
                                                           spec["head_dim"]), 16), dtype=torch.uint8, device=dev)
    T5 = int(ci.qo_indptr[-1])
    chunk = [int(ci.qo_indptr[b + 1] - ci.qo_indptr[b]) for b in range(len(ci.kv_lens))]
    kvl5 = ci.kv_lens.tolist()
    cases["scatter5"] = Case(
        "reshape_and_cache (chunked prefill, 16 req, hd 256)",
        lambda: pkv.reshape_and_cache(c5["k_new"], c5["v_new"], c5["kc"], c5["vc"], c5["slots"]),
        "hbm", scatter_bytes(T5, spec["num_kv_heads"], spec["head_dim"]), "GB/s", {"tokens_per_s": T5})
    cases["paged5"] = Case(
        "paged_prefill (16 req, prefix U[0,4096], chunk U[64,1024], 16/4 heads, hd 256)",
        lambda: pkv.paged_prefill(c5["q"], c5["kc"], c5["vc"], c5["bt"], c5["qi"], c5["kl"], True, c5["scale"],
                                  qo_indptr_h=c5["qi_h"], kv_lens_h=c5["kl_h"], out=c5["out"], workspace=c5["ws"]),
        "mfma", prefill_flops(chunk, kvl5, spec["num_q_heads"], spec["head_dim"], True), "TFLOP/s",
        {"q_tokens_per_s": T5})
    meta = {"T5": T5, "prefix_mean": float(ci.prefix_lens.float().mean()), "chunk_mean": T5 / len(chunk)}
    del ci

    # workload 2: ragged prefill
    ri = make_config(2)
    spec = CONFIGS[2]
    c2 = dict(q=ri.q.to(dev), k=ri.k.to(dev), v=ri.v.to(dev), qi=ri.qo_indptr.to(dev), ki=ri.kv_indptr.to(dev),
              qi_h=ri.qo_indptr, ki_h=ri.kv_indptr, scale=ri.scale)
    c2["out"] = torch.empty_like(c2["q"])
    c2["ws"] = torch.empty(max(pkv.prefill_workspace_bytes(ri.qo_indptr, spec["num_q_heads"], spec["num_kv_heads"],
                                                           spec["head_dim"]), 16), dtype=torch.uint8, device=dev)
    lens2 = [int(ri.qo_indptr[b + 1] - ri.qo_indptr[b]) for b in range(8)]
    cases["ragged2"] = Case(
        "ragged_prefill (8 req, U[128,2048], 32/8 heads, hd 128, causal)",
        lambda: pkv.ragged_prefill(c2["q"], c2["k"], c2["v"], c2["qi"], c2["ki"], True, c2["scale"],
                                   qo_indptr_h=c2["qi_h"], kv_indptr_h=c2["ki_h"], out=c2["out"], workspace=c2["ws"]),
        "mfma", prefill_flops(lens2, lens2, spec["num_q_heads"], spec["head_dim"], True), "TFLOP/s",
        {"q_tokens_per_s": sum(lens2)})
    meta["lens2"] = lens2
    del ri

    # workloads 3 and 4: decode
    for cid, key in ((3, "decode3"), (4, "decode4")):
        di = make_config(cid)
        spec = CONFIGS[cid]
        c = dict(q=di.q.to(dev), kc=di.k_cache.to(dev), vc=di.v_cache.to(dev), bt=di.block_tables.to(dev),
                 sl=di.seq_lens.to(dev), msl=di.max_seq_len, scale=di.scale)
        c["out"] = torch.empty_like(c["q"])
        B, Hq, D = di.q.shape
        Hkv = spec["num_kv_heads"]
        lens = di.seq_lens.tolist()
        pt = -1 if cid == 3 else 512
        need = pkv.decode_workspace_bytes(B, Hq, Hkv, D, di.max_seq_len, 512)
        c["ws"] = torch.empty(need, dtype=torch.uint8, device=dev)
        work = decode_bytes(lens, Hq, Hkv, D, di.block_size)

        def mk(c=c, pt=pt):
            return lambda: pkv.paged_attn_decode(c["q"], c["kc"], c["vc"], c["bt"], c["sl"], c["scale"],
                                                 max_seq_len=c["msl"], partition_tokens=pt, out=c["out"],
                                                 workspace=c["ws"])
        dtok = {"seqs_per_s": B, "kv_tokens_per_s": sum(lens)}
        cases[key] = Case(f"paged_attn_decode ({CONFIGS[cid]['name']}, B={B}, {Hq}/{Hkv} heads, hd {D})",
                          mk(), "hbm", work, "GB/s", dtok)
        # the measured plan for this shape (pkv_decode_tune, once at set-up); without tuning, the
        # library's default choice as a plan
        if tune:
            plan = pkv.decode_tune(c["q"], c["kc"], c["vc"], c["bt"], c["sl"], c["scale"], max_seq_len=c["msl"],
                                   repeats=5, out=c["out"])
        else:
            _, dpt, dws = pkv.decode_plan(lens, Hq, Hkv, D, pt)
            plan = pkv.DecodePlan(partition_tokens=dpt, partitions_per_wave=0, max_seq_len=di.max_seq_len,
                                  workspace_bytes=dws)
        c["plan"] = plan
        c["ws_plan"] = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device=dev)

        def mkp(c=c):
            return lambda: pkv.paged_attn_decode(c["q"], c["kc"], c["vc"], c["bt"], c["sl"], c["scale"],
                                                 max_seq_len=c["msl"], out=c["out"], workspace=c["ws_plan"],
                                                 plan=c["plan"])
        cases[key + "_tuned"] = Case(f"paged_attn_decode_tuned ({CONFIGS[cid]['name']}, plan: partition "
                                     f"{plan.partition_tokens}, {plan.partitions_per_wave} per wave)",
                                     mkp(), "hbm", work, "GB/s", dtok)
        meta[f"plan{cid}"] = {"partition_tokens": plan.partition_tokens,
                              "partitions_per_wave": plan.partitions_per_wave, "candidates": plan.candidates,
                              "tune_measured_us": round(plan.measured_us, 1),
                              "tune_default_us": round(plan.default_us, 1)}
        if cid == 3:
            cases["decode3_direct"] = Case("paged_attn_decode direct path (batched decode)", mk(c, 0), "hbm", work,
                                           "GB/s", dtok)
            cases["decode3_split"] = Case("paged_attn_decode split 512 (batched decode)", mk(c, 512), "hbm", work,
                                          "GB/s", dtok)
        if cid == 4:
            # sliding window of the last 8192 tokens over the long contexts (split 512)
            W = 8192
            wlens = [min(L, W) for L in lens]

            def mkw(c=c):
                return lambda: pkv.paged_attn_decode(c["q"], c["kc"], c["vc"], c["bt"], c["sl"], c["scale"],
                                                     max_seq_len=c["msl"], partition_tokens=512, out=c["out"],
                                                     workspace=c["ws"], window=W)
            cases["decode4_window"] = Case(f"paged_attn_decode_window (long-context, window {W}, split 512)",
                                           mkw(), "hbm", decode_bytes(wlens, Hq, Hkv, D, di.block_size), "GB/s",
                                           {"seqs_per_s": B, "kv_tokens_per_s": sum(wlens)})
        if cid == 3:
            # the batched workload streamed over tiles of 64 resident blocks (1024 tokens): one
            # launch per tile folded into a running state, then finalize
            cap = 64
            ntile = -(-max(lens) // (cap * di.block_size))
            tiles = []
            for i in range(ntile):
                t_tab = torch.zeros((B, cap), dtype=torch.int32)
                t_len = torch.zeros(B, dtype=torch.int32)
                for b_, L in enumerate(lens):
                    nblk = -(-L // di.block_size)
                    blocks = di.block_tables[b_, i * cap:min((i + 1) * cap, nblk)]
                    t_tab[b_, :len(blocks)] = blocks
                    t_len[b_] = max(0, min(L - i * cap * di.block_size, cap * di.block_size))
                tiles.append((t_tab.to(dev), t_len.to(dev)))
            sdec = pkv.StreamedDecode(c["q"], c["kc"], c["vc"], c["scale"])

            def streamed(sdec=sdec, tiles=tiles, c=c):
                sdec.begin()
                for t_tab, t_len in tiles:
                    sdec.step(t_tab, t_len)
                sdec.finalize(out=c["out"])
            cases["decode3_streamed"] = Case(f"streamed decode, batched workload over {ntile} tiles of {cap} blocks",
                                             streamed, "hbm", work, "GB/s", dtok)
        # the same workload over an fp8 (e4m3) cache (timed alone): codes of cache / scale, one byte
        # per element, so half the bytes of the bf16 cache
        c["k_scale"], c["v_scale"] = 0.02, 0.02
        c["kc8"] = (c["kc"].float() / c["k_scale"]).to(torch.float8_e4m3fn).view(torch.uint8)
        c["vc8"] = (c["vc"].float() / c["v_scale"]).to(torch.float8_e4m3fn).view(torch.uint8)

        # (the library's own path choice: direct for the batched workload, 4096-token partitions
        # for the long contexts)
        _, pt8, _ = pkv.decode_plan(lens, Hq, Hkv, D)

        def mk8(c=c):
            return lambda: pkv.paged_attn_decode(c["q"], c["kc8"], c["vc8"], c["bt"], c["sl"], c["scale"],
                                                 max_seq_len=c["msl"], partition_tokens=-1, out=c["out"],
                                                 workspace=c["ws"], k_scale=c["k_scale"], v_scale=c["v_scale"])
        path8 = "direct" if pt8 == 0 else f"split {pt8}"
        cases[key + "_fp8"] = Case(f"paged_attn_decode_fp8 ({CONFIGS[cid]['name']} over an e4m3 cache, library's "
                                   f"choice: {path8})", mk8(), "hbm",
                                   decode_bytes_fp8(lens, Hq, Hkv, D, di.block_size), "GB/s", dtok)
        meta[f"lens{cid}_sum"] = sum(lens)
        meta[f"flops{cid}"] = decode_flops(lens, Hq, D)
        del di
    # a small decode step (scatter of each sequence's new token, then decode), eager and replayed
    # from a HIP graph captured once with the planner's real maximum length
    from workloads import paged_decode_inputs
    cap = [int(x) for x in torch.randint(512, 2049, (8,), generator=torch.Generator().manual_seed(232200))]
    sd = paged_decode_inputs(232201, num_q_heads=32, num_kv_heads=8, head_dim=128, seq_lens=cap)
    ds = dict(q=sd.q.to(dev), kc=sd.k_cache.to(dev), vc=sd.v_cache.to(dev), bt=sd.block_tables.to(dev),
              sl=sd.seq_lens.to(dev), kn=torch.randn(8, 8, 128, device=dev).to(torch.bfloat16))
    ds["vn"] = ds["kn"].clone()
    pos = [L - 1 for L in cap]
    ds["slots"] = torch.tensor([int(sd.block_tables[b, p // 16]) * 16 + p % 16 for b, p in enumerate(pos)],
                               dtype=torch.int64, device=dev)
    mx, ptp, wsb = pkv.decode_plan(cap, 32, 8, 128)
    ds["ws"] = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    ds["out"] = torch.empty_like(ds["q"])

    def small_step(ds=ds, mx=mx, ptp=ptp):
        pkv.reshape_and_cache(ds["kn"], ds["vn"], ds["kc"], ds["vc"], ds["slots"])
        pkv.paged_attn_decode(ds["q"], ds["kc"], ds["vc"], ds["bt"], ds["sl"], sd.scale, max_seq_len=mx,
                              partition_tokens=ptp, out=ds["out"], workspace=ds["ws"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        small_step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        small_step()
    sbytes = decode_bytes(cap, 32, 8, 128, 16) + scatter_bytes(8, 8, 128)
    stok = {"seqs_per_s": 8, "kv_tokens_per_s": sum(cap)}
    cases["decode_step_eager"] = Case("decode step, eager launches (scatter + decode, B=8, U[512,2048])",
                                      small_step, "hbm", sbytes, "GB/s", stok)
    cases["decode_step_graph"] = Case("decode step replayed from a HIP graph (same step)", graph.replay, "hbm",
                                      sbytes, "GB/s", stok)
    meta["graph"] = graph  # keep the captured graph alive
    # the same step over 32 layers, each with its own K/V cache (a model's decode step runs it once
    # per layer): one graph launch then carries 96 kernels, so its fixed launch cost is shared
    nl = 32
    lkc = [ds["kc"].clone() for _ in range(nl)]
    lvc = [ds["vc"].clone() for _ in range(nl)]

    def layers_step(ds=ds, mx=mx, ptp=ptp):
        for kc_l, vc_l in zip(lkc, lvc):
            pkv.reshape_and_cache(ds["kn"], ds["vn"], kc_l, vc_l, ds["slots"])
            pkv.paged_attn_decode(ds["q"], kc_l, vc_l, ds["bt"], ds["sl"], sd.scale, max_seq_len=mx,
                                  partition_tokens=ptp, out=ds["out"], workspace=ds["ws"])
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layers_step()
    torch.cuda.current_stream().wait_stream(side)
    graph32 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph32):
        layers_step()
    ltok = {k: v * nl for k, v in stok.items()}
    cases["decode_step32_eager"] = Case(f"decode step over {nl} layers, eager launches", layers_step, "hbm",
                                        sbytes * nl, "GB/s", ltok)
    cases["decode_step32_graph"] = Case(f"decode step over {nl} layers replayed from one HIP graph",
                                        graph32.replay, "hbm", sbytes * nl, "GB/s", ltok)
    meta["graph32"] = (graph32, lkc, lvc)

    # block management around the cache (timed alone, outside the step): copy_blocks over 32
    # layers of the batched-decode cache shape, and a swap-out of 256 blocks to pinned host memory
    g = torch.Generator().manual_seed(232100)
    nb, layers, npairs = 2048, 32, 256
    blk_shape = (nb, 8, 16, 128)
    kcs = [torch.empty(blk_shape, dtype=torch.bfloat16, device=dev).normal_() for _ in range(layers)]
    vcs = [torch.empty(blk_shape, dtype=torch.bfloat16, device=dev).normal_() for _ in range(layers)]
    perm = torch.randperm(nb, generator=g)
    cmap = torch.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).to(torch.int64).to(dev)
    block_bytes = 8 * 16 * 128 * 2
    cases["copy_blocks"] = Case(
        f"copy_blocks ({layers} layers, {npairs} pairs, 32 KiB blocks, K and V)",
        lambda: pkv.copy_blocks(kcs, vcs, cmap), "hbm", 2 * 2 * layers * npairs * block_bytes, "GB/s")
    host = torch.empty((npairs,) + blk_shape[1:], dtype=torch.bfloat16, pin_memory=True)
    smap = torch.stack([perm[:npairs], torch.arange(npairs)], 1).to(torch.int64)
    cases["swap_out"] = Case(
        f"swap_blocks device -> pinned host ({npairs} scattered 32 KiB blocks)",
        lambda: pkv.swap_blocks(kcs[0], host, smap), "pcie", npairs * block_bytes, "GB/s")
    return cases, meta


STEP = ["scatter5", "paged5", "ragged2", "decode3", "decode4"]
# timed alone, outside the step
EXTRA = ["decode3_direct", "decode3_split", "decode3_tuned", "decode4_tuned", "decode3_fp8", "decode4_fp8",
         "decode4_window", "decode3_streamed", "decode_step_eager", "decode_step_graph", "decode_step32_eager",
         "decode_step32_graph", "copy_blocks", "swap_out"]
# host-inclusive latency (wall clock over many back-to-back calls, then one synchronisation)
HOST_TIMED = ["decode_step_eager", "decode_step_graph", "decode_step32_eager", "decode_step32_graph"]


def time_step(cases, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for k in STEP:
            cases[k].fn()
    torch.cuda.synchronize()
    ev = {k: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for k in STEP}
    whole0 = torch.cuda.Event(enable_timing=True)
    whole1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    whole0.record(stream)
    for s in range(steps):
        for k in STEP:
            ev[k][s][0].record(stream)
            cases[k].fn()
            ev[k][s][1].record(stream)
    whole1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for k in STEP:
        cases[k].ms = [a.elapsed_time(b) for a, b in ev[k]]
    return whole0.elapsed_time(whole1) / steps, wall


def time_host(case, reps=200, warmup=20):
    """Wall-clock microseconds per call, launch overhead included: reps calls back to back, then one
    synchronisation (the host's view of a serving loop)."""
    for _ in range(warmup):
        case.fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        case.fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps * 1e6


def time_alone(case, reps=20, warmup=5):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        case.fn()
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record(stream)
        case.fn()
        b.record(stream)
    torch.cuda.synchronize()
    case.ms = [a.elapsed_time(b) for a, b in pairs]


# ----------------------------------------------------------------------------------------------
def cpu_baseline(meta):
    """The fp64 oracle on the host cores, on a bounded sample of the decode workload."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    import oracle
    di = make_config(3)
    spec = CONFIGS[3]
    n = 32  # first 32 of the 64 sequences (about 10 s of the oracle on 8 to 16 host cores)
    lens = di.seq_lens[:n].tolist()
    t0 = time.perf_counter()
    oracle.paged_decode(di.q[:n], di.k_cache, di.v_cache, di.block_tables[:n], di.seq_lens[:n], di.scale)
    dt = time.perf_counter() - t0
    work = decode_bytes(lens, spec["num_q_heads"], spec["num_kv_heads"], spec["head_dim"], di.block_size)
    gbs = work / dt / 1e9
    # prefill sample: the longest request of the ragged workload
    ri = make_config(2)
    lens2 = meta["lens2"]
    b = int(np.argmax(lens2))
    q0, q1 = int(ri.qo_indptr[b]), int(ri.qo_indptr[b + 1])
    import torch as _t
    qi = _t.tensor([0, q1 - q0], dtype=_t.int32)
    t1 = time.perf_counter()
    oracle.ragged_prefill(ri.q[q0:q1], ri.k[q0:q1], ri.v[q0:q1], qi, qi, True, ri.scale)
    dt2 = time.perf_counter() - t1
    fl = prefill_flops([q1 - q0], [q1 - q0], 32, 128, True)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"batched decode workload, first {n} of 64 sequences ({sum(lens)} tokens), fp64 NumPy, "
                      f"{dt:.2f} s",
            "prefill": {"value": round(fl / dt2 / 1e12, 6), "unit": "TFLOP/s",
                        "sample": f"ragged prefill workload, request {b} ({q1 - q0} rows) alone, {dt2:.2f} s"}}


def copy_bandwidth(dev):
    """A plain 1 GiB device-to-device copy (the runtime's), timed with HIP events: the practical
    streaming rate of this machine, reported beside the nominal 8 TB/s."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_bytes_each_way": n, "ms": round(ms, 4), "GB/s_read_plus_write": round(2 * n / ms / 1e6, 1)}


def calibrate_copy(dev):
    print(json.dumps(copy_bandwidth(dev)))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the decode tuning sweep at set-up (for profiler runs; the *_tuned lines then "
                         "run the default plan)")
    ap.add_argument("--only", default="",
                    help="comma-separated calls to time (default: all); a profiler run of one call then sees "
                         "only that call's kernels in the timed region")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library's hot path runs on a single MI355X and no "
              "multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pkv.load_library()
    if args.calibrate_copy:
        calibrate_copy(dev)
        return
    print(f"# device: {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)
    cases, meta = build_cases(dev, tune=not args.no_tune)
    print("# inputs resident; timing", file=sys.stderr, flush=True)
    if args.only:
        only = [k for k in args.only.split(",") if k]
        unknown = [k for k in only if k not in cases]
        if unknown:
            sys.exit(f"unknown calls {unknown}; known: {sorted(cases)}")
        for k in only:
            time_alone(cases[k], reps=args.steps, warmup=args.warmup)
            c = cases[k]
            print(json.dumps({"call": k, "name": c.name, "avg_ms": round(statistics.fmean(c.ms), 5),
                              "rate": round(c.rate(statistics.fmean(c.ms)), 2), "unit": c.unit}), flush=True)
        return
    ms_step, wall = time_step(cases, args.steps, args.warmup)
    for k in EXTRA:
        time_alone(cases[k])
    host_us = {k: time_host(cases[k]) for k in HOST_TIMED}
    copy = copy_bandwidth(dev)

    def summary(k):
        c = cases[k]
        avg = statistics.fmean(c.ms)
        med = statistics.median(c.ms)
        peak = {"hbm": HBM_PEAK_GBS, "mfma": MFMA_BF16_PEAK_TFLOPS, "pcie": PCIE_PEAK_GBS}[c.kind]
        r = c.rate(avg)
        d = {"call": c.name, "avg_ms": round(avg, 5), "median_ms": round(med, 5), "work": c.work,
             "rate": round(r, 2), "unit": c.unit, "frac_of_peak": round(r / peak, 4),
             "hbm_traffic_bytes": measured_traffic(k)}
        for label, count in c.tokens.items():
            d[label] = round(count / (avg * 1e-3), 1)
        if k in host_us:
            d["host_inclusive_us"] = round(host_us[k], 2)
        return d

    per = {k: summary(k) for k in STEP + EXTRA}
    dec_ms = sum(statistics.fmean(cases[k].ms) for k in ("decode3", "decode4"))
    dec_bytes = cases["decode3"].work + cases["decode4"].work
    value = dec_bytes / (dec_ms * 1e-3) / 1e9
    pre = per["ragged2"]
    # dominant call of the step (largest share of the step time)
    dom = max(STEP, key=lambda k: statistics.fmean(cases[k].ms))
    dc = cases[dom]
    dpeak = HBM_PEAK_GBS if dc.kind == "hbm" else MFMA_BF16_PEAK_TFLOPS
    dach = dc.rate(statistics.fmean(dc.ms))
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, shuffled block pools; no dataset)",
        "config": {
            "workload": "paged-KV attention hot path per step: scatter + chunked paged prefill (16 req, "
                        "prefix U[0,4096], chunk U[64,1024], 16/4 heads, hd 256); ragged causal prefill (8 req, "
                        "U[128,2048], 32/8 heads, hd 128); batched paged decode (B=64, U[512,8192], 32/8 heads, "
                        "hd 128); long-context split decode (B=4, 131072, 64/8 heads, hd 128)",
            "global_batch": 64 + 4,
            "block_size": 16,
            "partition_tokens": 512,
            "parallelism": "none (1 GPU)",
        },
        "decode_hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "prefill": {"value": pre["rate"], "unit": "TFLOP/s", "frac": pre["frac_of_peak"],
                    "workload": "ragged causal prefill, 8 requests U[128,2048], 32/8 heads, hd 128"},
        "roofline": {"bound": "hbm" if dc.kind == "hbm" else "mfma", "kernel": dc.name,
                     "achieved": round(dach, 2), "peak": dpeak,
                     "unit": "GB/s" if dc.kind == "hbm" else "TFLOP/s", "frac": round(dach / dpeak, 4),
                     "traffic": measured_traffic(dom)},
        "tokens_per_s": {k: {t: v for t, v in per[k].items() if t.endswith("_per_s")} for k in STEP},
        "copy_1gib": copy,
        "decode_plans": {k: meta[k] for k in ("plan3", "plan4")},
        "context": {"pages_engine_prefill_tok_s": 3880, "hardware": "NVIDIA GB10 (sm_121)",
                    "note": "whole-engine prefill rate of an unnamed model quoted on the Atlas flashinfer page; "
                            "not comparable with a single attention kernel, not a target"},
        "per_call": per,
        "wall_s_timed": round(wall, 4),
    }
    line["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(meta)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
