#!/usr/bin/env python3
"""Benchmark of latent-cache decode (weight-absorbed MLA / TPLA) on one MI355X.

One step = one decode call through the C ABI over one batch of the workload (the
query rotation when the cache is Hadamard-rotated, the split-K decode kernel and the
log-sum-exp merge / shard sum), with the cache, block table and queries resident in
HBM.  Before every step, timed or not, a 1 GiB buffer is read so that no part of
the cache survives in the 256 MB last-level cache: the figures are HBM figures.
Steps are timed with HIP events on the call's stream around the whole call; the
split-K decode kernel is then timed alone, over as many further steps, with events
the library records around it on the same stream.

Cache eviction reads a 1 GiB buffer (a reduction with a scalar result): reading leaves only
clean lines behind, whereas overwriting a buffer would leave up to 256 MB of dirty lines whose
write-back then competes with the timed kernel's reads.

Prints ONE JSON line.  The headline workload is the paged TPLA decode with the Hadamard
reparameterisation (G = 2, batch 64, 128 heads, latent 512 + rope 64, 64-token pages with a
random block table, contexts uniform in [1024, 65536], bf16), the largest configuration of the
metric that fits one GPU and the one whose contexts reach the 32K regime the pages quote their
speedups at.  Its "roofline" object prices the split-K decode kernel's time against the HBM peak
with the algorithmic bytes (every cache element read once), and its "cpu_baseline" times the fp64
oracle on a bounded sample of the same sequences on the host cores; that leg also reports the
error of the timed output against the oracle on the sampled sequences.  The other workloads
(exact MLA at 4K context, TPLA G = 2 and G = 4 at 32K context) are reported in "workloads"
unless --headline-only is given, each with its own roofline object and oracle sample, and the
tiny fp32 case as call latency; the contiguous TPLA workloads also carry "per_device_share":
the call of one shard (what one of G devices would read and compute) and the G = 1 call over the
same cache.  "append" times latent_cache_append on its own on the paged Hadamard workload's rows:
the whole cache and one row per sequence, rotated and plain (and rotated with a per-shard RMS
norm); "value_up_projection" times the value up-projection that follows the decode
(DeepSeek-V3 shapes, bf16 weights); "projected_decode" (headline workload, and the 4K MLA one)
the decode with that projection fused into its merge against the two calls; "context_merge" the log-sum-exp merge of four decode results
over disjoint context parts (exact MLA shapes at 4K context); "prefill" the absorbed MLA prefill
of a chunked-prefill step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time
import types

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
METRIC = "latent-cache decode tokens/s and achieved HBM GB/s (% of peak), 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
# the decode kernel's sources: its file and the LDS-DMA helpers it includes
KERNEL_SRCS = [os.path.join(ROOT, "mla_latent_kv_13_amd", "csrc", f) for f in ("decode_mfma.hip", "lds_dma.h")] + [
    os.path.join(ROOT, "mla_latent_kv_13_amd", "build.py")]  # the compiler flags shape the kernel too


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=60,
                   help="untimed steps first (a process's decode kernels run slower over its first ~50 calls as the card settles)")
    p.add_argument("--config", type=int, default=5, choices=[2, 3, 4, 5], help="headline workload")
    p.add_argument("--shard-count", type=int, default=0,
                   help="headline call computes shards [0, n) only (0 = all): n = 1 is one device's share")
    p.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    p.add_argument("--extra-steps", type=int, default=10, help="timed steps of each other workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--chunk-tokens", type=int, default=0)
    p.add_argument("--no-flush", action="store_true", help="do not evict the last-level cache between steps")
    p.add_argument("--extras-only", action="store_true",
                   help="only the calls beside the decode: the append (paged Hadamard workload), the value "
                        "up-projection and the context merge")
    p.add_argument("--prefill-only", action="store_true",
                   help="only the absorbed MLA prefill step (4 sequences x 1024 new tokens of 4096 cached)")
    p.add_argument("--projected-only", action="store_true",
                   help="only the decode with the fused value up-projection against the two calls, on the "
                        "workload --config names")
    p.add_argument("--calibration-copy", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy three times (to scale HBM byte counters)")
    return p.parse_args()


def calibration_copy():
    """A plain copy of known size: each launch reads and writes exactly 1 GiB, so the byte
    counters a profiler reports for it give the scale factor of those counters."""
    import torch

    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_read": n, "calibration_copy_bytes_written": n, "launches": 3}))


class Workload:
    """Device-resident inputs of one seeded workload plus preallocated outputs and workspace."""

    def __init__(self, cfg: int, chunk_tokens: int = 0, shard_count: int = 0):
        import numpy as np
        import torch

        from mla_latent_kv_13_amd import binding, inputs

        self.cfg = cfg
        t0 = time.time()
        case = inputs.make_config(cfg)
        self.case = case
        dev = "cuda:0"

        def dev_t(a):
            if case.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

        self.desc = binding.Desc(case.dtype, case.d_latent, case.d_rope, case.page_size, case.num_pages,
                                 case.max_pages_per_seq, case.transform)
        self.q_lat = dev_t(case.q_lat)
        self.q_rope = dev_t(case.q_rope)
        self.seq_lens = torch.from_numpy(case.seq_lens).to(dev)
        self.block_table = None if case.block_table is None else torch.from_numpy(case.block_table).to(dev)
        if case.transform == "identity":
            self.pool = dev_t(case.pool)
        else:
            self.pool = dev_t(case.empty_pool())
            rows = dev_t(case.rows)
            slots = torch.from_numpy(case.slots).to(dev)
            binding.latent_cache_append(self.desc, self.pool, rows, slots)
            torch.cuda.synchronize()
            del rows, slots
        self.chunk_tokens = chunk_tokens
        self.shard_count = shard_count if shard_count > 0 else case.shards
        B, H = case.batch, case.heads
        self.out = torch.empty((B, H, case.d_latent), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, self.shard_count, H), dtype=torch.float32, device=dev)
        need = binding.workspace_size(self.desc, B, H, case.shards, self.shard_count, case.max_seq_len, chunk_tokens)
        self.workspace = binding.alloc_workspace(need, dev)
        self.tokens = case.total_tokens
        elem = 2 if case.dtype == "bf16" else 4
        # algorithmic bytes: every element of the shards' columns and the rope key read once
        width = self.shard_count * (case.d_latent // case.shards) + case.d_rope
        self.bytes = self.tokens * width * elem
        self.binding = binding
        log(f"workload {cfg} ({case.name}): {self.tokens} cached tokens, {self.bytes / 1e6:.1f} MB, "
            f"prepared in {time.time() - t0:.1f}s")

    def call(self, events=None):
        c = self.case
        self.binding.tpla_decode_sharded(self.desc, self.pool, self.block_table, self.seq_lens, self.q_lat,
                                         self.q_rope, c.scale, c.shards, c.max_seq_len, shard_begin=0,
                                         shard_count=self.shard_count, out=self.out, lse=self.lse,
                                         workspace=self.workspace, chunk_tokens=self.chunk_tokens, events=events)

    def config(self):
        c = self.case
        d = {"workload": c.name, "batch": c.batch, "heads": c.heads, "d_latent": c.d_latent, "d_rope": c.d_rope,
             "shards": c.shards, "dtype": c.dtype, "transform": c.transform,
             "layout": "paged" if c.paged else "contiguous", "cached_tokens": self.tokens}
        if self.shard_count != c.shards:
            d["shards_computed"] = [0, self.shard_count]
        if c.paged:
            d.update(page_size=c.page_size, context="uniform[1024,65536]", max_seq_len=c.max_seq_len)
        else:
            d.update(context=c.max_seq_len)
        return d


_FLUSH = []


def _flush_buffer():
    """A 1 GiB device buffer whose full read evicts the 256 MB last-level cache; allocated once."""
    import torch

    if not _FLUSH:
        _FLUSH.append(torch.zeros(1 << 28, dtype=torch.float32, device="cuda:0"))
    return _FLUSH[0]


def time_workload(w: Workload, steps: int, warmup: int, flush: bool):
    """Time `steps` whole calls (events around the call only), then the split-K decode kernel
    alone in `steps` further calls (events the library records around that kernel).  Event
    markers inside a call cost it several microseconds, so the two are measured apart."""
    import torch

    flush_buf = _flush_buffer() if flush else None

    def evict():
        if flush_buf is not None:
            flush_buf.sum()

    for _ in range(warmup):
        evict()
        w.call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev + kev:  # materialise the events outside the timed steps
        e[0].record()
        e[1].record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evict()
        ev[i][0].record()
        w.call()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for i in range(steps):
        evict()
        w.call(events=(kev[i][0], kev[i][1]))
    torch.cuda.synchronize()
    call_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[0].elapsed_time(e[1]) for e in kev]
    # the same call captured once in a HIP graph and replayed (how a serving loop would issue it)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        w.call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        w.call()
    # warm-up replays first: the host-side pause of the capture lets the card's clocks drop, and
    # the kernels then run slower for about twenty launches, as at the start of the process
    for _ in range(warmup):
        evict()
        graph.replay()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        evict()
        gev[i][0].record()
        graph.replay()
        gev[i][1].record()
    torch.cuda.synchronize()
    graph_ms = [e[0].elapsed_time(e[1]) for e in gev]
    del graph
    mean_call = statistics.fmean(call_ms)
    mean_dec = statistics.fmean(dec_ms)
    return {
        "call_ms_mean": mean_call, "call_ms_median": statistics.median(call_ms), "call_ms_min": min(call_ms),
        "decode_kernel_ms_mean": mean_dec, "decode_kernel_ms_min": min(dec_ms),
        "tokens_per_s": w.tokens / (mean_call * 1e-3),
        "query_tokens_per_s": w.case.batch / (mean_call * 1e-3),
        "call_gbs": w.bytes / (mean_call * 1e-3) / 1e9,
        "decode_kernel_gbs": w.bytes / (mean_dec * 1e-3) / 1e9,
        "graph_replay_ms_mean": statistics.fmean(graph_ms), "graph_replay_ms_median": statistics.median(graph_ms),
        "wall_s_with_flush": wall,
    }


def time_shard_calls(w: Workload, steps: int, warmup: int, flush: bool):
    """The one-GPU view of TPLA's device split on a contiguous workload: the call of a single
    shard (shard_begin = 0, shard_count = 1: the latent slice plus the rope, (w + d_r) * 2 bytes
    per token, what one device of G would read) and the G = 1 call (exact MLA, all 576 values
    per token) over the same cache, each timed like the full call (events around the call)."""
    import torch

    c = w.case
    binding = w.binding
    B, H = c.batch, c.heads
    flush_buf = _flush_buffer() if flush else None
    res = {}
    for name, num_shards in (("one_shard_of_g", c.shards), ("g1_same_cache", 1)):
        need = binding.workspace_size(w.desc, B, H, num_shards, 1, c.max_seq_len)
        ws = binding.alloc_workspace(need, "cuda:0")
        out = torch.empty((B, H, c.d_latent), dtype=torch.float32, device="cuda:0")
        lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda:0")

        def call():
            binding.tpla_decode_sharded(w.desc, w.pool, w.block_table, w.seq_lens, w.q_lat, w.q_rope, c.scale,
                                        num_shards, c.max_seq_len, shard_begin=0, shard_count=1, out=out, lse=lse,
                                        workspace=ws)

        for _ in range(warmup):
            if flush_buf is not None:
                flush_buf.sum()
            call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            if flush_buf is not None:
                flush_buf.sum()
            ev[i][0].record()
            call()
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
        width = c.d_latent // num_shards + c.d_rope
        nbytes = w.tokens * width * (2 if c.dtype == "bf16" else 4)
        res[name] = {"shards": num_shards, "values_per_token": width, "call_ms_mean": ms,
                     "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9}
        del ws, out, lse
    return res


def time_append(w: Workload, steps: int, warmup: int, flush: bool):
    """latent_cache_append timed on its own (events around each call) on the rows of a workload:
    the whole cache at once (as after a prefill) and one row per sequence (one decode step), with
    the workload's transform and, into a second pool, without rotation.  Re-appending a row at its
    own slot stores the value it already holds, so the decode inputs stay as they were.
    Algorithmic bytes: each row read once and written once."""
    import numpy as np
    import torch

    c = w.case
    binding = w.binding
    dev = "cuda:0"
    flush_buf = _flush_buffer() if flush else None
    elem = 2 if c.dtype == "bf16" else 4
    row_bytes = (c.d_latent + c.d_rope) * elem
    if c.dtype == "bf16":
        rows = torch.from_numpy(np.ascontiguousarray(c.rows).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        rows = torch.from_numpy(np.ascontiguousarray(c.rows, dtype=np.float32)).to(dev)
    slots = torch.from_numpy(c.slots).to(dev)
    ends = np.cumsum(c.seq_lens.astype(np.int64))
    last = torch.from_numpy(ends[c.seq_lens > 0] - 1).to(dev)  # the newest row of each non-empty sequence
    step_rows, step_slots = rows[last].contiguous(), slots[last].contiguous()
    plain = binding.Desc(c.dtype, c.d_latent, c.d_rope, c.page_size, c.num_pages, c.max_pages_per_seq, "identity")
    scratch = torch.empty_like(w.pool)

    def timed(desc, pool, r, sl, n_steps, norm=0):
        def call():
            if norm:
                binding.latent_cache_append_normed(desc, pool, r, sl, norm, 1e-6)
            else:
                binding.latent_cache_append(desc, pool, r, sl)

        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_steps)]
        for e in ev:
            if flush_buf is not None:
                flush_buf.sum()
            e[0].record()
            call()
            e[1].record()
        torch.cuda.synchronize()
        ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
        n = int(r.shape[0])
        gbs = 2 * n * row_bytes / (ms * 1e-3) / 1e9
        return {"rows": n, "ms_mean": ms, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}

    res = {"workload": c.name, "row_bytes": row_bytes}
    for name, desc, pool in ((c.transform, w.desc, w.pool), ("identity_into_second_pool", plain, scratch)):
        if name == "identity_into_second_pool" and c.transform == "identity":
            continue
        res[name] = {"whole_cache": timed(desc, pool, rows, slots, max(3, steps // 3)),
                     "one_row_per_sequence": timed(desc, pool, step_rows, step_slots, steps)}
    # rotated and normalised per shard slice (into the second pool: the decode inputs stay as they were)
    rdesc = binding.Desc(c.dtype, c.d_latent, c.d_rope, c.page_size, c.num_pages, c.max_pages_per_seq, "wht")
    res["wht_rms_norm_per_shard_into_second_pool"] = {
        "norm_slices": c.shards, "whole_cache": timed(rdesc, scratch, rows, slots, max(3, steps // 3), c.shards)}
    del rows, slots, step_rows, step_slots, scratch
    torch.cuda.empty_cache()
    return res


def time_value_projection(steps: int, warmup: int, flush: bool, batch=32, heads=128, d_latent=512, d_v=128):
    """tpla_value_up_projection timed on its own (events around each call) at DeepSeek-V3 shapes
    (value width 128 per head) with seeded bf16 weights, against its algorithmic bytes: the
    weights once, the latent-frame output read once and the projected output written once."""
    import torch

    from mla_latent_kv_13_amd import binding, inputs

    o, w = inputs.make_value_projection(2, batch=batch, heads=heads, d_latent=d_latent, d_v=d_v)
    o_t = torch.from_numpy(o).to("cuda:0")
    w_t = torch.from_numpy(w.view("int16")).view(torch.bfloat16).to("cuda:0")
    out = torch.empty((batch, heads, d_v), dtype=torch.float32, device="cuda:0")
    flush_buf = _flush_buffer() if flush else None
    for _ in range(warmup):
        binding.tpla_value_up_projection(o_t, w_t, out_v=out)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        if flush_buf is not None:
            flush_buf.sum()
        e[0].record()
        binding.tpla_value_up_projection(o_t, w_t, out_v=out)
        e[1].record()
    torch.cuda.synchronize()
    ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
    nbytes = heads * d_v * d_latent * 2 + batch * heads * d_latent * 4 + batch * heads * d_v * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del o_t, w_t, out
    return {"shape": {"batch": batch, "heads": heads, "d_latent": d_latent, "d_v": d_v, "weights": "bf16"},
            "ms_mean": ms, "algorithmic_bytes": nbytes, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
            "bound": "hbm"}


def time_projected(w: Workload, steps: int, warmup: int, flush: bool, d_v: int = 128):
    """tpla_decode_sharded_projected -- the decode with the value up-projection fused into its
    merge, writing [B, H, d_v] -- against the unfused pair (tpla_decode_sharded, then
    tpla_value_up_projection) on the same workload with seeded bf16 weights of DeepSeek-V3's value
    width.  The two alternate step by step (the decode kernel's own time drifts with the card's
    clock over a run, and alternating exposes both to the same drift).  Each step is timed with
    events around the whole call; a second set of steps times what follows the split-K decode
    kernel (from the event the library records at its end to the end of the call: the fused merge,
    or the merge and the up-projection), the part the fusion changes.  Algorithmic bytes of the
    fused call: the cache once, the weights once and the projected output once."""
    import numpy as np
    import torch

    from mla_latent_kv_13_amd import inputs

    c, binding = w.case, w.binding
    B, H = c.batch, c.heads
    _, wuv = inputs.make_value_projection(40 + w.cfg, batch=1, heads=H, d_latent=c.d_latent, d_v=d_v)
    w_t = torch.from_numpy(wuv.view("int16")).view(torch.bfloat16).to("cuda:0")
    out_f = torch.empty((B, H, d_v), dtype=torch.float32, device="cuda:0")
    out_p = torch.empty_like(out_f)
    flush_buf = _flush_buffer() if flush else None

    def fused(events=None):
        binding.tpla_decode_sharded_projected(w.desc, w.pool, w.block_table, w.seq_lens, w.q_lat, w.q_rope, c.scale,
                                              c.shards, c.max_seq_len, w_t, shard_begin=0,
                                              shard_count=w.shard_count, out_v=out_f, lse=w.lse,
                                              workspace=w.workspace, chunk_tokens=w.chunk_tokens, events=events)

    def pair(events=None):
        w.call(events=events)
        binding.tpla_value_up_projection(w.out, w_t, out_v=out_p)

    fns = (("fused", fused), ("unfused_pair", pair))
    for _ in range(warmup):
        for _, fn in fns:
            if flush_buf is not None:
                flush_buf.sum()
            fn()
    torch.cuda.synchronize()
    call = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)] for n, _ in fns}
    tail = {n: [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)] for n, _ in fns}
    for i in range(steps):
        for n, fn in fns:
            if flush_buf is not None:
                flush_buf.sum()
            call[n][i][0].record()
            fn()
            call[n][i][1].record()
    for i in range(steps):
        for n, fn in fns:
            if flush_buf is not None:
                flush_buf.sum()
            e = tail[n][i]
            fn(events=(e[0], e[1]))
            e[2].record()
    torch.cuda.synchronize()
    ms = {n: [e[0].elapsed_time(e[1]) for e in call[n]] for n, _ in fns}
    after = {n: [e[1].elapsed_time(e[2]) * 1e3 for e in tail[n]] for n, _ in fns}
    a, b = out_f.cpu().numpy().astype(np.float64), out_p.cpu().numpy().astype(np.float64)
    diff = float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))
    nbytes = w.bytes + H * d_v * c.d_latent * 2 + B * H * d_v * 4
    f_ms, p_ms = statistics.fmean(ms["fused"]), statistics.fmean(ms["unfused_pair"])
    del w_t, out_f, out_p
    return {"workload": c.name, "d_v": d_v, "weights": "bf16",
            "fused_call_ms_mean": f_ms, "fused_call_ms_median": statistics.median(ms["fused"]),
            "unfused_pair_ms_mean": p_ms, "unfused_pair_ms_median": statistics.median(ms["unfused_pair"]),
            "after_decode_us_median": {n: statistics.median(v) for n, v in after.items()},
            "algorithmic_bytes": nbytes, "fused_gbs": nbytes / (f_ms * 1e-3) / 1e9,
            "fused_frac_of_peak": nbytes / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "max_abs_diff_vs_pair_rel_to_max": diff}


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (no sparsity)


def time_prefill(steps: int, warmup: int, flush: bool, batch=4, context=4096, new=1024, heads=128):
    """mla_prefill_absorbed on a chunked-prefill step: `batch` sequences of `context` cached tokens
    (paged 64-token pages, Hadamard-rotated cache, DeepSeek-V3 widths) whose last `new` tokens are
    the new prompt tokens, each attending causally to its prefix.  The call is timed with events
    around it, the split-K kernel alone with the events the library records around it.  Prefill is
    compute-bound: priced against the dense bf16 matrix peak with 2*H*(2*d_c + d_r) flops per
    (query row, visible token) pair (logits over [latent | rope] plus the latent-valued output)."""
    import numpy as np
    import torch

    from mla_latent_kv_13_amd import binding, inputs

    dev = "cuda:0"
    case = inputs.make_case(91, batch=batch, heads=heads, d_latent=512, d_rope=64, shards=1, lens=context,
                            paged=True, page_size=64, transform="wht", scale=1.0 / np.sqrt(192),
                            place_rows=False, name=f"prefill-mla-{batch}x{new}-of-{context}-bf16")

    def dev_t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    desc = binding.Desc(case.dtype, case.d_latent, case.d_rope, case.page_size, case.num_pages,
                        case.max_pages_per_seq, case.transform)
    pool = dev_t(case.empty_pool())
    binding.latent_cache_append(desc, pool, dev_t(case.rows), torch.from_numpy(case.slots).to(dev))
    qs, q_lat, q_rope = inputs.make_prefill_queries(92, new_tokens=[new] * batch, heads=heads, d_latent=512,
                                                    d_rope=64)
    query_start = torch.from_numpy(qs).to(dev)
    q_lat_t, q_rope_t = dev_t(q_lat), dev_t(q_rope)
    seq_lens = torch.from_numpy(case.seq_lens).to(dev)
    block_table = torch.from_numpy(case.block_table).to(dev)
    nq = int(qs[-1])
    out = torch.empty((nq, heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((nq, heads), dtype=torch.float32, device=dev)
    ws = binding.alloc_workspace(binding.prefill_workspace_size(desc, nq, heads, case.max_seq_len), dev)

    def call(events=None):
        binding.mla_prefill_absorbed(desc, pool, block_table, seq_lens, query_start, q_lat_t, q_rope_t, case.scale,
                                     case.max_seq_len, out=out, lse=lse, workspace=ws, events=events)

    flush_buf = _flush_buffer() if flush else None
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(2 * steps)]
    for i in range(2 * steps):
        if flush_buf is not None:
            flush_buf.sum()
        if i < steps:
            ev[i][0].record()
            call()
            ev[i][1].record()
        else:
            call(events=(ev[i][0], ev[i][1]))
    torch.cuda.synchronize()
    call_ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev[:steps])
    kern_ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev[steps:])
    pairs = sum(context - new + j + 1 for j in range(new)) * batch  # (query row, visible token) pairs
    flops = 2.0 * heads * (2 * 512 + 64) * pairs
    tflops_call = flops / (call_ms * 1e-3) / 1e12
    tflops_kernel = flops / (kern_ms * 1e-3) / 1e12
    del pool, out, lse, ws
    return {"shape": {"workload": case.name, "sequences": batch, "context": context, "new_tokens_per_sequence": new,
                      "heads": heads, "d_latent": 512, "d_rope": 64, "layout": "paged", "page_size": 64,
                      "transform": "wht", "dtype": "bf16"},
            "call_ms_mean": call_ms, "kernel_ms_mean": kern_ms, "flops": flops,
            "prompt_tokens_per_s": nq / (call_ms * 1e-3),
            "tflops_call": tflops_call, "tflops_kernel": tflops_kernel,
            "roofline": {"bound": "mfma", "achieved": tflops_kernel, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": tflops_kernel / MFMA_BF16_PEAK_TFLOPS}}


def time_context_merge(steps: int, warmup: int, flush: bool, parts=4, batch=32, heads=128, d_latent=512):
    """tpla_merge_context_parts timed on its own (events around each call): the results of `parts`
    decode calls over disjoint context parts at the headline shapes (G = 1), against its
    algorithmic bytes: every part's output and log-sum-exp read once, the result written once."""
    import torch

    from mla_latent_kv_13_amd import binding, inputs

    out_p, lse_p = inputs.make_context_parts(3, parts=parts, batch=batch, heads=heads, d_latent=d_latent,
                                             shard_count=1, empty=0.0)
    op = torch.from_numpy(out_p).to("cuda:0")
    lp = torch.from_numpy(lse_p).to("cuda:0")
    out = torch.empty((batch, heads, d_latent), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((batch, 1, heads), dtype=torch.float32, device="cuda:0")
    flush_buf = _flush_buffer() if flush else None
    for _ in range(warmup):
        binding.tpla_merge_context_parts(op, lp, 1, out=out, lse=lse)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        if flush_buf is not None:
            flush_buf.sum()
        e[0].record()
        binding.tpla_merge_context_parts(op, lp, 1, out=out, lse=lse)
        e[1].record()
    torch.cuda.synchronize()
    ms = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
    nbytes = (parts + 1) * batch * heads * d_latent * 4 + (parts + 1) * batch * heads * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del op, lp, out, lse
    return {"shape": {"parts": parts, "batch": batch, "heads": heads, "d_latent": d_latent, "shards": 1,
                      "shard_count": 1, "transform": "identity", "seed": 3, "empty_parts": 0.0},
            "ms_mean": ms, "algorithmic_bytes": nbytes, "gbs": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
            "bound": "hbm"}


def streaming_bandwidth(steps: int = 10):
    """What plain streaming reaches on this card with the runtime's own kernels: a
    device-to-device copy of 1 GiB (1 GiB read plus 1 GiB written), and a full reduction of a
    1 GiB buffer (1 GiB read), each timed with events around it.  Neither kernel is tuned for
    the card, so these are reference points, not ceilings."""
    import torch

    buf = _flush_buffer()
    buf.sum()
    torch.cuda.synchronize()
    rev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in rev:
        e[0].record()
        buf.sum()
        e[1].record()
    torch.cuda.synchronize()
    read_ms = statistics.median(e[0].elapsed_time(e[1]) for e in rev)
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        dst.copy_(src)
        e[1].record()
    torch.cuda.synchronize()
    ms = statistics.median(e[0].elapsed_time(e[1]) for e in ev)
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": 2 * n / (ms * 1e-3) / 1e9, "copy_ms_median": ms,
            "read_gbs": buf.numel() * 4 / (read_ms * 1e-3) / 1e9, "read_ms_median": read_ms,
            "what": "torch device-to-device copy of 1 GiB (read + write) and torch sum of 1 GiB (read)"}


def traffic_for_current_kernel(workload_name: str):
    """HBM bytes per decode-kernel launch from the committed counter summary, if it was taken
    on the kernel source as it stands now (else None)."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
        h = hashlib.sha256()
        for path in KERNEL_SRCS:
            with open(path, "rb") as fh:
                h.update(fh.read())
        digest = h.hexdigest()
    except (OSError, ValueError):
        return None
    entry = rec.get("workloads", {}).get(workload_name)
    if entry is None or rec.get("decode_kernel_sources_sha256") != digest:
        return None
    return entry.get("hbm_bytes_per_launch")


def roofline_of(w: "Workload", res: dict) -> dict:
    """Roofline object of the split-K decode kernel of one workload: algorithmic bytes per launch
    (every cache element of the computed shards' columns and the rope key once) over the kernel's
    mean time between the events the library records around it, against the HBM peak; traffic =
    HBM bytes per launch from the committed counter summary when it was taken on this kernel."""
    gbs = w.bytes / (res["decode_kernel_ms_mean"] * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic_for_current_kernel(w.case.name) if w.shard_count == w.case.shards else None,
            "kernel": "split-K decode kernel (decode_mfma_kernel)", "algorithmic_bytes_per_launch": w.bytes,
            "kernel_ms_mean": res["decode_kernel_ms_mean"]}


def cpu_baseline(c, gpu_out=None, gpu_lse=None, shard_count=None, budget_s: float = 15.0, one_core_s: float = 0.0):
    """The fp64 oracle on the host cores, on whole sequences of a workload in a fixed seeded order,
    until about budget_s of decode computation (and, with one_core_s, the same with BLAS held to
    one thread, a per-core figure).  Each sequence's oracle cache is built from the raw rows before
    its timed decode (the rotated cache by the oracle's own append), so only the decode is timed.
    The oracle's outputs of the sampled sequences are compared with the GPU's timed output:
    relative L2 and max-abs errors over those sequences, against the bf16 bar of 2e-2 (1e-5 for
    fp32)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from mla_latent_kv_13_amd import inputs

    shard_count = shard_count or c.shards
    starts = np.concatenate([[0], np.cumsum(c.seq_lens.astype(np.int64))])
    q_lat = inputs.stored_to_f64(c.q_lat, c.dtype)
    q_rope = inputs.stored_to_f64(c.q_rope, c.dtype)
    order = [int(b) for b in np.random.default_rng([int(c.meta.get("seed", 0)), 99]).permutation(c.batch)
             if c.seq_lens[b] > 0]
    cache, cached_bytes = {}, [0]

    def prepared(b):
        if b in cache:
            return cache[b]
        r = inputs.stored_to_f64(c.rows[starts[b]:starts[b + 1]], c.dtype)
        pool = np.full((1, r.shape[0], c.width), np.nan)
        if c.transform == "identity":
            pool[0] = r
        else:
            pool = oracle.latent_cache_append(pool, r, np.arange(r.shape[0]), c.d_latent, c.transform, c.dtype)
        if cached_bytes[0] + pool.nbytes <= (2 << 30):
            cache[b] = pool
            cached_bytes[0] += pool.nbytes
        return pool

    def run(budget):
        done, spent, n, k, outs = 0, 0.0, 0, 0, {}
        while spent < budget or n == 0:
            b = order[k % len(order)]
            pool = prepared(b)
            t0 = time.perf_counter()
            o, l = oracle.tpla_decode_sharded(pool, None, c.seq_lens[b:b + 1], q_lat[b:b + 1], q_rope[b:b + 1],
                                              float(np.float32(c.scale)), c.shards, 0, shard_count,
                                              transform=c.transform)
            spent += time.perf_counter() - t0
            done += int(c.seq_lens[b])
            n += 1
            k += 1
            outs.setdefault(b, (o[0], l[0]))
        return done, spent, n, outs

    done, spent, n, outs = run(budget_s)
    threads = int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))
    res = {"value": done / spent, "unit": "cache-tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{n} whole-sequence decodes ({done} cached tokens, {len(outs)} distinct sequences) of the "
                     f"{c.name} workload, fp64 NumPy oracle, {spent:.1f}s of decode; oracle caches built from the "
                     f"raw rows outside the timing; host has {len(os.sched_getaffinity(0))} usable cores"}
    if one_core_s > 0:
        with threadpool_limits(limits=1):
            d1, s1, n1, _ = run(one_core_s)
        res["one_core"] = {"value": d1 / s1, "unit": "cache-tokens/s", "cores": 1,
                           "sample": f"{n1} whole-sequence decodes ({d1} cached tokens), {s1:.1f}s"}
    if gpu_out is not None:
        seqs = sorted(outs)
        ref = np.stack([outs[b][0] for b in seqs])
        ref_lse = np.stack([outs[b][1] for b in seqs])
        got = np.asarray(gpu_out, dtype=np.float64)[seqs]
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        mx = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
        tol = 2e-2 if c.dtype == "bf16" else 1e-5
        par = {"sequences": seqs, "rel_l2": rel, "max_abs_over_max_ref": mx, "tolerance": tol,
               "pass": bool(np.all(np.isfinite(got)) and rel <= tol and mx <= tol)}
        if gpu_lse is not None:
            gl = np.asarray(gpu_lse, dtype=np.float64)[seqs]
            fin = np.isfinite(ref_lse)
            par["lse_max_err_rel"] = float(np.max(np.abs(gl[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))))
        res["parity_of_timed_output"] = par
    return res


def cpu_baseline_extras(line, append_case=None, budget_s: float = 2.0):
    """The fp64 oracle timed beside each call the bench times besides the decode (the value
    up-projection, the context merge, the append and the prefill), each on a bounded sample of
    the same seeded inputs for about budget_s, scaled to the whole call; set-up (input generation,
    the rotated cache of the prefill sample) is not timed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from mla_latent_kv_13_amd import inputs

    threads = int(max([d.get("num_threads", 1) for d in threadpool_info()] or [1]))

    def timed(fn, sample, total, unit, what):
        runs, spent = 0, 0.0
        while spent < budget_s or runs == 0:
            t0 = time.perf_counter()
            fn()
            spent += time.perf_counter() - t0
            runs += 1
        ms = spent / runs * total / sample * 1e3
        return {"ms_whole_call": ms, "kind": "oracle", "cores": threads,
                "sample": f"{what}: {sample} of {total} {unit} per run, {runs} runs, {spent:.1f}s, scaled to the whole call"}

    if "value_up_projection" in line:
        sh = line["value_up_projection"]["shape"]
        o, w = inputs.make_value_projection(2, batch=sh["batch"], heads=sh["heads"], d_latent=sh["d_latent"], d_v=sh["d_v"])
        o64, w64 = o.astype(np.float64), inputs.stored_to_f64(w, "bf16")
        n = sh["batch"] * sh["heads"]
        line["value_up_projection"]["cpu_baseline"] = timed(lambda: oracle.value_up_projection(o64, w64), n, n,
                                                            "(sequence, head) rows", "the whole call")
    if "context_merge" in line:
        sh = line["context_merge"]["shape"]
        op, lp = inputs.make_context_parts(sh["seed"], parts=sh["parts"], batch=sh["batch"], heads=sh["heads"],
                                           d_latent=sh["d_latent"], shard_count=sh["shard_count"], empty=sh["empty_parts"])
        k = min(4, sh["batch"])
        line["context_merge"]["cpu_baseline"] = timed(
            lambda: oracle.merge_context_parts(op[:, :k], lp[:, :k], sh["shards"], 0, sh["shard_count"],
                                               transform=sh["transform"]), k, sh["batch"], "sequences", "merge")
    if "append" in line and append_case is not None:
        c = append_case
        rows = inputs.stored_to_f64(c.rows, c.dtype)
        n = rows.shape[0]
        target = np.full((1, n, c.width), np.nan)
        line["append"]["cpu_baseline"] = timed(
            lambda: oracle.latent_cache_append(target, rows, np.arange(n), c.d_latent, c.transform, c.dtype),
            n, c.total_rows, "rows", f"rotated append of {c.name}")
    if "prefill" in line:
        sh = line["prefill"]["shape"]
        case = inputs.make_case(91, batch=sh["sequences"], heads=sh["heads"], d_latent=sh["d_latent"], d_rope=sh["d_rope"],
                                shards=1, lens=sh["context"], paged=True, page_size=sh["page_size"],
                                transform=sh["transform"], scale=1.0 / np.sqrt(192), place_rows=False)
        qs, q_lat, q_rope = inputs.make_prefill_queries(92, new_tokens=[sh["new_tokens_per_sequence"]] * sh["sequences"],
                                                        heads=sh["heads"], d_latent=sh["d_latent"], d_rope=sh["d_rope"])
        T = sh["context"]
        raw = inputs.stored_to_f64(case.rows[:T], case.dtype)  # sequence 0, rotated once (set-up)
        pool = oracle.latent_cache_append(np.full((1, T, case.width), np.nan), raw, np.arange(T), case.d_latent,
                                          case.transform, case.dtype)
        picks = np.linspace(0, sh["new_tokens_per_sequence"] - 1, 8).astype(int)
        ql, qr = inputs.stored_to_f64(q_lat[picks], "bf16"), inputs.stored_to_f64(q_rope[picks], "bf16")
        vis = [T - sh["new_tokens_per_sequence"] + int(j) + 1 for j in picks]

        def rows_sample():
            for i in range(len(picks)):
                oracle.mla_prefill_absorbed(pool, None, [vis[i]], [0, 1], ql[i:i + 1], qr[i:i + 1], case.scale,
                                            transform=case.transform)

        line["prefill"]["cpu_baseline"] = timed(rows_sample, len(picks), int(qs[-1]), "query rows",
                                                "prefill rows spread over sequence 0's new tokens")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        log("bench.py measures the single-GPU hot path; runs on several GPUs are not supported")
        sys.exit(2)
    if args.calibration_copy:
        calibration_copy()
        return
    import torch

    from mla_latent_kv_13_amd import binding

    binding.load_library()
    torch.cuda.init()
    if args.projected_only:
        w = Workload(args.config, args.chunk_tokens, args.shard_count)
        print(json.dumps({"projected_decode": time_projected(w, args.extra_steps, args.warmup, not args.no_flush)}),
              flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": time_prefill(args.extra_steps, args.warmup, not args.no_flush)}), flush=True)
        return
    if args.extras_only:
        w = Workload(5, args.chunk_tokens)
        extras = {"append": time_append(w, args.extra_steps, args.warmup, not args.no_flush)}
        del w
        torch.cuda.empty_cache()
        extras["value_up_projection"] = time_value_projection(args.extra_steps, args.warmup, not args.no_flush)
        extras["context_merge"] = time_context_merge(args.extra_steps, args.warmup, not args.no_flush)
        extras["prefill"] = time_prefill(args.extra_steps, args.warmup, not args.no_flush)
        print(json.dumps(extras), flush=True)
        return
    head = Workload(args.config, args.chunk_tokens, args.shard_count)
    res = time_workload(head, args.steps, args.warmup, not args.no_flush)
    log(f"headline: {json.dumps(res)}")
    line = {
        "metric": METRIC,
        "value": res["tokens_per_s"],
        "unit": "cache-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["call_ms_mean"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.case.dtype,
        "data": "synthetic (seeded N(0,1) queries and cache rows of the workload's shapes)",
        "config": head.config(),
        "hbm_gbs": res["call_gbs"],
        "hbm_frac_of_peak": res["call_gbs"] / HBM_PEAK_GBS,
        "roofline": roofline_of(head, res),
        "timing": res,
    }
    head_case, head_shards = head.case, head.shard_count
    head_out, head_lse = head.out.cpu().numpy(), head.lse.cpu().numpy()
    if not args.headline_only:
        line["projected_decode"] = time_projected(head, args.extra_steps, args.warmup, not args.no_flush)
        log(f"projected decode: {json.dumps(line['projected_decode'])}")
    append_case = None
    del head
    torch.cuda.empty_cache()
    extra_cpu = {}
    if not args.headline_only:
        others = {}
        for cfg in (1, 2, 3, 4, 5):
            if cfg == args.config:
                continue
            w = Workload(cfg, args.chunk_tokens)
            if cfg == 1:
                # launch-bound: call latency, no cache eviction (the whole cache is 40 KB)
                r = time_workload(w, args.extra_steps * 3, args.warmup, False)
                others[w.case.name] = {"config": w.config(), "call_us_mean": r["call_ms_mean"] * 1e3,
                                       "call_us_median": r["call_ms_median"] * 1e3, "call_us_min": r["call_ms_min"] * 1e3,
                                       "graph_replay_us_median": r["graph_replay_ms_median"] * 1e3,
                                       "what": "latency of one call (tiny fp32 TPLA decode), launch-bound"}
            else:
                r = time_workload(w, args.extra_steps, args.warmup, not args.no_flush)
                others[w.case.name] = {"config": w.config(), "tokens_per_s": r["tokens_per_s"],
                                       "query_tokens_per_s": r["query_tokens_per_s"],
                                       "call_ms_mean": r["call_ms_mean"], "hbm_gbs": r["call_gbs"],
                                       "hbm_frac_of_peak": r["call_gbs"] / HBM_PEAK_GBS,
                                       "roofline": roofline_of(w, r)}
            extra_cpu[w.case.name] = (w.case, w.out.cpu().numpy(), w.lse.cpu().numpy())
            if cfg == 2:
                others[w.case.name]["projected_decode"] = time_projected(w, args.extra_steps, args.warmup,
                                                                         not args.no_flush)
            if w.case.shards > 1 and not w.case.paged and cfg != 1:
                others[w.case.name]["per_device_share"] = time_shard_calls(w, args.extra_steps, args.warmup,
                                                                           not args.no_flush)
            if w.case.transform != "identity" and w.case.paged:
                line["append"] = time_append(w, args.extra_steps, args.warmup, not args.no_flush)
            log(f"workload {cfg}: {json.dumps(others[w.case.name])}")
            del w
            torch.cuda.empty_cache()
        line["workloads"] = others
    if not args.headline_only and "append" not in line and head_case.transform != "identity":
        w = Workload(args.config, args.chunk_tokens)
        line["append"] = time_append(w, args.extra_steps, args.warmup, not args.no_flush)
        del w
        torch.cuda.empty_cache()
    if "append" in line:
        # the oracle's append is timed on a sample of the rows the append was timed on
        src = head_case if (head_case.paged and head_case.transform != "identity") else next(
            (cc for cc, _, _ in extra_cpu.values() if cc.paged and cc.transform != "identity"), None)
        if src is not None:
            append_case = types.SimpleNamespace(rows=src.rows[:2000].copy(), total_rows=int(src.rows.shape[0]),
                                                d_latent=src.d_latent, width=src.width, transform=src.transform,
                                                dtype=src.dtype, name=src.name)
    if not args.headline_only:
        line["value_up_projection"] = time_value_projection(args.extra_steps, args.warmup, not args.no_flush)
        line["context_merge"] = time_context_merge(args.extra_steps, args.warmup, not args.no_flush)
        line["prefill"] = time_prefill(args.extra_steps, args.warmup, not args.no_flush)
        log(f"prefill: {json.dumps(line['prefill'])}")
        line["achievable_streaming"] = streaming_bandwidth()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(head_case, head_out, head_lse, head_shards, budget_s=10.0, one_core_s=2.0)
        log(f"cpu_baseline: {json.dumps(line['cpu_baseline'])}")
        for name, (c, out, lse) in extra_cpu.items():
            line["workloads"][name]["cpu_baseline"] = cpu_baseline(c, out, lse, budget_s=1.0 if c.batch == 1 else 3.0)
        if not args.headline_only:
            cpu_baseline_extras(line, append_case=append_case)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
