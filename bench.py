#!/usr/bin/env python3
"""Benchmark of the paged, variable-length attention path on one MI355X.

A step is one pass of the whole path over one synthetic batch: cu_seqlens packing and the
load-sorted task table on the host (C++), the table's copy to the device, reshape_and_cache of
the step's new K/V, the attention launch (decode splits and/or prefill tiles) and the split
combine. Inputs are resident in HBM before timing starts; the host table build of step k+1
overlaps the GPU work of step k (two table slots, reused only after their event completes).

Headline (`value`): decode KV GB/s on the 64-sequence MHA decode batch (Hq = Hkv = 32, D 128,
16-token blocks, contexts U[128, 4096]): algorithmic bytes per step (every visible K/V row, q,
out, the block-table entries read) over the measured step time. Secondary workloads in the same
JSON line: GQA decode at block sizes 16 and 64, the packed varlen causal prefill (TFLOP/s) and
the mixed unified step (both). `roofline` covers the attention launch of the headline workload,
timed with HIP events on the launch stream, with L2/MALL evicted (a 1 GiB read) between launches.
The fp64 oracle is timed on this host's cores on a bounded sample: whole sequences of the
headline batch (`cpu_baseline`, GB/s) and sampled query rows of the prefill and mixed workloads
(their `cpu_baseline` entries, GFLOP/s). `context_sweep` runs the headline batch's shape at one
context per run (256 .. 16384 keys) and fits launch time against context length.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--only] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "decode KV GB/s (% of HBM peak) + prefill TFLOP/s (% of MFMA peak)"
HEADLINE = "decode_mha_bf16"
SECONDARY = ["decode_gqa_bf16_bs16", "decode_gqa_bf16_bs64", "prefill_varlen_bf16", "mixed_bf16",
             "verify_gqa_bf16", "verify_gqa_bf16:as_prefill_tiles", "decode_mha_fp8",
             "verify_gqa_fp8", "prefill_varlen_fp8", "mixed_fp8",
             "decode_shared_mha_bf16", "decode_shared_mha_bf16:no_sharing",
             "gemm_linear_prefill_qproj", "gemm_linear_mixed_oproj", "gemm_linear_1024x1024x1024",
             "gemm_linear_512x2048x1024", "gemm_linear_2048x512x2048"]
# Split sizes per workload, from a sweep on MI355X (decode: 512 .. 32768 keys; mixed: key
# splits of 4096 .. 32768 and none for prefill tiles). Larger decode splits amortise each task's
# query load, four-wave merge and partial write; the load-sorted table keeps the tail short. The
# MHA batches (contexts up to 4096) run unsplit: one task per sequence and head, writing `out`
# directly, with no partial rows and no combine.
TILING = {
    "decode_mha_bf16": dict(dec_split=4096),
    "decode_gqa_bf16_bs16": dict(dec_split=8192),
    "decode_gqa_bf16_bs64": dict(dec_split=8192),
    "prefill_varlen_bf16": dict(pf_q_tile=128, pf_kv_split=0),
    "mixed_bf16": dict(dec_split=4096, pf_q_tile=128, pf_kv_split=0),
    # 4-row drafts: verify tasks (one task reads each KV page once for 4 rows x 4 heads), and
    # for comparison the same batch decomposed into prefill tiles (one per query head)
    "verify_gqa_bf16": dict(dec_split=16384, verify_rows=4),
    "verify_gqa_bf16:as_prefill_tiles": dict(pf_q_tile=128, pf_kv_split=0, verify_rows=0),
    # the MHA decode batch over fp8 pages (half the KV bytes of the bf16 headline), and the
    # verify batch over fp8 pages
    "decode_mha_fp8": dict(dec_split=4096),
    "verify_gqa_fp8": dict(dec_split=32768, verify_rows=4),
    # the prefill batch and the mixed step over fp8 pages, through the unified fp8 launch
    "prefill_varlen_fp8": dict(pf_q_tile=128, pf_kv_split=0),
    "mixed_fp8": dict(dec_split=4096, pf_q_tile=128, pf_kv_split=0),
    # 8 prompts x 16 decoding requests that alias the prompt's blocks: the prefix is read once
    # per group and kv head; the variant runs the same batch without grouping
    "decode_shared_mha_bf16": dict(dec_split=4096, shared_min=64),
    "decode_shared_mha_bf16:no_sharing": dict(dec_split=1024),
}
# SmoothGEMM (C = A W^T, bf16, fp32 accumulation) on Linear shapes: the pages' own Linear table
# shapes and the q / o projections of this step's batches (synth.GEMM_SHAPES). Tiles per shape
# from a sweep on MI355X: 256-wide where there are enough of them to fill the chip, 128-wide
# where the product is small; in both, the blocks of the last partial round of 256 resident
# workgroups are cut into K pieces (tail_split), which also gives the small products their K
# pieces (256 or 512 deep).
GEMM_TILING = {
    "gemm_linear_prefill_qproj": dict(tile=256, k_split=0, tail_split=True),
    "gemm_linear_mixed_oproj": dict(tile=256, k_split=0, tail_split=True),
    "gemm_linear_1024x1024x1024": dict(tile=128, k_split=0, tail_split=True),
    "gemm_linear_512x2048x1024": dict(tile=128, k_split=0, tail_split=True),
    "gemm_linear_2048x512x2048": dict(tile=128, k_split=0, tail_split=True),
}
GEMM_WORKERS = 256      # resident workgroups: one per CU for both tiles
# workloads whose oracle baseline is timed on sampled query rows (GFLOP/s)
ROW_SAMPLED_BASELINE = ("prefill_varlen_bf16", "mixed_bf16")
KERNEL_SOURCE = os.path.join(ROOT, "paged_variable_length_amd", "csrc", "attention.hip")


def counter_traffic(workload, tiling):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of this workload, if it was taken on the current kernel source and tiling (else
    None). The summary's header records the source hash, the tiling and the calibrated bytes."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    meta = {}
    for line in open(path):
        if line.startswith("# ") and ":" in line:
            k, v = line[2:].split(":", 1)
            meta[k.strip()] = v.strip()
    src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    if meta.get("kernel source sha256") != src or meta.get("tiling") != json.dumps(tiling,
                                                                                   sort_keys=True):
        return None
    try:
        rd, wr = (float(x) for x in meta["launch traffic bytes (read, write)"].split(","))
    except (KeyError, ValueError):
        return None
    return {"read_bytes": rd, "write_bytes": wr, "bytes": rd + wr, "source": os.path.relpath(path, ROOT)}


def algorithmic_work(w, fp8_pages=False):
    """Bytes the method must move and flops it must do, counting valid data only: every
    visible K/V row once (one byte per element for fp8 pages, plus the K and V scale of each
    (block, kv head) page read), q and out once, the block-table entries a sequence needs, its
    length; flops = 4*D per unmasked (query row, key) pair per query head. A K/V row that
    several sequences alias (a shared prefix) is one row of HBM data: the bytes count distinct
    cached (block, slot) pairs, which equals the sum of the contexts when nothing is aliased."""
    esize = 2 if w.dtype == "bf16" else 4
    kv_size = 1 if fp8_pages else esize
    e_kv = 2 * w.num_kv_heads * w.head_dim * kv_size
    ctx = w.ctx_lens.astype(np.int64)
    # a slot is counted once if any sequence reads it; a sequence's last block holds only its
    # first ctx - (nblk - 1) * bs slots
    used = np.zeros((w.num_blocks, w.block_size), dtype=bool)
    for s_ in range(w.num_seqs):
        c = int(ctx[s_])
        nb_ = (c + w.block_size - 1) // w.block_size
        used[w.block_table[s_, :nb_ - 1]] = True
        used[w.block_table[s_, nb_ - 1], :c - (nb_ - 1) * w.block_size] = True
    distinct = int(used.sum())
    q = w.q_lens.astype(np.int64)
    nblk = (ctx + w.block_size - 1) // w.block_size
    T = int(q.sum())
    scale_bytes = int(nblk.sum()) * w.num_kv_heads * 2 * 4 if fp8_pages else 0
    B = distinct * e_kv + T * w.num_q_heads * w.head_dim * esize * 2 + int(nblk.sum()) * 4 \
        + 4 * w.num_seqs + scale_bytes
    P = ctx - q
    pairs = P * q + q * (q + 1) // 2                      # sum over rows i of (P + i + 1)
    dec = q == 1
    F_dec = int((pairs[dec]).sum()) * w.num_q_heads * 4 * w.head_dim
    F_pre = int((pairs[~dec]).sum()) * w.num_q_heads * 4 * w.head_dim
    B_dec = (distinct if np.all(dec) else int(ctx[dec].sum())) * e_kv \
        + int(dec.sum()) * w.num_q_heads * w.head_dim * esize * 2 \
        + int(nblk[dec].sum()) * 4 + 4 * int(dec.sum()) + (scale_bytes if np.all(dec) else 0)
    reshape = 2 * T * w.num_kv_heads * w.head_dim * esize * 2     # read the new rows, write them
    if fp8_pages:
        # the fp8 write reads the new rows once and reads and rewrites every valid row of each
        # page it touches, plus that page's scale
        rows = 0
        for s in range(w.num_seqs):
            p0, c = int(P[s]), int(ctx[s])
            for lb in range(p0 // w.block_size, (c - 1) // w.block_size + 1):
                rows += min(c, (lb + 1) * w.block_size) - lb * w.block_size
        pages = int(((ctx - 1) // w.block_size - P // w.block_size + 1).sum())
        reshape = 2 * w.num_kv_heads * (T * w.head_dim * esize + 2 * rows * w.head_dim
                                        + pages * 8)
    return dict(bytes=B, flops_prefill=F_pre, flops_decode=F_dec, bytes_decode=B_dec,
                reshape_bytes=reshape, logical_kv_bytes=int(ctx.sum()) * e_kv)


class Runner:
    """Everything one workload's step needs, resident on the GPU."""

    def __init__(self, name, seed=None, workload=None, tiling=None):
        import torch
        import synth
        import paged_variable_length_amd as pa
        self.torch, self.pa = torch, pa
        self.name = name
        # "name:variant" tilings; a caller-built workload (the context sweep) brings its tiling
        self.w = w = workload if workload is not None else synth.make_workload(name.split(":")[0], seed)
        self.vals = synth.make_values(w, device="cuda", nan_sentinels=True)
        self.fp8 = name.endswith("_fp8")
        if self.fp8:                     # fp8 pages with page scales replace the bf16 pool
            del self.vals["k_pages"], self.vals["v_pages"]
            self.vals.update(synth.make_fp8_pages(w, device="cuda"))
        self.tiling = dict(tiling if tiling is not None else TILING[name], num_workers=256 * 2)
        self.cu_host = pa.pack_seqlens(w.q_lens)
        self.ctx_host = w.ctx_lens.astype(np.int32)
        self.params = pa.make_params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                     **self.tiling)
        # a host copy of the block table lets the decomposer find shared prefixes
        self.bt_host = w.block_table if self.params.shared_min else None
        first = pa.build_task_table(self.params, self.cu_host, self.ctx_host,
                                    block_table=self.bt_host)
        self.balance = (first.balance_snake, first.balance_modulo)
        self.num_tasks, self.num_combines = len(first.tasks), len(first.combines)
        self.num_partials = first.num_partials
        dev = "cuda"
        self.cu = torch.from_numpy(self.cu_host).to(dev)
        self.ctx = torch.from_numpy(self.ctx_host).to(dev)
        self.bt = torch.from_numpy(w.block_table).to(dev)
        # one pinned and one device buffer per slot: task rows, then combine rows, so a
        # single copy carries the whole table
        self.cap_t, self.cap_c = max(self.num_tasks, 1), max(self.num_combines, 1)
        rows = self.cap_t + self.cap_c
        self.pin = [torch.zeros((rows, 8), dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.dev = [torch.zeros((rows, 8), dtype=torch.int32, device=dev) for _ in range(2)]
        self.copy_stream = torch.cuda.Stream()      # default priority
        self.copy_ev = [torch.cuda.Event(), torch.cuda.Event()]
        self.slot_ev = [None, None]
        nbytes = pa.workspace_bytes(self.num_partials, w.head_dim)
        self.ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(self.vals["q"])
        self.scale = 1.0 / math.sqrt(w.head_dim)
        self.decode_only = bool(np.all(w.q_lens == 1))
        # fp8 tables of decode and verify tasks only go to the verify entry, others (prefill
        # tiles) to the unified fp8 launch
        self.verify_kinds = (1 << pa.PA_TASK_DECODE) | (1 << pa.PA_TASK_VERIFY)
        self.work = algorithmic_work(w, self.fp8)
        self.step_no = 0
        self.graphs = None

    def build_table(self, k):
        """Host table for slot k into pinned memory, then one async copy to the device slot on
        the copy stream, so it overlaps the kernels of the step before."""
        pa, torch = self.pa, self.torch
        if self.slot_ev[k] is not None:
            self.slot_ev[k].synchronize()      # the slot's previous copy and kernels are done
        pin = self.pin[k].numpy()
        t = pa.build_task_table(self.params, self.cu_host, self.ctx_host, pin[:self.cap_t],
                                pin[self.cap_t:], with_balance=False, block_table=self.bt_host)
        nt, nc = len(t.tasks), len(t.combines)
        n = self.cap_t + nc
        with torch.cuda.stream(self.copy_stream):
            self.dev[k][:n].copy_(self.pin[k][:n], non_blocking=True)
            self.copy_ev[k].record()
        self.kinds = t.kinds
        return nt, nc, t.num_partials

    def write_cache(self):
        pa, v = self.pa, self.vals
        if self.fp8:
            pa.reshape_and_cache_fp8(v["k_new"], v["v_new"], v["k_codes"], v["v_codes"],
                                     v["scales"], self.bt, self.cu, self.ctx)
        else:
            pa.reshape_and_cache(v["k_new"], v["v_new"], v["k_pages"], v["v_pages"], self.bt,
                                 self.cu, self.ctx)

    def launch(self, k, nt, nc, nparts, ev_pair=None):
        """Cache write, then the attention launch (bracketed by ev_pair if given) once slot k's
        table copy has landed, all on the current stream. The cache write does not read the
        table, so it goes ahead of the wait for the copy (measured: ~4 us less per decode
        step)."""
        self.write_cache()
        self.torch.cuda.current_stream().wait_event(self.copy_ev[k])
        self.attention(k, nt, nc, nparts, ev_pair)

    def attention(self, k, nt, nc, nparts, ev_pair=None):
        """The attention launch (and its combine) over slot k's device table."""
        pa, v = self.pa, self.vals
        tasks = self.dev[k][:nt]
        combines = self.dev[k][self.cap_t:self.cap_t + nc]
        if ev_pair is not None:
            ev_pair[0].record()
        if self.fp8 and self.decode_only:
            pa.paged_attn_decode_fp8(v["q"], v["k_codes"], v["v_codes"], v["scales"],
                                     self.bt, self.ctx, self.scale, tasks,
                                     self.kinds, combines, nparts, self.ws, self.out)
        elif self.fp8 and self.kinds & ~self.verify_kinds:
            pa.paged_attn_varlen_prefill_fp8(v["q"], v["k_codes"], v["v_codes"], v["scales"],
                                             self.bt, self.cu, self.ctx, self.scale, tasks,
                                             self.kinds, combines, nparts, self.ws, self.out)
        elif self.fp8:
            pa.paged_attn_verify_fp8(v["q"], v["k_codes"], v["v_codes"], v["scales"],
                                     self.bt, self.cu, self.ctx, self.scale,
                                     tasks, self.kinds, combines, nparts, self.ws, self.out)
        elif self.decode_only:
            pa.paged_attn_decode(v["q"], v["k_pages"], v["v_pages"], self.bt, self.ctx, self.scale,
                                 tasks, self.kinds, combines, nparts, self.ws, self.out)
        else:
            pa.paged_attn_varlen_prefill(v["q"], v["k_pages"], v["v_pages"], self.bt, self.cu,
                                         self.ctx, self.scale, tasks, self.kinds, combines,
                                         nparts, self.ws, self.out)
        if ev_pair is not None:
            ev_pair[1].record()

    def capture(self):
        """One HIP graph per table slot holding the step's device work after the table copy:
        the cache write, the attention launch over that slot's device table and the combine.
        A step then builds its table on the host, copies it on the side stream and replays its
        slot's graph once the copy has landed; the batch (so the table's size) is the same every
        step, which the replay checks."""
        torch = self.torch
        self.graphs, self.graph_sizes = [None, None], [None, None]
        for k in range(2):
            sizes = self.build_table(k)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                self.write_cache()
                self.attention(k, *sizes)
            torch.cuda.synchronize()
            self.graphs[k], self.graph_sizes[k] = g, sizes

    def step(self):
        """One full step: host table (slot k), its copy, cache write, attention (replayed from
        the slot's graph once captured)."""
        k = self.step_no % 2
        self.step_no += 1
        nt, nc, nparts = self.build_table(k)
        if self.graphs is not None:
            if (nt, nc, nparts) != self.graph_sizes[k]:
                raise RuntimeError("the batch's table changed size: its graph no longer fits")
            self.torch.cuda.current_stream().wait_event(self.copy_ev[k])
            self.graphs[k].replay()
        else:
            self.launch(k, nt, nc, nparts)
        if self.slot_ev[k] is None:
            self.slot_ev[k] = self.torch.cuda.Event()
        self.slot_ev[k].record()

    def timed_steps(self, steps, warmup, graphs=False):
        torch = self.torch
        if graphs and self.graphs is None:
            self.capture()
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    def launch_times(self, launches, flush):
        """Average duration of the attention launch, from HIP events recorded on the current
        stream (the stream the library launches on). The table is built once; each iteration
        evicts L2/MALL by reading a 1 GiB buffer (a read leaves no dirty lines whose
        write-back would land on the timed kernel), rewrites the cache, and brackets the
        attention launch. Nothing synchronises the host inside the loop, so the queue stays
        full and the events time the GPU work, not host launch latency."""
        torch = self.torch
        torch.cuda.synchronize()
        nt, nc, nparts = self.build_table(0)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        for e in evs:
            flush.sum()
            self.launch(0, nt, nc, nparts, e)
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in evs]
        self.last_launch_median = float(np.median(ms))
        return float(np.mean(ms)), float(np.min(ms))

    def table_build_us(self, reps=20):
        """Median host time of one task-table build into a pinned slot (no copy)."""
        pin = self.pin[0].numpy()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            self.pa.build_task_table(self.params, self.cu_host, self.ctx_host, pin[:self.cap_t],
                                     pin[self.cap_t:], with_balance=False,
                                     block_table=self.bt_host)
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts) * 1e6)

    def reshape_times(self, launches, flush):
        """Average duration of reshape_and_cache alone (HIP events on the launch stream, L2/MALL
        evicted by a read between launches, as for the attention launch)."""
        torch, pa, v = self.torch, self.pa, self.vals
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(launches)]
        for a, b in evs:
            flush.sum()
            a.record()
            self.write_cache()
            b.record()
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))

    def finite(self):
        return bool(self.torch.isfinite(self.out).all())


def host_cpu():
    """BLAS threads the oracle's NumPy uses, the cores this process may run on, and the host
    CPU as /proc/cpuinfo names it (model name plus family / model / stepping numbers)."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (x.strip() for x in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
            if not line.strip() and fields:
                break
    except OSError:
        pass
    model = fields.get("model name", "unknown")
    if "cpu family" in fields:
        model += (f" (family {fields['cpu family']}, model {fields.get('model', '?')}, "
                  f"stepping {fields.get('stepping', '?')})")
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return threads, model, affinity


def cpu_baseline(name, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded seeded sample of the same workload's
    sequences (cache scatter + attention), timed on this host's cores."""
    import torch
    import synth
    from oracle import attention as oa
    from oracle import cache as oc
    w = synth.make_workload(name.split(":")[0])
    rng = np.random.default_rng(0)
    order = rng.permutation(w.num_seqs)
    vals = synth.make_values(w, device="cuda", nan_sentinels=False)
    esize = 2 if w.dtype == "bf16" else 4
    e_kv = 2 * w.num_kv_heads * w.head_dim * esize
    cu = oa.pack_lengths(w.q_lens)
    done_bytes, done_seqs, spent = 0, 0, 0.0
    threads, model, affinity = host_cpu()
    for s in order:
        s = int(s)
        nblk = oa.blocks_needed(int(w.ctx_lens[s]), w.block_size)
        ids = torch.from_numpy(w.block_table[s, :nblk].astype(np.int64)).cuda()
        kp = vals["k_pages"].index_select(0, ids).float().cpu().numpy().astype(np.float64)
        vp = vals["v_pages"].index_select(0, ids).float().cpu().numpy().astype(np.float64)
        rows = slice(int(cu[s]), int(cu[s + 1]))
        q = vals["q"][rows].float().cpu().numpy().astype(np.float64)
        kn = vals["k_new"][rows].float().cpu().numpy().astype(np.float64)
        vn = vals["v_new"][rows].float().cpu().numpy().astype(np.float64)
        table = np.arange(nblk)[None, :]
        ql, ctx = w.q_lens[s:s + 1], w.ctx_lens[s:s + 1]
        t0 = time.perf_counter()
        kp2, vp2 = oc.reshape_and_cache(kn, vn, kp, vp, table, ql, ctx)
        oa.paged_attention_fast(q, kp2, vp2, table, ql, ctx, 1.0 / math.sqrt(w.head_dim))
        spent += time.perf_counter() - t0
        done_bytes += int(ctx[0]) * e_kv + int(ql[0]) * w.num_q_heads * w.head_dim * esize * 2 \
            + nblk * 4 + 4
        done_seqs += 1
        if spent >= budget_s:
            break
    del vals
    torch.cuda.empty_cache()
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "cores_available": affinity,
            "sample": f"{done_seqs} of {w.num_seqs} sequences of {name} (seeded order), "
                      f"fp64 NumPy cache scatter + attention, {spent:.1f} s"}


def cpu_baseline_rows(name, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded seeded sample of a prefill or mixed
    workload's query rows, timed on this host's cores. The sequence with the longest context
    comes first, then the others in a seeded order; in the first pass each contributes its first
    and last row and one seeded row (a decode sequence its one row), and while the time budget
    lasts further passes add seeded rows of the multi-row sequences. Every sampled row runs for
    all query heads through the oracle's plain definition (gather through the block table,
    full-row softmax per row and head). Reported in GFLOP/s of the sampled rows' flops (4 * D
    per visible key per head); for sampled decode rows also their K/V bytes per second."""
    import torch
    import synth
    from oracle import attention as oa
    w = synth.make_workload(name.split(":")[0])
    vals = synth.make_values(w, device="cuda", nan_sentinels=False)
    rng = np.random.default_rng(0)
    longest = int(np.argmax(w.ctx_lens))
    order = [longest] + [int(x) for x in rng.permutation(w.num_seqs) if int(x) != longest]
    cu = oa.pack_lengths(w.q_lens)
    e_kv = 2 * w.num_kv_heads * w.head_dim * 2
    scale = 1.0 / math.sqrt(w.head_dim)
    flops, dec_bytes, dec_time, spent, nrows = 0, 0, 0.0, 0.0, 0
    seen, host = set(), {}
    threads, model, affinity = host_cpu()

    def host_copy(s):
        if s not in host:
            nblk = oa.blocks_needed(int(w.ctx_lens[s]), w.block_size)
            ids = torch.from_numpy(w.block_table[s, :nblk].astype(np.int64)).cuda()
            f64 = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
            host[s] = (f64(vals["k_pages"].index_select(0, ids)),
                       f64(vals["v_pages"].index_select(0, ids)),
                       f64(vals["q"][int(cu[s]):int(cu[s + 1])]), np.arange(nblk)[None, :])
        return host[s]

    for rnd in range(64):
        for s in order:
            ql, ctx = int(w.q_lens[s]), int(w.ctx_lens[s])
            if rnd > 0 and ql == 1:
                continue
            rows = sorted({0, ql - 1, int(rng.integers(0, ql))}) if rnd == 0 else \
                sorted({int(x) for x in rng.integers(0, ql, size=4)})
            kp, vp, q, table = host_copy(s)
            t0 = time.perf_counter()
            oa.paged_attention(q, kp, vp, table, w.q_lens[s:s + 1], w.ctx_lens[s:s + 1], scale,
                               rows={0: rows})
            dt = time.perf_counter() - t0
            spent += dt
            flops += sum(ctx - ql + i + 1 for i in rows) * w.num_q_heads * 4 * w.head_dim
            if ql == 1:
                dec_bytes += ctx * e_kv
                dec_time += dt
            seen.add(s)
            nrows += len(rows)
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    del vals, host
    torch.cuda.empty_cache()
    out = {"value": round(flops / spent / 1e9, 4), "unit": "GFLOP/s", "cores": threads,
           "kind": "oracle", "cpu_model": model, "cores_available": affinity,
           "sample": f"{nrows} query rows x {w.num_q_heads} heads from {len(seen)} of "
                     f"{w.num_seqs} sequences of {name} (longest context first, then seeded), "
                     f"fp64 NumPy gather + full-row softmax per row, {spent:.1f} s, "
                     f"{flops:.3e} flop"}
    if dec_time > 0:
        out["decode_rows_gbs"] = round(dec_bytes / dec_time / 1e9, 4)
    return out


# Context-length sweep of the headline decode batch's shape (cann-recipes-infer page, section
# 4.4, third check: the paged-attention kernel's time grows linearly with the sequence length
# while its read bandwidth stays steady): 64 sequences, all with the same context, MHA 32 heads,
# D 128, 16-token blocks, the headline tiling.
SWEEP_CTX = (256, 512, 1024, 2048, 4096, 8192, 16384)


def ctx_sweep(launches, flush):
    import synth
    points = []
    for ctx in SWEEP_CTX:
        w = synth.custom_workload([1] * 64, [ctx] * 64, 32, 32, 128, 16, seed=8,
                                  name=f"decode_mha_bf16_ctx{ctx}")
        r = Runner(w.name, workload=w, tiling=TILING[HEADLINE])
        avg, mn = r.launch_times(launches, flush)
        b = r.work["bytes"]
        points.append({"context": ctx, "launch_ms_avg": round(avg, 4),
                       "launch_ms_median": round(r.last_launch_median, 4),
                       "bytes": b, "gbs": round(b / (avg * 1e-3) / 1e9, 1)})
        del r
        import torch
        torch.cuda.empty_cache()
    x = np.array([p["context"] for p in points], dtype=np.float64)
    y = np.array([p["launch_ms_avg"] for p in points], dtype=np.float64)
    slope, icept = np.polyfit(x, y, 1)
    pred = slope * x + icept
    r2 = 1.0 - float(((y - pred) ** 2).sum() / ((y - y.mean()) ** 2).sum())
    gbs = [p["gbs"] for p in points]
    return {"batch": "64 decode sequences, one context each run, Hq=Hkv=32, D=128, bs=16",
            "points": points,
            "linear_fit_ms": {"per_1k_keys": round(slope * 1e3, 5), "intercept": round(icept, 5),
                              "r2": round(r2, 5)},
            "gbs_from_2048": {"min": min(g for p, g in zip(points, gbs) if p["context"] >= 2048),
                              "max": max(g for p, g in zip(points, gbs) if p["context"] >= 2048)}}


def run_gemm(name, steps, warmup, flush):
    """One SmoothGEMM workload: a step is the host Linear decomposition into a pinned buffer,
    its copy to the device and the GEMM launch (plus the partial-tile reduce when K is split).
    Launch time from HIP events on the launch stream with L2/MALL evicted (a 1 GiB read)
    between launches; torch.mm (hipBLASLt) on the same operands, warmed up, is timed the same
    way as a reference point."""
    import torch
    import synth
    import paged_variable_length_amd as pa
    shape = name[len("gemm_"):]
    M, N, K = synth.gemm_shape(shape)
    tl = GEMM_TILING[name]
    a, w = synth.make_gemm_operands(M, N, K, device="cuda", seed=1)
    c = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    plan = pa.GemmPlan(M, N, K, tile=tl["tile"], k_split=tl["k_split"], num_workers=GEMM_WORKERS,
                       tail_split=tl["tail_split"])
    nt = len(plan.table.tasks)
    pin = torch.zeros((max(nt, 1), 8), dtype=torch.int32, pin_memory=True)

    def step():
        t = pa.build_gemm_table(M, N, K, tl["tile"], tl["k_split"], GEMM_WORKERS,
                                tl["tail_split"])
        pin.numpy()[:nt] = t.tasks
        plan.tasks.copy_(pin[:nt], non_blocking=True)
        plan.run(a, w, c)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / steps

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for e0, e1 in evs:
            flush.sum()
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        ms = [x.elapsed_time(y) for x, y in evs]
        return float(np.mean(ms)), float(np.min(ms)), float(np.median(ms))

    n = max(steps, 10)
    avg, mn, med = timed(lambda: plan.run(a, w, c), n)
    # the library's first call picks its kernel (about 0.2 s); warm it up, write into a
    # preallocated output
    cref = torch.empty_like(c)
    for _ in range(3):
        torch.mm(a, w.t(), out=cref)
    lib_avg, _, _ = timed(lambda: torch.mm(a, w.t(), out=cref), n)
    del cref
    flops = 2.0 * M * N * K
    tf = flops / (avg * 1e-3) / 1e12
    res = {"workload": name, "shape_mnk": [M, N, K], "tiling": tl, "tasks": nt,
           "reduces": len(plan.table.reduces),
           "balance_snake": round(plan.table.balance_snake, 4),
           "balance_modulo": round(plan.table.balance_modulo, 4),
           "ms_per_step": round(step_s * 1e3, 4), "launch_ms_avg": round(avg, 4),
           "launch_ms_min": round(mn, 4), "launch_ms_median": round(med, 4),
           "flops": flops, "tflops": round(tf, 2), "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
           "bytes_min": 2 * (M * K + N * K + M * N),
           "finite": bool(torch.isfinite(c).all()),
           "torch_matmul_ms_avg": round(lib_avg, 4),
           "torch_matmul_tflops": round(flops / (lib_avg * 1e-3) / 1e12, 2)}
    del a, w, c, plan
    torch.cuda.empty_cache()
    return res


def run(name, steps, warmup, with_launch_timing=True, flush=None, graphs=False):
    if name.startswith("gemm_"):
        return run_gemm(name, steps, warmup, flush)
    r = Runner(name)
    step_s = r.timed_steps(steps, warmup, graphs)
    res = {"workload": name, "ms_per_step": round(step_s * 1e3, 4), "tasks": r.num_tasks,
           "combines": r.num_combines, "balance_snake": round(r.balance[0], 4),
           "balance_modulo": round(r.balance[1], 4), "finite": r.finite(), "work": r.work,
           "tiling": r.tiling, "step_device_work": "hip graph per table slot" if graphs else
           "eager launches"}
    if with_launch_timing:
        avg_ms, min_ms = r.launch_times(max(steps, 10), flush)
        res["attn_launch_ms_avg"] = round(avg_ms, 4)
        res["attn_launch_ms_min"] = round(min_ms, 4)
        res["attn_launch_ms_median"] = round(r.last_launch_median, 4)
        rs_ms = r.reshape_times(max(steps, 10), flush)
        res["reshape_ms_avg"] = round(rs_ms, 4)
        res["reshape_gbs"] = round(r.work["reshape_bytes"] / (rs_ms * 1e-3) / 1e9, 1)
    res["table_build_us"] = round(r.table_build_us(), 1)
    del r
    import torch
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dec-split", type=int, default=None, help="override decode key split")
    ap.add_argument("--pf-kv-split", type=int, default=None, help="override prefill key split")
    ap.add_argument("--pf-q-tile", type=int, default=None, help="override prefill query tile")
    ap.add_argument("--decode-weight", type=int, default=None, help="override decode load weight")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step's device work from a HIP graph per table slot "
                         "(measured on the headline batch: 0.422 ms per step against 0.415 ms "
                         "eager, so eager launches are the default)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB elementwise copy (for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    for tl in TILING.values():
        if args.dec_split is not None and "dec_split" in tl:
            tl["dec_split"] = args.dec_split
        if args.pf_kv_split is not None and "pf_kv_split" in tl:
            tl["pf_kv_split"] = args.pf_kv_split
        if args.pf_q_tile is not None and "pf_q_tile" in tl:
            tl["pf_q_tile"] = args.pf_q_tile
        if args.decode_weight is not None:
            tl["decode_weight"] = args.decode_weight
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    flush = torch.ones(2**28, dtype=torch.float32, device="cuda")     # 1 GiB, read to evict

    if args.calibrate_copy:
        src = torch.ones(2**28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
        print("[bench] calibration copy: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)

    head = run(args.workload, args.steps, args.warmup, True, flush, args.graph)
    if args.workload.startswith("gemm_"):
        # a SmoothGEMM workload on its own (for profiling): its result is the whole line
        print(f"[bench] {args.workload}: {head['launch_ms_avg']} ms launch, {head['tflops']} "
              f"TFLOP/s (torch.matmul {head['torch_matmul_tflops']})", file=sys.stderr,
              flush=True)
        print(json.dumps({"metric": "SmoothGEMM TFLOP/s", "value": head["tflops"],
                          "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": args.workload}, "detail": head}), flush=True)
        return
    print(f"[bench] {args.workload}: {head['ms_per_step']} ms/step, attention launch "
          f"{head['attn_launch_ms_avg']} ms", file=sys.stderr, flush=True)
    secondary = {}
    if not args.only:
        for name in SECONDARY:
            if name == args.workload:
                continue
            res = run(name, args.steps, args.warmup, True, flush, args.graph)
            if name.startswith("gemm_"):
                secondary[name] = res
                print(f"[bench] {name}: {res['launch_ms_avg']} ms launch, {res['tflops']} "
                      f"TFLOP/s ({res['mfma_frac']:.1%} of MFMA peak; torch.matmul "
                      f"{res['torch_matmul_tflops']})", file=sys.stderr, flush=True)
                continue
            wk = res["work"]
            t_launch = res["attn_launch_ms_avg"] * 1e-3
            res["attn_gbs"] = round(wk["bytes"] / t_launch / 1e9, 1)
            res["attn_tflops_prefill"] = round(wk["flops_prefill"] / t_launch / 1e12, 2)
            res["hbm_frac"] = round(res["attn_gbs"] / HBM_PEAK_GBS, 4)
            # K/V bytes as every sequence sees them (aliased prefix rows once per sequence)
            res["logical_kv_gbs"] = round(wk["logical_kv_bytes"] / t_launch / 1e9, 1)
            res["mfma_frac"] = round(res["attn_tflops_prefill"] / MFMA_BF16_PEAK_TFLOPS, 4)
            res["roofline_frac"] = round(max(wk["bytes"] / (HBM_PEAK_GBS * 1e9),
                                             wk["flops_prefill"] / (MFMA_BF16_PEAK_TFLOPS * 1e12))
                                         / t_launch, 4)
            if name in ROW_SAMPLED_BASELINE and not args.no_cpu_baseline:
                cb = cpu_baseline_rows(name)
                res["cpu_baseline"] = cb
                res["gpu_over_cpu_baseline"] = round(res["attn_tflops_prefill"] * 1e3 / cb["value"], 1)
                print(f"[bench] {name}: oracle {cb['value']} GFLOP/s on {cb['cores']} threads "
                      f"({cb['sample']})", file=sys.stderr, flush=True)
            secondary[name] = res
            print(f"[bench] {name}: {res['ms_per_step']} ms/step, launch "
                  f"{res['attn_launch_ms_avg']} ms, {res['attn_gbs']} GB/s, "
                  f"{res['attn_tflops_prefill']} TFLOP/s", file=sys.stderr, flush=True)

    sweep = None
    if not args.only:
        sweep = ctx_sweep(max(args.steps, 10), flush)
        fit = sweep["linear_fit_ms"]
        print(f"[bench] context sweep: {fit['per_1k_keys']} ms per 1k keys, r2 {fit['r2']}, "
              f"GB/s from 2k keys {sweep['gbs_from_2048']}", file=sys.stderr, flush=True)
    wk = head["work"]
    step_s = head["ms_per_step"] * 1e-3
    value = wk["bytes"] / step_s / 1e9
    achieved = wk["bytes"] / (head["attn_launch_ms_avg"] * 1e-3) / 1e9
    w = head
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload)
    import synth
    wl = synth.make_workload(args.workload.split(":")[0])
    traffic = counter_traffic(args.workload, head["tiling"])
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) values, seeded lengths and shuffled block pool)",
        "config": {"workload": args.workload, "num_seqs": wl.num_seqs,
                   "context_lens": "uniform [128, 4096]" if args.workload == HEADLINE else "see synth",
                   "sum_context": int(wl.ctx_lens.sum()), "num_q_heads": wl.num_q_heads,
                   "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
                   "block_size": wl.block_size, **TILING[args.workload]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_detail": traffic,
                     "kernel": "paged_attn_decode launch (decode_kernel + combine_kernel)",
                     "bytes_per_launch": wk["bytes"],
                     "launch_ms_avg": head["attn_launch_ms_avg"],
                     "launch_ms_min": head["attn_launch_ms_min"]},
        "cpu_baseline": cpu,
        "gpu_over_cpu_baseline": round(value / cpu["value"], 1) if cpu else None,
        "headline_detail": {k: head[k] for k in ("tasks", "combines", "balance_snake",
                                                 "balance_modulo", "finite", "table_build_us",
                                                 "attn_launch_ms_median",
                                                 "reshape_ms_avg", "reshape_gbs")},
        "secondary": secondary,
        "context_sweep": sweep,
    }
    # the metric names two halves: decode GB/s (the headline `value`, per step; the launch in
    # `roofline`) and prefill TFLOP/s (the packed varlen prefill launch)
    parts = {"decode": {"workload": args.workload, "launch_gbs": round(achieved, 1),
                        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4)}}
    pf = secondary.get("prefill_varlen_bf16")
    if pf:
        parts["prefill"] = {"workload": "prefill_varlen_bf16",
                            "launch_tflops": pf["attn_tflops_prefill"],
                            "mfma_frac": pf["mfma_frac"],
                            "launch_ms_avg": pf["attn_launch_ms_avg"]}
    line["metric_parts"] = parts
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
