"""Throughput of the paged-KV attention hot path on one MI355X.

A step is one decode pass of the long-context configuration (batch 1, 131072
keys, 32 query heads over 4 KV heads, K192/V128 bf16, block size 16):
  1. attn_cache_write of each sequence's new token (its K/V row),
  2. the split-KV partial kernel over the whole paged context,
  3. the log-sum-exp merge of its partitions into the bf16 output.
Inputs are resident in HBM before the timed region.  The step rotates over
several identical cache copies totalling >= 1 GB, so no step finds its K/V in
the 256 MB MALL left behind by the previous one.  Steps are launched eagerly: a
HIP graph per cache copy was measured no faster for this three-launch step.

value = algorithmic bytes per step / step time, where the algorithmic bytes are
the K/V rows read once per (sequence, KV head) plus Q, O and the block table.
The "roofline" object reports the split-KV kernel alone (HIP events on the
launch stream) against the 8 TB/s HBM peak; the oracle is timed on the
host's cores as a reported baseline.  Secondary lines (other decode shapes,
fp8 verify, MLA decode, chunked-prefill TFLOP/s) are printed under "extra".
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
MALL_BYTES = 256 << 20


# HBM bytes per launch of the split-KV kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# (scaled by a copy of known size), keyed by the sha256 of the kernel's sources and the
# partition count they were taken at: any later change reports traffic as null until
# re-measured.
MEASURED_TRAFFIC = {
    ("304008f8c75d5565", 128): 164006.6 * 1024 * 2 + 2178.7 * 1024,
}
KERNEL_SOURCES = ("splitkv_dma.hip", "common.hpp", "kernels.hpp", "lds_layout.hpp", "phase_stamps.hpp")


def _kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_176_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _copies(nbytes):
    return max(4, math.ceil((1 << 30) / max(1, nbytes)))


CUS = 256
# --partitions with --only: the split count of that one workload (a sweep), else auto
PARTITIONS_OVERRIDE = 0


def auto_partitions(batch, kv_heads, ctx, wgs_per_cu=1, min_keys=256, wave_keys=64):
    """Split count: as many 4-wave workgroups as the partial kernel keeps resident per CU
    (two for the bf16 DiffKV decode kernel, one for the MLA and fp8-verify kernels), with
    partitions of at least min_keys keys, then the partition size rounded up to a multiple
    of wave_keys (one 16-key tile per wave of the workgroup) so that the waves of a
    workgroup get equal tile counts (100K-key MLA at batch 1: 224 partitions of 448 keys
    instead of 256 of 400, whose waves got 7 or 6 tiles)."""
    if PARTITIONS_OVERRIDE:
        return PARTITIONS_OVERRIDE
    p = max(1, math.ceil(CUS * wgs_per_cu / max(1, batch * kv_heads)))
    p = min(p, max(1, ctx // min_keys), 4096)
    chunk = math.ceil(math.ceil(ctx / p) / wave_keys) * wave_keys
    return max(1, math.ceil(ctx / chunk))


class DecodeCase:
    """A decode (or MLA decode) workload on the GPU with rotating cache copies."""

    def __init__(self, w, P, dev="cuda:0", policy=None):
        import torch
        import paged_kv_cache_176_amd as pk
        import workloads
        self.w, self.P, self.policy = w, P, policy
        g = w.geom
        img = w.cache_init.clone()
        if "pre_slots" in w.extra:
            workloads.place_bf16_rows(img, g, w.extra["pre_slots"], w.extra["pre_key"], w.extra["pre_value"])
        self.cache_cpu = img
        nbytes = img.numel() * img.element_size()
        self.ncopy = 1 if nbytes > 4 * MALL_BYTES else _copies(nbytes)
        self.copies = [img.to(dev) for _ in range(self.ncopy)]
        self.descs = [pk.CacheDesc.from_geom(s, g) for s in self.copies]
        self.q = w.q.to(dev)
        self.key = w.key.to(dev)
        self.value = w.value.to(dev) if w.value is not None else None
        self.slots = w.slot_mapping.to(dev)
        assert self.key.shape[0] == w.q.shape[0], "one new token per sequence"
        self.bt = w.block_tables.to(dev)
        self.seq_lens = w.seq_lens.to(dev)
        B, Hq = w.q.shape[0], w.q.shape[1]
        self.ws = pk.new_workspace(B, Hq, g.head_dim_v, P, dev)
        from paged_kv_cache_176_amd.ops import workspace_views
        self.po, self.pl = workspace_views(self.ws, B, Hq, g.head_dim_v, P)
        self.out = torch.empty(B, Hq, g.head_dim_v, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        self.pk = pk
        kv_row = (g.head_dim_k + (g.head_dim_v if g.v_offset >= g.head_dim_k else 0)) * g.elem_bytes
        self.kv_bytes = int(w.seq_lens.sum().item()) * g.num_kv_heads * kv_row
        self.other_bytes = (w.q.numel() * 2 + B * Hq * g.head_dim_v * 2 +
                            sum(math.ceil(int(s) / g.block_size) for s in w.seq_lens.tolist()) * 4)
        # flops: QK^T and PV over every visible key of every query head
        self.flops = 2 * int(w.seq_lens.sum().item()) * Hq * (g.head_dim_k + g.head_dim_v)

        # every call checked and marshalled once per cache copy: a timed step is one ctypes call
        # (the binding's per-call Python checks would otherwise sit on the host's critical path
        # for the shorter steps)
        self.step_calls = [pk.decode_splitkv_append(self.q, self.key, self.value, self.slots, d, self.bt,
                                                    self.seq_lens, w.softmax_scale, P, out=self.out, out_lse=self.lse,
                                                    workspace=self.ws, split_policy=policy, prepare=True)
                           for d in self.descs]
        self.partial_calls = [pk.decode_splitkv_append(self.q, self.key, self.value, self.slots, d, self.bt,
                                                       self.seq_lens, w.softmax_scale, P, workspace=self.ws,
                                                       partials_only=True, split_policy=policy, prepare=True)
                              for d in self.descs]

    def partial(self, i):
        """The step's first kernel on cache copy i: the new token's write and the split-KV
        partials (attn_decode_splitkv_append with out=NULL; the write rides in the partial kernel)."""
        self.partial_calls[i % self.ncopy]()

    def time_partial(self, reps):
        """Average duration of the partial kernel alone: reps back-to-back launches (each on
        the next cache copy) between two HIP events on the launch stream."""
        import torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            self.partial(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    def partial_samples(self, reps):
        """Per-launch durations of the partial kernel (HIP events around each launch; the
        events' own cost is included, so these sit slightly above the back-to-back average)."""
        import torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record()
            self.partial(i)
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) / 1e3 for a, b in evs]

    def step(self, i, ev=None):
        """One decode step: attn_decode_splitkv_append with an output buffer -- the new
        token's K/V write and the split-KV partials in one kernel, then the merge (its own
        kernel, or folded into the partial kernel where the shape allows)."""
        if ev is not None:
            ev[0].record()
        self.step_calls[i % self.ncopy]()
        if ev is not None:
            ev[1].record()


SPINUP_MS = 200.0


def time_steps(fn, steps, warmup, events=False):
    """Warm up, then time exactly ``steps`` calls between two synchronisations.  Before the
    ``warmup`` calls the step runs untimed for SPINUP_MS of wall time: a GPU that has idled
    through the set-up runs its first ~10 ms slow (measured: a first timed pass 1% slower
    than later ones for the B1 decode step, 13% for the MLA verify B16 call)."""
    import torch
    t_end = time.perf_counter() + SPINUP_MS / 1e3
    i = 0
    while time.perf_counter() < t_end:            # back to back, the queue bounded to 16 calls
        fn(i, None)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    for i in range(warmup):
        fn(i, None)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)] \
        if events else [None] * steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + i, evs[i])
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    kern, per = None, None
    if events:
        per = [a.elapsed_time(b) / 1e3 for a, b in evs]
        kern = sum(per) / steps
    return dt, kern, per


def pcts(samples_s):
    """p10 / median / p90 of per-call durations, in microseconds."""
    import numpy as np
    a = np.asarray(samples_s, dtype=np.float64) * 1e6
    return {k: round(float(np.percentile(a, q)), 2) for k, q in (("p10", 10), ("p50", 50), ("p90", 90))}


def host_info():
    """The host the oracle runs on: CPU model, cores this process may use, BLAS threads."""
    import threadpoolctl
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [x.get("num_threads", 1) for x in threadpoolctl.threadpool_info() if x.get("user_api") == "blas"]
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": max(blas) if blas else 1}


def oracle_cache(w, write_new):
    """The cache image as the oracle sees it: the pre-placed context, and (write_new) the
    workload's new tokens written by the oracle's cache write."""
    import numpy as np
    import torch
    from oracle import paged_ref as R
    import workloads
    g = w.geom
    img = w.cache_init.clone()
    if "pre_slots" in w.extra:
        workloads.place_bf16_rows(img, g, w.extra["pre_slots"], w.extra["pre_key"], w.extra["pre_value"])
    base = img.numpy() if g.kv_dtype == "fp8" else img.numpy().view(np.uint16)
    if not write_new:
        return base
    kb = w.key.view(torch.int16).numpy().view(np.uint16)
    vb = w.value.view(torch.int16).numpy().view(np.uint16) if w.value is not None else None
    ks = w.k_scale.numpy() if w.k_scale is not None else None
    vs = w.v_scale.numpy() if w.v_scale is not None else None
    return R.cache_write(base, R.CacheSpec.from_geom(g), kb, vb, w.slot_mapping.numpy(), ks, vs)


def oracle_seconds(w, budget_s, with_write, rows=None):
    """Wall time of one oracle call on the workload (cache write of the new tokens when
    with_write, then fp64 attention of `rows`, default every query row), repeated until
    budget_s has passed; returns (seconds per call, calls)."""
    import numpy as np
    import torch
    from oracle import paged_ref as R
    spec = R.CacheSpec.from_geom(w.geom)
    ks = w.k_scale.numpy() if w.k_scale is not None else None
    vs = w.v_scale.numpy() if w.v_scale is not None else None
    qb = w.q.view(torch.int16).numpy().view(np.uint16)
    base = oracle_cache(w, write_new=False)
    written = None if with_write else oracle_cache(w, write_new=True)
    kb = w.key.view(torch.int16).numpy().view(np.uint16)
    vb = w.value.view(torch.int16).numpy().view(np.uint16) if w.value is not None else None
    n, t0 = 0, time.perf_counter()
    while True:
        c = R.cache_write(base, spec, kb, vb, w.slot_mapping.numpy(), ks, vs) if with_write else written
        R.paged_attention(qb, w.query_start_loc.numpy(), w.seq_lens.numpy(), w.block_tables.numpy(), c, spec,
                          w.softmax_scale, ks, vs, rows=rows)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return (time.perf_counter() - t0) / n, n


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on a bounded sample: whole decode steps of the same workload."""
    dt, n = oracle_seconds(w, budget_s, with_write=True)
    info = host_info()
    return dt, n, min(max(info["blas_threads"], 1), info["affinity_cores"]), info


# The oracle timings of the secondary lines run after every GPU measurement: a multithreaded
# BLAS call right before a timed GPU loop was seen to slow the loop's launches (its threads
# still spinning), so each line queues its oracle job here and main() runs them at the end.
DEFERRED = []


def defer_cpu(res, seconds_fn, algo, unit, sample, scale=1.0):
    """Queue an oracle timing whose result lands in res["cpu_oracle"]."""
    def job():
        sec, n = seconds_fn()
        res["cpu_oracle"] = cpu_line(sec, n, algo, unit, sample, scale)
        return res["cpu_oracle"]
    DEFERRED.append(job)


def cpu_line(seconds, n, algo, unit, sample, scale=1.0):
    """The oracle's figure for one measured line: `algo` bytes (GB/s) or flops (TFLOP/s) of
    the whole call, the sampled seconds scaled by `scale` to the whole call."""
    per_call = seconds * scale
    value = algo / per_call / (1e9 if unit == "GB/s" else 1e12)
    return {"value": round(value, 5), "unit": unit, "s_per_call": round(per_call, 3), "calls_timed": n,
            "sample": sample}


def run_prefill(steps, warmup, cpu=True):
    """Chunked prefill of 32768 tokens in 4096-token chunks: write + causal attention per chunk."""
    import numpy as np
    import torch
    import paged_kv_cache_176_amd as pk
    import workloads
    w = workloads.prefill_chunks()
    dev = "cuda:0"
    st = w.cache_init.to(dev)
    d = pk.CacheDesc.from_geom(st, w.geom)
    q, key, val, slots, bt = (w.q.to(dev), w.key.to(dev), w.value.to(dev), w.slot_mapping.to(dev),
                              w.block_tables.to(dev))
    C = w.extra["chunk"]
    T = q.shape[0]
    out = torch.empty(T, 32, 128, dtype=torch.bfloat16, device=dev)
    qsl = torch.tensor([0, C], dtype=torch.int32, device=dev)
    seqs = [torch.tensor([(c + 1) * C], dtype=torch.int32, device=dev) for c in range(T // C)]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T // C)]
    wev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(T // C)]

    def one(i, pev):
        if pev is not None:
            pev[0].record()
        for c in range(T // C):
            sl = slice(c * C, (c + 1) * C)
            wev[c][0].record()
            pk.cache_write(key[sl], val[sl], slots[sl], d)
            wev[c][1].record()
            ev[c][0].record()
            pk.prefill_causal(q[sl], qsl, seqs[c], bt, d, w.softmax_scale, C, out=out[sl], with_lse=False)
            ev[c][1].record()
        if pev is not None:
            pev[1].record()

    dt, _, _ = time_steps(one, steps, warmup)
    # per-chunk kernel times: median over instrumented passes
    passes, wpasses, totals = [], [], []
    for _ in range(max(5, steps)):
        one(0, None)
        torch.cuda.synchronize()
        passes.append([a.elapsed_time(b) / 1e3 for a, b in ev])
        wpasses.append([a.elapsed_time(b) / 1e3 for a, b in wev])
        totals.append(sum(passes[-1]))
    kern = [sorted(p[c] for p in passes)[len(passes) // 2] for c in range(T // C)]
    wmed = float(np.median([x for p in wpasses for x in p]))
    visible = sum((c * C) * C + C * (C + 1) // 2 for c in range(T // C))     # causal pairs per head
    flops = 2 * visible * 32 * (192 + 128)
    chunk_write_bytes = C * 4 * (192 + 128) * 2 * 2          # K/V sources read + cache rows written
    res = dict(workload="prefill_32768_in_4096_chunks_bs16", ms_per_pass=dt * 1e3, tflops=flops / dt / 1e12,
               kernel_ms=sum(kern) * 1e3, kernel_tflops=flops / sum(kern) / 1e12,
               frac_of_bf16_peak=flops / sum(kern) / 1e12 / BF16_PEAK_TFLOPS,
               kernel_ms_pcts={k: round(v / 1e3, 4) for k, v in pcts(totals).items()},
               per_chunk_kernel_ms=[round(k * 1e3, 4) for k in kern],
               cache_write_4096=dict(us=round(wmed * 1e6, 2), bytes=chunk_write_bytes,
                                     gbs=round(chunk_write_bytes / wmed / 1e9, 1)))
    if cpu:
        # the oracle on a 128-query slab of the last chunk (queries 28672..28799 over up to 28800 keys)
        rows = list(range(7 * C, 7 * C + 128))
        slab_flops = 2 * 32 * (192 + 128) * sum(r + 1 for r in rows)

        def job():
            sec, n = oracle_seconds(w, 2.0, with_write=False, rows=rows)
            line = cpu_line(sec, n, slab_flops, "TFLOP/s", "128 query rows of chunk 7 (all 32 heads), fp64 oracle")
            line["est_s_whole_prefill"] = round(flops / (line["value"] * 1e12), 1)
            res["cpu_oracle"] = line
        DEFERRED.append(job)
    return res


def fp8_verify_calls(mode, P):
    """The fp8 verify workload resident on the GPU (cache copies rotated past the MALL) and one
    prepared attn_verify call per copy; returns (workload, calls)."""
    import torch
    import paged_kv_cache_176_amd as pk
    import workloads
    w = workloads.fp8_verify(scale_mode=mode)
    dev = "cuda:0"
    st = w.cache_init.to(dev)
    ks, vs = w.k_scale.to(dev), w.v_scale.to(dev)
    d0 = pk.CacheDesc.from_geom(st, w.geom, ks, vs, mode)
    pk.cache_write(w.key.to(dev), w.value.to(dev), w.slot_mapping.to(dev), d0)
    torch.cuda.synchronize()
    nbytes = st.numel()
    copies = [st] + [st.clone() for _ in range(_copies(nbytes) - 1)]
    descs = [pk.CacheDesc.from_geom(s, w.geom, ks, vs, mode) for s in copies]
    q, qsl, sl, bt = w.q.to(dev), w.query_start_loc.to(dev), w.seq_lens.to(dev), w.block_tables.to(dev)
    T = q.shape[0]
    ws = pk.new_workspace(T, 32, 128, P, dev)
    out = torch.empty(T, 32, 128, dtype=torch.bfloat16, device=dev)

    calls = [pk.verify(q, qsl, sl, bt, d, w.softmax_scale, w.max_query_len, P, out=out, workspace=ws,
                       with_lse=False, prepare=True) for d in descs]
    return w, calls


def run_verify(mode, steps, warmup, P, cpu=True):
    w, calls = fp8_verify_calls(mode, P)

    def one(i, ev):
        if ev is not None:
            ev[0].record()
        calls[i % len(calls)]()
        if ev is not None:
            ev[1].record()

    dt, _, _ = time_steps(one, steps, warmup)
    _, kern, per = time_steps(one, steps, 0, events=True)
    kv = 4 * 46080 * 4 * 320
    res = dict(workload=f"fp8_verify_b4_s46080_l4_{mode}", P=P, us_per_call=round(dt * 1e6, 2),
               kernel_us=round(kern * 1e6, 2), kernel_us_pcts=pcts(per), kv_gbs=round(kv / kern / 1e9, 1),
               call_gbs=round(kv / dt / 1e9, 1))
    if cpu:
        defer_cpu(res, lambda: oracle_seconds(w, 2.0, with_write=False), kv, "GB/s",
                  "the whole verify call (4 x 4 query rows + 4 padded rows), fp64 oracle on the fp8 cache bytes")
    return res


def decode_line(c, name, steps, warmup, cpu, cpu_rows=None, cpu_scale=1.0, cpu_sample=None):
    """Timing of one DecodeCase: event-free steps, an instrumented pass (per-step events),
    the partial kernel back to back and per launch, and (cpu) the oracle on a sample."""
    d, _, _ = time_steps(c.step, steps, warmup)
    _, se, sper = time_steps(c.step, steps, 0, events=True)
    k = c.time_partial(steps)
    kper = c.partial_samples(steps)
    res = dict(workload=name, P=c.P, us_per_step=round(d * 1e6, 2), step_us_events=round(se * 1e6, 2),
               step_us_events_pcts=pcts(sper), partial_kernel_us=round(k * 1e6, 2),
               partial_kernel_us_pcts=pcts(kper), kv_gbs=round(c.kv_bytes / k / 1e9, 1),
               step_gbs=round((c.kv_bytes + c.other_bytes) / d / 1e9, 1),
               tflops=round(c.flops / k / 1e12, 2))
    if cpu:
        w = c.w
        defer_cpu(res, lambda: oracle_seconds(w, 2.0, with_write=cpu_rows is None, rows=cpu_rows),
                  c.kv_bytes + c.other_bytes, "GB/s", cpu_sample or "a whole decode step (cache write + fp64 attention)",
                  cpu_scale)
    return res


def run_mla(batch, steps, warmup, cpu=True):
    import workloads
    p = auto_partitions(batch, 1, 100000)
    c = DecodeCase(workloads.mla_decode(batch, 100000), p)
    if batch == 1:
        return decode_line(c, "mla_b1_s100000_h12", steps, warmup, cpu)
    return decode_line(c, f"mla_b{batch}_s100000_h12", steps, warmup, cpu, cpu_rows=[0], cpu_scale=batch,
                       cpu_sample=f"1 of the {batch} sequences (fp64 attention over its 100000 keys), x{batch}")


def mla_verify_calls(batch, qlen=4):
    """The MLA verify workload resident on the GPU (cache copies rotated past the MALL) and one
    prepared attn_verify call per copy; returns (workload, calls, P)."""
    import torch
    import paged_kv_cache_176_amd as pk
    import workloads
    w = workloads.mla_verify(batch, 100000, qlen=qlen)
    dev = "cuda:0"
    img = w.cache_init.clone()
    workloads.place_bf16_rows(img, w.geom, w.extra["pre_slots"], w.extra["pre_key"], w.extra["pre_value"])
    nbytes = img.numel() * img.element_size()
    copies = [img.to(dev) for _ in range(1 if nbytes > 4 * MALL_BYTES else _copies(nbytes))]
    descs = [pk.CacheDesc.from_geom(c, w.geom) for c in copies]
    key, slots = w.key.to(dev), w.slot_mapping.to(dev)
    for d in descs:
        pk.cache_write(key, None, slots, d)
    q, qsl, sl, bt = w.q.to(dev), w.query_start_loc.to(dev), w.seq_lens.to(dev), w.block_tables.to(dev)
    T = q.shape[0]
    P = auto_partitions(batch, 1, 100000)
    ws = pk.new_workspace(T, 12, 512, P, dev)
    out = torch.empty(T, 12, 512, dtype=torch.bfloat16, device=dev)

    calls = [pk.verify(q, qsl, sl, bt, d, w.softmax_scale, qlen, P, out=out, workspace=ws, with_lse=False,
                       prepare=True) for d in descs]
    return w, calls, P


def run_mla_verify(batch, steps, warmup, qlen=4, cpu=True):
    """MLA verify: qlen query tokens per sequence (drafts + 1) over the 12-head latent
    cache, S = 100000, rotating cache copies; one attn_verify call (partials, then the merge)."""
    w, calls, P = mla_verify_calls(batch, qlen)

    def one(i, ev):
        if ev is not None:
            ev[0].record()
        calls[i % len(calls)]()
        if ev is not None:
            ev[1].record()

    dt, _, _ = time_steps(one, steps, warmup)
    _, kern, per = time_steps(one, steps, 0, events=True)
    kv = batch * 100000 * 576 * 2
    flops = 2 * batch * qlen * 12 * 100000 * (576 + 512)
    res = dict(workload=f"mla_verify_b{batch}_s100000_l{qlen}_h12", P=P, us_per_call=round(dt * 1e6, 2),
               kernel_us=round(kern * 1e6, 2), kernel_us_pcts=pcts(per), kv_gbs=round(kv / dt / 1e9, 1),
               tflops=round(flops / dt / 1e12, 1))
    if cpu:
        rows = list(range(qlen))
        defer_cpu(res, lambda: oracle_seconds(w, 2.0, with_write=False, rows=rows), kv, "GB/s",
                  f"the {qlen} query rows of 1 of the {batch} sequence(s), fp64 oracle, x{batch}", scale=batch)
    return res


def run_decode_extra(b, s, bs, steps, warmup, cpu=True):
    import workloads
    p = auto_partitions(b, 4, s, wgs_per_cu=2)
    c = DecodeCase(workloads.long_decode(b, s, bs), p)
    return decode_line(c, f"decode_b{b}_s{s}_bs{bs}", steps, warmup, cpu)


MIXED_LENS = [131072, 65536, 16384, 8192, 4096, 2048, 1024, 256]
# context buckets -> active splits for the mixed decode batch (launch P 64), chosen by the
# measured sweep below (`--only policy_sweep`): the candidates that cut the splits of the
# mid-length sequences further, or that let the long ones take more than 64, all measured
# slower than a plain 64 (every inactive workgroup still costs a dispatch and a prologue);
# halving the splits of sequences up to 4096 keys ties or beats it
MIXED_POLICY = [(4096, 32), (1 << 30, 64)]
POLICY_CANDIDATES = [
    ("fixed64", 64, None),
    ("short32", 64, MIXED_POLICY),
    ("short16", 64, [(1024, 16), (1 << 30, 64)]),
    ("tail8", 64, [(256, 8), (2048, 32), (1 << 30, 64)]),
    ("512keys", 64, [(2048, 4), (8192, 16), (32768, 32), (1 << 30, 64)]),
    ("long96", 96, [(32768, 64), (1 << 30, 96)]),
    ("geo1024", 128, [(1024, 1), (2048, 2), (4096, 4), (8192, 8), (16384, 16), (32768, 32), (65536, 64),
                      (1 << 30, 128)]),
]


def run_decode_mixed(steps, warmup, cpu=True):
    """Decode over a batch of mixed context lengths: the split policy (launch P 64, active
    splits per sequence from MIXED_POLICY) against fixed split counts for every sequence."""
    import torch
    import workloads
    w = workloads.paged_workload("decode_mixed", workloads.diffkv_geom(0, 16), MIXED_LENS, [1] * len(MIXED_LENS), 32,
                                 1.0 / math.sqrt(192), seed=0, write_all=False)
    res = {"workload": "decode_mixed_b8_bs16", "lens": MIXED_LENS, "policy": MIXED_POLICY}
    for name, P, pol in (("policy_P64", 64, MIXED_POLICY), ("fixed_P16", 16, None), ("fixed_P64", 64, None)):
        c = DecodeCase(w, P, policy=pol)
        d, _, _ = time_steps(c.step, steps, warmup)
        _, _, sper = time_steps(c.step, steps, 0, events=True)
        res[name] = dict(us_per_step=round(d * 1e6, 2), step_us_events_pcts=pcts(sper),
                         kv_gbs=round(c.kv_bytes / d / 1e9, 1))
        algo = c.kv_bytes + c.other_bytes
        del c
        torch.cuda.empty_cache()
    if cpu:
        defer_cpu(res, lambda: oracle_seconds(w, 2.0, with_write=True), algo, "GB/s",
                  "a whole decode step of the 8 sequences (cache write + fp64 attention)")
    return res


def run_policy_sweep(steps, warmup):
    """The split-policy candidates on the mixed batch, each timed twice (event-free steps)."""
    import torch
    import workloads
    w = workloads.paged_workload("decode_mixed", workloads.diffkv_geom(0, 16), MIXED_LENS, [1] * len(MIXED_LENS), 32,
                                 1.0 / math.sqrt(192), seed=0, write_all=False)
    res = {"workload": "decode_mixed_b8_bs16", "lens": MIXED_LENS, "us_per_step": {}}
    for rep in range(2):
        for name, P, pol in POLICY_CANDIDATES:
            c = DecodeCase(w, P, policy=pol)
            d, _, _ = time_steps(c.step, steps, warmup)
            res["us_per_step"].setdefault(name, []).append(round(d * 1e6, 2))
            del c
            torch.cuda.empty_cache()
    res["policies"] = {name: {"P": P, "policy": pol} for name, P, pol in POLICY_CANDIDATES}
    return res


def copy_rate(dev="cuda:0", nbytes=2 << 30, reps=10):
    """A plain device-to-device copy (torch's copy kernel) of nbytes: (read + write bytes) /
    median time, the reference rate each HBM-bound line is also quoted against."""
    import numpy as np
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in evs:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    t = float(np.median([a.elapsed_time(b) / 1e3 for a, b in evs]))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_moved": 2 * nbytes, "us": round(t * 1e6, 1), "gbs": round(2 * nbytes / t / 1e9, 1),
            "kernel": "torch device-to-device copy_ of 2 GiB (read + write counted)"}


def sample_clocks(fn, seconds=1.5):
    """Engine clocks while `fn` runs back to back: `amd-smi metric -c` taken once, halfway
    through a window of `seconds` (current gfx clock of each XCD and the memory clock), or
    None where the tool is not available."""
    import subprocess
    import threading
    import torch
    sample = {}

    def probe():
        time.sleep(seconds / 2)
        try:
            r = subprocess.run(["amd-smi", "metric", "-c", "-g", "0", "--json"], capture_output=True, text=True,
                               timeout=20)
            sample["json"] = r.stdout
        except Exception as e:                       # noqa: BLE001 - the clocks are informative only
            sample["err"] = str(e)

    th = threading.Thread(target=probe)
    th.start()
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end or th.is_alive():
        fn(i, None)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    th.join()
    return parse_clocks(sample.get("json"))


def parse_clocks(text):
    """gfx clocks (MHz) of every XCD and the memory clock from amd-smi's JSON, or None."""
    if not text:
        return None
    try:
        d = json.loads(text)
        d = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else (d[0] if isinstance(d, list) else d)
        clk = d["clock"]
    except (ValueError, KeyError, IndexError, TypeError):
        return None
    gfx = [v["clk"]["value"] for k, v in clk.items() if k.startswith("gfx") and isinstance(v, dict)
           and isinstance(v.get("clk"), dict) and isinstance(v["clk"].get("value"), (int, float))]
    mem = [v["clk"]["value"] for k, v in clk.items() if k.startswith("mem") and isinstance(v, dict)
           and isinstance(v.get("clk"), dict) and isinstance(v["clk"].get("value"), (int, float))]
    if not gfx:
        return None
    return {"gfx_mhz_per_xcd": gfx, "gfx_mhz_mean": round(sum(gfx) / len(gfx), 1), "mem_mhz": mem[0] if mem else None,
            "source": "amd-smi metric -c, sampled mid-run"}


def run_only(name, steps, warmup):
    """One secondary workload alone, without the oracle (the profiling commands)."""
    if name == "prefill":
        return run_prefill(max(1, min(steps, 5)), max(1, min(warmup, 3)), cpu=False)
    if name == "fp8_verify":
        return run_verify("tensor", steps, warmup, auto_partitions(4, 4, 46080), cpu=False)
    if name == "mla_b1":
        return run_mla(1, steps, warmup, cpu=False)
    if name == "mla_b16":
        return run_mla(16, steps, warmup, cpu=False)
    if name == "mla_verify_b1":
        return run_mla_verify(1, steps, warmup, cpu=False)
    if name == "mla_verify_b16":
        return run_mla_verify(16, steps, warmup, cpu=False)
    if name == "decode_mixed":
        return run_decode_mixed(steps, warmup, cpu=False)
    if name == "copy":
        return copy_rate()
    if name == "policy_sweep":
        return run_policy_sweep(steps, warmup)
    return run_decode_extra(8, 8192, 16, steps, warmup, cpu=False)


def main():
    global SPINUP_MS, PARTITIONS_OVERRIDE
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partitions", type=int, default=0, help="split count (0 = auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-clocks", action="store_true", help="skip the amd-smi clock sample")
    ap.add_argument("--spinup-ms", type=float, default=SPINUP_MS,
                    help="untimed running of each measured step before its warmup steps (GPU clock spin-up)")
    ap.add_argument("--only", choices=["prefill", "fp8_verify", "mla_b1", "mla_b16", "mla_verify_b1", "mla_verify_b16",
                             "decode_mixed", "decode_b8", "copy", "policy_sweep"], default=None,
                    help="run just this secondary workload and print its JSON line (for profiling)")
    ap.add_argument("--phase-stamps", choices=sorted(STAMP_CASES), default=None,
                    help="load the library built with the partial kernels' phase stamps and print the per-wave "
                         "timeline of this workload (diagnostics; no timing line)")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="print the matrix-core issue probe's table (libmfma_probe.so) and exit")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed region, one device-to-device copy of this many MiB (a kernel of known "
                         "size that calibrates hardware byte counters)")
    args = ap.parse_args()
    SPINUP_MS = args.spinup_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_176_amd as pk
    import workloads
    if args.mfma_probe:
        assert torch.cuda.is_available(), "bench.py needs the GPU"
        print(json.dumps(mfma_probe()), flush=True)
        return
    if args.phase_stamps:
        from paged_kv_cache_176_amd import build as pkb
        pk.ops.use_library(pkb.STAMPS_LIB)
        assert torch.cuda.is_available(), "bench.py needs the GPU"
        print(json.dumps(phase_stamps(args.phase_stamps)), flush=True)
        return
    pk.load_library()
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.only:
        PARTITIONS_OVERRIDE = args.partitions
        res = run_only(args.only, args.steps, args.warmup)
        if args.copy_probe_mib:
            res["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
        print(json.dumps(res), flush=True)
        return

    B, S, BS = 1, 131072, 16
    P = args.partitions or auto_partitions(B, 4, S, wgs_per_cu=2)
    w = workloads.long_decode(B, S, BS)
    case = DecodeCase(w, P)
    # the timed steps (nothing but the step's kernels between the synchronisations); then,
    # outside the timed region, the partial kernel alone launched back to back (its
    # duration for the roofline) and per launch (its spread), a pass with HIP events around
    # each step (the per-step device figure, which carries the events' own overhead), and the
    # engine clocks while the step runs back to back
    dt, _, _ = time_steps(case.step, args.steps, args.warmup)
    kern = case.time_partial(args.steps)
    kper = case.partial_samples(max(args.steps, 20))
    _, step_ev, sper = time_steps(case.step, max(min(args.steps, 50), 20), 0, events=True)
    clocks = None if args.no_clocks else sample_clocks(case.step)
    algo = case.kv_bytes + case.other_bytes
    value = algo / dt / 1e9
    achieved = case.kv_bytes / kern / 1e9
    line = {
        "metric": "decode attn KV-read GB/s (% HBM peak) + prefill TFLOP/s, K192/V128 bf16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup_ms": SPINUP_MS,
        "ms_per_step": round(dt * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode_b{B}_s{S}_bs{BS}", "batch": B, "context": S, "q_heads": 32, "kv_heads": 4,
                   "head_dim_k": 192, "head_dim_v": 128, "block_size": BS, "partitions": P,
                   "cache_copies_rotated": case.ncopy, "step": "attn_decode_splitkv_append: split-KV partial kernel with the new token's K/V write fused in, then the merge",
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": MEASURED_TRAFFIC.get((_kernel_source_hash(), P)),
                     "kernel": "splitkv_dma_kernel<192,128,192,1 row group,2 stages,bf16,nontemporal>",
                     "kernel_us": round(kern * 1e6, 3), "kernel_us_per_launch_pcts": pcts(kper),
                     "step_us_with_events": round(step_ev * 1e6, 3), "step_us_with_events_pcts": pcts(sper),
                     "algorithmic_bytes_per_launch": case.kv_bytes},
        "clocks": clocks,
    }
    del case
    torch.cuda.empty_cache()
    copy = copy_rate()
    line["copy_reference"] = copy
    line["roofline"]["frac_of_copy"] = round(achieved / copy["gbs"], 4)
    line["config"]["frac_of_copy"] = round(value / copy["gbs"], 4)
    if not args.no_extra:
        cpu = not args.no_cpu_baseline
        extra = {}
        for (b2, s2, bs2) in [(1, 131072, 64), (8, 8192, 16), (8, 8192, 64)]:
            extra[f"decode_b{b2}_s{s2}_bs{bs2}"] = run_decode_extra(b2, s2, bs2, 100, 10, cpu=cpu)
            torch.cuda.empty_cache()
        for b2 in (1, 16):
            extra[f"mla_b{b2}_s100000_h12"] = run_mla(b2, 50, 5, cpu=cpu)
            torch.cuda.empty_cache()
        extra["decode_mixed_b8_bs16"] = run_decode_mixed(100, 10, cpu=cpu)
        torch.cuda.empty_cache()
        for b2 in (1, 16):
            extra[f"mla_verify_b{b2}_s100000_l4_h12"] = run_mla_verify(b2, 50, 5, cpu=cpu)
            torch.cuda.empty_cache()
        for mode in ("tensor", "head"):
            extra[f"fp8_verify_{mode}"] = run_verify(mode, 100, 10, auto_partitions(4, 4, 46080), cpu=cpu)
        extra["prefill"] = run_prefill(5, 3, cpu=cpu)
        for v in extra.values():                       # each HBM-bound line against the copy rate
            if "kv_gbs" in v:
                v["kv_frac_of_copy"] = round(v["kv_gbs"] / copy["gbs"], 4)
        line["extra"] = extra
        torch.cuda.empty_cache()
    # the oracle, after every GPU measurement: the headline's baseline, then the other lines'
    if not args.no_cpu_baseline:
        cdt, n, cores, info = cpu_baseline(w)
        line["cpu_baseline"] = {"value": round(algo / cdt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                                "sample": f"{n} whole decode step(s) of the same workload (cache write + fp64 "
                                          f"attention over all 131072 keys), {cdt:.2f} s each",
                                **info}
        for job in DEFERRED:
            job()
        DEFERRED.clear()
    if args.copy_probe_mib:
        line["copy_probe_bytes"] = copy_probe(args.copy_probe_mib)
    print(json.dumps(line), flush=True)


STAMP_CASES = {   # name -> (kernel's stamp reader, waves per workgroup, setup returning (grid size, launch fn))
    "decode_b1": ("attn_phase_stamps_read", 4, lambda: _stamp_decode(lambda w: w.long_decode(1, 131072, 16), 4, 2)),
    "decode_b8": ("attn_phase_stamps_read", 4, lambda: _stamp_decode(lambda w: w.long_decode(8, 8192, 16), 4, 2)),
    "mla_b1": ("attn_phase_stamps_read", 4, lambda: _stamp_decode(lambda w: w.mla_decode(1, 100000), 1, 1)),
    "mla_b16": ("attn_phase_stamps_read", 4, lambda: _stamp_decode(lambda w: w.mla_decode(16, 100000), 1, 1)),
    "fp8_verify": ("attn_phase_stamps_read_wide", 4, lambda: _stamp_fp8_verify()),
    "mla_verify_b1": ("attn_phase_stamps_read_tokens", 8, lambda: _stamp_mla_verify(1)),
    "mla_verify_b16": ("attn_phase_stamps_read_tokens", 8, lambda: _stamp_mla_verify(16)),
}


def _stamp_decode(make, kv_heads, wgs_per_cu):
    import workloads
    w = make(workloads)
    B, S = int(w.seq_lens.numel()), int(w.seq_lens.max())
    P = auto_partitions(B, kv_heads, S, wgs_per_cu=wgs_per_cu)
    c = DecodeCase(w, P)
    return P, P * kv_heads * B, c.partial


def _stamp_fp8_verify():
    P = auto_partitions(4, 4, 46080)
    w, calls = fp8_verify_calls("tensor", P)
    return P, P * 4 * int(w.seq_lens.numel()), lambda i: calls[i % len(calls)]()


def _stamp_mla_verify(batch):
    w, calls, P = mla_verify_calls(batch)
    return P, P * 1 * batch, lambda i: calls[i % len(calls)]()   # one token group of 4 per sequence


def mfma_probe():
    """The matrix-core issue probe (libmfma_probe.so, built beside the library): for each
    configuration, cycles per v_mfma_f32_32x32x16_bf16 per SIMD and, where a wave runs only
    VALU beside an MFMA wave, that wave's cycles per instruction."""
    import ctypes
    from paged_kv_cache_176_amd import build as pkb
    if not os.path.exists(pkb.PROBE_LIB):
        raise RuntimeError(f"{pkb.PROBE_LIB} is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(pkb.PROBE_LIB)
    lib.mfma_probe_label.restype = ctypes.c_char_p
    lib.mfma_probe_run.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    rows = []
    for i in range(lib.mfma_probe_count()):
        res = (ctypes.c_double * 3)()
        rc = lib.mfma_probe_run(i, res)
        if rc != 0:
            raise RuntimeError(f"mfma probe configuration {i} failed ({rc})")
        rows.append({"config": lib.mfma_probe_label(i).decode(), "cycles_per_mfma_per_simd": round(res[0], 1),
                     "valu_wave_cycles_per_instruction": round(res[1], 2) if res[1] >= 0 else None})
    return {"probe": "v_mfma_f32_32x32x16_bf16 issue, 256 workgroups x 2000 iterations, s_memtime cycles",
            "rows": rows}


def phase_stamps(name, launches=40):
    """Per-wave phase timeline of a split-KV partial kernel (decode, fp8 verify or MLA verify),
    from the library built with the kernels' phase stamps (the last of `launches` back-to-back
    launches): percentiles over the waves of each phase's time from the first wave's entry, of the
    per-tile (per-step for MLA verify) wait and compute, and the end time per XCC."""
    import ctypes
    import numpy as np
    import torch
    import paged_kv_cache_176_amd as pk
    lib = pk.load_library()
    reader_name, wpw, setup = STAMP_CASES[name]
    P, wgs, launch = setup()
    for i in range(launches):
        launch(i)
    reader = getattr(lib, reader_name)
    waves = wgs * wpw
    buf = np.zeros(waves * 64, dtype=np.uint32)
    torch.cuda.synchronize()
    reader.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    rc = reader(buf.ctypes.data, buf.size)
    if rc != 0:
        raise RuntimeError(f"reading the phase stamps failed ({rc})")
    st = buf.reshape(waves, 64).astype(np.int64)
    st = st[st[:, 58] > 0]             # workgroups with no key (the padded verify rows) exit at once
    waves = len(st)
    rel = (st - st[:, 0].min()) * 0.01                 # s_memrealtime ticks at 100 MHz -> us
    q = lambda a: {k: round(float(np.percentile(a, v)), 2) for k, v in (("min", 0), ("p10", 10), ("p50", 50),
                                                                         ("p90", 90), ("max", 100))}
    ntiles = st[:, 58]
    res = {"workload": name, "partitions": P, "waves": waves, "tiles_per_wave": sorted(set(ntiles.tolist())),
           "us_from_first_entry": {"entry": q(rel[:, 0]), "prologue_issued": q(rel[:, 1]),
                                   "q_landed": q(rel[:, 2]), "first_tile_ready": q(rel[:, 3]),
                                   "loop_end": q(rel[:, 60]),
                                   "epilogue_barrier": q(rel[:, 61]), "end": q(rel[:, 62])}}
    tiles = []
    for k in range(min(int(ntiles.max()), 27)):       # over the waves that consume a k-th tile
        r = rel[ntiles > k]
        # tile 0 waits from the later of Q's landing and the prologue's issue
        wait = r[:, 3 + 2 * k] - (np.maximum(r[:, 1], r[:, 2]) if k == 0 else r[:, 4 + 2 * (k - 1)])
        tiles.append({"tile": k, "waves": int(len(r)), "wait_us": q(wait),
                      "compute_us": q(r[:, 4 + 2 * k] - r[:, 3 + 2 * k])})
    res["tiles"] = tiles
    xcc = st[:, 59] & 0xF
    res["end_us_by_xcc"] = {int(x): q(rel[xcc == x, 62]) for x in np.unique(xcc)}
    res["corr_first_tile_vs_loop_end"] = round(float(np.corrcoef(rel[:, 3], rel[:, 60])[0, 1]), 3)
    return res


def copy_probe(mib):
    """One device-to-device copy of `mib` MiB after the measured work: a kernel of known size
    whose counter readings calibrate FETCH_SIZE / WRITE_SIZE in a profiled run."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n


if __name__ == "__main__":
    main()
