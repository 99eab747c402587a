"""Benchmark of the paged-attention hot path on one MI355X.

Headline workload: one LLaMA-2-7B-shaped attention layer at decode -- batch
64, 32 q = 32 kv heads, head_dim 128, fp16, block size 16, lengths uniform in
[512, 4096] (seed 2), blocks scattered by a seeded permutation over a pool of
16384 blocks.  One step = the cache write of the 64 new tokens followed by
paged decode (partition kernel + merge kernel).  ``value`` is effective KV
bandwidth: K+V bytes of all live tokens (each kv head's tile counted once)
divided by the step time, inputs resident in HBM.

Printed: one JSON line with the headline metric, a ``roofline`` object for
the dominant kernel (the decode partition kernel, timed with HIP events on
the stream it runs on), a ``cpu_baseline`` object (the float64 oracle on a
bounded sample of the same workload, on this host's cores) and
``secondary`` measurements of the other workloads (GQA + shared prefix,
chunked prefill, long-context split-KV, tiny decode, block copy) and of the
decode workloads over an FP8 (E4M3) cache.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--quick]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16/fp16 MFMA, TFLOP/s
METRIC = "paged-decode effective KV GB/s (% of MI355X HBM peak); decode tokens/s"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "decode_balanced_llama2_7b_layer_traffic.json")
# the decode kernels' sources: counter runs stay valid while these are unchanged
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_24_amd", "csrc", f)
                  for f in ("decode.hip", "common.h", "kernels.h")]


def _decode_sources_sha256():
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU budget of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM counters)")
    ap.add_argument("--workload", choices=sorted(_ONE_WORKLOAD),
                    help="run only this workload and print its line (for profilers)")
    ap.add_argument("--traffic-profile", metavar="DIR",
                    help="no GPU work: read the rocprofv3 FETCH_SIZE / WRITE_SIZE runs under "
                         "DIR/{dec,copy}_{FETCH_SIZE,WRITE_SIZE} and write the decode "
                         "partition kernel's HBM traffic JSON to stdout")
    return ap.parse_args()


def _dev(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.float16 if dtype == "f16" else torch.bfloat16)


def _i(a, dt=None):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dt or torch.int32).to("cuda")


class _Timer:
    """Per-kernel HIP events on the current stream, summed over steps."""

    def __init__(self, names):
        self.names = names
        self.events = []

    def step(self):
        import torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]
        self.events.append(ev)
        return ev

    def samples(self, name):
        i = self.names.index(name)
        return np.array([ev[i].elapsed_time(ev[i + 1]) for ev in self.events])

    def mean_ms(self):
        return {n: float(np.mean(self.samples(n))) for n in self.names}

    def spread_ms(self, name):
        x = self.samples(name)
        return {"p10": round(float(np.percentile(x, 10)), 4), "p50": round(float(np.median(x)), 4),
                "p90": round(float(np.percentile(x, 90)), 4)}


def _settle(step, min_s=0.3):
    """Run `step` untimed until the GPU has been busy for `min_s` seconds.  After
    the host-side set-up of a workload the GPU clock is still low and a few
    warm-up steps do not raise it: measured, the first configuration timed after
    a set-up ran up to 9% slower than the same configuration timed again."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


# ------------------------------------------------------------------ decode workloads

class DecodeRun:
    def __init__(self, case, partition_tokens=0, groups=False):
        import torch
        import paged_kv_cache_24_amd as pa
        self.pa = pa
        self.c = case
        self.q = _dev(case.q, case.dtype)
        self.kc = _dev(case.k_cache, case.dtype)
        self.vc = _dev(case.v_cache, case.dtype)
        self.key = _dev(case.key, case.dtype)
        self.value = _dev(case.value, case.dtype)
        self.slots = _i(case.slot_mapping, torch.int64)
        self.tables = _i(case.block_tables)
        self.lens = _i(case.seq_lens)
        self.out = torch.empty_like(self.q)
        # 0: the library's default split (the balanced split where fixed partitions
        # would need several rounds of waves); `split` records which one it makes
        self.part = partition_tokens
        split = pa.pa_decode_split(case.num_seqs, case.num_q_heads, case.num_kv_heads, case.head_dim,
                                   case.block_size, case.max_blocks_per_seq, self.part)
        self.split = "balanced" if split == pa.PA_PARTITION_BALANCED else f"partitions of {split} tokens"
        need = pa.pa_decode_workspace_size(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                           case.head_dim, case.block_size, case.max_blocks_per_seq,
                                           self.part)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        self.has_write = len(case.slot_mapping) > 0
        # the streaming hint is a promise that no physical block is read twice in the
        # call; a block manager knows it from its reference counts, here from the tables
        used = case.block_tables[case.block_tables >= 0]
        self.shared_blocks = len(np.unique(used)) < len(used)
        self.flags = 0 if self.shared_blocks else pa.PA_DECODE_STREAM_KV
        # sequence groups: a block manager with prefix caching knows that runs of
        # consecutive sequences share blocks; pa_decode then reads each shared
        # block once per group of 16 / (q heads per kv head) sequences, in one call
        # (plan, grouped split, merge)
        self.groups = groups
        if groups:
            self.flags |= pa.PA_DECODE_SHARED_PREFIX
            self.split = "sequence groups + balanced"

    def _write(self):
        self.pa.pa_reshape_and_cache(self.key, self.value, self.kc, self.vc, self.slots)

    def _partitions(self):
        pa, c = self.pa, self.c
        if self.groups:   # the phases run inside one call: all of it counts as "partitions"
            pa.pa_decode(self.out, self.q, self.kc, self.vc, self.tables, self.lens, c.scale, self.part,
                         workspace=self.ws, flags=self.flags)
            return
        pa.pa_decode_partitions(self.out, self.q, self.kc, self.vc, self.tables, self.lens, c.scale,
                                self.ws, self.part, flags=self.flags)

    def _merge(self):
        if not self.groups:
            c = self.c
            self.pa.pa_decode_merge(self.out, self.lens, c.num_kv_heads, c.max_blocks_per_seq, self.ws,
                                    self.part, block_size=c.block_size)

    def step(self, ev=None, part_only=False):
        """One step: cache write, decode partitions, merge.  ev: HIP events on the
        current stream -- four (before the write, after it, after the partitions,
        after the merge), or with part_only two, around the partitions alone."""
        full = ev is not None and not part_only
        if full:
            ev[0].record()
        if self.has_write:
            self._write()
        if ev is not None:
            ev[0 if part_only else 1].record()
        self._partitions()
        if ev is not None:
            ev[1 if part_only else 2].record()
        self._merge()
        if full:
            ev[3].record()

    def timed(self, steps, warmup):
        """Wall time per step over `steps` timed steps, with HIP events around the
        partition kernel only (events between kernels cost time: four per step
        add 3% here, two 1%); then the same number of untimed steps with events
        between every kernel for the per-kernel breakdown."""
        import torch
        _settle(self.step)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        part = _Timer(["partitions"])
        t0 = time.perf_counter()
        for _ in range(steps):
            self.step(part.step(), part_only=True)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
        timer = _Timer(["write", "partitions", "merge"])
        for _ in range(steps):
            self.step(timer.step())
        torch.cuda.synchronize()
        self.last_timer = part
        per = timer.mean_ms()
        per["partitions"] = part.mean_ms()["partitions"]   # the roofline's kernel: from the timed steps
        return wall_ms, per

    def timed_cold(self, steps, evict_bytes=512 << 20):
        """Per-step kernel times with a write of ``evict_bytes`` between steps
        (outside the events) so no K/V is left in the 256 MB Infinity Cache."""
        import torch
        scratch = torch.empty(evict_bytes, dtype=torch.uint8, device="cuda")
        timer = _Timer(["write", "partitions", "merge"])
        for _ in range(steps):
            scratch.fill_(1)
            self.step(timer.step())
        torch.cuda.synchronize()
        del scratch
        return timer

    def algorithmic_bytes(self):
        """Bytes any implementation of the decode partition kernel must move:
        K+V of the live tokens, q, the block-table entries read, the output."""
        c = self.c
        lens = c.seq_lens.astype(np.int64)
        elt = 2
        kv = int(lens.sum()) * 2 * c.num_kv_heads * c.head_dim * elt
        q = c.num_seqs * c.num_q_heads * c.head_dim * elt
        bs = c.block_size
        table = int(((lens + bs - 1) // bs).sum()) * 4
        out = c.num_seqs * c.num_q_heads * c.head_dim * elt
        return kv, kv + q + table + out

    def free(self):
        for k in ("q", "kc", "vc", "key", "value", "out", "ws"):
            setattr(self, k, None)


class Fp8DecodeRun(DecodeRun):
    """The same decode workload over an FP8 (E4M3) cache.  Set-up (untimed):
    the 16-bit pools after the cache write give every live token's k/v, which
    the library's FP8 cache write quantises into code and scale pools.  The
    timed step is the FP8 cache write of the new tokens plus FP8 decode."""

    def __init__(self, case, partition_tokens=0, groups=False):
        import torch
        super().__init__(case, partition_tokens, groups)
        pa, c = self.pa, case
        if self.has_write:
            pa.pa_reshape_and_cache(self.key, self.value, self.kc, self.vc, self.slots)
        lens = c.seq_lens.astype(np.int64)
        live = np.unique(np.concatenate([
            c.block_tables[b, np.arange(int(lens[b])) // 16].astype(np.int64) * 16
            + np.arange(int(lens[b])) % 16 for b in range(c.num_seqs)]))
        idx = _i(live, torch.int64)
        nb, hkv, d = c.num_blocks, c.num_kv_heads, c.head_dim
        self.kc8 = torch.full((nb, 16, hkv, d), 0x7F, dtype=torch.uint8, device="cuda")
        self.vc8 = torch.full_like(self.kc8, 0x7F)
        self.ks = torch.full((nb, hkv, 16), float("nan"), dtype=torch.float32, device="cuda")
        self.vs = torch.full_like(self.ks, float("nan"))
        for lo in range(0, len(live), 1 << 16):
            sl = idx[lo:lo + (1 << 16)]
            pa.pa_reshape_and_cache_fp8(
                self.kc.view(-1, hkv, d).index_select(0, sl).contiguous(),
                self.vc.view(-1, hkv, d).index_select(0, sl).contiguous(),
                self.kc8, self.vc8, self.ks, self.vs, sl.contiguous())
        torch.cuda.synchronize()
        self.kc = self.vc = None            # the 16-bit pools are not used by the timed step

    def _write(self):
        self.pa.pa_reshape_and_cache_fp8(self.key, self.value, self.kc8, self.vc8, self.ks, self.vs, self.slots)

    def _partitions(self):
        pa, c = self.pa, self.c
        if self.groups:   # the phases run inside one call: all of it counts as "partitions"
            pa.pa_decode_fp8(self.out, self.q, self.kc8, self.vc8, self.ks, self.vs, self.tables, self.lens,
                             c.scale, self.part, workspace=self.ws, flags=self.flags)
            return
        pa.pa_decode_partitions_fp8(self.out, self.q, self.kc8, self.vc8, self.ks, self.vs,
                                    self.tables, self.lens, c.scale, self.ws, self.part,
                                    flags=self.flags)

    def _merge(self):
        if not self.groups:
            c = self.c
            self.pa.pa_decode_merge(self.out, self.lens, c.num_kv_heads, c.max_blocks_per_seq, self.ws,
                                    self.part)

    def algorithmic_bytes(self):
        """K+V codes and their float32 scales of the live tokens, q, table, output."""
        c = self.c
        lens = c.seq_lens.astype(np.int64)
        kv = int(lens.sum()) * 2 * c.num_kv_heads * (c.head_dim + 4)
        q = c.num_seqs * c.num_q_heads * c.head_dim * 2
        table = int(((lens + 15) // 16).sum()) * 4
        return kv, kv + q + table + q

    def free(self):
        super().free()
        for k in ("kc8", "vc8", "ks", "vs"):
            setattr(self, k, None)


def _oracle_fp8_rate(case, budget_s=3.0):
    """The float64 oracle's FP8 decode on a bounded sample (whole sequences in
    order until the budget is spent; each sequence's tokens quantised by the
    oracle's cache write first, untimed): GB/s of codes + scales."""
    import oracle
    kc, vc = oracle.ref_reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                          case.slot_mapping)
    hkv, d = case.num_kv_heads, case.head_dim
    done, nbytes, spent = 0, 0, 0.0
    for b in range(case.num_seqs):
        n = int(case.seq_lens[b])
        nblk = (n + 15) // 16
        blocks = case.block_tables[b, :nblk]
        p = np.arange(n)
        slots = (p // 16) * 16 + p % 16                     # blocks renumbered 0..nblk-1
        key = kc[blocks[p // 16], p % 16]
        val = vc[blocks[p // 16], p % 16]
        codes0 = np.zeros((max(nblk, 1), 16, hkv, d), np.uint8)
        sc0 = np.ones((max(nblk, 1), hkv, 16), np.float32)
        k8, v8, ks, vs = oracle.ref_reshape_and_cache_fp8(key, val, codes0, codes0, sc0, sc0,
                                                          slots, case.dtype)
        table = np.arange(max(nblk, 1), dtype=np.int32)[None]
        t0 = time.perf_counter()
        oracle.ref_decode_fp8(case.q[b:b + 1], k8, v8, ks, vs, table, np.array([n]), case.scale,
                              case.dtype)
        spent += time.perf_counter() - t0
        done += 1
        nbytes += n * 2 * hkv * (d + 4)
        if spent > budget_s:
            break
    return {"value": round(nbytes / spent / 1e9, 3), "unit": "GB/s", "kind": "oracle",
            "sample": f"{done} of {case.num_seqs} sequences in {spent:.1f} s of attention "
                      "(the oracle's quantisation of their tokens not timed)"}


def _traffic_if_current():
    """HBM bytes per launch of the partition kernel from committed rocprofv3
    counter runs, valid only if the decode sources are unchanged since they were taken."""
    try:
        with open(PROFILE_TRAFFIC) as f:
            prof = json.load(f)
        if prof.get("decode_sources_sha256") != _decode_sources_sha256():
            return None
        return prof.get("hbm_bytes_per_launch")
    except (OSError, ValueError):
        return None


def _cpu_baseline(case, budget_s):
    """The float64 oracle on a bounded sample: sequences in order until the
    time budget is spent, after the same cache write."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    kc, vc = oracle.ref_reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                          case.slot_mapping)
    done, kv_bytes = 0, 0
    t0 = time.perf_counter()
    for b in range(case.num_seqs):
        n = int(case.seq_lens[b])
        oracle.ref_decode_one(case.q[b], kc, vc, case.block_tables[b], n, case.scale, case.dtype)
        done += 1
        kv_bytes += n * 2 * case.num_kv_heads * case.head_dim * 2
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": kv_bytes / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle decode of the first {done} of {case.num_seqs} sequences "
                      f"({kv_bytes / 1e9:.3f} GB of K+V) in {dt:.1f} s; "
                      f"{done / dt:.2f} sequences/s",
            "host": {"cpu_model": _cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}}


def _oracle_decode_rate(case, budget_s=3.0):
    """The float64 oracle on a bounded sample of a decode workload (whole
    sequences in order until the budget is spent): K+V GB/s."""
    import oracle
    kc, vc = oracle.ref_reshape_and_cache(case.key, case.value, case.k_cache, case.v_cache,
                                          case.slot_mapping)
    done, kv_bytes = 0, 0
    t0 = time.perf_counter()
    for b in range(case.num_seqs):
        n = int(case.seq_lens[b])
        oracle.ref_decode_one(case.q[b], kc, vc, case.block_tables[b], n, case.scale, case.dtype)
        done += 1
        kv_bytes += n * 2 * case.num_kv_heads * case.head_dim * 2
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(kv_bytes / dt / 1e9, 3), "unit": "GB/s", "kind": "oracle",
            "sample": f"{done} of {case.num_seqs} sequences in {dt:.1f} s"}


def _secondary_decode(builder, name, steps, warmup, note=None, cpu=True, fp8=False, groups=False):
    import torch
    case = builder()
    run = Fp8DecodeRun(case, groups=groups) if fp8 else DecodeRun(case, groups=groups)
    wall, per = run.timed(steps, warmup)
    kv, algo = run.algorithmic_bytes()
    dec_ms = per["partitions"] + per["merge"]
    res = {"workload": name, "ms_per_step": round(wall, 4), "decode_ms": round(dec_ms, 4),
           "partition_kernel_ms": round(per["partitions"], 4), "merge_ms": round(per["merge"], 4),
           "split": run.split, "block_size": case.block_size,
           "stream_kv": bool(run.flags & 1), "kv_bytes": kv,
           "kv_GBs": round(kv / (dec_ms * 1e-3) / 1e9, 1),
           "pct_hbm_peak": round(100 * kv / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
           "tokens_per_s": round(case.num_seqs / (dec_ms * 1e-3), 1)}
    if run.has_write:
        res["write_ms"] = round(per["write"], 4)
    if groups:
        del res["partition_kernel_ms"], res["merge_ms"]
        res["flags"] = "PA_DECODE_SHARED_PREFIX"
        res["phases"] = ("plan, grouped balanced split and merge in one pa_decode call; "
                         "kernel times in the rocprofv3 summary")
        run.free()
        plain = Fp8DecodeRun(case) if fp8 else DecodeRun(case)   # without the flag, for comparison
        _, pp = plain.timed(steps, warmup)
        res["decode_ms_without_groups"] = round(pp["partitions"] + pp["merge"], 4)
        plain.free()
    if note:
        res.update(note(case))
        if "unique_kv_bytes" in res:   # logical bytes can exceed the HBM peak where blocks are shared
            res["unique_kv_GBs"] = round(res["unique_kv_bytes"] / (dec_ms * 1e-3) / 1e9, 1)
    if fp8:
        res["kv_cache"] = "fp8 e4m3 codes + float32 scale per (token, kv head)"
        res["kv_bytes_16bit_equivalent"] = int(case.seq_lens.astype(np.int64).sum()) * 2 * \
            case.num_kv_heads * case.head_dim * 2
    if cpu:
        res["cpu_oracle"] = _oracle_fp8_rate(case) if fp8 else _oracle_decode_rate(case)
    run.free()
    del run, case
    torch.cuda.empty_cache()
    return res


def _secondary_tiny_latency(steps=200, warmup=20):
    """decode_tiny as a latency figure: one step (cache write of 4 tokens +
    decode) launched eagerly, and the same step captured once in a HIP graph
    and replayed; wall time per step with no events in between.  The same for
    pa_decode_step, whose decode kernels perform the cache write themselves
    (one kernel per step instead of two)."""
    import torch
    from workloads import decode_tiny
    case = decode_tiny()
    run = DecodeRun(case)
    assert len(case.slot_mapping) == case.num_seqs   # every sequence has a newest token

    def fused():
        run.pa.pa_decode_step(run.out, run.q, run.key, run.value, run.kc, run.vc, run.tables, run.lens,
                              case.scale, run.part, workspace=run.ws, flags=run.flags)

    def measure(step):
        _settle(step)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) * 1e6 / steps
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        replay = (time.perf_counter() - t0) * 1e6 / steps
        del graph
        return round(eager, 2), round(replay, 2)

    eager_us, graph_us = measure(run.step)
    fused_eager_us, fused_graph_us = measure(fused)
    run.free()
    del run
    torch.cuda.empty_cache()
    return {"workload": "decode_tiny_latency", "eager_us_per_step": eager_us,
            "graph_replay_us_per_step": graph_us,
            "decode_step_eager_us_per_step": fused_eager_us, "decode_step_graph_replay_us_per_step": fused_graph_us,
            "note": "write + decode of batch 4; wall clock over back-to-back steps, no events; "
                    "the graph holds the same kernel launches (one decode partition, no merge); "
                    "decode_step_*: pa_decode_step, the write inside the decode kernel"}


def _shared_prefix_note(case):
    used = np.unique(case.block_tables[case.block_tables >= 0])
    unique_tokens = 0
    lens = case.seq_lens.astype(np.int64)
    # unique bytes: each physical block read by any sequence, counting its live rows once
    rows = {}
    for b in range(case.num_seqs):
        n = int(lens[b])
        for j in range((n + 15) // 16):
            blk = int(case.block_tables[b, j])
            rows[blk] = max(rows.get(blk, 0), min(16, n - 16 * j))
    unique_tokens = sum(rows.values())
    unique = unique_tokens * 2 * case.num_kv_heads * case.head_dim * 2
    return {"unique_kv_bytes": unique, "blocks_used": int(len(used)),
            "note": "kv_GBs counts logical bytes (shared blocks once per sequence), so it can pass "
                    "the 8 TB/s HBM peak when shared blocks are read once for several sequences; "
                    "unique_kv_GBs counts each physical block once"}


def _oracle_prefill_rate(c, budget_s, fp8):
    """The float64 oracle's chunked prefill on a bounded sample: the first <= 64
    rows of each sequence, sequences in order until the budget is spent.  Over
    FP8 each sequence's keys are first quantised by the oracle's own FP8 cache
    write into blocks renumbered 0..n-1 (untimed); only the attention is timed."""
    import oracle
    L, ctxl = c.q_lens.astype(np.int64), c.ctx_lens.astype(np.int64)
    rk, rv = oracle.ref_reshape_and_cache(c.key, c.value, c.k_cache, c.v_cache, c.slot_mapping)
    hkv, d = c.num_kv_heads, c.head_dim
    done_pairs, spent, b = 0, 0.0, -1
    for b in range(c.num_seqs):
        lo = int(c.query_start_loc[b])
        rows = np.arange(min(int(L[b]), 64))
        if len(rows):
            table, kc, vc = c.block_tables[b], rk, rv
            n = int(ctxl[b]) + len(rows)
            if fp8:
                nblk = (n + 15) // 16
                p = np.arange(n)
                blocks = c.block_tables[b, p // 16]
                codes0 = np.zeros((nblk, 16, hkv, d), np.uint8)
                sc0 = np.ones((nblk, hkv, 16), np.float32)
                k8, v8, ks, vs = oracle.ref_reshape_and_cache_fp8(
                    rk[blocks, p % 16], rv[blocks, p % 16], codes0, codes0, sc0, sc0, p, c.dtype)
                table = np.arange(nblk, dtype=np.int32)
            t0 = time.perf_counter()
            if fp8:
                oracle.ref_prefill_rows_fp8(c.q, k8, v8, ks, vs, table, int(ctxl[b]), lo, rows,
                                            c.scale, c.dtype)
            else:
                oracle.ref_prefill_rows(c.q, kc, vc, table, int(ctxl[b]), lo, rows, c.scale,
                                        c.dtype)
            spent += time.perf_counter() - t0
            done_pairs += int((ctxl[b] + rows + 1).sum())
        if spent > budget_s:
            break
    return {"value": round(4 * c.num_q_heads * c.head_dim * done_pairs / spent / 1e12, 5),
            "unit": "TFLOP/s", "kind": "oracle",
            "sample": f"first <=64 rows of {b + 1} sequences ({done_pairs} (row, key) pairs per "
                      f"head) in {spent:.1f} s" + ("; keys quantised by the oracle's FP8 cache "
                                                   "write first, untimed" if fp8 else "")}


def _secondary_prefill(steps, warmup, oracle_budget_s=3.0, fp8=False):
    import torch
    import paged_kv_cache_24_amd as pa
    from workloads import prefill_chunked
    c = prefill_chunked()
    q = _dev(c.q, c.dtype)
    kc, vc = _dev(c.k_cache, c.dtype), _dev(c.v_cache, c.dtype)
    key, value = _dev(c.key, c.dtype), _dev(c.value, c.dtype)
    slots = _i(c.slot_mapping, torch.int64)
    tables, ctx, qsl = _i(c.block_tables), _i(c.ctx_lens), _i(c.query_start_loc)
    out = torch.empty_like(q)
    if fp8:
        # set-up (untimed): quantise the cached context into FP8 pools with the
        # library's FP8 cache write; the timed step writes the new tokens the same way
        hkv, d = c.num_kv_heads, c.head_dim
        kc8 = torch.full((c.num_blocks, 16, hkv, d), 0x7F, dtype=torch.uint8, device="cuda")
        vc8 = torch.full_like(kc8, 0x7F)
        ks8 = torch.full((c.num_blocks, hkv, 16), float("nan"), dtype=torch.float32, device="cuda")
        vs8 = torch.full_like(ks8, float("nan"))
        live = np.unique(np.concatenate([
            c.block_tables[b, np.arange(int(c.ctx_lens[b])) // 16].astype(np.int64) * 16
            + np.arange(int(c.ctx_lens[b])) % 16 for b in range(c.num_seqs)] + [np.zeros(0, np.int64)]))
        if len(live):
            idx = _i(live, torch.int64)
            pa.pa_reshape_and_cache_fp8(kc.view(-1, hkv, d).index_select(0, idx).contiguous(),
                                        vc.view(-1, hkv, d).index_select(0, idx).contiguous(),
                                        kc8, vc8, ks8, vs8, idx)
        torch.cuda.synchronize()
        kc = vc = None

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        if fp8:
            pa.pa_reshape_and_cache_fp8(key, value, kc8, vc8, ks8, vs8, slots)
        else:
            pa.pa_reshape_and_cache(key, value, kc, vc, slots)
        if ev is not None:
            ev[1].record()
        if fp8:
            pa.pa_prefill_paged_fp8(out, q, kc8, vc8, ks8, vs8, tables, ctx, qsl, c.scale, c.max_q_len)
        else:
            pa.pa_prefill_paged(out, q, kc, vc, tables, ctx, qsl, c.scale, c.max_q_len)
        if ev is not None:
            ev[2].record()

    _settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = _Timer(["write", "prefill"])
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer.step())
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = timer.mean_ms()
    L = c.q_lens.astype(np.int64)
    ctxl = c.ctx_lens.astype(np.int64)
    pairs = int((L * ctxl + L * (L + 1) // 2).sum())
    flops = 4 * c.num_q_heads * c.head_dim * pairs
    write_bytes = 2 * 2 * c.num_tokens * c.num_kv_heads * c.head_dim * 2   # read + write, K and V
    if fp8:   # 16-bit rows in, codes and scales out
        write_bytes = 2 * c.num_tokens * c.num_kv_heads * (c.head_dim * 2 + c.head_dim + 4)
    cpu = _oracle_prefill_rate(c, oracle_budget_s, fp8) if oracle_budget_s > 0 else None
    res = {"workload": "prefill_chunked_fp8" if fp8 else "prefill_chunked", "ms_per_step": round(wall, 4),
           "write_ms": round(per["write"], 4),
           "write_GBs": round(write_bytes / (per["write"] * 1e-3) / 1e9, 1),
           "write_pct_hbm_peak": round(100 * write_bytes / (per["write"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
           "prefill_ms": round(per["prefill"], 4), "prefill_flops": flops,
           "prefill_TFLOPs": round(flops / (per["prefill"] * 1e-3) / 1e12, 1),
           "prefill_pct_mfma_peak": round(100 * flops / (per["prefill"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 1),
           "new_tokens": c.num_tokens, "unmasked_pairs_per_head": pairs}
    if cpu:
        res["cpu_oracle"] = cpu
    if fp8:
        res["kv_cache"] = "fp8 e4m3 codes + float32 scale per (token, kv head)"
        del kc8, vc8, ks8, vs8
    del q, kc, vc, key, value, out
    torch.cuda.empty_cache()
    return res


def _secondary_copy_blocks(steps, warmup, pairs_n=2048):
    """Copy-on-write / swap block copy: 2048 random (src, dst) pairs in a
    32768-block bf16 pool with 8 kv heads of 128 (64 KiB of K+V per pair)."""
    import torch
    import paged_kv_cache_24_amd as pa
    nb, hkv, d = 32768, 8, 128
    kc = torch.empty((nb, 16, hkv, d), dtype=torch.bfloat16, device="cuda").normal_()
    vc = torch.empty_like(kc).normal_()
    perm = np.random.default_rng(6).permutation(nb)
    pairs = torch.from_numpy(np.stack([perm[:pairs_n], perm[pairs_n:2 * pairs_n]], 1).astype(np.int64)).cuda()
    _settle(lambda: pa.pa_copy_blocks(kc, vc, pairs))
    for _ in range(warmup):
        pa.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    timer = _Timer(["copy"])
    for _ in range(steps):
        ev = timer.step()
        ev[0].record()
        pa.pa_copy_blocks(kc, vc, pairs)
        ev[1].record()
    torch.cuda.synchronize()
    ms = timer.mean_ms()["copy"]
    moved = 2 * pairs_n * 2 * 16 * hkv * d * 2   # read + write, K and V
    del kc, vc
    torch.cuda.empty_cache()
    return {"workload": "copy_blocks", "pairs": pairs_n, "ms": round(ms, 4),
            "GBs_read_plus_write": round(moved / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}


def _secondary_multi(steps, warmup, nq=4):
    """Draft-token verification: the LLaMA-2-7B-shaped decode layer with nq
    queries per sequence (nq - 1 drafts plus the last accepted token), one
    pass over each sequence's cache."""
    import torch
    import paged_kv_cache_24_amd as pa
    from workloads import decode_llama2_7b_layer
    c = decode_llama2_7b_layer()
    run = DecodeRun(c)
    rng = np.random.default_rng(11)
    q = torch.from_numpy(rng.standard_normal((c.num_seqs, nq, c.num_q_heads, c.head_dim),
                                             dtype=np.float32)).to(torch.float16).cuda()
    out = torch.empty_like(q)
    # the library's own default partition for several queries (the size for
    # partition 0 of num_seqs * nq single-query sequences always suffices)
    need = pa.pa_decode_workspace_size(c.num_seqs * nq, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                       16, c.max_blocks_per_seq, 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    if run.has_write:
        pa.pa_reshape_and_cache(run.key, run.value, run.kc, run.vc, run.slots)

    def step():
        pa.pa_decode_multi(out, q, run.kc, run.vc, run.tables, run.lens, c.scale, 0, ws,
                           flags=run.flags)

    _settle(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = _Timer(["multi"])
    for _ in range(steps):
        ev = timer.step()
        ev[0].record()
        step()
        ev[1].record()
    torch.cuda.synchronize()
    ms = timer.mean_ms()["multi"]
    kv, _ = run.algorithmic_bytes()
    run.free()
    del run, q, out, ws
    torch.cuda.empty_cache()
    return {"workload": "decode_llama2_7b_layer_verify", "queries_per_seq": nq, "ms": round(ms, 4),
            "kv_bytes": kv, "kv_GBs": round(kv / (ms * 1e-3) / 1e9, 1),
            "pct_hbm_peak": round(100 * kv / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
            "query_tokens_per_s": round(c.num_seqs * nq / (ms * 1e-3), 1),
            "note": "all queries of a sequence share one read of its K/V (matrix-core kernel: "
                    "4 (query, head) columns per kv head; the balanced split at partition 0)"}


def _copy_probe(nbytes=4 << 30):
    """Achievable-bandwidth reference: a device-to-device copy of ``nbytes``
    (read + write counted), median of 5."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    ms = float(np.median(ts))
    return {"bytes": 2 * nbytes, "ms": round(ms, 3), "GBs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n}))


def _run_one(name, steps, warmup):
    from workloads import (decode_gqa_shared_prefix, decode_llama2_7b_layer,
                           decode_long_context, decode_tiny)
    table = {
        "decode_gqa_shared_prefix": lambda: _secondary_decode(
            decode_gqa_shared_prefix, name, steps, warmup, _shared_prefix_note, cpu=False, groups=True),
        "decode_long_context": lambda: _secondary_decode(decode_long_context, name, steps, warmup, cpu=False),
        "decode_tiny": lambda: _secondary_decode(decode_tiny, name, steps, warmup, cpu=False),
        "prefill_chunked": lambda: _secondary_prefill(steps, warmup, oracle_budget_s=0),
        "prefill_chunked_fp8": lambda: _secondary_prefill(steps, warmup, oracle_budget_s=0, fp8=True),
        "decode_llama2_7b_layer_fp8": lambda: _secondary_decode(
            decode_llama2_7b_layer, name, steps, warmup, cpu=False, fp8=True),
        "decode_gqa_shared_prefix_fp8": lambda: _secondary_decode(
            decode_gqa_shared_prefix, name, steps, warmup, cpu=False, fp8=True, groups=True),
        "decode_long_context_fp8": lambda: _secondary_decode(
            decode_long_context, name, steps, warmup, cpu=False, fp8=True),
        "decode_llama2_7b_layer_verify": lambda: _secondary_multi(steps, warmup),
        "copy_blocks": lambda: _secondary_copy_blocks(steps, warmup),
        "decode_llama2_7b_layer_bs32": lambda: _secondary_decode(
            lambda: decode_llama2_7b_layer(block_size=32), name, steps, warmup, cpu=False),
    }
    return table[name]()


_ONE_WORKLOAD = ("decode_gqa_shared_prefix", "decode_long_context", "decode_tiny", "prefill_chunked",
                 "prefill_chunked_fp8", "decode_llama2_7b_layer_fp8", "decode_gqa_shared_prefix_fp8",
                 "decode_long_context_fp8", "decode_llama2_7b_layer_verify", "copy_blocks",
                 "decode_llama2_7b_layer_bs32")


def _pmc_kib_per_dispatch(db_path, kernel_prefix, counter):
    """Mean of one counter (summed over its instances) per dispatch of the
    kernels whose name starts with kernel_prefix, from a rocprofv3 database."""
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = con.execute("select dispatch_id, name, counter_name, counter_value from pmc_events").fetchall()
    con.close()
    per = {}
    for disp, name, cname, val in rows:
        if cname == counter and name.startswith(kernel_prefix):
            per[disp] = per.get(disp, 0.0) + float(val)
    if not per:
        raise SystemExit(f"{db_path}: no {counter} samples for {kernel_prefix}")
    return sum(per.values()) / len(per), len(per)


def _traffic_profile(root):
    """HBM bytes per launch of the decode partition kernel: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) of the kernel, each scaled by what the same
    counter reads for a 1 GiB device copy (1 GiB read and 1 GiB written)."""
    import glob

    def db(sub):
        hits = glob.glob(os.path.join(root, sub, "**", "*_results.db"), recursive=True)
        if len(hits) != 1:
            raise SystemExit(f"expected one results database under {os.path.join(root, sub)}, found {hits}")
        return hits[0]

    kern = "void pa::decode_balanced_kernel<0, 128, 1, true>"
    copy = "__amd_rocclr_copyBuffer"
    f_dec, n_f = _pmc_kib_per_dispatch(db("dec_FETCH_SIZE"), kern, "FETCH_SIZE")
    w_dec, n_w = _pmc_kib_per_dispatch(db("dec_WRITE_SIZE"), kern, "WRITE_SIZE")
    f_copy, _ = _pmc_kib_per_dispatch(db("copy_FETCH_SIZE"), copy, "FETCH_SIZE")
    w_copy, _ = _pmc_kib_per_dispatch(db("copy_WRITE_SIZE"), copy, "WRITE_SIZE")
    n = 1 << 30
    fs, ws = n / (f_copy * 1024), n / (w_copy * 1024)
    from workloads import decode_llama2_7b_layer
    case = decode_llama2_7b_layer()
    lens = case.seq_lens.astype(np.int64)
    kv = int(lens.sum()) * 2 * case.num_kv_heads * case.head_dim * 2
    qo = 2 * case.num_seqs * case.num_q_heads * case.head_dim * 2
    algo = kv + qo + int(((lens + 15) // 16).sum()) * 4
    out = {
        "kernel": "decode_balanced_kernel<f16,128,1,stream> on decode_llama2_7b_layer (balanced split)",
        "decode_sources": [os.path.relpath(p, ROOT) for p in DECODE_SOURCES],
        "decode_sources_sha256": _decode_sources_sha256(),
        "fetch_size_kib_per_launch": round(f_dec, 1), "write_size_kib_per_launch": round(w_dec, 1),
        "dispatches": [n_f, n_w],
        "copy_calibration": {"bytes": n, "fetch_size_kib": round(f_copy, 1), "write_size_kib": round(w_copy, 1),
                             "fetch_scale": fs, "write_scale": ws},
        "hbm_fetch_bytes_per_launch": int(f_dec * 1024 * fs),
        "hbm_write_bytes_per_launch": int(w_dec * 1024 * ws),
        "hbm_bytes_per_launch": int(f_dec * 1024 * fs + w_dec * 1024 * ws),
        "algorithmic_bytes_per_launch": algo,
        # the runs that made the databases under `root` (the directory this was given)
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -d {root}/dec_FETCH_SIZE -o run -- python3 -u bench.py --quick --no-cpu-baseline --steps 5 --warmup 2",
            f"rocprofv3 --pmc WRITE_SIZE -d {root}/dec_WRITE_SIZE -o run -- python3 -u bench.py --quick --no-cpu-baseline --steps 5 --warmup 2",
            f"rocprofv3 --pmc FETCH_SIZE -d {root}/copy_FETCH_SIZE -o run -- python3 -u bench.py --copy-calibration",
            f"rocprofv3 --pmc WRITE_SIZE -d {root}/copy_WRITE_SIZE -o run -- python3 -u bench.py --copy-calibration",
            f"python3 bench.py --traffic-profile {root} > profiles/decode_balanced_llama2_7b_layer_traffic.json",
        ],
    }
    print(json.dumps(out, indent=1))


def main():
    args = _args()
    if args.traffic_profile:
        _traffic_profile(args.traffic_profile)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or kv head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        _copy_calibration()
        return
    if args.workload:
        import paged_kv_cache_24_amd  # noqa: F401  (raises if libpa.so is missing)
        print(json.dumps(_run_one(args.workload, args.steps, args.warmup)), flush=True)
        return
    import paged_kv_cache_24_amd  # noqa: F401  (raises if libpa.so is missing)
    from workloads import (decode_gqa_shared_prefix, decode_llama2_7b_layer,
                           decode_long_context, decode_tiny)

    t_gen = time.perf_counter()
    case = decode_llama2_7b_layer()
    gen_s = time.perf_counter() - t_gen
    run = DecodeRun(case)
    wall_ms, per = run.timed(args.steps, args.warmup)
    kv, algo = run.algorithmic_bytes()
    part_ms = per["partitions"]
    achieved = algo / (part_ms * 1e-3) / 1e9
    traffic = _traffic_if_current()
    value = kv / (wall_ms * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded N(0,1) q/k/v, random block placement)",
        "config": {"workload": "decode_llama2_7b_layer", "batch": case.num_seqs,
                   "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": 16,
                   "seq_lens": "uniform int [512, 4096], seed 2",
                   "num_blocks": case.num_blocks, "kv_bytes": kv,
                   "split": run.split, "stream_kv": bool(run.flags),
                   "step": "cache write of 64 tokens + paged decode (partitions + merge); HIP events "
                           "around the partition kernel only in the timed steps"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 1),
        "tokens_per_s": round(case.num_seqs / (wall_ms * 1e-3), 1),
        "kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "roofline": {"bound": "hbm",
                     "kernel": ("decode_balanced_kernel<f16,128,1>" if run.split == "balanced"
                                else "decode_partition_kernel<f16,128,1>"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": algo,
                     "traffic": traffic},
    }
    result["partition_kernel_ms_spread"] = run.last_timer.spread_ms("partitions")
    cold = run.timed_cold(max(5, args.steps // 2))
    cold_part = cold.spread_ms("partitions")
    result["cold_cache"] = {
        "note": "512 MiB written between steps (outside the events) to evict the Infinity Cache",
        "partition_kernel_ms": cold_part,
        "partition_kernel_GBs_p50": round(algo / (cold_part["p50"] * 1e-3) / 1e9, 1),
        "step_kernels_ms_p50": round(sum(cold.spread_ms(n)["p50"] for n in ("write", "partitions", "merge")), 4)}
    result["llama2_7b_attention_step_ms"] = round(32 * wall_ms, 3)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(case, args.cpu_seconds)
    run.free()
    del run, case
    torch.cuda.empty_cache()

    if not args.quick:
        sec = []
        s2, w2 = max(5, args.steps // 5), max(2, args.warmup // 2)
        sec.append(_secondary_decode(decode_gqa_shared_prefix, "decode_gqa_shared_prefix", s2, w2,
                                     _shared_prefix_note, groups=True))
        sec.append(_secondary_prefill(s2, w2))
        sec.append(_secondary_decode(decode_long_context, "decode_long_context", s2, w2))
        sec.append(_secondary_decode(decode_tiny, "decode_tiny", s2, w2))
        sec.append(_secondary_tiny_latency())
        sec.append(_secondary_copy_blocks(s2, w2))
        sec.append(_secondary_decode(decode_llama2_7b_layer, "decode_llama2_7b_layer_fp8", s2, w2,
                                     fp8=True))
        sec.append(_secondary_decode(decode_gqa_shared_prefix, "decode_gqa_shared_prefix_fp8", s2,
                                     w2, fp8=True, groups=True))
        sec.append(_secondary_decode(decode_long_context, "decode_long_context_fp8", s2, w2,
                                     fp8=True))
        sec.append(_secondary_prefill(s2, w2, fp8=True))
        sec.append(_secondary_multi(s2, w2))
        sec.append(_secondary_decode(lambda: decode_llama2_7b_layer(block_size=32),
                                     "decode_llama2_7b_layer_bs32", s2, w2, cpu=False))
        result["secondary"] = sec
    if not args.quick:
        result["achievable_copy_probe"] = _copy_probe()
    result["input_generation_s"] = round(gen_s, 1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
